"""Pins for the oracle's expert FFN, combine and whole-layer forward (CPU only)."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from synth import (get_config, draw_x, draw_wg, draw_sel_bias, draw_logit_bias, draw_w1_all,
                   draw_w2_all, draw_topk_given, f32_to_bf16_bits)
from tests import bruteforce as BF

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _c1():
    cfg = get_config("c1")
    return cfg, dict(x=draw_x(cfg), wg=draw_wg(cfg), sb=draw_sel_bias(cfg), lb=draw_logit_bias(cfg),
                     w1=draw_w1_all(cfg), w2=draw_w2_all(cfg))


def _fwd(cfg, d, **kw):
    return O.moe_forward(d["x"], d["w1"], d["w2"], T=cfg.T, H=cfg.H, E=cfg.E, K=cfg.K, I=cfg.I,
                         S=cfg.S, B=cfg.block_m, w_gate=d["wg"], logit_bias=d["lb"],
                         sel_bias=d["sb"], **kw)


def test_layer_matches_per_token_bruteforce_c1():
    cfg, d = _c1()
    out = _fwd(cfg, d)
    y, idx, w = BF.layer_forward(d["x"], d["wg"], d["lb"], d["sb"], d["w1"], d["w2"],
                                 cfg.T, cfg.E, cfg.K, cfg.I, cfg.S)
    np.testing.assert_array_equal(out["topk_idx"], idx)
    np.testing.assert_allclose(out["topk_w"], w, rtol=0, atol=1e-7)
    # Same rounding points on both sides: equal except, at most, a rare last-bit tie.
    diff = out["y"] != y
    assert diff.mean() < 1e-3
    np.testing.assert_allclose(out["y"], y, rtol=2**-7, atol=0)


def test_layer_matches_bruteforce_without_rounding():
    cfg, d = _c1()
    out = _fwd(cfg, d, rnd=None)
    y, _, _ = BF.layer_forward(d["x"], d["wg"], d["lb"], d["sb"], d["w1"], d["w2"],
                               cfg.T, cfg.E, cfg.K, cfg.I, cfg.S, rounding=False)
    np.testing.assert_allclose(out["y"], y, rtol=1e-12, atol=1e-14)


def test_grouped_ffn_equals_dense_per_expert_gemms():
    # Library routine as a pin: torch CPU float64 linear layers, one expert at a time.
    cfg = get_config("c1", T=96, E=6, K=3, S=1, block_m=32)
    x = draw_x(cfg)
    w1, w2 = draw_w1_all(cfg), draw_w2_all(cfg)
    idx = draw_topk_given(cfg.T, cfg.E, cfg.K, seed=4)
    Mcap = O.row_capacity(cfg.T, cfg.E, cfg.K, cfg.S, cfg.block_m)
    seg, _, total = O.build_segments(O.expert_counts(idx, cfg.E), cfg.T, cfg.E, cfg.S, cfg.block_m,
                                     Mcap)
    rt, _ = O.permute_maps(idx, seg, cfg.T, cfg.E, cfg.S, Mcap)
    xp = O.gather_rows(x, rt[:total])
    h, a, y = O.expert_ffn_forward(xp, seg, w1, w2, cfg.I)
    F = torch.nn.functional
    for g in range(cfg.G):
        r0, r1 = seg[g], seg[g + 1]
        xs = torch.from_numpy(xp[r0:r1])
        W1 = torch.from_numpy(O.bf16_to_f64(w1[g]))
        W2 = torch.from_numpy(O.bf16_to_f64(w2[g]))
        hh = F.linear(xs, W1)
        aa = F.silu(hh[:, :cfg.I]) * hh[:, cfg.I:]
        aa_r = torch.from_numpy(O.round_bf16(aa.numpy()))
        yy = O.round_bf16(F.linear(aa_r, W2).numpy())
        np.testing.assert_array_equal(a[r0:r1], aa_r.numpy())
        np.testing.assert_array_equal(y[r0:r1], yy)
        np.testing.assert_array_equal(h[r0:r1], O.round_bf16(hh.numpy()))
        pad = rt[r0:r1] < 0
        assert np.all(a[r0:r1][pad] == 0) and np.all(y[r0:r1][pad] == 0)


def test_single_expert_is_the_dense_swiglu_ffn():
    cfg = get_config("c1", E=1, K=1, S=0)
    x, w1, w2 = draw_x(cfg), draw_w1_all(cfg), draw_w2_all(cfg)
    idx = np.zeros((cfg.T, 1), np.int32)
    wts = np.ones((cfg.T, 1), np.float32)
    out = O.moe_forward(x, w1, w2, T=cfg.T, H=cfg.H, E=1, K=1, I=cfg.I, S=0, B=cfg.block_m,
                        topk_idx=idx, topk_w=wts)
    xv = O.bf16_to_f64(x)
    hh = xv @ O.bf16_to_f64(w1[0]).T
    a = O.round_bf16(O.silu(hh[:, :cfg.I]) * hh[:, cfg.I:])
    y = O.round_bf16(a @ O.bf16_to_f64(w2[0]).T)
    np.testing.assert_array_equal(out["y"], y)


def test_two_shared_experts_equal_one_of_twice_the_width():
    cfg = get_config("c1", S=2)
    rng = np.random.default_rng(0)
    T, H, I, E = cfg.T, cfg.H, cfg.I, cfg.E
    x = draw_x(cfg)
    w1, w2 = draw_w1_all(cfg), draw_w2_all(cfg)
    idx = draw_topk_given(T, E, cfg.K, seed=1)
    wts = rng.uniform(0.1, 1, (T, cfg.K)).astype(np.float32)
    kw = dict(T=T, H=H, E=E, K=cfg.K, B=cfg.block_m, topk_idx=idx, topk_w=wts, rnd=None)
    two = O.moe_forward(x, w1, w2, I=I, S=2, **kw)
    # One shared expert of width 2I: gate [G1; G2], up [U1; U2], down [D1 | D2]; routed experts get
    # zero-padded copies so every group has the same width.
    v1, v2 = O.bf16_to_f64(w1), O.bf16_to_f64(w2)
    G1 = np.zeros((E + 1, 4 * I, H))
    G2 = np.zeros((E + 1, H, 2 * I))
    for g in range(E):
        G1[g, :I], G1[g, 2 * I:3 * I] = v1[g, :I], v1[g, I:]
        G2[g, :, :I] = v2[g]
    s0, s1 = v1[E], v1[E + 1]
    G1[E] = np.concatenate([s0[:I], s1[:I], s0[I:], s1[I:]])
    G2[E] = np.concatenate([v2[E], v2[E + 1]], axis=1)
    one = O.moe_forward(x, G1, G2, I=2 * I, S=1, **kw)
    np.testing.assert_allclose(one["y"], two["y"], rtol=1e-12, atol=1e-13)


def test_identical_routed_experts_make_routing_irrelevant():
    cfg = get_config("c1", S=0)
    x = draw_x(cfg)
    w1 = np.repeat(draw_w1_all(cfg)[:1], cfg.E, axis=0)
    w2 = np.repeat(draw_w2_all(cfg)[:1], cfg.E, axis=0)
    kw = dict(T=cfg.T, H=cfg.H, E=cfg.E, K=cfg.K, I=cfg.I, S=0, B=cfg.block_m, rnd=None)
    ya = O.moe_forward(x, w1, w2, w_gate=draw_wg(cfg), sel_bias=draw_sel_bias(cfg), **kw)["y"]
    yb = O.moe_forward(x, w1, w2, w_gate=-draw_wg(cfg), sel_bias=None, **kw)["y"]
    # The weights are stored in fp32, so they sum to 1 only within a few fp32 ulps.
    np.testing.assert_allclose(ya, yb, rtol=5e-7, atol=1e-12)


def test_swiglu_golden():
    with open(os.path.join(GOLDEN, "swiglu_hand.json")) as f:
        g = json.load(f)
    x = np.array([g["x"]])
    w1 = np.array([g["w1"]])
    w2 = np.array([g["w2"]])
    seg = np.array([0, 1])
    h, a, y = O.expert_ffn_forward(x, seg, w1, w2, g["I"], rnd=None)
    np.testing.assert_allclose(a[0], g["a"], rtol=1e-14)
    np.testing.assert_allclose(y[0], g["y"], rtol=1e-14)
    dh, _ = O.expert_ffn_dgrad(np.array([g["dy"]]), h, seg, w1, w2, g["I"], rnd=None)
    np.testing.assert_allclose(dh[0], g["dh"], rtol=1e-14)


def test_combine_weights_and_shared_rows():
    # Combine on a hand-built permuted buffer: each row is a constant vector of its own index.
    T, E, K, S, H = 3, 2, 2, 1, 4
    idx = np.array([[0, 1], [1, 0], [1, 0]], np.int32)
    w = np.array([[0.5, 0.25], [1.0, 2.0], [0.0, 1.0]], np.float32)
    B = 4
    Mcap = O.row_capacity(T, E, K, S, B)
    seg, _, total = O.build_segments(O.expert_counts(idx, E), T, E, S, B, Mcap)
    _, pos = O.permute_maps(idx, seg, T, E, S, Mcap)
    yp = np.repeat(np.arange(total, dtype=np.float64)[:, None], H, axis=1)
    y = O.combine(yp, pos, w, seg, T, E, S, rnd=None)
    # expert 0 rows 0..2 (tokens 0,1,2), expert 1 rows 4..6, shared rows 8..10
    expect = [0.5 * 0 + 0.25 * 4 + 8, 1.0 * 5 + 2.0 * 1 + 9, 0.0 * 6 + 1.0 * 2 + 10]
    np.testing.assert_array_equal(y[:, 0], expect)


@pytest.mark.slow
def test_layer_bruteforce_skewed_small():
    cfg = get_config("c1", T=48, H=128, E=16, K=4, I=64, S=2, logit_bias="zipf", sel_bias="zero")
    d = dict(x=draw_x(cfg), wg=draw_wg(cfg), sb=draw_sel_bias(cfg), lb=draw_logit_bias(cfg),
             w1=draw_w1_all(cfg), w2=draw_w2_all(cfg))
    out = _fwd(cfg, d)
    y, idx, _ = BF.layer_forward(d["x"], d["wg"], d["lb"], d["sb"], d["w1"], d["w2"],
                                 cfg.T, cfg.E, cfg.K, cfg.I, cfg.S)
    np.testing.assert_array_equal(out["topk_idx"], idx)
    np.testing.assert_allclose(out["y"], y, rtol=2**-7, atol=0)
    assert (out["y"] != y).mean() < 1e-3
