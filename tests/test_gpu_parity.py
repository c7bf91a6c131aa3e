"""GPU parity of every stage of the HIP path against the CPU oracle, through the C ABI.

Bars: integer/index outputs and copies bit-exact; routing bit-exact where the oracle's ranking
margin between the K-th and (K+1)-th key is at least 1e-6 (elsewhere the GPU choice must be one of
the valid near-tied choices); fp32 logits rel-L2 <= 1e-5; bf16 GEMM outputs per
tests/gpu_helpers.assert_bf16_close (rel-L2 <= 2e-2 over the tensor and on every row).
"""
import numpy as np
import pytest
import torch

import grouped_gemm_fp32_amd as M
from oracle import moe_oracle as O
from synth import (get_config, draw_x, draw_wg, draw_sel_bias, draw_logit_bias, draw_w1_all,
                   draw_w2_all, draw_dy, draw_topk_given, draw_probs, draw_logits, uniform_topk)
from tests.gpu_helpers import (DEV, log, bf16_dev, f32_dev, i32_dev, bits_host, vals_host, rel_l2,
                               assert_bf16_close, validated_routing)

pytestmark = pytest.mark.gpu
DELTA = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    M.load_library()  # raises when the HIP library is missing: no fallback exists


def _np(t):
    return t.detach().cpu().numpy()


def _shape(T, H, E, K, I, S, B, normalize=True, probs_in=False):
    f = (M.MOE_NORM_TOPK if normalize else 0) | (M.MOE_PROBS_IN if probs_in else 0)
    return M.make_shape(T, H, E, K, I, S, B, f)


# ------------------------------------------------------------------------------------------------
# routing
# ------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("T,E,K,levels,normalize", [
    (777, 128, 6, 6, True), (777, 128, 6, 6, False), (300, 8, 8, 3, True), (513, 256, 8, 4, True),
    (64, 5, 2, 0, True), (1000, 128, 6, 0, True)])
def test_route_probs_input_bitexact(T, E, K, levels, normalize):
    log(f"route probs-in T={T} E={E} K={K} levels={levels} norm={normalize}")
    p = draw_probs(T, E, seed=T + E, levels=levels)
    b = (np.random.default_rng(E).integers(-3, 4, E) / 64).astype(np.float32)
    b[E // 3] = np.nan
    s = _shape(T, 128, E, K, 64, 0, 16, normalize, probs_in=True)
    idx, w = torch.empty(T, K, dtype=torch.int32, device=DEV), torch.empty(T, K, device=DEV)
    cnt = torch.empty(E, dtype=torch.int32, device=DEV)
    M.moe_route(s, None, None, None, f32_dev(b), None, f32_dev(p), idx, w, cnt)
    torch.cuda.synchronize()
    ref_idx, ref_w = O.select_topk(p, b, K, normalize)
    np.testing.assert_array_equal(_np(idx), ref_idx)
    if normalize:
        np.testing.assert_allclose(_np(w), ref_w, rtol=0, atol=1e-6)
    else:
        np.testing.assert_array_equal(_np(w), ref_w)
    np.testing.assert_array_equal(_np(cnt), O.expert_counts(ref_idx, E))


def test_route_logits_input():
    T, E, K = 1500, 128, 6
    z = draw_logits(T, E, seed=3, scale=2.0)
    b = np.random.default_rng(1).uniform(-0.02, 0.02, E).astype(np.float32)
    s = _shape(T, 128, E, K, 64, 0, 16)
    probs = torch.empty(T, E, device=DEV)
    idx, w = torch.empty(T, K, dtype=torch.int32, device=DEV), torch.empty(T, K, device=DEV)
    M.moe_route(s, None, None, None, f32_dev(b), f32_dev(z), probs, idx, w, None)
    torch.cuda.synchronize()
    ref_p = O.softmax_probs(z)
    gp = _np(probs).astype(np.float64)
    rel = np.abs(gp - ref_p) / np.maximum(ref_p, 1e-30)
    assert rel.max() < 4e-6, rel.max()
    # every token's weights, near-tied alternatives included: p renormalised over its experts
    vidx, vw, mism = validated_routing(_np(idx), ref_p, b, K, DELTA)
    np.testing.assert_allclose(_np(w), vw, rtol=0, atol=1e-6)


@pytest.mark.parametrize("name,T,over", [
    ("c1", None, {}), ("c3", 2048, {}), ("c5", None, {}), ("c5e", None, {}),
    # from 16384 tokens the logits kernel stages x and Wg in LDS (64 tokens per workgroup, all
    # experts): a ragged last token tile, and 200 experts (two expert blocks per wavefront, a
    # ragged last block)
    ("c3", 16384 + 77, {}), ("c3", 16400, {"E": 200, "K": 8})])
def test_route_from_x(name, T, over):
    cfg = get_config(name, **over) if T is None else get_config(name, T=T, **over)
    log(f"route from x: {cfg}")
    x, wg, sb, lb = draw_x(cfg), draw_wg(cfg), draw_sel_bias(cfg), draw_logit_bias(cfg)
    s = _shape(cfg.T, cfg.H, cfg.E, cfg.K, cfg.I, cfg.S, cfg.block_m)
    buf = M.alloc_buffers(s, DEV)
    M.moe_route(s, bf16_dev(x), f32_dev(wg), None if lb is None else f32_dev(lb), f32_dev(sb),
                buf["logits"], buf["probs"], buf["topk_idx"], buf["topk_w"], buf["expert_counts"])
    torch.cuda.synchronize()
    ref_logits = O.router_logits(x, wg, lb)
    r = rel_l2(_np(buf["logits"]), ref_logits)
    log(f"  logits rel-L2 {r:.2e}")
    assert r <= 1e-5
    ref_p = O.softmax_probs(ref_logits)
    vidx, vw, mism = validated_routing(_np(buf["topk_idx"]), ref_p, sb, cfg.K, DELTA)
    # Renormalised weights are the softmax of the selected logits, so first order
    # |dw_j| <= w_j (|dz_j| + sum_i w_i |dz_i|) <= 2 w_j max_i |dz_i|: the fp32-vs-fp64 logit
    # difference (bounded above by the rel-L2 bar) bounds the weight difference, plus fp32 rounding.
    # This holds for every token, near-tied alternatives included (their weights renormalise p
    # over the experts the GPU chose).
    dz = np.abs(_np(buf["logits"]).astype(np.float64) - ref_logits.astype(np.float64))
    dzmax = np.take_along_axis(dz, vidx.astype(np.int64), axis=1).max(axis=1, keepdims=True)
    bound = 2.0 * vw.astype(np.float64) * dzmax * 1.05 + 8 * 2.0 ** -24
    dw = np.abs(_np(buf["topk_w"]).astype(np.float64) - vw)
    assert np.all(dw <= bound), float((dw - bound).max())
    log(f"  weights: max |dw| {dw.max():.2e}, max logit diff {dz.max():.2e}")
    np.testing.assert_array_equal(_np(buf["expert_counts"]), O.expert_counts(vidx, cfg.E))
    if name == "c5e":
        assert np.all(_np(buf["expert_counts"])[list(cfg.forced_empty)] == 0)


# ------------------------------------------------------------------------------------------------
# permutation
# ------------------------------------------------------------------------------------------------
def _gpu_permute(s, idx, x_bits):
    buf = M.alloc_buffers(s, DEV)
    buf["row_token"].fill_(-7)
    M.moe_permute(s, i32_dev(idx), bf16_dev(x_bits), buf["seg_offsets"], buf["tile_group"],
                  buf["total_rows"], buf["row_token"], buf["pos"], buf["x_perm"], buf["ws"])
    return buf


@pytest.mark.parametrize("T,H,E,K,S,B,empty", [
    (64, 256, 8, 2, 1, 16, ()), (333, 256, 16, 4, 2, 32, (3, 9)), (1000, 128, 128, 6, 2, 128, ()),
    (4099, 128, 64, 8, 1, 64, tuple(range(0, 64, 5))), (257, 256, 256, 8, 4, 256, ()),
    (70000, 128, 128, 6, 2, 16, ()), (5, 128, 4, 4, 0, 16, ()),
    # the largest batch of one token block (the single-workgroup permutation) at the widest shape
    (256, 128, 256, 8, 4, 16, (1, 200))])
def test_permute_bitexact(T, H, E, K, S, B, empty):
    log(f"permute T={T} E={E} K={K} S={S} B={B}")
    idx = draw_topk_given(T, E, K, seed=T, forced_empty=empty)
    cfg = get_config("c1", T=T, H=H, E=E, K=K, S=S, block_m=B, seed=5)
    x = draw_x(cfg)
    s = _shape(T, H, E, K, 128, S, B)
    buf = _gpu_permute(s, idx, x)
    torch.cuda.synchronize()
    mcap = buf["mcap"]
    assert mcap == O.row_capacity(T, E, K, S, B)
    seg, tg, total = O.build_segments(O.expert_counts(idx, E), T, E, S, B, mcap)
    rt, pos = O.permute_maps(idx, seg, T, E, S, mcap)
    np.testing.assert_array_equal(_np(buf["seg_offsets"]), seg)
    assert int(_np(buf["total_rows"])[0]) == total
    np.testing.assert_array_equal(_np(buf["tile_group"]), tg)
    np.testing.assert_array_equal(_np(buf["row_token"])[:total], rt[:total])
    assert np.all(_np(buf["row_token"])[total:] == -7)   # rows past total_rows untouched
    np.testing.assert_array_equal(_np(buf["pos"]), pos)
    xp = bits_host(buf["x_perm"])[:total]
    np.testing.assert_array_equal(O.bf16_to_f64(xp), O.gather_rows(x, rt[:total]))


# ------------------------------------------------------------------------------------------------
# grouped GEMM forward / backward, combine
# ------------------------------------------------------------------------------------------------
def _layer_inputs(T, H, E, K, I, S, B, seed, empty=()):
    cfg = get_config("c1", T=T, H=H, E=E, K=K, I=I, S=S, block_m=B, seed=seed)
    idx = draw_topk_given(T, E, K, seed=seed, forced_empty=empty)
    w = np.random.default_rng(seed).uniform(0.05, 1.0, (T, K)).astype(np.float32)
    return cfg, idx, w, draw_x(cfg), draw_w1_all(cfg), draw_w2_all(cfg), draw_dy(cfg)


def _gpu_layer(s, idx, w, x, w1, w2, dy, backward=True):
    buf = M.alloc_buffers(s, DEV, backward=backward)
    M.moe_permute(s, i32_dev(idx), bf16_dev(x), buf["seg_offsets"], buf["tile_group"],
                  buf["total_rows"], buf["row_token"], buf["pos"], buf["x_perm"], buf["ws"])
    W1, W2, tw = bf16_dev(w1), bf16_dev(w2), f32_dev(w)
    M.grouped_gemm_fwd(s, M.MOE_FWD, buf["x_perm"], buf["seg_offsets"], buf["tile_group"], buf["total_rows"],
                       W1, W2, buf["h_save"], buf["a"], buf["y_perm"])
    M.moe_combine(s, buf["y_perm"], buf["pos"], tw, buf["seg_offsets"], buf["y"])
    if backward:
        M.moe_combine_bwd(s, bf16_dev(dy), buf["y_perm"], buf["pos"], tw, buf["seg_offsets"],
                          buf["row_token"], buf["total_rows"], buf["dy_perm"], buf["dtopk_w"])
        M.grouped_gemm_bwd(s, M.MOE_DGRAD | M.MOE_WGRAD, buf["x_perm"], buf["h_save"], buf["a"],
                           buf["dy_perm"], buf["seg_offsets"], buf["tile_group"],
                           buf["total_rows"], W1, W2, buf["dh"], buf["dx_perm"], buf["dw1"],
                           buf["dw2"])
        M.moe_unpermute_bwd(s, buf["dx_perm"], buf["pos"], buf["seg_offsets"], buf["dx"])
    torch.cuda.synchronize()
    return buf


def _oracle_layer(cfg, idx, w, x, w1, w2, dy, backward=True):
    kw = dict(T=cfg.T, H=cfg.H, E=cfg.E, K=cfg.K, I=cfg.I, S=cfg.S)
    f = O.moe_forward(x, w1, w2, B=cfg.block_m, topk_idx=idx, topk_w=w, **kw)
    b = O.moe_backward(f, dy, w1, w2, **kw) if backward else None
    return f, b


def _compare_layer(buf, f, b):
    total = f["total_rows"]
    assert int(_np(buf["total_rows"])[0]) == total
    pad = f["row_token"][:total] < 0
    for name, ref in (("h_save", f["h"]), ("a", f["a"]), ("y_perm", f["y_perm"])):
        got = vals_host(buf[name][:total])
        assert np.all(got[pad] == 0), f"{name}: padding rows not zero"
        assert_bf16_close(got, ref, name)
    assert_bf16_close(vals_host(buf["y"]), f["y"], "y")
    if b is None:
        return
    got = vals_host(buf["dy_perm"][:total])
    assert np.all(got[pad] == 0)
    assert_bf16_close(got, b["dy_perm"], "dy_perm")
    assert_bf16_close(_np(buf["dtopk_w"]), b["dtopk_w"], "dtopk_w", row_axis=0)
    assert_bf16_close(vals_host(buf["dh"][:total]), b["dh"], "dh")
    assert_bf16_close(vals_host(buf["dx_perm"][:total]), b["dx_perm"], "dx_perm")
    assert_bf16_close(vals_host(buf["dw1"]), b["dw1"], "dw1")
    assert_bf16_close(vals_host(buf["dw2"]), b["dw2"], "dw2")
    assert_bf16_close(vals_host(buf["dx"]), b["dx"], "dx")


@pytest.mark.parametrize("T,H,E,K,I,S,B,empty", [
    (64, 256, 8, 2, 128, 1, 16, ()),            # the tiny layer's sizes
    (333, 256, 8, 3, 192, 1, 16, (5,)),         # ragged: gate/up and down N tails, empty expert
    (333, 256, 8, 3, 192, 2, 32, ()),
    (500, 512, 16, 4, 256, 1, 64, (0, 15)),
    (700, 384, 12, 6, 320, 2, 128, (4,)),
    (300, 256, 6, 2, 128, 0, 256, ()),
    # more weight-gradient tiles (520 and 260) than persistent workgroups (256), skewed segments
    # from empty to 24 contraction stages: tiles chained and not chained within one workgroup
    (1500, 1024, 64, 4, 256, 1, 64, (3, 17, 40)),
    (1500, 1024, 64, 4, 256, 1, 128, (5,)),
    # one wave of tiles, so the host caps tiles at two 128-row blocks: the shared expert's 9
    # blocks split 2+2+2+2+1, a routed expert's 7 blocks 2+2+2+1
    (1100, 256, 4, 2, 128, 1, 128, (2,)),
    # tall tiles dealt to the XCDs in chunks of 4 row tiles (segments of about 6 blocks, two-block
    # tiles), skewed segments and a shared expert: 33 and 43 row tiles, a partial last chunk
    (1536, 256, 8, 4, 128, 1, 128, ()),
    (2000, 256, 8, 4, 128, 1, 128, ()),
    # a dense SwiGLU FFN as one group (E = K = 1): one segment of every token, many row tiles
    (1000, 512, 1, 1, 1024, 0, 128, ()),
    (777, 256, 1, 1, 320, 0, 64, ()),
])
def test_layer_parity(T, H, E, K, I, S, B, empty):
    log(f"layer T={T} H={H} E={E} K={K} I={I} S={S} B={B} empty={empty}")
    cfg, idx, w, x, w1, w2, dy = _layer_inputs(T, H, E, K, I, S, B, seed=T + B, empty=empty)
    s = _shape(T, H, E, K, I, S, B)
    buf = _gpu_layer(s, idx, w, x, w1, w2, dy)
    f, b = _oracle_layer(cfg, idx, w, x, w1, w2, dy)
    _compare_layer(buf, f, b)
    for e in empty:   # empty experts: zero weight gradients
        assert np.all(vals_host(buf["dw1"])[e] == 0) and np.all(vals_host(buf["dw2"])[e] == 0)


def test_full_tiny_layer_from_router():
    """The tiny configuration end to end: router on x, then every stage, forward and backward."""
    cfg = get_config("c1")
    x, wg, sb = draw_x(cfg), draw_wg(cfg), draw_sel_bias(cfg)
    w1, w2, dy = draw_w1_all(cfg), draw_w2_all(cfg), draw_dy(cfg)
    s = _shape(cfg.T, cfg.H, cfg.E, cfg.K, cfg.I, cfg.S, cfg.block_m)
    buf = M.alloc_buffers(s, DEV)
    M.moe_route(s, bf16_dev(x), f32_dev(wg), None, f32_dev(sb), buf["logits"], buf["probs"],
                buf["topk_idx"], buf["topk_w"], buf["expert_counts"])
    torch.cuda.synchronize()
    ref = O.moe_forward(x, w1, w2, T=cfg.T, H=cfg.H, E=cfg.E, K=cfg.K, I=cfg.I, S=cfg.S,
                        B=cfg.block_m, w_gate=wg, sel_bias=sb)
    np.testing.assert_array_equal(_np(buf["topk_idx"]), ref["topk_idx"])
    np.testing.assert_allclose(_np(buf["topk_w"]), ref["topk_w"], rtol=0, atol=1e-6)
    buf2 = _gpu_layer(s, ref["topk_idx"], _np(buf["topk_w"]), x, w1, w2, dy)
    f, b = _oracle_layer(cfg, ref["topk_idx"], ref["topk_w"], x, w1, w2, dy)
    _compare_layer(buf2, f, b)


def test_deterministic_bitwise():
    cfg, idx, w, x, w1, w2, dy = _layer_inputs(333, 256, 8, 3, 192, 1, 16, seed=1)
    s = _shape(333, 256, 8, 3, 192, 1, 16)
    b1 = _gpu_layer(s, idx, w, x, w1, w2, dy)
    b2 = _gpu_layer(s, idx, w, x, w1, w2, dy)
    total = int(_np(b1["total_rows"])[0])
    for k in ("y", "dx", "dw1", "dw2", "dtopk_w"):
        assert torch.equal(b1[k], b2[k]), k
    for k in ("a", "y_perm", "h_save", "dh", "dx_perm"):
        assert torch.equal(b1[k][:total], b2[k][:total]), k


def test_all_tokens_on_one_expert_and_k_equals_e():
    T, H, E, K, I, S, B = 200, 256, 4, 4, 128, 1, 16
    idx = np.tile(np.arange(K, dtype=np.int32)[::-1], (T, 1))
    cfg = get_config("c1", T=T, H=H, E=E, K=K, I=I, S=S, block_m=B, seed=9)
    w = np.full((T, K), 0.25, np.float32)
    x, w1, w2, dy = draw_x(cfg), draw_w1_all(cfg), draw_w2_all(cfg), draw_dy(cfg)
    buf = _gpu_layer(_shape(T, H, E, K, I, S, B), idx, w, x, w1, w2, dy)
    f, b = _oracle_layer(cfg, idx, w, x, w1, w2, dy)
    _compare_layer(buf, f, b)


def test_empty_batch():
    s = _shape(0, 256, 8, 2, 128, 1, 16)
    buf = M.alloc_buffers(s, DEV, backward=True)
    buf["seg_offsets"].fill_(5)
    buf["dw1"].fill_(1.0)
    buf["dw2"].fill_(1.0)
    idx = torch.empty(0, 2, dtype=torch.int32, device=DEV)
    M.moe_permute(s, idx, None, buf["seg_offsets"], buf["tile_group"], buf["total_rows"],
                  buf["row_token"], buf["pos"], None, buf["ws"])
    M.grouped_gemm_bwd(s, M.MOE_WGRAD, buf["x_perm"], buf["h_save"], buf["a"], buf["dy_perm"],
                       buf["seg_offsets"], None, None, None, None, buf["dh"], None, buf["dw1"],
                       buf["dw2"])
    counts = torch.full((8,), 7, dtype=torch.int32, device=DEV)
    M.moe_route(s, None, None, None, None, None, None, None, None, counts)
    torch.cuda.synchronize()
    assert np.all(_np(buf["seg_offsets"]) == 0) and int(_np(buf["total_rows"])[0]) == 0
    assert float(buf["dw1"].float().abs().sum()) == 0 and float(buf["dw2"].float().abs().sum()) == 0
    assert np.all(_np(counts) == 0)   # no token routed: every count is zero
