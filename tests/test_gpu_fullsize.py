"""GPU parity at the full workload sizes, in the launch configuration bench.py times, on outputs
the oracle computes one by one (sampled rows, sampled tokens, whole weight gradients of sampled
experts), plus exact checks of every integer map. Bars as in tests/gpu_helpers.py."""
import numpy as np
import pytest
import torch

import grouped_gemm_fp32_amd as M
from oracle import moe_oracle as O
from synth import (get_config, draw_probs, draw_x, draw_wg, draw_sel_bias, draw_logit_bias, draw_w1_all,
                   draw_w2_all, draw_dy, uniform_topk, uniform_logits, skewed_logits)
from tests.gpu_helpers import (DEV, log, bf16_dev, f32_dev, i32_dev, bits_host, vals_host, rel_l2,
                               assert_bf16_close, validated_routing)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    M.load_library()


def _np(t):
    return t.detach().cpu().numpy()


def _sample_rows(seg, rng, per_group=3, groups=24):
    """Rows to check: first, last and one random row of a spread of non-empty groups."""
    G = len(seg) - 1
    nonempty = [g for g in range(G) if seg[g + 1] > seg[g]]
    pick = sorted(set(np.linspace(0, len(nonempty) - 1, min(groups, len(nonempty))).astype(int)))
    rows = []
    for i in pick:
        g = nonempty[i]
        r0, r1 = int(seg[g]), int(seg[g + 1])
        rows += [r0, r1 - 1] + list(rng.integers(r0, r1, per_group - 2))
    return np.array(sorted(set(rows)))


def _oracle_rows(rows, seg, row_token, x_bits, cfg, w1_of, w2_of):
    """h, a, y_perm of the given permuted rows, each evaluated on its own."""
    H, I = cfg.H, cfg.I
    h = np.zeros((len(rows), 2 * I))
    a = np.zeros((len(rows), I))
    y = np.zeros((len(rows), H))
    groups = np.searchsorted(seg, rows, side="right") - 1
    for g in sorted(set(groups.tolist())):
        sel = np.nonzero(groups == g)[0]
        toks = row_token[rows[sel]]
        xr = np.zeros((len(sel), H))
        ok = toks >= 0
        xr[ok] = O.bf16_to_f64(x_bits[toks[ok]])
        h[sel], a[sel], y[sel] = O.expert_ffn_rows(xr, O.bf16_to_f64(w1_of(g)),
                                                    O.bf16_to_f64(w2_of(g)), I)
    return h, a, y


def _run_forward(cfg, s, X, W1, W2, route_kw):
    buf = M.alloc_buffers(s, DEV, backward=True)
    M.moe_route(s, **route_kw, probs=buf["probs"], topk_idx=buf["topk_idx"], topk_w=buf["topk_w"],
                expert_counts=buf["expert_counts"])
    M.moe_permute(s, buf["topk_idx"], X, buf["seg_offsets"], buf["tile_group"], buf["total_rows"],
                  buf["row_token"], buf["pos"], buf["x_perm"], buf["ws"])
    M.grouped_gemm_fwd(s, M.MOE_FWD, buf["x_perm"], buf["seg_offsets"], buf["tile_group"],
                       buf["total_rows"], W1, W2, buf["h_save"], buf["a"], buf["y_perm"])
    M.moe_combine(s, buf["y_perm"], buf["pos"], buf["topk_w"], buf["seg_offsets"], buf["y"])
    torch.cuda.synchronize()
    return buf


def _check_maps_exact(buf, idx, cfg):
    mcap = buf["mcap"]
    seg, tg, total = O.build_segments(O.expert_counts(idx, cfg.E), cfg.T, cfg.E, cfg.S,
                                      cfg.block_m, mcap)
    rt, pos = O.permute_maps(idx, seg, cfg.T, cfg.E, cfg.S, mcap)
    np.testing.assert_array_equal(_np(buf["seg_offsets"]), seg)
    assert int(_np(buf["total_rows"])[0]) == total
    np.testing.assert_array_equal(_np(buf["tile_group"]), tg)
    np.testing.assert_array_equal(_np(buf["row_token"])[:total], rt[:total])
    np.testing.assert_array_equal(_np(buf["pos"]), pos)
    return seg, rt, pos, total


def test_uniform_8192_tokens_forward_and_backward():
    """Bench workload: T=8192, hidden 4096, 128 experts top-6, intermediate 1408, block 128."""
    _uniform_layer(get_config("c2"), wgrad_groups=(0, 77, 127))


def test_expert_parallel_share_forward_and_backward():
    """One GPU's share of the bench layer under 8-way expert parallelism: 16 local experts with
    3072 rows each (8192 tokens top-6 over 16 experts), so each weight-gradient tile contracts
    over 48 stages of 64 rows."""
    _uniform_layer(get_config("ep8"), wgrad_groups=(5,), per_group=4)


def test_skewed_8192_tokens_forward_and_backward():
    """The bench workload's shapes under Zipf(1.1)-skewed routing (bench.py --workload c4z: 58 to
    6693 rows per expert). The most popular expert's weight-gradient tiles contract over more
    than a hundred 64-row stages and the least popular's over one, so the persistent weight-gradient kernel cuts its XCD
    ranges inside groups; both experts' whole weight gradients are checked."""
    cfg = get_config("c4z")
    idx, _ = O.select_topk(O.softmax_probs(skewed_logits(cfg)), None, cfg.K)
    counts = O.expert_counts(idx, cfg.E)
    hot, rare = int(np.argmax(counts)), int(np.argmin(counts))
    log(f"skewed routing: expert {hot} has {counts[hot]} rows, expert {rare} {counts[rare]}")
    _uniform_layer(cfg, wgrad_groups=(hot, rare), uniform=False)


def _uniform_layer(cfg, wgrad_groups, per_group=3, uniform=True):
    """Forward and backward at a full-size shape routed from logits that encode a given routing
    (uniform, or skewed with uniform=False): exact routing and maps, sampled rows through the FFN,
    the combine and the dgrad, and the whole weight gradients of wgrad_groups (the oracle runs
    their full segments)."""
    log(f"full size: {cfg}")
    s = M.make_shape(cfg.T, cfg.H, cfg.E, cfg.K, cfg.I, cfg.S, cfg.block_m)
    x, dy = draw_x(cfg), draw_dy(cfg)
    logits = uniform_logits(cfg) if uniform else skewed_logits(cfg)
    w1, w2 = draw_w1_all(cfg), draw_w2_all(cfg)
    X, W1, W2 = bf16_dev(x), bf16_dev(w1), bf16_dev(w2)
    buf = _run_forward(cfg, s, X, W1, W2, dict(x=None, w_gate=None, logit_bias=None, sel_bias=None,
                                               logits=f32_dev(logits)))
    # routing: the uniform assignment, exactly; weights from the oracle's own softmax
    probs = O.softmax_probs(logits)
    idx, w = O.select_topk(probs, None, cfg.K)
    if uniform:
        np.testing.assert_array_equal(np.sort(idx, 1), np.sort(uniform_topk(cfg.T, cfg.E, cfg.K), 1))
    np.testing.assert_array_equal(_np(buf["topk_idx"]), idx)
    np.testing.assert_allclose(_np(buf["topk_w"]), w, rtol=0, atol=1e-6)
    seg, rt, pos, total = _check_maps_exact(buf, idx, cfg)
    # the row copy, bit for bit: x[row_token[r]], zero bits on padding rows (skewed segments)
    want = np.where((rt[:total] >= 0)[:, None], x[np.maximum(rt[:total], 0)], 0).astype(x.dtype)
    np.testing.assert_array_equal(bits_host(buf["x_perm"][:total]), want)
    # sampled permuted rows through the expert FFN
    rng = np.random.default_rng(0)
    rows = _sample_rows(seg, rng, per_group=per_group)
    h_ref, a_ref, y_ref = _oracle_rows(rows, seg, rt, x, cfg, lambda g: w1[g], lambda g: w2[g])
    R = torch.from_numpy(rows).to(DEV)
    assert_bf16_close(vals_host(buf["h_save"][R]), O.round_bf16(h_ref), "h_save rows")
    assert_bf16_close(vals_host(buf["a"][R]), a_ref, "a rows")
    assert_bf16_close(vals_host(buf["y_perm"][R]), y_ref, "y_perm rows")
    # sampled tokens through the combine
    toks = rng.choice(cfg.T, 32, replace=False)
    y_tok = np.zeros((len(toks), cfg.H))
    for i, t in enumerate(toks):
        for j in range(cfg.K):
            e = idx[t, j]
            _, _, ye = O.expert_ffn_rows(O.bf16_to_f64(x[t:t + 1]), O.bf16_to_f64(w1[e]),
                                         O.bf16_to_f64(w2[e]), cfg.I)
            y_tok[i] += np.float64(w[t, j]) * ye[0]
    assert_bf16_close(vals_host(buf["y"][torch.from_numpy(toks).to(DEV)]), O.round_bf16(y_tok), "y tokens")

    # ---- backward in the same configuration --------------------------------------------------
    DY = bf16_dev(dy)
    M.moe_combine_bwd(s, DY, buf["y_perm"], buf["pos"], buf["topk_w"], buf["seg_offsets"],
                      buf["row_token"], buf["total_rows"], buf["dy_perm"], buf["dtopk_w"])
    M.grouped_gemm_bwd(s, M.MOE_DGRAD | M.MOE_WGRAD, buf["x_perm"], buf["h_save"], buf["a"],
                       buf["dy_perm"], buf["seg_offsets"], buf["tile_group"], buf["total_rows"],
                       W1, W2, buf["dh"], buf["dx_perm"], buf["dw1"], buf["dw2"])
    M.moe_unpermute_bwd(s, buf["dx_perm"], buf["pos"], buf["seg_offsets"], buf["dx"])
    torch.cuda.synchronize()
    # dgrad rows: dy_perm, dh, dx_perm from the oracle's per-row forward
    slot = {}
    for t in range(cfg.T):
        for j in range(cfg.K):
            slot[pos[t, j]] = (t, j)
    dyp_ref = np.zeros((len(rows), cfg.H))   # zero on padding rows (no slot)
    for i, r in enumerate(rows):
        if r in slot:
            t, j = slot[r]
            dyp_ref[i] = O.round_bf16(np.float64(w[t, j]) * O.bf16_to_f64(dy[t]))
    groups = np.searchsorted(seg, rows, side="right") - 1
    dh_ref = np.zeros((len(rows), 2 * cfg.I))
    dx_ref = np.zeros((len(rows), cfg.H))
    for g in sorted(set(groups.tolist())):
        sel = np.nonzero(groups == g)[0]
        dh_g, dx_g = O.expert_ffn_dgrad(dyp_ref[sel], O.round_bf16(h_ref[sel]), [0, len(sel)],
                                        [w1[g]], [w2[g]], cfg.I)
        dh_ref[sel], dx_ref[sel] = dh_g, dx_g
    assert_bf16_close(vals_host(buf["dy_perm"][R]), dyp_ref, "dy_perm rows")
    assert_bf16_close(vals_host(buf["dh"][R]), dh_ref, "dh rows")
    assert_bf16_close(vals_host(buf["dx_perm"][R]), dx_ref, "dx_perm rows")
    # wgrad: whole dW of the chosen experts (the oracle runs their full segments)
    for g in wgrad_groups:
        r0, r1 = int(seg[g]), int(seg[g + 1])
        seg_rows = np.arange(r0, r1)
        hg, ag, yg = _oracle_rows(seg_rows, seg, rt, x, cfg, lambda q: w1[q], lambda q: w2[q])
        dyp = np.zeros((r1 - r0, cfg.H))
        for i, r in enumerate(seg_rows):
            if r in slot:
                t, j = slot[r]
                dyp[i] = O.round_bf16(np.float64(w[t, j]) * O.bf16_to_f64(dy[t]))
        dhg, _ = O.expert_ffn_dgrad(dyp, O.round_bf16(hg), [0, r1 - r0], [w1[g]], [w2[g]], cfg.I)
        xg = O.gather_rows(x, rt[r0:r1])
        dw1, dw2 = O.expert_ffn_wgrad(xg, ag, dyp, dhg, [0, r1 - r0], cfg.I, cfg.H)
        assert_bf16_close(vals_host(buf["dw1"][g]), dw1[0], f"dw1[{g}]")
        assert_bf16_close(vals_host(buf["dw2"][g]), dw2[0], f"dw2[{g}]")


def test_dense_ffn_8192_tokens_forward_and_backward():
    """Dense SwiGLU FFN as one group (E = K = 1): T=8192, hidden 4096, intermediate 11264, block 128.

    With one expert of weight 1 the combine and the unpermute are exact copies (y = y_perm, dx =
    dx_perm, dy_perm = dy, bit for bit); sampled rows are checked through the FFN and its dgrad.
    """
    cfg = get_config("dense")
    log(f"full size: {cfg}")
    s = M.make_shape(cfg.T, cfg.H, cfg.E, cfg.K, cfg.I, cfg.S, cfg.block_m)
    x, dy, logits = draw_x(cfg), draw_dy(cfg), uniform_logits(cfg)
    w1, w2 = draw_w1_all(cfg), draw_w2_all(cfg)
    X, W1, W2 = bf16_dev(x), bf16_dev(w1), bf16_dev(w2)
    buf = _run_forward(cfg, s, X, W1, W2, dict(x=None, w_gate=None, logit_bias=None, sel_bias=None,
                                               logits=f32_dev(logits)))
    idx = np.zeros((cfg.T, 1), np.int32)
    np.testing.assert_array_equal(_np(buf["topk_idx"]), idx)
    assert np.all(_np(buf["topk_w"]) == 1.0)
    seg, rt, pos, total = _check_maps_exact(buf, idx, cfg)
    assert total == cfg.T and np.array_equal(rt[:total], np.arange(cfg.T))
    np.testing.assert_array_equal(bits_host(buf["x_perm"][:total]), x)
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([[0, 1, 383, 384, cfg.T - 1], rng.integers(0, cfg.T, 27)]))
    h_ref, a_ref, y_ref = _oracle_rows(rows, seg, rt, x, cfg, lambda g: w1[g], lambda g: w2[g])
    R = torch.from_numpy(rows).to(DEV)
    assert_bf16_close(vals_host(buf["h_save"][R]), O.round_bf16(h_ref), "h_save rows")
    assert_bf16_close(vals_host(buf["a"][R]), a_ref, "a rows")
    assert_bf16_close(vals_host(buf["y_perm"][R]), y_ref, "y_perm rows")
    assert torch.equal(buf["y"].view(torch.int16), buf["y_perm"][:cfg.T].view(torch.int16))
    DY = bf16_dev(dy)
    M.moe_combine_bwd(s, DY, buf["y_perm"], buf["pos"], buf["topk_w"], buf["seg_offsets"],
                      buf["row_token"], buf["total_rows"], buf["dy_perm"], buf["dtopk_w"])
    M.grouped_gemm_bwd(s, M.MOE_DGRAD | M.MOE_WGRAD, buf["x_perm"], buf["h_save"], buf["a"],
                       buf["dy_perm"], buf["seg_offsets"], buf["tile_group"], buf["total_rows"],
                       W1, W2, buf["dh"], buf["dx_perm"], buf["dw1"], buf["dw2"])
    M.moe_unpermute_bwd(s, buf["dx_perm"], buf["pos"], buf["seg_offsets"], buf["dx"])
    torch.cuda.synchronize()
    assert torch.equal(buf["dy_perm"][:cfg.T].view(torch.int16), DY.view(torch.int16))
    assert torch.equal(buf["dx"].view(torch.int16), buf["dx_perm"][:cfg.T].view(torch.int16))
    dh_ref, dx_ref = O.expert_ffn_dgrad(O.bf16_to_f64(dy[rows]), O.round_bf16(h_ref),
                                        [0, len(rows)], [w1[0]], [w2[0]], cfg.I)
    assert_bf16_close(vals_host(buf["dh"][R]), dh_ref, "dh rows")
    assert_bf16_close(vals_host(buf["dx_perm"][R]), dx_ref, "dx_perm rows")


def test_skewed_16384_tokens_full_layer():
    """Router with Zipf(1.1) logit offsets, two shared experts, block 128; forward."""
    cfg = get_config("c3")
    log(f"full size: {cfg}")
    s = M.make_shape(cfg.T, cfg.H, cfg.E, cfg.K, cfg.I, cfg.S, cfg.block_m)
    x, wg, sb, lb = draw_x(cfg), draw_wg(cfg), draw_sel_bias(cfg), draw_logit_bias(cfg)
    w1, w2 = draw_w1_all(cfg), draw_w2_all(cfg)
    w1_of, w2_of = (lambda g: w1[g]), (lambda g: w2[g])
    W1, W2 = bf16_dev(w1), bf16_dev(w2)
    X = bf16_dev(x)
    logits = torch.empty(cfg.T, cfg.E, device=DEV)
    buf = _run_forward(cfg, s, X, W1, W2, dict(x=X, w_gate=f32_dev(wg), logit_bias=f32_dev(lb),
                                               sel_bias=f32_dev(sb), logits=logits))
    ref_logits = O.router_logits(x, wg, lb)
    r = rel_l2(_np(logits), ref_logits)
    log(f"  logits rel-L2 {r:.2e}")
    assert r <= 1e-5
    ref_p = O.softmax_probs(ref_logits)
    # The oracle's routing, with near-tied tokens taken as the GPU chose them once shown valid;
    # every map and expected row below is then built by the oracle from that selection.
    idx, w, mism = validated_routing(_np(buf["topk_idx"]), ref_p, sb, cfg.K)
    dz = np.abs(_np(logits).astype(np.float64) - ref_logits.astype(np.float64))
    dzmax = np.take_along_axis(dz, idx.astype(np.int64), axis=1).max(axis=1, keepdims=True)
    bound = 2.0 * w.astype(np.float64) * dzmax * 1.05 + 8 * 2.0 ** -24   # see test_route_from_x
    assert np.all(np.abs(_np(buf["topk_w"]).astype(np.float64) - w) <= bound)
    np.testing.assert_array_equal(_np(buf["expert_counts"]), O.expert_counts(idx, cfg.E))
    seg, rt, pos, total = _check_maps_exact(buf, idx, cfg)
    # sampled tokens (every near-tied one among them): y[t] from per-token expert evaluations
    rng = np.random.default_rng(3)
    toks = np.union1d(rng.choice(cfg.T, 24, replace=False), np.nonzero(mism)[0][:8])
    y_tok = np.zeros((len(toks), cfg.H))
    for i, t in enumerate(toks):
        xt = O.bf16_to_f64(x[t:t + 1])
        for j in range(cfg.K):
            e = idx[t, j]
            y_tok[i] += np.float64(w[t, j]) * O.expert_ffn_rows(
                xt, O.bf16_to_f64(w1_of(e)), O.bf16_to_f64(w2_of(e)), cfg.I)[2][0]
        for sh in range(cfg.S):
            y_tok[i] += O.expert_ffn_rows(xt, O.bf16_to_f64(w1_of(cfg.E + sh)),
                                          O.bf16_to_f64(w2_of(cfg.E + sh)), cfg.I)[2][0]
    assert_bf16_close(vals_host(buf["y"][torch.from_numpy(toks).to(DEV)]), O.round_bf16(y_tok), "y tokens")
    # sampled permuted rows (including the heaviest expert and both shared experts)
    rows = _sample_rows(seg, rng, per_group=4, groups=20)
    h_ref, a_ref, y_ref = _oracle_rows(rows, seg, rt, x, cfg, w1_of, w2_of)
    R = torch.from_numpy(rows).to(DEV)
    assert_bf16_close(vals_host(buf["a"][R]), a_ref, "a rows")
    assert_bf16_close(vals_host(buf["y_perm"][R]), y_ref, "y_perm rows")


@pytest.mark.parametrize("name", ["c5", "c5e"])
def test_decode_256_tokens_full_layer(name):
    """Decode-sized layer (block 16): the whole forward output against the oracle."""
    cfg = get_config(name)
    log(f"full size: {cfg}")
    s = M.make_shape(cfg.T, cfg.H, cfg.E, cfg.K, cfg.I, cfg.S, cfg.block_m)
    x, wg, sb = draw_x(cfg), draw_wg(cfg), draw_sel_bias(cfg)
    w1, w2 = draw_w1_all(cfg), draw_w2_all(cfg)
    X = bf16_dev(x)
    logits = torch.empty(cfg.T, cfg.E, device=DEV)
    buf = _run_forward(cfg, s, X, bf16_dev(w1), bf16_dev(w2),
                       dict(x=X, w_gate=f32_dev(wg), logit_bias=None, sel_bias=f32_dev(sb),
                            logits=logits))
    ref = O.moe_forward(x, w1, w2, T=cfg.T, H=cfg.H, E=cfg.E, K=cfg.K, I=cfg.I, S=cfg.S,
                        B=cfg.block_m, w_gate=wg, sel_bias=sb)
    assert rel_l2(_np(logits), ref["logits"]) <= 1e-5
    np.testing.assert_array_equal(_np(buf["topk_idx"]), ref["topk_idx"])
    seg, rt, pos, total = _check_maps_exact(buf, ref["topk_idx"], cfg)
    if name == "c5e":
        for e in cfg.forced_empty:
            assert seg[e + 1] == seg[e]
    # rows past total_rows are never written: only the written rows are decoded
    assert_bf16_close(vals_host(buf["a"][:total]), ref["a"], "a")
    assert_bf16_close(vals_host(buf["y_perm"][:total]), ref["y_perm"], "y_perm")
    assert_bf16_close(vals_host(buf["y"]), ref["y"], "y")


def test_largest_shape_routing_permutation_and_forward():
    """The largest shape the library accepts in tokens, experts, slots and shared experts: T=262144,
    E=256, K=8, S=4, block 256 (hidden 128, intermediate 64 to keep it small). Routing from given
    probabilities and every integer map bit-exact; sampled rows through the expert FFN and sampled
    tokens through the combine."""
    cfg = get_config("c1", T=262144, H=128, E=256, K=8, I=64, S=4, block_m=256, seed=3)
    log(f"largest shape: {cfg}")
    s = M.make_shape(cfg.T, cfg.H, cfg.E, cfg.K, cfg.I, cfg.S, cfg.block_m,
                     M.MOE_NORM_TOPK | M.MOE_PROBS_IN)
    p = draw_probs(cfg.T, cfg.E, seed=3, levels=6)   # many ties: the index order decides them
    sb = (np.random.default_rng(3).integers(-3, 4, cfg.E) / 1024).astype(np.float32)
    x, w1, w2 = draw_x(cfg), draw_w1_all(cfg), draw_w2_all(cfg)
    X, W1, W2 = bf16_dev(x), bf16_dev(w1), bf16_dev(w2)
    buf = M.alloc_buffers(s, DEV)
    buf["probs"].copy_(f32_dev(p))
    M.moe_route(s, None, None, None, f32_dev(sb), None, buf["probs"], buf["topk_idx"], buf["topk_w"],
                buf["expert_counts"])
    M.moe_permute(s, buf["topk_idx"], X, buf["seg_offsets"], buf["tile_group"], buf["total_rows"],
                  buf["row_token"], buf["pos"], buf["x_perm"], buf["ws"])
    M.grouped_gemm_fwd(s, M.MOE_FWD, buf["x_perm"], buf["seg_offsets"], buf["tile_group"],
                       buf["total_rows"], W1, W2, buf["h_save"], buf["a"], buf["y_perm"])
    M.moe_combine(s, buf["y_perm"], buf["pos"], buf["topk_w"], buf["seg_offsets"], buf["y"])
    torch.cuda.synchronize()
    idx, w = O.select_topk(p, sb, cfg.K)
    np.testing.assert_array_equal(_np(buf["topk_idx"]), idx)
    np.testing.assert_array_equal(_np(buf["expert_counts"]), O.expert_counts(idx, cfg.E))
    np.testing.assert_allclose(_np(buf["topk_w"]), w, rtol=0, atol=1e-6)
    seg, rt, pos, total = _check_maps_exact(buf, idx, cfg)
    rng = np.random.default_rng(4)
    rows = _sample_rows(seg, rng, per_group=3, groups=40)
    R = torch.from_numpy(rows).to(DEV)
    ok = rt[rows] >= 0
    got_x = bits_host(buf["x_perm"][R])
    assert np.array_equal(got_x[ok], x[rt[rows][ok]]) and not got_x[~ok].any()
    h_ref, a_ref, y_ref = _oracle_rows(rows, seg, rt, x, cfg, lambda g: w1[g], lambda g: w2[g])
    assert_bf16_close(vals_host(buf["h_save"][R]), O.round_bf16(h_ref), "h_save rows")
    assert_bf16_close(vals_host(buf["a"][R]), a_ref, "a rows")
    assert_bf16_close(vals_host(buf["y_perm"][R]), y_ref, "y_perm rows")
    toks = np.concatenate([[0, cfg.T - 1], rng.choice(cfg.T, 14, replace=False)])
    y_tok = np.zeros((len(toks), cfg.H))
    for i, t in enumerate(toks):
        xt = O.bf16_to_f64(x[t:t + 1])
        for j in range(cfg.K):
            e = idx[t, j]
            y_tok[i] += np.float64(w[t, j]) * O.round_bf16(
                O.expert_ffn_rows(xt, O.bf16_to_f64(w1[e]), O.bf16_to_f64(w2[e]), cfg.I)[2][0])
        for sh in range(cfg.S):
            g = cfg.E + sh
            y_tok[i] += O.round_bf16(
                O.expert_ffn_rows(xt, O.bf16_to_f64(w1[g]), O.bf16_to_f64(w2[g]), cfg.I)[2][0])
    assert_bf16_close(vals_host(buf["y"][torch.from_numpy(toks).to(DEV)]), O.round_bf16(y_tok),
                      "y tokens")
