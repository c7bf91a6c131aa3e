"""The path under HIP graph capture: one forward + backward step (router from x, permutation,
grouped GEMMs, combine, their backward and the router backward) captured with torch.cuda.CUDAGraph
and replayed several times, with eager work and synchronisation between the replays.

Every output is overwritten with a marker before each replay, so a replay that skipped a write
would show. The kernels are deterministic (fixed summation orders, integer-only atomics), so each
replay must reproduce the eager step bit for bit; the eager step itself is pinned to the oracle by
the parity tests. The library records only kernel launches: no memset, copy or allocation.
"""
import pytest
import torch

import grouped_gemm_fp32_amd as M
from synth import get_config, draw_x, draw_wg, draw_sel_bias, draw_w1_all, draw_w2_all, draw_dy
from tests.gpu_helpers import DEV, log, bf16_dev, f32_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    M.load_library()  # raises when the HIP library is missing: no fallback exists


# (name, rows to compare: None = all, "total" = the first total_rows rows)
OUTS = [("logits", None), ("probs", None), ("topk_idx", None), ("topk_w", None),
        ("expert_counts", None), ("seg_offsets", None), ("total_rows", None), ("pos", None),
        ("row_token", "total"), ("x_perm", "total"), ("h_save", "total"), ("a", "total"),
        ("y_perm", "total"), ("y", None), ("dy_perm", "total"), ("dtopk_w", None),
        ("dh", "total"), ("dx_perm", "total"), ("dw1", None), ("dw2", None), ("dx", None),
        ("dlogits", None), ("dwg", None), ("dx_router", None)]


def _bits(t):
    return t.view(torch.int32) if t.element_size() == 4 else t.view(torch.int16)


@pytest.mark.parametrize("B", [16, 128])
def test_step_replays_in_a_graph(B):
    T, H, E, K, I, S = 333, 256, 8, 3, 192, 1
    log(f"graph capture T={T} H={H} E={E} K={K} I={I} S={S} B={B}")
    cfg = get_config("c1", T=T, H=H, E=E, K=K, I=I, S=S, block_m=B, seed=3)
    s = M.make_shape(T, H, E, K, I, S, B)
    X, WG, SB = bf16_dev(draw_x(cfg)), f32_dev(draw_wg(cfg)), f32_dev(draw_sel_bias(cfg))
    W1, W2, DY = bf16_dev(draw_w1_all(cfg)), bf16_dev(draw_w2_all(cfg)), bf16_dev(draw_dy(cfg))
    b = M.alloc_buffers(s, DEV, backward=True)
    b["dlogits"] = torch.empty(T, E, device=DEV)
    b["dwg"] = torch.empty(E, H, device=DEV)
    b["dx_router"] = torch.empty(T, H, device=DEV)

    def step():
        M.moe_route(s, X, WG, None, SB, b["logits"], b["probs"], b["topk_idx"], b["topk_w"],
                    b["expert_counts"])
        M.moe_permute(s, b["topk_idx"], X, b["seg_offsets"], b["tile_group"], b["total_rows"],
                      b["row_token"], b["pos"], b["x_perm"], b["ws"])
        M.grouped_gemm_fwd(s, M.MOE_FWD, b["x_perm"], b["seg_offsets"], b["tile_group"],
                           b["total_rows"], W1, W2, b["h_save"], b["a"], b["y_perm"])
        M.moe_combine(s, b["y_perm"], b["pos"], b["topk_w"], b["seg_offsets"], b["y"])
        M.moe_combine_bwd(s, DY, b["y_perm"], b["pos"], b["topk_w"], b["seg_offsets"],
                          b["row_token"], b["total_rows"], b["dy_perm"], b["dtopk_w"])
        M.grouped_gemm_bwd(s, M.MOE_DGRAD | M.MOE_WGRAD, b["x_perm"], b["h_save"], b["a"],
                           b["dy_perm"], b["seg_offsets"], b["tile_group"], b["total_rows"], W1,
                           W2, b["dh"], b["dx_perm"], b["dw1"], b["dw2"])
        M.moe_unpermute_bwd(s, b["dx_perm"], b["pos"], b["seg_offsets"], b["dx"])
        M.moe_route_bwd(s, b["dtopk_w"], b["topk_idx"], b["probs"], X, WG, b["dlogits"], b["dwg"],
                        b["dx_router"])

    def poison():
        for name, _ in OUTS:
            _bits(b[name]).fill_(-7)

    def snapshot():
        total = int(b["total_rows"][0])
        return total, {n: _bits(b[n][:total] if r == "total" else b[n]).clone() for n, r in OUTS}

    poison()
    step()
    torch.cuda.synchronize()
    total, ref = snapshot()
    log(f"  eager step: total_rows {total}")

    # capture (torch warms the capture stream up itself; buffers are all allocated already)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    filler = torch.randn(512, 512, device=DEV)
    for rep in range(3):
        poison()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        t_rep, got = snapshot()
        assert t_rep == total, (rep, t_rep, total)
        for name, _ in OUTS:
            assert torch.equal(got[name], ref[name]), (rep, name)
        filler = filler @ filler.T / 512.0   # unrelated eager work between the replays
        torch.cuda.synchronize()
    log("  three replays reproduce the eager step bit for bit")
