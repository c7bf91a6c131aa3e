"""moe_permute_noalloc (the permutation with its scratch in the library's fixed device array)
against moe_permute with a caller workspace, through the C ABI: bit for bit on every output, on
calls in a row with the second smaller than the first, with and without the row copy."""
import numpy as np
import pytest
import torch

import grouped_gemm_fp32_amd as M
from oracle import moe_oracle as O
from synth import get_config, draw_x, draw_topk_given
from tests.gpu_helpers import DEV, log, bf16_dev, i32_dev, bits_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    M.load_library()


def _np(t):
    return t.detach().cpu().numpy()


def _run(fn, s, idx, x):
    buf = M.alloc_buffers(s, DEV)
    for k in ("seg_offsets", "tile_group", "row_token", "pos", "total_rows"):
        buf[k].fill_(-7)
    X = None if x is None else bf16_dev(x)
    XP = None if x is None else buf["x_perm"]
    if fn == "ws":
        M.moe_permute(s, i32_dev(idx), X, buf["seg_offsets"], buf["tile_group"], buf["total_rows"],
                      buf["row_token"], buf["pos"], XP, buf["ws"])
    else:
        M.moe_permute_noalloc(s, i32_dev(idx), X, buf["seg_offsets"], buf["tile_group"],
                              buf["total_rows"], buf["row_token"], buf["pos"], XP)
    torch.cuda.synchronize()
    return buf


def _same(a, b, with_rows):
    total = int(_np(a["total_rows"])[0])
    assert total == int(_np(b["total_rows"])[0])
    for k in ("seg_offsets", "tile_group", "pos"):
        np.testing.assert_array_equal(_np(a[k]), _np(b[k]), err_msg=k)
    np.testing.assert_array_equal(_np(a["row_token"])[:total], _np(b["row_token"])[:total])
    if with_rows:
        np.testing.assert_array_equal(bits_host(a["x_perm"][:total]), bits_host(b["x_perm"][:total]))
    return total


# (T, H, E, K, S, B, forced-empty experts): the largest case first, then smaller ones, so each
# later call finds the previous call's histograms in the shared array
CASES = [(70000, 128, 256, 8, 4, 16, ()), (4099, 128, 64, 8, 1, 64, tuple(range(0, 64, 5))),
         (333, 256, 16, 4, 2, 32, (3, 9)), (5, 128, 4, 4, 0, 16, ())]


def test_noalloc_permute_matches_workspace_permute_on_calls_in_a_row():
    for T, H, E, K, S, B, empty in CASES:
        log(f"noalloc permute T={T} H={H} E={E} K={K} S={S} B={B}")
        s = M.make_shape(T, H, E, K, 128, S, B)
        idx = draw_topk_given(T, E, K, seed=T + 1, forced_empty=empty)
        x = draw_x(get_config("c1", T=T, H=H, E=E, K=K, S=S, block_m=B, seed=2))
        for with_rows in (True, False):
            ref = _run("ws", s, idx, x if with_rows else None)
            got = _run("noalloc", s, idx, x if with_rows else None)
            total = _same(got, ref, with_rows)
            # and the maps are the oracle's
            seg, tg, tot = O.build_segments(O.expert_counts(idx, E), T, E, S, B, got["mcap"])
            assert tot == total
            np.testing.assert_array_equal(_np(got["seg_offsets"]), seg)
            rt, pos = O.permute_maps(idx, seg, T, E, S, got["mcap"])
            np.testing.assert_array_equal(_np(got["row_token"])[:total], rt[:total])
            np.testing.assert_array_equal(_np(got["pos"]), pos)


def test_noalloc_permute_empty_batch():
    s = M.make_shape(0, 256, 8, 2, 128, 1, 16)
    buf = M.alloc_buffers(s, DEV)
    buf["seg_offsets"].fill_(5)
    buf["total_rows"].fill_(5)
    M.moe_permute_noalloc(s, None, None, buf["seg_offsets"], None, buf["total_rows"], None, None,
                          None)
    torch.cuda.synchronize()
    assert np.all(_np(buf["seg_offsets"]) == 0) and int(_np(buf["total_rows"])[0]) == 0
