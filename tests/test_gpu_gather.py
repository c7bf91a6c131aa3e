"""GPU parity of grouped_gemm_fwd_gather: the forward grouped GEMM with the gate/up product reading
its rows straight from x through the permutation map (moe_permute called with x == NULL), through
the C ABI, with and without its optional x_perm output.

Each case is checked three ways:
  * against the oracle's forward, with the bars every bf16 GEMM output has (rel-L2 <= 2e-2 over the
    tensor and on every row; padding rows exactly zero);
  * bit for bit against grouped_gemm_fwd on the x_perm that moe_permute writes from the same x:
    both read the same operand values in the same order and do the same arithmetic;
  * the x_perm output bit for bit against moe_permute's on rows < total_rows (a pure copy), the rows
    past total_rows left as they were. It is written from the gate/up product's own staged rows on
    tall tiles with at least twice as many 128-column tiles as 128-row blocks per tile, else by a
    separate row copy: the cases cover both.
Inputs are the seeded synthetic generators' and the oracle's; nothing expected comes from the GPU.
"""
import numpy as np
import pytest
import torch

import grouped_gemm_fp32_amd as M
from synth import get_config, draw_x, draw_w1_all, draw_w2_all, draw_topk_given
from tests.gpu_helpers import DEV, log, bf16_dev, i32_dev, vals_host, assert_bf16_close
from tests.test_gpu_parity import _layer_inputs, _oracle_layer, _shape

pytestmark = pytest.mark.gpu
OUTS = ("h_save", "a", "y_perm")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    M.load_library()  # raises when the HIP library is missing: no fallback exists


def _both_paths(s, idx, X, W1, W2, xperm=True):
    """(materialised buffers, gathered buffers) of one forward on the same inputs; with xperm the
    gathered forward also writes its x_perm output (pre-filled with all-ones bytes)."""
    IDX = i32_dev(idx)
    ref = M.alloc_buffers(s, DEV)
    M.moe_permute(s, IDX, X, ref["seg_offsets"], ref["tile_group"], ref["total_rows"],
                  ref["row_token"], ref["pos"], ref["x_perm"], ref["ws"])
    M.grouped_gemm_fwd(s, M.MOE_FWD, ref["x_perm"], ref["seg_offsets"], ref["tile_group"],
                       ref["total_rows"], W1, W2, ref["h_save"], ref["a"], ref["y_perm"])
    got = M.alloc_buffers(s, DEV)
    if xperm:
        got["x_perm"].view(torch.int16).fill_(-1)
    else:
        del got["x_perm"]   # no permuted copy of x at all
    M.moe_permute(s, IDX, None, got["seg_offsets"], got["tile_group"], got["total_rows"],
                  got["row_token"], got["pos"], None, got["ws"])
    M.grouped_gemm_fwd_gather(s, M.MOE_FWD, X, got["row_token"], got["seg_offsets"],
                              got["tile_group"], got["total_rows"], W1, W2, got["h_save"],
                              got["a"], got["y_perm"], x_perm=got.get("x_perm"))
    torch.cuda.synchronize()
    return ref, got


def _bitexact(ref, got):
    total = int(ref["total_rows"][0])
    assert int(got["total_rows"][0]) == total
    for name in OUTS + (("x_perm",) if "x_perm" in got else ()):
        a = ref[name][:total].view(torch.int16)
        b = got[name][:total].view(torch.int16)
        assert torch.equal(a, b), (name, int((a != b).sum()))
    if "x_perm" in got:
        rest = got["x_perm"][total:].view(torch.int16)
        assert bool((rest == -1).all()), "x_perm rows past total_rows were written"
    return total


@pytest.mark.parametrize("T,H,E,K,I,S,B,empty", [
    (64, 256, 8, 2, 128, 1, 16, ()),            # register-staged engine (block 16)
    (333, 256, 8, 3, 192, 2, 32, (5,)),         # block 32, ragged N tails, an empty expert
    (500, 512, 16, 4, 256, 1, 64, (0, 15)),     # 64-row DMA engine
    (700, 384, 12, 6, 320, 2, 128, (4,)),       # eight-wave engine, tiles of 128-384 rows
    (300, 256, 6, 2, 128, 0, 256, ()),
    (1000, 512, 1, 1, 1024, 0, 128, ()),        # a dense FFN as one group; x_perm from the stages
    (600, 256, 8, 2, 832, 0, 128, (3,)),        # x_perm from the stages, ragged last column tile
])
@pytest.mark.parametrize("xperm", [True, False])
def test_gather_forward_parity(T, H, E, K, I, S, B, empty, xperm):
    log(f"gather fwd T={T} H={H} E={E} K={K} I={I} S={S} B={B} empty={empty} xperm={xperm}")
    cfg, idx, w, x, w1, w2, dy = _layer_inputs(T, H, E, K, I, S, B, seed=T + B + 1, empty=empty)
    s = _shape(T, H, E, K, I, S, B)
    ref, got = _both_paths(s, idx, bf16_dev(x), bf16_dev(w1), bf16_dev(w2), xperm=xperm)
    total = _bitexact(ref, got)
    f, _ = _oracle_layer(cfg, idx, w, x, w1, w2, dy, backward=False)
    assert total == f["total_rows"]
    pad = f["row_token"][:total] < 0
    for name, r in (("h_save", f["h"]), ("a", f["a"]), ("y_perm", f["y_perm"])):
        g = vals_host(got[name][:total])
        assert np.all(g[pad] == 0), f"{name}: padding rows not zero"
        assert_bf16_close(g, r, name)


@pytest.mark.parametrize("name", ["c2", "c3", "c5"])
def test_gather_forward_full_size(name):
    """The 16384-token training layer and the skewed layer (block 128; x_perm from the staged
    rows) and the 256-token decode (block 16; x_perm by the row copy): bit for bit against the
    materialised path, which the full-size tests pin to the oracle."""
    cfg = get_config(name)
    log(f"gather fwd full size {cfg}")
    idx = draw_topk_given(cfg.T, cfg.E, cfg.K, seed=cfg.seed + 11)
    s = _shape(cfg.T, cfg.H, cfg.E, cfg.K, cfg.I, cfg.S, cfg.block_m)
    ref, got = _both_paths(s, idx, bf16_dev(draw_x(cfg)), bf16_dev(draw_w1_all(cfg)),
                           bf16_dev(draw_w2_all(cfg)))
    _bitexact(ref, got)


@pytest.mark.parametrize("I", [1024, 768])
def test_gather_forward_tile_heights(I):
    """12 blocks of 128 rows per expert: the tall tiles come out 384 rows high. Over eight
    128-column tiles the x_perm copy shares out 48 rows per workgroup and stage; over six, 64 (all
    512 lanes of each workgroup, the most it takes). Bit for bit against the materialised path."""
    T, H, E, K, S, B = 6144, 256, 8, 2, 0, 128
    cfg = get_config("c1", T=T, H=H, E=E, K=K, I=I, S=S, block_m=B, seed=9)
    idx = np.stack([(np.arange(T) + j) % E for j in range(K)], axis=1).astype(np.int32)
    log(f"gather fwd tile heights T={T} E={E} I={I}")
    ref, got = _both_paths(_shape(T, H, E, K, I, S, B), idx, bf16_dev(draw_x(cfg)),
                           bf16_dev(draw_w1_all(cfg)), bf16_dev(draw_w2_all(cfg)))
    assert int(ref["total_rows"][0]) == T * K
    _bitexact(ref, got)


def test_gather_forward_large_row_offsets():
    """65536 tokens of 4096 features: x is 512 MiB, so the gathered rows' byte offsets reach 2^29
    (the 32-bit offsets and the past-the-end marker at 2^31 stay apart)."""
    T, H, E, K, I, S, B = 65536, 4096, 8, 1, 64, 0, 128
    cfg = get_config("c1", T=T, H=H, E=E, K=K, I=I, S=S, block_m=B, seed=5)
    idx = draw_topk_given(T, E, K, seed=5)
    log(f"gather fwd T={T} H={H}")
    ref, got = _both_paths(_shape(T, H, E, K, I, S, B), idx, bf16_dev(draw_x(cfg)),
                           bf16_dev(draw_w1_all(cfg)), bf16_dev(draw_w2_all(cfg)))
    _bitexact(ref, got)
