"""C ABI checks that need no GPU: the library loads, exports every function include/moe.h declares,
and rejects bad arguments on the host before any HIP call."""
import ctypes
import os

import pytest

import grouped_gemm_fp32_amd as M
from oracle import moe_oracle as O


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(M.library_path()):
        from grouped_gemm_fp32_amd import build
        build.build()
    return M.load_library()


def test_exports_every_declared_function(lib):
    names = M.declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), f"libmoe.so does not export {n}"


def test_version_and_status_strings(lib):
    assert M.moe_abi_version() >= 1
    assert M.moe_status_string(0) == "MOE_OK"
    assert M.moe_status_string(-1) == "MOE_ERR_INVALID_ARG"
    assert M.moe_status_string(-3) == "MOE_ERR_WORKSPACE"


@pytest.mark.parametrize("T,E,K,S,B", [(64, 8, 2, 1, 16), (8192, 128, 6, 0, 128),
                                       (16384, 128, 6, 2, 128), (256, 128, 6, 2, 16),
                                       (0, 8, 2, 1, 16), (1, 4, 4, 4, 256), (1000, 256, 8, 3, 64)])
def test_row_capacity_matches_oracle(lib, T, E, K, S, B):
    s = M.make_shape(T, 256, E, K, 128, S, B)
    assert M.moe_row_capacity(s) == O.row_capacity(T, E, K, S, B)


def _call(lib, fn, *args):
    return getattr(lib, fn)(*args)


def test_shape_validation(lib):
    bad = [
        (M.make_shape(8, 256, 8, 9, 128, 0, 16), -1),     # K > E
        (M.make_shape(8, 256, 8, 0, 128, 0, 16), -1),     # K < 1
        (M.make_shape(-1, 256, 8, 2, 128, 0, 16), -1),    # T < 0
        (M.make_shape(8, 256, 8, 2, 128, 0, 48), -2),     # block_m not supported
        (M.make_shape(8, 200, 8, 2, 128, 0, 16), -2),     # H % 128
        (M.make_shape(8, 256, 8, 2, 96, 0, 16), -2),      # I % 64
        (M.make_shape(8, 256, 300, 2, 128, 0, 16), -2),   # E > 256
        (M.make_shape(8, 256, 8, 2, 128, 0, 16, flags=0x80), -1),
    ]
    dummy = ctypes.c_void_p(16)
    for s, code in bad:
        st = lib.moe_route(ctypes.byref(s), None, dummy, None, None, dummy, None, dummy, dummy,
                           None, None)
        assert st == code, (s, st)
        assert M.moe_row_capacity(s) == -1
    assert lib.moe_row_capacity(None) == -1
    assert lib.moe_route(None, *([None] * 10)) == -1


def test_null_required_pointers(lib):
    s = M.make_shape(8, 256, 8, 2, 128, 1, 16)
    d = ctypes.c_void_p(16)
    # moe_route: topk outputs required; x given needs w_gate and logits; x NULL needs logits
    assert lib.moe_route(ctypes.byref(s), d, None, None, None, d, None, d, d, None, None) == -1
    assert lib.moe_route(ctypes.byref(s), d, d, None, None, None, None, d, d, None, None) == -1
    assert lib.moe_route(ctypes.byref(s), None, None, None, None, None, None, d, d, None, None) == -1
    assert lib.moe_route(ctypes.byref(s), None, None, None, None, d, None, None, d, None, None) == -1
    s_probs = M.make_shape(8, 256, 8, 2, 128, 1, 16, flags=M.MOE_PROBS_IN)
    assert lib.moe_route(ctypes.byref(s_probs), None, None, None, None, None, None, d, d, None,
                         None) == -1
    # moe_permute
    args = [d] * 8
    for i in range(7):
        a = list(args)
        a[i] = None if i != 1 else d  # x (index 1) is optional
        if i == 1:
            continue
        assert lib.moe_permute(ctypes.byref(s), *a, d, 1 << 20, None) == -1
    # grouped_gemm_fwd: h_save (index 6) is optional, the rest required for both stages
    for i in range(9):
        if i == 6:
            continue
        a = [d] * 9
        a[i] = None
        assert lib.grouped_gemm_fwd(ctypes.byref(s), M.MOE_FWD, *a, None) == -1
    assert lib.grouped_gemm_fwd(ctypes.byref(s), 0, *([d] * 9), None) == -1
    assert lib.grouped_gemm_fwd(ctypes.byref(s), 4, *([d] * 9), None) == -1
    # grouped_gemm_bwd: which must be DGRAD and/or WGRAD
    assert lib.grouped_gemm_bwd(ctypes.byref(s), 0, *([d] * 13), None) == -1
    assert lib.grouped_gemm_bwd(ctypes.byref(s), 16, *([d] * 13), None) == -1
    a = [d] * 13
    a[1] = None   # h_save needed by DGRAD
    assert lib.grouped_gemm_bwd(ctypes.byref(s), M.MOE_DGRAD, *a, None) == -1
    a = [d] * 13
    a[11] = None  # dw1 needed by WGRAD
    assert lib.grouped_gemm_bwd(ctypes.byref(s), M.MOE_WGRAD, *a, None) == -1
    for fn, n in (("moe_combine", 5), ("moe_unpermute_bwd", 4), ("moe_combine_bwd", 9)):
        for i in range(n):
            a = [d] * n
            a[i] = None
            assert _call(lib, fn, ctypes.byref(s), *a, None) == -1, (fn, i)
    assert "NULL" in M.moe_last_error()


def test_router_backward_and_bias_update_checks(lib):
    s = M.make_shape(8, 256, 8, 2, 128, 1, 16)
    d = ctypes.c_void_p(16)
    # required: dtopk_w, topk_idx, probs, dlogits; dw_gate needs x, dx_router needs w_gate
    for i in range(4):
        a = [d, d, d, None, None, d, None, None]
        a[[0, 1, 2, 5][i]] = None
        assert lib.moe_route_bwd(ctypes.byref(s), *a, None) == -1, i
    assert lib.moe_route_bwd(ctypes.byref(s), d, d, d, None, d, d, d, None, None) == -1  # dw_gate, no x
    assert lib.moe_route_bwd(ctypes.byref(s), d, d, d, d, None, d, None, d, None) == -1  # dx, no w_gate
    s0 = M.make_shape(0, 256, 8, 2, 128, 1, 16)
    assert lib.moe_route_bwd(ctypes.byref(s0), *([None] * 8), None) == 0
    assert lib.moe_bias_update(ctypes.byref(s), None, 0.001, d, None) == -1
    assert lib.moe_bias_update(ctypes.byref(s), d, 0.001, None, None) == -1
    for bad in (-1.0, float("nan"), float("inf")):
        assert lib.moe_bias_update(ctypes.byref(s), d, bad, d, None) == -1
        assert "gamma" in M.moe_last_error()


def test_balance_loss_and_router_grads_checks(lib):
    s = M.make_shape(8, 256, 8, 2, 128, 1, 16)
    d = ctypes.c_void_p(16)
    f = ctypes.c_float
    need = M.moe_balance_workspace_size(s, 4)
    assert need == 4 * 2 * (1 + 8)                        # two sequences of one chunk each
    assert M.moe_balance_workspace_size(s, 3) == 0        # 3 does not divide 8
    ok = (d, d, d, d, d, need)

    def call(shape, seq_len, alpha, *args):
        return lib.moe_balance_loss(ctypes.byref(shape), seq_len, f(alpha), *args, None)

    assert call(s, 3, 0.1, *ok) == -1
    assert call(s, 0, 0.1, *ok) == -1
    assert call(s, 4, -1.0, *ok) == -1
    assert call(s, 4, float("nan"), *ok) == -1
    assert call(s, 4, 0.1, d, d, None, None, d, need) == -1      # nothing to compute
    assert call(s, 4, 0.1, None, d, d, None, d, need) == -1      # probs
    assert call(s, 4, 0.1, d, None, None, d, d, need) == -1      # topk_idx
    assert call(s, 4, 0.1, d, d, d, None, None, need) == -1      # ws
    assert call(s, 4, 0.1, d, d, d, None, d, need - 1) == -3     # ws too small
    s0 = M.make_shape(0, 256, 8, 2, 128, 1, 16)
    assert call(s0, 4, 0.1, None, None, d, None, None, 0) == 0
    assert lib.moe_router_grads(ctypes.byref(s), None, d, d, d, d, None) == -1
    assert lib.moe_router_grads(ctypes.byref(s), d, None, d, d, None, None) == -1
    assert lib.moe_router_grads(ctypes.byref(s), d, d, None, None, d, None) == -1
    assert lib.moe_router_grads(ctypes.byref(s), d, ctypes.c_void_p(18), d, d, None, None) == -1


def test_fp32_wgrad_checks(lib):
    s = M.make_shape(8, 256, 8, 2, 128, 1, 16)
    d, odd = ctypes.c_void_p(16), ctypes.c_void_p(24)
    assert lib.grouped_gemm_wgrad_f32(ctypes.byref(s), M.MOE_DGRAD_DOWN, *([d] * 7), None) == -1
    assert lib.grouped_gemm_wgrad_f32(ctypes.byref(s), 0, *([d] * 7), None) == -1
    for i in range(7):   # x_perm, a, dy_perm, dh, seg_offsets, dw1, dw2 all needed for both kinds
        a = [d] * 7
        a[i] = None
        assert lib.grouped_gemm_wgrad_f32(ctypes.byref(s), M.MOE_WGRAD, *a, None) == -1, i
    for i in (0, 1, 2, 3, 5, 6):
        a = [d] * 7
        a[i] = odd
        assert lib.grouped_gemm_wgrad_f32(ctypes.byref(s), M.MOE_WGRAD, *a, None) == -1, i
        assert "aligned" in M.moe_last_error()


def test_gemm_tensors_must_be_16_byte_aligned(lib):
    s = M.make_shape(8, 256, 8, 2, 128, 1, 16)
    d, odd = ctypes.c_void_p(16), ctypes.c_void_p(16 + 8)
    for i in (0, 4, 5, 7, 8):   # x_perm, w1, w2, a, y_perm
        a = [d] * 9
        a[i] = odd
        assert lib.grouped_gemm_fwd(ctypes.byref(s), M.MOE_FWD, *a, None) == -1
        assert "aligned" in M.moe_last_error()
    for i in (0, 1, 2, 3, 9, 10, 11, 12):   # x_perm, h_save, a, dy_perm, dh, dx_perm, dw1, dw2
        a = [d] * 13
        a[i] = odd
        assert lib.grouped_gemm_bwd(ctypes.byref(s), M.MOE_DGRAD | M.MOE_WGRAD, *a, None) == -1
        assert "aligned" in M.moe_last_error()
    for i in (0, 1):   # moe_route from x: x, w_gate (read with 16-byte vector loads)
        a = [d, d, None, None, d, None, d, d, None]
        a[i] = odd
        assert lib.moe_route(ctypes.byref(s), *a, None) == -1
        assert "aligned" in M.moe_last_error()
    # the row movers: gather (x, x_perm), combine (y_perm, y), combine backward (dy, y_perm,
    # dy_perm) and the backward unpermute (dx_perm, dx)
    for i in (1, 7):
        a = [d] * 8
        a[i] = odd
        assert lib.moe_permute(ctypes.byref(s), *a, d, 1 << 20, None) == -1
        assert "aligned" in M.moe_last_error()
    for fn, n, idx in (("moe_combine", 5, (0, 4)), ("moe_combine_bwd", 9, (0, 1, 7)),
                       ("moe_unpermute_bwd", 4, (0, 3))):
        for i in idx:
            a = [d] * n
            a[i] = odd
            assert _call(lib, fn, ctypes.byref(s), *a, None) == -1, (fn, i)
            assert "aligned" in M.moe_last_error()


def test_workspace_too_small(lib):
    s = M.make_shape(1000, 256, 8, 2, 128, 1, 16)
    need = M.moe_workspace_size(s)
    assert need == 4 * 4 * 8  # 4 token blocks of 256, 8 experts
    d = ctypes.c_void_p(16)
    assert lib.moe_permute(ctypes.byref(s), d, d, d, d, d, d, d, d, d, need - 1, None) == -3


def test_empty_batch_is_a_noop_on_the_host(lib):
    s = M.make_shape(0, 256, 8, 2, 128, 1, 16)
    d = ctypes.c_void_p(16)
    assert lib.moe_route(ctypes.byref(s), d, d, None, None, None, None, d, d, None, None) == 0
    assert lib.grouped_gemm_fwd(ctypes.byref(s), M.MOE_FWD, *([d] * 9), None) == 0
    assert lib.moe_combine(ctypes.byref(s), *([d] * 5), None) == 0
    assert lib.moe_unpermute_bwd(ctypes.byref(s), *([d] * 4), None) == 0
    assert lib.grouped_gemm_bwd(ctypes.byref(s), M.MOE_DGRAD, *([d] * 13), None) == 0


def test_binding_refuses_host_tensors(lib):
    import torch
    s = M.make_shape(4, 256, 8, 2, 128, 0, 16)
    t = torch.zeros(4, 2, dtype=torch.int32)
    with pytest.raises(ValueError):
        M.moe_route(s, None, None, None, None, torch.zeros(4, 8), None, t, torch.zeros(4, 2), None,
                    stream=0)


def test_binding_checks_tensor_sizes_against_the_shape(lib):
    """A tensor shorter than its layout needs is refused before any pointer reaches the library
    (the C entry points see bare pointers and could not tell)."""
    import torch
    s = M.make_shape(64, 256, 8, 2, 128, 1, 16)
    mcap = M.moe_row_capacity(s)
    T, H, E, K, I, G = 64, 256, 8, 2, 128, 9
    with pytest.raises(ValueError, match="topk_idx has 126 elements"):
        M.moe_route(s, None, None, None, None, torch.zeros(T, E), None,
                    torch.zeros(T * K - 2, dtype=torch.int32), torch.zeros(T, K), None, stream=0)
    with pytest.raises(ValueError, match="x_perm"):
        M.grouped_gemm_fwd(s, M.MOE_FWD, torch.zeros(mcap - 1, H), None, None, None, None, None,
                           None, None, None, stream=0)
    with pytest.raises(ValueError, match="w2"):
        M.grouped_gemm_fwd(s, M.MOE_FWD, None, None, None, None, None,
                           torch.zeros(G - 1, H, I), None, None, None, stream=0)
    with pytest.raises(ValueError, match="dw1"):
        M.grouped_gemm_wgrad_f32(s, M.MOE_WGRAD, None, None, None, None, None,
                                 torch.zeros(G, 2 * I, H - 1), None, stream=0)
    with pytest.raises(ValueError, match="seq_loss"):
        M.moe_balance_loss(s, 16, 0.1, None, None, torch.zeros(3), None, None, stream=0)
    with pytest.raises(ValueError, match="sel_bias"):
        M.moe_bias_update(s, None, 0.1, torch.zeros(E - 1), stream=0)
    # full-size host tensors pass the size check and are then refused as host memory
    with pytest.raises(ValueError, match="device tensor"):
        M.moe_bias_update(s, torch.zeros(E, dtype=torch.int32), 0.1, torch.zeros(E), stream=0)


def test_gather_forward_checks(lib):
    """grouped_gemm_fwd_gather: x and row_token replace x_perm for the gate/up product, and an
    optional x_perm output receives the permuted rows."""
    s = M.make_shape(8, 256, 8, 2, 128, 1, 16)
    d, odd = ctypes.c_void_p(16), ctypes.c_void_p(24)
    full = [d] * 10   # x, row_token, seg_offsets, tile_group, total_rows, w1, w2, h_save, a, y_perm

    def call(shape, which, args, x_perm=None):
        return lib.grouped_gemm_fwd_gather(ctypes.byref(shape), which, *args, x_perm, None)

    assert call(s, 0, full) == -1
    assert call(s, 4, full) == -1
    for i in range(10):
        if i == 7:        # h_save is optional
            continue
        a = list(full)
        a[i] = None
        assert call(s, M.MOE_FWD, a) == -1, i
        assert "NULL" in M.moe_last_error()
    for i in (0, 5, 6, 7, 8, 9):   # bf16 tensors: x, w1, w2, h_save, a, y_perm
        a = list(full)
        a[i] = odd
        assert call(s, M.MOE_FWD, a) == -1, i
        assert "aligned" in M.moe_last_error()
    # the optional x_perm output: 16-byte aligned and apart from x ([T,H] against [Mcap,H])
    assert call(s, M.MOE_FWD, full, x_perm=odd) == -1
    assert "aligned" in M.moe_last_error()
    x0 = 1 << 24
    with_x = [ctypes.c_void_p(x0)] + full[1:]
    for xp in (x0, x0 + 8 * 256 * 2 - 16, x0 - M.moe_row_capacity(s) * 256 * 2 + 16):
        assert call(s, M.MOE_FWD, with_x, x_perm=ctypes.c_void_p(xp)) == -1, xp
        assert "overlaps" in M.moe_last_error()
    # the down product alone reads neither x nor row_token, and writes no x_perm
    a = list(full)
    a[0] = a[1] = None
    st = M.make_shape(0, 256, 8, 2, 128, 1, 16)
    assert call(st, M.MOE_FWD_DOWN, a, x_perm=odd) == 0
    # x addressed with 32-bit byte offsets: T*H*2 <= 2^31
    big = M.make_shape(262144, 8192, 8, 2, 128, 1, 128)
    assert call(big, M.MOE_FWD, full) == -2
    assert "2^31" in M.moe_last_error()
    empty = M.make_shape(0, 256, 8, 2, 128, 1, 16)
    assert call(empty, M.MOE_FWD, [None] * 10) == 0


def test_gemm_32bit_span_limits(lib):
    """The GEMM engines address operands with 32-bit byte offsets (and mark masked lanes 2^31 past
    a buffer's start): shapes whose spans do not fit are refused with MOE_ERR_UNSUPPORTED before
    any launch, one case per span."""
    d = ctypes.c_void_p(16)

    def fwd(s):
        return lib.grouped_gemm_fwd(ctypes.byref(s), M.MOE_FWD, *([d] * 9), None)

    def gather(s):
        return lib.grouped_gemm_fwd_gather(ctypes.byref(s), M.MOE_FWD, *([d] * 11), None)

    def bwd(s, which):
        return lib.grouped_gemm_bwd(ctypes.byref(s), which, *([d] * 13), None)

    def wgrad32(s):
        return lib.grouped_gemm_wgrad_f32(ctypes.byref(s), M.MOE_WGRAD, *([d] * 7), None)

    # an expert's W1 (2I x H bf16) reaches 4 GiB: I*H = 2^30
    s = M.make_shape(8, 32768, 8, 2, 32768, 0, 128)
    for st in (fwd(s), gather(s), bwd(s, M.MOE_DGRAD), bwd(s, M.MOE_WGRAD), wgrad32(s)):
        assert st == -2 and "4 GiB" in M.moe_last_error()
    # ... one step below fits (T = 0: accepted, nothing launched)
    ok = M.make_shape(0, 32768, 8, 2, 32704, 0, 128)
    assert fwd(ok) == 0 and bwd(ok, M.MOE_DGRAD) == 0
    # a 384-row tile of a max(H, 2I)-wide operand reaches 4 GiB (the weights alone would fit)
    s = M.make_shape(8, 5592448, 8, 2, 64, 0, 128)
    assert fwd(s) == -2 and "384-row tile" in M.moe_last_error()
    assert bwd(s, M.MOE_DGRAD) == -2
    # weight gradients: a segment of ceil(T/B)*B rows reaches 4 GiB (the forward is unaffected)
    s = M.make_shape(262144, 8192, 8, 2, 64, 1, 128)
    for st in (bwd(s, M.MOE_WGRAD_DOWN), bwd(s, M.MOE_WGRAD_GATEUP), wgrad32(s)):
        assert st == -2 and "segment" in M.moe_last_error()
    assert bwd(M.make_shape(0, 8192, 8, 2, 64, 1, 128), M.MOE_DGRAD) == 0
    # weight gradients: one expert's bf16 dW1 exceeds 2^31 bytes (the 2^31 past-end marker)
    s = M.make_shape(8, 32768, 8, 2, 16448, 0, 128)
    assert bwd(s, M.MOE_WGRAD) == -2 and "2^31" in M.moe_last_error()
    assert fwd(M.make_shape(0, 32768, 8, 2, 16448, 0, 128)) == 0
    # ... and the fp32 dW1 of a shape whose bf16 dW1 still fits
    s = M.make_shape(8, 16384, 8, 2, 16448, 0, 128)
    assert wgrad32(s) == -2 and "2^31" in M.moe_last_error()
    assert bwd(M.make_shape(0, 16384, 8, 2, 16448, 0, 128), M.MOE_DGRAD) == 0


def test_noalloc_permute_host_checks(lib):
    """moe_permute_noalloc validates like moe_permute (no workspace argument) before any HIP call."""
    s = M.make_shape(8, 256, 8, 2, 128, 1, 16)
    d, odd = ctypes.c_void_p(16), ctypes.c_void_p(24)
    full = [d] * 8   # topk_idx, x, seg_offsets, tile_group, total_rows, row_token, pos, x_perm
    for i in (0, 2, 3, 4, 5, 6):
        a = list(full)
        a[i] = None
        assert lib.moe_permute_noalloc(ctypes.byref(s), *a, None) == -1, i
        assert "NULL" in M.moe_last_error()
    for i in (1, 7):
        a = list(full)
        a[i] = odd
        assert lib.moe_permute_noalloc(ctypes.byref(s), *a, None) == -1, i
        assert "aligned" in M.moe_last_error()
    bad = M.make_shape(8, 256, 8, 9, 128, 1, 16)
    assert lib.moe_permute_noalloc(ctypes.byref(bad), *full, None) == -1
