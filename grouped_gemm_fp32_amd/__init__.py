"""Python binding of libmoe.so, the gfx950 MoE feed-forward path of dots.llm1 (include/moe.h).

Argument marshalling only: every function here passes device pointers of torch tensors (PyTorch
provides device memory and streams) to the C entry point of the same name, which does all the work
in HIP kernels. Nothing falls back to a CPU path: if the library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import re

__all__ = [
    "MoeShape", "MoeError", "load_library", "library_path", "declared_functions",
    "MOE_NORM_TOPK", "MOE_PROBS_IN", "MOE_FWD_GATEUP", "MOE_FWD_DOWN", "MOE_FWD",
    "MOE_DGRAD_DOWN", "MOE_DGRAD_GATEUP", "MOE_WGRAD_DOWN", "MOE_WGRAD_GATEUP", "MOE_DGRAD",
    "MOE_WGRAD",
    "moe_abi_version", "moe_status_string", "moe_last_error", "moe_row_capacity",
    "moe_workspace_size", "moe_route", "moe_permute", "grouped_gemm_fwd",
    "grouped_gemm_fwd_gather", "grouped_gemm_bwd",
    "grouped_gemm_wgrad_f32", "moe_combine", "moe_combine_bwd", "moe_unpermute_bwd",
    "moe_route_bwd", "moe_router_grads", "moe_balance_loss",
    "moe_balance_workspace_size", "moe_bias_update",
    "make_shape", "alloc_buffers",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_HEADER = os.path.join(os.path.dirname(_PKG), "include", "moe.h")

MOE_NORM_TOPK = 0x1
MOE_PROBS_IN = 0x2
MOE_FWD_GATEUP, MOE_FWD_DOWN = 0x1, 0x2
MOE_FWD = MOE_FWD_GATEUP | MOE_FWD_DOWN
MOE_DGRAD_DOWN, MOE_DGRAD_GATEUP, MOE_WGRAD_DOWN, MOE_WGRAD_GATEUP = 0x1, 0x2, 0x4, 0x8
MOE_DGRAD = MOE_DGRAD_DOWN | MOE_DGRAD_GATEUP
MOE_WGRAD = MOE_WGRAD_DOWN | MOE_WGRAD_GATEUP


class MoeShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
                ("K", ctypes.c_int32), ("I", ctypes.c_int32), ("S", ctypes.c_int32),
                ("block_m", ctypes.c_int32), ("flags", ctypes.c_uint32)]

    @property
    def G(self):
        return self.E + self.S

    def __repr__(self):
        return ("MoeShape(T=%d, H=%d, E=%d, K=%d, I=%d, S=%d, block_m=%d, flags=%#x)"
                % (self.T, self.H, self.E, self.K, self.I, self.S, self.block_m, self.flags))


def make_shape(T, H, E, K, I, S, block_m, flags=MOE_NORM_TOPK) -> MoeShape:
    return MoeShape(T, H, E, K, I, S, block_m, flags)


class MoeError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed: {status} ({msg})")
        self.status = status


def library_path() -> str:
    return os.environ.get("MOE_LIB", os.path.join(_PKG, "libmoe.so"))


_lib = None
_P = ctypes.c_void_p
_SP = ctypes.POINTER(MoeShape)
_SIGS = {
    "moe_abi_version": (ctypes.c_int32, []),
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int32]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_row_capacity": (ctypes.c_int64, [_SP]),
    "moe_workspace_size": (ctypes.c_size_t, [_SP]),
    "moe_route": (ctypes.c_int, [_SP] + [_P] * 10),
    "moe_permute": (ctypes.c_int, [_SP] + [_P] * 9 + [ctypes.c_size_t, _P]),
    "moe_permute_noalloc": (ctypes.c_int, [_SP] + [_P] * 9),
    "grouped_gemm_fwd": (ctypes.c_int, [_SP, ctypes.c_uint32] + [_P] * 10),
    "grouped_gemm_fwd_gather": (ctypes.c_int, [_SP, ctypes.c_uint32] + [_P] * 12),
    "grouped_gemm_bwd": (ctypes.c_int, [_SP, ctypes.c_uint32] + [_P] * 14),
    "moe_combine": (ctypes.c_int, [_SP] + [_P] * 6),
    "moe_combine_bwd": (ctypes.c_int, [_SP] + [_P] * 10),
    "moe_unpermute_bwd": (ctypes.c_int, [_SP] + [_P] * 5),
    "moe_route_bwd": (ctypes.c_int, [_SP] + [_P] * 9),
    "grouped_gemm_wgrad_f32": (ctypes.c_int, [_SP, ctypes.c_uint32] + [_P] * 8),
    "moe_router_grads": (ctypes.c_int, [_SP] + [_P] * 6),
    "moe_balance_loss": (ctypes.c_int, [_SP, ctypes.c_int32, ctypes.c_float] + [_P] * 5
                         + [ctypes.c_size_t, _P]),
    "moe_balance_workspace_size": (ctypes.c_size_t, [_SP, ctypes.c_int32]),
    "moe_bias_update": (ctypes.c_int, [_SP, _P, ctypes.c_float, _P, _P]),
}


def load_library():
    """Load libmoe.so once. Raises if it is missing: there is no fallback implementation."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run `python -m grouped_gemm_fp32_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            f = getattr(lib, name)
            f.restype, f.argtypes = res, args
        _lib = lib
    return _lib


def declared_functions() -> list:
    """Function names declared in include/moe.h."""
    with open(_HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+|grouped_gemm_\w+)\s*\(", text)))


# ------------------------------------------------------------------------------------------------
# marshalling helpers
# ------------------------------------------------------------------------------------------------
def _ptr(t, name, dtype=None):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtype}")
    return t.data_ptr()


def _need(shape, **sizes):
    """Raise if a tensor argument holds fewer elements than its layout needs for this shape.

    The C entry points take bare pointers and cannot see sizes, so a short tensor would let a
    kernel read or write past it; this is checked here instead. Sizes are given as element counts
    per argument name; tensors passed as None or as raw integer addresses are not checked. An
    invalid shape is left to the C call to report."""
    if moe_row_capacity(shape) < 0:
        return
    for name, (t, n) in sizes.items():
        if t is None or isinstance(t, int):
            continue
        if t.numel() < n:
            raise ValueError(f"{name} has {t.numel()} elements; {shape!r} needs at least {n}")


def _dims(shape):
    """T, H, E, K, I, G and the row capacity of the permuted buffers."""
    return (shape.T, shape.H, shape.E, shape.K, shape.I, shape.E + shape.S,
            max(0, moe_row_capacity(shape)))


def _stream(stream, *tensors):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    dev = next((t.device for t in tensors if hasattr(t, "device")), None)
    return torch.cuda.current_stream(dev).cuda_stream


def _check(fn, status):
    if status != 0:
        lib = load_library()
        raise MoeError(fn, lib.moe_status_string(status).decode(), lib.moe_last_error().decode())


def _bf16():
    import torch
    return (torch.bfloat16, torch.int16, torch.uint16)


def _f32():
    import torch
    return (torch.float32,)


def _i32():
    import torch
    return (torch.int32,)


# ------------------------------------------------------------------------------------------------
# entry points (same names and argument order as include/moe.h)
# ------------------------------------------------------------------------------------------------
def moe_abi_version() -> int:
    return load_library().moe_abi_version()


def moe_status_string(status: int) -> str:
    return load_library().moe_status_string(status).decode()


def moe_last_error() -> str:
    return load_library().moe_last_error().decode()


def moe_row_capacity(shape: MoeShape) -> int:
    return int(load_library().moe_row_capacity(ctypes.byref(shape)))


def moe_workspace_size(shape: MoeShape) -> int:
    return int(load_library().moe_workspace_size(ctypes.byref(shape)))


def moe_route(shape, x, w_gate, logit_bias, sel_bias, logits, probs, topk_idx, topk_w,
              expert_counts, stream=None):
    lib = load_library()
    T, H, E, K, I, G, mcap = _dims(shape)
    _need(shape, x=(x, T * H), w_gate=(w_gate, E * H), logit_bias=(logit_bias, E),
          sel_bias=(sel_bias, E), logits=(logits, T * E), probs=(probs, T * E),
          topk_idx=(topk_idx, T * K), topk_w=(topk_w, T * K), expert_counts=(expert_counts, E))
    st = _stream(stream, topk_idx, expert_counts)
    _check("moe_route", lib.moe_route(
        ctypes.byref(shape), _ptr(x, "x", _bf16()), _ptr(w_gate, "w_gate", _f32()),
        _ptr(logit_bias, "logit_bias", _f32()), _ptr(sel_bias, "sel_bias", _f32()),
        _ptr(logits, "logits", _f32()), _ptr(probs, "probs", _f32()),
        _ptr(topk_idx, "topk_idx", _i32()), _ptr(topk_w, "topk_w", _f32()),
        _ptr(expert_counts, "expert_counts", _i32()), st))


def moe_permute(shape, topk_idx, x, seg_offsets, tile_group, total_rows, row_token, pos, x_perm,
                ws, stream=None):
    lib = load_library()
    T, H, E, K, I, G, mcap = _dims(shape)
    _need(shape, topk_idx=(topk_idx, T * K), x=(x, T * H), seg_offsets=(seg_offsets, G + 1),
          tile_group=(tile_group, mcap // shape.block_m), total_rows=(total_rows, 1),
          row_token=(row_token, mcap), pos=(pos, T * K), x_perm=(x_perm, mcap * H))
    st = _stream(stream, topk_idx)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("moe_permute", lib.moe_permute(
        ctypes.byref(shape), _ptr(topk_idx, "topk_idx", _i32()), _ptr(x, "x", _bf16()),
        _ptr(seg_offsets, "seg_offsets", _i32()), _ptr(tile_group, "tile_group", _i32()),
        _ptr(total_rows, "total_rows", _i32()), _ptr(row_token, "row_token", _i32()),
        _ptr(pos, "pos", _i32()), _ptr(x_perm, "x_perm", _bf16()), _ptr(ws, "ws"), ws_bytes, st))


def moe_permute_noalloc(shape, topk_idx, x, seg_offsets, tile_group, total_rows, row_token, pos,
                        x_perm, stream=None):
    lib = load_library()
    T, H, E, K, I, G, mcap = _dims(shape)
    _need(shape, topk_idx=(topk_idx, T * K), x=(x, T * H), seg_offsets=(seg_offsets, G + 1),
          tile_group=(tile_group, mcap // shape.block_m), total_rows=(total_rows, 1),
          row_token=(row_token, mcap), pos=(pos, T * K), x_perm=(x_perm, mcap * H))
    st = _stream(stream, topk_idx)
    _check("moe_permute_noalloc", lib.moe_permute_noalloc(
        ctypes.byref(shape), _ptr(topk_idx, "topk_idx", _i32()), _ptr(x, "x", _bf16()),
        _ptr(seg_offsets, "seg_offsets", _i32()), _ptr(tile_group, "tile_group", _i32()),
        _ptr(total_rows, "total_rows", _i32()), _ptr(row_token, "row_token", _i32()),
        _ptr(pos, "pos", _i32()), _ptr(x_perm, "x_perm", _bf16()), st))


def grouped_gemm_fwd(shape, which, x_perm, seg_offsets, tile_group, total_rows, w1, w2, h_save, a,
                     y_perm, stream=None):
    lib = load_library()
    T, H, E, K, I, G, mcap = _dims(shape)
    _need(shape, x_perm=(x_perm, mcap * H), seg_offsets=(seg_offsets, G + 1),
          tile_group=(tile_group, mcap // shape.block_m), total_rows=(total_rows, 1),
          w1=(w1, G * 2 * I * H), w2=(w2, G * H * I), h_save=(h_save, mcap * 2 * I),
          a=(a, mcap * I), y_perm=(y_perm, mcap * H))
    st = _stream(stream, a)
    _check("grouped_gemm_fwd", lib.grouped_gemm_fwd(
        ctypes.byref(shape), which, _ptr(x_perm, "x_perm", _bf16()),
        _ptr(seg_offsets, "seg_offsets", _i32()), _ptr(tile_group, "tile_group", _i32()),
        _ptr(total_rows, "total_rows", _i32()), _ptr(w1, "w1", _bf16()), _ptr(w2, "w2", _bf16()),
        _ptr(h_save, "h_save", _bf16()), _ptr(a, "a", _bf16()), _ptr(y_perm, "y_perm", _bf16()),
        st))


def grouped_gemm_fwd_gather(shape, which, x, row_token, seg_offsets, tile_group, total_rows, w1,
                            w2, h_save, a, y_perm, x_perm=None, stream=None):
    lib = load_library()
    T, H, E, K, I, G, mcap = _dims(shape)
    _need(shape, x=(x, T * H), row_token=(row_token, mcap), seg_offsets=(seg_offsets, G + 1),
          tile_group=(tile_group, mcap // shape.block_m), total_rows=(total_rows, 1),
          w1=(w1, G * 2 * I * H), w2=(w2, G * H * I), h_save=(h_save, mcap * 2 * I),
          a=(a, mcap * I), y_perm=(y_perm, mcap * H), x_perm=(x_perm, mcap * H))
    st = _stream(stream, a)
    _check("grouped_gemm_fwd_gather", lib.grouped_gemm_fwd_gather(
        ctypes.byref(shape), which, _ptr(x, "x", _bf16()), _ptr(row_token, "row_token", _i32()),
        _ptr(seg_offsets, "seg_offsets", _i32()), _ptr(tile_group, "tile_group", _i32()),
        _ptr(total_rows, "total_rows", _i32()), _ptr(w1, "w1", _bf16()), _ptr(w2, "w2", _bf16()),
        _ptr(h_save, "h_save", _bf16()), _ptr(a, "a", _bf16()), _ptr(y_perm, "y_perm", _bf16()),
        _ptr(x_perm, "x_perm", _bf16()), st))


def grouped_gemm_bwd(shape, which, x_perm, h_save, a, dy_perm, seg_offsets, tile_group, total_rows,
                     w1, w2, dh, dx_perm, dw1, dw2, stream=None):
    lib = load_library()
    T, H, E, K, I, G, mcap = _dims(shape)
    # The weight gradients follow a caller-supplied segment table, so their row operands are only
    # checked (against the capacity) when a data-gradient bit is also set.
    sizes = dict(w1=(w1, G * 2 * I * H), w2=(w2, G * H * I), dw1=(dw1, G * 2 * I * H),
                 dw2=(dw2, G * H * I), seg_offsets=(seg_offsets, G + 1))
    if int(which) & MOE_DGRAD:
        sizes.update(x_perm=(x_perm, mcap * H), h_save=(h_save, mcap * 2 * I), a=(a, mcap * I),
                     dy_perm=(dy_perm, mcap * H), tile_group=(tile_group, mcap // shape.block_m),
                     total_rows=(total_rows, 1), dh=(dh, mcap * 2 * I),
                     dx_perm=(dx_perm, mcap * H))
    _need(shape, **sizes)
    st = _stream(stream, dw1, dh)
    _check("grouped_gemm_bwd", lib.grouped_gemm_bwd(
        ctypes.byref(shape), which, _ptr(x_perm, "x_perm", _bf16()), _ptr(h_save, "h_save", _bf16()),
        _ptr(a, "a", _bf16()), _ptr(dy_perm, "dy_perm", _bf16()),
        _ptr(seg_offsets, "seg_offsets", _i32()), _ptr(tile_group, "tile_group", _i32()),
        _ptr(total_rows, "total_rows", _i32()), _ptr(w1, "w1", _bf16()), _ptr(w2, "w2", _bf16()),
        _ptr(dh, "dh", _bf16()), _ptr(dx_perm, "dx_perm", _bf16()), _ptr(dw1, "dw1", _bf16()),
        _ptr(dw2, "dw2", _bf16()), st))


def moe_combine(shape, y_perm, pos, topk_w, seg_offsets, y, stream=None):
    lib = load_library()
    T, H, E, K, I, G, mcap = _dims(shape)
    _need(shape, y_perm=(y_perm, mcap * H), pos=(pos, T * K), topk_w=(topk_w, T * K),
          seg_offsets=(seg_offsets, G + 1), y=(y, T * H))
    st = _stream(stream, y_perm)
    _check("moe_combine", lib.moe_combine(
        ctypes.byref(shape), _ptr(y_perm, "y_perm", _bf16()), _ptr(pos, "pos", _i32()),
        _ptr(topk_w, "topk_w", _f32()), _ptr(seg_offsets, "seg_offsets", _i32()),
        _ptr(y, "y", _bf16()), st))


def moe_combine_bwd(shape, dy, y_perm, pos, topk_w, seg_offsets, row_token, total_rows, dy_perm,
                    dtopk_w, stream=None):
    lib = load_library()
    T, H, E, K, I, G, mcap = _dims(shape)
    _need(shape, dy=(dy, T * H), y_perm=(y_perm, mcap * H), pos=(pos, T * K),
          topk_w=(topk_w, T * K), seg_offsets=(seg_offsets, G + 1), row_token=(row_token, mcap),
          total_rows=(total_rows, 1), dy_perm=(dy_perm, mcap * H), dtopk_w=(dtopk_w, T * K))
    st = _stream(stream, dy)
    _check("moe_combine_bwd", lib.moe_combine_bwd(
        ctypes.byref(shape), _ptr(dy, "dy", _bf16()), _ptr(y_perm, "y_perm", _bf16()),
        _ptr(pos, "pos", _i32()), _ptr(topk_w, "topk_w", _f32()),
        _ptr(seg_offsets, "seg_offsets", _i32()), _ptr(row_token, "row_token", _i32()),
        _ptr(total_rows, "total_rows", _i32()), _ptr(dy_perm, "dy_perm", _bf16()),
        _ptr(dtopk_w, "dtopk_w", _f32()), st))


def moe_unpermute_bwd(shape, dx_perm, pos, seg_offsets, dx, stream=None):
    lib = load_library()
    T, H, E, K, I, G, mcap = _dims(shape)
    _need(shape, dx_perm=(dx_perm, mcap * H), pos=(pos, T * K), seg_offsets=(seg_offsets, G + 1),
          dx=(dx, T * H))
    st = _stream(stream, dx_perm)
    _check("moe_unpermute_bwd", lib.moe_unpermute_bwd(
        ctypes.byref(shape), _ptr(dx_perm, "dx_perm", _bf16()), _ptr(pos, "pos", _i32()),
        _ptr(seg_offsets, "seg_offsets", _i32()), _ptr(dx, "dx", _bf16()), st))


def grouped_gemm_wgrad_f32(shape, which, x_perm, a, dy_perm, dh, seg_offsets, dw1, dw2,
                           stream=None):
    lib = load_library()
    T, H, E, K, I, G, mcap = _dims(shape)
    _need(shape, seg_offsets=(seg_offsets, G + 1), dw1=(dw1, G * 2 * I * H), dw2=(dw2, G * H * I))
    st = _stream(stream, dw1, dw2)
    _check("grouped_gemm_wgrad_f32", lib.grouped_gemm_wgrad_f32(
        ctypes.byref(shape), int(which), _ptr(x_perm, "x_perm", _bf16()), _ptr(a, "a", _bf16()),
        _ptr(dy_perm, "dy_perm", _bf16()), _ptr(dh, "dh", _bf16()),
        _ptr(seg_offsets, "seg_offsets", _i32()), _ptr(dw1, "dw1", _f32()),
        _ptr(dw2, "dw2", _f32()), st))


def moe_route_bwd(shape, dtopk_w, topk_idx, probs, x, w_gate, dlogits, dw_gate, dx_router,
                  stream=None):
    lib = load_library()
    T, H, E, K, I, G, mcap = _dims(shape)
    _need(shape, dtopk_w=(dtopk_w, T * K), topk_idx=(topk_idx, T * K), probs=(probs, T * E),
          x=(x, T * H), w_gate=(w_gate, E * H), dlogits=(dlogits, T * E), dw_gate=(dw_gate, E * H),
          dx_router=(dx_router, T * H))
    st = _stream(stream, dlogits, dw_gate)
    _check("moe_route_bwd", lib.moe_route_bwd(
        ctypes.byref(shape), _ptr(dtopk_w, "dtopk_w", _f32()), _ptr(topk_idx, "topk_idx", _i32()),
        _ptr(probs, "probs", _f32()), _ptr(x, "x", _bf16()), _ptr(w_gate, "w_gate", _f32()),
        _ptr(dlogits, "dlogits", _f32()), _ptr(dw_gate, "dw_gate", _f32()),
        _ptr(dx_router, "dx_router", _f32()), st))


def moe_router_grads(shape, dlogits, x, w_gate, dw_gate, dx_router, stream=None):
    lib = load_library()
    T, H, E, K, I, G, mcap = _dims(shape)
    _need(shape, dlogits=(dlogits, T * E), x=(x, T * H), w_gate=(w_gate, E * H),
          dw_gate=(dw_gate, E * H), dx_router=(dx_router, T * H))
    st = _stream(stream, dlogits, dw_gate, dx_router)
    _check("moe_router_grads", lib.moe_router_grads(
        ctypes.byref(shape), _ptr(dlogits, "dlogits", _f32()), _ptr(x, "x", _bf16()),
        _ptr(w_gate, "w_gate", _f32()), _ptr(dw_gate, "dw_gate", _f32()),
        _ptr(dx_router, "dx_router", _f32()), st))


def moe_balance_workspace_size(shape, seq_len) -> int:
    return int(load_library().moe_balance_workspace_size(ctypes.byref(shape), int(seq_len)))


def moe_balance_loss(shape, seq_len, alpha, probs, topk_idx, seq_loss, dlogits, ws, stream=None):
    lib = load_library()
    T, H, E, K, I, G, mcap = _dims(shape)
    n_seq = T // int(seq_len) if int(seq_len) > 0 else 0
    _need(shape, probs=(probs, T * E), topk_idx=(topk_idx, T * K), seq_loss=(seq_loss, n_seq),
          dlogits=(dlogits, T * E))
    st = _stream(stream, probs, seq_loss, dlogits)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("moe_balance_loss", lib.moe_balance_loss(
        ctypes.byref(shape), int(seq_len), float(alpha), _ptr(probs, "probs", _f32()),
        _ptr(topk_idx, "topk_idx", _i32()), _ptr(seq_loss, "seq_loss", _f32()),
        _ptr(dlogits, "dlogits", _f32()), _ptr(ws, "ws"), ws_bytes, st))


def moe_bias_update(shape, expert_counts, gamma, sel_bias, stream=None):
    lib = load_library()
    _need(shape, expert_counts=(expert_counts, shape.E), sel_bias=(sel_bias, shape.E))
    st = _stream(stream, sel_bias)
    _check("moe_bias_update", lib.moe_bias_update(
        ctypes.byref(shape), _ptr(expert_counts, "expert_counts", _i32()), float(gamma),
        _ptr(sel_bias, "sel_bias", _f32()), st))


# ------------------------------------------------------------------------------------------------
# device buffers (torch allocations sized by the capacity query)
# ------------------------------------------------------------------------------------------------
def alloc_buffers(shape: MoeShape, device, backward: bool = False, save_h: bool = True) -> dict:
    """Every buffer the forward (and optionally backward) calls write, on `device`."""
    import torch
    T, H, E, K, I, G, B = shape.T, shape.H, shape.E, shape.K, shape.I, shape.G, shape.block_m
    mcap = moe_row_capacity(shape)
    if mcap < 0:
        raise MoeError("moe_row_capacity", "MOE_ERR_INVALID_ARG", repr(shape))
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    e = lambda *s, dtype=bf: torch.empty(*s, dtype=dtype, device=device)  # noqa: E731
    buf = dict(
        mcap=mcap,
        logits=e(T, E, dtype=f32), probs=e(T, E, dtype=f32),
        topk_idx=e(T, K, dtype=i32), topk_w=e(T, K, dtype=f32), expert_counts=e(E, dtype=i32),
        seg_offsets=e(G + 1, dtype=i32), tile_group=e(max(1, mcap // B), dtype=i32),
        total_rows=e(1, dtype=i32), row_token=e(max(1, mcap), dtype=i32), pos=e(T, K, dtype=i32),
        ws=e(max(1, moe_workspace_size(shape)), dtype=torch.uint8),
        x_perm=e(mcap, H), a=e(mcap, I), y_perm=e(mcap, H), y=e(T, H),
        h_save=e(mcap, 2 * I) if (save_h or backward) else None,
    )
    if backward:
        buf.update(dy_perm=e(mcap, H), dtopk_w=e(T, K, dtype=f32), dh=e(mcap, 2 * I),
                   dx_perm=e(mcap, H), dx=e(T, H), dw1=e(G, 2 * I, H), dw2=e(G, H, I))
    return buf
