"""The ABI called from plain C: tests/c_abi/moe_c_example.c (gcc, the HIP runtime's C API, no
Python or torch in the process) runs a forward + backward step through the entry points of
include/moe.h. On the GPU its outputs are compared with the oracle, with the bars of the other
parity tests: routing bit-exact on the tiny layer (its ranking margins are all wide), the combine
weights within 1e-6, bf16 outputs per tests/gpu_helpers.assert_bf16_close. On the CPU it must
reject an impossible shape with the library's own message before any device call.
"""
import os
import subprocess

import numpy as np
import pytest

from grouped_gemm_fp32_amd import build as B
from oracle import moe_oracle as O
from synth import get_config, draw_x, draw_wg, draw_sel_bias, draw_w1_all, draw_w2_all, draw_dy


@pytest.fixture(scope="module")
def exe():
    if not os.path.exists(B.LIB):
        B.build()
    if not os.path.exists(B.C_EXAMPLE):
        B.build_c_example()
    return B.C_EXAMPLE


def _header(T, H, E, K, I, S, blk, flags=1):
    return np.array([T, H, E, K, I, S, blk, flags], dtype=np.int32).tobytes()


def test_c_caller_rejects_an_impossible_shape(exe, tmp_path):
    inp = tmp_path / "in.bin"
    inp.write_bytes(_header(64, 256, 8, 9, 128, 1, 16))   # K > E
    r = subprocess.run([exe, str(inp), str(tmp_path / "out.bin")], capture_output=True, text=True,
                       timeout=60)
    assert r.returncode == 1, (r.returncode, r.stdout, r.stderr)
    assert "invalid shape" in r.stderr and "1<=K<=E" in r.stderr, r.stderr
    assert not (tmp_path / "out.bin").exists()


@pytest.mark.gpu
def test_c_caller_matches_the_oracle(exe, tmp_path):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from tests.gpu_helpers import assert_bf16_close, log
    cfg = get_config("c1")
    T, H, E, K, I, S, blk = cfg.T, cfg.H, cfg.E, cfg.K, cfg.I, cfg.S, cfg.block_m
    G = E + S
    x, wg, sb = draw_x(cfg), draw_wg(cfg), draw_sel_bias(cfg)
    w1, w2, dy = draw_w1_all(cfg), draw_w2_all(cfg), draw_dy(cfg)
    inp, out = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(_header(T, H, E, K, I, S, blk))
        for a, dt in ((x, np.uint16), (wg, np.float32), (sb, np.float32), (w1, np.uint16),
                      (w2, np.uint16), (dy, np.uint16)):
            f.write(np.ascontiguousarray(a, dtype=dt).tobytes())
    log(f"C caller: T={T} H={H} E={E} K={K} I={I} S={S} block_m={blk}")
    r = subprocess.run([exe, str(inp), str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    log("  " + r.stdout.strip())
    buf = out.read_bytes()
    parts, off = {}, 0
    for name, n, dt in (("topk_idx", T * K, np.int32), ("topk_w", T * K, np.float32),
                        ("y", T * H, np.uint16), ("dtopk_w", T * K, np.float32),
                        ("dx", T * H, np.uint16), ("dw1", G * 2 * I * H, np.uint16),
                        ("dw2", G * H * I, np.uint16)):
        nb = n * np.dtype(dt).itemsize
        parts[name] = np.frombuffer(buf[off:off + nb], dtype=dt)
        off += nb
    assert off == len(buf)
    kw = dict(T=T, H=H, E=E, K=K, I=I, S=S)
    ref = O.moe_forward(x, w1, w2, B=blk, w_gate=wg, sel_bias=sb, **kw)
    bwd = O.moe_backward(ref, dy, w1, w2, **kw)
    np.testing.assert_array_equal(parts["topk_idx"].reshape(T, K), ref["topk_idx"])
    np.testing.assert_allclose(parts["topk_w"].reshape(T, K), ref["topk_w"], rtol=0, atol=1e-6)
    assert_bf16_close(O.bf16_to_f64(parts["y"].reshape(T, H)), ref["y"], "y")
    assert_bf16_close(parts["dtopk_w"].reshape(T, K), bwd["dtopk_w"], "dtopk_w", row_axis=0)
    assert_bf16_close(O.bf16_to_f64(parts["dx"].reshape(T, H)), bwd["dx"], "dx")
    assert_bf16_close(O.bf16_to_f64(parts["dw1"].reshape(G, 2 * I, H)), bwd["dw1"], "dw1")
    assert_bf16_close(O.bf16_to_f64(parts["dw2"].reshape(G, H, I)), bwd["dw2"], "dw2")
