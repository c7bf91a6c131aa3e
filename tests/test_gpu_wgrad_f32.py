"""GPU parity of the fp32 weight gradients (grouped_gemm_wgrad_f32), through the C ABI.

Inputs are seeded synthetic bf16 activations laid out in block-padded segments (zero padding
rows), never GPU outputs. The oracle is expert_ffn_wgrad with fp32 outputs. Bar, from fp32
accumulation (u = 2^-24) over a segment of n rows: |got - ref| <= n u sum_r |a_r b_r| + u |ref| per
element, and rel-L2 <= 1e-5 per group. Rounding the fp32 result to bf16 must reproduce the bf16
entry point's dW bit for bit (same accumulation, one rounding).
"""
import numpy as np
import pytest
import torch

import grouped_gemm_fp32_amd as M
from oracle import moe_oracle as O
from tests.gpu_helpers import DEV, log, bf16_dev, i32_dev, bits_host, rel_l2

pytestmark = pytest.mark.gpu
U = 2.0 ** -24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    M.load_library()


def _segments(counts, B):
    seg = [0]
    for c in counts:
        seg.append(seg[-1] + (c + B - 1) // B * B)
    return np.array(seg, np.int32)


def _rows(rng, seg, counts, width, scale):
    """bf16 bits [rows, width]: N(0, scale^2) on each segment's first counts[g] rows, 0 on padding."""
    v = np.zeros((int(seg[-1]), width))
    for g, c in enumerate(counts):
        v[seg[g]:seg[g] + c] = rng.standard_normal((c, width)) * scale
    return O.bf16_bits(O.round_bf16(v))


@pytest.mark.parametrize("H,I,B,counts", [
    (256, 128, 16, [5, 0, 37, 16, 1]),
    (512, 192, 64, [300, 0, 64, 129]),
    (1024, 256, 128, [384] * 6 + [0, 700]),
])
def test_wgrad_f32_parity(H, I, B, counts):
    log(f"wgrad fp32 H={H} I={I} B={B} counts={counts}")
    rng = np.random.default_rng(H + I + B)
    E = len(counts)
    seg = _segments(counts, B)
    x_perm, a = _rows(rng, seg, counts, H, 1.0), _rows(rng, seg, counts, I, 0.5)
    dy_perm, dh = _rows(rng, seg, counts, H, 1e-2), _rows(rng, seg, counts, 2 * I, 1e-2)
    T = max(1, max(counts))
    s = M.make_shape(T, H, E, 1, I, 0, B)
    X, A, DY, DH, SEG = bf16_dev(x_perm), bf16_dev(a), bf16_dev(dy_perm), bf16_dev(dh), i32_dev(seg)
    dw1 = torch.full((E, 2 * I, H), float("nan"), device=DEV)
    dw2 = torch.full((E, H, I), float("nan"), device=DEV)
    M.grouped_gemm_wgrad_f32(s, M.MOE_WGRAD, X, A, DY, DH, SEG, dw1, dw2)
    dw1_b = torch.empty(E, 2 * I, H, dtype=torch.bfloat16, device=DEV)
    dw2_b = torch.empty(E, H, I, dtype=torch.bfloat16, device=DEV)
    M.grouped_gemm_bwd(s, M.MOE_WGRAD, X, None, A, DY, SEG, None, None, None, None, DH, None,
                       dw1_b, dw2_b)
    torch.cuda.synchronize()
    xv, av, dyv, dhv = (O.bf16_to_f64(t) for t in (x_perm, a, dy_perm, dh))
    ref1, ref2 = O.expert_ffn_wgrad(xv, av, dyv, dhv, seg, I, H, rnd="fp32")
    got1, got2 = dw1.cpu().numpy(), dw2.cpu().numpy()
    for g in range(E):
        r0, r1 = int(seg[g]), int(seg[g + 1])
        n = r1 - r0
        b1 = n * U * (np.abs(dhv[r0:r1]).T @ np.abs(xv[r0:r1])) + U * np.abs(ref1[g])
        b2 = n * U * (np.abs(dyv[r0:r1]).T @ np.abs(av[r0:r1])) + U * np.abs(ref2[g])
        for got, ref, bound, name in ((got1[g], ref1[g], b1, "dW1"), (got2[g], ref2[g], b2, "dW2")):
            err = np.abs(got.astype(np.float64) - ref)
            assert np.all(err <= bound), (name, g, float((err - bound).max()))
            if n == 0:
                assert np.all(got == 0), (name, g)
            else:
                assert rel_l2(got, ref) <= 1e-5, (name, g, rel_l2(got, ref))
    # one rounding of the fp32 sums gives the bf16 entry point's result
    for f32, b16, name in ((dw1, dw1_b, "dW1"), (dw2, dw2_b, "dW2")):
        assert torch.equal(f32.to(torch.bfloat16).view(torch.int16), b16.view(torch.int16)), name
