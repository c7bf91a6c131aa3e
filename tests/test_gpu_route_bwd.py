"""GPU parity of the router backward and the load-balancing bias update, through the C ABI.

Bars, derived from fp32 arithmetic (u = 2^-24), against the float64 oracle rounded to fp32:
  * dlogits: per element |got - ref| <= 16 u (max_j |dw_j| + sum_j |dw_j|) + 2 u |ref| for the
    token (a handful of fp32 operations on values bounded by the slot gradients, p <= 1);
  * dWg = dlogits^T x (n = T/4 + 8 sequential fp32 additions per wavefront, then four partial sums)
    and dx_router = dlogits Wg (n = E + 4): |got - ref| <= n u sum_k |a_k b_k| + u |ref|, plus the
    dlogits bound carried through the product; and rel-L2 <= 1e-5;
  * bias update: bit-exact (integer comparison and one fp32 add on both sides);
  * balance loss: per sequence within (seq_len + E + 8) u of the oracle (all terms non-negative;
    partial sums per 256-token chunk, reduced in chunk order);
    its gradient as stated at the test.
Inputs come from the seeded generators and the oracle's own routing, never from the GPU.
"""
import numpy as np
import pytest
import torch

import grouped_gemm_fp32_amd as M
from oracle import moe_oracle as O
from synth import draw_logits
from tests.gpu_helpers import DEV, log, bf16_dev, f32_dev, i32_dev, rel_l2

pytestmark = pytest.mark.gpu
U = 2.0 ** -24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    M.load_library()  # raises when the HIP library is missing: no fallback exists


def _np(t):
    return t.detach().cpu().numpy()


def _inputs(T, H, E, K, seed):
    rng = np.random.default_rng(seed)
    z = draw_logits(T, E, seed=seed)
    p = O.softmax_probs(z)
    idx, _ = O.select_topk(p, None, K)
    dw = rng.standard_normal((T, K)).astype(np.float32)
    x = O.bf16_bits(O.round_bf16(rng.standard_normal((T, H))))
    wg = (rng.standard_normal((E, H)) / np.sqrt(H)).astype(np.float32)
    return p, idx, dw, x, wg


def _check_contraction(got, ref, bound, name):
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    bad = err > bound
    assert not bad.any(), (name, int(bad.sum()), float((err - bound).max()))
    r = rel_l2(got, ref)
    log(f"  {name}: rel-L2 {r:.2e}, worst err/bound {float((err / bound).max()):.3f}")
    assert r <= 1e-5, (name, r)


@pytest.mark.parametrize("normalize", [True, False])
@pytest.mark.parametrize("T,H,E,K", [
    (64, 256, 8, 2),          # the tiny layer's routing
    (333, 256, 20, 4),        # ragged tokens, experts not a multiple of 32
    (101, 128, 256, 8),       # the most experts and slots a shape may have
    (77, 128, 13, 3),         # E % 4 != 0: dlogits rows not 16-byte aligned (scalar loads)
    (8192, 4096, 128, 6),     # the benchmark shape
])
def test_route_bwd_parity(T, H, E, K, normalize):
    log(f"route bwd T={T} H={H} E={E} K={K} norm={normalize}")
    p, idx, dw, x, wg = _inputs(T, H, E, K, seed=T + E + K)
    s = M.make_shape(T, H, E, K, 128, 0, 16, M.MOE_NORM_TOPK if normalize else 0)
    dz_d = torch.empty(T, E, device=DEV)
    dwg_d = torch.empty(E, H, device=DEV)
    dx_d = torch.empty(T, H, device=DEV)
    M.moe_route_bwd(s, f32_dev(dw), i32_dev(idx), f32_dev(p), bf16_dev(x), f32_dev(wg), dz_d, dwg_d,
                    dx_d)
    torch.cuda.synchronize()
    dz_ref = O.route_backward(p, idx, dw, normalize)
    dz = _np(dz_d)
    scale = 16 * U * (np.abs(dw).max(axis=1) + np.abs(dw).sum(axis=1))
    dz_bound = scale[:, None] + 2 * U * np.abs(dz_ref)
    _check_contraction(dz, dz_ref, dz_bound, "dlogits")
    if normalize:   # unselected experts get exactly nothing
        off = np.ones((T, E), bool)
        np.put_along_axis(off, idx.astype(np.int64), False, axis=1)
        assert np.all(dz[off] == 0)
    xv = O.bf16_to_f64(x)
    adz, adzb = np.abs(dz_ref.astype(np.float64)), dz_bound
    dwg_ref = O.router_weight_grad(dz_ref, x)
    n = T / 4 + 8
    dwg_bound = n * U * (adz.T @ np.abs(xv)) + adzb.T @ np.abs(xv) + U * np.abs(dwg_ref)
    _check_contraction(_np(dwg_d), dwg_ref, dwg_bound, "dWg")
    dx_ref = O.router_input_grad(dz_ref, wg)
    awg = np.abs(wg.astype(np.float64))
    dx_bound = (E + 4) * U * (adz @ awg) + adzb @ awg + U * np.abs(dx_ref)
    _check_contraction(_np(dx_d), dx_ref, dx_bound, "dx_router")


def test_route_bwd_optional_outputs_and_empty_batch():
    T, H, E, K = 50, 128, 16, 3
    p, idx, dw, x, wg = _inputs(T, H, E, K, seed=5)
    s = M.make_shape(T, H, E, K, 128, 0, 16)
    dz_d = torch.empty(T, E, device=DEV)
    M.moe_route_bwd(s, f32_dev(dw), i32_dev(idx), f32_dev(p), None, None, dz_d, None, None)
    torch.cuda.synchronize()
    np.testing.assert_allclose(_np(dz_d), O.route_backward(p, idx, dw), rtol=1e-5, atol=1e-7)
    # an empty batch: the weight gradient is a sum over no tokens
    s0 = M.make_shape(0, H, E, K, 128, 0, 16)
    dwg_d = torch.full((E, H), 7.0, device=DEV)
    M.moe_route_bwd(s0, None, None, None, None, None, None, dwg_d, None)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dwg_d).item() == 0


@pytest.mark.parametrize("T,K,E", [(8192, 6, 128), (3, 2, 4), (1000, 8, 256), (7, 1, 5)])
def test_bias_update_bitexact(T, K, E):
    log(f"bias update T={T} K={K} E={E}")
    rng = np.random.default_rng(T + K + E)
    mean = T * K / E
    counts = rng.integers(max(0, int(mean) - 3), int(mean) + 4, E).astype(np.int32)
    if float(mean).is_integer():
        counts[: E // 4] = int(mean)          # experts exactly at the mean keep their bias
    b = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    s = M.make_shape(T, 128, E, K, 128, 0, 16)
    for gamma in (1e-3, 0.0, 0.25):
        b_d = f32_dev(b)
        M.moe_bias_update(s, i32_dev(counts), gamma, b_d)
        torch.cuda.synchronize()
        ref = O.bias_update(b, counts, T, K, gamma)
        assert np.array_equal(_np(b_d).view(np.uint32), ref.view(np.uint32)), gamma


@pytest.mark.parametrize("T,E,K,seq_len", [(64, 8, 2, 16), (300, 20, 4, 100), (8192, 128, 6, 4096),
                                           (8192, 128, 6, 1024), (257, 256, 8, 257)])
def test_balance_loss_parity(T, E, K, seq_len):
    """Loss: every term f_e P_e is >= 0, so fp32 sums of n terms are within n u of the result.
    Gradient (added to an existing dlogits): |got - ref| <= 2 u |ref| + (E + 8) u p_e (g_e + sum_i
    p_i g_i), all of those terms non-negative."""
    log(f"balance loss T={T} E={E} K={K} seq_len={seq_len}")
    rng = np.random.default_rng(T + E + seq_len)
    p = O.softmax_probs(draw_logits(T, E, seed=T + 3))
    idx, _ = O.select_topk(p, None, K)
    base = rng.standard_normal((T, E)).astype(np.float32) * np.float32(1e-4)
    alpha = 1e-3
    s = M.make_shape(T, 128, E, K, 128, 0, 16)
    loss_d = torch.empty(T // seq_len, device=DEV)
    dz_d = f32_dev(base)
    ws = torch.empty(M.moe_balance_workspace_size(s, seq_len) // 4, device=DEV)
    M.moe_balance_loss(s, seq_len, alpha, f32_dev(p), i32_dev(idx), loss_d, dz_d, ws)
    torch.cuda.synchronize()
    ref_loss, ref_dz = O.balance_loss(p, idx, seq_len, alpha)
    got_loss = _np(loss_d).astype(np.float64)
    assert np.all(np.abs(got_loss - ref_loss) <= (seq_len + E + 8) * U * np.abs(ref_loss)), \
        (got_loss, ref_loss)
    ref = base.astype(np.float64) + ref_dz
    n_seq = T // seq_len
    pv = p.astype(np.float64)
    g = np.zeros((T, E))
    for q in range(n_seq):
        f = np.bincount(idx[q * seq_len:(q + 1) * seq_len].reshape(-1), minlength=E) * (E / (K * seq_len))
        g[q * seq_len:(q + 1) * seq_len] = alpha * f / (seq_len * n_seq)
    bound = 2 * U * np.abs(ref) + (E + 8) * U * pv * (g + (pv * g).sum(axis=1, keepdims=True))
    err = np.abs(_np(dz_d).astype(np.float64) - ref)
    assert np.all(err <= bound), float((err - bound).max())
    log(f"  loss {got_loss[:4]}, worst err/bound {float((err / bound).max()):.3f}")


@pytest.mark.parametrize("offset", [0, 1])
def test_router_grads_from_given_dlogits(offset):
    """offset 1: dlogits starts 4 bytes past a 16-byte boundary (the scalar-load path)."""
    T, H, E, K = 512, 256, 32, 4
    p, idx, dw, x, wg = _inputs(T, H, E, K, seed=11)
    dz = O.route_backward(p, idx, dw) + O.balance_loss(p, idx, 128, 1e-2)[1].astype(np.float32)
    dz = dz.astype(np.float32)
    s = M.make_shape(T, H, E, K, 128, 0, 16)
    dwg_d, dx_d = torch.empty(E, H, device=DEV), torch.empty(T, H, device=DEV)
    dz_d = torch.empty(T * E + offset, device=DEV)
    dz_d[offset:] = f32_dev(dz).reshape(-1)
    M.moe_router_grads(s, dz_d[offset:], bf16_dev(x), f32_dev(wg), dwg_d, dx_d)
    torch.cuda.synchronize()
    xv, adz, awg = O.bf16_to_f64(x), np.abs(dz.astype(np.float64)), np.abs(wg.astype(np.float64))
    ref = O.router_weight_grad(dz, x)
    _check_contraction(_np(dwg_d), ref, (T / 4 + 8) * U * (adz.T @ np.abs(xv)) + U * np.abs(ref), "dWg")
    ref = O.router_input_grad(dz, wg)
    _check_contraction(_np(dx_d), ref, (E + 4) * U * (adz @ awg) + U * np.abs(ref), "dx_router")
