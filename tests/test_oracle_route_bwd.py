"""Pins for the oracle's router backward and load-balancing bias update (CPU only).

The backward is checked against two things the oracle does not use: PyTorch's float64 autograd of
the forward definition (softmax over the routed experts, the K selected probabilities, optionally
renormalised), and central finite differences of that forward in float64. The bias update is
checked on hand-worked loads.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from synth import draw_logits


def _routing(T, E, K, seed):
    z = draw_logits(T, E, seed=seed)
    p = O.softmax_probs(z)
    idx, _ = O.select_topk(p, None, K)
    dw = np.random.default_rng(seed + 1).standard_normal((T, K)).astype(np.float32)
    return z, p, idx, dw


def _weights64(z, idx, normalize):
    """Forward definition in float64: w = the selected softmax probabilities (renormalised)."""
    p = torch.softmax(z, dim=1)
    sel = torch.gather(p, 1, idx)
    return sel / sel.sum(dim=1, keepdim=True) if normalize else sel


@pytest.mark.parametrize("normalize", [True, False])
@pytest.mark.parametrize("T,E,K", [(50, 8, 2), (40, 128, 6), (16, 256, 8), (10, 6, 6)])
def test_route_backward_matches_autograd(T, E, K, normalize):
    z, p, idx, dw = _routing(T, E, K, seed=T + E + K)
    # Autograd at the fp32 probabilities' own logits: softmax of log(p) is p itself, so the
    # reference sees exactly the probabilities the oracle is given.
    zt = torch.tensor(np.log(p.astype(np.float64)), dtype=torch.float64, requires_grad=True)
    w = _weights64(zt, torch.tensor(idx, dtype=torch.int64), normalize)
    (w * torch.tensor(dw, dtype=torch.float64)).sum().backward()
    ref = zt.grad.numpy()
    got = O.route_backward(p, idx, dw, normalize).astype(np.float64)
    np.testing.assert_allclose(got, ref, rtol=2e-6, atol=2e-7 * np.abs(ref).max())


@pytest.mark.parametrize("normalize", [True, False])
def test_route_backward_finite_differences(normalize):
    T, E, K = 6, 10, 3
    z, p, idx, dw = _routing(T, E, K, seed=3)
    z64 = np.log(p.astype(np.float64))

    def loss(zz):
        ez = np.exp(zz - zz.max(axis=1, keepdims=True))
        pp = ez / ez.sum(axis=1, keepdims=True)
        sel = np.take_along_axis(pp, idx.astype(np.int64), axis=1)
        w = sel / sel.sum(axis=1, keepdims=True) if normalize else sel
        return float((w * dw.astype(np.float64)).sum())

    h = 1e-6
    fd = np.zeros((T, E))
    for t in range(T):
        for e in range(E):
            zp, zm = z64.copy(), z64.copy()
            zp[t, e] += h
            zm[t, e] -= h
            fd[t, e] = (loss(zp) - loss(zm)) / (2 * h)
    got = O.route_backward(p, idx, dw, normalize).astype(np.float64)
    np.testing.assert_allclose(got, fd, rtol=1e-5, atol=1e-8)


def test_route_backward_invariants():
    T, E, K = 300, 64, 6
    z, p, idx, dw = _routing(T, E, K, seed=9)
    for normalize in (True, False):
        dz = O.route_backward(p, idx, dw, normalize).astype(np.float64)
        # softmax gradients sum to zero over the experts
        assert np.abs(dz.sum(axis=1)).max() <= 1e-6 * np.abs(dz).max()
    dz = O.route_backward(p, idx, dw, True)
    off = np.ones((T, E), bool)
    np.put_along_axis(off, idx.astype(np.int64), False, axis=1)
    # renormalised weights: the selected probabilities' gradients sum to zero against p, so the
    # unselected logits get nothing (up to float64 rounding of that zero sum)
    assert np.abs(dz[off]).max() <= 1e-12 * np.abs(dz).max()
    # renormalised weights sum to one, so a gradient equal on every slot has no effect
    flat = np.repeat(dw[:, :1], K, axis=1)
    assert np.abs(O.route_backward(p, idx, flat, True)).max() <= 1e-7 * np.abs(flat).max()


@pytest.mark.parametrize("T,H,E", [(37, 64, 8), (64, 256, 128)])
def test_router_weight_and_input_grads_match_autograd(T, H, E):
    rng = np.random.default_rng(T * H + E)
    x = O.bf16_bits(O.round_bf16(rng.standard_normal((T, H))))
    wg = (rng.standard_normal((E, H)) / np.sqrt(H)).astype(np.float32)
    dz = rng.standard_normal((T, E)).astype(np.float32)
    xt = torch.tensor(O.bf16_to_f64(x), requires_grad=True)
    wt = torch.tensor(wg.astype(np.float64), requires_grad=True)
    ((xt @ wt.T) * torch.tensor(dz, dtype=torch.float64)).sum().backward()
    np.testing.assert_allclose(O.router_weight_grad(dz, x), wt.grad.numpy(), rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(O.router_input_grad(dz, wg), xt.grad.numpy(), rtol=1e-6, atol=1e-6)


def test_bias_update_hand_worked():
    # T=4 tokens, K=2: 8 routed slots over E=4 experts, mean load 2.
    counts = np.array([3, 2, 1, 2], np.int32)
    b = np.array([0.5, -0.25, 0.0, 1.0], np.float32)
    got = O.bias_update(b, counts, T=4, K=2, gamma=0.125)
    assert got.tolist() == [0.375, -0.25, 0.125, 1.0]   # overloaded down, underloaded up
    # a mean load that is not an integer: T*K/E = 6/4 = 1.5, so no expert sits at the mean
    got = O.bias_update(np.zeros(4, np.float32), np.array([2, 1, 2, 1]), T=3, K=2, gamma=0.5)
    assert got.tolist() == [-0.5, 0.5, -0.5, 0.5]


def test_bias_update_is_one_fp32_add():
    rng = np.random.default_rng(4)
    E, T, K = 128, 8192, 6
    b = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    counts = rng.integers(300, 470, E).astype(np.int32)
    got = O.bias_update(b, counts, T, K, 1e-3)
    step = np.abs(got.astype(np.float64) - b.astype(np.float64))
    ulp = np.spacing(np.abs(b)).astype(np.float64)
    moved = counts != 384
    # the step is gamma to within half an ulp of the result (one correctly rounded fp32 add)
    assert np.all(np.abs(step[moved] - np.float64(np.float32(1e-3))) <= 0.5 * np.maximum(ulp, np.spacing(np.abs(got)))[moved] + 1e-12)
    assert np.all(got[~moved] == b[~moved])
    assert np.all((got > b) == (counts < 384))


# --- sequence-wise balance loss ------------------------------------------------------------------
def _balance_autograd(p, idx, seq_len, alpha):
    """float64 autograd of the loss definition at the logits log(p) (the counts f held fixed)."""
    T, E = p.shape
    K = idx.shape[1]
    zt = torch.tensor(np.log(p.astype(np.float64)), dtype=torch.float64, requires_grad=True)
    pt = torch.softmax(zt, dim=1)
    n_seq = T // seq_len
    total = 0
    for q in range(n_seq):
        sl = slice(q * seq_len, (q + 1) * seq_len)
        f = torch.tensor(np.bincount(idx[sl].reshape(-1), minlength=E) * (E / (K * seq_len)),
                         dtype=torch.float64)
        total = total + alpha * (f * pt[sl].mean(dim=0)).sum()
    (total / n_seq).backward()
    return zt.grad.numpy()


@pytest.mark.parametrize("T,E,K,seq_len", [(64, 8, 2, 16), (96, 128, 6, 96), (40, 20, 4, 8)])
def test_balance_loss_gradient_matches_autograd(T, E, K, seq_len):
    z, p, idx, _ = _routing(T, E, K, seed=T + E)
    _, dz = O.balance_loss(p, idx, seq_len, 1e-2)
    ref = _balance_autograd(p, idx, seq_len, 1e-2)
    # the probabilities are fp32, so their softmax-of-log reproduction sums to 1 only to fp32 accuracy
    np.testing.assert_allclose(dz, ref, rtol=1e-5, atol=1e-6 * np.abs(ref).max())


def test_balance_loss_finite_differences():
    T, E, K, seq_len, alpha = 12, 6, 2, 4, 0.3
    z, p, idx, _ = _routing(T, E, K, seed=21)
    z64 = np.log(p.astype(np.float64))
    f = [np.bincount(idx[q * seq_len:(q + 1) * seq_len].reshape(-1), minlength=E) * (E / (K * seq_len))
         for q in range(T // seq_len)]

    def loss(zz):
        ez = np.exp(zz - zz.max(axis=1, keepdims=True))
        pp = ez / ez.sum(axis=1, keepdims=True)
        return np.mean([alpha * f[q] @ pp[q * seq_len:(q + 1) * seq_len].mean(axis=0)
                        for q in range(T // seq_len)])

    h = 1e-6
    fd = np.zeros((T, E))
    for t in range(T):
        for e in range(E):
            zp, zm = z64.copy(), z64.copy()
            zp[t, e] += h
            zm[t, e] -= h
            fd[t, e] = (loss(zp) - loss(zm)) / (2 * h)
    _, dz = O.balance_loss(p, idx, seq_len, alpha)
    np.testing.assert_allclose(dz, fd, rtol=1e-5, atol=1e-10)


def test_balance_loss_closed_forms():
    T, E, K, seq_len, alpha = 64, 8, 2, 32, 0.5
    # perfectly balanced routing with uniform affinities: f = 1, P = 1/E, so L = alpha
    idx = ((K * np.arange(T)[:, None] + np.arange(K)[None, :]) % E).astype(np.int32)
    p = np.full((T, E), 1.0 / E, np.float32)
    losses, dz = O.balance_loss(p, idx, seq_len, alpha)
    np.testing.assert_allclose(losses, alpha, rtol=1e-7)
    assert np.abs(dz).max() <= 1e-12          # uniform p: the softmax passes no gradient
    # collapse: every token on experts 0..K-1 with p = 1/K there: f = E/K, P = 1/K, L = alpha E / K
    idx = np.tile(np.arange(K, dtype=np.int32), (T, 1))
    p = np.zeros((T, E), np.float32)
    p[:, :K] = 1.0 / K
    losses, _ = O.balance_loss(p, idx, seq_len, alpha)
    np.testing.assert_allclose(losses, alpha * E / K, rtol=1e-7)
    # the gradient sums to zero over the experts (softmax; the fp32 probabilities sum to 1 only to
    # fp32 accuracy)
    z, p, idx, _ = _routing(T, E, K, seed=2)
    _, dz = O.balance_loss(p, idx, seq_len, alpha)
    assert np.abs(dz.sum(axis=1)).max() <= 1e-6 * np.abs(dz).max()
