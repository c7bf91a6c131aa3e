"""Pins for the oracle's backward: central finite differences of L = <dy, y> in float64 with the
bf16 roundings turned off and the routing held fixed (CPU only)."""
import numpy as np
import pytest

from oracle import moe_oracle as O
from synth import draw_topk_given

T, H, E, K, I, S, B = 6, 8, 4, 2, 4, 1, 4


@pytest.fixture(scope="module")
def problem():
    rng = np.random.default_rng(123)
    x = rng.standard_normal((T, H))
    w1 = rng.standard_normal((E + S, 2 * I, H)) / np.sqrt(H)
    w2 = rng.standard_normal((E + S, H, I)) / np.sqrt(I)
    idx = draw_topk_given(T, E, K, seed=5)
    w = np.round(rng.uniform(0.1, 0.9, (T, K)) * 4096) / 4096   # exact in fp32, also after +-2^-8
    dy = rng.standard_normal((T, H))
    return x, w1, w2, idx, w, dy


def _loss(x, w1, w2, idx, w, dy):
    out = O.moe_forward(x, w1, w2, T=T, H=H, E=E, K=K, I=I, S=S, B=B, topk_idx=idx,
                        topk_w=w.astype(np.float64), rnd=None)
    return float(np.sum(dy * out["y"])), out


def _grads(problem):
    x, w1, w2, idx, w, dy = problem
    # The oracle takes fp32 weights; use values exactly representable so the FD sees the same w.
    _, fwd = _loss(x, w1, w2, idx, w, dy)
    fwd["topk_w"] = w
    return O.moe_backward(fwd, dy, w1, w2, T=T, H=H, E=E, K=K, I=I, S=S, rnd=None)


def _fd(f, arr, index, eps=1e-5):
    a0 = arr[index]
    arr[index] = a0 + eps
    lp = f()
    arr[index] = a0 - eps
    lm = f()
    arr[index] = a0
    return (lp - lm) / (2 * eps)


def test_fd_dx_dw1_dw2_dw(problem):
    x, w1, w2, idx, w, dy = [np.array(v, copy=True) for v in problem]
    w = w.astype(np.float32).astype(np.float64)   # weights pass through fp32 in the oracle
    g = _grads((x, w1, w2, idx, w, dy))
    rng = np.random.default_rng(7)

    def L():
        return _loss(x, w1, w2, idx, w, dy)[0]

    for _ in range(12):
        t, hh = rng.integers(T), rng.integers(H)
        np.testing.assert_allclose(g["dx"][t, hh], _fd(L, x, (t, hh)), rtol=1e-6, atol=1e-9)
    for _ in range(12):
        gg, j, hh = rng.integers(E + S), rng.integers(2 * I), rng.integers(H)
        np.testing.assert_allclose(g["dw1"][gg, j, hh], _fd(L, w1, (gg, j, hh)), rtol=1e-6, atol=1e-9)
    for _ in range(12):
        gg, hh, i = rng.integers(E + S), rng.integers(H), rng.integers(I)
        np.testing.assert_allclose(g["dw2"][gg, hh, i], _fd(L, w2, (gg, hh, i)), rtol=1e-6, atol=1e-9)


def test_fd_dtopk_w(problem):
    x, w1, w2, idx, w, dy = [np.array(v, copy=True) for v in problem]
    g = _grads((x, w1, w2, idx, w, dy))
    for t in range(T):
        for j in range(K):
            def L():
                return _loss(x, w1, w2, idx, w, dy)[0]
            # L is linear in w, so the difference quotient is exact up to float64 rounding; dtopk_w
            # itself is stored in fp32.
            np.testing.assert_allclose(g["dtopk_w"][t, j], _fd(L, w, (t, j), eps=2**-8), rtol=2e-7,
                                       atol=1e-9)


def test_directional_derivative_of_the_whole_layer(problem):
    # <grad, v> over all inputs equals d/ds L(theta + s v) at s = 0.
    x, w1, w2, idx, w, dy = [np.array(v, copy=True) for v in problem]
    g = _grads((x, w1, w2, idx, w, dy))
    rng = np.random.default_rng(9)
    vx, v1, v2 = rng.standard_normal(x.shape), rng.standard_normal(w1.shape), rng.standard_normal(w2.shape)
    lin = np.sum(g["dx"] * vx) + np.sum(g["dw1"] * v1) + np.sum(g["dw2"] * v2)
    eps = 1e-6
    lp = _loss(x + eps * vx, w1 + eps * v1, w2 + eps * v2, idx, w, dy)[0]
    lm = _loss(x - eps * vx, w1 - eps * v1, w2 - eps * v2, idx, w, dy)[0]
    np.testing.assert_allclose(lin, (lp - lm) / (2 * eps), rtol=1e-6)


def test_padding_rows_of_gradients_are_zero(problem):
    x, w1, w2, idx, w, dy = problem
    _, fwd = _loss(x, w1, w2, idx, w, dy)
    g = O.moe_backward(fwd, dy, w1, w2, T=T, H=H, E=E, K=K, I=I, S=S)
    pad = fwd["row_token"][:fwd["total_rows"]] < 0
    assert pad.any()
    for k in ("dy_perm", "dh", "dx_perm"):
        assert np.all(g[k][pad] == 0)
