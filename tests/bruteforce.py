"""Brute-force per-token evaluator of the MoE layer, used only to pin the oracle.

It shares no code with the oracle: per token it computes the router logits with exactly rounded
sums (math.fsum), the softmax with math.exp, picks the top-K by repeated arg-max (ties to the lower
index), evaluates every selected expert and every shared expert on that one token, and adds the
weighted outputs. No permutation, no padding, no grouping. bf16 rounding is done per scalar with
math.frexp/ldexp and Python's round-half-even.
"""
from __future__ import annotations

import math

import numpy as np


def bits_to_float(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f32(v: float) -> float:
    return float(np.float32(v))


def bf16_scalar(v: float) -> float:
    """Nearest bf16 value, ties to even (finite inputs in the normal range and zero)."""
    if v == 0.0 or not math.isfinite(v):
        return v
    m, e = math.frexp(v)             # v = m 2^e, 0.5 <= |m| < 1
    q = max(e - 8, -133)             # 8 significant bits; subnormal grid 2^-133
    return math.ldexp(round(math.ldexp(v, -q)), q)


def bf16_vec(a) -> np.ndarray:
    return np.array([bf16_scalar(float(v)) for v in np.asarray(a).ravel()]).reshape(np.shape(a))


def _beats(ke: float, kb: float) -> bool:
    """Strictly better key: a number beats NaN, NaN never beats anything, else larger wins."""
    if math.isnan(kb):
        return not math.isnan(ke)
    if math.isnan(ke):
        return False
    return ke > kb


def pick_topk(key, K):
    """K rounds of arg-max over the remaining experts; scanning upward and replacing only on a
    strictly better key keeps the lower index on ties."""
    chosen = []
    for _ in range(K):
        best = None
        for e in range(len(key)):
            if e in chosen:
                continue
            if best is None or _beats(key[e], key[best]):
                best = e
        chosen.append(best)
    return chosen


def route_token(x_t, wg, logit_bias, sel_bias, K, normalize=True):
    E = wg.shape[0]
    logits = []
    for e in range(E):
        z = math.fsum(float(a) * float(b) for a, b in zip(x_t, wg[e]))
        if logit_bias is not None:
            z += float(logit_bias[e])
        logits.append(f32(z))
    m = max(logits)
    ex = [math.exp(z - m) for z in logits]
    s = math.fsum(ex)
    p = [f32(v / s) for v in ex]
    key = [f32(np.float32(p[e]) + np.float32(sel_bias[e])) for e in range(E)]
    chosen = pick_topk(key, K)
    sp = [p[e] for e in chosen]
    if normalize:
        tot = math.fsum(sp)
        w = [f32(v / tot) for v in sp]
    else:
        w = sp
    return chosen, w, logits, p


def expert_on_token(x_t, w1, w2, I, rounding=True):
    """SwiGLU expert on one token: h = W1 x, a = silu(h_gate) h_up, y = W2 a."""
    h = w1 @ x_t
    g, u = h[:I], h[I:]
    a = g / (1.0 + np.exp(-g)) * u
    if rounding:
        a = bf16_vec(a)
    y = w2 @ a
    if rounding:
        y = bf16_vec(y)
    return y


def layer_forward(x_bits, wg, logit_bias, sel_bias, w1_bits, w2_bits, T, E, K, I, S,
                  rounding=True, normalize=True):
    """Returns (y [T,H] float64, topk_idx [T,K], topk_w [T,K])."""
    x = bits_to_float(x_bits)
    wg64 = np.asarray(wg, dtype=np.float32).astype(np.float64)
    H = x.shape[1]
    y = np.zeros((T, H))
    idx = np.zeros((T, K), dtype=np.int64)
    wts = np.zeros((T, K))
    for t in range(T):
        chosen, w, _, _ = route_token(x[t], wg64, logit_bias, sel_bias, K, normalize)
        idx[t], wts[t] = chosen, w
        acc = np.zeros(H)
        for j, e in enumerate(chosen):
            acc += w[j] * expert_on_token(x[t], bits_to_float(w1_bits[e]), bits_to_float(w2_bits[e]),
                                          I, rounding)
        for s in range(S):
            acc += expert_on_token(x[t], bits_to_float(w1_bits[E + s]),
                                   bits_to_float(w2_bits[E + s]), I, rounding)
        y[t] = bf16_vec(acc) if rounding else acc
    return y, idx, wts
