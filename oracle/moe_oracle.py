"""Plain CPU oracle of the dots.llm1 MoE feed-forward path.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check in __graft_entry__ and bench.py's CPU-baseline leg may import
this module. The product path (the HIP library and its binding) never calls it, shares no code with
it and fails loudly when its own extension is missing.

What it computes, and where that is stated (TR = the dots.llm1 Technical Report notes page):
  * TR section A2 "Architecture", mixture-of-experts paragraph: the FFN is a MoE with routed experts
    and always-on shared experts; each expert is a two-layer FFN with SwiGLU; the router picks the
    top-6 routed experts per token; the gating is computed in FP32, not BF16.
  * TR section A2, load-balancing paragraph: a per-expert bias is added to the affinity scores only
    to decide the top-k; no token is dropped.
  * TR section 3.2 "Efficient grouped GEMM": each expert's token segment M_i is padded to a fixed
    block size so every tile of rows belongs to one expert. Padding and permutation only reorganise
    the work; the result is the plain MoE definition.
  * TR section 6 "MoE analysis": the per-expert token count N_{E_i} behind the expert-load figure.
  * TR section A2, load-balancing paragraph, again: the per-expert bias is adjusted during training
    to keep the expert loads balanced (the router backward and the bias update below).

Where the pages leave a step open the oracle takes one reading, stated at the function:
softmax affinities over the routed experts; the bias added to the probability; weights renormalised
over the K selected experts (optional); ties to the lower expert index, NaN below every number;
SwiGLU(x) = W2 (silu(W1_gate x) * W1_up x) with no biases; shared experts weight 1; ascending token
order inside a segment with shared groups last; bf16 round-to-nearest-even at the stored tensors
(h, a, y_perm, y, dy_perm, dh, dx_perm, dx, dW1, dW2) and fp32 for logits, probabilities and weights;
the selection passes no gradient and the selection bias gets none; the bias moves by a fixed step
gamma toward the mean load (sign of mean load minus the expert's load).

Arithmetic is float64 (products of bf16 values are exact in it); rounding to bf16 or fp32 happens
only where the path stores a tensor. Passing ``rnd=None`` turns every bf16 rounding off, which the
finite-difference and identity checks use.

bf16 tensors are passed in as uint16 bit patterns and float tensors as float32 arrays; outputs that
the path stores in bf16 are returned as float64 arrays holding bf16 values (see ``bf16_bits``).
"""
from __future__ import annotations

import numpy as np

# ------------------------------------------------------------------------------------------------
# Number formats
# ------------------------------------------------------------------------------------------------
_BF16_MANT = 7          # stored mantissa bits of bfloat16
_BF16_EMIN = -126       # smallest normal exponent (same as fp32)
_BF16_MAX = float.fromhex("0x1.fep127")


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 values (exact): a bf16 is the top half of an fp32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_bf16(v) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even (returned as float64).

    Written from the format's definition: a finite bf16 is m * 2^(e-7) with an 8-bit significand m,
    e >= -126, and subnormals on the grid 2^-133. We scale by the grid spacing of each value's binade,
    round half-to-even to an integer and scale back (both scalings are exact powers of two).
    Magnitudes that round beyond the largest finite bf16 become +-inf.
    """
    v = np.asarray(v, dtype=np.float64)
    out = v.copy()
    fin = np.isfinite(v) & (v != 0.0)
    x = v[fin]
    _, e = np.frexp(x)                     # x = m * 2^e, 0.5 <= |m| < 1, so the binade is 2^(e-1)
    q = np.maximum(e - 1 - _BF16_MANT, _BF16_EMIN - _BF16_MANT)  # spacing exponent
    r = np.ldexp(np.rint(np.ldexp(x, -q)), q)
    r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, r), r)
    out[fin] = r
    return out


def bf16_bits(v) -> np.ndarray:
    """float64 values already on the bf16 grid -> bf16 bit patterns."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def _identity(v):
    return np.asarray(v, dtype=np.float64)


def round_fp32(v) -> np.ndarray:
    """Round float64 values to the nearest fp32 value (returned as float64)."""
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def _rounder(rnd):
    if rnd is None:
        return _identity
    if rnd == "bf16":
        return round_bf16
    if rnd == "fp32":
        return round_fp32
    return rnd


def _as_values(a):
    """bf16 bit patterns (uint16) -> float64 values; any float array -> float64."""
    a = np.asarray(a)
    return bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def _w(weights, g):
    """Group g of a weight given as an array [G, ...] (bf16 bits or floats) or a callable g -> array."""
    return _as_values(weights(g) if callable(weights) else weights[g])


# ------------------------------------------------------------------------------------------------
# a1-a5: router (TR section A2: FP32 gating; load balancing by a selection-only bias)
# ------------------------------------------------------------------------------------------------
def router_logits(x_bits, w_gate, logit_bias=None) -> np.ndarray:
    """logits[T,E] = x . Wg^T (+ logit_bias) in float64, rounded once to fp32.

    "FP32 gating" (TR section A2, MoE paragraph): the bf16 activations are widened exactly and the
    router weight is fp32. logit_bias is an optional per-expert offset used by the skewed workload
    (the model has no gate bias).
    """
    x = _as_values(x_bits)
    wg = np.asarray(w_gate, dtype=np.float32).astype(np.float64)
    z = x @ wg.T
    if logit_bias is not None:
        z = z + np.asarray(logit_bias, dtype=np.float32).astype(np.float64)[None, :]
    return z.astype(np.float32)


def softmax_probs(logits) -> np.ndarray:
    """Affinity scores p[T,E] = softmax over the routed experts, float64 rounded to fp32.

    Reading: the pages call them "affinity scores" (TR section A2, load balancing) without naming
    the function; we take the softmax over the E routed experts. The maximum is subtracted first,
    which changes nothing mathematically and keeps exp finite.
    """
    z = np.asarray(logits, dtype=np.float32).astype(np.float64)
    z = z - z.max(axis=1, keepdims=True)
    ez = np.exp(z)
    return (ez / ez.sum(axis=1, keepdims=True)).astype(np.float32)


def selection_keys(probs, sel_bias) -> np.ndarray:
    """key = p + b as one IEEE fp32 addition (TR section A2, load balancing: bias only for top-k)."""
    p = np.asarray(probs, dtype=np.float32)
    b = np.zeros(p.shape[1], np.float32) if sel_bias is None else np.asarray(sel_bias, np.float32)
    return (p + b[None, :]).astype(np.float32)


def select_topk(probs, sel_bias, K: int, normalize: bool = True):
    """Top-K experts per token by (key descending, expert index ascending); weights from p alone.

    Ordering: every number ranks above NaN; equal keys (including +0 and -0) go to the lower expert
    index; NaN keys tie among themselves by index. Slot j of a token holds its j-th ranked expert.
    Weights: w_j = p_{e_j} / sum_i p_{e_i} over the K selected experts when ``normalize`` (reading:
    renormalised, so the routed weights sum to 1), else w_j = p_{e_j}. The bias never enters w.
    Returns (topk_idx int32 [T,K], topk_w float32 [T,K]).
    """
    p = np.asarray(probs, dtype=np.float32)
    T, E = p.shape
    key = selection_keys(p, sel_bias).astype(np.float64)
    nan = np.isnan(key)
    # Full sort per token with a composite key: (is_nan asc, key desc, index asc).
    key_for_sort = np.where(nan, 0.0, -key)
    idx_all = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((idx_all, key_for_sort, nan), axis=1)
    topk_idx = order[:, :K].astype(np.int32)
    return topk_idx, combine_weights(p, topk_idx, normalize)


def combine_weights(probs, topk_idx, normalize: bool = True) -> np.ndarray:
    """Weights of a given selection: w_j = p_{e_j} / sum_i p_{e_i} over the token's K selected
    experts (renormalised) or w_j = p_{e_j}, from the affinities alone (TR section A2, load
    balancing: the bias decides the selection only). float64, rounded once to fp32."""
    p = np.asarray(probs, dtype=np.float32)
    sel_p = np.take_along_axis(p, np.asarray(topk_idx, dtype=np.int64), axis=1).astype(np.float64)
    w = sel_p / sel_p.sum(axis=1, keepdims=True) if normalize else sel_p
    return w.astype(np.float32)


def expert_counts(topk_idx, E: int) -> np.ndarray:
    """c_e = number of (token, slot) pairs routed to expert e (TR section 6: N_{E_i})."""
    idx = np.asarray(topk_idx).reshape(-1)
    return np.bincount(idx, minlength=E).astype(np.int32)


# ------------------------------------------------------------------------------------------------
# a6-a7: block-aligned segments and permutation (TR section 3.2)
# ------------------------------------------------------------------------------------------------
def row_capacity(T: int, E: int, K: int, S: int, B: int) -> int:
    """Rows reserved for the permuted buffers whatever the routing.

    Routed experts take sum_e ceil(c_e/B) blocks with sum_e c_e = T*K; that sum is at most
    floor((T*K + E*(B-1))/B) and at most T*K (a non-empty block holds a row). Each shared expert
    takes ceil(T/B) blocks. Never drops a token (TR section A2, load balancing: no token dropped).
    """
    R = T * K
    routed_blocks = min(R, (R + E * (B - 1)) // B)
    return B * (routed_blocks + S * (-(-T // B)))


def build_segments(counts, T: int, E: int, S: int, B: int, Mcap: int):
    """seg_offsets[G+1], tile_group[Mcap/B] and total_rows.

    Groups 0..E-1 are the routed experts in index order, groups E..E+S-1 the shared experts (each
    holding all T tokens). Each group's rows are padded up to a multiple of the block size B, so a
    block of B rows never spans two experts (TR section 3.2). tile_group[i] is the group whose
    segment contains rows i*B .. i*B+B-1, or -1 past the last segment.
    """
    c = list(np.asarray(counts, dtype=np.int64)) + [T] * S
    seg = [0]
    for cg in c:
        seg.append(seg[-1] + (-(-cg // B)) * B)
    seg = np.asarray(seg, dtype=np.int64)
    total = int(seg[-1])
    nblk = Mcap // B
    tile_group = np.full(nblk, -1, dtype=np.int32)
    for g in range(len(c)):
        tile_group[seg[g] // B: seg[g + 1] // B] = g
    return seg.astype(np.int32), tile_group, total


def permute_maps(topk_idx, seg_offsets, T: int, E: int, S: int, Mcap: int):
    """row_token[Mcap] (-1 on padding and unused rows) and pos[T,K] (row of each token-slot).

    Inside a routed expert's segment the rows hold the tokens routed to it in ascending token
    order (reading: the pages leave the order free; ascending is stable and deterministic).
    Shared expert s holds token t at row seg_offsets[E+s] + t.
    """
    idx = np.asarray(topk_idx, dtype=np.int64)
    K = idx.shape[1] if idx.ndim == 2 else 0
    seg = np.asarray(seg_offsets, dtype=np.int64)
    row_token = np.full(Mcap, -1, dtype=np.int32)
    pos = np.full((T, K), -1, dtype=np.int32)
    fill = seg[:E].copy()
    for t in range(T):
        for j in range(K):
            e = idx[t, j]
            pos[t, j] = fill[e]
            row_token[fill[e]] = t
            fill[e] += 1
    for s in range(S):
        base = seg[E + s]
        row_token[base: base + T] = np.arange(T, dtype=np.int32)
    return row_token, pos


def gather_rows(x_bits, row_token) -> np.ndarray:
    """x_perm[r] = x[row_token[r]] (bf16 values as float64), zero on padding rows."""
    x = _as_values(x_bits)
    rt = np.asarray(row_token, dtype=np.int64)
    out = np.zeros((len(rt), x.shape[1]), dtype=np.float64)
    ok = rt >= 0
    out[ok] = x[rt[ok]]
    return out


# ------------------------------------------------------------------------------------------------
# a8-a10: expert SwiGLU FFN per segment (TR section A2 MoE paragraph; TR section 3.2 grouped GEMM)
# ------------------------------------------------------------------------------------------------
def silu(z):
    return z / (1.0 + np.exp(-z))


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def expert_ffn_rows(x_rows, w1g, w2g, I: int, rnd="bf16"):
    """One expert's SwiGLU FFN on rows of bf16 values (float64 arrays).

    h = x W1^T ([gate | up], width 2I), a = silu(h_gate) * h_up, y = a W2^T; h, a and y are stored
    in bf16 (rounded here), a is computed from the unrounded h (fp32 accumulators on the device).
    Returns (h_stored, a, y).
    """
    R = _rounder(rnd)
    h = x_rows @ w1g.T
    a = R(silu(h[:, :I]) * h[:, I:])
    y = R(a @ w2g.T)
    return R(h), a, y


def expert_ffn_forward(x_perm, seg_offsets, w1, w2, I: int, rnd="bf16"):
    """Grouped GEMM forward: for every group g, its segment rows through that group's FFN.

    Equivalent by construction to separate dense per-expert GEMMs on each segment (TR section 3.2:
    the padding only aligns scheduling). Padding rows are zero inputs and give zero outputs.
    Returns (h [M,2I], a [M,I], y_perm [M,H]) over the rows covered by the segments.
    """
    seg = np.asarray(seg_offsets, dtype=np.int64)
    M, H = x_perm.shape
    h = np.zeros((M, 2 * I))
    a = np.zeros((M, I))
    y = np.zeros((M, H))
    for g in range(len(seg) - 1):
        r0, r1 = seg[g], seg[g + 1]
        if r1 == r0:
            continue
        hg, ag, yg = expert_ffn_rows(x_perm[r0:r1], _w(w1, g), _w(w2, g), I, rnd)
        h[r0:r1], a[r0:r1], y[r0:r1] = hg, ag, yg
    return h, a, y


# ------------------------------------------------------------------------------------------------
# a11: weighted combine
# ------------------------------------------------------------------------------------------------
def combine(y_perm, pos, topk_w, seg_offsets, T: int, E: int, S: int, rnd="bf16"):
    """y[t] = sum_j w[t,j] y_perm[pos[t,j]] + sum_s y_perm[seg_offsets[E+s] + t], stored in bf16.

    Shared experts enter with weight 1 (TR section A2: always active for every token).
    """
    R = _rounder(rnd)
    H = y_perm.shape[1]
    w = np.asarray(topk_w, dtype=np.float32).astype(np.float64)
    p = np.asarray(pos, dtype=np.int64)
    acc = np.zeros((T, H))
    for j in range(p.shape[1] if p.ndim == 2 else 0):
        acc += w[:, j:j + 1] * y_perm[p[:, j]]
    seg = np.asarray(seg_offsets, dtype=np.int64)
    for s in range(S):
        acc += y_perm[seg[E + s]: seg[E + s] + T]
    return R(acc)


# ------------------------------------------------------------------------------------------------
# b1-b6: backward with the routing held fixed (gradients of L = <dy, y>)
# ------------------------------------------------------------------------------------------------
def combine_backward(dy_bits_or_vals, y_perm, pos, topk_w, seg_offsets, total_rows: int,
                     T: int, E: int, S: int, rnd="bf16"):
    """dy_perm (rows of each token-slot, bf16) and dtopk_w [T,K] (fp32).

    dy_perm[pos[t,j]] = w[t,j] dy[t]; dy_perm[shared row of t] = dy[t]; padding rows 0.
    dtopk_w[t,j] = <dy[t], y_perm[pos[t,j]]>.
    """
    R = _rounder(rnd)
    dy = _as_values(dy_bits_or_vals)
    H = dy.shape[1]
    w = np.asarray(topk_w, dtype=np.float32).astype(np.float64)
    p = np.asarray(pos, dtype=np.int64)
    dy_perm = np.zeros((total_rows, H))
    K = p.shape[1] if p.ndim == 2 else 0
    dw = np.zeros((T, K))
    for j in range(K):
        dy_perm[p[:, j]] = R(w[:, j:j + 1] * dy)
        dw[:, j] = np.einsum("th,th->t", dy, y_perm[p[:, j]])
    seg = np.asarray(seg_offsets, dtype=np.int64)
    for s in range(S):
        dy_perm[seg[E + s]: seg[E + s] + T] = dy
    return dy_perm, dw.astype(np.float32)


def swiglu_backward(da, h, I: int):
    """d(silu(g) u)/d[g, u] times da, with g = h[:, :I], u = h[:, I:] and s = sigmoid(g):
    dg = da u s (1 + g (1 - s)), du = da g s."""
    g, u = h[:, :I], h[:, I:]
    s = sigmoid(g)
    return np.concatenate([da * u * s * (1.0 + g * (1.0 - s)), da * g * s], axis=1)


def expert_ffn_dgrad(dy_perm, h, seg_offsets, w1, w2, I: int, rnd="bf16"):
    """dgrad: da = dy_perm W2_g, dh = swiglu_backward(da, h) (stored bf16), dx_perm = dh W1_g."""
    R = _rounder(rnd)
    seg = np.asarray(seg_offsets, dtype=np.int64)
    M, H = dy_perm.shape
    dh = np.zeros((M, 2 * I))
    dx = np.zeros((M, H))
    for g in range(len(seg) - 1):
        r0, r1 = seg[g], seg[g + 1]
        if r1 == r0:
            continue
        da = dy_perm[r0:r1] @ _w(w2, g)
        dhg = R(swiglu_backward(da, h[r0:r1], I))
        dh[r0:r1] = dhg
        dx[r0:r1] = R(dhg @ _w(w1, g))
    return dh, dx


def expert_ffn_wgrad(x_perm, a, dy_perm, dh, seg_offsets, I: int, H: int, rnd="bf16"):
    """wgrad per group: dW2_g = dy_perm_seg^T a_seg [H,I]; dW1_g = dh_seg^T x_perm_seg [2I,H].
    A group with an empty segment gets zeros. rnd="fp32" gives the fp32-gradient variant (the
    same sums stored in fp32 instead of bf16)."""
    R = _rounder(rnd)
    seg = np.asarray(seg_offsets, dtype=np.int64)
    G = len(seg) - 1
    dw1 = np.zeros((G, 2 * I, H))
    dw2 = np.zeros((G, H, I))
    for g in range(G):
        r0, r1 = seg[g], seg[g + 1]
        if r1 == r0:
            continue
        dw2[g] = R(dy_perm[r0:r1].T @ a[r0:r1])
        dw1[g] = R(dh[r0:r1].T @ x_perm[r0:r1])
    return dw1, dw2


def unpermute_backward(dx_perm, pos, seg_offsets, T: int, E: int, S: int, rnd="bf16"):
    """dx[t] = sum_j dx_perm[pos[t,j]] + sum_s dx_perm[seg_offsets[E+s] + t], stored bf16.
    (The router's own contribution to dx is not part of this path.)"""
    R = _rounder(rnd)
    H = dx_perm.shape[1]
    p = np.asarray(pos, dtype=np.int64)
    acc = np.zeros((T, H))
    for j in range(p.shape[1] if p.ndim == 2 else 0):
        acc += dx_perm[p[:, j]]
    seg = np.asarray(seg_offsets, dtype=np.int64)
    for s in range(S):
        acc += dx_perm[seg[E + s]: seg[E + s] + T]
    return R(acc)


# ------------------------------------------------------------------------------------------------
# Router backward and the load-balancing bias update (TR section A2, load-balancing paragraph)
# ------------------------------------------------------------------------------------------------
def route_backward(probs, topk_idx, dtopk_w, normalize: bool = True) -> np.ndarray:
    """dlogits[T,E]: gradient of a loss with respect to the router logits, given dL/dw = dtopk_w.

    The routing weights depend on the logits only through the softmax probabilities p (the
    selection is piecewise constant, so it passes no gradient, and the selection bias, which the
    pages use only to pick the top-k, gets none). Two chain-rule steps, in float64:
      1. g = dL/dp, zero off the K selected experts. Renormalised weights w_j = p_{e_j} / S with
         S = sum_i p_{e_i}: dw_j/dp_{e_k} = (delta_jk - w_j) / S, so g_{e_k} = (dw_k - sum_j w_j
         dw_j) / S. Unnormalised weights w_j = p_{e_j}: g_{e_k} = dw_k.
      2. Softmax: dp_e/dz_f = p_e (delta_ef - p_f), so dz_f = p_f (g_f - sum_e p_e g_e).
    Rounded once to fp32.
    """
    p = np.asarray(probs, dtype=np.float32).astype(np.float64)
    idx = np.asarray(topk_idx, dtype=np.int64)
    dw = np.asarray(dtopk_w, dtype=np.float32).astype(np.float64)
    T, E = p.shape
    sel_p = np.take_along_axis(p, idx, axis=1)
    if normalize:
        S = sel_p.sum(axis=1, keepdims=True)
        w = sel_p / S
        g_sel = (dw - (w * dw).sum(axis=1, keepdims=True)) / S
    else:
        g_sel = dw
    g = np.zeros((T, E))
    np.put_along_axis(g, idx, g_sel, axis=1)
    dz = p * (g - (p * g).sum(axis=1, keepdims=True))
    return dz.astype(np.float32)


def router_weight_grad(dlogits, x_bits) -> np.ndarray:
    """dWg[E,H] = dlogits^T x (the logits are x . Wg^T), float64 rounded once to fp32."""
    dz = np.asarray(dlogits, dtype=np.float32).astype(np.float64)
    return (dz.T @ _as_values(x_bits)).astype(np.float32)


def router_input_grad(dlogits, w_gate) -> np.ndarray:
    """The router's share of dx: dlogits Wg [T,H], float64 rounded once to fp32."""
    dz = np.asarray(dlogits, dtype=np.float32).astype(np.float64)
    return (dz @ np.asarray(w_gate, dtype=np.float32).astype(np.float64)).astype(np.float32)


def balance_loss(probs, topk_idx, seq_len: int, alpha: float):
    """Sequence-wise balance loss and its gradient with respect to the router logits.

    The pages add a sequence-wise balance loss to keep any one sequence from routing too unevenly
    but give no formula. Reading (the form of the cited aux-loss-free method family): the batch is
    T / seq_len sequences of seq_len consecutive tokens; in each sequence
        f_e = E / (K * seq_len) * #{(t, j) in the sequence : topk_idx[t, j] = e}   (1 when balanced)
        P_e = mean over the sequence's tokens of p[t, e]
        L_seq = alpha * sum_e f_e P_e,
    and the batch loss is the mean of L_seq over the sequences. The selection counts f are piecewise
    constant in the logits, so the gradient flows through P only:
        dL/dp[t, e] = alpha f_e / (seq_len * n_seq), then through the softmax as in route_backward.
    Returns (per-sequence losses [n_seq] float64, dlogits [T,E] float64).
    """
    p = np.asarray(probs, dtype=np.float32).astype(np.float64)
    idx = np.asarray(topk_idx, dtype=np.int64)
    T, E = p.shape
    K = idx.shape[1]
    n_seq = T // seq_len
    losses = np.zeros(n_seq)
    dz = np.zeros((T, E))
    for q in range(n_seq):
        t0, t1 = q * seq_len, (q + 1) * seq_len
        f = np.bincount(idx[t0:t1].reshape(-1), minlength=E) * (E / (K * seq_len))
        P = p[t0:t1].mean(axis=0)
        losses[q] = alpha * float(f @ P)
        g = np.broadcast_to(alpha * f / (seq_len * n_seq), (seq_len, E))
        pq = p[t0:t1]
        dz[t0:t1] = pq * (g - (pq * g).sum(axis=1, keepdims=True))
    return losses, dz


def bias_update(sel_bias, counts, T: int, K: int, gamma: float) -> np.ndarray:
    """One step of the aux-loss-free balance: b_e + gamma * sign(mean load - c_e), in fp32.

    The pages say only that each expert's bias is adjusted during training to keep the load
    balanced. Reading (the update of the cited aux-loss-free method): an expert with fewer than
    the mean T*K/E routed tokens has its bias raised by the update speed gamma, one with more has
    it lowered, one at the mean keeps it. The comparison is exact in integers (T*K vs E*c_e) and
    the update is one fp32 addition.
    """
    b = np.asarray(sel_bias, dtype=np.float32)
    c = np.asarray(counts, dtype=np.int64)
    E = b.shape[0]
    sgn = np.sign(T * K - E * c).astype(np.float32)
    return (b + np.float32(gamma) * sgn).astype(np.float32)


# ------------------------------------------------------------------------------------------------
# Whole layer
# ------------------------------------------------------------------------------------------------
def moe_forward(x_bits, w1, w2, *, T, H, E, K, I, S, B, topk_idx=None, topk_w=None,
                w_gate=None, logit_bias=None, sel_bias=None, probs=None, normalize=True,
                rnd="bf16"):
    """Forward of the MoE FFN: route (unless topk_idx/topk_w are given), permute, experts, combine.

    Returns a dict with every intermediate the path stores.
    """
    out = {}
    if topk_idx is None:
        if probs is None:
            out["logits"] = router_logits(x_bits, w_gate, logit_bias)
            probs = softmax_probs(out["logits"])
        out["probs"] = probs
        topk_idx, topk_w = select_topk(probs, sel_bias, K, normalize)
    topk_idx = np.asarray(topk_idx, dtype=np.int32).reshape(T, K)
    out["topk_idx"], out["topk_w"] = topk_idx, np.asarray(topk_w, dtype=np.float32)
    out["expert_counts"] = expert_counts(topk_idx, E)
    Mcap = row_capacity(T, E, K, S, B)
    seg, tile_group, total = build_segments(out["expert_counts"], T, E, S, B, Mcap)
    row_token, pos = permute_maps(topk_idx, seg, T, E, S, Mcap)
    out.update(Mcap=Mcap, seg_offsets=seg, tile_group=tile_group, total_rows=total,
               row_token=row_token, pos=pos)
    x_perm = gather_rows(x_bits, row_token[:total])
    h, a, y_perm = expert_ffn_forward(x_perm, seg, w1, w2, I, rnd)
    out.update(x_perm=x_perm, h=h, a=a, y_perm=y_perm)
    out["y"] = combine(y_perm, pos, out["topk_w"], seg, T, E, S, rnd)
    return out


def moe_backward(fwd, dy, w1, w2, *, T, H, E, K, I, S, rnd="bf16"):
    """Backward of the MoE FFN with the forward's routing held fixed (dgrad and wgrad)."""
    seg, total = fwd["seg_offsets"], fwd["total_rows"]
    dy_perm, dtopk_w = combine_backward(dy, fwd["y_perm"], fwd["pos"], fwd["topk_w"], seg, total,
                                        T, E, S, rnd)
    dh, dx_perm = expert_ffn_dgrad(dy_perm, fwd["h"], seg, w1, w2, I, rnd)
    dw1, dw2 = expert_ffn_wgrad(fwd["x_perm"], fwd["a"], dy_perm, dh, seg, I, H, rnd)
    dx = unpermute_backward(dx_perm, fwd["pos"], seg, T, E, S, rnd)
    return dict(dy_perm=dy_perm, dtopk_w=dtopk_w, dh=dh, dx_perm=dx_perm, dw1=dw1, dw2=dw2, dx=dx)
