"""Plausible mistakes planted in the CPU oracle, each with the pins that must catch it.

Each mutant replaces one oracle function (in this process only) with a version that makes one
mistake a reimplementation could make: a dropped term, a wrong sign or index, a transposed
operand, a wrong tie rule. test_oracle_mutations.py runs the listed pin tests with the mutant
applied (in a subprocess, ORACLE_MUTANT=<name>) and requires them to fail; tests/conftest.py
applies the mutant named in the environment.
"""
from __future__ import annotations

import numpy as np

from oracle import moe_oracle as O

_ORIG = {name: getattr(O, name) for name in (
    "softmax_probs", "selection_keys", "select_topk", "expert_counts", "permute_maps",
    "expert_ffn_rows", "combine", "combine_backward", "swiglu_backward", "expert_ffn_dgrad",
    "expert_ffn_wgrad", "round_bf16", "route_backward", "router_weight_grad", "bias_update",
    "balance_loss")}


# --- routing --------------------------------------------------------------------------------------
def softmax_temperature(logits):
    # softmax of logits / 2
    return _ORIG["softmax_probs"](np.asarray(logits, np.float32) * np.float32(0.5))


def bias_ignored(probs, sel_bias):
    return _ORIG["selection_keys"](probs, None)


def bias_subtracted(probs, sel_bias):
    b = None if sel_bias is None else -np.asarray(sel_bias, np.float32)
    return _ORIG["selection_keys"](probs, b)


def weights_from_keys(probs, sel_bias, K, normalize=True):
    # selection as before, but the weights taken from p + b instead of p
    keys = _ORIG["selection_keys"](probs, sel_bias)
    idx, _ = _ORIG["select_topk"](probs, sel_bias, K, normalize)
    sel = np.take_along_axis(keys.astype(np.float64), idx, axis=1)
    w = sel / sel.sum(axis=1, keepdims=True) if normalize else sel
    return idx, w.astype(np.float32)


def ties_to_higher_index(probs, sel_bias, K, normalize=True):
    # reverse the expert axis, select, map back: equal keys now go to the higher index
    p = np.asarray(probs, np.float32)[:, ::-1]
    b = None if sel_bias is None else np.asarray(sel_bias, np.float32)[::-1]
    idx, w = _ORIG["select_topk"](np.ascontiguousarray(p), b if b is None else b.copy(), K, normalize)
    return (p.shape[1] - 1 - idx).astype(np.int32), w


def weights_not_renormalised(probs, sel_bias, K, normalize=True):
    return _ORIG["select_topk"](probs, sel_bias, K, False)


def counts_off_by_one(topk_idx, E):
    c = _ORIG["expert_counts"](topk_idx, E).copy()
    c[0] += 1
    return c


# --- permutation ----------------------------------------------------------------------------------
def segments_descending(topk_idx, seg_offsets, T, E, S, Mcap):
    # tokens inside each routed segment in descending instead of ascending order
    row_token, pos = _ORIG["permute_maps"](topk_idx, seg_offsets, T, E, S, Mcap)
    row_token, pos = row_token.copy(), pos.copy()
    seg = np.asarray(seg_offsets, np.int64)
    for e in range(E):
        r0, r1 = seg[e], seg[e + 1]
        used = r0 + int(np.sum(row_token[r0:r1] >= 0))
        if used - r0 < 2:
            continue
        old = row_token[r0:used].copy()
        row_token[r0:used] = old[::-1]
    # pos follows the rows: find each (token, slot) in its expert's segment again
    idx = np.asarray(topk_idx, np.int64)
    K = idx.shape[1]
    new_pos = np.full_like(pos, -1)
    for e in range(E):
        r0, r1 = seg[e], seg[e + 1]
        rows = {}
        for r in range(r0, r1):
            t = row_token[r]
            if t >= 0:
                rows.setdefault(int(t), []).append(r)
        for t, rs in rows.items():
            js = [j for j in range(K) if idx[t, j] == e]
            for j, r in zip(js, rs):
                new_pos[t, j] = r
    return row_token, new_pos


# --- forward ---------------------------------------------------------------------------------------
def swiglu_gate_up_swapped(x_rows, w1g, w2g, I, rnd="bf16"):
    # silu applied to the up half and multiplied by the gate half
    w = np.concatenate([w1g[I:], w1g[:I]], axis=0)
    h, a, y = _ORIG["expert_ffn_rows"](x_rows, w, w2g, I, rnd)
    return np.concatenate([h[:, I:], h[:, :I]], axis=1), a, y


def shared_experts_dropped(y_perm, pos, topk_w, seg_offsets, T, E, S, rnd="bf16"):
    return _ORIG["combine"](y_perm, pos, topk_w, seg_offsets, T, E, 0, rnd)


# --- backward --------------------------------------------------------------------------------------
def swiglu_bwd_missing_term(da, h, I):
    # dg without the g (1 - s) term of d silu / d g
    g, u = h[:, :I], h[:, I:]
    s = O.sigmoid(g)
    return np.concatenate([da * u * s, da * g * s], axis=1)


def swiglu_bwd_sign(da, h, I):
    d = _ORIG["swiglu_backward"](da, h, I)
    return np.concatenate([d[:, :I], -d[:, I:]], axis=1)


def dgrad_up_half_dropped(dy_perm, h, seg_offsets, w1, w2, I, rnd="bf16"):
    # dx_perm = dh W1 with the up half of W1 left out (W1 given as float64 values)
    w1m = np.asarray(w1, dtype=np.float64).copy()
    w1m[:, I:, :] = 0.0
    return _ORIG["expert_ffn_dgrad"](dy_perm, h, seg_offsets, w1m, w2, I, rnd)


def wgrad_gate_up_swapped(x_perm, a, dy_perm, dh, seg_offsets, I, H, rnd="bf16"):
    dhs = np.concatenate([dh[:, I:], dh[:, :I]], axis=1)
    return _ORIG["expert_ffn_wgrad"](x_perm, a, dy_perm, dhs, seg_offsets, I, H, rnd)


def dtopk_w_halved(*args, **kwargs):
    dy_perm, dw = _ORIG["combine_backward"](*args, **kwargs)
    return dy_perm, (dw * np.float32(0.5)).astype(np.float32)


def dy_perm_unweighted(dy_bits_or_vals, y_perm, pos, topk_w, *args, **kwargs):
    ones = np.ones_like(np.asarray(topk_w, np.float32))
    dy_perm, _ = _ORIG["combine_backward"](dy_bits_or_vals, y_perm, pos, ones, *args, **kwargs)
    _, dw = _ORIG["combine_backward"](dy_bits_or_vals, y_perm, pos, topk_w, *args, **kwargs)
    return dy_perm, dw


# --- router backward and bias update ---------------------------------------------------------------
def route_bwd_uncentred(probs, topk_idx, dtopk_w, normalize=True):
    # the renormalisation's -sum_j w_j dw_j term dropped (as if dw/dp were 1/S on the diagonal)
    p = np.asarray(probs, np.float32).astype(np.float64)
    idx = np.asarray(topk_idx, np.int64)
    dw = np.asarray(dtopk_w, np.float32).astype(np.float64)
    sel = np.take_along_axis(p, idx, axis=1)
    g_sel = dw / sel.sum(axis=1, keepdims=True) if normalize else dw
    g = np.zeros_like(p)
    np.put_along_axis(g, idx, g_sel, axis=1)
    return (p * (g - (p * g).sum(axis=1, keepdims=True))).astype(np.float32)


def route_bwd_no_softmax(probs, topk_idx, dtopk_w, normalize=True):
    # dL/dp returned as if it were dL/dz (softmax Jacobian skipped)
    p = np.asarray(probs, np.float32).astype(np.float64)
    idx = np.asarray(topk_idx, np.int64)
    dw = np.asarray(dtopk_w, np.float32).astype(np.float64)
    sel = np.take_along_axis(p, idx, axis=1)
    if normalize:
        S = sel.sum(axis=1, keepdims=True)
        g_sel = (dw - (sel / S * dw).sum(axis=1, keepdims=True)) / S
    else:
        g_sel = dw
    g = np.zeros_like(p)
    np.put_along_axis(g, idx, g_sel, axis=1)
    return g.astype(np.float32)


def router_weight_grad_mean(dlogits, x_bits):
    # averaged over the tokens instead of summed
    dw = _ORIG["router_weight_grad"](dlogits, x_bits)
    return (dw / np.float32(np.asarray(dlogits).shape[0])).astype(np.float32)


def balance_loss_summed(probs, topk_idx, seq_len, alpha):
    # gradient of the sum over sequences while the loss reported is their mean
    losses, dz = _ORIG["balance_loss"](probs, topk_idx, seq_len, alpha)
    return losses, dz * (np.asarray(probs).shape[0] // seq_len)


def balance_loss_raw_counts(probs, topk_idx, seq_len, alpha):
    # f as raw counts, without the E / (K seq_len) normalisation
    p = np.asarray(probs, np.float32)
    K = np.asarray(topk_idx).shape[1]
    scale = p.shape[1] / (K * seq_len)
    losses, dz = _ORIG["balance_loss"](probs, topk_idx, seq_len, alpha / scale)
    return losses, dz


def bias_update_sign_flipped(sel_bias, counts, T, K, gamma):
    return _ORIG["bias_update"](sel_bias, counts, T, K, -gamma)


# --- number format ---------------------------------------------------------------------------------
def round_toward_zero(v):
    # truncate to bf16 instead of rounding to nearest even
    x = np.asarray(v, dtype=np.float64)
    f = x.astype(np.float32)
    bits = (f.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)
    return np.where(np.isfinite(x), bits, x)


# name -> (oracle attribute, replacement, pin tests that must fail)
MUTANTS = {
    "softmax_temperature": ("softmax_probs", softmax_temperature,
                            ["test_oracle_numerics.py::test_softmax_closed_forms",
                             "test_oracle_routing.py::test_routing_golden"]),
    "bias_ignored": ("selection_keys", bias_ignored,
                     ["test_oracle_routing.py::test_routing_golden"]),
    "bias_subtracted": ("selection_keys", bias_subtracted,
                        ["test_oracle_routing.py::test_routing_golden"]),
    "weights_from_keys": ("select_topk", weights_from_keys,
                          ["test_oracle_routing.py::test_bias_only_changes_selection_not_weights",
                           "test_oracle_routing.py::test_routing_golden"]),
    "ties_to_higher_index": ("select_topk", ties_to_higher_index,
                             ["test_oracle_routing.py::test_all_equal_logits",
                              "test_oracle_routing.py::test_selection_equals_repeated_argmax",
                              "test_oracle_routing.py::test_routing_golden"]),
    "weights_not_renormalised": ("select_topk", weights_not_renormalised,
                                 ["test_oracle_routing.py::test_renormalised_weights_are_softmax_of_selected_logits",
                                  "test_oracle_routing.py::test_routing_golden"]),
    "counts_off_by_one": ("expert_counts", counts_off_by_one,
                          ["test_oracle_routing.py::test_expert_counts_sum",
                           "test_oracle_permute.py::test_maps_invariants_random_routing"]),
    "segments_descending": ("permute_maps", segments_descending,
                            ["test_oracle_permute.py::test_maps_invariants_random_routing"]),
    "swiglu_gate_up_swapped": ("expert_ffn_rows", swiglu_gate_up_swapped,
                               ["test_oracle_layer.py::test_layer_matches_per_token_bruteforce_c1",
                                "test_oracle_layer.py::test_swiglu_golden",
                                "test_oracle_layer.py::test_single_expert_is_the_dense_swiglu_ffn"]),
    "shared_experts_dropped": ("combine", shared_experts_dropped,
                               ["test_oracle_layer.py::test_layer_matches_per_token_bruteforce_c1",
                                "test_oracle_layer.py::test_combine_weights_and_shared_rows"]),
    "swiglu_bwd_missing_term": ("swiglu_backward", swiglu_bwd_missing_term,
                                ["test_oracle_backward.py::test_fd_dx_dw1_dw2_dw"]),
    "swiglu_bwd_sign": ("swiglu_backward", swiglu_bwd_sign,
                        ["test_oracle_backward.py::test_fd_dx_dw1_dw2_dw"]),
    "dgrad_up_half_dropped": ("expert_ffn_dgrad", dgrad_up_half_dropped,
                              ["test_oracle_backward.py::test_fd_dx_dw1_dw2_dw"]),
    "wgrad_gate_up_swapped": ("expert_ffn_wgrad", wgrad_gate_up_swapped,
                              ["test_oracle_backward.py::test_fd_dx_dw1_dw2_dw"]),
    "dtopk_w_halved": ("combine_backward", dtopk_w_halved,
                       ["test_oracle_backward.py::test_fd_dtopk_w"]),
    "dy_perm_unweighted": ("combine_backward", dy_perm_unweighted,
                           ["test_oracle_backward.py::test_fd_dx_dw1_dw2_dw"]),
    "route_bwd_uncentred": ("route_backward", route_bwd_uncentred,
                            ["test_oracle_route_bwd.py::test_route_backward_matches_autograd",
                             "test_oracle_route_bwd.py::test_route_backward_finite_differences"]),
    "route_bwd_no_softmax": ("route_backward", route_bwd_no_softmax,
                             ["test_oracle_route_bwd.py::test_route_backward_matches_autograd",
                              "test_oracle_route_bwd.py::test_route_backward_invariants"]),
    "router_weight_grad_mean": ("router_weight_grad", router_weight_grad_mean,
                                ["test_oracle_route_bwd.py::test_router_weight_and_input_grads_match_autograd"]),
    "bias_update_sign_flipped": ("bias_update", bias_update_sign_flipped,
                                 ["test_oracle_route_bwd.py::test_bias_update_hand_worked",
                                  "test_oracle_route_bwd.py::test_bias_update_is_one_fp32_add"]),
    "balance_loss_summed": ("balance_loss", balance_loss_summed,
                            ["test_oracle_route_bwd.py::test_balance_loss_gradient_matches_autograd",
                             "test_oracle_route_bwd.py::test_balance_loss_finite_differences"]),
    "balance_loss_raw_counts": ("balance_loss", balance_loss_raw_counts,
                                ["test_oracle_route_bwd.py::test_balance_loss_closed_forms"]),
    "round_toward_zero": ("round_bf16", round_toward_zero,
                          ["test_oracle_numerics.py::test_round_bf16_known_values",
                           "test_oracle_numerics.py::test_round_bf16_matches_torch_on_fp32_inputs"]),
}


def apply(name: str) -> None:
    attr, fn, _ = MUTANTS[name]
    setattr(O, attr, fn)
