"""Pins for the oracle's biased top-k selection and combine weights (CPU only)."""
import json
import math
import os

import numpy as np
import pytest

from oracle import moe_oracle as O
from synth import draw_probs, draw_logits
from tests import bruteforce as BF

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_cases():
    with open(os.path.join(GOLDEN, "routing_hand.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_routing_golden(case):
    ratios = np.array(case["ratios"], dtype=np.float64)
    logits = np.log(ratios).astype(np.float32)[None, :]
    b = np.array([float(v) for v in case["sel_bias"]], dtype=np.float32)
    p = O.softmax_probs(logits)
    np.testing.assert_allclose(p[0], case["probs"], rtol=1e-6)
    idx, w = O.select_topk(p, b, case["K"], case["normalize"])
    assert idx[0].tolist() == case["topk_idx"]
    np.testing.assert_allclose(w[0], case["topk_w"], rtol=0, atol=1e-6)
    if "keys" in case:
        np.testing.assert_allclose(O.selection_keys(p, b)[0], case["keys"], rtol=1e-6)


@pytest.mark.parametrize("levels", [0, 3, 8])
@pytest.mark.parametrize("normalize", [True, False])
def test_selection_equals_repeated_argmax(levels, normalize):
    # A different algorithm (K rounds of arg-max with an upward scan) must give the same slots.
    T, E, K = 200, 12, 4
    p = draw_probs(T, E, seed=11 + levels, levels=levels)
    b = (np.random.default_rng(levels).integers(-2, 3, E) / 16).astype(np.float32)
    idx, w = O.select_topk(p, b, K, normalize)
    key = O.selection_keys(p, b)
    for t in range(T):
        ref = BF.pick_topk([float(k) for k in key[t]], K)
        assert idx[t].tolist() == ref
        sp = p[t, ref].astype(np.float64)
        ref_w = sp / sp.sum() if normalize else sp
        np.testing.assert_allclose(w[t], ref_w, rtol=0, atol=1e-7)


def test_selection_with_nan_and_signed_zero():
    p = np.array([[0.0, 0.5, np.nan, 0.5, 0.0, np.nan]], dtype=np.float32)
    b = np.array([-0.0, 0.0, 0.0, 0.0, 0.0, 0.0], dtype=np.float32)
    idx, _ = O.select_topk(p, b, 6, normalize=False)
    # numbers first (0.5 at 1 and 3, then the zeros at 0 and 4), then the NaNs by index
    assert idx[0].tolist() == [1, 3, 0, 4, 2, 5]
    key = O.selection_keys(p, b)[0]
    assert BF.pick_topk([float(k) for k in key], 6) == [1, 3, 0, 4, 2, 5]


def test_selection_is_a_full_sort_prefix():
    T, E, K = 300, 16, 5
    p = draw_probs(T, E, seed=3, levels=5)
    b = np.zeros(E, np.float32)
    idx, _ = O.select_topk(p, b, K)
    idx_all, _ = O.select_topk(p, b, E, normalize=False)
    np.testing.assert_array_equal(idx, idx_all[:, :K])
    key = O.selection_keys(p, b)
    for t in range(T):
        s = sorted(range(E), key=lambda e: (-float(key[t, e]), e))
        assert idx_all[t].tolist() == s


def test_all_equal_logits():
    T, E, K = 4, 10, 3
    idx, w = O.select_topk(O.softmax_probs(np.zeros((T, E), np.float32)), np.zeros(E, np.float32), K)
    np.testing.assert_array_equal(idx, np.tile(np.arange(K), (T, 1)))
    np.testing.assert_allclose(w, 1.0 / K, atol=1e-7)


def test_renormalised_weights_are_softmax_of_selected_logits():
    # Closed form: p_e / sum_sel p = exp(z_e) / sum_sel exp(z), computed here from the logits alone.
    T, E, K = 500, 128, 6
    z = draw_logits(T, E, seed=9, scale=2.0)
    b = np.random.default_rng(0).uniform(-0.01, 0.01, E).astype(np.float32)
    idx, w = O.select_topk(O.softmax_probs(z), b, K)
    zs = np.take_along_axis(z.astype(np.float64), idx.astype(np.int64), axis=1)
    ref = np.exp(zs - zs.max(1, keepdims=True))
    ref /= ref.sum(1, keepdims=True)
    np.testing.assert_allclose(w, ref, rtol=0, atol=1e-6)
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) < 1e-6)


def test_bias_only_changes_selection_not_weights():
    T, E, K = 400, 32, 4
    p = O.softmax_probs(draw_logits(T, E, seed=5))
    b0 = np.zeros(E, np.float32)
    idx0, w0 = O.select_topk(p, b0, K)
    # A uniform shift of every bias keeps each token's ranking up to rounding of p + b; where the
    # selection is unchanged the weights must be bit-identical.
    b1 = np.full(E, 0.125, np.float32)
    idx1, w1 = O.select_topk(p, b1, K)
    same = np.all(np.sort(idx0, 1) == np.sort(idx1, 1), axis=1)
    assert same.mean() > 0.99
    for t in np.nonzero(same)[0]:
        m0 = dict(zip(idx0[t].tolist(), w0[t].tolist()))
        m1 = dict(zip(idx1[t].tolist(), w1[t].tolist()))
        assert m0 == m1
    # A large negative bias removes an expert from every selection.
    b2 = b0.copy()
    b2[[0, 5]] = -10.0
    idx2, _ = O.select_topk(p, b2, K)
    assert not np.isin(idx2, [0, 5]).any()


def test_expert_counts_sum():
    T, E, K = 1000, 20, 3
    p = draw_probs(T, E, seed=1)
    idx, _ = O.select_topk(p, None, K)
    c = O.expert_counts(idx, E)
    assert c.sum() == T * K
    for e in range(E):
        assert c[e] == int((idx == e).sum())
