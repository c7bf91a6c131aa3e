"""Pins for the oracle's block-aligned segments and permutation maps (CPU only)."""
import itertools

import numpy as np
import pytest

from oracle import moe_oracle as O
from synth import draw_topk_given, uniform_topk


def _check_maps(idx, T, E, K, S, B):
    Mcap = O.row_capacity(T, E, K, S, B)
    c = O.expert_counts(idx, E)
    seg, tg, total = O.build_segments(c, T, E, S, B, Mcap)
    row_token, pos = O.permute_maps(idx, seg, T, E, S, Mcap)
    G = E + S
    assert Mcap % B == 0 and total <= Mcap
    assert c.sum() == T * K
    assert seg[0] == 0 and np.all(seg % B == 0) and np.all(np.diff(seg) >= 0)
    sizes = list(c) + [T] * S
    for g in range(G):
        n = seg[g + 1] - seg[g]
        assert n == -(-sizes[g] // B) * B                       # padded to a multiple of B
        rows = row_token[seg[g]:seg[g + 1]]
        real = rows[:sizes[g]]
        assert np.all(rows[sizes[g]:] == -1)                     # padding rows
        assert np.all(np.diff(real) > 0)                          # ascending tokens
        if g < E:
            assert set(real.tolist()) == set(np.nonzero((idx == g).any(1))[0].tolist())
        else:
            np.testing.assert_array_equal(real, np.arange(T))
    assert np.all(row_token[total:] == -1)
    # pos is a bijection from (t, j) onto the routed non-padding rows and row_token inverts it.
    flat = pos.reshape(-1)
    assert len(set(flat.tolist())) == T * K
    for t in range(T):
        for j in range(K):
            r = pos[t, j]
            assert row_token[r] == t and seg[idx[t, j]] <= r < seg[idx[t, j] + 1]
    # tile_group by a direct scan of the offsets
    for i in range(Mcap // B):
        r = i * B
        expect = -1
        for g in range(G):
            if seg[g] <= r < seg[g + 1]:
                expect = g
        assert tg[i] == expect
    return seg, total, Mcap


@pytest.mark.parametrize("T,E,K,S,B", [(64, 8, 2, 1, 16), (100, 16, 4, 2, 32), (37, 5, 5, 0, 16),
                                       (1, 4, 1, 1, 16), (300, 128, 6, 2, 128)])
def test_maps_invariants_random_routing(T, E, K, S, B):
    idx = draw_topk_given(T, E, K, seed=T + E)
    _check_maps(idx, T, E, K, S, B)


def test_uniform_routing_has_no_padding():
    T, E, K, B = 8192, 128, 6, 128
    idx = uniform_topk(T, E, K)
    assert np.all(O.expert_counts(idx, E) == 384)
    assert all(len(set(r)) == K for r in idx[:200].tolist())
    Mcap = O.row_capacity(T, E, K, 0, B)
    seg, tg, total = O.build_segments(O.expert_counts(idx, E), T, E, 0, B, Mcap)
    assert total == T * K and np.all(np.diff(seg) == 384)


def test_forced_empty_experts_have_empty_segments():
    T, E, K, S, B = 200, 16, 3, 1, 16
    idx = draw_topk_given(T, E, K, seed=2, forced_empty=(3, 7, 15))
    seg, total, Mcap = _check_maps(idx, T, E, K, S, B)
    for e in (3, 7, 15):
        assert seg[e + 1] == seg[e]


def test_all_tokens_on_the_same_experts_and_empty_input():
    T, E, K, S, B = 50, 8, 3, 2, 16
    idx = np.tile(np.array([5, 0, 2], np.int32), (T, 1))
    seg, total, _ = _check_maps(idx, T, E, K, S, B)
    assert total == 3 * 64 + 2 * 64
    T = 0
    idx = np.zeros((0, K), np.int32)
    assert O.row_capacity(T, E, K, S, B) == 0
    seg, tg, total = O.build_segments(O.expert_counts(idx, E), T, E, S, B, 0)
    assert total == 0 and np.all(seg == 0)


def test_capacity_bounds_every_count_vector():
    # Brute force over every way to spread R rows over E experts (tiny sizes): padded total <= cap.
    for T, E, K, B in [(3, 3, 2, 4), (4, 4, 2, 2), (5, 3, 1, 4)]:
        R = T * K
        cap = O.row_capacity(T, E, K, 0, B)
        worst = 0
        for c in itertools.product(range(R + 1), repeat=E):
            if sum(c) != R or max(c) > T:
                continue
            worst = max(worst, sum(-(-ci // B) * B for ci in c))
        assert worst <= cap
