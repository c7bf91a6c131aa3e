"""Pins for the oracle's number handling and router arithmetic (CPU only)."""
import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle import moe_oracle as O
from synth import f32_to_bf16_bits, bf16_bits_to_f32
from tests import bruteforce as BF

h = float.fromhex


@pytest.mark.parametrize("v,expect", [
    (1.0, 1.0),
    (1 + 2**-8, 1.0),                      # exact tie, round to even (mantissa 0)
    (1 + 3 * 2**-8, 1 + 2**-6),            # exact tie, round to even (mantissa 2)
    (1 + 2**-8 + 2**-40, 1 + 2**-7),       # just above the tie
    (-(1 + 2**-8 + 2**-40), -(1 + 2**-7)),
    (h("0x1.fep127"), h("0x1.fep127")),    # largest finite bf16
    (h("0x1.ffp127"), math.inf),           # tie above the largest finite rounds to even = overflow
    (2.0**-133, 2.0**-133),                # smallest subnormal
    (2.0**-134, 0.0),                      # tie between 0 and 2^-133 -> even (0)
    (3 * 2.0**-134, 2.0**-132),            # tie between 1 and 2 units of 2^-133 -> 2
    (2.0**-126 * (1 + 2**-9), 2.0**-126),  # smallest normal binade
    (0.0, 0.0), (-0.0, -0.0), (math.inf, math.inf),
])
def test_round_bf16_known_values(v, expect):
    got = float(O.round_bf16(np.array([v]))[0])
    assert got == expect and math.copysign(1, got) == math.copysign(1, expect)


def test_round_bf16_nan():
    assert np.isnan(O.round_bf16(np.array([np.nan]))[0])


def test_round_bf16_matches_torch_on_fp32_inputs():
    # Library routine as a pin: torch's CPU float32 -> bfloat16 conversion is round-to-nearest-even.
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        rng.standard_normal(1000) * 2.0**-128]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_bf16(v.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_round_bf16_agrees_with_scalar_bruteforce():
    rng = np.random.default_rng(2)
    v = rng.standard_normal(3000) * 10.0 ** rng.integers(-5, 5, 3000)
    got = O.round_bf16(v)
    ref = np.array([BF.bf16_scalar(float(t)) for t in v])
    np.testing.assert_array_equal(got, ref)


def test_bf16_bits_roundtrip_and_generator_rounding():
    rng = np.random.default_rng(3)
    v = rng.standard_normal(5000).astype(np.float32)
    bits = f32_to_bf16_bits(v)
    np.testing.assert_array_equal(O.bf16_to_f64(bits), O.round_bf16(v.astype(np.float64)))
    np.testing.assert_array_equal(O.bf16_bits(O.bf16_to_f64(bits)), bits)
    np.testing.assert_array_equal(bf16_bits_to_f32(bits).astype(np.float64), O.bf16_to_f64(bits))


def test_router_logits_against_exact_sums():
    rng = np.random.default_rng(4)
    T, H, E = 5, 24, 6
    x = f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    wg = rng.standard_normal((E, H)).astype(np.float32)
    lb = rng.standard_normal(E).astype(np.float32)
    got = O.router_logits(x, wg, lb)
    xv = BF.bits_to_float(x)
    for t in range(T):
        for e in range(E):
            exact = math.fsum([float(a) * float(b) for a, b in zip(xv[t], wg[e])] + [float(lb[e])])
            assert got[t, e] == np.float32(exact)


def test_softmax_closed_forms():
    # Equal logits give 1/E; two experts give the logistic of the difference.
    E = 7
    p = O.softmax_probs(np.zeros((1, E), np.float32))
    np.testing.assert_array_equal(p, np.float32(1.0 / E))
    d = np.linspace(-20, 20, 41, dtype=np.float32)
    z = np.stack([d, np.zeros_like(d)], axis=1)
    p2 = O.softmax_probs(z)
    np.testing.assert_allclose(p2[:, 0], 1.0 / (1.0 + np.exp(-d.astype(np.float64))), rtol=1e-7)
    # Shift invariance and agreement with scipy's softmax.
    rng = np.random.default_rng(5)
    z = rng.standard_normal((50, 128)).astype(np.float32) * 4
    np.testing.assert_allclose(O.softmax_probs(z), scipy.special.softmax(z.astype(np.float64), axis=1),
                               rtol=1e-7, atol=0)
    zq = (rng.integers(-64, 64, (50, 128)) / 8).astype(np.float32)   # shifts by 64 stay exact
    np.testing.assert_array_equal(O.softmax_probs(zq + np.float32(64)), O.softmax_probs(zq))
    assert np.all(np.abs(O.softmax_probs(z).astype(np.float64).sum(1) - 1) < 1e-6)
