"""Helpers shared by the GPU parity tests: host<->device transfers and the comparison bars.

Bars (written out here and in the tests that use them):
  * integer and index outputs, and copies: bit-exact;
  * bf16 GEMM outputs: relative L2 error <= 2e-2 over the whole tensor (the stated bar), and, to
    catch a localised fault that a global norm would hide, <= 2e-2 on every row and at most 0.1 %
    of elements further than 2^-6 relative + 2^-8 of the tensor's RMS from the oracle;
  * fp32 router logits: relative L2 <= 1e-5.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import moe_oracle as O

DEV = "cuda:0"


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns (host) -> bf16 device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(DEV).view(torch.bfloat16)


def f32_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def i32_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def bits_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def vals_host(t: torch.Tensor) -> np.ndarray:
    """bf16 device tensor -> float64 values (through the oracle's exact decoder)."""
    return O.bf16_to_f64(bits_host(t))


def rel_l2(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / den) if den > 0 else float(np.linalg.norm(got))


def assert_bf16_close(got, ref, name, tol=2e-2, row_axis=-1):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    if ref.size == 0:
        return
    r = rel_l2(got, ref)
    assert r <= tol, f"{name}: rel-L2 {r:.3e} > {tol}"
    g2 = got.reshape(-1, got.shape[row_axis]) if got.ndim > 1 else got[None]
    r2 = ref.reshape(-1, ref.shape[row_axis]) if ref.ndim > 1 else ref[None]
    num = np.linalg.norm(g2 - r2, axis=1)
    den = np.linalg.norm(r2, axis=1)
    zero = den == 0
    assert np.all(num[zero] == 0), f"{name}: rows that must be zero are not"
    worst = float(np.max(num[~zero] / den[~zero])) if (~zero).any() else 0.0
    assert worst <= tol, f"{name}: worst row rel-L2 {worst:.3e} > {tol}"
    rms = float(np.sqrt(np.mean(ref ** 2)))
    far = np.abs(got - ref) > 2.0 ** -6 * np.abs(ref) + 2.0 ** -8 * rms
    assert far.mean() <= 1e-3, f"{name}: {far.sum()} elements ({far.mean():.2e}) off"
    log(f"  {name}: rel-L2 {r:.2e}, worst row {worst:.2e}, far {int(far.sum())}")


def validated_routing(idx_gpu, probs_ref, sel_bias, K, delta=1e-6, normalize=True):
    """The oracle's routing with every near-tied token taken as the GPU chose it, once that choice
    is shown to be valid.

    A token whose oracle margin between the K-th and (K+1)-th key is at least ``delta`` must match
    the oracle exactly. Elsewhere the GPU's experts must be K distinct ones, each keyed within
    ``delta`` of the oracle's K-th key, in slots whose keys do not increase by more than ``delta``.
    Returns (idx, w, mism): the selection (the oracle's, with those valid alternatives), the
    oracle's weights of that selection (the affinities p renormalised over the chosen experts),
    and the mask of tokens that took an alternative. Every expected map and row of a test is then
    built by the oracle from ``idx``."""
    idx_gpu = np.asarray(idx_gpu)
    key = O.selection_keys(probs_ref, sel_bias).astype(np.float64)
    key = np.nan_to_num(key, nan=-np.inf)
    ref_idx, _ = O.select_topk(probs_ref, sel_bias, K, normalize)
    T, E = key.shape
    srt = -np.sort(-key, axis=1)
    margin = srt[:, K - 1] - (srt[:, K] if K < E else -np.inf)
    mism = np.any(idx_gpu != ref_idx, axis=1)
    assert not np.any(mism & (margin >= delta)), \
        f"{int((mism & (margin >= delta)).sum())} tokens with a decided ranking differ"
    for t in np.nonzero(mism)[0]:
        row = idx_gpu[t]
        assert np.all((row >= 0) & (row < E)) and len(set(row.tolist())) == K, (t, row)
        chosen = key[t, row]
        assert chosen.min() >= srt[t, K - 1] - delta, (t, row)
        assert np.all(np.diff(chosen) <= delta), (t, row)
    idx = ref_idx.copy()
    idx[mism] = idx_gpu[mism]
    log(f"  routing: {int(mism.sum())} of {T} tokens took a valid near-tie alternative "
        f"({int((margin < delta).sum())} with margin < {delta})")
    return idx, O.combine_weights(probs_ref, idx, normalize), mism
