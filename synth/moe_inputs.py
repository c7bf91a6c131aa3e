"""Seeded synthetic inputs for the MoE feed-forward path (data only, no method arithmetic).

Every tensor comes from its own NumPy stream ``default_rng([seed, tag, index])``, so one slice of a
workload (the weights of one expert, one block of tokens) can be regenerated without drawing the
rest. bf16 tensors are returned as their uint16 bit patterns, rounded from float32 draws with
round-to-nearest-even; fp32 tensors are float32 arrays.

The workloads follow the dots.llm1 MoE layer: 128 routed experts with top-6 selection plus 2
shared experts, expert intermediate 1408 (dots.llm1 Technical Report, section A2 "Architecture",
mixture-of-experts paragraph). Value distributions: weights N(0,1)/sqrt(fan_in), activations
N(0,1), upstream gradients N(0, 1e-2).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

__all__ = [
    "MoEConfig", "CONFIGS", "get_config",
    "f32_to_bf16_bits", "bf16_bits_to_f32",
    "draw_x", "draw_wg", "draw_sel_bias", "draw_logit_bias", "draw_w1", "draw_w2",
    "draw_w1_all", "draw_w2_all", "draw_dy", "draw_topk_given", "draw_probs", "draw_logits",
    "uniform_topk", "uniform_logits", "skewed_logits", "num_groups",
]

# Stream tags: one per tensor kind.
TAG_X, TAG_WG, TAG_SEL, TAG_W1, TAG_W2, TAG_DY, TAG_TOPK, TAG_PROBS, TAG_LOGITS = range(1, 10)
ROW_CHUNK = 1024  # token rows per stream for x and dy


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    H: int
    E: int
    K: int
    I: int
    S: int
    block_m: int
    seed: int
    routing: str = "router"      # "router" (x . Wg -> softmax -> biased top-k) or "uniform"
    logit_bias: str = "none"     # "none" or "zipf" (per-expert offsets -s*ln(e+1), s = 1.1)
    sel_bias: str = "zero"       # "zero", "uniform0.1" or "forced_empty"
    forced_empty: tuple = field(default=())  # experts whose selection bias is -10

    @property
    def G(self) -> int:
        return self.E + self.S


def num_groups(cfg: MoEConfig) -> int:
    return cfg.E + cfg.S


CONFIGS = {
    # Tiny layer forward: the size the oracle and the brute-force checker finish in well under a second.
    "c1": MoEConfig("c1", T=64, H=256, E=8, K=2, I=128, S=1, block_m=16, seed=0,
                    routing="router", sel_bias="uniform0.1"),
    # Grouped GEMM with uniform routing: 49152 rows, exactly 384 per expert.
    "c2": MoEConfig("c2", T=8192, H=4096, E=128, K=6, I=1408, S=0, block_m=128, seed=0,
                    routing="uniform"),
    # Full layer, router with Zipf(1.1)-skewed per-expert logit offsets and two shared experts.
    "c3": MoEConfig("c3", T=16384, H=4096, E=128, K=6, I=1408, S=2, block_m=128, seed=0,
                    routing="router", logit_bias="zipf"),
    # Backward at the c2 shapes (upstream gradient N(0, 1e-2)).
    "c4": MoEConfig("c4", T=8192, H=4096, E=128, K=6, I=1408, S=0, block_m=128, seed=0,
                    routing="uniform"),
    # Decode-sized sparse layer.
    "c5": MoEConfig("c5", T=256, H=4096, E=128, K=6, I=1408, S=2, block_m=16, seed=7,
                    routing="router"),
    # A dense SwiGLU FFN (the model's first layer) run as one group: E = K = 1. The pages do not give
    # its width; the reading is the active experts' total width per token, 8 x 1408 = 11264.
    "dense": MoEConfig("dense", T=8192, H=4096, E=1, K=1, I=11264, S=0, block_m=128, seed=0,
                       routing="uniform"),
    # One GPU's share of c2 under 8-way expert parallelism: its 16 local experts receive
    # 8 x 8192 x 6 / 128 = 3072 rows each, modelled as 8192 local tokens routed top-6 uniformly
    # over the 16 experts (the GEMMs see exactly that shape; the exchange itself is not modelled).
    "ep8": MoEConfig("ep8", T=8192, H=4096, E=16, K=6, I=1408, S=0, block_m=128, seed=0,
                     routing="uniform"),
    # The c4 training step with Zipf(1.1)-skewed routing (a router early in training, before the
    # bias balances the load): expert popularity ~ rank^-1.1, K distinct experts per token.
    "c4z": MoEConfig("c4z", T=8192, H=4096, E=128, K=6, I=1408, S=0, block_m=128, seed=0,
                     routing="zipf"),
    # Decode with 16 experts forced empty by a -10 selection bias (empty-group skipping).
    "c5e": MoEConfig("c5e", T=256, H=4096, E=128, K=6, I=1408, S=2, block_m=16, seed=7,
                     routing="router", sel_bias="forced_empty",
                     forced_empty=tuple(range(7, 128, 8))),
}


def get_config(name: str, **overrides) -> MoEConfig:
    cfg = CONFIGS[name]
    return replace(cfg, **overrides) if overrides else cfg


# ----------------------------------------------------------------------------------------------
# bf16 bit patterns
# ----------------------------------------------------------------------------------------------
def f32_to_bf16_bits(a) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest, ties to even; NaN -> quiet NaN 0x7fc0."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _rng(seed: int, tag: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(tag), int(index)])


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ----------------------------------------------------------------------------------------------
# Activations and gradients (row-chunked streams)
# ----------------------------------------------------------------------------------------------
def _rows_bf16(seed, tag, T, H, scale, rows=None) -> np.ndarray:
    """[T,H] (or the selected rows) of N(0, scale^2) rounded to bf16 bits."""
    if rows is None:
        out = np.empty((T, H), dtype=np.uint16)
        chunks = range((T + ROW_CHUNK - 1) // ROW_CHUNK)

        def fill(c):
            r0 = c * ROW_CHUNK
            n = min(ROW_CHUNK, T - r0)
            v = _rng(seed, tag, c).standard_normal((ROW_CHUNK, H), dtype=np.float32)[:n]
            out[r0:r0 + n] = f32_to_bf16_bits(v * np.float32(scale))

        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, chunks))
        return out
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows), H), dtype=np.uint16)
    cache = {}
    for i, r in enumerate(rows):
        c = int(r) // ROW_CHUNK
        if c not in cache:
            cache[c] = _rng(seed, tag, c).standard_normal((ROW_CHUNK, H), dtype=np.float32)
        out[i] = f32_to_bf16_bits(cache[c][int(r) % ROW_CHUNK] * np.float32(scale))
    return out


def draw_x(cfg: MoEConfig, rows=None) -> np.ndarray:
    """Token activations x [T,H], bf16 bits, N(0,1)."""
    return _rows_bf16(cfg.seed, TAG_X, cfg.T, cfg.H, 1.0, rows)


def draw_dy(cfg: MoEConfig, rows=None) -> np.ndarray:
    """Upstream gradient of the layer output dy [T,H], bf16 bits, N(0, 1e-2)."""
    return _rows_bf16(cfg.seed, TAG_DY, cfg.T, cfg.H, 1e-2, rows)


# ----------------------------------------------------------------------------------------------
# Router parameters
# ----------------------------------------------------------------------------------------------
def draw_wg(cfg: MoEConfig) -> np.ndarray:
    """Router weight Wg [E,H], float32, N(0,1)/sqrt(H)."""
    v = _rng(cfg.seed, TAG_WG).standard_normal((cfg.E, cfg.H), dtype=np.float32)
    return (v * np.float32(1.0 / math.sqrt(cfg.H))).astype(np.float32)


def draw_sel_bias(cfg: MoEConfig) -> np.ndarray:
    """Per-expert selection bias b [E], float32."""
    if cfg.sel_bias == "uniform0.1":
        return _rng(cfg.seed, TAG_SEL).uniform(-0.1, 0.1, cfg.E).astype(np.float32)
    b = np.zeros(cfg.E, dtype=np.float32)
    if cfg.sel_bias == "forced_empty":
        b[list(cfg.forced_empty)] = np.float32(-10.0)
    elif cfg.sel_bias != "zero":
        raise ValueError(cfg.sel_bias)
    return b


def draw_logit_bias(cfg: MoEConfig):
    """Per-expert additive logit offsets [E] or None. 'zipf': -1.1*ln(e+1) (popularity ~ rank^-1.1)."""
    if cfg.logit_bias == "none":
        return None
    if cfg.logit_bias == "zipf":
        e = np.arange(cfg.E, dtype=np.float64)
        return (-1.1 * np.log(e + 1.0)).astype(np.float32)
    raise ValueError(cfg.logit_bias)


# ----------------------------------------------------------------------------------------------
# Expert weights (one stream per group so a single expert can be regenerated)
# ----------------------------------------------------------------------------------------------
def draw_w1(cfg: MoEConfig, g: int) -> np.ndarray:
    """Gate/up weight of group g, [2I, H] bf16 bits (rows 0..I-1 gate, I..2I-1 up), N(0,1)/sqrt(H)."""
    v = _rng(cfg.seed, TAG_W1, g).standard_normal((2 * cfg.I, cfg.H), dtype=np.float32)
    return f32_to_bf16_bits(v * np.float32(1.0 / math.sqrt(cfg.H)))


def draw_w2(cfg: MoEConfig, g: int) -> np.ndarray:
    """Down weight of group g, [H, I] bf16 bits, N(0,1)/sqrt(I)."""
    v = _rng(cfg.seed, TAG_W2, g).standard_normal((cfg.H, cfg.I), dtype=np.float32)
    return f32_to_bf16_bits(v * np.float32(1.0 / math.sqrt(cfg.I)))


def _all_groups(cfg, fn, shape) -> np.ndarray:
    out = np.empty((cfg.G,) + shape, dtype=np.uint16)

    def fill(g):
        out[g] = fn(cfg, g)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(cfg.G)))
    return out


def draw_w1_all(cfg: MoEConfig) -> np.ndarray:
    return _all_groups(cfg, draw_w1, (2 * cfg.I, cfg.H))


def draw_w2_all(cfg: MoEConfig) -> np.ndarray:
    return _all_groups(cfg, draw_w2, (cfg.H, cfg.I))


# ----------------------------------------------------------------------------------------------
# Routing inputs for stage-level tests
# ----------------------------------------------------------------------------------------------
def uniform_topk(T: int, E: int, K: int) -> np.ndarray:
    """Uniform routing: slot j of token t goes to expert (K*t + j) mod E.

    (t, j) -> K*t + j is a bijection onto 0..T*K-1, so each expert receives exactly T*K/E rows when
    E divides T*K, and a token's K experts are K consecutive residues, hence distinct when K <= E.
    """
    t = np.arange(T, dtype=np.int64)[:, None]
    j = np.arange(K, dtype=np.int64)[None, :]
    return ((K * t + j) % E).astype(np.int32)


def uniform_logits(cfg: MoEConfig) -> np.ndarray:
    """Router logits [T,E] float32 whose top-K experts are exactly the uniform assignment.

    N(0,1) noise everywhere plus +16 on the token's K assigned experts; the host checks that every
    assigned logit exceeds every other logit of its row, so any monotone score keeps the set.
    """
    idx = uniform_topk(cfg.T, cfg.E, cfg.K)
    v = _rng(cfg.seed, TAG_LOGITS).standard_normal((cfg.T, cfg.E), dtype=np.float32)
    rows = np.arange(cfg.T)[:, None]
    v[rows, idx] += np.float32(16.0)
    mask = np.zeros_like(v, dtype=bool)
    mask[rows, idx] = True
    lo_sel = np.where(mask, v, np.inf).min(axis=1)
    hi_rest = np.where(mask, -np.inf, v).max(axis=1)
    assert np.all(lo_sel > hi_rest + 1.0), "uniform_logits: assignment margin too small"
    return v


def skewed_logits(cfg: MoEConfig, skew: float = 1.1) -> np.ndarray:
    """Router logits [T,E] float32 whose top-K experts are a Zipf(skew) routing (draw_topk_given
    with the config's seed): N(0,1) noise plus +16 on the token's K chosen experts, as in
    uniform_logits."""
    idx = draw_topk_given(cfg.T, cfg.E, cfg.K, cfg.seed, skew)
    v = _rng(cfg.seed, TAG_LOGITS).standard_normal((cfg.T, cfg.E), dtype=np.float32)
    rows = np.arange(cfg.T)[:, None]
    v[rows, idx] += np.float32(16.0)
    mask = np.zeros_like(v, dtype=bool)
    mask[rows, idx] = True
    lo_sel = np.where(mask, v, np.inf).min(axis=1)
    hi_rest = np.where(mask, -np.inf, v).max(axis=1)
    assert np.all(lo_sel > hi_rest + 1.0), "skewed_logits: assignment margin too small"
    return v


def draw_topk_given(T: int, E: int, K: int, seed: int, skew: float = 1.1,
                    forced_empty=()) -> np.ndarray:
    """Random routing [T,K] int32 with K distinct experts per token, popularity ~ rank^-skew.

    Gumbel-top-K over log-popularities (sampling without replacement); experts in forced_empty are
    never chosen. Used as a given routing for permutation and combine tests.
    """
    rng = _rng(seed, TAG_TOPK)
    logp = -skew * np.log(np.arange(1, E + 1, dtype=np.float64))
    if len(forced_empty):
        logp[list(forced_empty)] = -np.inf
    g = rng.gumbel(size=(T, E))
    keys = logp[None, :] + g
    idx = np.argsort(-keys, axis=1, kind="stable")[:, :K]
    return idx.astype(np.int32)


def draw_probs(T: int, E: int, seed: int, levels: int = 0) -> np.ndarray:
    """Routing probabilities [T,E] float32, rows summing to about 1.

    levels > 0 quantises each row's values to multiples of 1/levels before normalising, so equal
    values (ties) are common.
    """
    rng = _rng(seed, TAG_PROBS)
    v = rng.exponential(size=(T, E))
    if levels:
        v = np.floor(v * levels / v.max(axis=1, keepdims=True))
        v[:, 0] += 1.0  # no all-zero row
    v = v / v.sum(axis=1, keepdims=True)
    return v.astype(np.float32)


def draw_logits(T: int, E: int, seed: int, scale: float = 1.0) -> np.ndarray:
    """Router logits [T,E] float32, N(0, scale^2)."""
    return (_rng(seed, TAG_LOGITS, 1).standard_normal((T, E), dtype=np.float32)
            * np.float32(scale)).astype(np.float32)
