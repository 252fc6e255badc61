"""Seeded synthetic inputs for one draft-tree construction round.

This module only draws random numbers and packs them into the layouts the
library consumes. It holds none of the method's arithmetic, so both the HIP
path and the CPU oracle can take their inputs from it.

Workload shapes follow the DARTree pages (marsggbo blog, section 3.1: top-K
candidates per block position with K=64 by default, per-depth width W=12 or
4, global budget B=64; section 4.4: concurrency C=4 with B=32, W=3; the
AINews summary: a 16-token block from the drafter). The vocabulary size is
Qwen3's (151936). The correction head is not defined on the pages; the
stand-in used here is a low-rank recurrent head:

    root state      s_0 = h_0
    child state     s   = tanh(A s_parent + E[u] + h_d)      (d = child depth)
    corrected logit z_c = Lbase_d[c] + <s_parent, U[c]>,  log-softmax over
                          the K candidates of that depth

with h_d = P^T H_d, H_d the drafter's hidden state at block position d.

Conventions shared by both sides (layouts, not arithmetic):
  * logits[n][L][V]: row i is the base logit vector of depth i+1.
  * H[n][L][D] (bf16 bits) or h[n][L][r] (fp32, when D == 0): row d feeds
    the states of depth-d nodes (row 0 is the root state).
  * weights: A[r][r] (A[j][m] multiplies s[m] into output j), E[V][r],
    U[V][r], Pt[r][D] (the projection stored output-major: Pt[j][i] = P[i][j]).
  * bf16 tensors are carried as uint16 bit patterns, rounded from fp32
    with round-to-nearest-even.

Random streams: round t of config c under seed s is drawn from
``np.random.default_rng([s, c, t])``; the head from
``np.random.default_rng([s, c, 2**32 - 1])``. Draw order is fixed and
documented in each function.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

HEAD_STREAM = 2**32 - 1

F32 = "f32"
BF16 = "bf16"


@dataclass(frozen=True)
class Config:
    """One workload: tree-construction hyper-parameters plus input recipe."""

    name: str
    cfg_id: int
    n_req: int
    V: int
    L: int
    K: int
    W: int
    B: int
    beta: float
    r: int
    D: int                  # 0: h is supplied directly (no projection)
    logits_dtype: str       # "f32" | "bf16"
    weight_dtype: str       # "f32" | "bf16"
    sigma: float = 2.0      # std of the base-logit noise
    n_boost: int = 32       # boosted ids per (request, position)
    boost_lo: float = 4.0
    boost_hi: float = 12.0
    decay: float = 0.9      # boost multiplier decay**d, d = 1-based depth
    temperature: float = 1.0

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


# The five workloads. Sizes: V=151936 is the Qwen3 vocabulary; L=16 the
# drafter block; K/W/B/beta from the blog's section 3.1 and 4.4.
CONFIGS = {
    "tiny": Config("tiny", 0, n_req=1, V=1024, L=6, K=8, W=3, B=16, beta=-0.1, r=16, D=0,
                   logits_dtype=F32, weight_dtype=F32, sigma=2.0, n_boost=8, decay=0.9),
    "qwen3_4b": Config("qwen3_4b", 1, n_req=1, V=151936, L=16, K=64, W=12, B=64, beta=-0.15,
                       r=256, D=2560, logits_dtype=BF16, weight_dtype=BF16, sigma=2.0,
                       n_boost=32, decay=0.9),
    "fixed_w4_qwen3_8b": Config("fixed_w4_qwen3_8b", 2, n_req=1, V=151936, L=16, K=64, W=4, B=64,
                                beta=-0.1, r=256, D=4096, logits_dtype=BF16, weight_dtype=BF16,
                                sigma=2.0, n_boost=32, decay=0.85),
    "concurrent_c4": Config("concurrent_c4", 3, n_req=4, V=151936, L=16, K=64, W=3, B=32,
                            beta=-0.2, r=256, D=2560, logits_dtype=BF16, weight_dtype=BF16,
                            sigma=3.0, n_boost=32, decay=0.9, temperature=1.0),
    "stress_64req": Config("stress_64req", 4, n_req=64, V=151936, L=16, K=512, W=12, B=64,
                           beta=-0.2, r=512, D=4096, logits_dtype=BF16, weight_dtype=BF16,
                           sigma=2.0, n_boost=32, decay=0.9),
}
CONFIG_ORDER = ["tiny", "qwen3_4b", "fixed_w4_qwen3_8b", "concurrent_c4", "stress_64req"]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32 values."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x32) if dtype == BF16 else np.ascontiguousarray(x32, dtype=np.float32)


@dataclass
class Head:
    """Correction-head weights in their storage dtype (uint16 bits or fp32)."""

    A: np.ndarray           # [r][r]
    E: np.ndarray           # [V][r]
    U: np.ndarray           # [V][r]
    Pt: Optional[np.ndarray]  # [r][D] or None when D == 0
    dtype: str


@dataclass
class Round:
    """Per-round drafter outputs in storage dtype."""

    logits: np.ndarray      # [n][L][V]
    H: Optional[np.ndarray]  # [n][L][D] bf16 bits/fp32, or None when D == 0
    h: Optional[np.ndarray]  # [n][L][r] fp32 when D == 0, else None
    boost_ids: np.ndarray = field(default=None)  # [n][L][n_boost] (for tests)


def make_head(cfg: Config, seed: int = 0) -> Head:
    """Draw order: A ~ N(0, 1/r) [r,r]; E ~ N(0,1) [V,r]; U ~ N(0,1/r) [V,r];
    then, if D > 0, P ~ N(0, 1/D) drawn as [D,r] and stored transposed."""
    rng = np.random.default_rng([seed, cfg.cfg_id, HEAD_STREAM])
    r, V, D = cfg.r, cfg.V, cfg.D
    A = rng.standard_normal((r, r), dtype=np.float32) * np.float32(1.0 / np.sqrt(r))
    E = rng.standard_normal((V, r), dtype=np.float32)
    U = rng.standard_normal((V, r), dtype=np.float32) * np.float32(1.0 / np.sqrt(r))
    Pt = None
    if D > 0:
        P = rng.standard_normal((D, r), dtype=np.float32) * np.float32(1.0 / np.sqrt(D))
        Pt = np.ascontiguousarray(P.T)
    wd = cfg.weight_dtype
    return Head(A=_store(A, wd), E=_store(E, wd), U=_store(U, wd),
                Pt=None if Pt is None else _store(Pt, wd), dtype=wd)


def make_round(cfg: Config, seed: int = 0, t: int = 0) -> Round:
    """Draw order: noise N(0, sigma^2) [n,L,V]; per row (request-major, then
    depth) n_boost distinct ids without replacement; boost values
    U(lo,hi) [n,L,n_boost] scaled by decay**d (d = row index + 1); the sum is
    divided by the temperature; then H ~ N(0,1) [n,L,D] (or h ~ N(0,1)
    [n,L,r] when D == 0)."""
    rng = np.random.default_rng([seed, cfg.cfg_id, t])
    n, L, V = cfg.n_req, cfg.L, cfg.V
    x = rng.standard_normal((n, L, V), dtype=np.float32) * np.float32(cfg.sigma)
    nb = min(cfg.n_boost, V)
    ids = np.empty((n, L, nb), dtype=np.int64)
    for q in range(n):
        for i in range(L):
            ids[q, i] = rng.choice(V, size=nb, replace=False)
    vals = rng.uniform(cfg.boost_lo, cfg.boost_hi, size=(n, L, nb)).astype(np.float32)
    depth = np.arange(1, L + 1, dtype=np.float64)
    vals = (vals * (cfg.decay ** depth)[None, :, None]).astype(np.float32)
    qi = np.arange(n)[:, None, None]
    li = np.arange(L)[None, :, None]
    x[qi, li, ids] += vals
    if cfg.temperature != 1.0:
        x = x / np.float32(cfg.temperature)
    logits = _store(x, cfg.logits_dtype)
    H = h = None
    if cfg.D > 0:
        H = f32_to_bf16_bits(rng.standard_normal((n, L, cfg.D), dtype=np.float32)) \
            if cfg.weight_dtype == BF16 else rng.standard_normal((n, L, cfg.D), dtype=np.float32)
    else:
        h = rng.standard_normal((n, L, cfg.r), dtype=np.float32)
    return Round(logits=logits, H=H, h=h, boost_ids=ids)


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 values of a stored tensor (uint16 bf16 bits or fp32)."""
    if dtype == BF16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def small_variant(base: str = "tiny", **kw) -> Config:
    """A config derived from a preset, for parity tests at oracle-friendly sizes."""
    return CONFIGS[base].with_(**kw)


# ----------------------------------------------------------------------------
# the drafter's LM head (the step before the candidates): hidden states X and
# head rows Wlm, both bf16
# ----------------------------------------------------------------------------
LMHEAD_STREAM = 2**32 - 2


def make_lmhead(cfg: Config, seed: int = 0, chunk_rows: int = 16384) -> np.ndarray:
    """Wlm [V][D] bf16 bits, entries N(0, sigma^2 / D) rounded to bf16, drawn
    in chunks of rows (so a full-vocabulary head never holds fp32 copies of
    more than one chunk)."""
    rng = np.random.default_rng([seed, cfg.cfg_id, LMHEAD_STREAM])
    V, D = cfg.V, cfg.D
    out = np.empty((V, D), np.uint16)
    scale = np.float32(cfg.sigma / np.sqrt(D))
    for v0 in range(0, V, chunk_rows):
        v1 = min(V, v0 + chunk_rows)
        out[v0:v1] = f32_to_bf16_bits(rng.standard_normal((v1 - v0, D), dtype=np.float32) * scale)
    return out


def make_lmhead_states(cfg: Config, Wlm: np.ndarray, seed: int = 0, t: int = 0) -> np.ndarray:
    """Hidden states X [n][L][D] bf16 bits whose logits look like the
    configs' base logits: noise N(0, 1) plus, per (request, position), n_boost
    distinct ids u with boost a_u ~ U(lo, hi) * decay^d (d = 1-based row of
    the block) added along Wlm[u] / sigma^2, so that token u's logit gains
    about a_u. Draw order: noise [n,L,D]; ids per row without replacement;
    boosts [n,L,n_boost]."""
    rng = np.random.default_rng([seed, cfg.cfg_id, t, 1])
    n, L, V, D = cfg.n_req, cfg.L, cfg.V, cfg.D
    x = rng.standard_normal((n, L, D), dtype=np.float32)
    nb = min(cfg.n_boost, V)
    ids = np.empty((n, L, nb), dtype=np.int64)
    for q in range(n):
        for i in range(L):
            ids[q, i] = rng.choice(V, size=nb, replace=False)
    a = rng.uniform(cfg.boost_lo, cfg.boost_hi, size=(n, L, nb)).astype(np.float32)
    a = (a * (cfg.decay ** np.arange(1, L + 1, dtype=np.float64))[None, :, None]).astype(np.float32)
    w32 = bf16_bits_to_f32(Wlm[ids.reshape(-1)]).reshape(n, L, nb, D)
    x += np.einsum("qlb,qlbd->qld", a, w32).astype(np.float32) / np.float32(cfg.sigma ** 2)
    return f32_to_bf16_bits(x)

