"""Seeded synthetic inputs for the RDA token mixer (host side, NumPy only).

This module is the one piece shared by the GPU path's tests/bench and the
fp64 oracle: it draws inputs and nothing else.  It contains none of the
recurrence's arithmetic.  Every tensor is drawn in float64, cast to float32,
and (for bf16 inputs) rounded to bfloat16 with round-to-nearest-even on the
host, so the GPU kernels and the oracle consume exactly the same bits.

Workload recipe (the shapes follow the Raon-1 nano spec table on the
"Raon-1-nano-gguf" page: 16 RDA heads of dimension 128; the state is one
128 x 128 fp32 matrix per head per the "Raon-1 nano" teardown, section "The
cache is small if the runtime keeps it small"):

* q, k ~ N(0, 1), then L2-normalised per token and head;  v ~ N(0, 1).
* a = exp(-softplus(x)), b = sigmoid(y) with x, y ~ N(0, 1), fp32, one value
  per token per head.
* Initial states S0 ~ N(0, 0.02) (0.02 is the standard deviation, matching
  the normal_(std=0.02) initialisation printed on the tiny-random Raon-1 mini
  model card) where a workload asks for one.

Seeding: ``np.random.default_rng`` on ``SeedSequence([20261203, config_id])``
with one spawned child stream per tensor in the order q, k, v, a, b, S0,
lengths.  Decode draws each step's token from ``SeedSequence([20261203,
config_id, 1 + step])``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

SEED_ROOT = 20261203


# --------------------------------------------------------------------------
# bfloat16 helpers (bit-level, round to nearest even)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (RNE); returns uint16 bit patterns."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    rounding = ((u >> 16) & 1) + 0x7FFF
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (bits.astype(np.uint32) << 16).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16 (returned as float32)."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


# --------------------------------------------------------------------------
# elementary draws
# --------------------------------------------------------------------------
def _rng(*key) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([SEED_ROOT, *key]))


def _children(*key, n: int):
    return [np.random.default_rng(s)
            for s in np.random.SeedSequence([SEED_ROOT, *key]).spawn(n)]


def unit_rows(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) draws L2-normalised along the last axis (float64)."""
    x = rng.standard_normal(shape)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    n[n == 0] = 1.0
    return x / n


def gates(rng_a: np.random.Generator, rng_b: np.random.Generator, shape):
    """a = exp(-softplus(x)), b = sigmoid(y), x, y ~ N(0,1); float32."""
    x = rng_a.standard_normal(shape)
    y = rng_b.standard_normal(shape)
    softplus = np.logaddexp(0.0, x)
    a = np.exp(-softplus)
    b = 1.0 / (1.0 + np.exp(-y))
    return a.astype(np.float32), b.astype(np.float32)


def varlen_lengths(rng: np.random.Generator, n: int = 8, lo: int = 512,
                   hi: int = 8192, total: int = 32768) -> np.ndarray:
    """n lengths in [lo, hi] summing to `total`: n-1 uniform draws, the last
    fills the remainder; redraw until the last is also within [lo, hi]."""
    while True:
        head = rng.integers(lo, hi + 1, size=n - 1)
        last = total - int(head.sum())
        if lo <= last <= hi:
            return np.concatenate([head, [last]]).astype(np.int64)


def cu_from_lengths(lengths) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


# --------------------------------------------------------------------------
# prefill / decode input bundles
# --------------------------------------------------------------------------
@dataclass
class PrefillInputs:
    """Host arrays for one prefill call.

    q, k, v hold float32 values; when ``bf16`` is set they are exact
    bfloat16 values and ``*_bits`` hold the uint16 patterns.
    """
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    a: np.ndarray
    b: np.ndarray
    cu_seqlens: Optional[np.ndarray]
    S0: Optional[np.ndarray]
    bf16: bool
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def total_tokens(self) -> int:
        return self.q.shape[0]

    @property
    def num_heads(self) -> int:
        return self.q.shape[1]

    @property
    def num_seqs(self) -> int:
        return 1 if self.cu_seqlens is None else len(self.cu_seqlens) - 1

    def bits(self, name: str) -> np.ndarray:
        return f32_to_bf16_bits(getattr(self, name))


def make_prefill(T: int = 0, H: int = 16, dk: int = 128, dv: int = 128, *,
                 lengths=None, bf16: bool = True, s0_std: float = 0.0,
                 key=(0,), name: str = "") -> PrefillInputs:
    """Generic seeded prefill inputs.

    lengths: per-sequence lengths for a packed varlen batch (cu_seqlens is
    then set); otherwise one sequence of T tokens with cu_seqlens None.
    s0_std > 0 draws per-sequence S0 ~ N(0, s0_std); 0 means S0 = None.
    """
    rq, rk, rv, ra, rb, rs, _ = _children(*key, n=7)
    if lengths is not None:
        lengths = np.asarray(lengths, dtype=np.int64)
        T = int(lengths.sum())
        cu = cu_from_lengths(lengths)
        N = len(lengths)
    else:
        cu = None
        N = 1
    q = unit_rows(rq, (T, H, dk)).astype(np.float32)
    k = unit_rows(rk, (T, H, dk)).astype(np.float32)
    v = rv.standard_normal((T, H, dv)).astype(np.float32)
    if bf16:
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    a, b = gates(ra, rb, (T, H))
    S0 = None
    if s0_std > 0:
        S0 = (rs.standard_normal((N, H, dv, dk)) * s0_std).astype(np.float32)
    return PrefillInputs(q, k, v, a, b, cu, S0, bf16, name=name)


# The five workloads.  Config 1 is the small single-head case, 2-4 are the
# Raon-1 nano RDA prefill shapes, 5 is the batched decode workload.
def config1() -> PrefillInputs:
    """Single head, T=64, d=128, fp32 q/k/v, S0 = 0."""
    return make_prefill(64, 1, 128, 128, bf16=False, key=(1,),
                        name="c1: single-head T=64 H=1 d=128 fp32")


def config2() -> PrefillInputs:
    """Raon-1 nano RDA layer prefill: T=2048, H=16, d=128, bf16, S0 = 0."""
    return make_prefill(2048, 16, 128, 128, bf16=True, key=(2,),
                        name="c2: prefill T=2048 H=16 d=128 bf16")


def config3() -> PrefillInputs:
    """Long prompt: T=16384, H=16, d=128, bf16, S0 ~ N(0, 0.02)."""
    return make_prefill(16384, 16, 128, 128, bf16=True, s0_std=0.02, key=(3,),
                        name="c3: long-prompt prefill T=16384 H=16 d=128 bf16")


def config4_lengths() -> np.ndarray:
    rngs = _children(4, n=7)
    return varlen_lengths(rngs[6], 8, 512, 8192, 32768)


def config4() -> PrefillInputs:
    """Varlen: 8 sequences, lengths uniform in 512..8192, total 32768."""
    lengths = config4_lengths()
    p = make_prefill(H=16, dk=128, dv=128, lengths=lengths, bf16=True,
                     s0_std=0.02, key=(4,),
                     name="c4: varlen prefill 8 seqs total 32768 H=16 d=128 bf16")
    p.meta["lengths"] = [int(x) for x in lengths]
    return p


@dataclass
class DecodeStepInputs:
    q: np.ndarray   # [B, H, dk] float32 (exact bf16 values)
    k: np.ndarray
    v: np.ndarray   # [B, H, dv]
    a: np.ndarray   # [B, H]
    b: np.ndarray


def decode_state(B: int = 256, H: int = 16, dk: int = 128, dv: int = 128,
                 std: float = 0.02, key=(5,)) -> np.ndarray:
    """Initial decode states S ~ N(0, std), float32 [B, H, dv, dk]."""
    rng = _rng(*key, 0)
    out = np.empty((B, H, dv, dk), dtype=np.float32)
    # drawn in slabs to bound host memory for the 256 MiB workload
    for bi in range(B):
        out[bi] = (rng.standard_normal((H, dv, dk)) * std).astype(np.float32)
    return out


def decode_step_inputs(step: int, B: int = 256, H: int = 16, dk: int = 128,
                       dv: int = 128, key=(5,)) -> DecodeStepInputs:
    """One decode token per (batch, head) for step `step` (bf16 q/k/v)."""
    rq, rk, rv, ra, rb = _children(*key, 1 + step, n=5)
    q = round_bf16(unit_rows(rq, (B, H, dk)).astype(np.float32))
    k = round_bf16(unit_rows(rk, (B, H, dk)).astype(np.float32))
    v = round_bf16(rv.standard_normal((B, H, dv)).astype(np.float32))
    a, b = gates(ra, rb, (B, H))
    return DecodeStepInputs(q, k, v, a, b)


@dataclass
class DecodeTokensInputs:
    q: np.ndarray   # [B, T, H, dk] float32 (exact bf16 values)
    k: np.ndarray
    v: np.ndarray   # [B, T, H, dv]
    a: np.ndarray   # [B, T, H]
    b: np.ndarray
    accept: np.ndarray  # int32 [B], uniform in [0, T]


def decode_tokens_inputs(B: int = 256, T: int = 3, H: int = 16, dk: int = 128,
                         dv: int = 128, bf16: bool = True, key=(6,)) -> DecodeTokensInputs:
    """T tokens per (batch, head) for a verify of drafted tokens (one token
    plus T - 1 drafts), with a per-sequence accepted count."""
    rq, rk, rv, ra, rb, rc = _children(*key, n=6)
    q = unit_rows(rq, (B, T, H, dk)).astype(np.float32)
    k = unit_rows(rk, (B, T, H, dk)).astype(np.float32)
    v = rv.standard_normal((B, T, H, dv)).astype(np.float32)
    if bf16:
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    a, b = gates(ra, rb, (B, T, H))
    accept = rc.integers(0, T + 1, size=B).astype(np.int32)
    return DecodeTokensInputs(q, k, v, a, b, accept)


def diag_alpha(T: int, H: int = 16, dk: int = 128, key=(10,)) -> np.ndarray:
    """Per-channel decays [T, H, dk]: alpha = exp(-softplus(x)), x ~ N(-1,
    1.5^2) per element (median about 0.73, a long tail of fast channels)."""
    x = _rng(*key).standard_normal((T, H, dk)) * 1.5 - 1.0
    return np.exp(-np.logaddexp(0.0, x)).astype(np.float32)


@dataclass
class EpilogueInputs:
    o: np.ndarray       # [rows, dv] float32, row scales spread over 1e-3 .. 1e2
    g: np.ndarray       # [rows, dv] float32 (exact bf16 values when bf16)
    weight: np.ndarray  # [dv] float32, uniform in [0.5, 1.5]


def epilogue_inputs(rows: int, dv: int = 128, bf16: bool = True, key=(7,)) -> EpilogueInputs:
    """Mixer outputs and gates for the output norm and gate: N(0, 1) rows
    scaled by a log-uniform factor, gate N(0, 2), weight U(0.5, 1.5)."""
    ro, rs, rg, rw = _children(*key, n=4)
    scale = np.exp(rs.uniform(np.log(1e-3), np.log(1e2), size=(rows, 1)))
    o = (ro.standard_normal((rows, dv)) * scale).astype(np.float32)
    g = (rg.standard_normal((rows, dv)) * 2.0).astype(np.float32)
    if bf16:
        g = round_bf16(g)
    w = rw.uniform(0.5, 1.5, size=dv).astype(np.float32)
    return EpilogueInputs(o, g, w)


@dataclass
class PrologueInputs:
    xq: np.ndarray        # raw projections [T, H, d] float32 (exact bf16 values)
    xk: np.ndarray
    xv: np.ndarray
    conv_w: np.ndarray    # [3, H, d, K] float32
    beta_raw: np.ndarray  # [T, H]
    delta: np.ndarray     # [T, H]
    g_log: np.ndarray     # [T, H], some below the -5 floor
    hist: np.ndarray      # [N, 3, K-1, H, d] float32 (exact bf16 values)


def prologue_inputs(T: int, H: int = 16, K: int = 4, N: int = 1, d: int = 128,
                    key=(8,)) -> PrologueInputs:
    """Raw projections and gates for the prologue: q, k, v N(0, 1) in bf16,
    conv weights N(0, 0.5^2), beta_raw and delta N(0, 1), log decay
    -Exp(mean 1.5) (about 4 % below -5), a bf16 N(0, 1) history."""
    r = _children(*key, n=8)
    xq, xk, xv = (round_bf16(r[i].standard_normal((T, H, d)).astype(np.float32)) for i in range(3))
    conv_w = (r[3].standard_normal((3, H, d, K)) * 0.5).astype(np.float32)
    beta_raw = r[4].standard_normal((T, H)).astype(np.float32)
    delta = r[5].standard_normal((T, H)).astype(np.float32)
    g_log = (-r[6].exponential(1.5, (T, H))).astype(np.float32)
    hist = round_bf16(r[7].standard_normal((N, 3, max(K - 1, 0), H, d)).astype(np.float32))
    return PrologueInputs(xq, xk, xv, conv_w, beta_raw, delta, g_log, hist)


CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4}
