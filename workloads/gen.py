"""Seeded synthetic logits and per-row k / p controls.

The five named workloads stand in for the large-vocabulary serving runs that
the Qrita summary evaluates (Llama, Qwen, GPT-OSS, Gemma logits; "Resultados"
section). No dataset or trained weights are involved: each row is drawn from a
stated distribution with NumPy's PCG64, from a seed sequence rooted at
``1000 + config_index``, so any subset of rows can be regenerated alone.

Values are drawn in float64, cast to float32 with round-to-nearest-even, and
for bf16 workloads rounded float32 -> bf16 with round-to-nearest-even; f16
workloads round float64 -> IEEE binary16 (NumPy's cast, nearest-even). The
resulting bit patterns are the data for both the GPU path and the oracle.

Two more named workloads (EXTRA) have the shapes of the same selection in
other systems: top-512 marginals of a block drafter over a full vocabulary,
and top-B pruning of a beam search over BW x K scored proposals.

This module only draws numbers. It contains none of the selection method's
arithmetic (no ordering, no thresholds, no softmax).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Optional, Sequence

import numpy as np

__all__ = [
    "CONFIGS",
    "EXTRA",
    "Inputs",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "make_config",
    "make_rows",
]


@dataclass
class Inputs:
    """One batch of rows.

    logits: [B, V] array. float32 values for dtype "f32"; uint16 bit
            patterns for dtypes "bf16" and "f16". Rows are contiguous (C order).
    k:      int32 [B] per-row top-k (<= 0 or >= V means top-k off).
    p:      float32 [B] per-row top-p (>= 1 or NaN means top-p off).
    """

    name: str
    dtype: str
    logits: np.ndarray
    k: np.ndarray
    p: np.ndarray

    @property
    def batch(self) -> int:
        return int(self.logits.shape[0])

    @property
    def vocab(self) -> int:
        return int(self.logits.shape[1])

    def values_f32(self) -> np.ndarray:
        """The logits widened to float32 (exact for every dtype)."""
        if self.dtype == "bf16":
            return bf16_bits_to_f32(self.logits)
        if self.dtype == "f16":
            return self.logits.view(np.float16).astype(np.float32)
        return self.logits

    def take_rows(self, rows: Sequence[int]) -> "Inputs":
        rows = np.asarray(rows, dtype=np.int64)
        return Inputs(self.name, self.dtype, np.ascontiguousarray(self.logits[rows]),
                      self.k[rows].copy(), self.p[rows].copy())


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round-to-nearest-even); returns uint16 bits.

    Inputs here are always finite, so the NaN case of the rounding is not
    handled.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _cast(z64: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return z64.astype(np.float16).view(np.uint16)
    z32 = z64.astype(np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(z32)
    return z32


def _store_dtype(dtype: str):
    return np.uint16 if dtype in ("bf16", "f16") else np.float32


def _row_rngs(seed_root: int, batch: int) -> list:
    children = np.random.SeedSequence([seed_root, 0]).spawn(batch)
    return [np.random.Generator(np.random.PCG64(c)) for c in children]


def _ctl_rng(seed_root: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed_root, 1])))


# ---------------------------------------------------------------------------
# Row distributions of the five named workloads
# ---------------------------------------------------------------------------

def _row_c0(rng, V):
    z = rng.standard_normal(V)
    pos = rng.choice(V, 20, replace=False)
    z[pos] = rng.normal(8.0, 2.0, 20)
    return z


def _row_c1(rng, V):
    z = rng.normal(0.0, 2.5, V)
    n = int(round(0.01 * V))
    pos = rng.choice(V, n, replace=False)
    z[pos] = rng.normal(10.0, 3.0, n)
    return z


def _row_c2(rng, V):
    # quantised to steps of 1/16: exactly representable in bf16 while |z| < 16,
    # and np.round keeps the sign of small negatives, so -0.0 appears.
    return np.round(rng.normal(0.0, 2.0, V) * 16.0) / 16.0


def _row_c3(rng, V):
    return rng.uniform(-1.0, 1.0, V)


def _row_c4(rng, V):
    z = 3.0 * rng.standard_t(3.0, V)
    n = int(round(0.005 * V))
    pos = rng.choice(V, n, replace=False)
    z[pos] = 15.0
    return z


def _ctl_c0(rng, B):
    return np.full(B, 50, np.int32), np.full(B, 0.9, np.float32)


def _ctl_c1(rng, B):
    k = rng.integers(1, 1025, B).astype(np.int32)
    p = rng.uniform(0.5, 1.0, B).astype(np.float32)
    return k, p


def _ctl_c2(rng, B):
    return np.full(B, 50, np.int32), np.full(B, 0.95, np.float32)


def _ctl_c3(rng, B):
    return np.full(B, 4096, np.int32), np.full(B, 1.0, np.float32)


def _ctl_c4(rng, B):
    r = np.arange(B)
    k = np.where(r < 256, np.array([1, 20, 1000, 8192])[r % 4], 0).astype(np.int32)
    p = np.where(r < 256, 1.0, np.array([0.1, 0.9, 0.99])[(r - 256) % 3]).astype(np.float32)
    return k, p


CONFIGS = [
    dict(index=0, name="b1_v32000_f32_gauss_outliers", batch=1, vocab=32000, dtype="f32",
         row=_row_c0, ctl=_ctl_c0,
         text="1 x 32000 fp32, N(0,1) with 20 positions set to N(8, sd 2); k=50, p=0.9"),
    dict(index=1, name="b64_v128256_bf16_gauss_tail", batch=64, vocab=128256, dtype="bf16",
         row=_row_c1, ctl=_ctl_c1,
         text="64 x 128256 bf16, N(0, sd 2.5) with 1283 positions set to N(10, sd 3); "
              "k ~ U{1..1024}, p ~ U[0.5, 1.0) per row"),
    dict(index=2, name="b256_v151936_bf16_ties16", batch=256, vocab=151936, dtype="bf16",
         row=_row_c2, ctl=_ctl_c2,
         text="256 x 151936 bf16, N(0, sd 2) quantised to 1/16 (heavy ties, signed zeros); "
              "k=50, p=0.95"),
    dict(index=3, name="b1024_v201088_f32_uniform", batch=1024, vocab=201088, dtype="f32",
         row=_row_c3, ctl=_ctl_c3,
         text="1024 x 201088 fp32, U(-1,1) (non-Gaussian: truncation miss); k=4096, top-p off"),
    dict(index=4, name="b512_v262144_bf16_heavy", batch=512, vocab=262144, dtype="bf16",
         row=_row_c4, ctl=_ctl_c4,
         text="512 x 262144 bf16, 3*StudentT(3) with 1311 positions at +15; rows 0-255 top-k "
              "k in {1,20,1000,8192}; rows 256-511 top-p p in {0.1,0.9,0.99}"),
]


def make_config(index: int, rows: Optional[Sequence[int]] = None) -> Inputs:
    """Generate named workload ``index`` (all rows, or only ``rows``)."""
    c = CONFIGS[index]
    B, V, dt = c["batch"], c["vocab"], c["dtype"]
    seed_root = 1000 + index
    rngs = _row_rngs(seed_root, B)
    k, p = c["ctl"](_ctl_rng(seed_root), B)
    sel = np.arange(B) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((len(sel), V), dtype=_store_dtype(dt))
    for j, r in enumerate(sel):
        out[j] = _cast(c["row"](rngs[int(r)], V), dt)
    return Inputs(c["name"], dt, out, k[sel].copy(), p[sel].copy())


# ---------------------------------------------------------------------------
# The second workload: the same selection at other systems' shapes
# ---------------------------------------------------------------------------

def _row_marginals(rng, V):
    # a drafter's per-position logits: a broad N(0, sd 2.5) body with about
    # 0.5 % plausible tokens lifted to N(9, sd 2.5)
    z = rng.normal(0.0, 2.5, V)
    n = int(round(0.005 * V))
    z[rng.choice(V, n, replace=False)] = rng.normal(9.0, 2.5, n)
    return z


def _row_beam(rng, V, K=64):
    # BW = V / K beams, each with K proposals in beam-major order: the score
    # is the beam's cumulative log-probability plus the proposal's
    # log-probability, both modelled as decreasing sums of exponential steps
    # (about 30 % of the proposals fail validation and score -inf)
    BW = V // K
    beam = -np.cumsum(rng.exponential(0.15, BW))
    lp = -np.cumsum(rng.exponential(0.4, (BW, K)), axis=1)
    s = (beam[:, None] + lp).reshape(-1)
    s[rng.random(V) < 0.3] = -np.inf
    return s


def _ctl_marginals(rng, B):
    return np.full(B, 512, np.int32), np.full(B, 1.0, np.float32)


def _ctl_beam(rng, B):
    return np.full(B, 64, np.int32), np.full(B, 1.0, np.float32)


EXTRA = [
    dict(index=0, name="b2048_v151936_f16_marginals_top512", batch=2048, vocab=151936, dtype="f16",
         row=_row_marginals, ctl=_ctl_marginals, idx_order=1,
         text="2048 x 151936 f16 (128 sequences x 16 block positions of drafter logits: N(0, sd 2.5), "
              "0.5 % at N(9, sd 2.5)); k=512, indices in ascending vocabulary order"),
    dict(index=1, name="b4096_v4096_f32_beam_prune_top64", batch=4096, vocab=4096, dtype="f32",
         row=_row_beam, ctl=_ctl_beam, idx_order=1,
         text="4096 x 4096 fp32 (64 beams x 64 proposals: cumulative beam log-prob + sorted "
              "proposal log-softmax, 30 % -inf); k=64, indices in ascending (beam-major) order"),
]


def make_extra(index: int, rows: Optional[Sequence[int]] = None) -> Inputs:
    """Generate the second-workload shape ``index`` (all rows, or only ``rows``)."""
    c = EXTRA[index]
    B, V, dt = c["batch"], c["vocab"], c["dtype"]
    seed_root = 2000 + index
    rngs = _row_rngs(seed_root, B)
    k, p = c["ctl"](_ctl_rng(seed_root), B)
    sel = np.arange(B) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((len(sel), V), dtype=_store_dtype(dt))
    for j, r in enumerate(sel):
        out[j] = _cast(c["row"](rngs[int(r)], V), dt)
    return Inputs(c["name"], dt, out, k[sel].copy(), p[sel].copy())


# ---------------------------------------------------------------------------
# Extra row kinds for tests (edge cases and adversarial layouts)
# ---------------------------------------------------------------------------

def _kind_fn(kind: str) -> Callable:
    def gauss(rng, V):
        return rng.normal(0.0, 1.5, V)

    def gauss_outliers(rng, V):
        return _row_c1(rng, V)

    def ties16(rng, V):
        return _row_c2(rng, V)

    def uniform(rng, V):
        return _row_c3(rng, V)

    def gauss2(rng, V):
        # the 1/16-grid rows' distribution before quantisation (distinct in float32)
        return rng.normal(0.0, 2.0, V)

    def heavy(rng, V):
        return _row_c4(rng, V)

    def equal(rng, V):
        return np.full(V, float(rng.integers(-4, 5)) * 0.5)

    def twolevel(rng, V):
        z = np.full(V, -1.0)
        a = int(rng.integers(1, max(2, V // 3)))
        z[rng.choice(V, a, replace=False)] = 2.0
        return z

    def smallint(rng, V):
        return rng.integers(-3, 4, V).astype(np.float64)

    def neginf(rng, V):
        z = rng.normal(0.0, 1.0, V)
        n = int(rng.integers(0, V + 1))
        z[rng.choice(V, n, replace=False)] = -np.inf
        return z

    def allneginf(rng, V):
        return np.full(V, -np.inf)

    def zeros(rng, V):
        z = np.where(rng.random(V) < 0.5, -0.0, 0.0)
        n = int(rng.integers(0, max(1, V // 50) + 1))
        z[rng.choice(V, n, replace=False)] = rng.normal(0.0, 1.0, n)
        return z

    def ascending(rng, V):
        return np.sort(rng.normal(0.0, 1.0, V))

    def descending(rng, V):
        return np.sort(rng.normal(0.0, 1.0, V))[::-1].copy()

    def spike(rng, V):
        z = rng.normal(0.0, 1.0, V)
        z[int(rng.integers(0, V))] = 200.0
        return z

    def flat(rng, V):
        return rng.normal(0.0, 0.05, V)

    def marginals(rng, V):
        return _row_marginals(rng, V)

    def beam(rng, V):
        return _row_beam(rng, V, K=64 if V % 64 == 0 else 1)

    def f16_edges(rng, V):
        # binary16 extremes: subnormals, the largest finite values, signed zeros
        z = rng.normal(0.0, 1.0, V)
        pick = rng.integers(0, 5, V)
        z = np.where(pick == 0, rng.integers(-1023, 1024, V) * 2.0**-24, z)
        z = np.where(pick == 1, np.where(rng.random(V) < 0.5, -0.0, 0.0), z)
        z = np.where(pick == 2, rng.choice([65504.0, 65472.0, -65504.0], V), z)
        return z

    table = dict(gauss=gauss, gauss_outliers=gauss_outliers, ties16=ties16, uniform=uniform, gauss2=gauss2,
                 heavy=heavy, equal=equal, twolevel=twolevel, smallint=smallint, neginf=neginf,
                 allneginf=allneginf, zeros=zeros, ascending=ascending, descending=descending,
                 spike=spike, flat=flat, marginals=marginals, beam=beam, f16_edges=f16_edges)
    return table[kind]


ROW_KINDS = ("gauss", "gauss_outliers", "ties16", "uniform", "gauss2", "heavy", "equal", "twolevel",
             "smallint", "neginf", "allneginf", "zeros", "ascending", "descending", "spike",
             "flat", "marginals", "beam", "f16_edges")


def make_rows(batch: int, vocab: int, dtype: str, kind: str, seed: int,
              k=None, p=None) -> Inputs:
    """``batch`` rows of one kind. ``k``/``p`` may be scalars, arrays, or None.

    None draws per-row controls: k uniform over {-1, 0, 1, .., vocab + 1} and
    p from a mix of off (1.0), 0, small, mid and near-1 values.
    """
    fn = _kind_fn(kind)
    rngs = _row_rngs(seed, batch)
    out = np.empty((batch, vocab), dtype=_store_dtype(dtype))
    for r in range(batch):
        out[r] = _cast(fn(rngs[r], vocab), dtype)
    crng = _ctl_rng(seed)
    if k is None:
        k = crng.integers(-1, vocab + 2, batch)
    if p is None:
        choices = np.array([1.0, 1.0, 0.0, 0.1, 0.5, 0.9, 0.99, 0.999], dtype=np.float64)
        p = choices[crng.integers(0, len(choices), batch)]
    k = np.broadcast_to(np.asarray(k, dtype=np.int32), (batch,)).copy()
    p = np.broadcast_to(np.asarray(p, dtype=np.float32), (batch,)).copy()
    return Inputs(f"{kind}_b{batch}_v{vocab}_{dtype}", dtype, out, k, p)
