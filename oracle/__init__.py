"""Python handle on the plain CPU oracle (``oracle/oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the package smoke check and the
benchmark's CPU-baseline leg are the only callers. The GPU path neither
imports nor links anything here, and nothing here touches the GPU path.

The oracle is the sort-based definition of top-k / top-p that the Qrita
summary says its output matches ("Resultados"; "Contribuciones Clave" 1):
stable descending order by value with ties by ascending index, top-k prefix,
then the minimal rank prefix whose float64 softmax mass reaches p.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def _stale() -> bool:
    """True when liboracle.so is missing or older than oracle.c."""
    return not os.path.exists(_LIB) or os.path.getmtime(_SRC) > os.path.getmtime(_LIB)


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc; returns the path."""
    if force or _stale():
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if _stale():
                build(force=True)
            lib = ctypes.CDLL(_LIB)
            vp, i64, i32p = ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(ctypes.c_int32)
            lib.oracle_select.restype = ctypes.c_int
            lib.oracle_select.argtypes = [vp, i64, i64, ctypes.c_int, vp, vp, vp, vp, i64, vp,
                                          vp, vp, ctypes.c_int, ctypes.POINTER(i64),
                                          ctypes.POINTER(i64)]
            lib.oracle_sample.restype = ctypes.c_int
            lib.oracle_sample.argtypes = [vp, i64, i64, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64,
                                          ctypes.c_int, ctypes.POINTER(i64), ctypes.POINTER(i64)]
            lib.oracle_hardware_threads.restype = ctypes.c_int
            _lib = lib
        return _lib


def hardware_threads() -> int:
    return int(_load().oracle_hardware_threads())


def _host_logits(logits, dtype):
    """Host array and dtype code: "f32" float32 values; "bf16" and "f16"
    uint16 bit patterns (an f16 array of float16 values is taken as its bits)."""
    if dtype == "f32":
        return np.ascontiguousarray(logits, dtype=np.float32), 0
    if dtype == "bf16":
        return np.ascontiguousarray(logits, dtype=np.uint16), 1
    if dtype == "f16":
        a = np.asarray(logits)
        if a.dtype == np.float16:
            a = a.view(np.uint16)
        return np.ascontiguousarray(a, dtype=np.uint16), 2
    raise ValueError(f"unknown dtype {dtype!r}")


class OracleInputError(ValueError):
    pass


@dataclass
class OracleResult:
    mask: np.ndarray      # uint8 [B, V]
    idx: np.ndarray       # int32 [B, idx_cap]; entries past min(count, idx_cap) are -1
    count: np.ndarray     # int32 [B]
    band_lo: np.ndarray   # int32 [B]
    band_hi: np.ndarray   # int32 [B]

    @property
    def band_rows(self) -> np.ndarray:
        return np.nonzero(self.band_lo != self.band_hi)[0]


def select(logits: np.ndarray, dtype: str, k: Optional[np.ndarray], p: Optional[np.ndarray],
           idx_cap: int, nthreads: int = 0, want_mask: bool = True) -> OracleResult:
    """Run the oracle on host arrays.

    logits: [B, V] float32 (dtype "f32") or uint16 bf16 bits (dtype "bf16").
    k: int32 [B] or None (top-k off); p: float32 [B] or None (top-p off).
    """
    lib = _load()
    x, dt = _host_logits(logits, dtype)
    B, V = x.shape
    kk = None if k is None else np.ascontiguousarray(k, dtype=np.int32)
    pp = None if p is None else np.ascontiguousarray(p, dtype=np.float32)
    mask = np.empty((B, V), np.uint8) if want_mask else None
    idx = np.full((B, max(idx_cap, 0)), -1, np.int32)
    count = np.empty(B, np.int32)
    lo = np.empty(B, np.int32)
    hi = np.empty(B, np.int32)
    bad_r, bad_c = ctypes.c_int64(-1), ctypes.c_int64(-1)

    def ptr(a):
        return None if a is None else a.ctypes.data

    rc = lib.oracle_select(ptr(x), B, V, dt, ptr(kk), ptr(pp), ptr(mask),
                           ptr(idx) if idx_cap > 0 else None, int(idx_cap), ptr(count), ptr(lo),
                           ptr(hi), int(nthreads), ctypes.byref(bad_r), ctypes.byref(bad_c))
    if rc == 2:
        raise OracleInputError(f"NaN or +inf logit at row {bad_r.value}, column {bad_c.value}")
    if rc != 0:
        raise RuntimeError(f"oracle_select failed with status {rc}")
    return OracleResult(mask, idx, count, lo, hi)


def uniforms(seed: int, offset: int, batch: int) -> np.ndarray:
    """The draw's uniforms from NumPy's own Philox4x64-10 (the generator of
    Salmon et al., SC 2011, as NumPy implements it): for row b, the first
    64-bit output at counter (b, offset, 0, 0) under key (seed, 0), top 53
    bits times 2^-53. NumPy advances its counter before each block of four
    outputs, so the generator starts one counter value earlier."""
    out = np.empty(batch, np.float64)
    for b in range(batch):
        ctr = ((int(b) | (int(offset) % 2**64) << 64) - 1) % 2**256
        g = np.random.Philox(counter=ctr, key=int(seed) % 2**64)
        x = int(g.random_raw())
        out[b] = (x >> 11) * 2.0**-53
    return out


@dataclass
class SampleResult:
    token: np.ndarray     # int32 [B] drawn vocabulary index
    rank: np.ndarray      # int32 [B] its rank in the kept set
    rank_lo: np.ndarray   # int32 [B] draw rank at u - 1e-6
    rank_hi: np.ndarray   # int32 [B] draw rank at u + 1e-6
    count: np.ndarray     # int32 [B] kept count
    idx: np.ndarray       # int32 [B, idx_cap] kept indices in rank order (-1 past the count)
    prob: np.ndarray      # float32 [B, idx_cap] renormalised probabilities beside idx


def sample(logits: np.ndarray, dtype: str, k: Optional[np.ndarray], p: Optional[np.ndarray],
           u: np.ndarray, idx_cap: int, nthreads: int = 0) -> SampleResult:
    """Select, then draw by inverse CDF over the kept set with the given uniforms."""
    lib = _load()
    x, dt = _host_logits(logits, dtype)
    B, V = x.shape
    kk = None if k is None else np.ascontiguousarray(k, dtype=np.int32)
    pp = None if p is None else np.ascontiguousarray(p, dtype=np.float32)
    uu = np.ascontiguousarray(u, dtype=np.float64)
    if uu.shape != (B,):
        raise ValueError("u must have one uniform per row")
    token = np.empty(B, np.int32)
    lo = np.empty(B, np.int32)
    hi = np.empty(B, np.int32)
    count = np.empty(B, np.int32)
    cap = max(int(idx_cap), 1)
    idx = np.full((B, cap), -1, np.int32)
    prob = np.zeros((B, cap), np.float32)
    bad_r, bad_c = ctypes.c_int64(-1), ctypes.c_int64(-1)

    def ptr(a):
        return None if a is None else a.ctypes.data

    rank = np.empty(B, np.int32)
    rc = lib.oracle_sample(ptr(x), B, V, dt, ptr(kk), ptr(pp), ptr(uu), ptr(token), ptr(rank), ptr(lo), ptr(hi),
                           ptr(count), ptr(idx), ptr(prob), cap, int(nthreads), ctypes.byref(bad_r),
                           ctypes.byref(bad_c))
    if rc == 2:
        raise OracleInputError(f"NaN or +inf logit at row {bad_r.value}, column {bad_c.value}")
    if rc != 0:
        raise RuntimeError(f"oracle_sample failed with status {rc}")
    return SampleResult(token, rank, lo, hi, count, idx[:, :idx_cap] if idx_cap > 0 else idx[:, :0],
                        prob[:, :idx_cap] if idx_cap > 0 else prob[:, :0])
