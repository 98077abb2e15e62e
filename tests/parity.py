"""Helpers for GPU-vs-oracle parity tests (imported by the gpu tests only).

The GPU side is called through the C ABI (the ctypes binding); the expected
side is the CPU oracle on the same seeded host arrays.

The bar (from the method's exactness claim): top-k masks, indices and counts
bit-exact; top-p exact except on rows where the oracle's float64 cumulative
mass at the cut lies within 1e-5 of p (band rows). On a band row the GPU must
return a rank prefix of the oracle's order whose length lies in
[band_lo, band_hi].
"""
from dataclasses import dataclass

import numpy as np

import oracle


@dataclass
class GpuOut:
    mask: np.ndarray
    idx: np.ndarray
    count: np.ndarray
    diag: np.ndarray


def device_logits(x, dev):
    """The batch's logits as a device tensor of its dtype (bit patterns kept)."""
    import torch

    if x.dtype == "bf16":
        return torch.from_numpy(x.logits.view(np.int16)).to(dev).view(torch.bfloat16)
    if x.dtype == "f16":
        return torch.from_numpy(x.logits.view(np.int16)).to(dev).view(torch.float16)
    return torch.from_numpy(x.logits).to(dev)


def run_gpu(x, idx_cap, options=None, want_mask=True, want_idx=True, stream=None):
    import torch

    import top_selection_sigma_amd as q

    dev = torch.device("cuda", 0)
    logits = device_logits(x, dev)
    k = torch.from_numpy(x.k).to(dev)
    p = torch.from_numpy(x.p).to(dev)
    if options is None:
        options = q.Options()
    diag = torch.full((x.batch, q.DIAG_FIELDS), -7, dtype=torch.int32, device=dev)
    options.diag = diag
    cap = idx_cap if want_idx else None
    mask, idx, count = q.select(logits, k, p, want_mask=want_mask, idx_cap=cap,
                                options=options, stream=stream)
    torch.cuda.synchronize()
    return GpuOut(None if mask is None else mask.cpu().numpy(),
                  None if idx is None else idx.cpu().numpy(), count.cpu().numpy(),
                  diag.cpu().numpy())


def oracle_for(x, idx_cap):
    return oracle.select(x.logits, x.dtype, x.k, x.p, idx_cap)


def check(x, g: GpuOut, ref, idx_cap, label=""):
    """Assert parity; returns the list of band rows."""
    B = x.batch
    band = ref.band_lo != ref.band_hi
    exact = ~band
    cnt = g.count
    bad = np.nonzero(exact & (cnt != ref.count))[0]
    assert len(bad) == 0, f"{label}: count mismatch rows {bad[:10]} gpu {cnt[bad[:10]]} ref {ref.count[bad[:10]]}"
    if g.mask is not None:
        rows_bad = np.nonzero(exact & np.any(g.mask != ref.mask, axis=1))[0]
        assert len(rows_bad) == 0, f"{label}: mask mismatch rows {rows_bad[:10]}"
    if g.idx is not None and idx_cap > 0:
        for b in np.nonzero(exact)[0]:
            n = min(int(ref.count[b]), idx_cap)
            if not np.array_equal(g.idx[b, :n], ref.idx[b, :n]):
                raise AssertionError(f"{label}: idx mismatch row {b}: gpu {g.idx[b, :min(n, 12)]} "
                                     f"ref {ref.idx[b, :min(n, 12)]}")
    brows = np.nonzero(band)[0]
    if len(brows):
        hi = int(ref.band_hi[brows].max())
        sub = x.take_rows(brows)
        full = oracle.select(sub.logits, sub.dtype, sub.k, sub.p, max(hi, 1), want_mask=False)
        for j, b in enumerate(brows):
            c = int(cnt[b])
            assert ref.band_lo[b] <= c <= ref.band_hi[b], f"{label}: band row {b} count {c}"
            order = full.idx[j, :c]
            if g.mask is not None:
                m = np.zeros(x.vocab, np.uint8)
                m[order] = 1
                assert np.array_equal(g.mask[b], m), f"{label}: band row {b} mask not a rank prefix"
            if g.idx is not None and idx_cap > 0:
                n = min(c, idx_cap)
                assert np.array_equal(g.idx[b, :n], full.idx[j, :n]), f"{label}: band row {b} idx"
    return list(brows)


def check_index_order(x, g: GpuOut, ref, idx_cap, label=""):
    """Parity of index-ordered output: the kept set as in check(), and idx
    holding the first min(count, idx_cap) kept indices in ascending order."""
    band = ref.band_lo != ref.band_hi
    cnt = g.count
    bad = np.nonzero(~band & (cnt != ref.count))[0]
    assert len(bad) == 0, f"{label}: count mismatch rows {bad[:10]}"
    if g.mask is not None:
        rows_bad = np.nonzero(~band & np.any(g.mask != ref.mask, axis=1))[0]
        assert len(rows_bad) == 0, f"{label}: mask mismatch rows {rows_bad[:10]}"
    brows = np.nonzero(band)[0]
    full = None
    if len(brows):
        sub = x.take_rows(brows)
        full = oracle.select(sub.logits, sub.dtype, sub.k, sub.p, max(int(ref.band_hi[brows].max()), 1),
                             want_mask=False)
    j = 0
    for b in range(x.batch):
        c = int(cnt[b])
        if band[b]:
            assert ref.band_lo[b] <= c <= ref.band_hi[b], f"{label}: band row {b} count {c}"
            kept = np.sort(full.idx[j, :c])
            j += 1
            if g.mask is not None:
                m = np.zeros(x.vocab, np.uint8)
                m[kept] = 1
                assert np.array_equal(g.mask[b], m), f"{label}: band row {b} mask not a rank prefix"
        else:
            kept = np.nonzero(ref.mask[b])[0]
        if g.idx is not None and idx_cap > 0:
            n = min(c, idx_cap)
            if not np.array_equal(g.idx[b, :n], kept[:n]):
                raise AssertionError(f"{label}: index-ordered idx mismatch row {b}: gpu {g.idx[b, :min(n, 12)]} "
                                     f"want {kept[:min(n, 12)]}")
