"""Pins for the CPU oracle against things other than itself.

Each test ties the oracle to one of: the hand-derived worked examples in
tests/golden (with their citations), a brute-force O(V^2) rank definition on
exhaustive tiny rows, NumPy / PyTorch stable sorts, closed forms for top-p,
and invariants that the mathematics fixes. The test ids name which plausible
mistake each one would catch.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads as w

HERE = os.path.dirname(os.path.abspath(__file__))


def _parse(s):
    return float(s)


def _golden_cases():
    with open(os.path.join(HERE, "golden", "worked_examples.json")) as f:
        return json.load(f)["cases"]


def _row_from_case(c):
    if c["dtype"] == "bf16":
        return np.array([int(b, 16) for b in c["row_bits"]], dtype=np.uint16)
    if "row_spec" in c:
        spec = c["row_spec"]
        vals = [_parse(v) for v in spec["head"]] + [_parse(spec["fill"])] * spec["fill_count"]
    else:
        vals = [_parse(v) for v in c["row"]]
    return np.array(vals, dtype=np.float32)


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["id"])
def test_golden_worked_examples(case):
    row = _row_from_case(case)[None, :]
    k = np.array([case["k"]], np.int32)
    p = np.array([_parse(case["p"])], np.float32)
    r = oracle.select(row, case["dtype"], k, p, case["idx_cap"])
    n = min(case["count"], case["idx_cap"])
    assert int(r.count[0]) == case["count"]
    assert r.idx[0, :n].tolist() == case["idx"]
    assert [int(r.band_lo[0]), int(r.band_hi[0])] == case["band"]
    kept = np.zeros(row.shape[1], np.uint8)
    # the mask is the set of the first `count` ranks; check it against idx when idx_cap covers it
    if case["idx_cap"] >= case["count"]:
        kept[case["idx"]] = 1
        assert np.array_equal(r.mask[0], kept)
    assert int(r.mask[0].sum()) == case["count"]


# ---------------------------------------------------------------------------
# Brute force: rank(i) = #{j: z_j > z_i} + #{j < i: z_j == z_i}
# ---------------------------------------------------------------------------

ALPHABET = np.array([-np.inf, -1.0, -0.0, 0.0, 0.5, 1.0, 2.0], dtype=np.float32)


def _brute_ranks(z):
    """z: float64 [B, V] -> rank [B, V] by the counting definition (no sort)."""
    zi = z[:, :, None]
    zj = z[:, None, :]
    V = z.shape[1]
    lower = np.tri(V, V, -1, dtype=bool)  # lower[i, j] = j < i
    gt = (zj > zi).sum(axis=2)
    eq_before = ((zj == zi) & lower[None, :, :]).sum(axis=2)
    return gt + eq_before


def _exhaustive_rows(V, limit=None, seed=0):
    if limit is None or len(ALPHABET) ** V <= limit:
        rows = np.array(list(itertools.product(range(len(ALPHABET)), repeat=V)), dtype=np.int64)
    else:
        rows = np.random.default_rng(seed).integers(0, len(ALPHABET), (limit, V))
    return ALPHABET[rows]


@pytest.mark.parametrize("V", [1, 2, 3, 4, 5, 6])
def test_topk_matches_brute_force_rank_definition(V):
    """Catches: wrong sort direction, ties by descending index, -0/+0 or -inf misordered,
    off-by-one in K, k edge values (<=0, >=V) handled wrongly."""
    z = _exhaustive_rows(V, limit=20000, seed=V)
    B = z.shape[0]
    rank = _brute_ranks(z.astype(np.float64))
    for kval in range(-1, V + 2):
        k = np.full(B, kval, np.int32)
        r = oracle.select(z, "f32", k, None, V)
        K = V if (kval <= 0 or kval >= V) else kval
        assert np.array_equal(r.mask.astype(bool), rank < K), kval
        assert np.all(r.count == K)
        order = np.argsort(rank, axis=1)  # ranks are a permutation: unique order
        assert np.array_equal(r.idx[:, :K], order[:, :K]), kval


def _brute_top_p_cut(vals_sorted, K, p):
    """Minimal prefix with mass >= p, masses summed exactly with math.fsum."""
    if p <= 0.0:
        return 1
    m = vals_sorted[0]
    if m == -math.inf:
        return 1
    e = [math.exp(v - m) for v in vals_sorted[:K]]
    S = math.fsum(e)
    for r in range(K):
        if math.fsum(e[: r + 1]) / S >= p:
            return r + 1
    return K


@pytest.mark.parametrize("V", [1, 2, 3, 4, 5])
def test_top_p_matches_exact_summation_within_band(V):
    """Catches: cut with '>' instead of '>=', missing renormalisation over the top-k set,
    top-p applied before top-k, p compared as a float64 literal instead of the float32 value.
    Also shows that the band captures every rounding-sensitive row."""
    z = _exhaustive_rows(V, limit=3000, seed=10 + V)
    B = z.shape[0]
    rank = _brute_ranks(z.astype(np.float64))
    order = np.argsort(rank, axis=1)
    rng = np.random.default_rng(V)
    for trial in range(4):
        k = rng.integers(-1, V + 2, B).astype(np.int32)
        p = rng.choice(np.array([0.0, 0.2, 0.3, 0.5, 0.6, 0.75, 0.9, 0.999], np.float32), B)
        r = oracle.select(z, "f32", k, p, V)
        for b in range(B):
            K = V if (k[b] <= 0 or k[b] >= V) else int(k[b])
            srt = [float(z[b, i]) for i in order[b]]
            Lb = _brute_top_p_cut(srt, K, float(p[b]))
            lo, hi = int(r.band_lo[b]), int(r.band_hi[b])
            assert lo <= Lb <= hi
            assert lo <= int(r.count[b]) <= hi
            if lo == hi:
                assert int(r.count[b]) == Lb
            assert np.array_equal(np.nonzero(r.mask[b])[0], np.sort(order[b, : r.count[b]]))


# ---------------------------------------------------------------------------
# Library stable sorts on mid-size rows
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kind", ["gauss", "ties16", "smallint", "zeros", "neginf", "heavy",
                                  "equal", "twolevel"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_order_matches_numpy_and_torch_stable_sort(kind, dtype):
    import torch

    x = w.make_rows(6, 3001, dtype, kind, seed=hash((kind, dtype)) % 10000, k=0, p=1.0)
    vals = x.values_f32().astype(np.float64)
    r = oracle.select(x.logits, dtype, x.k, x.p, 3001)
    ref_np = np.argsort(-vals, axis=1, kind="stable")
    assert np.array_equal(r.idx, ref_np)
    _, ref_t = torch.sort(torch.from_numpy(vals), dim=1, descending=True, stable=True)
    assert np.array_equal(r.idx, ref_t.numpy())
    # top-k prefixes of the same order
    for K in (1, 7, 50, 1000, 3000):
        k = np.full(6, K, np.int32)
        rk = oracle.select(x.logits, dtype, k, None, K)
        assert np.array_equal(rk.idx, ref_np[:, :K])


def test_topk_distinct_values_match_torch_topk():
    import torch

    rng = np.random.default_rng(3)
    z = np.stack([rng.permutation(5000) for _ in range(4)]).astype(np.float32) * 0.25 - 300.0
    vals = torch.from_numpy(z.astype(np.float64))
    assert all(len(torch.unique(vals[b])) == 5000 for b in range(4))
    for K in (1, 10, 333):
        r = oracle.select(z, "f32", np.full(4, K, np.int32), None, K)
        ref = torch.topk(vals, K, dim=1, largest=True, sorted=True).indices.numpy()
        assert np.array_equal(r.idx, ref)


# ---------------------------------------------------------------------------
# Closed forms for top-p
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("c", [0.25, 0.5, 1.0, 2.0])
@pytest.mark.parametrize("K", [5, 40, 1000])
def test_top_p_geometric_row_closed_form(c, K):
    """z_i = -c*i: masses r^i with r = e^-c, so the minimal L with
    (1 - r^L) / (1 - r^K) >= p is ceil(ln(1 - p (1 - r^K)) / ln r).
    Catches: a dropped max-subtraction or a sum over the wrong range."""
    V = 1200
    z = (-c * np.arange(V, dtype=np.float64)).astype(np.float32)[None, :]
    r_ = math.exp(-c)
    for p in np.array([0.1, 0.37, 0.5, 0.8, 0.9, 0.95, 0.99], np.float32):
        pd = float(p)
        exact = math.log(1.0 - pd * (1.0 - r_ ** K)) / math.log(r_)
        L = min(max(1, math.ceil(exact)), K)
        res = oracle.select(z, "f32", np.array([K], np.int32), np.array([p]), 8)
        if abs(exact - round(exact)) < 1e-6:
            assert res.band_lo[0] <= L <= res.band_hi[0]
        else:
            assert int(res.count[0]) == L, (c, K, pd)


@pytest.mark.parametrize("K", [3, 7, 64, 999])
def test_top_p_all_equal_row_closed_form(K):
    """All-equal row: every token has mass 1/K, so L = ceil(p K)."""
    V = 1000
    z = np.zeros((1, V), np.float32)
    for p in np.array([0.013, 0.3, 0.501, 0.77, 0.9, 0.999], np.float32):
        pk = float(p) * min(K, V)
        res = oracle.select(z, "f32", np.array([K], np.int32), np.array([p]), 4)
        if abs(pk - round(pk)) > 1e-5 * min(K, V):
            assert int(res.count[0]) == math.ceil(pk)
            assert res.band_lo[0] == res.band_hi[0]
        assert np.array_equal(res.idx[0, : min(4, res.count[0])],
                              np.arange(min(4, res.count[0])))


# ---------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------

def _check_output_invariants(x, r, idx_cap):
    vals = x.values_f32().astype(np.float64)
    for b in range(x.batch):
        n = int(r.count[b])
        kept = np.nonzero(r.mask[b])[0]
        assert len(kept) == n >= 1
        m = min(n, idx_cap)
        ids = r.idx[b, :m]
        assert np.all(r.mask[b, ids] == 1)
        v = vals[b, ids]
        assert np.all(v[:-1] >= v[1:])
        same = v[:-1] == v[1:]
        assert np.all(np.diff(ids)[same] > 0)
        if n < x.vocab:
            assert vals[b, kept].min() >= vals[b, r.mask[b] == 0].max()


@pytest.mark.parametrize("kind", ["gauss", "ties16", "smallint", "neginf", "spike", "flat"])
def test_output_invariants_and_nesting(kind):
    """count == popcount(mask); idx in rank order and inside the mask; every kept value >=
    every dropped value; topk(K) is contained in topk(K+1)."""
    x = w.make_rows(5, 700, "bf16", kind, seed=77)
    r = oracle.select(x.logits, "bf16", x.k, x.p, 700)
    _check_output_invariants(x, r, 700)
    prev = None
    for K in range(1, 60):
        rk = oracle.select(x.logits, "bf16", np.full(5, K, np.int32), None, 0)
        if prev is not None:
            assert np.all(rk.mask >= prev)
            assert np.all(rk.mask.sum(1) == K)
        prev = rk.mask


def test_top_p_monotone_in_p():
    x = w.make_rows(8, 2000, "f32", "gauss_outliers", seed=5, k=0, p=1.0)
    ps = np.linspace(0.05, 0.999, 25).astype(np.float32)
    prev = np.zeros(8, np.int64)
    for p in ps:
        r = oracle.select(x.logits, "f32", None, np.full(8, p, np.float32), 0)
        assert np.all(r.count >= prev)
        prev = r.count.astype(np.int64)


@pytest.mark.parametrize("shift", [4.0, -16.0, 1024.0])
def test_exact_shift_invariance(shift):
    """Adding a constant that is exact in the dtype leaves every output unchanged;
    with shift 1024 a missing max-subtraction overflows exp."""
    x = w.make_rows(6, 1500, "f32", "ties16", seed=9)
    vals = x.values_f32()
    assert np.all(np.abs(vals) < 16)
    y = (vals.astype(np.float64) + shift).astype(np.float32)
    assert np.array_equal(y.astype(np.float64) - shift, vals.astype(np.float64))
    a = oracle.select(vals, "f32", x.k, x.p, 1500)
    b = oracle.select(y, "f32", x.k, x.p, 1500)
    assert np.array_equal(a.mask, b.mask)
    assert np.array_equal(a.idx, b.idx)
    assert np.array_equal(a.count, b.count)


def test_top_k_full_then_top_p_equals_top_p_alone():
    x = w.make_rows(6, 900, "bf16", "gauss_outliers", seed=11, p=0.8)
    a = oracle.select(x.logits, "bf16", np.full(6, 900, np.int32), x.p, 900)
    b = oracle.select(x.logits, "bf16", None, x.p, 900)
    assert np.array_equal(a.mask, b.mask) and np.array_equal(a.idx, b.idx)


def test_rejects_nan_and_pos_inf_with_position():
    z = np.zeros((3, 10), np.float32)
    z[1, 7] = np.nan
    with pytest.raises(oracle.OracleInputError, match="row 1, column 7"):
        oracle.select(z, "f32", None, None, 0)
    z[1, 7] = np.inf
    with pytest.raises(oracle.OracleInputError, match="row 1, column 7"):
        oracle.select(z, "f32", None, None, 0)
    z[1, 7] = -np.inf
    oracle.select(z, "f32", None, None, 0)


def test_threads_do_not_change_results():
    x = w.make_rows(13, 1000, "bf16", "ties16", seed=21)
    a = oracle.select(x.logits, "bf16", x.k, x.p, 100, nthreads=1)
    b = oracle.select(x.logits, "bf16", x.k, x.p, 100, nthreads=5)
    for f in ("mask", "idx", "count", "band_lo", "band_hi"):
        assert np.array_equal(getattr(a, f), getattr(b, f))


# ---------------------------------------------------------------------------
# IEEE binary16 logits: the oracle's own decode of the bit patterns against
# NumPy's float16 -> float32 conversion (exact), over every finite pattern
# ---------------------------------------------------------------------------

def _all_finite_f16_bits():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = b.view(np.float16)
    keep = np.isfinite(v) | (v == -np.inf)
    return b[keep]


def test_f16_decode_matches_numpy_over_every_pattern():
    """Every finite binary16 pattern (and -inf), shuffled into rows: the full
    order, masks and top-p cuts from the f16 bits equal those from the same
    values widened by NumPy and passed as float32."""
    bits = _all_finite_f16_bits()
    rng = np.random.default_rng(5)
    bits = bits[rng.permutation(len(bits))]
    V = 2048
    n = (len(bits) // V) * V
    X16 = bits[:n].reshape(-1, V)
    X32 = X16.view(np.float16).astype(np.float32)
    B = X16.shape[0]
    k = rng.integers(0, V + 1, B).astype(np.int32)
    p = np.where(rng.random(B) < 0.5, rng.uniform(0.01, 1.0, B), 1.0).astype(np.float32)
    a = oracle.select(X16, "f16", k, p, V)
    b = oracle.select(X32, "f32", k, p, V)
    assert np.array_equal(a.count, b.count)
    assert np.array_equal(a.mask, b.mask)
    assert np.array_equal(a.idx, b.idx)
    assert np.array_equal(a.band_lo, b.band_lo) and np.array_equal(a.band_hi, b.band_hi)
    # and the full order is NumPy's stable descending sort of the float64 values
    full = oracle.select(X16, "f16", None, None, V)
    for r in range(0, B, 7):
        want = np.argsort(-X16[r].view(np.float16).astype(np.float64), kind="stable")
        assert np.array_equal(full.idx[r], want)


def test_f16_rejects_nan_and_pos_inf():
    x = np.zeros((2, 8), np.float16)
    x[1, 3] = np.inf
    with pytest.raises(oracle.OracleInputError, match="row 1, column 3"):
        oracle.select(x, "f16", None, None, 4)
    x[1, 3] = np.nan
    with pytest.raises(oracle.OracleInputError):
        oracle.select(x, "f16", None, None, 4)


def test_f16_decoded_values_through_a_closed_form():
    """Each finite binary16 value v with |v| <= 16 (subnormals included) in a
    two-logit row [v, 0]: the kept set's renormalised probability of the
    first logit is 1 / (1 + exp(-v)) for v >= 0 (v is rank 0) and
    1 / (1 + exp(v)) for v < 0 (0 is rank 0), with v from NumPy's conversion.
    A decode that is off in scale, bias or subnormal step moves the value."""
    bits = _all_finite_f16_bits()
    v = bits.view(np.float16).astype(np.float64)
    sel = np.abs(v) <= 16.0
    bits, v = bits[sel], v[sel]
    X = np.zeros((len(bits), 2), np.uint16)
    X[:, 0] = bits
    X[:, 1] = np.float16(0.0).view(np.uint16)
    u = np.zeros(len(bits))
    r = oracle.sample(X, "f16", None, None, u, 2)
    top = r.prob[:, 0].astype(np.float64)
    want = np.where(v >= 0, 1.0 / (1.0 + np.exp(-v)), 1.0 / (1.0 + np.exp(v)))
    np.testing.assert_allclose(top, want, rtol=2e-7, atol=0)
    # subnormals are not flushed: the smallest one still moves the rank-0 logit
    sub = (np.abs(v) > 0) & (np.abs(v) < 2.0**-14)
    assert np.any(sub)
    assert np.all(r.idx[sub & (v > 0), 0] == 0) and np.all(r.idx[sub & (v < 0), 0] == 1)
