"""Pins for the oracle's draw from the kept set (oracle_sample) and for the
Philox4x64-10 uniforms the draw consumes.

The draw: the token of smallest rank r in the kept set with c_r >= u, c_r the
cumulative softmax mass renormalised over the kept set (the rule the library
header states; the pages motivate returning the whole candidate set for the
sampler that draws from it, "Declaración del Problema"). Pinned by
hand-derived cases (tests/golden/sampling_cases.json), by NumPy's
searchsorted over an exactly summed CDF on small random rows, by the
frequencies of a grid of uniforms, and by the kept set of the already pinned
selection oracle. The uniforms are pinned by NumPy's own Philox.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads as w

HERE = os.path.dirname(os.path.abspath(__file__))


def _cases():
    with open(os.path.join(HERE, "golden", "sampling_cases.json")) as f:
        return json.load(f)["cases"]


def _row(c):
    if "row_log" in c:
        return np.array([math.log(v) for v in c["row_log"]], np.float32)
    return np.array([float(v) for v in c["row"]], np.float32)


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["id"])
def test_hand_derived_draws(case):
    x = _row(case)[None, :]
    V = x.shape[1]
    r = oracle.sample(x, "f32", np.array([case["k"]], np.int32), np.array([case["p"]], np.float32),
                      np.array([case["u"]]), V)
    assert int(r.token[0]) == case["token"]
    assert int(r.rank[0]) == case["rank"]
    if "prob" in case:
        n = int(r.count[0])
        got = r.prob[0, :n].astype(np.float64)
        want = np.array(case["prob"][:n], np.float64)
        assert got.shape == want.shape
        np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-7)


def _exact_cdf_rank(z, kept, u):
    """Independent route: exact softmax over the kept ranks with math.fsum,
    then NumPy's searchsorted (leftmost c_r >= u)."""
    zz = z[kept].astype(np.float64)
    m = zz.max()
    if m == -np.inf:
        return 0
    e = np.exp(zz - m)
    S = math.fsum(e.tolist())
    c = np.array([math.fsum(e[: r + 1].tolist()) / S for r in range(len(e))])
    r = int(np.searchsorted(c, u, side="left"))
    return min(r, len(e) - 1), c


@pytest.mark.parametrize("seed", range(6))
def test_draw_matches_searchsorted_over_exact_cdf(seed):
    rng = np.random.default_rng(seed)
    B, V = 64, 40
    x = w.make_rows(B, V, "f32", ["gauss", "ties16", "smallint", "neginf"][seed % 4], seed=seed)
    k = rng.integers(0, V + 2, B).astype(np.int32)
    p = np.where(rng.random(B) < 0.5, rng.uniform(0.05, 1.0, B), 1.0).astype(np.float32)
    u = rng.random(B)
    sel = oracle.select(x.logits, "f32", k, p, V)
    r = oracle.sample(x.logits, "f32", k, p, u, V)
    assert np.array_equal(r.count, sel.count)
    for b in range(B):
        n = int(sel.count[b])
        kept = sel.idx[b, :n]
        assert np.array_equal(r.idx[b, :n], kept)
        if sel.band_lo[b] != sel.band_hi[b]:
            continue  # the kept set's length is exact here, but its band is not this test's subject
        got = _exact_cdf_rank(x.logits[b].astype(np.float64), kept, u[b])
        rank = got if isinstance(got, int) else got[0]
        if not isinstance(got, int):
            c = got[1]
            # within 1e-9 of a step the two summation orders may disagree
            if np.any(np.abs(c - u[b]) < 1e-9):
                continue
        assert int(r.rank[b]) == rank, (seed, b)
        assert int(r.token[b]) == int(kept[rank])
        assert int(r.rank_lo[b]) <= rank <= int(r.rank_hi[b])


def test_draw_frequencies_follow_the_renormalised_probabilities():
    """A grid of N uniforms u_j = (j + 1/2)/N lands on rank r about p_r N times
    (exactly within one): the draw inverts the CDF of the kept set."""
    x = np.array([[0.0, -0.5, -1.0, -1.0, -3.0, -0.25, 2.0, -10.0]], np.float32)
    k = np.array([6], np.int32)
    p = np.array([0.95], np.float32)
    N = 4000
    u = (np.arange(N) + 0.5) / N
    X = np.repeat(x, N, axis=0)
    r = oracle.sample(X, "f32", np.repeat(k, N), np.repeat(p, N), u, 8)
    L = int(r.count[0])
    assert np.all(r.count == L)
    freq = np.bincount(r.rank, minlength=L)
    probs = r.prob[0, :L].astype(np.float64)
    assert abs(probs.sum() - 1.0) < 1e-6
    assert np.all(np.abs(freq - probs * N) <= 1.0 + 1e-3 * N * 1e-3)
    # ranks are drawn in order of u
    assert np.all(np.diff(r.rank) >= 0)


def test_band_ranks_bracket_the_draw():
    x = w.make_rows(200, 300, "bf16", "ties16", seed=4)
    u = np.random.default_rng(4).random(200)
    r = oracle.sample(x.logits, "bf16", x.k, x.p, u, 300)
    assert np.all(r.rank_lo <= r.rank) and np.all(r.rank <= r.rank_hi)
    assert np.all(r.rank < r.count)


def test_uniforms_are_numpy_philox():
    """oracle.uniforms is NumPy's Philox4x64-10 at counter (row, offset, 0, 0),
    key (seed, 0): checked here against a generator advanced to that counter
    by NumPy's own `advance`."""
    seed, offset = 123456789, 77
    u = oracle.uniforms(seed, offset, 5)
    for b in range(5):
        g = np.random.Philox(counter=0, key=seed)
        # the counter is a 256-bit integer with word 0 least significant; NumPy
        # increments it before the first block
        g.advance(b + (offset << 64) - 1)
        x = int(g.random_raw())
        assert u[b] == (x >> 11) * 2.0**-53
    assert np.all((u >= 0) & (u < 1))
    assert len(set(u.tolist())) == 5
