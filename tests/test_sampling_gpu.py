"""GPU parity of the draw from the kept set (qrita_sample) against the oracle.

The GPU draws its uniforms itself (Philox4x64-10 on the device); the oracle
takes NumPy's Philox uniforms for the same (seed, offset, row). Per row:
the selection outputs match as for qrita_select; the drawn token is the
oracle's, except on band draws (u within 1e-6 of a cumulative mass), where
its rank lies in the oracle's band, and on top-p band rows (the kept set's
length itself lies in a band), where the token lies in the GPU's kept set;
the probabilities beside the indices agree to 1e-6 relative plus 1e-12.
"""
import numpy as np
import pytest

import oracle
import workloads as w
from parity import GpuOut, check, oracle_for

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def run_sample(x, idx_cap, seed, offset, options=None, want_mask=True):
    import torch

    import top_selection_sigma_amd as q

    dev = torch.device("cuda", 0)
    if x.dtype == "bf16":
        logits = torch.from_numpy(x.logits.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        logits = torch.from_numpy(x.logits).to(dev)
    k = torch.from_numpy(x.k).to(dev)
    p = torch.from_numpy(x.p).to(dev)
    token, idx, prob, count, mask = q.sample(logits, k, p, seed=seed, offset=offset, idx_cap=idx_cap,
                                             want_mask=want_mask, options=options)
    torch.cuda.synchronize()
    f = lambda t: None if t is None else t.cpu().numpy()  # noqa: E731
    return f(token), f(idx), f(prob), f(count), f(mask)


def _rank_of(x, b, t):
    """Rank of token t in row b: #{z > z_t} + #{j < t: z_j == z_t}."""
    if x.dtype == "bf16":
        z = (x.logits[b].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    else:
        z = x.logits[b].astype(np.float64)
    return int(np.sum(z > z[t]) + np.sum(z[:t] == z[t]))


def check_sample(x, idx_cap, seed, offset, got, label):
    token, idx, prob, count, mask = got
    B = x.batch
    ref = oracle_for(x, idx_cap)
    check(x, GpuOut(mask, idx, count, None), ref, idx_cap, label)
    u = oracle.uniforms(seed, offset, B)
    s = oracle.sample(x.logits, x.dtype, x.k, x.p, u, max(idx_cap, 1))
    band_rows = ref.band_lo != ref.band_hi
    n_band_draws = 0
    for b in range(B):
        t = int(token[b])
        assert 0 <= t < x.vocab, f"{label}: row {b} token {t}"
        if band_rows[b]:
            # the kept set itself differs within the top-p band: the token is kept
            if mask is not None:
                assert mask[b, t] == 1, f"{label}: band row {b} token {t} not kept"
            continue
        if s.rank_lo[b] == s.rank_hi[b]:
            assert t == int(s.token[b]), (f"{label}: row {b} token {t} oracle {int(s.token[b])} "
                                          f"u {u[b]!r} count {int(ref.count[b])}")
        else:
            n_band_draws += 1
            rank = _rank_of(x, b, t)
            assert s.rank_lo[b] <= rank <= s.rank_hi[b], f"{label}: row {b} band draw rank {rank}"
        if prob is not None and idx_cap > 0:
            n = min(int(ref.count[b]), idx_cap)
            want = s.prob[b, :n].astype(np.float64)
            gotp = prob[b, :n].astype(np.float64)
            err = np.abs(gotp - want)
            assert np.all(err <= 1e-6 * want + 1e-12), f"{label}: row {b} prob max err {err.max()}"
    return n_band_draws


KINDS = ["gauss", "gauss_outliers", "ties16", "uniform", "heavy", "equal", "twolevel", "smallint", "neginf",
         "allneginf", "zeros", "spike", "flat"]


@pytest.mark.parametrize("search,launches", [(0, 1), (1, 1), (0, 2)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_sample_all_kinds_mixed_controls(dtype, search, launches):
    import top_selection_sigma_amd as q

    for i, kind in enumerate(KINDS):
        x = w.make_rows(24, 6007, dtype, kind, seed=300 + i)
        _say(f"sample {kind} {dtype} search {search} launches {launches}")
        got = run_sample(x, 6007, seed=1000 + i, offset=i,
                         options=q.Options(pivot_search_only=search, launches=launches))
        check_sample(x, 6007, 1000 + i, i, got, f"sample {kind} {dtype} search {search} launches {launches}")


@pytest.mark.parametrize("search", [0, 1])
@pytest.mark.parametrize("kind", ["gauss", "gauss_outliers", "heavy", "ties16"])
def test_sample_keep_all_rows(kind, search):
    """Rows with top-k and top-p off: the draw covers the whole row, so its
    candidates are collected for a mass of 0.999 and the logits left out are
    summed; draws past the candidates' mass take the slow path."""
    import top_selection_sigma_amd as q

    x = w.make_rows(64, 32000, "bf16", kind, seed=77, k=0, p=1.0)
    _say(f"keep-all {kind} search {search}")
    got = run_sample(x, 64, seed=5, offset=9, options=q.Options(pivot_search_only=search))
    n = check_sample(x, 64, 5, 9, got, f"keep-all {kind} search {search}")
    _say(f"band draws {n}")


def test_sample_keep_all_rows_token_only():
    """No mask, no indices: the token is the only output."""
    import torch

    import top_selection_sigma_amd as q

    x = w.make_rows(40, 50000, "f32", "gauss_outliers", seed=8, k=0, p=1.0)
    dev = torch.device("cuda", 0)
    logits = torch.from_numpy(x.logits).to(dev)
    token = torch.empty(40, dtype=torch.int32, device=dev)
    ws = q.workspace_for(40, 50000, q.QRITA_F32, 0, dev)
    q.qrita_sample(logits, None, None, 42, 3, token, None, None, None, None, 0, ws)
    torch.cuda.synchronize()
    u = oracle.uniforms(42, 3, 40)
    s = oracle.sample(x.logits, "f32", None, None, u, 1)
    t = token.cpu().numpy()
    ok = (t == s.token) | (s.rank_lo != s.rank_hi)
    assert np.all(ok), np.nonzero(~ok)[0]


@pytest.mark.parametrize("tier", [1, 2])
@pytest.mark.parametrize("force_miss", [False, True])
def test_sample_tiers_and_fallback(tier, force_miss):
    import top_selection_sigma_amd as q

    x = w.make_rows(16, 20000, "bf16", "ties16", seed=3 + tier)
    x.k[:4] = 0
    x.p[:4] = 1.0
    _say(f"tier {tier} miss {force_miss}")
    got = run_sample(x, 20000, seed=9, offset=tier, options=q.Options(tier=tier, force_miss=force_miss))
    check_sample(x, 20000, 9, tier, got, f"tier {tier} miss {force_miss}")


def test_sample_bitmap_batch():
    """512 rows: the tail writes masks from its LDS bitmap."""
    x = w.make_rows(512, 4099, "bf16", "gauss_outliers", seed=12)
    got = run_sample(x, 4099, seed=2, offset=0)
    check_sample(x, 4099, 2, 0, got, "bitmap batch")


def test_sample_is_deterministic_and_offset_changes_draws():
    x = w.make_rows(256, 8192, "f32", "gauss", seed=21, k=0, p=0.99)
    a = run_sample(x, 0, seed=7, offset=0, want_mask=False)
    b = run_sample(x, 0, seed=7, offset=0, want_mask=False)
    c = run_sample(x, 0, seed=7, offset=1, want_mask=False)
    d = run_sample(x, 0, seed=8, offset=0, want_mask=False)
    assert np.array_equal(a[0], b[0])
    assert np.mean(a[0] != c[0]) > 0.5
    assert np.mean(a[0] != d[0]) > 0.5


def test_sample_duplicate_heavy_rows_draw_lowest_kept_duplicates():
    """Ties at the top-k boundary: draws land only on the kept (lowest-index)
    duplicates, with equal probabilities."""
    B, V = 64, 5000
    logits = np.zeros((B, V), np.float32)
    logits[:, ::7] = 1.0  # 715 tokens tied at the top
    from workloads.gen import Inputs

    x = Inputs("ties_top", "f32", logits, np.full(B, 100, np.int32), np.ones(B, np.float32))
    got = run_sample(x, 128, seed=3, offset=4)
    check_sample(x, 128, 3, 4, got, "top ties")
    token, idx, prob = got[0], got[1], got[2]
    assert np.all(token % 7 == 0) and np.all(token < 7 * 100)
    np.testing.assert_allclose(prob[:, :100], 0.01, rtol=1e-6)


@pytest.mark.parametrize("tier,B", [(1, 700), (2, 400)])
def test_sample_counted_tail_rows(tier, B):
    """Batches whose tail workgroups take their rows from the counter: each
    row's draw uses the uniform of its own batch row, whichever workgroup
    handles it."""
    import top_selection_sigma_amd as q

    x = w.make_rows(B, 2003, "bf16", "gauss_outliers", seed=600 + tier)
    _say(f"counted rows sample tier {tier} B {B}")
    got = run_sample(x, 2003, seed=11, offset=4, options=q.Options(tier=tier))
    check_sample(x, 2003, 11, 4, got, f"counted rows sample tier {tier} B {B}")
