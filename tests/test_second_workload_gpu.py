"""GPU parity of the float16 dtype, index-ordered output and the second
workload's shapes (top-512 marginals of a block drafter over a full
vocabulary; top-64 pruning of BW x K = 64 x 64 beam proposals), against the
oracle, through the C ABI."""
import numpy as np
import pytest

import oracle
import workloads as w
from parity import GpuOut, check, check_index_order, device_logits, oracle_for, run_gpu

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


KINDS = ["gauss", "gauss_outliers", "ties16", "uniform", "heavy", "equal", "twolevel", "smallint", "neginf",
         "allneginf", "zeros", "ascending", "spike", "flat", "marginals", "f16_edges"]


@pytest.mark.parametrize("tier", [0, 1, 2])
def test_f16_all_kinds(tier):
    import top_selection_sigma_amd as q

    for i, kind in enumerate(KINDS):
        x = w.make_rows(8, 9001, "f16", kind, seed=500 + i)
        _say(f"f16 {kind} tier {tier}")
        g = run_gpu(x, 500, options=q.Options(tier=tier))
        check(x, g, oracle_for(x, 500), 500, f"f16 {kind} tier {tier}")


def test_f16_truncation_misses_and_full_row_fallback():
    import top_selection_sigma_amd as q

    x = w.make_rows(6, 30000, "f16", "f16_edges", seed=2, k=np.array([1, 50, 3000, 0, 0, 29999]),
                    p=np.array([1.0, 0.9, 1.0, 0.5, 0.999, 1.0]))
    for fm in (False, True):
        g = run_gpu(x, 3000, options=q.Options(force_miss=fm))
        check(x, g, oracle_for(x, 3000), 3000, f"f16 miss {fm}")


def test_f16_bitmap_batch():
    x = w.make_rows(512, 12000, "f16", "marginals", seed=8, k=512, p=1.0)
    g = run_gpu(x, 512)
    check(x, g, oracle_for(x, 512), 512, "f16 bitmap")


@pytest.mark.parametrize("tier", [0, 1, 2])
@pytest.mark.parametrize("kind,dtype", [("gauss_outliers", "bf16"), ("ties16", "bf16"), ("smallint", "f32"),
                                        ("neginf", "f32"), ("beam", "f32"), ("marginals", "f16")])
def test_index_order(tier, kind, dtype):
    import top_selection_sigma_amd as q

    x = w.make_rows(16, 12288, dtype, kind, seed=40 + tier)
    x.k[:3] = 0
    x.p[:3] = 1.0  # keep-all rows: indices 0, 1, ...
    for cap in (64, 4096):
        for search in (0, 1):
            _say(f"index order {kind} {dtype} tier {tier} cap {cap} search {search}")
            g = run_gpu(x, cap, options=q.Options(tier=tier, idx_order=1, pivot_search_only=search))
            check_index_order(x, g, oracle_for(x, cap), cap, f"index order {kind} tier {tier} cap {cap} s {search}")


@pytest.mark.parametrize("mask_mode", [0, 1])
def test_index_order_large_batch_masks(mask_mode):
    """512 rows: light tier, mask from the bitmap or scattered bytes."""
    import top_selection_sigma_amd as q

    x = w.make_rows(512, 4096, "f32", "beam", seed=77, k=64, p=1.0)
    g = run_gpu(x, 64, options=q.Options(idx_order=1, mask_mode=mask_mode))
    check_index_order(x, g, oracle_for(x, 64), 64, f"index order 512 rows mask {mask_mode}")


def test_index_order_heavy_tier_for_long_rows():
    """Rows beyond the light tier's bitmap take the heavy tier with index order."""
    import top_selection_sigma_amd as q

    x = w.make_rows(300, 400000, "bf16", "gauss_outliers", seed=5, k=512, p=0.95)
    rows = np.arange(0, 300, 29)
    g = run_gpu(x, 512, options=q.Options(idx_order=1))
    sub = x.take_rows(rows)
    gs = GpuOut(g.mask[rows], g.idx[rows], g.count[rows], None)
    check_index_order(sub, gs, oracle_for(sub, 512), 512, "index order 400000")


def test_index_order_with_sampling_probabilities():
    import torch

    import top_selection_sigma_amd as q

    x = w.make_rows(32, 20000, "f16", "marginals", seed=3, k=300, p=0.9)
    logits = device_logits(x, torch.device("cuda", 0))
    k = torch.from_numpy(x.k).cuda()
    p = torch.from_numpy(x.p).cuda()
    tok, idx, prob, cnt, mask = q.sample(logits, k, p, seed=4, offset=2, idx_cap=300, want_mask=True,
                                         options=q.Options(idx_order=1))
    torch.cuda.synchronize()
    g = GpuOut(mask.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy(), None)
    ref = oracle_for(x, 300)
    check_index_order(x, g, ref, 300, "index order sampling")
    s = oracle.sample(x.logits, "f16", x.k, x.p, oracle.uniforms(4, 2, 32), 300)
    pr = prob.cpu().numpy()
    tk = tok.cpu().numpy()
    for b in range(32):
        if ref.band_lo[b] != ref.band_hi[b]:
            continue
        n = int(ref.count[b])
        # the oracle's probabilities are in rank order: reorder by index
        order = np.argsort(s.idx[b, :n], kind="stable")
        want = s.prob[b, :n][order].astype(np.float64)
        np.testing.assert_allclose(pr[b, :n].astype(np.float64), want, rtol=1e-6, atol=1e-12)
        if s.rank_lo[b] == s.rank_hi[b]:
            assert tk[b] == s.token[b]


def test_marginals_top512_full_shape():
    """The drafter-marginals shape at full size (2048 x 151936 f16, k = 512,
    index order); sampled rows against the oracle."""
    import top_selection_sigma_amd as q

    c = w.EXTRA[0]
    x = w.make_extra(0)
    g = run_gpu(x, 512, options=q.Options(idx_order=1), want_mask=False)
    rows = np.arange(0, c["batch"], 97)
    sub = x.take_rows(rows)
    gs = GpuOut(None, g.idx[rows], g.count[rows], None)
    check_index_order(sub, gs, oracle_for(sub, 512), 512, "marginals full shape")
    assert np.all(g.count == 512)


def test_beam_prune_top64_full_shape():
    """The beam-pruning shape at full size (4096 x 4096 f32, k = 64, index
    order); sampled rows against the oracle, and every row's kept indices name
    64 distinct proposals."""
    import top_selection_sigma_amd as q

    x = w.make_extra(1)
    g = run_gpu(x, 64, options=q.Options(idx_order=1), want_mask=False)
    rows = np.arange(0, x.batch, 61)
    sub = x.take_rows(rows)
    gs = GpuOut(None, g.idx[rows], g.count[rows], None)
    check_index_order(sub, gs, oracle_for(sub, 64), 64, "beam full shape")
    assert np.all(np.diff(g.idx, axis=1) > 0)
