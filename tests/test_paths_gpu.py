"""GPU parity of every tail path and option, through the C ABI, against the oracle.

Each test names the path it drives: the two tail tiers, the whole-row bitmap
mask (with unaligned and odd-length rows) and the byte-scattered mask, the
three pivot placements (key quartiles, value quartiles, one pivot), windowed
index output for kept sets larger than one sort, workspaces left dirty by other
calls or filled with garbage, and calls on two streams.
"""
import numpy as np
import pytest

import workloads as w
from parity import check, oracle_for, run_gpu

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


KINDS = ["gauss", "gauss_outliers", "ties16", "uniform", "heavy", "equal", "twolevel", "smallint",
         "neginf", "allneginf", "zeros", "ascending", "descending", "spike", "flat"]


@pytest.mark.parametrize("search", [0, 1])
@pytest.mark.parametrize("tier", [1, 2])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forced_tiers_all_kinds(tier, dtype, search):
    """Light (1) and heavy (2) tail tiers on the same rows as the default tier,
    with small candidate sets sorted and scanned (search 0) or searched with
    pivots like every other row (search 1)."""
    import top_selection_sigma_amd as q

    for i, kind in enumerate(KINDS):
        x = w.make_rows(6, 7001, dtype, kind, seed=900 + i)
        _say(f"tier {tier} {kind} {dtype} search {search}")
        g = run_gpu(x, 400, options=q.Options(tier=tier, pivot_search_only=search))
        check(x, g, oracle_for(x, 400), 400, f"tier {tier} {kind} {dtype} search {search}")


@pytest.mark.parametrize("V", [3001, 4099, 20000])
@pytest.mark.parametrize("tier", [1, 2])
def test_bitmap_mask_rows(V, tier):
    """512 rows switch the mask to whole-row writes from an LDS bitmap; odd V makes
    every other row start unaligned (head and tail bytes around 16-byte stores)."""
    import top_selection_sigma_amd as q

    x = w.make_rows(512, V, "bf16", "gauss_outliers", seed=V + tier)
    ref = oracle_for(x, 64)
    for search in (0, 1):
        _say(f"bitmap V={V} tier {tier} search {search}")
        g = run_gpu(x, 64, options=q.Options(tier=tier, pivot_search_only=search))
        check(x, g, ref, 64, f"bitmap V={V} tier {tier} search {search}")


@pytest.mark.parametrize("kind", ["ties16", "smallint", "neginf", "equal"])
def test_bitmap_and_scattered_masks_agree_with_oracle(kind):
    """The same 512-row batch with the bitmap mask and with byte-scattered masks
    (pass 1 zero-fills, the tail stores the kept bytes)."""
    import top_selection_sigma_amd as q

    x = w.make_rows(512, 2500, "f32", kind, seed=31)
    ref = oracle_for(x, 100)
    for mode in (0, 1):
        for search in (0, 1):
            _say(f"mask mode {mode} {kind} search {search}")
            g = run_gpu(x, 100, options=q.Options(mask_mode=mode, pivot_search_only=search))
            check(x, g, ref, 100, f"mask mode {mode} {kind} search {search}")


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("kind,dtype", [("ties16", "bf16"), ("gauss_outliers", "bf16"), ("uniform", "f32"),
                                        ("heavy", "bf16"), ("smallint", "f32")])
def test_pivot_modes_match_oracle(mode, kind, dtype):
    """Key quartiles (0), value quartiles (1) and a single key midpoint (2, the
    binary search) all reach the oracle's result."""
    import top_selection_sigma_amd as q

    x = w.make_rows(8, 30000, dtype, kind, seed=12 + mode)
    g = run_gpu(x, 300, options=q.Options(pivot_mode=mode, pivot_search_only=1))
    check(x, g, oracle_for(x, 300), 300, f"pivot mode {mode} {kind}")


@pytest.mark.parametrize("mode", [0, 2])
def test_pivot_modes_on_truncation_misses(mode):
    """The fallback search over the full row with quaternary and binary pivots."""
    import top_selection_sigma_amd as q

    x = w.make_rows(4, 20000, "f32", "uniform", seed=44, k=3000, p=1.0)
    g = run_gpu(x, 3000, options=q.Options(pivot_mode=mode, force_miss=True))
    check(x, g, oracle_for(x, 3000), 3000, f"miss pivot mode {mode}")
    assert np.all(g.diag[:, 4] >= 2)


def test_nan_p_turns_top_p_off():
    x = w.make_rows(8, 5000, "bf16", "gauss_outliers", seed=71)
    x.p[:] = np.float32("nan")
    x.k[:] = np.array([0, 1, 10, 100, 0, 4999, 5000, 37], np.int32)
    g = run_gpu(x, 200)
    ref = oracle_for(x, 200)
    check(x, g, ref, 200, "nan p")
    K = np.where((x.k <= 0) | (x.k >= 5000), 5000, x.k)
    assert np.array_equal(g.count, K)


def test_mask_only_and_idx_only():
    x = w.make_rows(6, 3000, "bf16", "gauss", seed=17)
    ref = oracle_for(x, 50)
    g = run_gpu(x, 0, want_mask=True, want_idx=False)
    check(x, g, ref, 0, "mask only")
    g = run_gpu(x, 50, want_mask=False, want_idx=True)
    check(x, g, ref, 50, "idx only")


@pytest.mark.parametrize("tier", [1, 2])
def test_windowed_index_output(tier):
    """Kept sets larger than one sort (4096 light, 8704 heavy) with heavy ties at
    the boundary: the indices come out in rank windows, each with its own tie
    boundary."""
    import top_selection_sigma_amd as q

    x = w.make_rows(3, 40000, "f32", "smallint", seed=5, k=np.array([10000, 20000, 25000]), p=1.0)
    cap = 22000
    g = run_gpu(x, cap, options=q.Options(tier=tier))
    check(x, g, oracle_for(x, cap), cap, f"windows tier {tier}")


@pytest.mark.parametrize("tier,k", [(1, 8192), (2, 10000)])
def test_windowed_index_output_from_lds_candidates(tier, k):
    """Windows when the row's candidates sit in LDS (heavy-tailed rows whose
    single pass keeps 9-20 K candidates, at most the tier's LDS capacity) and
    the kept set with its boundary duplicates exceeds one sort: the windows'
    gathers and sorts reuse that LDS, so their boundary searches must not read
    it."""
    import top_selection_sigma_amd as q

    x = w.make_rows(4, 262144, "bf16", "heavy", seed=6, k=k, p=1.0)
    g = run_gpu(x, k, options=q.Options(tier=tier))
    check(x, g, oracle_for(x, k), k, f"lds windows tier {tier}")
    _say(f"paths {g.diag[:, 4].tolist()} candidates {g.diag[:, 3].tolist()}")
    assert np.sum(g.diag[:, 4] == 0) >= 3  # most rows on the LDS path


def test_workspace_left_dirty_by_a_smaller_batch():
    """A call on 9 rows of 17 logits, then one on 17 rows of top-p-only rows on
    the same workspace: nothing an earlier call wrote is read by a later one."""
    import torch

    import top_selection_sigma_amd as q

    dev = torch.device("cuda", 0)
    ws = torch.empty(q.qrita_workspace_bytes(17, 64, q.QRITA_F32, 17), dtype=torch.uint8, device=dev)
    a = w.make_rows(9, 17, "f32", "gauss", seed=1, p=1.0)
    a.k[1] = 1
    b = w.make_rows(17, 64, "f32", "gauss_outliers", seed=2, k=0, p=0.9)
    for x in (a, b):
        logits = torch.from_numpy(x.logits).to(dev)
        k = torch.from_numpy(x.k).to(dev)
        p = torch.from_numpy(x.p).to(dev)
        B, V = x.batch, x.vocab
        mask = torch.empty((B, V), dtype=torch.uint8, device=dev)
        idx = torch.empty((B, 17), dtype=torch.int32, device=dev)
        cnt = torch.empty(B, dtype=torch.int32, device=dev)
        diag = torch.zeros((B, q.DIAG_FIELDS), dtype=torch.int32, device=dev)
        q.qrita_select_ex(logits, k, p, mask, idx, cnt, 17, ws, None, q.Options(diag=diag))
        torch.cuda.synchronize()
        from parity import GpuOut

        g = GpuOut(mask.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy(), diag.cpu().numpy())
        check(x, g, oracle_for(x, 17), 17, f"dirty workspace {B}x{V}")
        assert np.all(g.diag[:, 4] <= 1)


def test_workspace_filled_with_garbage():
    """Every word a call reads from the workspace is written earlier in the call."""
    import torch

    import top_selection_sigma_amd as q

    dev = torch.device("cuda", 0)
    x = w.make_rows(40, 20000, "bf16", "ties16", seed=3)
    for fill in (0x00, 0xFF, 0x5A):
        ws = torch.full((q.qrita_workspace_bytes(40, 20000, q.QRITA_BF16, 100),), fill, dtype=torch.uint8,
                        device=dev)
        logits = torch.from_numpy(x.logits.view(np.int16)).to(dev).view(torch.bfloat16)
        k = torch.from_numpy(x.k).to(dev)
        p = torch.from_numpy(x.p).to(dev)
        mask = torch.empty((40, 20000), dtype=torch.uint8, device=dev)
        idx = torch.empty((40, 100), dtype=torch.int32, device=dev)
        cnt = torch.empty(40, dtype=torch.int32, device=dev)
        q.qrita_select(logits, k, p, mask, idx, cnt, 100, ws)
        torch.cuda.synchronize()
        from parity import GpuOut

        g = GpuOut(mask.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy(), None)
        check(x, g, oracle_for(x, 100), 100, f"garbage 0x{fill:02x}")


def test_two_streams_ten_calls_each_are_identical():
    """Two streams, each with its own workspace and outputs, ten calls each,
    interleaved: every output is byte-identical to the others and to the oracle
    (the selection is deterministic; the pages require it)."""
    import torch

    import top_selection_sigma_amd as q

    dev = torch.device("cuda", 0)
    x = w.make_rows(64, 50000, "bf16", "ties16", seed=19)
    logits = torch.from_numpy(x.logits.view(np.int16)).to(dev).view(torch.bfloat16)
    k = torch.from_numpy(x.k).to(dev)
    p = torch.from_numpy(x.p).to(dev)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)]
    outs = []
    for i in range(10):
        for s in streams:
            m, ix, c = q.select(logits, k, p, idx_cap=256, stream=s)
            outs.append((m, ix, c))
    torch.cuda.synchronize()
    ref = oracle_for(x, 256)
    first = None
    from parity import GpuOut

    for m, ix, c in outs:
        g = GpuOut(m.cpu().numpy(), ix.cpu().numpy(), c.cpu().numpy(), None)
        if first is None:
            first = g
            check(x, g, ref, 256, "two streams")
        else:
            assert np.array_equal(g.mask, first.mask)
            assert np.array_equal(g.count, first.count)
            for r in range(x.batch):
                n = min(int(g.count[r]), 256)
                assert np.array_equal(g.idx[r, :n], first.idx[r, :n])
    assert len(q._ws_cache) >= 2


@pytest.mark.parametrize("chunks", [2, 3, 16])
def test_chunked_tails_overlap_and_agree(chunks):
    """Row chunks whose tails run on the library's second stream: the same
    outputs as one chunk, draws included (the draw's counter is the batch row),
    and parity with the oracle; diagnostics land on the right rows."""
    import torch

    import top_selection_sigma_amd as q

    x = w.make_rows(300, 9000, "bf16", "gauss_outliers", seed=60)
    g1 = run_gpu(x, 300, options=q.Options(chunks=1))
    gc = run_gpu(x, 300, options=q.Options(chunks=chunks))
    check(x, gc, oracle_for(x, 300), 300, f"chunks {chunks}")
    assert np.array_equal(g1.mask, gc.mask) and np.array_equal(g1.count, gc.count)
    assert np.array_equal(g1.diag[:, 3], gc.diag[:, 3])
    from parity import device_logits

    dev = torch.device("cuda", 0)
    lg = device_logits(x, dev)
    k = torch.from_numpy(x.k).to(dev)
    p = torch.from_numpy(x.p).to(dev)
    t1 = q.sample(lg, k, p, seed=3, offset=1, idx_cap=300, options=q.Options(chunks=1))
    tc = q.sample(lg, k, p, seed=3, offset=1, idx_cap=300, options=q.Options(chunks=chunks))
    torch.cuda.synchronize()
    assert np.array_equal(t1[0].cpu().numpy(), tc[0].cpu().numpy())
    n = np.minimum(t1[3].cpu().numpy(), 300)
    pa, pb = t1[2].cpu().numpy(), tc[2].cpu().numpy()
    for b in range(300):
        assert np.array_equal(pa[b, :n[b]], pb[b, :n[b]])


@pytest.mark.parametrize("n_kind", ["gauss", "ties16", "smallint", "twolevel", "neginf", "zeros"])
def test_small_sets_sorted_and_searched_agree(n_kind):
    """The sort-and-scan path and the pivot searches give identical outputs
    (masks, indices, counts) on rows whose candidate sets straddle the limits
    of the sort-and-scan path (2048 candidates on the light tier, 4096 on the
    heavy one)."""
    import top_selection_sigma_amd as q

    for B, tier in ((40, 2), (40, 1)):
        x = w.make_rows(B, 60000, "f32", n_kind, seed=8 + tier)
        x.k[:] = np.array([1, 5, 50, 500, 1500, 2047, 0, 0, 1000, 1900] * 4, np.int32)
        x.p[:] = np.array([1.0, 0.9, 0.5, 1.0, 0.99, 1.0, 0.7, 0.999, 1.0, 1.0] * 4, np.float32)
        ref = oracle_for(x, 2100)
        a = run_gpu(x, 2100, options=q.Options(pivot_search_only=0, tier=tier))
        b = run_gpu(x, 2100, options=q.Options(pivot_search_only=1, tier=tier))
        check(x, a, ref, 2100, f"sorted {n_kind} tier {tier}")
        check(x, b, ref, 2100, f"searched {n_kind} tier {tier}")
        assert np.array_equal(a.count, b.count) and np.array_equal(a.mask, b.mask)
        _say(f"{n_kind} tier {tier}: candidates {sorted(a.diag[:, 3].tolist())[::8]}")


@pytest.mark.parametrize("tier,B", [(1, 700), (1, 1024), (2, 300), (2, 512)])
def test_counted_rows_cover_every_row_once(tier, B):
    """Batches of one to two rounds of resident tail workgroups take their rows
    from a counter that pass 1 zeroes: every row is handled exactly once, on a
    mix of cheap and expensive rows (k cycling over 1, 20, 1000, 3000 and top-p
    rows), in two calls in a row."""
    import top_selection_sigma_amd as q

    ks = np.array([1, 20, 1000, 3000, 0], dtype=np.int32)[np.arange(B) % 5]
    ps = np.where(np.arange(B) % 5 == 4, 0.9, 1.0)
    x = w.make_rows(B, 6007, "bf16", "gauss_outliers", seed=B + 31 * tier, k=ks, p=ps)
    ref = oracle_for(x, 3000)
    for call in range(2):
        _say(f"counted rows tier {tier} B {B} call {call}")
        g = run_gpu(x, 3000, options=q.Options(tier=tier))
        check(x, g, ref, 3000, f"counted rows tier {tier} B {B} call {call}")


@pytest.mark.parametrize("launches", [1, 2])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_one_and_two_launches_all_kinds(launches, dtype):
    """One launch (each row's tail workgroup streams the row itself) and two
    launches (the streaming pass over (row, slice) workgroups, then the tail)
    on every kind of row, against the oracle."""
    import top_selection_sigma_amd as q

    for i, kind in enumerate(KINDS):
        x = w.make_rows(6, 7001, dtype, kind, seed=1300 + i)
        _say(f"launches {launches} {kind} {dtype}")
        g = run_gpu(x, 400, options=q.Options(launches=launches))
        check(x, g, oracle_for(x, 400), 400, f"launches {launches} {kind} {dtype}")


@pytest.mark.parametrize("case", ["bitmap", "misses", "overflow", "long_rows"])
def test_one_launch_paths(case):
    """One launch through the tail's other paths: whole-row bitmap masks (512
    rows), forced truncation misses (re-collection and full-row search), a
    list too small for the candidates, and rows long enough for several tiles
    per thread with a ragged end."""
    import top_selection_sigma_amd as q

    if case == "bitmap":
        x = w.make_rows(512, 3001, "bf16", "gauss_outliers", seed=77)
        opts = q.Options(launches=1)
    elif case == "misses":
        x = w.make_rows(24, 20000, "bf16", "gauss_outliers", seed=78)
        opts = q.Options(launches=1, force_miss=True)
    elif case == "overflow":
        x = w.make_rows(24, 20000, "f32", "ties16", seed=79)
        opts = q.Options(launches=1, list_cap=64)
    else:
        x = w.make_rows(8, 262144 + 37, "bf16", "heavy", seed=80)
        opts = q.Options(launches=1)
    ref = oracle_for(x, 300)
    _say(f"one launch {case}")
    g = run_gpu(x, 300, options=opts)
    check(x, g, ref, 300, f"one launch {case}")
