"""qrita_select_noalloc (static scratch, no allocation) against qrita_select.

Both entry points run the same kernels, so outputs must be identical: masks,
counts, and the indices up to each row's count. Two calls in a row on the
same GPU, the second with a smaller input, show that what one call leaves in
the shared static scratch does not affect the next.
"""
import numpy as np
import pytest

import workloads as w

pytestmark = pytest.mark.gpu


def _dev_inputs(x):
    import torch

    dev = torch.device("cuda", 0)
    if x.dtype == "bf16":
        logits = torch.from_numpy(x.logits.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        logits = torch.from_numpy(x.logits).to(dev)
    return logits, torch.from_numpy(x.k).to(dev), torch.from_numpy(x.p).to(dev)


def _call(x, cap, noalloc):
    import torch

    import top_selection_sigma_amd as q

    logits, k, p = _dev_inputs(x)
    B, V = x.batch, x.vocab
    dev = logits.device
    # outputs prefilled with values no selection produces
    mask = torch.full((B, V), 7, dtype=torch.uint8, device=dev)
    idx = torch.full((B, cap), -5, dtype=torch.int32, device=dev)
    count = torch.full((B,), -9, dtype=torch.int32, device=dev)
    if noalloc:
        q.qrita_select_noalloc(logits, k, p, mask, idx, count, cap)
    else:
        ws = torch.empty(q.qrita_workspace_bytes(B, V, q.dtype_code(logits), cap), dtype=torch.uint8, device=dev)
        q.qrita_select(logits, k, p, mask, idx, count, cap, ws)
    torch.cuda.synchronize()
    return mask.cpu().numpy(), idx.cpu().numpy(), count.cpu().numpy()


def _same(a, b, cap, label):
    ma, ia, ca = a
    mb, ib, cb = b
    assert np.array_equal(ca, cb), f"{label}: counts differ"
    assert np.all(ca >= 1), f"{label}: counts not written"
    assert np.array_equal(ma, mb), f"{label}: masks differ"
    for r in range(len(ca)):
        n = min(int(ca[r]), cap)
        assert np.array_equal(ia[r, :n], ib[r, :n]), f"{label}: indices differ in row {r}"


def test_noalloc_matches_select_on_two_calls_second_smaller():
    cases = [
        (w.make_rows(48, 100000, "bf16", "gauss_outliers", seed=501), 512, "48 x 100000 bf16"),
        (w.make_rows(5, 20000, "f32", "ties16", seed=502), 300, "5 x 20000 f32"),
    ]
    for x, cap, label in cases:
        print(f"noalloc case {label}", flush=True)
        ref = _call(x, cap, noalloc=False)
        got = _call(x, cap, noalloc=True)
        _same(ref, got, cap, label)


def test_noalloc_rejects_shapes_beyond_its_scratch():
    import top_selection_sigma_amd as q

    # 300 rows of 262144 logits need far more than the static scratch
    need = q.qrita_workspace_bytes(300, 262144, q.QRITA_BF16, 64)
    assert need > q.NOALLOC_SCRATCH_BYTES
    import torch

    dev = torch.device("cuda", 0)
    logits = torch.zeros((300, 262144), dtype=torch.bfloat16, device=dev)
    count = torch.empty(300, dtype=torch.int32, device=dev)
    with pytest.raises(q.QritaError) as e:
        q.qrita_select_noalloc(logits, None, None, None, None, count, 0)
    assert e.value.status == q.QRITA_ESCRATCH


def test_noalloc_matches_select_with_counted_tail_rows():
    """700 rows take their tail rows from the counter in the scratch (zeroed by
    pass 1 in the same call); then a smaller call on the same scratch."""
    cases = [
        (w.make_rows(700, 3001, "bf16", "gauss_outliers", seed=503), 200, "700 x 3001 bf16"),
        (w.make_rows(20, 3001, "bf16", "ties16", seed=504), 200, "20 x 3001 bf16"),
    ]
    for x, cap, label in cases:
        print(f"noalloc case {label}", flush=True)
        ref = _call(x, cap, noalloc=False)
        got = _call(x, cap, noalloc=True)
        _same(ref, got, cap, label)
