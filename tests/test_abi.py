"""The C-ABI library: it loads, exports every function include/qrita.h declares,
and rejects bad arguments before touching the GPU (no compute calls here)."""
import ctypes
import os
import re

import pytest

import top_selection_sigma_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qrita.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(qrita_[a-z0-9_]+)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_api():
    names = _declared_functions()
    assert names == ["qrita_philox4x64_10", "qrita_sample", "qrita_select", "qrita_select_ex",
                     "qrita_select_noalloc", "qrita_strerror", "qrita_uniform", "qrita_workspace_bytes"]


def test_library_exports_every_declared_symbol():
    lib = q.lib()
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_strerror():
    assert q.qrita_strerror(0) == "success"
    assert "invalid" in q.qrita_strerror(1)
    assert "workspace" in q.qrita_strerror(2)
    assert q.qrita_strerror(99) == "unknown status"


def test_workspace_bytes():
    a = q.qrita_workspace_bytes(1, 32000, q.QRITA_F32, 64)
    assert a >= 64 + 16384 * 8
    b = q.qrita_workspace_bytes(1024, 201088, q.QRITA_F32, 4096)
    # O(batch) scratch: far below a value+index buffer of the whole batch
    assert b < 1024 * 201088 * 8 // 4
    assert q.qrita_workspace_bytes(10, 100, q.QRITA_BF16, 0) >= 10 * (64 + 100 * 8)
    assert q.qrita_workspace_bytes(-1, 100, 0, 0) == 0
    assert q.qrita_workspace_bytes(1, 0, 0, 0) == 0
    assert q.qrita_workspace_bytes(1, 100, 7, 0) == 0
    assert q.qrita_workspace_bytes(0, 100, 0, 0) == 0 or q.qrita_workspace_bytes(0, 100, 0, 0) < 256


# Fake, aligned, never-dereferenced addresses: every call below must return
# before any HIP call.
FAKE = 0x7F0000000000


def _call(logits=FAKE, batch=4, vocab=100, dtype=0, k=FAKE + 4096, p=FAKE + 8192,
          mask=FAKE + 16384, idx=FAKE + 65536, count=FAKE + 131072, idx_cap=8,
          ws=FAKE + (1 << 20), ws_bytes=None, opt=None):
    lib = q.lib()
    if ws_bytes is None:
        ws_bytes = q.qrita_workspace_bytes(max(batch, 0), max(vocab, 1), 0, idx_cap)
    args = (logits, batch, vocab, dtype, k, p, mask, idx, count, idx_cap, ws, ws_bytes, None)
    if opt is None:
        return lib.qrita_select(*args)
    return lib.qrita_select_ex(*args, ctypes.byref(opt))


@pytest.mark.parametrize("kw,code", [
    (dict(logits=None), q.QRITA_EINVAL),
    (dict(batch=-1), q.QRITA_EINVAL),
    (dict(vocab=0), q.QRITA_EINVAL),
    (dict(vocab=-5), q.QRITA_EINVAL),
    (dict(vocab=1 << 31), q.QRITA_EINVAL),
    (dict(dtype=3), q.QRITA_EINVAL),
    (dict(idx_cap=-1), q.QRITA_EINVAL),
    (dict(count=None), q.QRITA_EINVAL),                    # idx without count
    (dict(mask=None, idx=None, count=None), q.QRITA_EINVAL),
    (dict(logits=FAKE + 4), q.QRITA_EINVAL),               # logits not 16-byte aligned
    (dict(mask=FAKE + 16384 + 8), q.QRITA_EINVAL),         # mask not 16-byte aligned
    (dict(k=FAKE + 4096 + 2), q.QRITA_EINVAL),
    (dict(ws=None), q.QRITA_EWORKSPACE),
    (dict(ws_bytes=100), q.QRITA_EWORKSPACE),
    (dict(batch=0), q.QRITA_OK),                           # empty batch: no-op
])
def test_argument_errors_return_before_launch(kw, code):
    assert _call(**kw) == code


def test_options_are_validated():
    bad = [q._Options(0, 0.0, 3, 0, 0, 0, None, None, 0, 0, 0), q._Options(0, 0.0, 0, -1, 0, 0, None, None, 0, 0, 0),
           q._Options(0, float("nan"), 0, 0, 0, 0, None, None, 0, 0, 0),
           q._Options(0, 0.0, 0, 0, -3, 0, None, None, 0, 0, 0),
           q._Options(0, 0.0, 0, 0, 0, 0, None, None, 3, 0, 0),
           q._Options(0, 0.0, 0, 0, 0, 0, None, None, 0, 2, 0),
           q._Options(0, 0.0, 0, 0, 0, 0, None, None, 0, 0, 2),
           q._Options(0, 0.0, 0, 0, 0, 0, None, None, 0, 0, -1),
           q._Options(0, 0.0, 0, 0, 0, 0, None, None, 0, 0, 0, 17),
           q._Options(0, 0.0, 0, 0, 0, 0, None, None, 0, 0, 0, -1),
           q._Options(0, 0.0, 0, 0, 0, 0, None, None, 0, 0, 0, 0, 2),
           q._Options(0, 0.0, 0, 0, 0, 0, None, None, 0, 0, 0, 0, 0, 3),
           q._Options(0, 0.0, 0, 0, 0, 0, None, None, 0, 0, 0, 0, 0, -1)]
    for o in bad:
        assert _call(opt=o) == q.QRITA_EINVAL


def test_index_order_rejects_rows_beyond_the_lds_bitmap():
    """Index-ordered output keeps the row's bitmap in LDS: at most 688192
    logits (the heavy tier); longer rows are refused before any HIP call."""
    o = q._Options(0, 0.0, 0, 0, 0, 0, None, None, 0, 0, 1)
    assert _call(vocab=688193, opt=o) == q.QRITA_EINVAL
    assert _call(vocab=1 << 24, opt=o) == q.QRITA_EINVAL
    # the light tier forced on a row beyond its bitmap
    o = q._Options(0, 0.0, 0, 0, 0, 0, None, None, 1, 0, 1)
    assert _call(vocab=400000, opt=o) == q.QRITA_EINVAL


def test_product_path_has_no_cpu_fallback():
    """The binding must not import the oracle or any CPU implementation."""
    import ast

    pkg = os.path.join(ROOT, "top_selection_sigma_amd")
    for fn in os.listdir(pkg):
        if fn.endswith(".py"):
            tree = ast.parse(open(os.path.join(pkg, fn)).read())
            for node in ast.walk(tree):
                if isinstance(node, (ast.Import, ast.ImportFrom)):
                    mods = [a.name for a in node.names] if isinstance(node, ast.Import) else [node.module or ""]
                    for m in mods:
                        assert not m.startswith("oracle"), (fn, m)
                        assert not m.startswith("workloads"), (fn, m)


def test_noalloc_rejects_oversize_and_bad_arguments_before_launch():
    lib = q.lib()
    # 300 x 262144 needs more than the static scratch: refused before any HIP call
    assert lib.qrita_select_noalloc(FAKE, 300, 262144, 1, None, None, None, None, FAKE + 4096, 0, None) == \
        q.QRITA_ESCRATCH
    assert lib.qrita_select_noalloc(None, 4, 100, 0, None, None, None, None, FAKE, 0, None) == q.QRITA_EINVAL
    assert lib.qrita_select_noalloc(FAKE, 4, 100, 9, None, None, None, None, FAKE, 0, None) == q.QRITA_EINVAL
    assert lib.qrita_select_noalloc(FAKE, 0, 100, 0, None, None, None, None, FAKE, 0, None) == q.QRITA_OK
    assert "static scratch" in q.qrita_strerror(q.QRITA_ESCRATCH)


def _sample(token=FAKE + (2 << 20), prob=None, opt=None, **kw):
    lib = q.lib()
    a = dict(logits=FAKE, batch=4, vocab=100, dtype=0, k=FAKE + 4096, p=FAKE + 8192, mask=FAKE + 16384,
             idx=FAKE + 65536, count=FAKE + 131072, idx_cap=8, ws=FAKE + (1 << 20), ws_bytes=None)
    a.update(kw)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = q.qrita_workspace_bytes(max(a["batch"], 0), max(a["vocab"], 1), 0, a["idx_cap"])
    return lib.qrita_sample(a["logits"], a["batch"], a["vocab"], a["dtype"], a["k"], a["p"], 5, 6, token, prob,
                            a["mask"], a["idx"], a["count"], a["idx_cap"], a["ws"], a["ws_bytes"], None,
                            None if opt is None else ctypes.byref(opt))


def test_sample_argument_errors_return_before_launch():
    assert _sample(token=None) == q.QRITA_EINVAL                       # no token output
    assert _sample(token=FAKE + 2) == q.QRITA_EINVAL                   # misaligned token output
    assert _sample(prob=FAKE + (3 << 20), idx=None, count=None) == q.QRITA_EINVAL  # prob without idx
    assert _sample(logits=None) == q.QRITA_EINVAL
    assert _sample(ws=None) == q.QRITA_EWORKSPACE
    assert _sample(opt=q._Options(0, 0.0, 7, 0, 0, 0, None, None, 0, 0, 0)) == q.QRITA_EINVAL
    assert _sample(batch=0) == q.QRITA_OK
    # token alone is a valid output set (checked up to the workspace)
    assert _sample(mask=None, idx=None, count=None, ws=None) == q.QRITA_EWORKSPACE


def test_host_philox_matches_numpy():
    """The library's Philox4x64-10 (the routine its device draw runs) against
    NumPy's independent implementation of the same published generator, over
    counters and keys with every word in use."""
    import numpy as np

    rng = np.random.default_rng(11)
    for t in range(40):
        ctr = [int(x) for x in rng.integers(0, 2**63, 4, dtype=np.int64)]
        if t % 4 == 0:
            ctr = [t, 0, 0, 0]
        if t % 4 == 1:
            ctr = [2**64 - 1, 2**64 - 1, t, 2**63]
        key = [int(x) for x in rng.integers(0, 2**63, 2, dtype=np.int64)]
        if t % 3 == 0:
            key[1] = 0
        c = sum(w << (64 * i) for i, w in enumerate(ctr))
        g = np.random.Philox(counter=(c - 1) % 2**256, key=key[0] | key[1] << 64)
        want = [int(x) for x in g.random_raw(4)]
        assert list(q.qrita_philox4x64_10(ctr, key)) == want, t


def test_host_uniform_matches_oracle_uniforms():
    import numpy as np

    import oracle

    for seed, offset in [(0, 0), (1, 2), (2**64 - 1, 2**63 + 5), (987654321, 12)]:
        u = oracle.uniforms(seed, offset, 9)
        assert [q.qrita_uniform(seed, offset, b) for b in range(9)] == u.tolist()
        assert np.all((u >= 0) & (u < 1))
