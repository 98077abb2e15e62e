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
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(qrita_[a-z_]+)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_api():
    names = _declared_functions()
    assert names == ["qrita_select", "qrita_select_ex", "qrita_select_noalloc", "qrita_strerror",
                     "qrita_workspace_bytes"]


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
    (dict(dtype=2), q.QRITA_EINVAL),
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
    bad = [q._Options(0, 0.0, 3, 0, 0, 0, None, None, 0, 0), q._Options(0, 0.0, 0, -1, 0, 0, None, None, 0, 0),
           q._Options(0, float("nan"), 0, 0, 0, 0, None, None, 0, 0),
           q._Options(0, 0.0, 0, 0, -3, 0, None, None, 0, 0),
           q._Options(0, 0.0, 0, 0, 0, 0, None, None, 3, 0),
           q._Options(0, 0.0, 0, 0, 0, 0, None, None, 0, 2)]
    for o in bad:
        assert _call(opt=o) == q.QRITA_EINVAL


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
