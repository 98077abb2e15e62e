"""Python binding of libqrita: exact top-k / top-p candidate-set selection on MI355X.

The functions below carry the C ABI's names (``include/qrita.h``) and only
marshal arguments: tensors become device pointers, the current torch stream
becomes the hipStream_t, and nonzero status codes become exceptions. Every
step of the selection runs in the library's HIP kernels; there is no other
implementation behind these calls, and importing fails loudly if the compiled
library is missing.
"""
from __future__ import annotations

import ctypes
import os
import threading
from dataclasses import dataclass
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqrita.so")

QRITA_F32 = 0
QRITA_BF16 = 1
QRITA_F16 = 2
QRITA_OK = 0
QRITA_EINVAL = 1
QRITA_EWORKSPACE = 2
QRITA_ELAUNCH = 3
QRITA_EUNSUPPORTED = 4
QRITA_ESCRATCH = 5
NOALLOC_SCRATCH_BYTES = 32 << 20
DIAG_FIELDS = 8
DIAG_NAMES = ("t", "tc", "n_t", "n_cand", "path", "hit", "iters", "predicted")

_lib = None
_lock = threading.Lock()


class QritaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {qrita_strerror(status)} (status {status})")


class _Options(ctypes.Structure):
    _fields_ = [
        ("force_miss", ctypes.c_int32),
        ("delta_scale", ctypes.c_float),
        ("pivot_mode", ctypes.c_int32),
        ("slices", ctypes.c_int32),
        ("lds_cap", ctypes.c_int32),
        ("list_cap", ctypes.c_int32),
        ("diag", ctypes.c_void_p),
        ("mid_event", ctypes.c_void_p),
        ("tier", ctypes.c_int32),
        ("mask_mode", ctypes.c_int32),
        ("idx_order", ctypes.c_int32),
        ("chunks", ctypes.c_int32),
        ("pivot_search_only", ctypes.c_int32),
        ("launches", ctypes.c_int32),
    ]


@dataclass
class Options:
    """Mirror of ``qrita_options`` (ablation and test controls)."""

    force_miss: bool = False
    delta_scale: float = 0.0
    pivot_mode: int = 0
    slices: int = 0
    lds_cap: int = 0
    list_cap: int = 0
    diag: object = None       # device int32 tensor [batch, 8] or None
    mid_event: object = None  # torch.cuda.Event (already recorded once) or None
    tier: int = 0             # 0 automatic, 1 light, 2 heavy
    mask_mode: int = 0        # 0 automatic, 1 mask bytes stored one by one
    idx_order: int = 0        # 0 rank order, 1 ascending vocabulary index
    chunks: int = 0           # 0 automatic, 1 no overlap, n row chunks overlapping tail and pass 1
    pivot_search_only: int = 0  # 1: no sort-and-scan path for small candidate sets
    launches: int = 0         # 0 automatic (two), 1 one launch (the tail streams its row), 2 two launches

    def to_c(self) -> _Options:
        return _Options(int(self.force_miss), float(self.delta_scale), int(self.pivot_mode),
                        int(self.slices), int(self.lds_cap), int(self.list_cap),
                        None if self.diag is None else self.diag.data_ptr(),
                        None if self.mid_event is None else self.mid_event.cuda_event,
                        int(self.tier), int(self.mask_mode), int(self.idx_order), int(self.chunks), int(self.pivot_search_only),
                        int(self.launches))


def lib() -> ctypes.CDLL:
    """Load libqrita.so (built in-tree by ``top_selection_sigma_amd.build``)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(f"{LIB_PATH} is missing: build it with "
                                  "`python -m top_selection_sigma_amd.build`")
            L = ctypes.CDLL(LIB_PATH)
            i64, vp, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
            L.qrita_workspace_bytes.restype = sz
            L.qrita_workspace_bytes.argtypes = [i64, i64, ctypes.c_int, i64]
            sel = [vp, i64, i64, ctypes.c_int, vp, vp, vp, vp, vp, i64, vp, sz, vp]
            L.qrita_select.restype = ctypes.c_int
            L.qrita_select.argtypes = sel
            L.qrita_select_ex.restype = ctypes.c_int
            L.qrita_select_ex.argtypes = sel + [ctypes.POINTER(_Options)]
            L.qrita_select_noalloc.restype = ctypes.c_int
            L.qrita_select_noalloc.argtypes = [vp, i64, i64, ctypes.c_int, vp, vp, vp, vp, vp, i64, vp]
            u64 = ctypes.c_uint64
            L.qrita_sample.restype = ctypes.c_int
            L.qrita_sample.argtypes = [vp, i64, i64, ctypes.c_int, vp, vp, u64, u64, vp, vp, vp, vp, vp, i64,
                                       vp, sz, vp, ctypes.POINTER(_Options)]
            L.qrita_philox4x64_10.restype = None
            L.qrita_philox4x64_10.argtypes = [ctypes.POINTER(u64), ctypes.POINTER(u64), ctypes.POINTER(u64)]
            L.qrita_uniform.restype = ctypes.c_double
            L.qrita_uniform.argtypes = [u64, u64, u64]
            L.qrita_strerror.restype = ctypes.c_char_p
            L.qrita_strerror.argtypes = [ctypes.c_int]
            _lib = L
        return _lib


def qrita_strerror(status: int) -> str:
    return lib().qrita_strerror(int(status)).decode()


def qrita_workspace_bytes(batch: int, vocab: int, dtype: int, idx_cap: int) -> int:
    return int(lib().qrita_workspace_bytes(int(batch), int(vocab), int(dtype), int(idx_cap)))


def _stream_ptr(stream) -> Optional[int]:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float32:
        return QRITA_F32
    if t.dtype == torch.bfloat16:
        return QRITA_BF16
    if t.dtype == torch.float16:
        return QRITA_F16
    raise TypeError(f"logits must be float32, bfloat16 or float16, got {t.dtype}")


def qrita_select(logits, k, p, out_mask, out_idx, out_count, idx_cap: int, workspace,
                 stream=None) -> None:
    """Call ``qrita_select`` on torch device tensors (asynchronous on ``stream``)."""
    qrita_select_ex(logits, k, p, out_mask, out_idx, out_count, idx_cap, workspace, stream, None)


def qrita_select_ex(logits, k, p, out_mask, out_idx, out_count, idx_cap: int, workspace,
                    stream=None, options: Optional[Options] = None) -> None:
    if logits.dim() != 2 or not logits.is_contiguous():
        raise ValueError("logits must be a contiguous [batch, vocab] tensor")
    B, V = logits.shape
    ws_bytes = workspace.numel() * workspace.element_size()
    args = (logits.data_ptr(), B, V, dtype_code(logits), _ptr(k), _ptr(p), _ptr(out_mask),
            _ptr(out_idx), _ptr(out_count), int(idx_cap), workspace.data_ptr(), ws_bytes,
            _stream_ptr(stream))
    if options is None:
        st = lib().qrita_select(*args)
    else:
        opt = options.to_c()
        st = lib().qrita_select_ex(*args, ctypes.byref(opt))
    if st != QRITA_OK:
        raise QritaError(st, "qrita_select")


def qrita_select_noalloc(logits, k, p, out_mask, out_idx, out_count, idx_cap: int, stream=None) -> None:
    """Call ``qrita_select_noalloc`` (the library's static scratch as workspace)."""
    if logits.dim() != 2 or not logits.is_contiguous():
        raise ValueError("logits must be a contiguous [batch, vocab] tensor")
    B, V = logits.shape
    st = lib().qrita_select_noalloc(logits.data_ptr(), B, V, dtype_code(logits), _ptr(k), _ptr(p),
                                    _ptr(out_mask), _ptr(out_idx), _ptr(out_count), int(idx_cap),
                                    _stream_ptr(stream))
    if st != QRITA_OK:
        raise QritaError(st, "qrita_select_noalloc")


def qrita_sample(logits, k, p, seed: int, offset: int, out_token, out_prob, out_mask, out_idx, out_count,
                 idx_cap: int, workspace, stream=None, options: Optional[Options] = None) -> None:
    """Call ``qrita_sample``: the selection plus one draw per row from the kept set."""
    if logits.dim() != 2 or not logits.is_contiguous():
        raise ValueError("logits must be a contiguous [batch, vocab] tensor")
    B, V = logits.shape
    ws_bytes = workspace.numel() * workspace.element_size()
    opt = None if options is None else ctypes.byref(options.to_c())
    st = lib().qrita_sample(logits.data_ptr(), B, V, dtype_code(logits), _ptr(k), _ptr(p),
                            int(seed) % 2**64, int(offset) % 2**64, _ptr(out_token), _ptr(out_prob),
                            _ptr(out_mask), _ptr(out_idx), _ptr(out_count), int(idx_cap),
                            workspace.data_ptr(), ws_bytes, _stream_ptr(stream), opt)
    if st != QRITA_OK:
        raise QritaError(st, "qrita_sample")


def qrita_philox4x64_10(counter, key) -> Tuple[int, int, int, int]:
    """Philox4x64-10 of a 4-word counter under a 2-word key (host, through the library)."""
    u64 = ctypes.c_uint64
    c = (u64 * 4)(*[int(x) % 2**64 for x in counter])
    k = (u64 * 2)(*[int(x) % 2**64 for x in key])
    o = (u64 * 4)()
    lib().qrita_philox4x64_10(c, k, o)
    return tuple(int(x) for x in o)


def qrita_uniform(seed: int, offset: int, row: int) -> float:
    """The uniform ``qrita_sample`` draws for ``row`` under (seed, offset)."""
    return float(lib().qrita_uniform(int(seed) % 2**64, int(offset) % 2**64, int(row) % 2**64))


_ws_cache = {}


def workspace_for(batch: int, vocab: int, dtype: int, idx_cap: int, device=None, stream=None):
    """A workspace large enough for this shape, cached per (device, stream).

    Calls on one stream run in order, so they can share a workspace; calls on
    different streams get different ones. The workspace is allocated on that
    stream, so torch reuses its memory only in that stream's order. Its
    contents never matter to the library.
    """
    import torch

    device = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    if stream is None:
        stream = torch.cuda.current_stream(device)
    need = max(qrita_workspace_bytes(batch, vocab, dtype, idx_cap), 256)
    key = (device, stream.cuda_stream)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < need:
        with torch.cuda.stream(stream):
            ws = torch.empty(need, dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def select(logits, k=None, p=None, want_mask: bool = True, idx_cap: Optional[int] = None,
           options: Optional[Options] = None, stream=None) -> Tuple:
    """Allocate outputs and run the selection.

    Returns (mask uint8 [B, V] or None, idx int32 [B, idx_cap] or None, count int32 [B]).
    ``idx_cap`` None means no index output; entries of idx past min(count, idx_cap)
    are unspecified.
    """
    import torch

    B, V = logits.shape
    dev = logits.device
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    idx = None
    cap = 0
    # outputs are allocated on the stream the kernels run on
    with torch.cuda.stream(stream):
        mask = torch.empty((B, V), dtype=torch.uint8, device=dev) if want_mask else None
        if idx_cap is not None and idx_cap > 0:
            cap = int(idx_cap)
            idx = torch.empty((B, cap), dtype=torch.int32, device=dev)
        count = torch.empty(B, dtype=torch.int32, device=dev)
    ws = workspace_for(B, V, dtype_code(logits), cap, dev, stream)
    qrita_select_ex(logits, k, p, mask, idx, count, cap, ws, stream, options)
    return mask, idx, count


def sample(logits, k=None, p=None, seed: int = 0, offset: int = 0, idx_cap: Optional[int] = None,
           want_mask: bool = False, options: Optional[Options] = None, stream=None) -> Tuple:
    """Allocate outputs, select and draw one token per row.

    Returns (token int32 [B], idx int32 [B, idx_cap] or None, prob float32
    [B, idx_cap] or None, count int32 [B], mask uint8 [B, V] or None).
    """
    import torch

    B, V = logits.shape
    dev = logits.device
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    idx = prob = None
    cap = 0
    with torch.cuda.stream(stream):
        token = torch.empty(B, dtype=torch.int32, device=dev)
        mask = torch.empty((B, V), dtype=torch.uint8, device=dev) if want_mask else None
        if idx_cap is not None and idx_cap > 0:
            cap = int(idx_cap)
            idx = torch.empty((B, cap), dtype=torch.int32, device=dev)
            prob = torch.empty((B, cap), dtype=torch.float32, device=dev)
        count = torch.empty(B, dtype=torch.int32, device=dev)
    ws = workspace_for(B, V, dtype_code(logits), cap, dev, stream)
    qrita_sample(logits, k, p, seed, offset, token, prob, mask, idx, count, cap, ws, stream, options)
    return token, idx, prob, count, mask
