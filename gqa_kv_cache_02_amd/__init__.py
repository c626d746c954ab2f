"""Grouped-query attention over a KV cache on MI355X (gfx950).

A thin ctypes binding over libgqa.so (declared in include/gqa.h).  It only
marshals arguments: tensor pointers, sizes and the current HIP stream.  Every
step of the computation runs in the library's HIP kernels; there is no CPU or
PyTorch fallback, and every entry point raises if the library is missing.

Layouts (contiguous, d innermost):
    prefill:        q [B, Hq, T, d],  k/v [B, Hkv, C, d] -> out [B, T, Hq, d]
    prefill_prefix: q [B, Hq, Tq, d], k/v [B, Hkv, C, d] -> out [B, Tq, Hq, d]
    decode:         q [B, Hq, d],     k/v [B, Hkv, C, d] -> out [B, Hq, d]
    decode_cache:   as decode, plus k_new/v_new [B, Hkv, d] and a rolling cache
``seqlens`` is an int32 device tensor of per-sequence lengths n_b (decode:
cells in use including the newly appended one).  ``window=None`` means no local
window; ``window >= 1`` counts the current cell and at most window-1 earlier
cells.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgqa.so")

GQA_F32, GQA_BF16 = 0, 1
GQA_NO_WINDOW = -1
KERNELS = {0: "none", 1: "generic", 2: "decode_split", 3: "prefill_mfma"}
STATUS = {
    0: "GQA_OK", 1: "GQA_ERR_NULL", 2: "GQA_ERR_HEADS", 3: "GQA_ERR_ZERO_WINDOW",
    4: "GQA_ERR_HEAD_DIM", 5: "GQA_ERR_DTYPE", 6: "GQA_ERR_SHAPE", 7: "GQA_ERR_OVERFLOW",
    8: "GQA_ERR_WORKSPACE", 9: "GQA_ERR_ALIGN", 10: "GQA_ERR_HIP", 11: "GQA_ERR_SCALE",
}

_lib = None


class GQAError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = _load().gqa_status_string(status).decode()
        super().__init__(f"{where}: {STATUS.get(status, status)} ({msg})")
        self.status = status


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"libgqa.so is not built ({LIB_PATH}); run `python -m gqa_kv_cache_02_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, u64, f32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                              ctypes.c_uint64, ctypes.c_float)
    sz = ctypes.c_size_t
    L.gqa_prefill.argtypes = [vp] * 5 + [i32] * 7 + [f32, i32, vp]
    L.gqa_prefill.restype = ctypes.c_int
    L.gqa_prefill_records.argtypes = [vp] * 5 + [i32] * 7 + [f32, i32, vp, vp]
    L.gqa_prefill_records.restype = ctypes.c_int
    L.gqa_decode_workspace_bytes.argtypes = [i32] * 7
    L.gqa_decode_workspace_bytes.restype = sz
    L.gqa_decode.argtypes = [vp] * 5 + [i32] * 6 + [f32, i32, vp, sz, vp]
    L.gqa_decode.restype = ctypes.c_int
    L.gqa_decode_no_alloc.argtypes = [vp] * 5 + [i32] * 6 + [f32, i32, vp]
    L.gqa_decode_no_alloc.restype = ctypes.c_int
    L.gqa_decode_records.argtypes = [vp] * 5 + [i32] * 6 + [f32, i32, vp, sz, vp, vp]
    L.gqa_decode_records.restype = ctypes.c_int
    L.gqa_prefill_prefix.argtypes = [vp] * 7 + [i32] * 7 + [f32, i32, vp, sz, vp, vp]
    L.gqa_prefill_prefix_workspace_bytes.argtypes = [i32] * 8
    L.gqa_prefill_prefix_workspace_bytes.restype = sz
    L.gqa_prefill_prefix.restype = ctypes.c_int
    L.gqa_decode_cache.argtypes = [vp] * 7 + [i32] * 6 + [f32, i32, i32, vp, sz, vp, vp]
    L.gqa_decode_cache.restype = ctypes.c_int
    L.gqa_prefill_kernel.argtypes = [i32] * 8
    L.gqa_prefill_kernel.restype = ctypes.c_int
    L.gqa_decode_kernel.argtypes = [i32] * 7
    L.gqa_decode_kernel.restype = ctypes.c_int
    L.gqa_kv_head_for_query.argtypes = [i32, i32, i32]
    L.gqa_kv_head_for_query.restype = i32
    L.gqa_window_start.argtypes = [i64, i64, i64]
    L.gqa_window_start.restype = i64
    L.gqa_kv_cache_bytes.argtypes = [u64] * 6 + [ctypes.POINTER(u64)]
    L.gqa_kv_cache_bytes.restype = ctypes.c_int
    L.gqa_status_string.argtypes = [ctypes.c_int]
    L.gqa_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


def lib():
    """The loaded ctypes library (raises if it is not built)."""
    return _load()


# ---------------------------------------------------------------------------
# host helpers
# ---------------------------------------------------------------------------

def kv_head_for_query(h: int, hq: int, hkv: int):
    g = _load().gqa_kv_head_for_query(h, hq, hkv)
    return None if g < 0 else int(g)


def window_start(t: int, seg_start: int, w: int):
    x = _load().gqa_window_start(t, seg_start, w)
    return None if x < 0 else int(x)


def kv_cache_bytes(L: int, B: int, T: int, hkv: int, d: int, e: int) -> int:
    out = ctypes.c_uint64(0)
    rc = _load().gqa_kv_cache_bytes(L, B, T, hkv, d, e, ctypes.byref(out))
    if rc:
        raise GQAError(rc, "kv_cache_bytes")
    return int(out.value)


def decode_workspace_bytes(B, C, hq, hkv, d, window=None, dtype=torch.bfloat16) -> int:
    return int(_load().gqa_decode_workspace_bytes(B, C, hq, hkv, d, _win(window), _dt(dtype)))


def prefill_kernel(B, T, C, hq, hkv, d, window=None, dtype=torch.bfloat16) -> str:
    return KERNELS[_load().gqa_prefill_kernel(B, T, C, hq, hkv, d, _win(window), _dt(dtype))]


def decode_kernel(B, C, hq, hkv, d, window=None, dtype=torch.bfloat16) -> str:
    return KERNELS[_load().gqa_decode_kernel(B, C, hq, hkv, d, _win(window), _dt(dtype))]


# ---------------------------------------------------------------------------
# device entry points
# ---------------------------------------------------------------------------

def _dt(dtype) -> int:
    if dtype == torch.float32:
        return GQA_F32
    if dtype == torch.bfloat16:
        return GQA_BF16
    return 99  # refused by the library with GQA_ERR_DTYPE


def _win(window) -> int:
    return GQA_NO_WINDOW if window is None else int(window)


# The per-call checks below use the cheapest tensor queries (is_cuda,
# get_device, plain integer pointers): a decode call on a small cache runs for
# about as long as the Python side takes to issue it.
def _ptr(t):
    return None if t is None else t.data_ptr()


def _check_tensor(name, t, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        # the library takes device pointers only; host memory is never passed on
        raise ValueError(f"{name} is on {t.device}; the kernels need GPU tensors")
    if t.get_device() != device.index:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device):
    if _raw_stream is not None:
        return _raw_stream(device.index)
    return torch.cuda.current_stream(device).cuda_stream


def _seq(seqlens, B, device):
    if seqlens is None:
        return None
    if not isinstance(seqlens, torch.Tensor):
        seqlens = torch.tensor(list(seqlens), dtype=torch.int32, device=device)
    _check_tensor("seqlens", seqlens, torch.int32, device)
    if seqlens.shape != (B,):
        raise ValueError(f"seqlens must have shape ({B},), got {tuple(seqlens.shape)}")
    return seqlens


def prefill(q, k, v, *, seqlens=None, window=None, scale=None, out=None, records=None):
    """Causal prefill.  q [B,Hq,T,d], k/v [B,Hkv,C,d] -> out [B,T,Hq,d].

    ``records`` (optional int32 [B,T,Hq,5] device tensor) receives the
    index-set records of every row."""
    L = _load()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D")
    B, hq, T, d = q.shape
    hkv, C = k.shape[1], k.shape[2]
    if k.shape != (B, hkv, C, d) or v.shape != k.shape:
        raise ValueError(f"k/v shape {tuple(k.shape)}/{tuple(v.shape)} does not match q {tuple(q.shape)}")
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, q.dtype, dev)
    if out is None:
        out = torch.empty((B, T, hq, d), dtype=q.dtype, device=dev)
    _check_tensor("out", out, q.dtype, dev)
    if out.shape != (B, T, hq, d):
        raise ValueError("out must be [B,T,Hq,d]")
    sl = _seq(seqlens, B, dev)
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(sl), B, T, C, hq, hkv, d,
            _win(window), sc, _dt(q.dtype))
    if records is not None:
        _check_tensor("records", records, torch.int32, dev)
        if records.shape != (B, T, hq, 5):
            raise ValueError("records must be int32 [B,T,Hq,5]")
        rc = L.gqa_prefill_records(*args, _ptr(records), _stream(dev))
    else:
        rc = L.gqa_prefill(*args, _stream(dev))
    if rc:
        raise GQAError(rc, "gqa_prefill")
    return out


def decode(q, k, v, *, seqlens=None, window=None, scale=None, out=None, workspace=None,
           records=None):
    """Single-token decode.  q [B,Hq,d], k/v [B,Hkv,C,d] -> out [B,Hq,d].

    ``workspace`` is an optional uint8 device tensor of at least
    ``decode_workspace_bytes(...)`` bytes (any contents); one is allocated
    when omitted."""
    L = _load()
    if q.dim() != 3 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q must be 3-D and k, v 4-D")
    B, hq, d = q.shape
    hkv, C = k.shape[1], k.shape[2]
    if k.shape != (B, hkv, C, d) or v.shape != k.shape:
        raise ValueError(f"k/v shape {tuple(k.shape)}/{tuple(v.shape)} does not match q {tuple(q.shape)}")
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, q.dtype, dev)
    if out is None:
        out = torch.empty((B, hq, d), dtype=q.dtype, device=dev)
    _check_tensor("out", out, q.dtype, dev)
    if out.shape != (B, hq, d):
        raise ValueError("out must be [B,Hq,d]")
    sl = _seq(seqlens, B, dev)
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    w = _win(window)
    if workspace is None:
        need = int(L.gqa_decode_workspace_bytes(B, C, hq, hkv, d, w, _dt(q.dtype)))
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check_tensor("workspace", workspace, torch.uint8, dev)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(sl), B, C, hq, hkv, d, w, sc,
            _dt(q.dtype), _ptr(workspace), workspace.numel())
    if records is not None:
        _check_tensor("records", records, torch.int32, dev)
        if records.shape != (B, hq, 5):
            raise ValueError("records must be int32 [B,Hq,5]")
        rc = L.gqa_decode_records(*args, _ptr(records), _stream(dev))
    else:
        rc = L.gqa_decode(*args, _stream(dev))
    if rc:
        raise GQAError(rc, "gqa_decode")
    return out


def decode_no_alloc(q, k, v, *, seqlens=None, window=None, scale=None, out=None):
    """decode() without a workspace: the library keeps the split partials in
    its own device array (one per GPU), so the call allocates nothing when
    ``out`` and ``seqlens`` are given as device tensors.  Calls that may
    overlap in time on one GPU share that array and must be serialised."""
    L = _load()
    if q.dim() != 3 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q must be 3-D and k, v 4-D")
    B, hq, d = q.shape
    hkv, C = k.shape[1], k.shape[2]
    if k.shape != (B, hkv, C, d) or v.shape != k.shape:
        raise ValueError(f"k/v shape {tuple(k.shape)}/{tuple(v.shape)} does not match q {tuple(q.shape)}")
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, q.dtype, dev)
    if out is None:
        out = torch.empty((B, hq, d), dtype=q.dtype, device=dev)
    _check_tensor("out", out, q.dtype, dev)
    if out.shape != (B, hq, d):
        raise ValueError("out must be [B,Hq,d]")
    sl = _seq(seqlens, B, dev)
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    rc = L.gqa_decode_no_alloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(sl), B, C, hq, hkv, d,
                               _win(window), sc, _dt(q.dtype), _stream(dev))
    if rc:
        raise GQAError(rc, "gqa_decode_no_alloc")
    return out


def _rowmeta(name, t, shape, device):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        t = torch.tensor(t, dtype=torch.int32, device=device)
    _check_tensor(name, t, torch.int32, device)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def prefill_prefix_workspace_bytes(B, Tq, C, hq, hkv, d, window=None,
                                   dtype=torch.bfloat16) -> int:
    return int(_load().gqa_prefill_prefix_workspace_bytes(B, Tq, C, hq, hkv, d, _win(window),
                                                          _dt(dtype)))


def prefill_prefix(q, k, v, *, seqlens=None, qlens=None, seg_starts=None, window=None,
                   scale=None, out=None, workspace=None, records=None):
    """Queries against a cached prefix (chunked prefill / several new tokens),
    optionally with packed segments.  q [B,Hq,Tq,d], k/v [B,Hkv,C,d] ->
    out [B,Tq,Hq,d].  Query row i of the t_b = qlens[b] new ones sits at cell
    seqlens[b] - t_b + i; seg_starts [B,Tq] gives each row's segment start."""
    L = _load()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D")
    B, hq, Tq, d = q.shape
    hkv, C = k.shape[1], k.shape[2]
    if k.shape != (B, hkv, C, d) or v.shape != k.shape:
        raise ValueError(f"k/v shape {tuple(k.shape)}/{tuple(v.shape)} does not match q {tuple(q.shape)}")
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, q.dtype, dev)
    if out is None:
        out = torch.empty((B, Tq, hq, d), dtype=q.dtype, device=dev)
    _check_tensor("out", out, q.dtype, dev)
    if out.shape != (B, Tq, hq, d):
        raise ValueError("out must be [B,Tq,Hq,d]")
    sl = _rowmeta("seqlens", seqlens, (B,), dev)
    ql = _rowmeta("qlens", qlens, (B,), dev)
    sg = _rowmeta("seg_starts", seg_starts, (B, Tq), dev)
    if records is not None:
        _check_tensor("records", records, torch.int32, dev)
        if records.shape != (B, Tq, hq, 5):
            raise ValueError("records must be int32 [B,Tq,Hq,5]")
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if workspace is None:
        need = int(L.gqa_prefill_prefix_workspace_bytes(B, Tq, C, hq, hkv, d, _win(window),
                                                        _dt(q.dtype)))
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check_tensor("workspace", workspace, torch.uint8, dev)
    rc = L.gqa_prefill_prefix(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(sl), _ptr(ql),
                              _ptr(sg), B, Tq, C, hq, hkv, d, _win(window), sc, _dt(q.dtype),
                              _ptr(workspace), workspace.numel(), _ptr(records), _stream(dev))
    if rc:
        raise GQAError(rc, "gqa_prefill_prefix")
    return out


def decode_cache(q, k, v, *, k_new=None, v_new=None, seqlens=None, window=None, ring=False,
                 scale=None, out=None, workspace=None, records=None):
    """Decode that reads the new cell from k_new/v_new [B,Hkv,d] and commits
    them to the cache (k and v are updated in place), and/or addresses a
    rolling cache (ring=True: cell j in slot j mod C, 1 <= window <= C)."""
    L = _load()
    if q.dim() != 3 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q must be 3-D and k, v 4-D")
    B, hq, d = q.shape
    hkv, C = k.shape[1], k.shape[2]
    if k.shape != (B, hkv, C, d) or v.shape != k.shape:
        raise ValueError(f"k/v shape {tuple(k.shape)}/{tuple(v.shape)} does not match q {tuple(q.shape)}")
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, q.dtype, dev)
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new go together")
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if t is not None:
            _check_tensor(name, t, q.dtype, dev)
            if t.shape != (B, hkv, d):
                raise ValueError(f"{name} must be [B,Hkv,d]")
    if out is None:
        out = torch.empty((B, hq, d), dtype=q.dtype, device=dev)
    _check_tensor("out", out, q.dtype, dev)
    if out.shape != (B, hq, d):
        raise ValueError("out must be [B,Hq,d]")
    sl = _rowmeta("seqlens", seqlens, (B,), dev)
    if records is not None:
        _check_tensor("records", records, torch.int32, dev)
        if records.shape != (B, hq, 5):
            raise ValueError("records must be int32 [B,Hq,5]")
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    w = _win(window)
    if workspace is None:
        need = int(L.gqa_decode_workspace_bytes(B, C, hq, hkv, d, w, _dt(q.dtype)))
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check_tensor("workspace", workspace, torch.uint8, dev)
    rc = L.gqa_decode_cache(_ptr(q), _ptr(k), _ptr(v), _ptr(k_new), _ptr(v_new), _ptr(out),
                            _ptr(sl), B, C, hq, hkv, d, w, sc, _dt(q.dtype), int(bool(ring)),
                            _ptr(workspace), workspace.numel(), _ptr(records), _stream(dev))
    if rc:
        raise GQAError(rc, "gqa_decode_cache")
    return out
