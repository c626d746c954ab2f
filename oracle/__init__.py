"""fp64 CPU oracle for grouped-query attention over a KV cache.

TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the benchmark's
CPU-baseline leg are the only code allowed to import this package.  It shares
nothing with the HIP library: the arithmetic lives in ``gqa_oracle.c`` (plain C,
built with gcc, no HIP headers) and in ``brute.py`` (pure Python).

Inputs are numpy arrays; they are widened to float64 exactly before the call,
so the oracle sees the same values the GPU sees.  See ``gqa_oracle.c`` for the
passages of the pages each function follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gqa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

GCC_CMD = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
           "-o", _LIB, _SRC, "-lm"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no HIP) into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        subprocess.run(GCC_CMD, check=True)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int32)
        i64, i32 = ctypes.c_int64, ctypes.c_int
        L.oracle_kv_head_for_query.argtypes = [i64, i64, i64]
        L.oracle_kv_head_for_query.restype = i64
        L.oracle_window_start.argtypes = [i64, i64, i64]
        L.oracle_window_start.restype = i64
        u64 = ctypes.c_uint64
        L.oracle_kv_cache_bytes.argtypes = [u64] * 6 + [ctypes.POINTER(u64)]
        L.oracle_kv_cache_bytes.restype = i32
        L.oracle_prefill.argtypes = [dp, dp, dp, dp, dp, ip, ip] + [i32] * 7 + [ctypes.c_double]
        L.oracle_prefill.restype = i32
        L.oracle_decode.argtypes = [dp, dp, dp, dp, dp, ip, ip] + [i32] * 6 + [ctypes.c_double]
        L.oracle_decode.restype = i32
        L.oracle_expanded.argtypes = ([dp, dp, dp, dp, ip] + [i32] * 7 + [ctypes.c_double]
                                      + [i32, i32])
        L.oracle_expanded.restype = i32
        L.oracle_attend_prefix.argtypes = ([dp, dp, dp, dp, dp, ip, ip, ip, ip] + [i32] * 7
                                           + [ctypes.c_double])
        L.oracle_attend_prefix.restype = i32
        L.oracle_decode_cache.argtypes = ([dp, dp, dp, dp, dp, dp, ip, ip] + [i32] * 6
                                          + [ctypes.c_double, i32])
        L.oracle_decode_cache.restype = i32
        _lib = L
    return _lib


def threads() -> int:
    """OpenMP threads the oracle's parallel loops use in this process."""
    f = lib().omp_get_max_threads
    f.restype = ctypes.c_int
    return int(f())


class OracleError(RuntimeError):
    def __init__(self, code: int):
        super().__init__(f"oracle refused the call (code {code})")
        self.code = code


def _f64(a) -> np.ndarray:
    a = np.asarray(a, dtype=np.float64)
    return np.ascontiguousarray(a)


def _dp(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _ip(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _seq(seqlens):
    if seqlens is None:
        return None
    return np.ascontiguousarray(np.asarray(seqlens, dtype=np.int32))


def kv_head_for_query(h: int, hq: int, hkv: int):
    g = lib().oracle_kv_head_for_query(h, hq, hkv)
    return None if g < 0 else int(g)


def window_start(t: int, s: int, w: int):
    x = lib().oracle_window_start(t, s, w)
    return None if x < 0 else int(x)


def kv_cache_bytes(L: int, B: int, T: int, hkv: int, d: int, e: int):
    out = ctypes.c_uint64(0)
    rc = lib().oracle_kv_cache_bytes(L, B, T, hkv, d, e, ctypes.byref(out))
    return None if rc else int(out.value)


def prefill(q, k, v, seqlens=None, window=None, scale=None, want_probs=False,
            want_records=False):
    """q [B,Hq,T,d], k/v [B,Hkv,C,d] -> out [B,T,Hq,d] (float64).

    Returns (out, probs or None, records or None)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, hq, T, d = q.shape
    _, hkv, C, _ = k.shape
    w = -1 if window is None else int(window)
    sc = 1.0 / np.sqrt(d) if scale is None else float(scale)
    out = np.zeros((B, T, hq, d), np.float64)
    probs = np.zeros((B, hq, T, C), np.float64) if want_probs else None
    rec = np.zeros((B, T, hq, 5), np.int32) if want_records else None
    sl = _seq(seqlens)
    rc = lib().oracle_prefill(_dp(q), _dp(k), _dp(v), _dp(out),
                              _dp(probs) if probs is not None else None,
                              _ip(rec), _ip(sl), B, T, C, hq, hkv, d, w, sc)
    if rc:
        raise OracleError(rc)
    return out, probs, rec


def decode(q, k, v, seqlens=None, window=None, scale=None, want_probs=False,
           want_records=False):
    """q [B,Hq,d], k/v [B,Hkv,C,d] -> out [B,Hq,d] (float64)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, hq, d = q.shape
    _, hkv, C, _ = k.shape
    w = -1 if window is None else int(window)
    sc = 1.0 / np.sqrt(d) if scale is None else float(scale)
    out = np.zeros((B, hq, d), np.float64)
    probs = np.zeros((B, hq, C), np.float64) if want_probs else None
    rec = np.zeros((B, hq, 5), np.int32) if want_records else None
    sl = _seq(seqlens)
    rc = lib().oracle_decode(_dp(q), _dp(k), _dp(v), _dp(out),
                             _dp(probs) if probs is not None else None,
                             _ip(rec), _ip(sl), B, C, hq, hkv, d, w, sc)
    if rc:
        raise OracleError(rc)
    return out, probs, rec


def expanded(q, k, v, seqlens=None, window=None, scale=None, decode=False, tiled=False):
    """The repeat-then-mask formulation.  Prefill: q [B,Hq,T,d] -> [B,T,Hq,d].
    Decode: q [B,Hq,d] -> [B,Hq,d]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    if decode:
        B, hq, d = q.shape
        tq = 1
    else:
        B, hq, tq, d = q.shape
    _, hkv, C, _ = k.shape
    w = -1 if window is None else int(window)
    sc = 1.0 / np.sqrt(d) if scale is None else float(scale)
    out = np.zeros((B, tq, hq, d), np.float64)
    sl = _seq(seqlens)
    rc = lib().oracle_expanded(_dp(q), _dp(k), _dp(v), _dp(out), _ip(sl), B, tq, C, hq,
                               hkv, d, w, sc, int(decode), int(tiled))
    if rc:
        raise OracleError(rc)
    return out.reshape(B, hq, d) if decode else out


def attend_prefix(q, k, v, seqlens=None, qlens=None, segs=None, window=None, scale=None,
                  want_probs=False, want_records=False):
    """Queries against a cached prefix: q [B,Hq,Tq,d], k/v [B,Hkv,C,d] ->
    out [B,Tq,Hq,d].  seqlens: cells s_b in the cache (new ones included);
    qlens: new query rows t_b; segs [B,Tq]: each query row's segment start.
    Query row i sits at position s_b - t_b + i."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, hq, tq, d = q.shape
    _, hkv, C, _ = k.shape
    w = -1 if window is None else int(window)
    sc = 1.0 / np.sqrt(d) if scale is None else float(scale)
    out = np.zeros((B, tq, hq, d), np.float64)
    probs = np.zeros((B, hq, tq, C), np.float64) if want_probs else None
    rec = np.zeros((B, tq, hq, 5), np.int32) if want_records else None
    sl, ql = _seq(seqlens), _seq(qlens)
    sg = None if segs is None else np.ascontiguousarray(np.asarray(segs, dtype=np.int32))
    if sg is not None and sg.shape != (B, tq):
        raise ValueError("segs must be [B, Tq]")
    rc = lib().oracle_attend_prefix(_dp(q), _dp(k), _dp(v), _dp(out),
                                    _dp(probs) if probs is not None else None, _ip(rec),
                                    _ip(sl), _ip(ql), _ip(sg), B, tq, C, hq, hkv, d, w, sc)
    if rc:
        raise OracleError(rc)
    return out, probs, rec


def decode_cache(q, k, v, knew=None, vnew=None, seqlens=None, window=None, scale=None,
                 ring=False, want_records=False):
    """Decode that first commits a candidate (knew/vnew [B,Hkv,d]) at cell
    n_b - 1 and/or addresses a rolling cache (cell j in slot j mod C).
    Returns (out [B,Hq,d], updated k, updated v, records or None); the
    inputs are not modified."""
    q = _f64(q)
    k, v = _f64(k).copy(), _f64(v).copy()
    B, hq, d = q.shape
    _, hkv, C, _ = k.shape
    if (knew is None) != (vnew is None):
        raise ValueError("knew and vnew go together")
    kn = None if knew is None else _f64(knew)
    vn = None if vnew is None else _f64(vnew)
    w = -1 if window is None else int(window)
    sc = 1.0 / np.sqrt(d) if scale is None else float(scale)
    out = np.zeros((B, hq, d), np.float64)
    rec = np.zeros((B, hq, 5), np.int32) if want_records else None
    sl = _seq(seqlens)
    rc = lib().oracle_decode_cache(_dp(q), _dp(k), _dp(v),
                                   _dp(kn) if kn is not None else None,
                                   _dp(vn) if vn is not None else None, _dp(out), _ip(rec),
                                   _ip(sl), B, C, hq, hkv, d, w, sc, int(bool(ring)))
    if rc:
        raise OracleError(rc)
    return out, k, v, rec
