"""Seeded random shapes through every entry point, against the fp64 oracle.

Each case draws its own form (decode, prefill, queries against a cached
prefix, decode with a committed candidate or over a rolling cache), dtype,
head counts (group sizes 1 to 16, powers of two and not), head width, batch, capacity, ragged
lengths and window from a fixed seed, so a failure names a reproducible
case.  Tolerances as in test_gpu_parity: max-abs 1e-5 (fp32 storage) and
2e-2 (bf16 storage); index-set records and committed cache cells exact.  Every
case also runs the record-free instantiation, which must give the same output
(and committed caches) bit for bit.
"""
import os

import numpy as np
import pytest
import torch

import gqa_kv_cache_02_amd as gqa
import oracle
from gqa_kv_cache_02_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"
# more cases for a longer run: GQA_RANDOM_CASES=2000 (case i uses seed i)
NCASES = int(os.environ.get("GQA_RANDOM_CASES", "128"))


def _np(t):
    return t.detach().float().cpu().numpy()


def _tol(dtype):
    return 1e-5 if dtype == torch.float32 else 2e-2


def _maxerr(a, b):
    a = np.asarray(a, np.float64)
    return float(np.max(np.abs(a - np.asarray(b, np.float64)))) if a.size else 0.0


def _i32(x):
    return torch.tensor(np.asarray(x), dtype=torch.int32, device=DEV)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gqa.lib()
    yield
    torch.cuda.synchronize()


def draw(case):
    """The shape of one case; every draw comes from a generator seeded by the
    case number."""
    r = np.random.RandomState(9000 + case)
    form = ["decode", "prefill", "prefix", "cache"][case % 4]
    kind = r.choice(["mfma", "mfma", "generic_bf16", "f32"])
    if kind == "mfma":
        dtype, d = torch.bfloat16, int(r.choice([64, 128]))
    elif kind == "generic_bf16":
        dtype, d = torch.bfloat16, int(r.choice([16, 40, 96, 256]))
    else:
        dtype, d = torch.float32, int(r.choice([8, 64, 128, 200]))
    hkv = int(r.choice([1, 2, 4, 8]))
    g = int(r.choice([1, 2, 3, 4, 5, 6, 8, 12, 16]))
    while hkv * g > 64:
        g //= 2
    B = int(r.randint(1, 5))
    window = None if r.rand() < 0.35 else int(r.randint(1, 700))
    return r, dict(form=form, dtype=dtype, d=d, hq=hkv * g, hkv=hkv, B=B, window=window)


@pytest.mark.parametrize("case", range(NCASES))
def test_random_case(case):
    r, s = draw(case)
    dtype, d, hq, hkv, B, w = s["dtype"], s["d"], s["hq"], s["hkv"], s["B"], s["window"]
    tol = _tol(dtype)
    seed = 700 + case
    what = (case, s)
    print("case", what, flush=True)

    if s["form"] == "decode":
        C = int(r.randint(1, 3000))
        seqlens = [int(x) for x in r.randint(0, C + 1, size=B)]
        seqlens[0] = C                                   # one row at full capacity
        q, k, v = synth.decode_inputs(B, C, hq, hkv, d, dtype, seed, DEV)
        rec = torch.full((B, hq, 5), -7, dtype=torch.int32, device=DEV)
        out = gqa.decode(q, k, v, seqlens=_i32(seqlens), window=w, records=rec)
        plain = gqa.decode(q, k, v, seqlens=_i32(seqlens), window=w)
        torch.cuda.synchronize()
        assert torch.equal(plain, out), what
        ref, _, rrec = oracle.decode(_np(q), _np(k), _np(v), seqlens=seqlens, window=w,
                                     want_records=True)
        assert _maxerr(_np(out), ref) <= tol, what
        assert np.array_equal(_np(rec).astype(np.int32), rrec), what

    elif s["form"] == "prefill":
        T = int(r.randint(1, 400))
        C = T + int(r.randint(0, 3)) * 17
        seqlens = [int(x) for x in r.randint(0, T + 1, size=B)]
        seqlens[0] = T
        q, k, v = synth.prefill_inputs(B, T, hq, hkv, d, dtype, seed, DEV, C=C)
        rec = torch.full((B, T, hq, 5), -7, dtype=torch.int32, device=DEV)
        out = gqa.prefill(q, k, v, seqlens=_i32(seqlens), window=w, records=rec)
        plain = gqa.prefill(q, k, v, seqlens=_i32(seqlens), window=w)
        torch.cuda.synchronize()
        assert torch.equal(plain, out), what
        ref, _, rrec = oracle.prefill(_np(q), _np(k), _np(v), seqlens=seqlens, window=w,
                                      want_records=True)
        assert _maxerr(_np(out), ref) <= tol, what
        assert np.array_equal(_np(rec).astype(np.int32), rrec), what

    elif s["form"] == "prefix":
        Tq = int(r.randint(1, 130))
        C = Tq + int(r.randint(0, 1500))
        seqlens = [int(x) for x in r.randint(0, C + 1, size=B)]
        qlens = [int(x) for x in r.randint(0, Tq + 1, size=B)]
        seqlens[0], qlens[0] = C, Tq
        segs = None
        if r.rand() < 0.5:
            # packed segments: per batch row, boundaries drawn over its cells;
            # a row's start is the last boundary at or before its position
            segs = np.zeros((B, Tq), np.int32)
            for b in range(B):
                bounds = np.sort(r.randint(0, max(seqlens[b], 1), size=int(r.randint(0, 4))))
                for i in range(Tq):
                    p = seqlens[b] - qlens[b] + i
                    below = bounds[bounds <= p]
                    segs[b, i] = int(below[-1]) if below.size else 0
        q, k, v = synth.prefill_inputs(B, Tq, hq, hkv, d, dtype, seed, DEV, C=C)
        rec = torch.full((B, Tq, hq, 5), -7, dtype=torch.int32, device=DEV)
        out = gqa.prefill_prefix(q, k, v, seqlens=_i32(seqlens), qlens=_i32(qlens),
                                 seg_starts=None if segs is None else _i32(segs), window=w,
                                 records=rec)
        plain = gqa.prefill_prefix(q, k, v, seqlens=_i32(seqlens), qlens=_i32(qlens),
                                   seg_starts=None if segs is None else _i32(segs), window=w)
        torch.cuda.synchronize()
        assert torch.equal(plain, out), what
        ref, _, rrec = oracle.attend_prefix(_np(q), _np(k), _np(v), seqlens=seqlens,
                                            qlens=qlens, segs=segs, window=w,
                                            want_records=True)
        assert _maxerr(_np(out), ref) <= tol, what
        assert np.array_equal(_np(rec).astype(np.int32), rrec), what

    else:
        ring = bool(r.rand() < 0.5)
        C = int(r.randint(2, 1200))
        if ring:
            w = int(r.randint(1, C + 1))
            seqlens = [int(x) for x in r.randint(1, 4 * C, size=B)]
        else:
            seqlens = [int(x) for x in r.randint(1, C + 1, size=B)]
        candidate = bool(r.rand() < 0.7)
        q, k, v = synth.decode_inputs(B, C, hq, hkv, d, dtype, seed, DEV)
        kn = vn = None
        if candidate:
            kn = synth.randn((B, hkv, d), seed + 50, dtype, DEV)
            vn = synth.randn((B, hkv, d), seed + 51, dtype, DEV)
        k0, v0 = _np(k), _np(v)
        kc, vc = k.clone(), v.clone()
        rec = torch.full((B, hq, 5), -7, dtype=torch.int32, device=DEV)
        out = gqa.decode_cache(q, k, v, k_new=kn, v_new=vn, seqlens=_i32(seqlens), window=w,
                               ring=ring, records=rec)
        plain = gqa.decode_cache(q, kc, vc, k_new=kn, v_new=vn, seqlens=_i32(seqlens), window=w,
                                 ring=ring)
        torch.cuda.synchronize()
        assert torch.equal(plain, out) and torch.equal(kc, k) and torch.equal(vc, v), what
        ref, rk, rv, rrec = oracle.decode_cache(
            _np(q), k0, v0, None if kn is None else _np(kn), None if vn is None else _np(vn),
            seqlens=seqlens, window=w, ring=ring, want_records=True)
        assert _maxerr(_np(out), ref) <= tol, what
        assert np.array_equal(_np(rec).astype(np.int32), rrec), what
        assert np.array_equal(_np(k), rk) and np.array_equal(_np(v), rv), what
