"""Parity of the HIP kernels with the fp64 oracle for queries against a cached
prefix (chunked prefill, packed segments), decode with a committed candidate,
and decode over a rolling cache -- all through the C-ABI.

Tolerances as in test_gpu_parity: max-abs 1e-5 (fp32 storage) and 2e-2 (bf16
storage, fp32 arithmetic); index-set records and cache contents exact.
"""
import numpy as np
import pytest
import torch

import gqa_kv_cache_02_amd as gqa
import oracle
from gqa_kv_cache_02_amd import synth

pytestmark = pytest.mark.gpu

F32_TOL = 1e-5
BF16_TOL = 2e-2
DEV = "cuda"


def _np(t):
    return t.detach().float().cpu().numpy()


def _tol(dtype):
    return F32_TOL if dtype == torch.float32 else BF16_TOL


def _maxerr(a, b):
    a = np.asarray(a, np.float64)
    return float(np.max(np.abs(a - np.asarray(b, np.float64)))) if a.size else 0.0


def _i32(x):
    return None if x is None else torch.tensor(np.asarray(x), dtype=torch.int32, device=DEV)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gqa.lib()
    yield
    torch.cuda.synchronize()


def run_prefix(q, k, v, seqlens=None, qlens=None, segs=None, window=None):
    B, hq, Tq, d = q.shape
    rec = torch.full((B, Tq, hq, 5), -7, dtype=torch.int32, device=DEV)
    out = gqa.prefill_prefix(q, k, v, seqlens=_i32(seqlens), qlens=_i32(qlens),
                             seg_starts=_i32(segs), window=window, records=rec)
    torch.cuda.synchronize()
    return out, rec


def check_prefix(q, k, v, seqlens=None, qlens=None, segs=None, window=None, what=""):
    out, rec = run_prefix(q, k, v, seqlens, qlens, segs, window)
    ref, _, rrec = oracle.attend_prefix(_np(q), _np(k), _np(v), seqlens=seqlens, qlens=qlens,
                                        segs=segs, window=window, want_records=True)
    err = _maxerr(_np(out), ref)
    assert err <= _tol(q.dtype), (what, window, err)
    assert np.array_equal(_np(rec).astype(np.int32), rrec), (what, window)
    return out


# ---------------------------------------------------------------------------
# queries against a cached prefix
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,d", [(torch.float32, 8), (torch.float32, 128), (torch.bfloat16, 40),
                                     (torch.bfloat16, 64), (torch.bfloat16, 128)])
def test_prefix_sweep(dtype, d):
    # new rows at the end of longer caches, ragged t_b, a single new token,
    # more new rows than cells (rows before cell 0), windows across tiles
    B, Tq, C = 4, 70, 333
    seqlens = [333, 200, 50, 30]
    qlens = [70, 1, 50, 70]
    for hq, hkv in ((4, 4), (8, 2), (6, 2)):
        q, k, v = synth.prefill_inputs(B, Tq, hq, hkv, d, dtype, 3100 + d + hq, DEV, C=C)
        for w in (None, 1, 63, 64, 65, 100):
            check_prefix(q, k, v, seqlens, qlens, None, w, (hq, hkv))
        # default lengths: s_b = C, t_b = Tq
        check_prefix(q, k, v, None, None, None, 17, (hq, hkv, "defaults"))


@pytest.mark.parametrize("d", [64, 128])
def test_prefix_full_prompt_is_prefill(d):
    # t_b = s_b = n_b is the ordinary prefill, row for row (same kernel, same
    # arithmetic order: equal bits)
    B, T, hq, hkv = 2, 300, 8, 2
    q, k, v = synth.prefill_inputs(B, T, hq, hkv, d, torch.bfloat16, 3200 + d, DEV)
    n = [300, 131]
    for w in (None, 64):
        a, ra = run_prefix(q, k, v, n, n, None, w)
        b = gqa.prefill(q, k, v, seqlens=_i32(n), window=w)
        torch.cuda.synchronize()
        assert torch.equal(a, b)


def test_prefix_one_token_matches_decode():
    B, C, hq, hkv, d = 3, 1000, 8, 2, 128
    q, k, v = synth.decode_inputs(B, C, hq, hkv, d, torch.bfloat16, 3300, DEV)
    n = [1000, 513, 1]
    for w in (None, 100):
        a, _ = run_prefix(q[:, :, None, :].contiguous(), k, v, n, [1] * B, None, w)
        b = gqa.decode(q, k, v, seqlens=_i32(n), window=w)
        torch.cuda.synchronize()
        assert _maxerr(_np(a)[:, 0], _np(b)) <= BF16_TOL


@pytest.mark.parametrize("d", [64, 128])
def test_prefix_split_key_range(d):
    # few new rows against long caches: the key range of every block is split
    # over several workgroups and merged; ragged lengths leave whole splits
    # empty, rows before cell 0 and windows leave rows with no key in a split
    B, Tq, C = 2, 64, 2000
    for hq, hkv in ((8, 2), (4, 4), (6, 2)):
        q, k, v = synth.prefill_inputs(B, Tq, hq, hkv, d, torch.bfloat16, 3150 + d + hq, DEV, C=C)
        for w in (None, 1000, 64):
            assert gqa.prefill_prefix_workspace_bytes(B, Tq, C, hq, hkv, d, w) > 0 or w == 64
            for seqlens, qlens in (([2000, 1500], [64, 64]), ([2000, 40], [1, 64]), (None, None)):
                check_prefix(q, k, v, seqlens, qlens, None, w, ("split", hq, hkv))
        segs = _packed_segments(B, Tq, 3160 + d, 30) + 1900
        check_prefix(q, k, v, [2000, 2000], [64, 64], segs, None, ("split+segments", hq, hkv))


# ---------------------------------------------------------------------------
# packed segments
# ---------------------------------------------------------------------------

def _packed_segments(B, T, seed, max_len):
    """Segment starts of examples packed back to back (lengths 1..max_len)."""
    rng = np.random.default_rng(seed)
    segs = np.zeros((B, T), np.int32)
    for b in range(B):
        t = 0
        while t < T:
            L = int(rng.integers(1, max_len + 1))
            segs[b, t:t + L] = t
            t += L
    return segs


@pytest.mark.parametrize("dtype,d", [(torch.float32, 8), (torch.bfloat16, 64), (torch.bfloat16, 128)])
def test_segments_sweep(dtype, d):
    B, T = 3, 260
    hq, hkv = 8, 2
    q, k, v = synth.prefill_inputs(B, T, hq, hkv, d, dtype, 3400 + d, DEV)
    n = [260, 190, 77]
    for max_len in (1, 7, 70, 300):
        segs = _packed_segments(B, T, 3500 + max_len, max_len)
        for w in (None, 1, 33, 64, 65):
            check_prefix(q, k, v, n, n, segs, w, ("packed", max_len))
    # arbitrary (not packed) starts, some after their row: those rows are empty
    rng = np.random.default_rng(3600)
    segs = rng.integers(0, T, size=(B, T)).astype(np.int32)
    for w in (None, 40):
        check_prefix(q, k, v, n, n, segs, w, "arbitrary")


@pytest.mark.parametrize("d", [64, 128])
def test_many_head_chunks(d):
    """64 query heads on one KV head: the decode splits them into 4 chunks of
    16, the prefill into 8 chunks of 8 heads, and packed segments (4-wavefront
    workgroups) into 16 chunks of 4; every chunk must land on its own heads."""
    hq, hkv = 64, 1
    B, C = 2, 300
    q, k, v = synth.decode_inputs(B, C, hq, hkv, d, torch.bfloat16, 3800 + d, DEV)
    n = [300, 77]
    for w in (None, 65):
        rec = torch.full((B, hq, 5), -7, dtype=torch.int32, device=DEV)
        out = gqa.decode(q, k, v, seqlens=_i32(n), window=w, records=rec)
        torch.cuda.synchronize()
        ref, _, rrec = oracle.decode(_np(q), _np(k), _np(v), seqlens=n, window=w, want_records=True)
        assert _maxerr(_np(out), ref) <= BF16_TOL, ("decode", w)
        assert np.array_equal(_np(rec).astype(np.int32), rrec), ("decode", w)
    T = 150
    q, k, v = synth.prefill_inputs(B, T, hq, hkv, d, torch.bfloat16, 3810 + d, DEV)
    n = [150, 61]
    for w in (None, 65):
        rec = torch.full((B, T, hq, 5), -7, dtype=torch.int32, device=DEV)
        out = gqa.prefill(q, k, v, seqlens=_i32(n), window=w, records=rec)
        torch.cuda.synchronize()
        ref, _, rrec = oracle.prefill(_np(q), _np(k), _np(v), seqlens=n, window=w, want_records=True)
        assert _maxerr(_np(out), ref) <= BF16_TOL, ("prefill", w)
        assert np.array_equal(_np(rec).astype(np.int32), rrec), ("prefill", w)
    segs = _packed_segments(B, T, 3820 + d, 40)
    check_prefix(q, k, v, n, n, segs, None, ("packed", hq, hkv))


def test_packing_equals_separate_runs():
    hq, hkv, d = 8, 2, 128
    la, lb = 137, 200
    qa, ka, va = synth.prefill_inputs(1, la, hq, hkv, d, torch.bfloat16, 3700, DEV)
    qb, kb, vb = synth.prefill_inputs(1, lb, hq, hkv, d, torch.bfloat16, 3701, DEV)
    q = torch.cat([qa, qb], dim=2).contiguous()
    k = torch.cat([ka, kb], dim=2).contiguous()
    v = torch.cat([va, vb], dim=2).contiguous()
    segs = np.array([[0] * la + [la] * lb], np.int32)
    for w in (None, 50):
        out, _ = run_prefix(q, k, v, [la + lb], [la + lb], segs, w)
        oa = gqa.prefill(qa, ka, va, window=w)
        ob = gqa.prefill(qb, kb, vb, window=w)
        torch.cuda.synchronize()
        assert _maxerr(_np(out)[0, :la], _np(oa)[0]) <= BF16_TOL
        assert _maxerr(_np(out)[0, la:], _np(ob)[0]) <= BF16_TOL


# ---------------------------------------------------------------------------
# decode with a committed candidate, and over a rolling cache
# ---------------------------------------------------------------------------

def run_cache(q, k, v, kn=None, vn=None, seqlens=None, window=None, ring=False, workspace=None):
    B, hq, d = q.shape
    rec = torch.full((B, hq, 5), -7, dtype=torch.int32, device=DEV)
    out = gqa.decode_cache(q, k, v, k_new=kn, v_new=vn, seqlens=_i32(seqlens), window=window,
                           ring=ring, records=rec, workspace=workspace)
    torch.cuda.synchronize()
    return out, rec


def check_cache(q, k, v, kn, vn, seqlens, window, ring, what=""):
    k0, v0 = _np(k), _np(v)
    out, rec = run_cache(q, k, v, kn, vn, seqlens, window, ring)
    ref, kref, vref, rrec = oracle.decode_cache(
        _np(q), k0, v0, None if kn is None else _np(kn), None if vn is None else _np(vn),
        seqlens=seqlens, window=window, ring=ring, want_records=True)
    err = _maxerr(_np(out), ref)
    assert err <= _tol(q.dtype), (what, window, ring, err)
    assert np.array_equal(_np(rec).astype(np.int32), rrec), (what, window, ring)
    # the caches: the committed slot holds the candidate's bits, nothing else moved
    assert np.array_equal(_np(k), kref) and np.array_equal(_np(v), vref), (what, "cache")


def _cand(B, hkv, d, dtype, seed):
    return (synth.randn((B, hkv, d), seed, dtype, DEV), synth.randn((B, hkv, d), seed + 1, dtype, DEV))


@pytest.mark.parametrize("dtype,d", [(torch.float32, 8), (torch.bfloat16, 40), (torch.bfloat16, 64),
                                     (torch.bfloat16, 128)])
def test_decode_candidate(dtype, d):
    B, C, hq, hkv = 9, 700, 8, 2
    seqlens = [700, 513, 129, 128, 127, 33, 32, 1, 0]
    q, k, v = synth.decode_inputs(B, C, hq, hkv, d, dtype, 3800 + d, DEV)
    # stale contents in the candidate's slot: the step must not read them
    for b, n in enumerate(seqlens):
        if n:
            k[b, :, n - 1] = 1000.0
            v[b, :, n - 1] = -1000.0
    kn, vn = _cand(B, hkv, d, dtype, 3900 + d)
    for w in (None, 1, 100):
        check_cache(q, k.clone(), v.clone(), kn, vn, seqlens, w, False, "candidate")


@pytest.mark.parametrize("dtype,d", [(torch.float32, 8), (torch.bfloat16, 64), (torch.bfloat16, 128)])
def test_decode_ring(dtype, d):
    B, hq, hkv = 8, 8, 2
    for w, C in ((100, 100), (100, 107), (256, 256)):
        # wrap points anywhere, including inside a 32-key tile, and n_b < C
        seqlens = [1, w - 1, w, w + 1, 3 * w + 5, 10 * w + 17, C + 31, 7 * C - 3]
        q, k, v = synth.decode_inputs(B, C, hq, hkv, d, dtype, 4000 + w + C + d, DEV)
        check_cache(q, k.clone(), v.clone(), None, None, seqlens, w, True, ("ring", w, C))
        kn, vn = _cand(B, hkv, d, dtype, 4100 + w + d)
        check_cache(q, k.clone(), v.clone(), kn, vn, seqlens, w, True, ("ring+cand", w, C))


def test_ring_streaming_decode():
    # a rolling cache of capacity w filled one candidate per step gives, at
    # every step, the windowed decode of the whole history
    B, hq, hkv, d, w, steps = 2, 8, 2, 64, 48, 130
    ks = synth.randn((B, hkv, steps, d), 4200, torch.bfloat16, DEV)
    vs = synth.randn((B, hkv, steps, d), 4201, torch.bfloat16, DEV)
    qs = synth.randn((steps, B, hq, d), 4202, torch.bfloat16, DEV)
    rk = torch.zeros((B, hkv, w, d), dtype=torch.bfloat16, device=DEV)
    rv = torch.zeros_like(rk)
    ws = torch.empty(max(1, gqa.decode_workspace_bytes(B, w, hq, hkv, d, w)), dtype=torch.uint8,
                     device=DEV)
    kn_np, vn_np = _np(ks), _np(vs)
    for t in range(steps):
        out, _ = run_cache(qs[t].contiguous(), rk, rv, ks[:, :, t].contiguous(),
                           vs[:, :, t].contiguous(), [t + 1] * B, w, True, workspace=ws)
        ref, _, _ = oracle.decode(_np(qs[t]), kn_np[:, :, :t + 1], vn_np[:, :, :t + 1], window=w)
        assert _maxerr(_np(out), ref) <= BF16_TOL, t


# ---------------------------------------------------------------------------
# full-size workloads of the three forms (every element, record and cache cell)
# ---------------------------------------------------------------------------

def test_full_chunked_prefill_t512_c4096():
    cfg = synth.CONFIGS["chunk_b1_tq512_c4096_hq32_hkv8_d128"]
    B, Tq, C, hq, hkv, d = cfg["B"], cfg["Tq"], cfg["C"], cfg["Hq"], cfg["Hkv"], cfg["d"]
    q, k, v = synth.prefill_inputs(B, Tq, hq, hkv, d, torch.bfloat16, cfg["seed"], DEV, C=C)
    out, rec = run_prefix(q, k, v, [C], [Tq], None, None)
    # the instantiation bench.py times (no records), called as it calls it:
    # bit for bit the output of the record-writing one
    ws = torch.empty(max(1, gqa.prefill_prefix_workspace_bytes(B, Tq, C, hq, hkv, d)),
                     dtype=torch.uint8, device=DEV)
    plain = torch.empty_like(out)
    gqa.prefill_prefix(q, k, v, out=plain, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(plain, out)
    # every output element and every row's record against the oracle
    ref, _, rrec = oracle.attend_prefix(_np(q), _np(k), _np(v), seqlens=[C], qlens=[Tq],
                                        want_records=True)
    err = _maxerr(_np(out), ref)
    assert err <= BF16_TOL, err
    r = _np(rec).astype(np.int32)
    assert np.array_equal(r, rrec)
    # closed form of the index sets: row i sits at p = C - Tq + i and reads
    # keys 0..p, whose XOR is p, 1, p + 1 or 0 as p mod 4 is 0, 1, 2, 3
    p = (C - Tq + np.arange(Tq))[None, :, None]
    xor_to = np.where(p % 4 == 0, p, np.where(p % 4 == 1, 1, np.where(p % 4 == 2, p + 1, 0)))
    assert (r[..., 1] == 0).all() and (r[..., 2] == p).all() and (r[..., 3] == p + 1).all()
    assert (r[..., 4] == xor_to).all()


def test_full_packed_prefill_t4096():
    cfg = synth.CONFIGS["packed_b1_t4096_hq32_hkv8_d128"]
    B, T, hq, hkv, d = cfg["B"], cfg["T"], cfg["Hq"], cfg["Hkv"], cfg["d"]
    lo, hi = cfg["seg_len"]
    q, k, v = synth.prefill_inputs(B, T, hq, hkv, d, torch.bfloat16, cfg["seed"], DEV)
    segs = synth.packed_segment_starts(B, T, lo, hi, cfg["seed"]).numpy()
    out, rec = run_prefix(q, k, v, None, None, segs, None)
    # the instantiation bench.py times (no records), called as it calls it
    plain = torch.empty_like(out)
    gqa.prefill_prefix(q, k, v, seg_starts=torch.from_numpy(segs).to(DEV), out=plain)
    torch.cuda.synchronize()
    assert torch.equal(plain, out)
    # every output element and every row's record against the oracle
    ref, _, rrec = oracle.attend_prefix(_np(q), _np(k), _np(v), segs=segs, want_records=True)
    err = _maxerr(_np(out), ref)
    assert err <= BF16_TOL, err
    r = _np(rec).astype(np.int32)
    assert np.array_equal(r, rrec)
    # closed form: cell t reads keys s..t of its own segment (start s), so the
    # count is t - s + 1 and the XOR is that of s..t
    t = np.arange(T)[None, :, None]
    s0 = segs[:, :, None].astype(np.int64)

    def xor_upto(n):  # XOR of 0..n (n >= -1)
        return np.where(n % 4 == 0, n, np.where(n % 4 == 1, 1, np.where(n % 4 == 2, n + 1, 0)))

    assert (r[..., 1] == s0).all() and (r[..., 2] == t).all() and (r[..., 3] == t - s0 + 1).all()
    assert (r[..., 4] == (xor_upto(t) ^ xor_upto(s0 - 1))).all()


def test_full_ring_decode_ragged_w4096():
    cfg = synth.CONFIGS["ring_b32_hq8_hkv2_d64_w4096"]
    B, hq, hkv, d, w = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["window"]
    C = w
    lo, hi = cfg["n"]
    seqlens = synth.ragged_lengths(B, lo, hi, cfg["seed"]).tolist()
    q, k, v = synth.decode_inputs(B, C, hq, hkv, d, torch.bfloat16, cfg["seed"], DEV)
    kn, vn = _cand(B, hkv, d, torch.bfloat16, cfg["seed"] + 50)
    k0, v0 = k.clone(), v.clone()
    out, rec = run_cache(q, k, v, kn, vn, seqlens, w, True)
    # the instantiation bench.py times (no records) on a second copy of the
    # original cache: the same output bit for bit and the same committed cache
    k2, v2 = k0.clone(), v0.clone()
    plain = gqa.decode_cache(q, k2, v2, k_new=kn, v_new=vn,
                             seqlens=torch.tensor(seqlens, dtype=torch.int32, device=DEV),
                             window=w, ring=True)
    torch.cuda.synchronize()
    assert torch.equal(plain, out) and torch.equal(k2, k) and torch.equal(v2, v)
    # every output element, every record and both committed caches against
    # the oracle
    ref, kr, vr, rrec = oracle.decode_cache(_np(q), _np(k0), _np(v0), _np(kn), _np(vn),
                                            seqlens=seqlens, window=w, ring=True,
                                            want_records=True)
    err = _maxerr(_np(out), ref)
    assert err <= BF16_TOL, err
    assert np.array_equal(_np(rec).astype(np.int32), rrec)
    assert np.array_equal(_np(k), kr) and np.array_equal(_np(v), vr)
