"""The C-ABI library on the host: it loads, exports every declared symbol, its
host helpers reproduce the pages' tables, and every refusal happens on the
host before anything is launched (so these run without a GPU: each call below
returns an error before touching the device)."""
import ctypes
import json
import os
import re

import pytest

import gqa_kv_cache_02_amd as gqa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa.h")

# Refusal codes (include/gqa.h)
OK, NULL, HEADS, ZERO_WINDOW, HEAD_DIM, DTYPE, SHAPE, OVERFLOW, WORKSPACE, ALIGN, HIP, SCALE = range(12)

P = ctypes.c_void_p(4096)  # a non-NULL, 4 KiB-aligned placeholder; never dereferenced
P_ODD = ctypes.c_void_p(4097)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gqa_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = gqa.lib()
    names = declared_functions()
    assert set(names) >= {"gqa_prefill", "gqa_decode", "gqa_decode_workspace_bytes",
                          "gqa_prefill_records", "gqa_decode_records", "gqa_kv_head_for_query",
                          "gqa_window_start", "gqa_kv_cache_bytes", "gqa_status_string"}
    for n in names:
        assert hasattr(L, n), f"{n} declared in gqa.h but not exported"
    # and the exports are the C names, not mangled C++ ones
    out = os.popen(f"nm -D --defined-only {gqa.LIB_PATH}").read()
    for n in names:
        assert re.search(rf"\bT {n}$", out, flags=re.M), n


def test_host_head_map_matches_pages(golden_dir):
    gold = json.load(open(os.path.join(golden_dir, "worked_example_4token.json")))
    assert [gqa.kv_head_for_query(h, 4, 2) for h in range(4)] == gold["head_mapping"]
    assert [gqa.kv_head_for_query(h, 8, 2) for h in range(8)] == [0] * 4 + [1] * 4
    assert [gqa.kv_head_for_query(h, 32, 8) for h in range(32)] == [h // 4 for h in range(32)]
    for bad in ((0, 4, 0), (0, 0, 1), (0, 6, 4), (4, 4, 2), (-1, 4, 2)):
        assert gqa.kv_head_for_query(*bad) is None


def test_host_window_start_matches_pages():
    ws = gqa.window_start
    assert ws(4, 2, 2) == 3 and ws(5, 5, 2) == 5
    assert all(ws(t, 0, 1) == t for t in range(20))
    assert ws(3, 0, 0) is None and ws(3, 4, 2) is None
    assert ws(1, 0, 5) == 0 and ws(9, 7, 5) == 7 and ws(9, 2, 5) == 5
    assert all(ws(t, 0, 10 ** 9) == 0 for t in range(20))


def test_host_kv_cache_bytes_matches_pages(golden_dir):
    gold = json.load(open(os.path.join(golden_dir, "kv_cache_bytes.json")))
    for c in gold["cases"]:
        assert gqa.kv_cache_bytes(c["L"], c["B"], c["T"], c["Hkv"], c["d"], c["e"]) == c["bytes"]
    with pytest.raises(gqa.GQAError) as e:
        gqa.kv_cache_bytes(2 ** 40, 2 ** 30, 1, 1, 1, 1)
    assert e.value.status == OVERFLOW


def _prefill(**kw):
    a = dict(q=P, k=P, v=P, out=P, seqlens=None, B=1, T=4, C=4, Hq=4, Hkv=2, d=8, window=-1,
             scale=0.5, dtype=0)
    a.update(kw)
    return gqa.lib().gqa_prefill(a["q"], a["k"], a["v"], a["out"], a["seqlens"], a["B"], a["T"],
                                 a["C"], a["Hq"], a["Hkv"], a["d"], a["window"], a["scale"],
                                 a["dtype"], None)


def _decode(**kw):
    a = dict(q=P, k=P, v=P, out=P, seqlens=None, B=2, C=64, Hq=8, Hkv=2, d=128, window=-1,
             scale=0.5, dtype=1, ws=P, wsb=1 << 30)
    a.update(kw)
    return gqa.lib().gqa_decode(a["q"], a["k"], a["v"], a["out"], a["seqlens"], a["B"], a["C"],
                                a["Hq"], a["Hkv"], a["d"], a["window"], a["scale"], a["dtype"],
                                a["ws"], a["wsb"], None)


def test_refusals_prefill():
    assert _prefill(Hq=6, Hkv=4) == HEADS
    assert _prefill(Hq=0) == HEADS
    assert _prefill(Hkv=0) == HEADS
    assert _prefill(Hkv=-2) == HEADS
    assert _prefill(window=0) == ZERO_WINDOW
    assert _prefill(d=0) == HEAD_DIM
    assert _prefill(d=257) == HEAD_DIM
    assert _prefill(dtype=7) == DTYPE
    assert _prefill(scale=float("nan")) == SCALE
    assert _prefill(scale=float("inf")) == SCALE
    assert _prefill(T=5, C=4) == SHAPE
    assert _prefill(B=-1) == SHAPE
    assert _prefill(B=2 ** 31 - 1, T=2 ** 30, C=2 ** 30, d=256) == OVERFLOW
    assert _prefill(T=4, C=2 ** 30 + 1) == SHAPE  # past GQA_MAX_CELLS
    assert _prefill(q=None) == NULL
    assert _prefill(out=None) == NULL
    assert _prefill(k=P_ODD) == ALIGN
    # precedence: head counts are reported before the window and the shape
    assert _prefill(Hq=6, Hkv=4, window=0, T=9) == HEADS
    # empty inputs are a no-op, whatever the pointers
    assert _prefill(B=0, q=None, k=None, v=None, out=None) == OK
    assert _prefill(T=0, q=None, k=None, v=None, out=None) == OK
    assert gqa.lib().gqa_prefill_records(P, P, P, P, None, 1, 4, 4, 4, 2, 8, -1, 0.5, 0,
                                         None, None) == NULL


def test_refusals_decode():
    assert _decode(Hq=8, Hkv=3) == HEADS
    assert _decode(window=0) == ZERO_WINDOW
    assert _decode(d=300) == HEAD_DIM
    assert _decode(dtype=-1) == DTYPE
    assert _decode(scale=float("-inf")) == SCALE
    assert _decode(C=-1) == SHAPE
    assert _decode(v=None) == NULL
    assert _decode(seqlens=ctypes.c_void_p(4098)) == ALIGN
    # a cache long enough to be split over several workgroups needs a
    # workspace; a short one has no split and needs none
    need = gqa.lib().gqa_decode_workspace_bytes(2, 8000, 8, 2, 128, -1, 1)
    assert need > 0
    assert gqa.lib().gqa_decode_workspace_bytes(2, 64, 8, 2, 128, -1, 1) == 0
    assert _decode(C=8000, wsb=need - 1) == WORKSPACE
    assert _decode(C=8000, ws=None) == NULL
    assert _decode(C=8000, ws=ctypes.c_void_p(4096 + 16)) == ALIGN
    assert _decode(B=20_000_000) == SHAPE  # more workgroups than a 32-bit grid holds
    # cells past GQA_MAX_CELLS: refused, no kernel, no workspace
    assert _decode(C=2 ** 30 + 1) == SHAPE
    assert gqa.lib().gqa_decode_kernel(2, 2 ** 30 + 1, 8, 2, 128, -1, 1) == 0
    assert gqa.lib().gqa_decode_workspace_bytes(2, 2 ** 30 + 1, 8, 2, 128, -1, 1) == 0
    assert _decode(B=0, q=None, k=None, v=None, out=None) == OK
    assert gqa.lib().gqa_decode_records(P, P, P, P, None, 2, 64, 8, 2, 128, -1, 0.5, 1, P,
                                        1 << 30, None, None) == NULL


def test_matrix_core_shapes_refuse_misaligned_pointers():
    # bf16 with d = 64 or 128 runs the matrix-core kernels, which move 16
    # bytes per lane: a pointer aligned to its element size but not to 16
    # bytes is refused, never rerouted to another kernel
    P2 = ctypes.c_void_p(4096 + 2)
    for name in ("q", "k", "v", "out"):
        assert _decode(**{name: P2}) == ALIGN, name
        assert _decode(C=8000, **{name: P2}) == ALIGN, name
        for d in (64, 128):
            assert _prefill(dtype=1, d=d, **{name: P2}) == ALIGN, (name, d)
            assert _prefix(dtype=1, d=d, **{name: P2}) == ALIGN, (name, d)
    assert _dcache(kn=P2, vn=P) == ALIGN
    assert _dcache(kn=P, vn=P2) == ALIGN
    # the kernel a call runs depends on its arguments only
    assert gqa.decode_kernel(2, 64, 8, 2, 128) == "decode_split"
    assert gqa.prefill_kernel(1, 4, 4, 4, 2, 64) == "prefill_mfma"


def test_workspace_size_and_kernel_choice():
    L = gqa.lib()
    # the split decode path is used for bf16 with d in {64, 128}
    assert gqa.decode_kernel(8, 8000, 32, 8, 128) == "decode_split"
    assert gqa.decode_kernel(32, 32768, 8, 2, 64, window=4096) == "decode_split"
    assert gqa.decode_kernel(8, 8000, 32, 8, 128, dtype=__import__("torch").float32) == "generic"
    assert gqa.decode_kernel(8, 8000, 32, 8, 96) == "generic"
    assert gqa.decode_kernel(0, 10, 4, 2, 64) == "none"
    # workspace: partial outputs, log-sum-exp values and record slots per split
    ws = L.gqa_decode_workspace_bytes(8, 8000, 32, 8, 128, -1, 1)
    assert ws >= 8 * 32 * 128 * 4  # at least one fp32 partial row per (b, h)
    assert L.gqa_decode_workspace_bytes(8, 8000, 32, 8, 96, -1, 1) == 0
    assert L.gqa_decode_workspace_bytes(8, 8000, 32, 8, 128, 0, 1) == 0  # refused arguments
    # a window bounds the work, so it can only shrink the workspace
    assert (L.gqa_decode_workspace_bytes(32, 32768, 8, 2, 64, 4096, 1)
            <= L.gqa_decode_workspace_bytes(32, 32768, 8, 2, 64, -1, 1))


def _prefix(**kw):
    a = dict(q=P, k=P, v=P, out=P, seqlens=None, qlens=None, segs=None, B=1, Tq=4, C=8, Hq=4,
             Hkv=2, d=8, window=-1, scale=0.5, dtype=0, ws=None, wsb=0, rec=None)
    a.update(kw)
    return gqa.lib().gqa_prefill_prefix(a["q"], a["k"], a["v"], a["out"], a["seqlens"],
                                        a["qlens"], a["segs"], a["B"], a["Tq"], a["C"], a["Hq"],
                                        a["Hkv"], a["d"], a["window"], a["scale"], a["dtype"],
                                        a["ws"], a["wsb"], a["rec"], None)


def _dcache(**kw):
    a = dict(q=P, k=P, v=P, kn=None, vn=None, out=P, seqlens=None, B=2, C=64, Hq=8, Hkv=2,
             d=128, window=16, scale=0.5, dtype=1, ring=1, ws=P, wsb=1 << 30, rec=None)
    a.update(kw)
    return gqa.lib().gqa_decode_cache(a["q"], a["k"], a["v"], a["kn"], a["vn"], a["out"],
                                      a["seqlens"], a["B"], a["C"], a["Hq"], a["Hkv"], a["d"],
                                      a["window"], a["scale"], a["dtype"], a["ring"], a["ws"],
                                      a["wsb"], a["rec"], None)


def test_refusals_prefill_prefix():
    assert _prefix(Hq=6, Hkv=4) == HEADS
    assert _prefix(window=0) == ZERO_WINDOW
    assert _prefix(Tq=9, C=8) == SHAPE          # more query rows than cells
    assert _prefix(Tq=4, C=2 ** 30 + 1) == SHAPE  # past GQA_MAX_CELLS
    assert _prefix(q=None) == NULL
    assert _prefix(qlens=ctypes.c_void_p(4098)) == ALIGN
    assert _prefix(segs=ctypes.c_void_p(4098)) == ALIGN
    assert _prefix(rec=ctypes.c_void_p(4098)) == ALIGN
    assert _prefix(B=0, q=None, k=None, v=None, out=None) == OK
    assert _prefix(Tq=0, q=None, k=None, v=None, out=None) == OK
    # few new rows against a long cache split the key range and need a workspace
    L = gqa.lib()
    need = L.gqa_prefill_prefix_workspace_bytes(1, 512, 4096, 32, 8, 128, -1, 1)
    assert need > 0
    assert L.gqa_prefill_prefix_workspace_bytes(1, 4096, 4096, 32, 8, 128, -1, 1) == 0
    assert L.gqa_prefill_prefix_workspace_bytes(1, 512, 4096, 32, 8, 128, -1, 0) == 0  # fp32
    big = dict(B=1, Tq=512, C=4096, Hq=32, Hkv=8, d=128, dtype=1)
    assert _prefix(**big, ws=None, wsb=0) == NULL
    assert _prefix(**big, ws=P, wsb=need - 1) == WORKSPACE
    assert _prefix(**big, ws=ctypes.c_void_p(4096 + 16), wsb=need) == ALIGN


def _prefix_plan(B, T, C, hq, hkv, window):
    """The key-range plan of queries against a cached prefix, restated: with
    fewer than 256 blocks (8 wavefronts: heads x 32-row blocks) and at least 8
    tiles of 64 keys, the key range is cut over ns workgroups while
    blocks x ns stays under 256 and every split keeps 4 tiles.  Returns
    (nsplit, workspace bytes)."""
    r = hq // hkv
    hpw = 8
    while r % hpw:
        hpw //= 2
    rb = 8 // hpw
    units = -(-T // (32 * rb)) * B * hkv * (r // hpw)
    elig = window if 0 < window < C else C
    mt = min(-(-C // 64), (elig + 32 * rb) // 64 + 2)
    if not (0 < units < 256 and mt >= 8):
        return 1, 0
    ns = min(-(-256 // units), mt // 4)
    if ns <= 1:
        return 1, 0
    tps = -(-mt // ns)
    ns = -(-mt // tps)
    rows = ns * B * T * hq
    a = lambda x: (x + 255) // 256 * 256
    return ns, a(rows * 128 * 4) + a(rows * 4) + a(rows * 16)


def test_prefix_plan_splits():
    L = gqa.lib()
    for B, T, C, hq, hkv in ((1, 512, 4096, 32, 8), (2, 64, 700, 8, 2), (2, 64, 2100, 8, 2),
                             (1, 4096, 4096, 32, 8), (2, 64, 2000, 4, 4), (2, 64, 2000, 6, 2),
                             (1, 16, 30000, 64, 8), (3, 200, 5000, 16, 16), (1, 1, 9000, 8, 1)):
        for w in (-1, 64, 700, 1200, 3000):
            ns, want = _prefix_plan(B, T, C, hq, hkv, w)
            got = L.gqa_prefill_prefix_workspace_bytes(B, T, C, hq, hkv, 128, w, 1)
            assert got == want, (B, T, C, hq, hkv, w, ns)
    # the chunked-prefill workload: 64 blocks, 4 splits of 16 tiles
    assert _prefix_plan(1, 512, 4096, 32, 8, -1)[0] == 4


def test_refusals_decode_cache():
    assert _dcache(ring=2) == SHAPE
    assert _dcache(window=-1) == SHAPE           # a rolling cache needs a window
    assert _dcache(window=65) == SHAPE           # ... no longer than the capacity
    assert _dcache(window=0) == ZERO_WINDOW
    assert _dcache(C=2 ** 30 + 1, window=4) == SHAPE  # past GQA_MAX_CELLS
    assert _dcache(kn=P) == NULL                 # the key without the value
    assert _dcache(vn=P) == NULL
    assert _dcache(kn=P_ODD, vn=P) == ALIGN
    assert _dcache(ring=0, window=-1, C=8000, wsb=0) == WORKSPACE
    assert _dcache(B=0, q=None, k=None, v=None, out=None) == OK
    # a rolling cache sizes its workspace from the window, like gqa_decode
    L = gqa.lib()
    need = L.gqa_decode_workspace_bytes(2, 8000, 8, 2, 128, 4000, 1)
    assert need > 0
    assert _dcache(C=8000, window=4000, wsb=need - 1) == WORKSPACE
    assert _dcache(C=8000, window=4000, ws=None) == NULL


def _decode_plan_bytes(B, C, hq, hkv, d, window):
    """The split plan the decode kernel follows, restated: the number of
    splits ns minimises rounds(ns) / ns, rounds = ceil(groups * ns / 256) (one
    workgroup per CU of 256), ties to fewer splits, with at most two
    workgroups per CU in all and at most one split per 128 keys (a 32-key tile
    per wavefront); the permitted range is cut evenly."""
    from fractions import Fraction
    elig = window if 0 < window < C else C
    units = B * hkv * -(-(hq // hkv) // 16)
    max_ns = max(1, min(-(-elig // 128), 512 // units))
    ns = min(range(1, max_ns + 1), key=lambda c: (Fraction(-(-units * c // 256), c), c))
    chunk = max(128, -(-elig // ns))
    nsplit = -(-elig // chunk) if elig > 0 else 0
    rows = B * hq * nsplit
    a256 = lambda x: (x + 255) // 256 * 256
    # without a split every row finishes in one workgroup: no workspace
    need = a256(rows * d * 4) + a256(rows * 4) + a256(rows * 16) if nsplit > 1 else 0
    return need, nsplit, chunk


def test_decode_plan_even_chunks():
    L = gqa.lib()
    shapes = [(8, 8000, 32, 8, 128, -1), (1, 200, 8, 8, 64, -1), (64, 8000, 32, 8, 128, -1),
              (2, 5000, 64, 2, 64, -1), (4, 10000, 8, 2, 128, 1000), (32, 32768, 8, 2, 64, 4096),
              (3, 129, 6, 2, 128, -1), (1, 1, 4, 2, 64, -1), (5, 777, 12, 3, 64, 300)]
    for B, C, hq, hkv, d, w in shapes:
        want, nsplit, chunk = _decode_plan_bytes(B, C, hq, hkv, d, w)
        assert L.gqa_decode_workspace_bytes(B, C, hq, hkv, d, w, 1) == want, (B, C, hq, hkv, d, w)
        elig = w if 0 < w < C else C
        assert chunk >= 128 and (nsplit - 1) * chunk < elig <= nsplit * chunk
    # the headline decode: 4 chunks of 2000 keys for 64 groups, one
    # workgroup per CU; 16 groups (the MQA endpoint) take 16 splits
    assert _decode_plan_bytes(8, 8000, 32, 8, 128, -1)[1:] == (4, 2000)
    assert _decode_plan_bytes(16, 8000, 8, 1, 128, -1)[1:] == (16, 500)
    # 129 groups: 3 splits (387 workgroups, 2 rounds) beat 1 or 2 (1 or 2 rounds of a full range)
    assert _decode_plan_bytes(129, 4000, 4, 1, 64, -1)[1] == 3


def test_binding_refuses_host_tensors():
    """The binding passes device pointers only: CPU tensors are refused in
    Python, before any library call (no CPU path exists to fall back to)."""
    import torch
    q = torch.zeros((1, 4, 4, 8), dtype=torch.float32)
    k = torch.zeros((1, 2, 4, 8), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU tensors"):
        gqa.prefill(q, k, k.clone())
    with pytest.raises(ValueError, match="GPU tensors"):
        gqa.decode(q[:, :, 0].contiguous(), k, k.clone())
    with pytest.raises(ValueError, match="GPU tensors"):
        gqa.prefill_prefix(q, k, k.clone())
    with pytest.raises(ValueError, match="GPU tensors"):
        gqa.decode_cache(q[:, :, 0].contiguous(), k, k.clone())


def test_missing_library_raises(monkeypatch):
    """Without the built library every entry point raises: there is no
    fallback path to run instead."""
    import torch
    monkeypatch.setattr(gqa, "_lib", None)
    monkeypatch.setattr(gqa, "LIB_PATH", "/nonexistent/libgqa.so")
    with pytest.raises(RuntimeError, match="not built"):
        gqa.lib()
    q = torch.zeros((1, 4, 4, 8), dtype=torch.float32)
    k = torch.zeros((1, 2, 4, 8), dtype=torch.float32)
    with pytest.raises((RuntimeError, ValueError)):
        gqa.prefill(q, k, k.clone())


def _native_check():
    import __graft_entry__ as entry
    if not os.path.exists(entry.NATIVE_BIN):
        entry.build_native_check()
    return entry.NATIVE_BIN


def test_native_program_refusals():
    """The C ABI from native code (tests/native/abi_check.cpp, no Python in
    the call path): refusals come back before any launch and the host helpers
    reproduce the pages' tables."""
    import subprocess
    res = subprocess.run([_native_check(), "refusals"], capture_output=True, text=True,
                         timeout=60)
    assert res.returncode == 0, res.stderr
    assert res.stdout.strip() == "refusals ok"
