"""The entry points under HIP graph capture.

With caller-provided output and workspace buffers and device-side lengths, a
decode or prefill call launches kernels only: no allocation, no copy, no
memset, no synchronisation.  It can then be captured in a graph and replayed.
The captured graph is replayed several times, with new inputs written into the
captured buffers and eager work and synchronisations between the replays; every
replay must equal the eager call on the same inputs bit for bit (same kernels,
no atomics), and one replay is also held to the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import gqa_kv_cache_02_amd as gqa
import oracle
from gqa_kv_cache_02_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gqa.lib()
    yield
    torch.cuda.synchronize()


def _np(t):
    return t.detach().float().cpu().numpy()


def test_decode_and_prefill_replay_in_a_graph():
    B, C, hq, hkv, d = 4, 1000, 16, 4, 128
    q, k, v = synth.decode_inputs(B, C, hq, hkv, d, torch.bfloat16, 5100, DEV)
    seqlens = torch.tensor([1000, 700, 33, 1], dtype=torch.int32, device=DEV)
    out = torch.empty((B, hq, d), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(max(1, gqa.decode_workspace_bytes(B, C, hq, hkv, d, window=300)),
                     dtype=torch.uint8, device=DEV)
    qp, kp, vp = synth.prefill_inputs(2, 300, 8, 2, 64, torch.bfloat16, 5101, DEV)
    plens = torch.tensor([300, 129], dtype=torch.int32, device=DEV)
    outp = torch.empty((2, 300, 8, 64), dtype=torch.bfloat16, device=DEV)

    def calls():
        gqa.decode(q, k, v, seqlens=seqlens, window=300, out=out, workspace=ws)
        gqa.prefill(qp, kp, vp, seqlens=plens, out=outp)

    # warm up on a side stream of default priority, as capture requires
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()

    for i in range(5):
        # new query rows in the captured buffers (eager work between replays)
        q.copy_(synth.randn((B, hq, d), 5200 + i, torch.bfloat16, DEV))
        qp.copy_(synth.randn((2, 8, 300, 64), 5300 + i, torch.bfloat16, DEV))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = gqa.decode(q, k, v, seqlens=seqlens, window=300)
        refp = gqa.prefill(qp, kp, vp, seqlens=plens)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"decode replay {i} differs from the eager call"
        assert torch.equal(outp, refp), f"prefill replay {i} differs from the eager call"
        if i == 2:
            od, _, _ = oracle.decode(_np(q), _np(k), _np(v), seqlens=[1000, 700, 33, 1],
                                     window=300)
            op, _, _ = oracle.prefill(_np(qp), _np(kp), _np(vp), seqlens=[300, 129])
            assert float(np.max(np.abs(_np(out) - od))) <= 2e-2
            assert float(np.max(np.abs(_np(outp) - op))) <= 2e-2


def test_prefix_and_rolling_decode_replay_in_a_graph():
    # queries against a long cache (key range split over workgroups, second
    # merge kernel) and a rolling-cache decode that commits a candidate; a
    # replay commits the same candidate into the same slot again
    Bq, Tq, C, hq, hkv, d = 1, 64, 2000, 8, 2, 128
    q, k, v = synth.prefill_inputs(Bq, Tq, hq, hkv, d, torch.bfloat16, 5400, DEV, C=C)
    s_lens = torch.tensor([1900], dtype=torch.int32, device=DEV)
    q_lens = torch.tensor([64], dtype=torch.int32, device=DEV)
    need = gqa.prefill_prefix_workspace_bytes(Bq, Tq, C, hq, hkv, d)
    assert need > 0  # the split path
    wsp = torch.empty(need, dtype=torch.uint8, device=DEV)
    outp = torch.empty((Bq, Tq, hq, d), dtype=torch.bfloat16, device=DEV)

    B, W = 3, 64
    qd, kc, vc = synth.decode_inputs(B, W, 8, 2, 64, torch.bfloat16, 5401, DEV)
    kn = synth.randn((B, 2, 64), 5402, torch.bfloat16, DEV)
    vn = synth.randn((B, 2, 64), 5403, torch.bfloat16, DEV)
    r_lens = torch.tensor([150, 40, 64], dtype=torch.int32, device=DEV)
    wsd = torch.empty(max(1, gqa.decode_workspace_bytes(B, W, 8, 2, 64, window=W)),
                      dtype=torch.uint8, device=DEV)
    outd = torch.empty((B, 8, 64), dtype=torch.bfloat16, device=DEV)

    def calls():
        gqa.prefill_prefix(q, k, v, seqlens=s_lens, qlens=q_lens, out=outp, workspace=wsp)
        gqa.decode_cache(qd, kc, vc, k_new=kn, v_new=vn, seqlens=r_lens, window=W, ring=True,
                         out=outd, workspace=wsd)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()

    for i in range(4):
        q.copy_(synth.randn((Bq, hq, Tq, d), 5500 + i, torch.bfloat16, DEV))
        qd.copy_(synth.randn((B, 8, 64), 5600 + i, torch.bfloat16, DEV))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = gqa.prefill_prefix(q, k, v, seqlens=s_lens, qlens=q_lens)
        refd = gqa.decode_cache(qd, kc, vc, k_new=kn, v_new=vn, seqlens=r_lens, window=W,
                                ring=True)
        torch.cuda.synchronize()
        assert torch.equal(outp, ref), f"prefix replay {i} differs from the eager call"
        assert torch.equal(outd, refd), f"rolling decode replay {i} differs from the eager call"
        if i == 1:
            o, _, _ = oracle.attend_prefix(_np(q), _np(k), _np(v), seqlens=[1900], qlens=[64])
            assert float(np.max(np.abs(_np(outp) - o))) <= 2e-2


def test_packed_segments_replay_in_a_graph():
    # packed segments run the 4-wavefront workgroups: once over a whole packed
    # row, once as new rows against a long cache (key range split, merge)
    B, T, hq, hkv, d = 2, 300, 8, 2, 128
    q, k, v = synth.prefill_inputs(B, T, hq, hkv, d, torch.bfloat16, 5700, DEV)
    segs_np = np.zeros((B, T), np.int32)
    for b, cuts in enumerate(([0, 37, 120, 121, 250], [0, 64, 65, 200])):
        for i, c in enumerate(cuts):
            end = cuts[i + 1] if i + 1 < len(cuts) else T
            segs_np[b, c:end] = c
    segs = torch.from_numpy(segs_np).to(DEV)
    out = torch.empty((B, T, hq, d), dtype=torch.bfloat16, device=DEV)

    Tq, C = 64, 2000
    qs, ks, vs = synth.prefill_inputs(1, Tq, hq, hkv, d, torch.bfloat16, 5701, DEV, C=C)
    s_lens = torch.tensor([1900], dtype=torch.int32, device=DEV)
    q_lens = torch.tensor([64], dtype=torch.int32, device=DEV)
    segs_s_np = np.full((1, Tq), 1850, np.int32)
    segs_s_np[0, 40:] = 1876
    segs_s = torch.from_numpy(segs_s_np).to(DEV)
    need = gqa.prefill_prefix_workspace_bytes(1, Tq, C, hq, hkv, d)
    assert need > 0  # the split path
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    outs = torch.empty((1, Tq, hq, d), dtype=torch.bfloat16, device=DEV)

    def calls():
        gqa.prefill_prefix(q, k, v, seg_starts=segs, out=out)
        gqa.prefill_prefix(qs, ks, vs, seqlens=s_lens, qlens=q_lens, seg_starts=segs_s, out=outs,
                           workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()

    for i in range(4):
        q.copy_(synth.randn((B, hq, T, d), 5800 + i, torch.bfloat16, DEV))
        qs.copy_(synth.randn((1, hq, Tq, d), 5900 + i, torch.bfloat16, DEV))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = gqa.prefill_prefix(q, k, v, seg_starts=segs)
        refs = gqa.prefill_prefix(qs, ks, vs, seqlens=s_lens, qlens=q_lens, seg_starts=segs_s)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"packed replay {i} differs from the eager call"
        assert torch.equal(outs, refs), f"split packed replay {i} differs from the eager call"
        if i == 2:
            o, _, _ = oracle.attend_prefix(_np(q), _np(k), _np(v), segs=segs_np)
            assert float(np.max(np.abs(_np(out) - o))) <= 2e-2
            o, _, _ = oracle.attend_prefix(_np(qs), _np(ks), _np(vs), seqlens=[1900], qlens=[64],
                                           segs=segs_s_np)
            assert float(np.max(np.abs(_np(outs) - o))) <= 2e-2
