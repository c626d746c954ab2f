"""Seeded synthetic inputs for grouped-query attention over a KV cache.

This module only draws numbers and lays them out; it holds none of the
attention arithmetic.  The same bits are handed to the HIP path and to the
fp64 oracle.

Workloads (no public dataset is involved; shapes follow the pages' examples):

* ``fixture_4token`` -- the zero-Q/K example of "Share key/value heads and make
  context explicit", section "Follow four query heads into two shared groups":
  four cells, Hq = 4, Hkv = 2, d = 2, Q = K = 0.  The value of cell j is
  (j+1, 0) on KV head 0 and (0, 10(j+1)) on KV head 1 (embedding feature 0 of
  cell j is j+1 and the value projection maps it to features 0 and 3, as the
  worked_example code in that section builds them).
* ``CONFIGS`` -- the measured or checked workloads, Q/K/V iid N(0,1)
  drawn in float32 from a seeded generator and rounded to bf16 (round to
  nearest even) where the dtype is bf16.
"""
from __future__ import annotations

import torch

CONFIGS = {
    # fp32 causal prefill, small enough for every check to run in the oracle.
    "prefill_f32_small": dict(kind="prefill", dtype="f32", B=1, T=16, Hq=4, Hkv=2,
                              d=8, windows=(None, 2), seed=1001),
    # bf16 single-token decode, Llama-3-8B-like head shape, 8000 cached cells.
    "decode_b8_hq32_hkv8_d128_n8000": dict(kind="decode", dtype="bf16", B=8, Hq=32,
                                           Hkv=8, d=128, n=8000, C=8000, window=None,
                                           seed=1002),
    # bf16 causal prefill over 4096 cells.
    "prefill_b1_t4096_hq32_hkv8_d128": dict(kind="prefill", dtype="bf16", B=1, T=4096,
                                            Hq=32, Hkv=8, d=128, window=None, seed=1003),
    # endpoint sweep: MHA, GQA group 4, MQA at the same query side.
    "decode_sweep_b16_hq8_d128_n8000": dict(kind="decode", dtype="bf16", B=16, Hq=8,
                                            Hkv=(8, 2, 1), d=128, n=8000, C=8000,
                                            window=None, seed=1004),
    # ragged lengths in [1, 32768] with an inclusive-self window of 4096.
    "decode_ragged_b32_hq8_hkv2_d64_w4096": dict(kind="decode", dtype="bf16", B=32, Hq=8,
                                                 Hkv=2, d=64, n=(1, 32768), C=32768,
                                                 window=4096, seed=1005),
    # Queries against a cached prefix: the last 512 cells of a 4096-cell
    # sequence as new rows (a chunk of a chunked prefill), the prefill shape
    # above otherwise.
    "chunk_b1_tq512_c4096_hq32_hkv8_d128": dict(kind="prefix", dtype="bf16", B=1, Tq=512,
                                                C=4096, Hq=32, Hkv=8, d=128, window=None,
                                                seed=1006),
    # The ragged sliding-window decode above over a rolling cache of capacity
    # w = 4096 (cell j in slot j mod w), with the new cell's key/value
    # committed in the same call.
    "ring_b32_hq8_hkv2_d64_w4096": dict(kind="ring", dtype="bf16", B=32, Hq=8, Hkv=2, d=64,
                                        n=(1, 32768), window=4096, seed=1007),
    # Packed segments: independent sequences of 64..1024 cells (uniform,
    # seeded; the last one cut to fill the row) back to back in one causal
    # prefill row of 4096 cells, each attending only within itself.
    "packed_b1_t4096_hq32_hkv8_d128": dict(kind="packed", dtype="bf16", B=1, T=4096, Hq=32,
                                           Hkv=8, d=128, seg_len=(64, 1024), window=None,
                                           seed=1008),
}

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(name: str) -> torch.dtype:
    return _DT[name]


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def randn(shape, seed: int, dtype=torch.float32, device="cpu") -> torch.Tensor:
    """iid N(0,1) in float32 from a seeded generator, then cast (RNE for bf16)."""
    g = _gen(seed, device)
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32, device=device)
    return x.to(dtype)


def prefill_inputs(B, T, Hq, Hkv, d, dtype=torch.float32, seed=0, device="cpu", C=None):
    """Q [B,Hq,T,d], K and V [B,Hkv,C,d] (C defaults to T)."""
    C = T if C is None else C
    q = randn((B, Hq, T, d), seed, dtype, device)
    k = randn((B, Hkv, C, d), seed + 7919, dtype, device)
    v = randn((B, Hkv, C, d), seed + 15838, dtype, device)
    return q, k, v


def decode_inputs(B, C, Hq, Hkv, d, dtype=torch.float32, seed=0, device="cpu"):
    """Q [B,Hq,d], K and V [B,Hkv,C,d]."""
    q = randn((B, Hq, d), seed, dtype, device)
    k = randn((B, Hkv, C, d), seed + 7919, dtype, device)
    v = randn((B, Hkv, C, d), seed + 15838, dtype, device)
    return q, k, v


def ragged_lengths(B: int, lo: int, hi: int, seed: int) -> torch.Tensor:
    """Per-sequence lengths uniform in [lo, hi] (inclusive), int32, on the CPU."""
    g = _gen(seed, "cpu")
    return torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)


def packed_segment_starts(B: int, T: int, lo: int, hi: int, seed: int) -> torch.Tensor:
    """Segment starts [B, T] int32 (CPU) of sequences packed back to back:
    lengths uniform in [lo, hi], the last one of each row cut at T."""
    g = _gen(seed, "cpu")
    starts = torch.empty((B, T), dtype=torch.int32)
    for b in range(B):
        t = 0
        while t < T:
            n = int(torch.randint(lo, hi + 1, (1,), generator=g))
            starts[b, t:t + n] = t
            t += n
    return starts


def fixture_4token(dtype=torch.float32, device="cpu"):
    """The four-cell zero-Q/K example; returns (q, k, v) with C = T = 4."""
    B, Hq, Hkv, T, d = 1, 4, 2, 4, 2
    q = torch.zeros((B, Hq, T, d), dtype=torch.float32)
    k = torch.zeros((B, Hkv, T, d), dtype=torch.float32)
    v = torch.zeros((B, Hkv, T, d), dtype=torch.float32)
    for j in range(T):
        v[0, 0, j, 0] = float(j + 1)
        v[0, 1, j, 1] = float(10 * (j + 1))
    return q.to(dtype).to(device), k.to(dtype).to(device), v.to(dtype).to(device)
