"""Pure-Python brute force for tiny grouped-query attention cases.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

This is a deliberately different way of writing the same definition as
``gqa_oracle.c`` so that each can catch the other's slips:

* the KV head of query head h is found by searching for the group whose
  adjacent block of r = Hq/Hkv query heads contains h ("Share key/value heads
  and make context explicit", section "Give each query head an explicit shared
  KV head"), not by integer division;
* the permitted set is found by testing every key cell against the membership
  rules (causal j <= t, window t - j < w, active t < n_b; section "Intersect
  the window with the context already permitted"), not by a range;
* softmax is exp(s_j) / sum_u exp(s_u) without subtracting the maximum, summed
  with math.fsum (correctly rounded sums), which is fine for the small scores
  of tiny inputs.
"""
from __future__ import annotations

import math


def group_of(h: int, hq: int, hkv: int) -> int:
    r = hq // hkv
    for g in range(hkv):
        if g * r <= h < (g + 1) * r:
            return g
    raise ValueError("query head out of range")


def permitted(t: int, n: int, window, ncells: int):
    if t >= n:
        return []
    keys = []
    for j in range(ncells):
        if j > t:
            continue
        if window is not None and t - j >= window:
            continue
        keys.append(j)
    return keys


def attend(qv, kcells, vcells, keys, scale):
    d = len(qv)
    if not keys:
        return [0.0] * d, {}
    s = {j: scale * math.fsum(qv[c] * kcells[j][c] for c in range(d)) for j in keys}
    ex = {j: math.exp(s[j]) for j in keys}
    z = math.fsum(ex.values())
    p = {j: ex[j] / z for j in keys}
    out = [math.fsum(p[j] * vcells[j][c] for j in keys) for c in range(d)]
    return out, p


def prefill(q, k, v, seqlens=None, window=None, scale=None):
    """q nested [B][Hq][T][d], k/v [B][Hkv][C][d] -> out [B][T][Hq][d]."""
    B, hq, T, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    hkv, C = len(k[0]), len(k[0][0])
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    out = [[[None] * hq for _ in range(T)] for _ in range(B)]
    for b in range(B):
        n = T if seqlens is None else seqlens[b]
        for h in range(hq):
            g = group_of(h, hq, hkv)
            for t in range(T):
                keys = permitted(t, n, window, C)
                out[b][t][h], _ = attend(q[b][h][t], k[b][g], v[b][g], keys, sc)
    return out


def decode(q, k, v, seqlens=None, window=None, scale=None):
    """q nested [B][Hq][d], k/v [B][Hkv][C][d] -> out [B][Hq][d]."""
    B, hq, d = len(q), len(q[0]), len(q[0][0])
    hkv, C = len(k[0]), len(k[0][0])
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    out = [[None] * hq for _ in range(B)]
    for b in range(B):
        n = C if seqlens is None else seqlens[b]
        for h in range(hq):
            g = group_of(h, hq, hkv)
            keys = permitted(n - 1, n, window, C) if n > 0 else []
            out[b][h], _ = attend(q[b][h], k[b][g], v[b][g], keys, sc)
    return out


def prefix(q, k, v, seqlens=None, qlens=None, segs=None, window=None, scale=None):
    """Queries against a cached prefix, by membership tests.

    q nested [B][Hq][Tq][d], k/v [B][Hkv][C][d] -> out [B][Tq][Hq][d].  Query
    row i of t_b new ones sits at position p = s_b - t_b + i ("How do you
    implement grouped query attention (GQA)?", section "Worked example": the
    tril(s - t) mask); key j is permitted when j <= p, j is not before the
    row's segment start and p - j < w (section "Intersect the window with the
    context already permitted")."""
    B, hq, T, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    hkv, C = len(k[0]), len(k[0][0])
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    out = [[[None] * hq for _ in range(T)] for _ in range(B)]
    for b in range(B):
        s = C if seqlens is None else seqlens[b]
        t = T if qlens is None else qlens[b]
        for h in range(hq):
            g = group_of(h, hq, hkv)
            for i in range(T):
                p = s - t + i
                seg = 0 if segs is None else segs[b][i]
                keys = []
                if i < t:
                    for j in range(C):
                        if j > p or j < seg:
                            continue
                        if window is not None and p - j >= window:
                            continue
                        keys.append(j)
                out[b][i][h], _ = attend(q[b][h][i], k[b][g], v[b][g], keys, sc)
    return out


def decode_ring(q, k, v, seqlens, window, scale=None):
    """Decode over a rolling cache: the cell with index j lives in slot j mod C
    (the rolling buffer of the Mistral 7B paragraph in "Share key/value heads
    and make context explicit").  The logical cells are looked up one by one
    from their slots; the permitted ones are those within the window."""
    B, hq, d = len(q), len(q[0]), len(q[0][0])
    hkv, C = len(k[0]), len(k[0][0])
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    out = [[None] * hq for _ in range(B)]
    for b in range(B):
        n = seqlens[b]
        for h in range(hq):
            g = group_of(h, hq, hkv)
            cells_k, cells_v, keys = {}, {}, []
            for j in range(n):
                if n - 1 - j < window:
                    keys.append(j)
                    cells_k[j] = k[b][g][j % C]
                    cells_v[j] = v[b][g][j % C]
            out[b][h], _ = attend(q[b][h], cells_k, cells_v, keys, sc)
    return out
