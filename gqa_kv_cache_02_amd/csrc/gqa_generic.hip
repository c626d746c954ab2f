// gqa_generic.hip -- the general kernel: fp32 or bf16 storage, any head width
// d <= 256, decode or causal prefill, optional window.
//
// Prefill rows may be queries against a cached prefix (row i of the t_b new
// ones at cell s_b - t_b + i) with a per-row segment start; decode may read
// the new cell from a separate candidate buffer and commit it, and may
// address a rolling cache (cell j in slot j mod C).
//
// One 64-lane wavefront owns one output row t of one batch row b and up to
// kGroupHeads query heads of one KV group g.  Lane c holds features
// c, c+64, c+128, c+192.  Each permitted key cell is loaded from HBM once per
// wavefront and used by every query head the wavefront owns (the group's
// heads share the K/V lane; "Share key/value heads and make context
// explicit", "Give each query head an explicit shared KV head").  Softmax is
// the running (online) form: a running maximum m, running sum l and a running
// value mix rescaled by exp2(m_old - m_new), which gives the same result as
// normalising over the whole permitted set ("GQA, FlashAttention and the KV
// cache", section "FlashAttention").
#include "gqa_common.hpp"
#include "gqa_internal.hpp"

namespace gqa {

constexpr int kGroupHeads = 8;

struct GenericArgs {
    const void *q;
    const void *k;
    const void *v;
    void *out;
    const int32_t *seqlens;
    const int32_t *qlens;
    const int32_t *segs;
    int32_t *records;
    const void *knew;
    const void *vnew;
    void *kw;
    void *vw;
    int T, C, Hq, Hkv, d, window, r, nchunk;
    float scale_log2;
    int decode, prefix, ring;
};

template <typename T, int DPL, bool kRecord>
__global__ __launch_bounds__(64) void generic_kernel(GenericArgs a) {
    const int lane = threadIdx.x;
    const int b = blockIdx.z;
    const int g = blockIdx.y / a.nchunk;
    const int chunk = blockIdx.y % a.nchunk;
    const int h0 = g * a.r + chunk * kGroupHeads;
    int nh = a.r - chunk * kGroupHeads;
    nh = nh < kGroupHeads ? nh : kGroupHeads;

    const int tq = a.decode ? 1 : a.T;         // query rows per (b, h)
    const int trow = a.decode ? 0 : static_cast<int>(blockIdx.x); // row within q/out
    const int d = a.d;
    // t: the query's cell; lo: its first permitted key
    int t, lo;
    bool active;
    if (a.decode) {
        const int nb = a.seqlens ? a.seqlens[b] : a.C;
        t = nb - 1;
        active = nb >= 1;
        lo = window_lo(t, a.window);
    } else {
        int s_b, t_b;
        if (a.prefix) {
            s_b = a.seqlens ? a.seqlens[b] : a.C;
            t_b = a.qlens ? a.qlens[b] : a.T;
        } else {
            s_b = a.seqlens ? a.seqlens[b] : a.T;
            t_b = s_b;
        }
        t = s_b - t_b + trow;
        const int seg = a.segs ? a.segs[(int64_t)b * a.T + trow] : 0;
        lo = segment_lo(t, seg, a.window);
        active = trow < t_b && t >= 0 && lo >= 0;
    }

    const T *q = static_cast<const T *>(a.q);
    const T *kc = static_cast<const T *>(a.k) + ((int64_t)b * a.Hkv + g) * a.C * d;
    const T *vc = static_cast<const T *>(a.v) + ((int64_t)b * a.Hkv + g) * a.C * d;
    T *out = static_cast<T *>(a.out);
    // The candidate (decode): cell t is read from its own buffer and, by the
    // first head chunk of the group, committed to its cache slot.  Nothing
    // else in this launch reads that slot: the cell it held before (t - C in
    // a rolling cache) is outside the window.
    const T *kcand = a.knew ? static_cast<const T *>(a.knew) + ((int64_t)b * a.Hkv + g) * d : nullptr;
    const T *vcand = a.vnew ? static_cast<const T *>(a.vnew) + ((int64_t)b * a.Hkv + g) * d : nullptr;
    if (kcand && active && chunk == 0) {
        const int64_t slot = a.ring ? t % a.C : t;
        T *kd = static_cast<T *>(a.kw) + (((int64_t)b * a.Hkv + g) * a.C + slot) * d;
        T *vd = static_cast<T *>(a.vw) + (((int64_t)b * a.Hkv + g) * a.C + slot) * d;
        for (int c = lane; c < d; c += 64) {
            kd[c] = kcand[c];
            vd[c] = vcand[c];
        }
    }

    if (!active) {
        for (int hh = 0; hh < nh; ++hh) {
            T *o = out + (((int64_t)b * tq + trow) * a.Hq + h0 + hh) * d;
            for (int c = lane; c < d; c += 64)
                Elem<T>::store(o + c, 0.f);
            if (kRecord && lane == 0) {
                int32_t *rec = a.records + (((int64_t)b * tq + trow) * a.Hq + h0 + hh) * 5;
                rec[0] = g; rec[1] = -1; rec[2] = -1; rec[3] = 0; rec[4] = 0;
            }
        }
        return;
    }

    float qf[kGroupHeads][DPL];
    float acc[kGroupHeads][DPL];
    float m[kGroupHeads], l[kGroupHeads];
#pragma unroll
    for (int hh = 0; hh < kGroupHeads; ++hh) {
        const T *qrow = q + (((int64_t)b * a.Hq + h0 + hh) * tq + trow) * d;
#pragma unroll
        for (int i = 0; i < DPL; ++i) {
            const int c = lane + 64 * i;
            qf[hh][i] = (hh < nh && c < d) ? Elem<T>::load(qrow + c) : 0.f;
            acc[hh][i] = 0.f;
        }
        m[hh] = -INFINITY;
        l[hh] = 0.f;
    }

    int rcount = 0, rxor = 0;
    for (int j = lo; j <= t; ++j) {
        const T *kj = kc + (int64_t)(a.ring ? j % a.C : j) * d;
        const T *vj = vc + (int64_t)(a.ring ? j % a.C : j) * d;
        if (kcand && j == t) {
            kj = kcand;
            vj = vcand;
        }
        float kk[DPL], vv[DPL];
#pragma unroll
        for (int i = 0; i < DPL; ++i) {
            const int c = lane + 64 * i;
            kk[i] = c < d ? Elem<T>::load(kj + c) : 0.f;
            vv[i] = c < d ? Elem<T>::load(vj + c) : 0.f;
        }
#pragma unroll
        for (int hh = 0; hh < kGroupHeads; ++hh) {
            if (hh >= nh)
                break;
            float part = 0.f;
#pragma unroll
            for (int i = 0; i < DPL; ++i)
                part = fmaf(qf[hh][i], kk[i], part);
            const float s = wave_sum(part) * a.scale_log2;
            const float mn = fmaxf(m[hh], s);
            const float alpha = fast_exp2(m[hh] - mn);
            const float p = fast_exp2(s - mn);
            l[hh] = fmaf(l[hh], alpha, p);
#pragma unroll
            for (int i = 0; i < DPL; ++i)
                acc[hh][i] = fmaf(acc[hh][i], alpha, p * vv[i]);
            m[hh] = mn;
        }
        if (kRecord) {
            rcount += 1;
            rxor ^= j;
        }
    }

#pragma unroll
    for (int hh = 0; hh < kGroupHeads; ++hh) {
        if (hh >= nh)
            break;
        const float inv = 1.f / l[hh];
        T *o = out + (((int64_t)b * tq + trow) * a.Hq + h0 + hh) * d;
#pragma unroll
        for (int i = 0; i < DPL; ++i) {
            const int c = lane + 64 * i;
            if (c < d)
                Elem<T>::store(o + c, acc[hh][i] * inv);
        }
        if (kRecord && lane == 0) {
            int32_t *rec = a.records + (((int64_t)b * tq + trow) * a.Hq + h0 + hh) * 5;
            rec[0] = g; rec[1] = lo; rec[2] = t; rec[3] = rcount; rec[4] = rxor;
        }
    }
}

template <typename T, bool kRecord>
static hipError_t launch_typed(const GenericArgs &a, dim3 grid, int dpl, hipStream_t s) {
    switch (dpl) {
    case 1: generic_kernel<T, 1, kRecord><<<grid, 64, 0, s>>>(a); break;
    case 2: generic_kernel<T, 2, kRecord><<<grid, 64, 0, s>>>(a); break;
    case 3: generic_kernel<T, 3, kRecord><<<grid, 64, 0, s>>>(a); break;
    default: generic_kernel<T, 4, kRecord><<<grid, 64, 0, s>>>(a); break;
    }
    return hipGetLastError();
}

hipError_t launch_generic(const Problem &p, hipStream_t stream) {
    GenericArgs a;
    a.q = p.q; a.k = p.k; a.v = p.v; a.out = p.out;
    a.seqlens = p.seqlens; a.records = p.records;
    a.qlens = p.qlens; a.segs = p.segs; a.prefix = p.prefix ? 1 : 0;
    a.knew = p.knew; a.vnew = p.vnew; a.kw = p.kw; a.vw = p.vw; a.ring = p.ring ? 1 : 0;
    a.T = p.T; a.C = p.C; a.Hq = p.Hq; a.Hkv = p.Hkv; a.d = p.d; a.window = p.window;
    a.r = p.Hq / p.Hkv;
    a.nchunk = (a.r + kGroupHeads - 1) / kGroupHeads;
    a.scale_log2 = p.scale * kLog2e;
    a.decode = p.decode ? 1 : 0;
    const int dpl = (p.d + 63) / 64;
    dim3 grid(p.decode ? 1 : p.T, p.Hkv * a.nchunk, p.B);
    const bool rec = p.records != nullptr;
    if (p.dtype == 0)
        return rec ? launch_typed<float, true>(a, grid, dpl, stream)
                   : launch_typed<float, false>(a, grid, dpl, stream);
    return rec ? launch_typed<uint16_t, true>(a, grid, dpl, stream)
               : launch_typed<uint16_t, false>(a, grid, dpl, stream);
}

} // namespace gqa
