// gqa_decode.hip -- bf16 single-token decode over a KV cache, split along the
// cache length, with matrix-core (MFMA) dot products and a log-sum-exp merge.
//
// Work decomposition.  A row (b, query head h) reads the key cells
// lo..n_b-1 of KV head g = floor(h / r) (lo = max(0, n_b - w) with a window;
// "Share key/value heads and make context explicit", "Intersect the window
// with the context already permitted", and "Extend the existing full and
// cached attention paths" for the query's position).  That range is cut into
// chunks of `chunk` keys counted from lo; workgroup (split, g, b) takes chunk
// `split` for ALL query heads of group g at once (up to 16 per workgroup), so
// every K/V cell is fetched from HBM once per group and feeds the r heads that
// share it -- the saving GQA exists for ("How do you implement grouped query
// attention (GQA)?", Step 4: the cache stores G heads and is repeated on
// read; here the repeat never materialises).
//
// Inside a workgroup, 4 wavefronts take interleaved 32-key tiles.  Per tile:
//   S^T[32 keys x 16 heads] = K_tile[32 x d] . Q^T[d x 16]   (MFMA 16x16x32 bf16)
//   online softmax per head in base 2 (running max m, running sum l)
//   O^T[d x 16] += V_tile^T[d x 32] . P^T[32 x 16]            (MFMA 16x16x32 bf16)
// The transposed products keep every per-head quantity in the lanes that own
// that head (lane & 15), so the softmax rescale never crosses lanes.  K is
// read straight from HBM into the MFMA operand layout; V is staged through a
// wavefront-private LDS tile to be read back transposed.  The 4 wavefronts'
// states are merged through LDS and one (normalised partial, log2-sum-exp)
// pair per (row, split) goes to the workspace.  A second kernel merges the
// splits of each row with weights 2^(lse_s - max lse) ("GQA, FlashAttention
// and the KV cache", section "FlashAttention": blockwise softmax with a
// numerically stable running normalisation gives the dense result).
#include <limits.h>

#include "gqa_common.hpp"
#include "gqa_internal.hpp"

namespace gqa {

struct DecodeArgs {
    const uint16_t *q;
    const uint16_t *k;
    const uint16_t *v;
    const int32_t *seqlens;
    float *o_part;     // [B, Hq, nsplit, D]
    float *lse_part;   // [B, Hq, nsplit]
    int32_t *rec_part; // [B, Hq, nsplit, 4]  (record instantiation only)
    int C, Hq, Hkv, window, r, nhc, nsplit, chunk;
    float scale_log2;
};

struct CombineArgs {
    const float *o_part;
    const float *lse_part;
    const int32_t *rec_part;
    const int32_t *seqlens;
    uint16_t *out;     // [B, Hq, D]
    int32_t *records;  // [B, Hq, 5]
    int B, C, Hq, r, window, nsplit, chunk;
};

template <int D> struct DecodeSmem {
    static constexpr int LDV = D + 8; // padded LDS row (u16) of a V tile
    static constexpr int kVBytes = kDecodeWaves * kDecodeTile * LDV * 2;
    static constexpr int kOBytes = kDecodeWaves * kDecodeHeads * D * 4;
    static constexpr int kBytes = (kVBytes > kOBytes ? kVBytes : kOBytes);
};

template <int D, bool kRecord>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
    constexpr int KS = D / 32;               // 32-feature k-steps of Q.K
    constexpr int DB = D / 16;               // 16-column blocks of P.V
    constexpr int LDV = DecodeSmem<D>::LDV;
    constexpr int VPI = 1024 / (2 * D);      // keys per 1 KiB wavefront load
    constexpr int LPK = 64 / VPI;            // lanes per key row
    constexpr int VIT = kDecodeTile / VPI;   // V loads per tile

    __shared__ __attribute__((aligned(16))) unsigned char smem[DecodeSmem<D>::kBytes];
    __shared__ float sm_m[kDecodeWaves][kDecodeHeads];
    __shared__ float sm_l[kDecodeWaves][kDecodeHeads];
    __shared__ int sm_rec[kDecodeWaves][4];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int hl = lane & 15; // head within the 16-head chunk (MFMA column)
    const int qg = lane >> 4; // lane group (MFMA k/row group)

    const int b = blockIdx.z;
    const int g = blockIdx.y / a.nhc;
    const int hc = blockIdx.y % a.nhc;
    const int split = blockIdx.x;
    const int h0 = g * a.r + hc * kDecodeHeads;
    const int nh = min(kDecodeHeads, a.r - hc * kDecodeHeads);

    const int nb = a.seqlens ? a.seqlens[b] : a.C;
    if (nb <= 0)
        return;
    const int hi = nb - 1;
    const int lo = window_lo(hi, a.window);
    const int c_lo = lo + split * a.chunk;
    if (c_lo > hi)
        return; // this row has fewer chunks; the combine step knows
    const int c_hi = min(hi, c_lo + a.chunk - 1);

    // Q^T operand: lane (hl, qg) holds features s*32 + qg*8 .. +8 of head hl.
    bf16x8 qb[KS];
    {
        const uint16_t *qrow = a.q + ((int64_t)b * a.Hq + h0 + hl) * D;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if (hl < nh)
                qb[s] = *reinterpret_cast<const bf16x8 *>(qrow + s * 32 + qg * 8);
            else
                qb[s] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
    }

    const int64_t lane_off = ((int64_t)b * a.Hkv + g) * (int64_t)a.C * D;
    const uint16_t *kbase = a.k + lane_off;
    const uint16_t *vbase = a.v + lane_off;
    uint16_t *vs = reinterpret_cast<uint16_t *>(smem) + wave * kDecodeTile * LDV;

    float m = -INFINITY;
    float lsum = 0.f;
    f32x4 oacc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i)
        oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    int r_cnt = 0, r_xor = 0, r_lo = INT_MAX, r_hi = -1;

    for (int tile = wave;; tile += kDecodeWaves) {
        const int j0 = c_lo + tile * kDecodeTile;
        if (j0 > c_hi)
            break;

        // K operand straight from HBM: lane (hl, qg) of key block kb holds
        // key j0 + kb*16 + hl, features s*32 + qg*8 .. +8.
        bf16x8 ka[2][KS];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int key = j0 + kb * 16 + hl;
            const uint16_t *krow = kbase + (int64_t)key * D + qg * 8;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                if (key <= c_hi)
                    ka[kb][s] = *reinterpret_cast<const bf16x8 *>(krow + s * 32);
                else
                    ka[kb][s] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
            }
        }
        // V tile in its natural layout, 16 B per lane, 1 KiB per load.
        uint4 vr[VIT];
#pragma unroll
        for (int it = 0; it < VIT; ++it) {
            const int key = j0 + it * VPI + lane / LPK;
            const int col = (lane % LPK) * 8;
            if (key <= c_hi)
                vr[it] = *reinterpret_cast<const uint4 *>(vbase + (int64_t)key * D + col);
            else
                vr[it] = uint4{0u, 0u, 0u, 0u};
        }

        // S^T = K . Q^T ; lane (hl, qg) gets keys kb*16 + qg*4 + i of head hl.
        f32x4 sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s)
                sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kb][s], qb[s], sacc[kb], 0, 0, 0);
        }

        // Stage V (wavefront-private tile).  The fences keep the compiler
        // from moving LDS accesses across tiles; LDS operations of one
        // wavefront complete in order.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int it = 0; it < VIT; ++it) {
            const int row = it * VPI + lane / LPK;
            const int col = (lane % LPK) * 8;
            *reinterpret_cast<uint4 *>(vs + row * LDV + col) = vr[it];
        }

        // Scale, mask cells past the chunk end, online softmax update.
        float x[2][4];
        float tmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = j0 + kb * 16 + qg * 4 + i;
                x[kb][i] = (key <= c_hi) ? sacc[kb][i] * a.scale_log2 : -INFINITY;
                tmax = fmaxf(tmax, x[kb][i]);
            }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float mn = fmaxf(m, tmax); // finite: key j0 is always permitted
        const float alpha = fast_exp2(m - mn);
        m = mn;
        float psum = 0.f;
        uint32_t pw[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
                const float p0 = fast_exp2(x[kb][i] - mn);
                const float p1 = fast_exp2(x[kb][i + 1] - mn);
                psum += p0 + p1;
                pw[kb * 2 + i / 2] = pack_bf16x2(p0, p1);
            }
        const bf16x8 pb = __builtin_bit_cast(bf16x8, (uint4){pw[0], pw[1], pw[2], pw[3]});
        lsum = fmaf(lsum, alpha, psum);
#pragma unroll
        for (int i = 0; i < DB; ++i)
            oacc[i] *= alpha;

        if (kRecord) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = j0 + kb * 16 + qg * 4 + i;
                    if (key <= c_hi) {
                        r_cnt += 1;
                        r_xor ^= key;
                        r_lo = min(r_lo, key);
                        r_hi = max(r_hi, key);
                    }
                }
        }

        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // O^T += V^T . P^T.  P^T k-slot qg*8 + e is key qg*4 + e (e < 4) or
        // 16 + qg*4 + (e - 4): exactly the keys this lane already holds, so
        // V^T is gathered from LDS in the same key order.
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            bf16x8 va;
            const uint16_t *vcol = vs + db * 16 + hl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int key = (e < 4) ? (qg * 4 + e) : (16 + qg * 4 + (e - 4));
                va[e] = static_cast<short>(vcol[key * LDV]);
            }
            oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, oacc[db], 0, 0, 0);
        }
    }

    // Per-head running sum: add the 4 lane groups that share head hl.
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);

    if (kRecord) {
        // every head folds the same keys; gather the 4 lane groups
#pragma unroll
        for (int msk = 16; msk <= 32; msk <<= 1) {
            r_cnt += __shfl_xor(r_cnt, msk, 64);
            r_xor ^= __shfl_xor(r_xor, msk, 64);
            r_lo = min(r_lo, __shfl_xor(r_lo, msk, 64));
            r_hi = max(r_hi, __shfl_xor(r_hi, msk, 64));
        }
        if (lane == 0) {
            sm_rec[wave][0] = r_cnt;
            sm_rec[wave][1] = r_lo;
            sm_rec[wave][2] = r_hi;
            sm_rec[wave][3] = r_xor;
        }
    }

    // Merge the 4 wavefronts of the workgroup.
    if (qg == 0) {
        sm_m[wave][hl] = m;
        sm_l[wave][hl] = lsum;
    }
    __syncthreads(); // also ends every wavefront's use of the V tiles
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w)
        mx = fmaxf(mx, sm_m[w][hl]);
    const float my_scale = fast_exp2(m - mx);
    float *os = reinterpret_cast<float *>(smem);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            os[(wave * kDecodeHeads + hl) * D + db * 16 + qg * 4 + i] = oacc[db][i] * my_scale;
    __syncthreads();

    const int64_t row0 = (int64_t)b * a.Hq + h0;
    for (int idx = tid; idx < kDecodeHeads * D; idx += 256) {
        const int h = idx / D;
        const int c = idx % D;
        if (h >= nh)
            break;
        float hm = -INFINITY;
#pragma unroll
        for (int w = 0; w < kDecodeWaves; ++w)
            hm = fmaxf(hm, sm_m[w][h]);
        float hl_sum = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < kDecodeWaves; ++w) {
            hl_sum += fast_exp2(sm_m[w][h] - hm) * sm_l[w][h];
            o += os[(w * kDecodeHeads + h) * D + c];
        }
        a.o_part[((row0 + h) * a.nsplit + split) * D + c] = o / hl_sum;
        if (c == 0)
            a.lse_part[(row0 + h) * a.nsplit + split] = hm + log2f(hl_sum);
    }
    if (kRecord && tid < nh) {
        int cnt = 0, x = 0, rl = INT_MAX, rh = -1;
#pragma unroll
        for (int w = 0; w < kDecodeWaves; ++w) {
            cnt += sm_rec[w][0];
            rl = min(rl, sm_rec[w][1]);
            rh = max(rh, sm_rec[w][2]);
            x ^= sm_rec[w][3];
        }
        int32_t *rp = a.rec_part + ((row0 + tid) * a.nsplit + split) * 4;
        rp[0] = cnt; rp[1] = rl; rp[2] = rh; rp[3] = x;
    }
}

// One wavefront per (b, h): weights 2^(lse_s - max_s lse_s) over the row's
// splits, output = sum_s w_s o_s / sum_s w_s, rounded to bf16.
template <int D, bool kRecord>
__global__ __launch_bounds__(256) void decode_combine_kernel(CombineArgs a) {
    constexpr int CPL = D / 64; // output features per lane
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + wave;
    if (row >= (int64_t)a.B * a.Hq)
        return;
    const int b = static_cast<int>(row / a.Hq);
    const int h = static_cast<int>(row % a.Hq);
    const int nb = a.seqlens ? a.seqlens[b] : a.C;
    uint16_t *orow = a.out + row * D;
    if (nb <= 0) {
#pragma unroll
        for (int i = 0; i < CPL; ++i)
            orow[lane + 64 * i] = 0;
        if (kRecord && lane == 0) {
            int32_t *rec = a.records + row * 5;
            rec[0] = h / a.r; rec[1] = -1; rec[2] = -1; rec[3] = 0; rec[4] = 0;
        }
        return;
    }
    const int hi = nb - 1;
    const int lo = window_lo(hi, a.window);
    const int ns = (hi - lo) / a.chunk + 1;
    const float *lse = a.lse_part + row * a.nsplit;
    const float *op = a.o_part + row * a.nsplit * D;

    float mx = -INFINITY;
    for (int s = lane; s < ns; s += 64)
        mx = fmaxf(mx, lse[s]);
    mx = wave_max(mx);

    float den = 0.f;
    float acc[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i)
        acc[i] = 0.f;
    for (int s = 0; s < ns; ++s) {
        const float w = fast_exp2(lse[s] - mx);
        den += w;
#pragma unroll
        for (int i = 0; i < CPL; ++i)
            acc[i] = fmaf(w, op[(int64_t)s * D + lane + 64 * i], acc[i]);
    }
    const float inv = 1.f / den;
#pragma unroll
    for (int i = 0; i < CPL; ++i)
        orow[lane + 64 * i] = f32_to_bf16(acc[i] * inv);

    if (kRecord && lane == 0) {
        int cnt = 0, x = 0, rl = INT_MAX, rh = -1;
        for (int s = 0; s < ns; ++s) {
            const int32_t *rp = a.rec_part + (row * a.nsplit + s) * 4;
            cnt += rp[0];
            rl = min(rl, rp[1]);
            rh = max(rh, rp[2]);
            x ^= rp[3];
        }
        int32_t *rec = a.records + row * 5;
        rec[0] = h / a.r; rec[1] = rl; rec[2] = rh; rec[3] = cnt; rec[4] = x;
    }
}

static size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

DecodePlan plan_decode(int B, int C, int Hq, int Hkv, int d, int window) {
    DecodePlan p{};
    const int elig = (window > 0 && window < C) ? window : C;
    const int r = Hq / Hkv;
    p.nhc = (r + kDecodeHeads - 1) / kDecodeHeads;
    // Aim for at least two 4-wavefront workgroups per compute unit on a
    // 256-CU part, with as long a chunk as that allows (fewer partials).
    const int64_t units = (int64_t)B * Hkv * p.nhc;
    const int64_t target = 512;
    int tpw = 1;
    for (int t = 16; t >= 1; t >>= 1) {
        const int64_t chunk = (int64_t)kDecodeWaves * kDecodeTile * t;
        const int64_t ns = (elig + chunk - 1) / chunk;
        if (units * ns >= target) {
            tpw = t;
            break;
        }
    }
    p.tiles_per_wave = tpw;
    p.chunk = kDecodeWaves * kDecodeTile * tpw;
    p.nsplit = elig > 0 ? (elig + p.chunk - 1) / p.chunk : 0;
    const size_t rows = (size_t)B * Hq * (size_t)p.nsplit;
    p.o_off = 0;
    p.lse_off = align256(rows * d * sizeof(float));
    p.rec_off = p.lse_off + align256(rows * sizeof(float));
    p.bytes = p.rec_off + align256(rows * 4 * sizeof(int32_t));
    if (p.nsplit == 0)
        p.bytes = 256; // the combine step still runs (it writes zero rows)
    return p;
}

template <int D, bool kRecord>
static hipError_t launch_d(const Problem &p, const DecodePlan &plan, void *ws, hipStream_t s) {
    unsigned char *w = static_cast<unsigned char *>(ws);
    DecodeArgs a;
    a.q = static_cast<const uint16_t *>(p.q);
    a.k = static_cast<const uint16_t *>(p.k);
    a.v = static_cast<const uint16_t *>(p.v);
    a.seqlens = p.seqlens;
    a.o_part = reinterpret_cast<float *>(w + plan.o_off);
    a.lse_part = reinterpret_cast<float *>(w + plan.lse_off);
    a.rec_part = reinterpret_cast<int32_t *>(w + plan.rec_off);
    a.C = p.C; a.Hq = p.Hq; a.Hkv = p.Hkv; a.window = p.window;
    a.r = p.Hq / p.Hkv; a.nhc = plan.nhc; a.nsplit = plan.nsplit; a.chunk = plan.chunk;
    a.scale_log2 = p.scale * kLog2e;
    if (plan.nsplit > 0) {
        dim3 grid(plan.nsplit, p.Hkv * plan.nhc, p.B);
        decode_split_kernel<D, kRecord><<<grid, 256, 0, s>>>(a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    CombineArgs c;
    c.o_part = a.o_part; c.lse_part = a.lse_part; c.rec_part = a.rec_part;
    c.seqlens = p.seqlens;
    c.out = static_cast<uint16_t *>(p.out);
    c.records = p.records;
    c.B = p.B; c.C = p.C; c.Hq = p.Hq; c.r = a.r; c.window = p.window;
    c.nsplit = plan.nsplit; c.chunk = plan.chunk;
    const int64_t rows = (int64_t)p.B * p.Hq;
    decode_combine_kernel<D, kRecord><<<dim3((unsigned)((rows + 3) / 4)), 256, 0, s>>>(c);
    return hipGetLastError();
}

hipError_t launch_decode_split(const Problem &p, const DecodePlan &plan, void *workspace,
                               hipStream_t stream) {
    const bool rec = p.records != nullptr;
    if (p.d == 128)
        return rec ? launch_d<128, true>(p, plan, workspace, stream)
                   : launch_d<128, false>(p, plan, workspace, stream);
    return rec ? launch_d<64, true>(p, plan, workspace, stream)
               : launch_d<64, false>(p, plan, workspace, stream);
}

} // namespace gqa
