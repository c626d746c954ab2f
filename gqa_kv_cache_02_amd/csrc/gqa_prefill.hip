// gqa_prefill.hip -- bf16 causal prefill with matrix cores (MFMA), in the
// blockwise online-softmax form ("GQA, FlashAttention and the KV cache",
// section "FlashAttention": blocks and a numerically stable running
// normalisation give the dense result without materialising the score
// matrix; the dense pairwise work remains).
//
// Work decomposition.  A workgroup owns one batch row b, one KV group g and
// one block of query rows, and runs NW wavefronts: 8 (one workgroup per CU,
// two wavefronts per SIMD), or 4 for packed segments (two workgroups per CU).
// They are `hpw` query heads of group g times `rb` blocks of 32 rows
// (hpw * rb = NW).  All its wavefronts read the same K/V tiles, which are
// staged once in LDS per workgroup -- the r query heads that share a KV head
// ("Share key/value heads and make context explicit", "Give each query head
// an explicit shared KV head") never cause a second read or a repeated copy,
// and one staged tile feeds every wavefront of the workgroup.
//
// Per 64-key tile and wavefront (32 query rows):
//   S^T[64 keys x 32 rows] = K[64 x d] . Q^T[d x 32]     (MFMA 32x32x16 bf16)
//   mask (diagonal, window edge and padded rows only), base-2 online softmax
//   O^T[d x 32] += V^T[d x 64] . P^T[64 x 32]            (MFMA 32x32x16 bf16)
// The transposed products keep every row's running max and sum in the two
// lanes that own the row (l and l ^ 32).  K/V tiles are double-buffered in
// LDS and filled by direct global-to-LDS loads one tile ahead; V^T comes
// straight out of the natural-layout LDS tile with ds_read_b64_tr_b16.  Tiles entirely above the
// causal diagonal or entirely before every row's window start are never
// visited; only diagonal and window-edge tiles are masked ("Intersect the
// window with the context already permitted").
#include <limits.h>

#include <algorithm>
#include <type_traits>

#include "gqa_common.hpp"
#include "gqa_internal.hpp"

namespace gqa {

constexpr int kPBN = 64;   // keys per K/V tile
constexpr int kPRows = 32; // query rows per wavefront
constexpr int kPWaves = 8; // wavefronts per workgroup (4 for packed segments, see
                           // prefill_waves)

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;

struct PrefillArgs {
    const uint16_t *q;
    const uint16_t *k;
    const uint16_t *v;
    uint16_t *out;
    const int32_t *seqlens;
    const int32_t *qlens;   // prefix queries only (nullable)
    const int32_t *segs;    // nullable: segment start of each query row [B,T]
    int32_t *records;
    int B, T, C, Hq, Hkv, window, r, hpw, rb, nhc, nqb;
    int prefix;             // query rows sit at s_b - t_b + i (else at i, t_b = s_b = n_b)
    // Split of each block's key range over nsplit workgroups of tps tiles
    // (nsplit > 1: partials to the workspace, merged by prefix_merge_kernel).
    int nsplit, tps;
    float *o_part;          // [nsplit, B, T, Hq, D] normalised partial outputs
    float *lse_part;        // [nsplit, B, T, Hq] log2-sum-exp (-inf: no key)
    int32_t *rec_part;      // [nsplit, B, T, Hq, 4] {count, lowest, highest, xor}
    float scale_log2; // |scale| * log2(e)
    uint32_t qneg;    // 0x80008000 when scale < 0: Q's sign bits are flipped on load
};

// Direct global-to-LDS 16-byte load (lane i lands at lds_addr + 16*i).  It is
// issued from inline assembly so that the compiler, which cannot tell which
// LDS bytes the transfer writes, does not put a wait for it in front of every
// transposing LDS read of the other stage.  It has no register result; the
// kernel itself waits for it (vmcnt(0), then a workgroup barrier) before the
// stage it fills is read.
__device__ __forceinline__ void dma16(const uint16_t *gptr, uint32_t lds_addr) {
    asm volatile("global_load_lds_dwordx4 %1, off" : : "{m0}"(lds_addr), "v"(gptr) : "memory");
}
// Same, with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane byte
// offset (no per-lane 64-bit address arithmetic on interior tiles).
__device__ __forceinline__ void dma16s(const void *sbase, uint32_t voff, uint32_t lds_addr) {
    asm volatile("global_load_lds_dwordx4 %1, %2" : : "{m0}"(lds_addr), "v"(voff), "s"(sbase) : "memory");
}

// Byte offset of an LDS object in the workgroup's LDS allocation.
__device__ __forceinline__ uint32_t lds_offset(const void *p) {
    return static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void *)p));
}

__device__ __forceinline__ s16x4 ds_read_tr(const uint16_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(p));
}

// LDS tiles are unpadded (64 rows x d bf16 each) and filled by direct
// global-to-LDS loads, which place lane i's 16 bytes at base + 16*i.  The
// bank spread comes from XOR-swizzling the 16-byte chunks of each row instead
// of padding: chunk c of row r lives in slot c ^ f(r).
//   K rows are read 16 B per lane, 16 consecutive rows per pass:
//     f_K(r) = (r / RPL) % CPR puts those 16 reads on 16 distinct bank groups.
//   V rows are read with ds_read_b64_tr_b16, 4 consecutive rows x 4 chunks
//   per half-wavefront: f_V(r) = ((r / RPL) % (4 / RPL)) * 4 does the same.
// (CPR = d/8 chunks per row, RPL = 16/CPR rows per 256-byte bank line.)
template <int D> struct PrefillLayout {
    static constexpr int CPR = D / 8;
    static constexpr int RPL = 16 / CPR;
    static constexpr int kTileBytes = kPBN * D * 2;
    __device__ static int fk(int r) { return (r / RPL) % CPR; }
    __device__ static int fv(int r) { return ((r / RPL) % (4 / RPL)) * 4; }
};

// Per-wavefront tile math: one wavefront owns 32 query rows (lane l holds row
// l & 31 together with lane l ^ 32) and works through one 64-key tile in
// three steps -- scores, softmax, P.V.
template <int D, bool kRecord> struct TileMath {
    using L = PrefillLayout<D>;
    static constexpr int KS = D / 16; // 16-feature k-steps of Q.K (32x32x16)
    static constexpr int DB = D / 32; // 32-column blocks of P.V
    static constexpr int CPR = L::CPR;

    __device__ __forceinline__ static bf16x8 kread(const unsigned char *kst, int s, int kb, int lane) {
        const int row = kb * 32 + (lane & 31);
        const int c = 2 * s + (lane >> 5);
        return *reinterpret_cast<const bf16x8 *>(kst + (row * CPR + (c ^ L::fk(row))) * 16);
    }

    // S^T = K . Q^T for the tile's two 32-key blocks, chains interleaved.
    // The K operands are read one k-step ahead of their MFMAs; the
    // scheduling barriers keep the compiler from hoisting every read of the
    // tile up front, which would hold 16 operands in registers.
    __device__ __forceinline__ static void scores(const unsigned char *kst, const bf16x8 (&qb)[KS],
                                                  f32x16 (&sacc)[2], int lane) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                sacc[kb][e] = 0.f;
        bf16x8 kc0 = kread(kst, 0, 0, lane), kc1 = kread(kst, 0, 1, lane);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            bf16x8 kn0 = kc0, kn1 = kc1;
            if (s + 1 < KS) {
                kn0 = kread(kst, s + 1, 0, lane);
                kn1 = kread(kst, s + 1, 1, lane);
            }
            sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kc0, qb[s], sacc[0], 0, 0, 0);
            sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kc1, qb[s], sacc[1], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            kc0 = kn0;
            kc1 = kn1;
        }
    }

    // Mask (edge tiles only), the row's max, lazy rescale, exponentials and
    // the bf16 P^T operands (plus the index-set records).
    template <bool full>
    __device__ __forceinline__ static void softmax(f32x16 (&sacc)[2], bf16x8 (&pb)[2][2],
                                                   f32x16 (&oacc)[DB], float &m, float &lsum,
                                                   int &r_cnt, int &r_xor, int &r_lo, int &r_hi,
                                                   int j0, int my_pos, int lo_row, int lane,
                                                   float scale_log2) {
        const int qq = lane >> 5;
        // Mask (diagonal, window-edge and padded-row tiles only) and the
        // row's max.  Lane l holds row r0 + (l & 31) and keys
        // j0 + kb*32 + 8*(v/4) + 4*(l>>5) + v%4.  Scores stay unscaled;
        // the scale (>= 0 after the sign flip of Q) is folded into one FMA
        // in front of the exponential.
        float tmax = -INFINITY;
        if constexpr (full) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    tmax = fmaxf(tmax, sacc[kb][v]);
        } else {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int j = j0 + kb * 32 + 8 * (v / 4) + 4 * qq + (v % 4);
                    // lo_row is INT_MAX on inactive rows: nothing kept
                    const bool keep = (j <= my_pos) && (j >= lo_row);
                    sacc[kb][v] = keep ? sacc[kb][v] : -INFINITY;
                    tmax = fmaxf(tmax, sacc[kb][v]);
                }
        }
        {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax),
                                                             __float_as_uint(tmax), false, false);
            tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])); // lanes l and l^32
        }
        tmax = (tmax == -INFINITY) ? -INFINITY : tmax * scale_log2;

        // Lazy rescale: the reference maximum m only moves when a row's new
        // scores exceed it by more than 2^8, so every p = 2^(x - m) stays
        // <= 256 and the accumulators are touched only on those rare
        // tiles.  The final division by the running sum uses the same m,
        // so the result is the same softmax.
        const bool grow = tmax > m + 8.f;
        if (__builtin_amdgcn_ballot_w64(grow)) {
            // rows that do not grow keep m and alpha = 1 (m may still be
            // -inf there, where m - m would be NaN)
            const float mn = grow ? tmax : m;
            const float alpha = grow ? fast_exp2(m - mn) : 1.f; // 0 when m was -inf
            lsum *= alpha;
#pragma unroll
            for (int i = 0; i < DB; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    oacc[i][e] *= alpha;
            m = mn;
        }
        const float mneg = (m == -INFINITY) ? 0.f : -m;
        float psum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int stp = 0; stp < 2; ++stp) {
                uint32_t w[4];
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    const int v = 8 * stp + 2 * e2;
                    float p0 = fast_exp2(fmaf(sacc[kb][v], scale_log2, mneg));
                    float p1 = fast_exp2(fmaf(sacc[kb][v + 1], scale_log2, mneg));
                    if constexpr (!full) { // masked cells contribute exactly 0
                        p0 = (sacc[kb][v] == -INFINITY) ? 0.f : p0;
                        p1 = (sacc[kb][v + 1] == -INFINITY) ? 0.f : p1;
                    }
                    psum += p0 + p1;
                    w[e2] = pack_bf16x2(p0, p1);
                    if (kRecord) {
#pragma unroll
                        for (int u = 0; u < 2; ++u) {
                            if (sacc[kb][v + u] != -INFINITY) { // a permitted cell
                                const int j = j0 + kb * 32 + 8 * ((v + u) / 4) + 4 * qq + ((v + u) % 4);
                                r_cnt += 1;
                                r_xor ^= j;
                                r_lo = min(r_lo, j);
                                r_hi = max(r_hi, j);
                            }
                        }
                    }
                }
                pb[kb][stp] = __builtin_bit_cast(bf16x8, (uint4){w[0], w[1], w[2], w[3]});
            }
        lsum += psum;
    }

    // O^T += V^T . P^T for the tile.
    __device__ __forceinline__ static void pv(const unsigned char *vst, const bf16x8 (&pb)[2][2],
                                              f32x16 (&oacc)[DB], int lane) {
        const int qq = lane >> 5;
        const int gl = lane & 15;
        const int cgrp = (lane >> 4) & 1; // which 16 columns of a 32-column block
        // O^T += V^T . P^T.  For key block kb and k-step stp, P^T k-slot
        // 8*(l>>5) + e is key kb*32 + 16*stp + 8*(e/4) + 4*(l>>5) + e%4, so
        // V^T needs two runs of 4 consecutive keys per lane: one
        // transposing LDS read per run.  In each 16-lane group, lane j
        // supplies row k0 + j/4, columns c0 + 4*(j%4) .. +3 and receives
        // column c0 + (lane & 15).
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int stp = 0; stp < 2; ++stp) {
                const int k0 = kb * 32 + 16 * stp + 4 * qq;
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const int col = db * 32 + 16 * cgrp + 4 * (gl & 3);
                    const int ra = k0 + (gl >> 2);
                    const int rb2 = ra + 8;
                    const unsigned char *pa =
                        vst + (ra * CPR + ((col >> 3) ^ L::fv(ra))) * 16 + (col & 7) * 2;
                    const unsigned char *pb2 =
                        vst + (rb2 * CPR + ((col >> 3) ^ L::fv(rb2))) * 16 + (col & 7) * 2;
                    const s16x4 lo4 = ds_read_tr(reinterpret_cast<const uint16_t *>(pa));
                    const s16x4 hi4 = ds_read_tr(reinterpret_cast<const uint16_t *>(pb2));
                    const bf16x8 va = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[kb][stp], oacc[db], 0, 0, 0);
                }
            }
    }
};

// NW wavefronts per workgroup: 8 (one workgroup per CU, two wavefronts per
// SIMD) or 4 (two workgroups per CU, so that one's row loads and output
// writes overlap the other's tiles; used where blocks carry little work).
template <int D, bool kRecord, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_mfma_kernel(PrefillArgs a) {
    using L = PrefillLayout<D>;
    using TM = TileMath<D, kRecord>;
    constexpr int KS = D / 16;   // 16-feature k-steps of Q.K (32x32x16)
    constexpr int DB = D / 32;   // 32-column blocks of P.V
    constexpr int CPR = L::CPR;
    constexpr int NLD = CPR / NW; // 1 KiB direct loads per wavefront per tensor per tile

    // Two stages of [K | V] tiles.  Separate objects (and a loop unrolled by
    // two) let the compiler see that reads of one stage never alias the
    // direct loads in flight into the other.
    __shared__ __attribute__((aligned(1024))) unsigned char stage0[2 * L::kTileBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char stage1[2 * L::kTileBytes];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave); // same value, kept in an SGPR
    const int lane = tid & 63;
    const int nwaves = a.hpw * a.rb;

    // One-dimensional grid, query block slowest: workgroups are dispatched
    // in order of their linear index, so every head's heaviest (latest)
    // causal blocks start first and the light ones fill the tail.  Adjacent
    // indices differ in (batch row, KV group, head chunk); with 8 or a
    // multiple of them per query block, each XCD keeps seeing the same KV
    // groups, whose K/V then stay in that XCD's L2.
    // (With a split key range the split index sits between the query block
    // and the (b, g, head chunk) index.)
    const int per_blk = a.B * a.Hkv * a.nhc;
    const int lin_id = static_cast<int>(blockIdx.x);
    const int qblk = a.nqb - 1 - lin_id / (per_blk * a.nsplit); // heaviest blocks first
    const int split = (lin_id / per_blk) % a.nsplit;
    const int rest = lin_id % per_blk;
    const int b = rest / (a.Hkv * a.nhc);
    const int g = (rest / a.nhc) % a.Hkv;
    const int hc = rest % a.nhc;
    const int rows_wg = kPRows * a.rb;
    const int q0 = qblk * rows_wg;

    const bool wave_on = wave < nwaves;
    const int hh = wave % a.hpw;            // head within the workgroup
    const int rsub = wave / a.hpw;          // 32-row block within the workgroup
    const int h = g * a.r + hc * a.hpw + hh;
    const int r0 = q0 + rsub * kPRows;
    const int my_row = r0 + (lane & 31);    // query row index (output row)

    // The row's cell: query row i of the t_b new ones sits at cell
    // s_b - t_b + i, the offset rule of "How do you implement grouped query
    // attention (GQA)?", section "Worked example" (a plain prefill has
    // t_b = s_b = n_b, so row i is cell i).  It reads keys lo..p with lo the
    // later of its segment start and its window start.
    int s_b, t_b;
    if (a.prefix) {
        s_b = a.seqlens ? a.seqlens[b] : a.C;
        t_b = a.qlens ? a.qlens[b] : a.T;
    } else {
        s_b = a.seqlens ? a.seqlens[b] : a.T;
        t_b = s_b;
    }
    const int my_pos = s_b - t_b + my_row;
    const int my_seg = (a.segs && my_row < a.T) ? a.segs[(int64_t)b * a.T + my_row] : 0;
    const int lo_cand = segment_lo(my_pos, my_seg, a.window);
    const bool row_on = wave_on && my_row < t_b && my_pos >= 0 && lo_cand >= 0;
    const int lo_row = row_on ? lo_cand : INT_MAX;

    // The wavefront's key range (lanes l and l ^ 32 share a row) and whether
    // all its rows are active; then the workgroup's, through LDS.
    const bool w_all = __builtin_amdgcn_ballot_w64(row_on) == ~0ull;
    const int w_lo = wave_min_i(lo_row);                        // INT_MAX: no active row
    const int w_lo_last = wave_max_i(row_on ? lo_row : -1);
    const int w_last = wave_max_i(row_on ? my_pos : -1);        // -1: no active row
    const int w_first = wave_min_i(row_on ? my_pos : INT_MAX);
    __shared__ int sm_range[NW][2];
    if (lane == 0) {
        sm_range[wave][0] = w_lo;
        sm_range[wave][1] = w_last;
    }
    __syncthreads();
    int wg_lo = INT_MAX, wg_last = -1;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        wg_lo = min(wg_lo, sm_range[w][0]);
        wg_last = max(wg_last, sm_range[w][1]);
    }
    const int64_t out_stride = (int64_t)a.Hq * D; // between cells in [B,T,Hq,D]

    // This workgroup's tiles: the block's key range, or its split-th part.
    int tile_lo = wg_lo / kPBN;
    int tile_hi = wg_last / kPBN;
    if (a.nsplit > 1) {
        tile_lo += split * a.tps;
        tile_hi = min(tile_hi, tile_lo + a.tps - 1);
    }
    // Partial results of a split key range: this split's normalised output,
    // its log2-sum-exp (-inf when it folded no key) and its index-set part.
    auto write_part = [&](int row, const float *o4, float lse, int cnt, int klo, int khi, int kx,
                          bool with_o) {
        const int64_t prow = (((int64_t)split * a.B + b) * a.T + row) * a.Hq + h;
        if (with_o) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) {
                    const int col = db * 32 + 8 * v4 + 4 * (lane >> 5);
                    *reinterpret_cast<float4 *>(a.o_part + prow * D + col) =
                        make_float4(o4[(db * 4 + v4) * 4 + 0], o4[(db * 4 + v4) * 4 + 1],
                                    o4[(db * 4 + v4) * 4 + 2], o4[(db * 4 + v4) * 4 + 3]);
                }
        }
        if ((lane >> 5) == 0) {
            a.lse_part[prow] = lse;
            if (kRecord) {
                int32_t *rp = a.rec_part + prow * 4;
                rp[0] = cnt; rp[1] = klo; rp[2] = khi; rp[3] = kx;
            }
        }
    };

    if (a.nsplit > 1 && (wg_last < 0 || tile_lo > tile_hi)) {
        // nothing to fold in this split: an empty partial for every row
        if (wave_on && (lane >> 5) == 0 && my_row < a.T)
            write_part(my_row, nullptr, -INFINITY, 0, INT_MAX, -1, 0, false);
        return;
    }
    if (wg_last < 0) {
        // no active row: the whole block is padding, write zeros
        if (wave_on) {
            for (int i = lane; i < kPRows * (D / 4); i += 64) {
                const int row = r0 + i / (D / 4);
                const int c4 = (i % (D / 4)) * 4;
                if (row < a.T) {
                    uint16_t *o = a.out + ((int64_t)b * a.T + row) * out_stride + (int64_t)h * D + c4;
                    *reinterpret_cast<uint2 *>(o) = uint2{0u, 0u};
                    if (kRecord && c4 == 0) {
                        int32_t *rec = a.records + (((int64_t)b * a.T + row) * a.Hq + h) * 5;
                        rec[0] = g; rec[1] = -1; rec[2] = -1; rec[3] = 0; rec[4] = 0;
                    }
                }
            }
        }
        return;
    }

    // Q^T operand, kept for the whole loop: lane l holds row r0 + (l & 31),
    // features s*16 + 8*(l >> 5) .. +8 (sign bits flipped for a negative scale).
    // The loads are issued unconditionally from a valid row (row 0 of a head
    // of this group for idle lanes) so that all of them are in flight at
    // once; lanes without a row zero their operand afterwards.
    bf16x8 qb[KS];
    {
        const bool ok = wave_on && my_row < a.T;
        const int hq = wave_on ? h : g * a.r;
        const uint16_t *qrow = a.q + (((int64_t)b * a.Hq + hq) * a.T + (ok ? my_row : 0)) * D;
        uint4 raw[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s)
            raw[s] = *reinterpret_cast<const uint4 *>(qrow + s * 16 + 8 * (lane >> 5));
        const uint32_t keep = ok ? 0xFFFFFFFFu : 0u;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            raw[s].x = (raw[s].x ^ a.qneg) & keep;
            raw[s].y = (raw[s].y ^ a.qneg) & keep;
            raw[s].z = (raw[s].z ^ a.qneg) & keep;
            raw[s].w = (raw[s].w ^ a.qneg) & keep;
            qb[s] = __builtin_bit_cast(bf16x8, raw[s]);
        }
    }

    const int64_t kv_off = ((int64_t)b * a.Hkv + g) * (int64_t)a.C * D;
    const uint16_t *kbase = a.k + kv_off;
    const uint16_t *vbase = a.v + kv_off;

    // Direct loads of one tile into a stage: wavefront w issues loads
    // ii = it*NW + w; lane l fills linear chunk ii*64 + l, i.e. row
    // (ii*64 + l) / CPR and slot (ii*64 + l) % CPR, with the global chunk the
    // swizzle puts there.  An interior tile uses per-lane byte offsets fixed
    // for the whole loop; the workgroup's last tile repeats its last key in
    // the rows past it (finite data, always masked).
    uint32_t koffs[NLD], voffs[NLD];
#pragma unroll
    for (int it = 0; it < NLD; ++it) {
        const int ii = it * NW + wave_u;
        const int lin = ii * 64 + lane;
        const int row = lin / CPR;
        const int slot = lin % CPR;
        koffs[it] = static_cast<uint32_t>(row * D * 2 + (slot ^ L::fk(row)) * 16);
        voffs[it] = static_cast<uint32_t>(row * D * 2 + (slot ^ L::fv(row)) * 16);
    }
    auto load_tile = [&](int tile, uint32_t dst) {
        const int j0 = tile * kPBN;
        if (j0 + kPBN - 1 <= wg_last) {
            const void *kb0 = kbase + (int64_t)j0 * D;
            const void *vb0 = vbase + (int64_t)j0 * D;
#pragma unroll
            for (int it = 0; it < NLD; ++it) {
                const int ii = it * NW + wave_u;
                dma16s(kb0, koffs[it], dst + ii * 1024);
                dma16s(vb0, voffs[it], dst + L::kTileBytes + ii * 1024);
            }
        } else {
#pragma unroll
            for (int it = 0; it < NLD; ++it) {
                const int ii = it * NW + wave_u;
                const int lin = ii * 64 + lane;
                const int row = lin / CPR;
                const int slot = lin % CPR;
                const int key = min(j0 + row, wg_last);
                dma16(kbase + (int64_t)key * D + (slot ^ L::fk(row)) * 8, dst + ii * 1024);
                dma16(vbase + (int64_t)key * D + (slot ^ L::fv(row)) * 8, dst + L::kTileBytes + ii * 1024);
            }
        }
    };

    f32x16 oacc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            oacc[i][e] = 0.f;
    float m = -INFINITY; // reference max of this lane's row (base-2 scaled)
    float lsum = 0.f;    // this lane's share of the running sum
    int r_cnt = 0, r_xor = 0, r_lo = INT_MAX, r_hi = -1;
    const int qq = lane >> 5;

    // One tile: start the direct loads of the next tile into the other stage,
    // compute on this stage, then wait until every wavefront's loads landed
    // and every wavefront is done with this stage.
    auto step = [&](int tile, const unsigned char *src, unsigned char *nxt) {
        if (tile < tile_hi)
            load_tile(tile + 1, lds_offset(nxt));
        const unsigned char *kst = src;
        const unsigned char *vst = src + L::kTileBytes;
        const int j0 = tile * kPBN;
        const bool work = w_last >= 0 && j0 <= w_last && j0 + kPBN - 1 >= w_lo;
        // Interior tiles (every key permitted for every row of the wavefront)
        // and edge tiles (diagonal, window edge, padded rows) are separate
        // instantiations so that interior tiles carry no masking code.
        auto compute = [&](auto full_tag) {
            constexpr bool full = decltype(full_tag)::value;
            f32x16 sacc[2];
            bf16x8 pb[2][2];
            TM::scores(kst, qb, sacc, lane);
            TM::template softmax<full>(sacc, pb, oacc, m, lsum, r_cnt, r_xor, r_lo, r_hi, j0, my_pos,
                                       lo_row, lane, a.scale_log2);
            TM::pv(vst, pb, oacc, lane);
        };
        if (work) {
            if (w_all && (j0 + kPBN - 1 <= w_first) && (j0 >= w_lo_last))
                compute(std::true_type{});
            else
                compute(std::false_type{});
        }
        __builtin_amdgcn_s_waitcnt(0x0F70); // vmcnt(0): next tile's loads of this wavefront landed
        __syncthreads();                     // ... of every wavefront; this stage is free again
    };

    load_tile(tile_lo, lds_offset(stage0));
    __builtin_amdgcn_s_waitcnt(0x0F70); // vmcnt(0): this wavefront's tile loads landed
    __syncthreads();
    for (int tile = tile_lo; tile <= tile_hi; tile += 2) {
        step(tile, stage0, stage1);
        if (tile + 1 > tile_hi)
            break;
        step(tile + 1, stage1, stage0);
    }

    if (!wave_on)
        return;
    lsum += __shfl_xor(lsum, 32, 64);
    if (kRecord) {
        r_cnt += __shfl_xor(r_cnt, 32, 64);
        r_xor ^= __shfl_xor(r_xor, 32, 64);
        r_lo = min(r_lo, __shfl_xor(r_lo, 32, 64));
        r_hi = max(r_hi, __shfl_xor(r_hi, 32, 64));
    }
    if (my_row >= a.T)
        return;
    const bool active = row_on;
    const float inv = (active && lsum > 0.f) ? 1.f / lsum : 0.f;
    if (a.nsplit > 1) {
        float o4[DB * 16];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                o4[db * 16 + e] = oacc[db][e] * inv;
        const bool folded = active && lsum > 0.f;
        write_part(my_row, o4, folded ? m + __builtin_amdgcn_logf(lsum) : -INFINITY,
                   folded ? r_cnt : 0, r_lo, r_hi, r_xor, true);
        return;
    }
    uint16_t *orow = a.out + ((int64_t)b * a.T + my_row) * out_stride + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
            const int col = db * 32 + 8 * v4 + 4 * qq;
            uint2 pk;
            pk.x = pack_bf16x2(oacc[db][4 * v4 + 0] * inv, oacc[db][4 * v4 + 1] * inv);
            pk.y = pack_bf16x2(oacc[db][4 * v4 + 2] * inv, oacc[db][4 * v4 + 3] * inv);
            *reinterpret_cast<uint2 *>(orow + col) = pk;
        }
    if (kRecord && qq == 0) {
        int32_t *rec = a.records + (((int64_t)b * a.T + my_row) * a.Hq + h) * 5;
        rec[0] = g;
        if (active) {
            rec[1] = r_lo; rec[2] = r_hi; rec[3] = r_cnt; rec[4] = r_xor;
        } else {
            rec[1] = -1; rec[2] = -1; rec[3] = 0; rec[4] = 0;
        }
    }
}

// Merge of a split key range: one thread per 4 output features of a row
// (b, i, h); out = sum_s w_s o_s / sum_s w_s with w_s = 2^(lse_s - max lse)
// ("GQA, FlashAttention and the KV cache", section "FlashAttention").  A row
// no split folded a key into is inactive: zero output.
template <int D, bool kRecord>
__global__ __launch_bounds__(256) void prefix_merge_kernel(PrefillArgs a) {
    constexpr int Q4 = D / 4;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t rows = (int64_t)a.B * a.T * a.Hq;
    if (idx >= rows * Q4)
        return;
    const int64_t row = idx / Q4; // (b * T + i) * Hq + h
    const int c4 = static_cast<int>(idx % Q4) * 4;
    // The partials are loaded kChunk splits at a time, every load of a chunk
    // in flight together (a loop that waits on each load in turn makes the
    // kernel a chain of memory round trips).  The first chunk's outputs stay
    // in registers for the second pass.  A split with lse = -inf never wrote
    // its output slot; that slot is loaded (it lies inside the workspace) but
    // not used.  The arithmetic is the plain two-pass order: the maximum over
    // all splits, then the weighted sums in split order.
    constexpr int kChunk = 8;
    const float *lse = a.lse_part + row;
    const float *op = a.o_part + row * D + c4;
    const int64_t ostride = rows * D;
    float lc[kChunk];
    float4 oc[kChunk];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
        if (i < a.nsplit) {
            lc[i] = lse[i * rows];
            oc[i] = *reinterpret_cast<const float4 *>(op + i * ostride);
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < kChunk; ++i)
        if (i < a.nsplit)
            mx = fmaxf(mx, lc[i]);
    for (int s0 = kChunk; s0 < a.nsplit; s0 += kChunk) {
        float t[kChunk];
#pragma unroll
        for (int i = 0; i < kChunk; ++i)
            if (s0 + i < a.nsplit)
                t[i] = lse[(s0 + i) * rows];
#pragma unroll
        for (int i = 0; i < kChunk; ++i)
            if (s0 + i < a.nsplit)
                mx = fmaxf(mx, t[i]);
    }
    uint2 pk = uint2{0u, 0u};
    if (mx != -INFINITY) {
        float den = 0.f;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int s0 = 0; s0 < a.nsplit; s0 += kChunk) {
            if (s0 > 0) {
#pragma unroll
                for (int i = 0; i < kChunk; ++i) {
                    if (s0 + i < a.nsplit) {
                        lc[i] = lse[(s0 + i) * rows];
                        oc[i] = *reinterpret_cast<const float4 *>(op + (s0 + i) * ostride);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < kChunk; ++i) {
                if (s0 + i >= a.nsplit || lc[i] == -INFINITY)
                    continue; // past the last split, or nothing folded
                const float w = fast_exp2(lc[i] - mx);
                const float4 o = oc[i];
                den += w;
                acc.x = fmaf(w, o.x, acc.x);
                acc.y = fmaf(w, o.y, acc.y);
                acc.z = fmaf(w, o.z, acc.z);
                acc.w = fmaf(w, o.w, acc.w);
            }
        }
        const float inv = 1.f / den;
        pk.x = pack_bf16x2(acc.x * inv, acc.y * inv);
        pk.y = pack_bf16x2(acc.z * inv, acc.w * inv);
    }
    *reinterpret_cast<uint2 *>(a.out + row * D + c4) = pk;
    if (kRecord && c4 == 0) {
        // record partials: 16 bytes per split, kChunk splits in flight
        // together; a split with lse = -inf wrote none (its slot is loaded,
        // inside the workspace, and skipped)
        int cnt = 0, x = 0, rl = INT_MAX, rh = -1;
        const int4 *rp = reinterpret_cast<const int4 *>(a.rec_part) + row;
        for (int s0 = 0; s0 < a.nsplit; s0 += kChunk) {
            int4 rc[kChunk];
            float rlse[kChunk];
#pragma unroll
            for (int i = 0; i < kChunk; ++i) {
                if (s0 + i < a.nsplit) {
                    rc[i] = rp[(s0 + i) * rows];
                    rlse[i] = lse[(s0 + i) * rows];
                }
            }
#pragma unroll
            for (int i = 0; i < kChunk; ++i) {
                if (s0 + i < a.nsplit && rlse[i] != -INFINITY) {
                    cnt += rc[i].x;
                    rl = min(rl, rc[i].y);
                    rh = max(rh, rc[i].z);
                    x ^= rc[i].w;
                }
            }
        }
        int32_t *rec = a.records + row * 5;
        rec[0] = static_cast<int>(row % a.Hq) / a.r;
        if (cnt > 0) {
            rec[1] = rl; rec[2] = rh; rec[3] = cnt; rec[4] = x;
        } else {
            rec[1] = -1; rec[2] = -1; rec[3] = 0; rec[4] = 0;
        }
    }
}

// Wavefronts per workgroup.  Packed segments leave each block of rows only
// the tiles of its own segment, often a few, against a fixed cost per
// workgroup (its rows' queries loaded, its output written); two 4-wavefront
// workgroups per CU overlap that cost with the other's tiles (57.3 -> 50.9
// us on 4096 cells of 7 packed sequences, against 138.7 -> 149.4 us for a
// plain causal prefill, whose blocks are heavy).
int prefill_waves(bool segmented) { return segmented ? 4 : kPWaves; }

// Heads per workgroup: the largest power of two (at most nw) that divides r;
// the remaining wavefronts take further 32-row blocks of the same heads, so
// every workgroup runs all nw wavefronts.  (One staged tile feeds every
// wavefront whatever the split between heads and rows; more heads mean
// fewer rows per workgroup and less work on the causal diagonal.)
static void prefill_shape(int r, int nw, int *hpw, int *rb) {
    int x = nw;
    while (r % x != 0)
        x /= 2;
    *hpw = x;
    *rb = nw / x;
}

// The grid is one-dimensional: ceil(T / (32*rb)) * B * Hkv * (r/hpw)
// workgroups of nw*64 work-items, whose total must fit a 32-bit count.
static int64_t prefill_workgroups(int B, int T, int Hq, int Hkv, int nw) {
    int hpw, rb;
    prefill_shape(Hq / Hkv, nw, &hpw, &rb);
    const int64_t nqb = ((int64_t)T + kPRows * rb - 1) / (kPRows * rb);
    return nqb * B * Hkv * ((Hq / Hkv) / hpw);
}

bool prefill_grid_ok(int B, int T, int Hq, int Hkv, int nsplit, int nw) {
    const int64_t wgs = prefill_workgroups(B, T, Hq, Hkv, nw) * (nsplit > 1 ? nsplit : 1);
    return T >= 0 && wgs * nw * 64 <= (int64_t)UINT32_MAX &&
           (int64_t)B * T * Hq * 64 <= (int64_t)UINT32_MAX; // merge grid
}

static size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Split of the key range for queries against a cached prefix: when the
// blocks alone give fewer than 256 workgroups (one per CU), each block's key
// range is cut into nsplit parts of tps tiles (at least 4).  The
// plan depends only on the arguments (the workspace size is a function of
// them).
PrefixPlan plan_prefix(int B, int T, int C, int Hq, int Hkv, int d, int window) {
    PrefixPlan p{};
    p.nsplit = 1;
    p.tps = 0;
    // (counted for 8-wavefront workgroups whatever the call runs, so that the
    // workspace size depends on the shape arguments only)
    int hpw, rb;
    prefill_shape(Hq / Hkv, kPWaves, &hpw, &rb);
    const int64_t nqb = ((int64_t)T + kPRows * rb - 1) / (kPRows * rb);
    const int64_t units = nqb * B * Hkv * ((Hq / Hkv) / hpw);
    const int64_t elig = (window > 0 && window < C) ? window : C;
    // tiles a block can span: its rows' key ranges, at most the cache
    const int64_t maxtiles = std::min<int64_t>((C + kPBN - 1) / kPBN,
                                               (elig + kPRows * rb) / kPBN + 2);
    const int64_t target = 256;
    if (units > 0 && units < target && maxtiles >= 8) {
        int64_t ns = (target + units - 1) / units;
        ns = std::min<int64_t>(ns, maxtiles / 4);
        if (ns > 1) {
            p.tps = static_cast<int>((maxtiles + ns - 1) / ns);
            p.nsplit = static_cast<int>((maxtiles + p.tps - 1) / p.tps);
        }
    }
    if (p.nsplit > 1) {
        const size_t rows = (size_t)p.nsplit * B * T * Hq;
        p.o_off = 0;
        p.lse_off = align256(rows * d * sizeof(float));
        p.rec_off = p.lse_off + align256(rows * sizeof(float));
        p.bytes = p.rec_off + align256(rows * 4 * sizeof(int32_t));
    }
    return p;
}

template <int D, bool kRecord, int NW>
static hipError_t launch_p(const PrefillArgs &a, dim3 grid, hipStream_t s) {
    prefill_mfma_kernel<D, kRecord, NW><<<grid, NW * 64, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit <= 1)
        return e;
    const int64_t threads = (int64_t)a.B * a.T * a.Hq * (D / 4);
    prefix_merge_kernel<D, kRecord><<<dim3((unsigned)((threads + 255) / 256)), 256, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_prefill_mfma(const Problem &p, const PrefixPlan &plan, void *workspace,
                               hipStream_t stream) {
    PrefillArgs a;
    a.q = static_cast<const uint16_t *>(p.q);
    a.k = static_cast<const uint16_t *>(p.k);
    a.v = static_cast<const uint16_t *>(p.v);
    a.out = static_cast<uint16_t *>(p.out);
    a.seqlens = p.seqlens;
    a.qlens = p.qlens;
    a.segs = p.segs;
    a.prefix = p.prefix ? 1 : 0;
    a.records = p.records;
    a.T = p.T; a.C = p.C; a.Hq = p.Hq; a.Hkv = p.Hkv; a.window = p.window;
    a.r = p.Hq / p.Hkv;
    const int nw = prefill_waves(p.segs != nullptr);
    prefill_shape(a.r, nw, &a.hpw, &a.rb);
    a.nhc = a.r / a.hpw;
    a.nqb = (p.T + kPRows * a.rb - 1) / (kPRows * a.rb);
    a.scale_log2 = fabsf(p.scale) * kLog2e;
    a.qneg = p.scale < 0.f ? 0x80008000u : 0u;
    a.B = p.B;
    a.nsplit = plan.nsplit > 1 ? plan.nsplit : 1;
    a.tps = plan.tps;
    unsigned char *w = static_cast<unsigned char *>(workspace);
    a.o_part = a.nsplit > 1 ? reinterpret_cast<float *>(w + plan.o_off) : nullptr;
    a.lse_part = a.nsplit > 1 ? reinterpret_cast<float *>(w + plan.lse_off) : nullptr;
    a.rec_part = a.nsplit > 1 ? reinterpret_cast<int32_t *>(w + plan.rec_off) : nullptr;
    dim3 grid(static_cast<uint32_t>(prefill_workgroups(p.B, p.T, p.Hq, p.Hkv, nw) * a.nsplit), 1, 1);
    const bool rec = p.records != nullptr;
    if (nw == 4) {
        if (p.d == 128)
            return rec ? launch_p<128, true, 4>(a, grid, stream) : launch_p<128, false, 4>(a, grid, stream);
        return rec ? launch_p<64, true, 4>(a, grid, stream) : launch_p<64, false, 4>(a, grid, stream);
    }
    if (p.d == 128)
        return rec ? launch_p<128, true, 8>(a, grid, stream) : launch_p<128, false, 8>(a, grid, stream);
    return rec ? launch_p<64, true, 8>(a, grid, stream) : launch_p<64, false, 8>(a, grid, stream);
}

} // namespace gqa
