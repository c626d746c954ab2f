// gqa_decode.hip -- bf16 single-token decode over a KV cache, split along the
// cache length, with matrix-core (MFMA) dot products and a log-sum-exp merge.
//
// Work decomposition.  A row (b, query head h) reads the key cells
// lo..n_b-1 of KV head g = floor(h / r) (lo = max(0, n_b - w) with a window;
// "Share key/value heads and make context explicit", "Intersect the window
// with the context already permitted", and "Extend the existing full and
// cached attention paths" for the query's position).  That range is cut into
// chunks of `chunk` keys counted from lo; a workgroup takes one chunk of one
// unit (batch row b, KV group g, up to 16 of the group's query heads) for all
// of the unit's heads at once, so every K/V cell is fetched from HBM once per
// group and feeds the r heads that share it -- the saving GQA exists for
// ("How do you implement grouped query attention (GQA)?", Step 4: the cache
// stores G heads and is repeated on read; here the repeat never
// materialises).
//
// Inside a workgroup, 4 wavefronts take interleaved 32-key tiles; each
// wavefront prefetches its next tile while it computes the current one.
// Per tile:
//   S^T[32 keys x 16 heads] = K_tile[32 x d] . Q^T[d x 16]   (MFMA 16x16x32 bf16)
//   online softmax per head in base 2 (running max m, running sum l)
//   O^T[d x 16] += V_tile^T[d x 32] . P^T[32 x 16]            (MFMA 16x16x32 bf16)
// The transposed products keep every per-head quantity in the lanes that own
// that head (lane & 15), so the softmax rescale never crosses lanes.  K is
// read straight from HBM into the MFMA operand layout; V goes through a
// wavefront-private LDS tile and comes back transposed (ds_read_b64_tr_b16).
// K/V are streamed with non-temporal loads: each cell is used once.
//
// The 4 wavefronts' states are merged through LDS.  A row with a single chunk
// is finished right there.  Otherwise each workgroup writes its normalised
// partial and log2-sum-exp to the workspace, and a second, small kernel
// merges the chunks of every row with weights 2^(lse_s - max lse) ("GQA,
// FlashAttention and the KV cache", section "FlashAttention": blockwise
// softmax with a numerically stable running normalisation gives the dense
// result).  The kernel boundary orders the two steps; no workgroup waits on
// another.
//
// The extended instantiation (kExt) adds two cache forms.  A candidate: the
// new cell n_b - 1 is read from its own key/value buffers and committed to
// its cache slot in the same launch, as the incremental step of "Extend the
// existing full and cached attention paths" includes the candidate key before
// the cache commits.  A rolling cache: cell j lives in slot j mod C (the
// rolling buffer of the Mistral 7B paragraph in "Share key/value heads and
// make context explicit"), with a window of at most C cells.
#include <limits.h>

#include <algorithm>
#include <mutex>

#include "gqa_common.hpp"
#include "gqa_internal.hpp"

namespace gqa {

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

struct DecodeArgs {
    const uint16_t *q;
    const uint16_t *k;
    const uint16_t *v;
    const int32_t *seqlens;
    uint16_t *out;      // [B, Hq, D]
    int32_t *records;   // [B, Hq, 5] (record instantiation only)
    float *o_part;      // [B, Hq, nsplit, D]
    float *lse_part;    // [B, Hq, nsplit]
    int32_t *rec_part;  // [B, Hq, nsplit, 4] (record instantiation only)
    int C, Hq, Hkv, window, r, nhc, nsplit, chunk;
    int units; // B * Hkv * nhc
    float scale_log2;
    // kExt only
    const uint16_t *knew; // [B, Hkv, D] candidate key (nullable)
    const uint16_t *vnew; // [B, Hkv, D] candidate value
    uint16_t *kw;         // the K/V caches again, writable, for the commit
    uint16_t *vw;
    int ring;             // cell j in slot j mod C
};

template <int D> struct DecodeSmem {
    // V tile pitch (u16): 72 dwords puts the 8 rows one half-wavefront reads
    // with ds_read_b64_tr_b16 on disjoint banks.
    static constexpr int LDV = D + 16;
    static constexpr int kVBytes = kDecodeWaves * kDecodeTile * LDV * 2;
    // Staged partial outputs: rows of D + 4 floats, so that the 16 heads'
    // 16-byte writes fall on distinct banks.
    static constexpr int LDO = D + 4;
    static constexpr int kOBytes = kDecodeWaves * kDecodeHeads * LDO * 4;
    static constexpr int kBytes = (kVBytes > kOBytes ? kVBytes : kOBytes);
};

__device__ __forceinline__ s16x4 ds_read_tr_d(const uint16_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(p));
}

template <int D, bool kRecord, bool kExt>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
    constexpr int KS = D / 32;               // 32-feature k-steps of Q.K
    constexpr int DB = D / 16;               // 16-column blocks of P.V
    constexpr int LDV = DecodeSmem<D>::LDV;
    constexpr int LDO = DecodeSmem<D>::LDO;
    constexpr int VPI = 1024 / (2 * D);      // keys per 1 KiB wavefront load
    constexpr int LPK = 64 / VPI;            // lanes per key row
    constexpr int VIT = kDecodeTile / VPI;   // V loads per tile
    constexpr int STEP = kDecodeWaves * kDecodeTile;

    __shared__ __attribute__((aligned(16))) unsigned char smem[DecodeSmem<D>::kBytes];
    __shared__ float sm_m[kDecodeWaves][kDecodeHeads];
    __shared__ float sm_l[kDecodeWaves][kDecodeHeads];
    __shared__ float sm_lse[kDecodeHeads];
    __shared__ int sm_rec[kDecodeWaves][4];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int hl = lane & 15; // head within the 16-head chunk (MFMA column)
    const int qg = lane >> 4; // lane group (MFMA k/row group)

    // One-dimensional grid.  Workgroups are dispatched to the 8 XCDs in turn
    // (linear id mod 8), so all splits of a (b, g, head chunk) unit u run on
    // XCD u mod 8, where the merge kernel's workgroup for u runs too: the
    // merge then finds the partials in that XCD's cache.
    const int ns_grid = a.nsplit > 0 ? a.nsplit : 1;
    const int wid = static_cast<int>(blockIdx.x);
    const int split = (wid >> 3) % ns_grid;
    const int unit = ((wid >> 3) / ns_grid) * 8 + (wid & 7);
    if (unit >= a.units)
        return; // the grid is rounded up to whole groups of 8 units
    const int b = unit / (a.Hkv * a.nhc);
    const int g = (unit / a.nhc) % a.Hkv;
    const int hc = unit % a.nhc;
    const int h0 = g * a.r + hc * kDecodeHeads;
    const int nh = min(kDecodeHeads, a.r - hc * kDecodeHeads);
    const int64_t row0 = (int64_t)b * a.Hq + h0; // first (b, h) row of this workgroup

    const int nb = a.seqlens ? a.seqlens[b] : a.C;
    if (nb <= 0) {
        // empty row: no key is permitted, the output row is zero
        if (split == 0) {
            for (int idx = tid; idx < nh * D; idx += 256)
                a.out[row0 * D + idx] = 0;
            if (kRecord && tid < nh) {
                int32_t *rec = a.records + (row0 + tid) * 5;
                rec[0] = g; rec[1] = -1; rec[2] = -1; rec[3] = 0; rec[4] = 0;
            }
        }
        return;
    }
    const int hi = nb - 1;
    const int lo = window_lo(hi, a.window);
    const int c_lo = lo + split * a.chunk;
    if (c_lo > hi)
        return; // this row has fewer chunks than the grid
    const int c_hi = min(hi, c_lo + a.chunk - 1);
    const int ns = (hi - lo) / a.chunk + 1; // chunks of this row

    // Q^T operand: lane (hl, qg) holds features s*32 + qg*8 .. +8 of head hl.
    bf16x8 qb[KS];
    {
        // columns past the group's last head read that head and are zeroed
        const uint16_t *qrow = a.q + (row0 + min(hl, nh - 1)) * D;
        const bf16x8 zero = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const bf16x8 t = *reinterpret_cast<const bf16x8 *>(qrow + s * 32 + qg * 8);
            qb[s] = (hl < nh) ? t : zero;
        }
    }

    const int64_t lane_off = ((int64_t)b * a.Hkv + g) * (int64_t)a.C * D;
    const uint16_t *kbase = a.k + lane_off;
    const uint16_t *vbase = a.v + lane_off;

    // Cache row of key cell `key` (relative to kbase/vbase), and where the
    // candidate cell reads from.  In a rolling cache the permitted cells
    // lo..hi (fewer than C of them) map to slots key - base or key - base - C
    // with base = C * floor(lo / C).
    const uint16_t *kcand = nullptr, *vcand = nullptr;
    int ring_base = 0;
    if constexpr (kExt) {
        if (a.ring)
            ring_base = (lo / a.C) * a.C;
        if (a.knew) {
            kcand = a.knew + ((int64_t)b * a.Hkv + g) * D;
            vcand = a.vnew + ((int64_t)b * a.Hkv + g) * D;
            // Commit by the workgroup whose chunk holds the new cell (first
            // head chunk only).  No workgroup of this launch reads that slot:
            // the new cell is read from the candidate buffers, and the cell
            // the slot held before (hi - C, rolling cache) is outside the
            // window.
            if (hc == 0 && c_hi == hi && tid < D / 8) {
                int64_t slot = hi;
                if (a.ring)
                    slot = hi - ring_base >= a.C ? hi - ring_base - a.C : hi - ring_base;
                *reinterpret_cast<uint4 *>(a.kw + lane_off + slot * D + tid * 8) =
                    *reinterpret_cast<const uint4 *>(kcand + tid * 8);
                *reinterpret_cast<uint4 *>(a.vw + lane_off + slot * D + tid * 8) =
                    *reinterpret_cast<const uint4 *>(vcand + tid * 8);
            }
        }
    }
    auto cell = [&](int key) -> int64_t {
        if constexpr (kExt) {
            if (a.ring) {
                const int sl = key - ring_base;
                return sl >= a.C ? sl - a.C : sl;
            }
        }
        return key;
    };
    uint16_t *vs = reinterpret_cast<uint16_t *>(smem) + wave * kDecodeTile * LDV;

    // One tile's loads: K in the MFMA operand layout (lane (hl, qg) of key
    // block kb holds key j0 + kb*16 + hl, features s*32 + qg*8 .. +8) and V in
    // its natural layout (16 B per lane, 1 KiB per load).  Keys past the chunk
    // end re-read the chunk's last cell instead of branching around the load:
    // their scores are masked to -inf and their values get weight 0, and that
    // cell is permitted, so its values are the caller's data.
    auto load_tile = [&](int j0, bf16x8 (&ka)[2][KS], u32x4 (&vr)[VIT]) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int key = min(j0 + kb * 16 + hl, c_hi);
            const uint16_t *krow = kbase + cell(key) * D + qg * 8;
            if constexpr (kExt)
                if (kcand && key == hi)
                    krow = kcand + qg * 8;
#pragma unroll
            for (int s = 0; s < KS; ++s)
                ka[kb][s] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8 *>(krow + s * 32));
        }
#pragma unroll
        for (int it = 0; it < VIT; ++it) {
            const int key = min(j0 + it * VPI + lane / LPK, c_hi);
            const int col = (lane % LPK) * 8;
            const uint16_t *vrow = vbase + cell(key) * D;
            if constexpr (kExt)
                if (vcand && key == hi)
                    vrow = vcand;
            vr[it] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(vrow + col));
        }
    };

    // The extended instantiation computes a tile's addresses (rolling-cache
    // slots, candidate substitution: about twice the plain arithmetic) before
    // the wait for the previous tile, so that its loads issue as soon as that
    // tile has landed: 17.5 -> 16.4 us on a ragged rolling-cache decode.  In
    // the plain kernel the same split measured 1.5-6% slower on every shape,
    // so it keeps load_tile.  Early addresses of a tile past the chunk end
    // are clamped like any other, so they are always valid.  The loads name
    // global memory (address space 1) explicitly: behind the empty asm
    // statements that pin the addresses the compiler would otherwise see only
    // generic pointers, and it would issue flat loads.
    typedef __attribute__((address_space(1))) const bf16x8 gbf16x8;
    typedef __attribute__((address_space(1))) const u32x4 gu32x4;
    struct TilePtrs {
        const uint16_t *k[2];
        const uint16_t *v[VIT];
    };
    auto tile_ptrs = [&](int j0) {
        TilePtrs t;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int key = min(j0 + kb * 16 + hl, c_hi);
            const uint16_t *krow = kbase + cell(key) * D + qg * 8;
            if (kcand && key == hi)
                krow = kcand + qg * 8;
            t.k[kb] = krow;
            asm volatile("" : "+v"(t.k[kb]));
        }
#pragma unroll
        for (int it = 0; it < VIT; ++it) {
            const int key = min(j0 + it * VPI + lane / LPK, c_hi);
            const uint16_t *vrow = vbase + cell(key) * D;
            if (vcand && key == hi)
                vrow = vcand;
            t.v[it] = vrow + (lane % LPK) * 8;
            asm volatile("" : "+v"(t.v[it]));
        }
        return t;
    };
    auto load_ptrs = [&](const TilePtrs &t, bf16x8 (&ka)[2][KS], u32x4 (&vr)[VIT]) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int s = 0; s < KS; ++s)
                ka[kb][s] = __builtin_nontemporal_load((gbf16x8 *)(t.k[kb] + s * 32));
#pragma unroll
        for (int it = 0; it < VIT; ++it)
            vr[it] = __builtin_nontemporal_load((gu32x4 *)t.v[it]);
    };

    float m = -INFINITY;
    float lsum = 0.f;
    f32x4 oacc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i)
        oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    int r_cnt = 0, r_xor = 0, r_lo = INT_MAX, r_hi = -1;

    // Wait until one tile's registers have landed.  The scheduling barrier
    // keeps the next tile's loads behind the wait: each wavefront then has
    // one tile (16 KiB at d = 128) in flight while it computes, ~32 MiB over
    // the chip.  With two tiles per wavefront HBM delivered less.
    auto wait_tile = [&](const bf16x8 (&ka)[2][KS], const u32x4 (&vr)[VIT]) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int s = 0; s < KS; ++s)
                asm volatile("" ::"v"(ka[kb][s]));
#pragma unroll
        for (int it = 0; it < VIT; ++it)
            asm volatile("" ::"v"(vr[it]));
        __builtin_amdgcn_sched_barrier(0);
    };

    auto compute_tile = [&](int j0, const bf16x8 (&ka)[2][KS], const u32x4 (&vr)[VIT]) {
        // S^T = K . Q^T ; lane (hl, qg) gets keys kb*16 + qg*4 + i of head hl.
        f32x4 sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kb][s], qb[s], sacc[kb], 0, 0, 0);

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
            *reinterpret_cast<u32x4 *>(vs + row * LDV + col) = vr[it];
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
        // Lazy rescale: the reference maximum m moves only when a head's new
        // scores exceed it by more than 2^8, so every p = 2^(x - m) stays
        // <= 256 and the accumulators are rescaled only on those tiles.  The
        // partial's log2-sum-exp is m + log2(lsum) for whatever m is held,
        // so the result is the same softmax.  Key j0 is always permitted, so
        // a wavefront's first tile has a finite tmax and sets m.
        const bool grow = tmax > m + 8.f;
        if (__builtin_amdgcn_ballot_w64(grow)) {
            const float mn = grow ? tmax : m;
            const float alpha = grow ? fast_exp2(m - mn) : 1.f; // 0 when m was -inf
            lsum *= alpha;
#pragma unroll
            for (int i = 0; i < DB; ++i)
                oacc[i] *= alpha;
            m = mn;
        }
        float psum = 0.f;
        uint32_t pw[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
                const float p0 = fast_exp2(x[kb][i] - m);
                const float p1 = fast_exp2(x[kb][i + 1] - m);
                psum += p0 + p1;
                pw[kb * 2 + i / 2] = pack_bf16x2(p0, p1);
            }
        const bf16x8 pb = __builtin_bit_cast(bf16x8, (uint4){pw[0], pw[1], pw[2], pw[3]});
        lsum += psum;

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
        // 16 + qg*4 + (e - 4): exactly the keys this lane already holds.  A
        // transposing read gives lane hl of group qg the 4 consecutive keys
        // k0..k0+3 of column c0 + hl when lane j supplies row k0 + j/4,
        // columns c0 + 4*(j%4) .. +3.
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const uint16_t *src = vs + (qg * 4 + (hl >> 2)) * LDV + db * 16 + 4 * (hl & 3);
            const s16x4 lo4 = ds_read_tr_d(src);
            const s16x4 hi4 = ds_read_tr_d(src + 16 * LDV);
            const bf16x8 va = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
            oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, oacc[db], 0, 0, 0);
        }
    };

    // Two register sets take alternate tiles, so no register copy (which
    // would wait for the loads in flight) sits between tiles.
    bf16x8 ka0[2][KS], ka1[2][KS];
    u32x4 vr0[VIT], vr1[VIT];
    // j0 is the same in every lane of a wavefront; saying so keeps it in
    // scalar registers
    int j0 = __builtin_amdgcn_readfirstlane(c_lo + wave * kDecodeTile);
    if (j0 <= c_hi)
        load_tile(j0, ka0, vr0);
    while (j0 <= c_hi) {
        if constexpr (kExt) {
            const TilePtrs p1 = tile_ptrs(j0 + STEP);
            wait_tile(ka0, vr0);
            if (j0 + STEP <= c_hi)
                load_ptrs(p1, ka1, vr1);
        } else {
            wait_tile(ka0, vr0);
            if (j0 + STEP <= c_hi)
                load_tile(j0 + STEP, ka1, vr1);
        }
        compute_tile(j0, ka0, vr0);
        j0 += STEP;
        if (j0 > c_hi)
            break;
        if constexpr (kExt) {
            const TilePtrs p0 = tile_ptrs(j0 + STEP);
            wait_tile(ka1, vr1);
            if (j0 + STEP <= c_hi)
                load_ptrs(p0, ka0, vr0);
        } else {
            wait_tile(ka1, vr1);
            if (j0 + STEP <= c_hi)
                load_tile(j0 + STEP, ka0, vr0);
        }
        compute_tile(j0, ka1, vr1);
        j0 += STEP;
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

    // Merge the 4 wavefronts of the workgroup.  Each wavefront weights its
    // partial by 2^(m_w - max m) / sum_w' 2^(m_w' - max m) l_w', so that the
    // workgroup's normalised result is the plain sum of the 4 weighted
    // partials; only the group's nh real heads are staged.
    if (qg == 0) {
        sm_m[wave][hl] = m;
        sm_l[wave][hl] = lsum;
    }
    __syncthreads(); // also ends every wavefront's use of the V tiles
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w)
        mx = fmaxf(mx, sm_m[w][hl]);
    float tot = 0.f; // > 0: wavefront 0 folded at least key c_lo
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w)
        tot += fast_exp2(sm_m[w][hl] - mx) * sm_l[w][hl];
    const float my_w = fast_exp2(m - mx) / tot; // 0 for a wavefront that folded no key
    if (wave == 0 && qg == 0)
        sm_lse[hl] = mx + __builtin_amdgcn_logf(tot); // log2-sum-exp of the chunk
    float *os = reinterpret_cast<float *>(smem);
    if (hl < nh) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
            *reinterpret_cast<float4 *>(os + (wave * kDecodeHeads + hl) * LDO + db * 16 + qg * 4) =
                make_float4(oacc[db][0] * my_w, oacc[db][1] * my_w, oacc[db][2] * my_w,
                            oacc[db][3] * my_w);
    }
    __syncthreads();

    int rec_cnt = 0, rec_lo = INT_MAX, rec_hi = -1, rec_xor = 0;
    if (kRecord) {
#pragma unroll
        for (int w = 0; w < kDecodeWaves; ++w) {
            rec_cnt += sm_rec[w][0];
            rec_lo = min(rec_lo, sm_rec[w][1]);
            rec_hi = max(rec_hi, sm_rec[w][2]);
            rec_xor ^= sm_rec[w][3];
        }
    }

    // 4 output features per work-item.
    for (int idx = tid; idx < nh * (D / 4); idx += 256) {
        const int h = idx / (D / 4);
        const int c = (idx % (D / 4)) * 4;
        float4 o = *reinterpret_cast<const float4 *>(os + h * LDO + c);
#pragma unroll
        for (int w = 1; w < kDecodeWaves; ++w) {
            const float4 t = *reinterpret_cast<const float4 *>(os + (w * kDecodeHeads + h) * LDO + c);
            o.x += t.x;
            o.y += t.y;
            o.z += t.z;
            o.w += t.w;
        }
        if (ns == 1) {
            // the whole row was this chunk: finished
            uint2 pk;
            pk.x = pack_bf16x2(o.x, o.y);
            pk.y = pack_bf16x2(o.z, o.w);
            *reinterpret_cast<uint2 *>(a.out + (row0 + h) * D + c) = pk;
        } else {
            *reinterpret_cast<float4 *>(a.o_part + ((row0 + h) * a.nsplit + split) * D + c) = o;
            if (c == 0)
                a.lse_part[(row0 + h) * a.nsplit + split] = sm_lse[h];
        }
    }
    if (kRecord && tid < nh) {
        if (ns == 1) {
            int32_t *rec = a.records + (row0 + tid) * 5;
            rec[0] = g; rec[1] = rec_lo; rec[2] = rec_hi; rec[3] = rec_cnt; rec[4] = rec_xor;
        } else {
            int32_t *rp = a.rec_part + ((row0 + tid) * a.nsplit + split) * 4;
            rp[0] = rec_cnt; rp[1] = rec_lo; rp[2] = rec_hi; rp[3] = rec_xor;
        }
    }
}

struct MergeArgs {
    const float *o_part;
    const float *lse_part;
    const int32_t *rec_part;
    const int32_t *seqlens;
    uint16_t *out;
    int32_t *records;
    int B, C, Hq, Hkv, nhc, r, window, nsplit, chunk;
};

// Workgroup u merges the rows of unit u (batch row b, KV group g, head chunk
// hc: up to 16 query heads), on the XCD where that unit's splits ran (see
// decode_kernel).  One thread per 4 output features of a row with more than
// one chunk: out = sum_s w_s o_s / sum_s w_s with w_s = 2^(lse_s - max lse).
template <int D> constexpr int merge_threads() { return kDecodeHeads * (D / 4); }

template <int D, bool kRecord>
__global__ __launch_bounds__(merge_threads<D>()) void decode_merge_kernel(MergeArgs a) {
    constexpr int Q4 = D / 4;
    const int unit = static_cast<int>(blockIdx.x);
    const int b = unit / (a.Hkv * a.nhc);
    const int g = (unit / a.nhc) % a.Hkv;
    const int hc = unit % a.nhc;
    const int h0 = g * a.r + hc * kDecodeHeads;
    const int nh = min(kDecodeHeads, a.r - hc * kDecodeHeads);
    const int hl = static_cast<int>(threadIdx.x) / Q4;
    if (hl >= nh)
        return;
    const int64_t row = (int64_t)b * a.Hq + h0 + hl;
    const int c4 = (static_cast<int>(threadIdx.x) % Q4) * 4;
    const float *lse = a.lse_part + row * a.nsplit;
    const float *op = a.o_part + row * a.nsplit * D + c4;
    // Partials are loaded in unrolled chunks of kChunk splits, every load of
    // a chunk in flight together.  The first chunk does not wait for the row
    // length: all nsplit slots of the row are in the workspace, and only the
    // first ns of them (those written by this call) are used.
    constexpr int kChunk = 8;
    float lc[kChunk];
    float4 oc[kChunk];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
        if (i < a.nsplit) {
            lc[i] = lse[i];
            oc[i] = *reinterpret_cast<const float4 *>(op + (int64_t)i * D);
        }
    }
    const int nb = a.seqlens ? a.seqlens[b] : a.C;
    if (nb <= 0)
        return; // written by the split kernel
    const int hi = nb - 1;
    const int lo = window_lo(hi, a.window);
    const int ns = (hi - lo) / a.chunk + 1;
    if (ns == 1)
        return; // finished by the split kernel
    // One pass with a running maximum.  Every chunk of a row with ns > 1
    // folded at least one key, so each lse_s is finite.
    float mx = -INFINITY;
    float den = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = 0; s0 < ns; s0 += kChunk) {
        if (s0 > 0) {
#pragma unroll
            for (int i = 0; i < kChunk; ++i) {
                if (s0 + i < ns) {
                    lc[i] = lse[s0 + i];
                    oc[i] = *reinterpret_cast<const float4 *>(op + (int64_t)(s0 + i) * D);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < kChunk; ++i) {
            if (s0 + i < ns) {
                const float l = lc[i];
                const float4 o = oc[i];
                const float mn = fmaxf(mx, l);
                const float sc = fast_exp2(mx - mn); // 0 on the first chunk (mx = -inf)
                const float w = fast_exp2(l - mn);
                den = fmaf(den, sc, w);
                acc.x = fmaf(acc.x, sc, w * o.x);
                acc.y = fmaf(acc.y, sc, w * o.y);
                acc.z = fmaf(acc.z, sc, w * o.z);
                acc.w = fmaf(acc.w, sc, w * o.w);
                mx = mn;
            }
        }
    }
    const float inv = 1.f / den;
    uint2 pk;
    pk.x = pack_bf16x2(acc.x * inv, acc.y * inv);
    pk.y = pack_bf16x2(acc.z * inv, acc.w * inv);
    *reinterpret_cast<uint2 *>(a.out + row * D + c4) = pk;
    if (kRecord && c4 == 0) {
        // record partials: 16 bytes per split, kChunk splits in flight together
        int cnt = 0, x = 0, rl = INT_MAX, rh = -1;
        const int4 *rp = reinterpret_cast<const int4 *>(a.rec_part) + row * a.nsplit;
        for (int s0 = 0; s0 < ns; s0 += kChunk) {
            int4 rc[kChunk];
#pragma unroll
            for (int i = 0; i < kChunk; ++i)
                if (s0 + i < ns)
                    rc[i] = rp[s0 + i];
#pragma unroll
            for (int i = 0; i < kChunk; ++i) {
                if (s0 + i < ns) {
                    cnt += rc[i].x;
                    rl = min(rl, rc[i].y);
                    rh = max(rh, rc[i].z);
                    x ^= rc[i].w;
                }
            }
        }
        int32_t *rec = a.records + row * 5;
        rec[0] = static_cast<int>(row % a.Hq) / a.r;
        rec[1] = rl; rec[2] = rh; rec[3] = cnt; rec[4] = x;
    }
}

// The split workspace of gqa_decode_no_alloc, for callers that cannot
// allocate.  Every GPU holds its own copy until the process ends; its
// contents on entry never matter (each call writes the partials it reads).
// In host code `scratch` names a host-side stand-in, not device memory: the
// kernels are only ever given the address hipGetSymbolAddress returns.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

constexpr int kMaxDevices = 64;

hipError_t decode_scratch(hipStream_t stream, void **ptr) {
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess)
            return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
            return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess)
                e = e2;
        }
        if (e != hipSuccess)
            return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

static size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

DecodePlan plan_decode(int B, int C, int Hq, int Hkv, int d, int window) {
    DecodePlan p{};
    const int elig = (window > 0 && window < C) ? window : C;
    const int r = Hq / Hkv;
    p.nhc = (r + kDecodeHeads - 1) / kDecodeHeads;
    // Number of splits ns.  The launch runs ceil(units * ns / 256) rounds of
    // one 4-wavefront workgroup per CU (256 CUs), each round 1/ns of a row's
    // range, so its time goes as rounds(ns) / ns: pick the ns that minimises
    // it, ties to fewer splits (less to merge).  At most two workgroups per
    // CU in all: with one tile in flight per wavefront, one workgroup per CU
    // holds ~16 MiB of reads in flight over the chip, where a streaming read
    // peaks, and more is slower.  Chunks hold at least one tile per wavefront
    // and split the range evenly: a round lasts as long as its longest chunk.
    const int64_t units = (int64_t)B * Hkv * p.nhc;
    const int64_t cus = kDecodeCUs;
    const int64_t step = (int64_t)kDecodeWaves * kDecodeTile;
    const int64_t max_ns = std::max<int64_t>(
        1, std::min<int64_t>((elig + step - 1) / step, units > 0 ? 2 * cus / units : 1));
    int64_t ns = 1, ns_rounds = units > 0 ? (units + cus - 1) / cus : 1;
    for (int64_t c = 2; c <= max_ns; ++c) {
        const int64_t rounds = (units * c + cus - 1) / cus;
        if (rounds * ns < ns_rounds * c) { // rounds / c < ns_rounds / ns
            ns = c;
            ns_rounds = rounds;
        }
    }
    p.chunk = static_cast<int>(std::max<int64_t>(step, (elig + ns - 1) / ns));
    p.nsplit = elig > 0 ? (elig + p.chunk - 1) / p.chunk : 0;
    const size_t rows = (size_t)B * Hq * (size_t)p.nsplit;
    p.o_off = 0;
    p.lse_off = p.o_off + align256(rows * d * sizeof(float));
    p.rec_off = p.lse_off + align256(rows * sizeof(float));
    p.bytes = p.rec_off + align256(rows * 4 * sizeof(int32_t));
    return p;
}

// The split kernel's grid is one-dimensional: units rounded up to groups of
// 8, times the splits, workgroups of 256 work-items; the merge kernel's is
// one workgroup of up to 512 work-items per unit.  Both totals must fit a
// 32-bit count.
bool decode_grid_ok(int B, int Hkv, const DecodePlan &plan) {
    const int64_t units = (int64_t)B * Hkv * plan.nhc;
    const int64_t ns = plan.nsplit > 0 ? plan.nsplit : 1;
    const int64_t wgs = (units + 7) / 8 * 8 * ns;
    return units <= INT_MAX && wgs * 256 <= (int64_t)UINT32_MAX &&
           units * merge_threads<128>() <= (int64_t)UINT32_MAX;
}

template <int D, bool kRecord, bool kExt>
static hipError_t launch_d(const Problem &p, const DecodePlan &plan, void *ws, hipStream_t s) {
    // no workspace without a split (every row finishes in the split kernel)
    unsigned char *w = static_cast<unsigned char *>(ws);
    DecodeArgs a;
    a.q = static_cast<const uint16_t *>(p.q);
    a.k = static_cast<const uint16_t *>(p.k);
    a.v = static_cast<const uint16_t *>(p.v);
    a.seqlens = p.seqlens;
    a.out = static_cast<uint16_t *>(p.out);
    a.records = p.records;
    a.o_part = w ? reinterpret_cast<float *>(w + plan.o_off) : nullptr;
    a.lse_part = w ? reinterpret_cast<float *>(w + plan.lse_off) : nullptr;
    a.rec_part = w ? reinterpret_cast<int32_t *>(w + plan.rec_off) : nullptr;
    a.C = p.C; a.Hq = p.Hq; a.Hkv = p.Hkv; a.window = p.window;
    a.r = p.Hq / p.Hkv; a.nhc = plan.nhc; a.nsplit = plan.nsplit; a.chunk = plan.chunk;
    a.units = p.B * p.Hkv * plan.nhc;
    a.scale_log2 = p.scale * kLog2e;
    a.knew = static_cast<const uint16_t *>(p.knew);
    a.vnew = static_cast<const uint16_t *>(p.vnew);
    a.kw = static_cast<uint16_t *>(p.kw);
    a.vw = static_cast<uint16_t *>(p.vw);
    a.ring = p.ring ? 1 : 0;
    // at least one split so that empty rows still get their zero output;
    // units in whole groups of 8 (one per XCD)
    const int64_t ns_grid = plan.nsplit > 0 ? plan.nsplit : 1;
    const int64_t wgs = ((int64_t)a.units + 7) / 8 * 8 * ns_grid;
    decode_kernel<D, kRecord, kExt><<<dim3((unsigned)wgs), 256, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || plan.nsplit <= 1)
        return e; // every row finished inside the split kernel
    MergeArgs m;
    m.o_part = a.o_part; m.lse_part = a.lse_part; m.rec_part = a.rec_part;
    m.seqlens = p.seqlens; m.out = a.out; m.records = p.records;
    m.B = p.B; m.C = p.C; m.Hq = p.Hq; m.Hkv = p.Hkv; m.nhc = plan.nhc; m.r = a.r;
    m.window = p.window; m.nsplit = plan.nsplit; m.chunk = plan.chunk;
    decode_merge_kernel<D, kRecord><<<dim3((unsigned)a.units), merge_threads<D>(), 0, s>>>(m);
    return hipGetLastError();
}

hipError_t launch_decode_split(const Problem &p, const DecodePlan &plan, void *workspace,
                               hipStream_t stream) {
    const bool rec = p.records != nullptr;
    const bool ext = p.ring || p.knew != nullptr;
    if (p.d == 128) {
        if (ext)
            return rec ? launch_d<128, true, true>(p, plan, workspace, stream)
                       : launch_d<128, false, true>(p, plan, workspace, stream);
        return rec ? launch_d<128, true, false>(p, plan, workspace, stream)
                   : launch_d<128, false, false>(p, plan, workspace, stream);
    }
    if (ext)
        return rec ? launch_d<64, true, true>(p, plan, workspace, stream)
                   : launch_d<64, false, true>(p, plan, workspace, stream);
    return rec ? launch_d<64, true, false>(p, plan, workspace, stream)
               : launch_d<64, false, false>(p, plan, workspace, stream);
}

} // namespace gqa
