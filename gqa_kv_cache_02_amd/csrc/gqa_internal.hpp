// gqa_internal.hpp -- launch descriptions shared by the host entry points and
// the kernel translation units of libgqa.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gqa {

// One call, after validation.  Decode uses T = 1 and reads the query at cell
// n_b - 1; prefill reads query t of cell t.
struct Problem {
    const void *q;
    const void *k;
    const void *v;
    void *out;
    const int32_t *seqlens; // nullable: n_b = T (prefill) or C (decode)
    int32_t *records;       // nullable: index-set records
    int B, T, C, Hq, Hkv, d, window;
    float scale;
    int dtype; // 0 fp32, 1 bf16
    bool decode;
};

// Split-K decode plan: the eligible key range of a row is cut into chunks of
// `chunk` keys starting at the row's window start; each chunk is one
// workgroup of 4 wavefronts, each wavefront taking 32-key tiles.
// Workspace layout: partial outputs [B, Hq, nsplit, d] fp32, their
// log2-sum-exp values [B, Hq, nsplit] fp32 and index-set partials
// [B, Hq, nsplit, 4] int32 (each region 256-byte aligned).
struct DecodePlan {
    int tiles_per_wave;
    int chunk;    // keys per workgroup = 4 * 32 * tiles_per_wave
    int nsplit;   // chunks per row at the longest eligible range
    int nhc;      // head chunks of up to 16 query heads per KV group
    size_t o_off, lse_off, rec_off, bytes;
};

constexpr int kDecodeTile = 32;
constexpr int kDecodeWaves = 4;
constexpr int kDecodeHeads = 16;

DecodePlan plan_decode(int B, int C, int Hq, int Hkv, int d, int window);

hipError_t launch_generic(const Problem &p, hipStream_t stream);
hipError_t launch_decode_split(const Problem &p, const DecodePlan &plan, void *workspace,
                               hipStream_t stream);
hipError_t launch_prefill_mfma(const Problem &p, hipStream_t stream);
bool prefill_grid_ok(int B, int T, int Hq, int Hkv);

} // namespace gqa
