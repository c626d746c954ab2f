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
    const int32_t *seqlens; // nullable: n_b = T (prefill), C (decode, prefix queries)
    int32_t *records;       // nullable: index-set records
    int B, T, C, Hq, Hkv, d, window;
    float scale;
    int dtype; // 0 fp32, 1 bf16
    bool decode;
    // Prefill against a cached prefix: query row i of the t_b new ones sits
    // at cell s_b - t_b + i (s_b = seqlens, default C; t_b = qlens, default
    // T) and its keys start no earlier than segs[b][i] (default 0).  When
    // prefix is false, t_b = s_b = n_b and every row i sits at cell i.
    bool prefix = false;
    const int32_t *qlens = nullptr;
    const int32_t *segs = nullptr;
    // Decode: the candidate's key/value [B,Hkv,d] (both or neither) are read
    // for cell n_b - 1 and committed to its slot of kw/vw (the same caches
    // as k/v); ring stores cell j in slot j mod C.
    const void *knew = nullptr;
    const void *vnew = nullptr;
    void *kw = nullptr;
    void *vw = nullptr;
    bool ring = false;
};

// Split-K decode plan: the eligible key range of a row is cut into chunks of
// `chunk` keys starting at the row's window start; each chunk is one
// workgroup of 4 wavefronts, each wavefront taking 32-key tiles (the last tile
// of a chunk may be partial: chunks are sized to split the range evenly).
// Workspace layout: partial outputs [B, Hq, nsplit, d] fp32, their
// log2-sum-exp values [B, Hq, nsplit] fp32 and index-set partials
// [B, Hq, nsplit, 4] int32 (each region 256-byte aligned).
struct DecodePlan {
    int chunk;    // keys per workgroup, at least 128
    int nsplit;   // chunks per row at the longest eligible range
    int nhc;      // head chunks of up to 16 query heads per KV group
    size_t o_off, lse_off, rec_off, bytes;
};

constexpr int kDecodeTile = 32;
constexpr int kDecodeWaves = 4;
constexpr int kDecodeHeads = 16;
constexpr int kDecodeCUs = 256; // compute units of the MI355X the decode plan targets

DecodePlan plan_decode(int B, int C, int Hq, int Hkv, int d, int window);
bool decode_grid_ok(int B, int Hkv, const DecodePlan &plan);

// Library-owned split workspace of the no-allocation decode entry point: a
// file-scope device array of this many bytes on each GPU the library runs on.
// The split plan keeps at most two workgroups of at most 16 heads per CU, so
// a call's partials hold at most 16 * 512 rows of (d + 5) * 4 bytes: 4.4 MB
// at d = 128.
constexpr size_t kDecodeScratchBytes = size_t{8} << 20;
// Device address of that array on the GPU of `stream` (looked up once per
// device, with that device current).
hipError_t decode_scratch(hipStream_t stream, void **ptr);

hipError_t launch_generic(const Problem &p, hipStream_t stream);
hipError_t launch_decode_split(const Problem &p, const DecodePlan &plan, void *workspace,
                               hipStream_t stream);
// Key-range split of the MFMA prefill for queries against a cached prefix:
// nsplit parts of tps tiles; workspace layout: normalised partial outputs
// [nsplit, B, T, Hq, d] fp32, their log2-sum-exp [nsplit, B, T, Hq] fp32 and
// index-set partials [nsplit, B, T, Hq, 4] int32 (each 256-byte aligned).
// nsplit == 1: no split, no workspace.
struct PrefixPlan {
    int nsplit;
    int tps;
    size_t o_off, lse_off, rec_off, bytes;
};
PrefixPlan plan_prefix(int B, int T, int C, int Hq, int Hkv, int d, int window);

hipError_t launch_prefill_mfma(const Problem &p, const PrefixPlan &plan, void *workspace,
                               hipStream_t stream);
bool prefill_grid_ok(int B, int T, int Hq, int Hkv, int nsplit, int nw);
int prefill_waves(bool segmented);

} // namespace gqa
