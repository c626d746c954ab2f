// gqa_api.cpp -- the C entry points of libgqa: host-side argument checks,
// kernel selection and launches on the caller's stream.  Nothing here
// allocates, frees or synchronises.
//
// Refusals follow the pages: zero window ("Intersect the window with the
// context already permitted": a zero window is refused), head counts that do
// not divide (kv_head_for_query in "Extend the existing full and cached
// attention paths" returns None), sizes that overflow (the pages' checked
// multiplications), and T > C (generation refuses to exceed the cache bound).
// Every check runs before any launch, so a refused call leaves the output
// untouched.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <hip/hip_runtime.h>

#include "gqa.h"
#include "gqa_internal.hpp"

static_assert(gqa::kDecodeScratchBytes == GQA_DECODE_SCRATCH_BYTES,
              "the header states the no-allocation decode's array size");

namespace {

using gqa::Problem;

constexpr int64_t kMaxGridYZ = 65535;

bool mul_ok(int64_t a, int64_t b, int64_t *out) { return !__builtin_mul_overflow(a, b, out); }

int elem_size(int32_t dtype) { return dtype == GQA_F32 ? 4 : 2; }

bool aligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// Scalar checks shared by prefill and decode, in a fixed order.
int check_scalars(int32_t Hq, int32_t Hkv, int32_t d, int32_t window, float scale,
                  int32_t dtype) {
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0)
        return GQA_ERR_HEADS;
    if (window == 0)
        return GQA_ERR_ZERO_WINDOW;
    if (d < 1 || d > GQA_MAX_HEAD_DIM)
        return GQA_ERR_HEAD_DIM;
    if (dtype != GQA_F32 && dtype != GQA_BF16)
        return GQA_ERR_DTYPE;
    if (!isfinite(scale))
        return GQA_ERR_SCALE;
    return GQA_OK;
}

// Element counts of every array must fit in int64 (kernels index with int64).
int check_sizes(int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t C, int64_t d,
                int32_t dtype) {
    // every kernel counts cells in int, with room past C for a tile's reach
    if (C > GQA_MAX_CELLS)
        return GQA_ERR_SHAPE;
    int64_t x;
    const int64_t es = elem_size(dtype);
    if (!mul_ok(B, Hq, &x) || !mul_ok(x, T, &x) || !mul_ok(x, d, &x) || !mul_ok(x, es, &x))
        return GQA_ERR_OVERFLOW;
    if (!mul_ok(B, Hkv, &x) || !mul_ok(x, C, &x) || !mul_ok(x, d, &x) || !mul_ok(x, es, &x))
        return GQA_ERR_OVERFLOW;
    return GQA_OK;
}

// k and v may be NULL only when the cache has no cells (C == 0): nothing is
// read from them then.
int check_pointers(const void *q, const void *k, const void *v, const void *out,
                   const int32_t *seqlens, int32_t dtype, bool need_kv) {
    if (!q || !out || (need_kv && (!k || !v)))
        return GQA_ERR_NULL;
    const uintptr_t es = static_cast<uintptr_t>(elem_size(dtype));
    if (!aligned(q, es) || !aligned(k, es) || !aligned(v, es) || !aligned(out, es))
        return GQA_ERR_ALIGN;
    if (seqlens && !aligned(seqlens, 4))
        return GQA_ERR_ALIGN;
    return GQA_OK;
}

bool fast_shape(int32_t d, int32_t dtype) {
    return dtype == GQA_BF16 && (d == 64 || d == 128);
}

// The matrix-core kernels move 16 bytes per lane: q, k, v and out (and a
// decode candidate) must be 16-byte aligned.  A call of their shape with a
// pointer that is not is refused (GQA_ERR_ALIGN), never rerouted to another
// kernel behind the caller's back.
bool fast_aligned(const void *q, const void *k, const void *v, const void *out) {
    return aligned(q, 16) && aligned(k, 16) && aligned(v, 16) && aligned(out, 16);
}

int prefill_kernel_for(int32_t d, int32_t dtype) {
    return fast_shape(d, dtype) ? GQA_KERNEL_PREFILL_MFMA : GQA_KERNEL_GENERIC;
}

int decode_kernel_for(int32_t d, int32_t dtype) {
    return fast_shape(d, dtype) ? GQA_KERNEL_DECODE_SPLIT : GQA_KERNEL_GENERIC;
}

int status_of(hipError_t e) { return e == hipSuccess ? GQA_OK : GQA_ERR_HIP; }

// Extra inputs of the prefix-query and cache-update forms.
struct PrefixExtra {
    bool prefix = false;
    const int32_t *qlens = nullptr;
    const int32_t *segs = nullptr;
    void *workspace = nullptr; // key-range split partials (prefix form only)
    size_t workspace_bytes = 0;
};
struct CacheExtra {
    const void *knew = nullptr;
    const void *vnew = nullptr;
    void *kw = nullptr;
    void *vw = nullptr;
    bool ring = false;
};

int prefill_impl(const void *q, const void *k, const void *v, void *out, const int32_t *seqlens,
                 int32_t B, int32_t T, int32_t C, int32_t Hq, int32_t Hkv, int32_t d,
                 int32_t window, float scale, int32_t dtype, int32_t *records, bool want_records,
                 void *stream, const PrefixExtra &x = PrefixExtra()) {
    int rc = check_scalars(Hq, Hkv, d, window, scale, dtype);
    if (rc)
        return rc;
    if (B < 0 || T < 0 || C < 0 || T > C)
        return GQA_ERR_SHAPE;
    if ((rc = check_sizes(B, Hq, Hkv, T, C, d, dtype)))
        return rc;
    if (B == 0 || T == 0)
        return GQA_OK;
    if ((rc = check_pointers(q, k, v, out, seqlens, dtype, true)))
        return rc;
    if ((x.qlens && !aligned(x.qlens, 4)) || (x.segs && !aligned(x.segs, 4)))
        return GQA_ERR_ALIGN;
    if (want_records) {
        if (!records)
            return GQA_ERR_NULL;
        if (!aligned(records, 4))
            return GQA_ERR_ALIGN;
    }
    const int r = Hq / Hkv;
    Problem p{q, k, v, out, seqlens, want_records ? records : nullptr,
              B, T, C, Hq, Hkv, d, window, scale, dtype, false};
    p.prefix = x.prefix;
    p.qlens = x.qlens;
    p.segs = x.segs;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (prefill_kernel_for(d, dtype) == GQA_KERNEL_PREFILL_MFMA) {
        if (!fast_aligned(q, k, v, out))
            return GQA_ERR_ALIGN;
        gqa::PrefixPlan plan{};
        plan.nsplit = 1;
        if (x.prefix)
            plan = gqa::plan_prefix(B, T, C, Hq, Hkv, d, window);
        if (!gqa::prefill_grid_ok(B, T, Hq, Hkv, plan.nsplit, gqa::prefill_waves(x.segs != nullptr)))
            return GQA_ERR_SHAPE;
        if (plan.nsplit > 1) {
            if (!x.workspace)
                return GQA_ERR_NULL;
            if (!aligned(x.workspace, 256))
                return GQA_ERR_ALIGN;
            if (x.workspace_bytes < plan.bytes)
                return GQA_ERR_WORKSPACE;
        }
        return status_of(gqa::launch_prefill_mfma(p, plan, x.workspace, s));
    }
    if (B > kMaxGridYZ || (int64_t)Hkv * ((r + 7) / 8) > kMaxGridYZ)
        return GQA_ERR_SHAPE;
    return status_of(gqa::launch_generic(p, s));
}

int decode_impl(const void *q, const void *k, const void *v, void *out, const int32_t *seqlens,
                int32_t B, int32_t C, int32_t Hq, int32_t Hkv, int32_t d, int32_t window,
                float scale, int32_t dtype, void *workspace, size_t workspace_bytes,
                int32_t *records, bool want_records, void *stream,
                const CacheExtra &x = CacheExtra(), bool use_scratch = false) {
    int rc = check_scalars(Hq, Hkv, d, window, scale, dtype);
    if (rc)
        return rc;
    if (B < 0 || C < 0)
        return GQA_ERR_SHAPE;
    // a rolling cache must hold every cell the window reaches
    if (x.ring && (window < 1 || window > C))
        return GQA_ERR_SHAPE;
    if ((rc = check_sizes(B, Hq, Hkv, 1, C, d, dtype)))
        return rc;
    if (B == 0)
        return GQA_OK;
    if ((rc = check_pointers(q, k, v, out, seqlens, dtype, C > 0)))
        return rc;
    if ((x.knew == nullptr) != (x.vnew == nullptr))
        return GQA_ERR_NULL;
    const uintptr_t es = static_cast<uintptr_t>(elem_size(dtype));
    if (x.knew && (!aligned(x.knew, es) || !aligned(x.vnew, es)))
        return GQA_ERR_ALIGN;
    if (want_records) {
        if (!records)
            return GQA_ERR_NULL;
        if (!aligned(records, 4))
            return GQA_ERR_ALIGN;
    }
    Problem p{q, k, v, out, seqlens, want_records ? records : nullptr,
              B, 1, C, Hq, Hkv, d, window, scale, dtype, true};
    p.knew = x.knew;
    p.vnew = x.vnew;
    p.kw = x.kw;
    p.vw = x.vw;
    p.ring = x.ring;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int r = Hq / Hkv;
    if (decode_kernel_for(d, dtype) == GQA_KERNEL_DECODE_SPLIT) {
        const bool cand_aligned = !x.knew || (aligned(x.knew, 16) && aligned(x.vnew, 16));
        if (!fast_aligned(q, k, v, out) || !cand_aligned)
            return GQA_ERR_ALIGN;
        const gqa::DecodePlan plan = gqa::plan_decode(B, C, Hq, Hkv, d, window);
        if (!gqa::decode_grid_ok(B, Hkv, plan))
            return GQA_ERR_SHAPE;
        // the workspace holds split partials only: without a split it is
        // never touched and may be NULL
        if (plan.nsplit > 1 && use_scratch) {
            // the library's own array instead of a caller's workspace
            if (plan.bytes > gqa::kDecodeScratchBytes)
                return GQA_ERR_WORKSPACE;
            if (gqa::decode_scratch(s, &workspace) != hipSuccess)
                return GQA_ERR_HIP;
        } else if (plan.nsplit > 1) {
            if (!workspace)
                return GQA_ERR_NULL;
            if (!aligned(workspace, 256))
                return GQA_ERR_ALIGN;
            if (workspace_bytes < plan.bytes)
                return GQA_ERR_WORKSPACE;
        } else {
            workspace = nullptr;
        }
        return status_of(gqa::launch_decode_split(p, plan, workspace, s));
    }
    if (B > kMaxGridYZ || (int64_t)Hkv * ((r + 7) / 8) > kMaxGridYZ)
        return GQA_ERR_SHAPE;
    return status_of(gqa::launch_generic(p, s));
}

} // namespace

extern "C" {

int gqa_prefill(const void *q, const void *k_cache, const void *v_cache, void *out,
                const int32_t *seqlens, int32_t B, int32_t T, int32_t C, int32_t Hq,
                int32_t Hkv, int32_t d, int32_t window, float scale, int32_t dtype,
                void *stream) {
    return prefill_impl(q, k_cache, v_cache, out, seqlens, B, T, C, Hq, Hkv, d, window, scale,
                        dtype, nullptr, false, stream);
}

int gqa_prefill_records(const void *q, const void *k_cache, const void *v_cache, void *out,
                        const int32_t *seqlens, int32_t B, int32_t T, int32_t C, int32_t Hq,
                        int32_t Hkv, int32_t d, int32_t window, float scale, int32_t dtype,
                        int32_t *records, void *stream) {
    return prefill_impl(q, k_cache, v_cache, out, seqlens, B, T, C, Hq, Hkv, d, window, scale,
                        dtype, records, true, stream);
}

size_t gqa_decode_workspace_bytes(int32_t B, int32_t C, int32_t Hq, int32_t Hkv, int32_t d,
                                  int32_t window, int32_t dtype) {
    if (check_scalars(Hq, Hkv, d, window, 1.0f, dtype) || B < 0 || C < 0 ||
        check_sizes(B, Hq, Hkv, 1, C, d, dtype))
        return 0;
    if (B == 0 || decode_kernel_for(d, dtype) != GQA_KERNEL_DECODE_SPLIT)
        return 0;
    const gqa::DecodePlan plan = gqa::plan_decode(B, C, Hq, Hkv, d, window);
    return plan.nsplit > 1 ? plan.bytes : 0;
}

int gqa_decode(const void *q, const void *k_cache, const void *v_cache, void *out,
               const int32_t *seqlens, int32_t B, int32_t C, int32_t Hq, int32_t Hkv,
               int32_t d, int32_t window, float scale, int32_t dtype, void *workspace,
               size_t workspace_bytes, void *stream) {
    return decode_impl(q, k_cache, v_cache, out, seqlens, B, C, Hq, Hkv, d, window, scale, dtype,
                       workspace, workspace_bytes, nullptr, false, stream);
}

int gqa_decode_no_alloc(const void *q, const void *k_cache, const void *v_cache, void *out,
                        const int32_t *seqlens, int32_t B, int32_t C, int32_t Hq, int32_t Hkv,
                        int32_t d, int32_t window, float scale, int32_t dtype, void *stream) {
    return decode_impl(q, k_cache, v_cache, out, seqlens, B, C, Hq, Hkv, d, window, scale, dtype,
                       nullptr, 0, nullptr, false, stream, CacheExtra(), true);
}

int gqa_decode_records(const void *q, const void *k_cache, const void *v_cache, void *out,
                       const int32_t *seqlens, int32_t B, int32_t C, int32_t Hq, int32_t Hkv,
                       int32_t d, int32_t window, float scale, int32_t dtype, void *workspace,
                       size_t workspace_bytes, int32_t *records, void *stream) {
    return decode_impl(q, k_cache, v_cache, out, seqlens, B, C, Hq, Hkv, d, window, scale, dtype,
                       workspace, workspace_bytes, records, true, stream);
}

size_t gqa_prefill_prefix_workspace_bytes(int32_t B, int32_t Tq, int32_t C, int32_t Hq,
                                          int32_t Hkv, int32_t d, int32_t window,
                                          int32_t dtype) {
    if (check_scalars(Hq, Hkv, d, window, 1.0f, dtype) || B < 0 || Tq < 0 || C < 0 || Tq > C ||
        check_sizes(B, Hq, Hkv, Tq, C, d, dtype))
        return 0;
    if (B == 0 || Tq == 0 || prefill_kernel_for(d, dtype) != GQA_KERNEL_PREFILL_MFMA)
        return 0;
    const gqa::PrefixPlan plan = gqa::plan_prefix(B, Tq, C, Hq, Hkv, d, window);
    return plan.nsplit > 1 ? plan.bytes : 0;
}

int gqa_prefill_prefix(const void *q, const void *k_cache, const void *v_cache, void *out,
                       const int32_t *seqlens, const int32_t *qlens, const int32_t *seg_starts,
                       int32_t B, int32_t Tq, int32_t C, int32_t Hq, int32_t Hkv, int32_t d,
                       int32_t window, float scale, int32_t dtype, void *workspace,
                       size_t workspace_bytes, int32_t *records, void *stream) {
    PrefixExtra x;
    x.prefix = true;
    x.qlens = qlens;
    x.segs = seg_starts;
    x.workspace = workspace;
    x.workspace_bytes = workspace_bytes;
    return prefill_impl(q, k_cache, v_cache, out, seqlens, B, Tq, C, Hq, Hkv, d, window, scale,
                        dtype, records, records != nullptr, stream, x);
}

int gqa_decode_cache(const void *q, void *k_cache, void *v_cache, const void *k_new,
                     const void *v_new, void *out, const int32_t *seqlens, int32_t B, int32_t C,
                     int32_t Hq, int32_t Hkv, int32_t d, int32_t window, float scale,
                     int32_t dtype, int32_t ring, void *workspace, size_t workspace_bytes,
                     int32_t *records, void *stream) {
    if (ring != 0 && ring != 1)
        return GQA_ERR_SHAPE;
    CacheExtra x;
    x.knew = k_new;
    x.vnew = v_new;
    x.kw = k_cache;
    x.vw = v_cache;
    x.ring = ring != 0;
    return decode_impl(q, k_cache, v_cache, out, seqlens, B, C, Hq, Hkv, d, window, scale, dtype,
                       workspace, workspace_bytes, records, records != nullptr, stream, x);
}

int gqa_prefill_kernel(int32_t B, int32_t T, int32_t C, int32_t Hq, int32_t Hkv, int32_t d,
                       int32_t window, int32_t dtype) {
    if (check_scalars(Hq, Hkv, d, window, 1.0f, dtype) || B < 0 || T < 0 || C < 0 || T > C ||
        check_sizes(B, Hq, Hkv, T, C, d, dtype))
        return GQA_KERNEL_NONE;
    if (B == 0 || T == 0)
        return GQA_KERNEL_NONE;
    return prefill_kernel_for(d, dtype);
}

int gqa_decode_kernel(int32_t B, int32_t C, int32_t Hq, int32_t Hkv, int32_t d, int32_t window,
                      int32_t dtype) {
    if (check_scalars(Hq, Hkv, d, window, 1.0f, dtype) || B < 0 || C < 0 ||
        check_sizes(B, Hq, Hkv, 1, C, d, dtype))
        return GQA_KERNEL_NONE;
    if (B == 0)
        return GQA_KERNEL_NONE;
    return decode_kernel_for(d, dtype);
}

int32_t gqa_kv_head_for_query(int32_t h, int32_t Hq, int32_t Hkv) {
    if (Hkv <= 0 || Hq <= 0 || Hq % Hkv != 0 || h < 0 || h >= Hq)
        return -1;
    return h / (Hq / Hkv);
}

int64_t gqa_window_start(int64_t t, int64_t seg_start, int64_t w) {
    if (t < 0 || seg_start < 0 || w <= 0 || seg_start > t)
        return -1;
    const int64_t lo = (t >= w - 1) ? t - (w - 1) : 0;
    return lo > seg_start ? lo : seg_start;
}

int gqa_kv_cache_bytes(uint64_t L, uint64_t B, uint64_t T, uint64_t Hkv, uint64_t d, uint64_t e,
                       uint64_t *bytes) {
    if (!bytes)
        return GQA_ERR_NULL;
    uint64_t acc = 2;
    const uint64_t f[6] = {L, B, T, Hkv, d, e};
    for (int i = 0; i < 6; ++i)
        if (__builtin_mul_overflow(acc, f[i], &acc))
            return GQA_ERR_OVERFLOW;
    *bytes = acc;
    return GQA_OK;
}

const char *gqa_status_string(int status) {
    switch (status) {
    case GQA_OK: return "ok";
    case GQA_ERR_NULL: return "a required pointer is NULL";
    case GQA_ERR_HEADS: return "head counts must be positive with Hq divisible by Hkv";
    case GQA_ERR_ZERO_WINDOW: return "a zero window is refused (window < 0 means none)";
    case GQA_ERR_HEAD_DIM: return "head width d must be in 1..256";
    case GQA_ERR_DTYPE: return "dtype must be GQA_F32 or GQA_BF16";
    case GQA_ERR_SHAPE: return "shape out of range (negative size, T > C, or grid limit)";
    case GQA_ERR_OVERFLOW: return "element count or byte size overflows int64";
    case GQA_ERR_WORKSPACE: return "decode workspace is smaller than gqa_decode_workspace_bytes";
    case GQA_ERR_ALIGN: return "pointer misaligned";
    case GQA_ERR_HIP: return "HIP launch error";
    case GQA_ERR_SCALE: return "scale must be finite";
    default: return "unknown status";
    }
}

} // extern "C"
