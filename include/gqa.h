/*
 * gqa.h -- C interface of libgqa: grouped-query attention over a KV cache on
 * AMD Instinct MI355X (gfx950), for single-token decode and causal prefill,
 * with an optional local window that includes the current cell.
 *
 * What is computed ("Share key/value heads and make context explicit",
 * sections "Give each query head an explicit shared KV head" and "Intersect
 * the window with the context already permitted"):
 *
 *   r = Hq / Hkv; query head h reads KV head g(h) = floor(h / r).
 *   An active query at cell t of batch row b (t < n_b) may read the key cells
 *   l..t, where l = 0 without a window and l = max(0, t - (w - 1)) with a
 *   window of w >= 1 cells (the current cell plus at most w - 1 earlier ones).
 *   s_j = scale * <q_{h,t}, k_{g(h),j}>, p = softmax of s over l..t only
 *   (every other cell has probability exactly 0), z_{h,t} = sum_j p_j v_{g,j}.
 *   The output row of cell t concatenates z_{0,t} .. z_{Hq-1,t} in head order.
 *   Inactive (padded) queries, t >= n_b, produce a zero row.
 *
 * Conventions shared by every entry point:
 *   - Pointers named q, k_cache, v_cache, out, seqlens, workspace and records
 *     are DEVICE pointers owned by the caller; the library never allocates,
 *     frees or keeps them.  All arrays are dense and contiguous with the last
 *     axis (d) innermost.
 *   - dtype selects the element type of q, k_cache, v_cache and out together:
 *     GQA_F32 (IEEE binary32) or GQA_BF16 (bfloat16).  Arithmetic is fp32
 *     throughout; bf16 outputs are rounded to nearest even.
 *   - window < 0 means no local window; window == 0 is refused
 *     (GQA_ERR_ZERO_WINDOW); window >= 1 is the window length in cells.
 *   - scale multiplies the dot products; pass 1/sqrt(d) for the usual scaled
 *     dot product.  It must be finite.
 *   - stream is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls only enqueue work on it and return; they never synchronise.
 *   - Alignment: every array to its element size; the workspace to 256
 *     bytes.  bf16 calls with d = 64 or 128 run the matrix-core kernels,
 *     which need q, k_cache, v_cache, out (and k_new, v_new) 16-byte
 *     aligned; such a call with any of them misaligned is refused with
 *     GQA_ERR_ALIGN (it is never rerouted to another kernel).
 *   - C (cache cells) is at most GQA_MAX_CELLS = 2^30 for every entry point
 *     (else GQA_ERR_SHAPE): the kernels count cells in 32-bit integers.
 *   - Every argument check happens on the host before anything is enqueued;
 *     on any error nothing is launched and out is left untouched (a failed
 *     call never half-advances anything, as the pages require of the cache).
 *   - Preconditions that live in device memory are NOT checked (checking would
 *     need a synchronisation): 0 <= seqlens[b] <= T for prefill and
 *     0 <= seqlens[b] <= C for decode (see each entry point for the rest).
 *   - Calls are thread-safe; the library holds no mutable state (except the
 *     device array of gqa_decode_no_alloc, see there).
 */
#ifndef GQA_H
#define GQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Largest cache length C (cells) any entry point accepts. */
#define GQA_MAX_CELLS ((int32_t)1 << 30)

typedef enum {
    GQA_OK = 0,
    GQA_ERR_NULL = 1,        /* a required pointer is NULL                         */
    GQA_ERR_HEADS = 2,       /* Hq <= 0, Hkv <= 0 or Hq % Hkv != 0                 */
    GQA_ERR_ZERO_WINDOW = 3, /* window == 0                                        */
    GQA_ERR_HEAD_DIM = 4,    /* d < 1 or d > 256                                   */
    GQA_ERR_DTYPE = 5,       /* dtype is not GQA_F32 or GQA_BF16                   */
    GQA_ERR_SHAPE = 6,       /* negative B/T/C, T > C, C > GQA_MAX_CELLS, or a
                                grid limit exceeded                                */
    GQA_ERR_OVERFLOW = 7,    /* an element count or byte size overflows int64      */
    GQA_ERR_WORKSPACE = 8,   /* workspace smaller than gqa_decode_workspace_bytes  */
    GQA_ERR_ALIGN = 9,       /* a pointer is misaligned: to its element size, or to
                                16 bytes for a matrix-core shape (bf16, d 64/128)  */
    GQA_ERR_HIP = 10,        /* the HIP runtime reported an error at launch        */
    GQA_ERR_SCALE = 11       /* scale is NaN or infinite                           */
} gqa_status;

typedef enum { GQA_F32 = 0, GQA_BF16 = 1 } gqa_dtype;

#define GQA_NO_WINDOW (-1)
#define GQA_MAX_HEAD_DIM 256

/* Which kernel family a call would run (for tests and reports). */
typedef enum {
    GQA_KERNEL_NONE = 0,       /* nothing to launch (empty batch or no rows)      */
    GQA_KERNEL_GENERIC = 1,    /* one wavefront per row and KV group, fp32 or bf16 */
    GQA_KERNEL_DECODE_SPLIT = 2, /* bf16 MFMA split-K decode + LSE merge kernel      */
    GQA_KERNEL_PREFILL_MFMA = 3  /* bf16 MFMA flash prefill                         */
} gqa_kernel;

/*
 * Causal prefill.  "Share key/value heads and make context explicit",
 * "Intersect the window with the context already permitted" (active lengths,
 * window rule) and "Give each query head an explicit shared KV head" (scores,
 * permitted-set softmax, value mix, merged heads).
 *
 *   q        [B, Hq, T, d]   queries of cells 0..T-1 (already rotated)
 *   k_cache  [B, Hkv, C, d]  keys; cells 0..n_b-1 are read
 *   v_cache  [B, Hkv, C, d]  values
 *   out      [B, T, Hq, d]   = merged rows [B, T, Hq*d]; rows t >= n_b are 0
 *   seqlens  [B] int32 active lengths n_b (0 <= n_b <= T), or NULL for n_b = T
 *   Requires 0 <= T <= C.  B == 0 or T == 0 is a no-op returning GQA_OK.
 */
int gqa_prefill(const void *q, const void *k_cache, const void *v_cache, void *out,
                const int32_t *seqlens, int32_t B, int32_t T, int32_t C, int32_t Hq,
                int32_t Hkv, int32_t d, int32_t window, float scale, int32_t dtype,
                void *stream);

/*
 * Workspace size in bytes that gqa_decode needs for these arguments (0 when
 * the chosen kernel needs none).  Depends only on the arguments.  Returns 0
 * for arguments gqa_decode would refuse.
 */
size_t gqa_decode_workspace_bytes(int32_t B, int32_t C, int32_t Hq, int32_t Hkv, int32_t d,
                                  int32_t window, int32_t dtype);

/*
 * Single-token decode against a cached prefix.  "Share key/value heads and
 * make context explicit", "Extend the existing full and cached attention
 * paths" (the new query reads every permitted earlier key plus its own
 * candidate key) and "GQA, FlashAttention and the KV cache", "The important
 * mask bug with a cache" (the one new query sees all previous keys).
 *
 *   q        [B, Hq, d]      the new token's queries
 *   k_cache  [B, Hkv, C, d]  keys; the caller has already written the new
 *                            token's key and value at cell n_b - 1
 *   v_cache  [B, Hkv, C, d]
 *   out      [B, Hq, d]      = merged row [B, Hq*d]
 *   seqlens  [B] int32 n_b = cells in use including the new one
 *            (0 <= n_b <= C; n_b == 0 gives a zero row), or NULL for n_b = C
 *   The query sits at cell n_b - 1 and reads cells max(0, n_b - w)..n_b - 1
 *   (all n_b cells without a window).
 *   workspace: device scratch of at least gqa_decode_workspace_bytes(...)
 *   bytes, 256-byte aligned (may be NULL when that size is 0).  Its contents
 *   on entry do not matter.  Calls that may overlap in time must not share
 *   one workspace.
 *   B == 0 is a no-op returning GQA_OK.
 */
int gqa_decode(const void *q, const void *k_cache, const void *v_cache, void *out,
               const int32_t *seqlens, int32_t B, int32_t C, int32_t Hq, int32_t Hkv,
               int32_t d, int32_t window, float scale, int32_t dtype, void *workspace,
               size_t workspace_bytes, void *stream);

/*
 * Decode that allocates nothing and takes no workspace: for callers that
 * cannot allocate device memory at call time (work being captured into a HIP
 * graph, tight serving loops, harnesses that forbid hipMalloc).  It runs the
 * kernels of gqa_decode with their split partials kept in a library-owned
 * device array of GQA_DECODE_SCRATCH_BYTES, one per GPU the library runs on
 * (set up on the first call on that GPU, held until the process ends).
 * Arguments, results and refusals are those of gqa_decode; a split plan whose
 * partials would not fit the array is refused with GQA_ERR_WORKSPACE (the
 * plans of every decode shape need at most about 4.4 MB).  All calls on one GPU
 * share its array, which keeps the last call's contents (no call depends on
 * them): calls that may overlap in time on one GPU -- other streams or other
 * host threads -- race, and the caller must serialise them.
 */
#define GQA_DECODE_SCRATCH_BYTES ((size_t)8 << 20)
int gqa_decode_no_alloc(const void *q, const void *k_cache, const void *v_cache, void *out,
                        const int32_t *seqlens, int32_t B, int32_t C, int32_t Hq, int32_t Hkv,
                        int32_t d, int32_t window, float scale, int32_t dtype, void *stream);

/*
 * Index-set records: the same kernels, instantiated to also write, for every
 * output row, five int32 values {KV head read, lowest key folded in, highest
 * key folded in, number of keys folded in, XOR of the folded key indices}
 * counted at the point of accumulation ({g, -1, -1, 0, 0} for an inactive
 * row).  records is [B, T, Hq, 5] for prefill and [B, Hq, 5] for decode.
 * Everything else is as for gqa_prefill / gqa_decode, and out is written too.
 */
int gqa_prefill_records(const void *q, const void *k_cache, const void *v_cache, void *out,
                        const int32_t *seqlens, int32_t B, int32_t T, int32_t C, int32_t Hq,
                        int32_t Hkv, int32_t d, int32_t window, float scale, int32_t dtype,
                        int32_t *records, void *stream);
int gqa_decode_records(const void *q, const void *k_cache, const void *v_cache, void *out,
                       const int32_t *seqlens, int32_t B, int32_t C, int32_t Hq, int32_t Hkv,
                       int32_t d, int32_t window, float scale, int32_t dtype, void *workspace,
                       size_t workspace_bytes, int32_t *records, void *stream);

/*
 * Queries against a cached prefix: chunked prefill, or checking several new
 * tokens at once, with optional packed segments.
 * "How do you implement grouped query attention (GQA)?", section "Worked
 * example" (query i of the t new ones sits at absolute position s - t + i and
 * sees the keys up to it) and "GQA, FlashAttention and the KV cache",
 * "The important mask bug with a cache" (several new tokens need that
 * offset); "Share key/value heads and make context explicit", "Intersect the
 * window with the context already permitted" (segment starts, intersected
 * with the window).
 *
 *   q          [B, Hq, Tq, d]  the new queries (rows past t_b are padding)
 *   k_cache    [B, Hkv, C, d]  keys; the caller has already written the new
 *                              cells, so cells 0..s_b-1 hold the sequence
 *   v_cache    [B, Hkv, C, d]
 *   out        [B, Tq, Hq, d]  = merged rows; inactive rows are 0
 *   seqlens    [B] int32 s_b = cells in the cache including the new ones
 *              (0 <= s_b <= C), or NULL for s_b = C
 *   qlens      [B] int32 t_b = new query rows (0 <= t_b <= Tq), or NULL for
 *              t_b = Tq
 *   seg_starts [B, Tq] int32: the first cell of each query row's segment
 *              (packed unrelated examples), or NULL for 0
 *   workspace  device scratch of at least gqa_prefill_prefix_workspace_bytes(...)
 *              bytes, 256-byte aligned (may be NULL when that size is 0).  When
 *              the blocks of new rows alone cannot fill the GPU, their key
 *              ranges are split over several workgroups whose partial results
 *              go here and are merged by a second kernel.  Contents on entry
 *              do not matter; calls that may overlap must not share it.
 *   records    NULL, or [B, Tq, Hq, 5] index-set records as for
 *              gqa_prefill_records
 *   Query row i < t_b sits at cell p = s_b - t_b + i and reads cells lo..p,
 *   lo = max(seg, p - (w - 1), 0) with a window, lo = seg without.  A row is
 *   inactive (zero output) when i >= t_b, when p < 0, or when its segment
 *   starts after it (seg > p).  With qlens == seqlens and no segments this is
 *   gqa_prefill with cache capacity C; with Tq = 1 it is the decode query.
 *   Requires 0 <= Tq <= C.  B == 0 or Tq == 0 is a no-op returning GQA_OK.
 *   Device-side preconditions (not checked): the bounds above on s_b, t_b.
 */
size_t gqa_prefill_prefix_workspace_bytes(int32_t B, int32_t Tq, int32_t C, int32_t Hq,
                                          int32_t Hkv, int32_t d, int32_t window,
                                          int32_t dtype);
int gqa_prefill_prefix(const void *q, const void *k_cache, const void *v_cache, void *out,
                       const int32_t *seqlens, const int32_t *qlens, const int32_t *seg_starts,
                       int32_t B, int32_t Tq, int32_t C, int32_t Hq, int32_t Hkv, int32_t d,
                       int32_t window, float scale, int32_t dtype, void *workspace,
                       size_t workspace_bytes, int32_t *records, void *stream);

/*
 * Decode with the new token's key and value committed in the same call,
 * and/or over a rolling cache.
 * "Extend the existing full and cached attention paths": the incremental
 * step reads the candidate key and value at the new position from their own
 * buffers and commits them to the cache as part of the step.  "Share
 * key/value heads and make context explicit", the paragraph on the Mistral 7B
 * report: a rolling buffer that overwrites the oldest entries; with a window
 * of w cells a buffer of capacity C >= w holds every key the query reads,
 * cell j in slot j mod C.
 *
 *   q        [B, Hq, d]       the new token's queries
 *   k_cache  [B, Hkv, C, d]   keys (written: the candidate's slot)
 *   v_cache  [B, Hkv, C, d]   values (written likewise)
 *   k_new    [B, Hkv, d]      the candidate's key, or NULL (then v_new must
 *   v_new    [B, Hkv, d]      be NULL too and the cache already holds cell
 *                             n_b - 1)
 *   out      [B, Hq, d]
 *   seqlens  [B] int32 n_b = cells of the sequence including the new one, or
 *            NULL for n_b = C.  ring == 0: 0 <= n_b <= C, cell j in slot j.
 *            ring == 1: any n_b >= 0, cell j in slot j mod C; requires
 *            1 <= window <= C (else GQA_ERR_SHAPE).
 *   ring     0 or 1 (anything else: GQA_ERR_SHAPE)
 *   workspace, workspace_bytes: as for gqa_decode, sized by
 *            gqa_decode_workspace_bytes(B, C, Hq, Hkv, d, window, dtype)
 *   records  NULL, or [B, Hq, 5] records as for gqa_decode_records (key
 *            cells, not slots)
 *   The query sits at cell n_b - 1 and reads cells max(0, n_b - w)..n_b - 1,
 *   taking cell n_b - 1 from k_new/v_new when they are given; those are also
 *   copied, bit for bit, into the slot of cell n_b - 1 (n_b == 0 commits
 *   nothing).  No other cache element changes.  k_new/v_new must not
 *   overlap the caches.
 */
int gqa_decode_cache(const void *q, void *k_cache, void *v_cache, const void *k_new,
                     const void *v_new, void *out, const int32_t *seqlens, int32_t B, int32_t C,
                     int32_t Hq, int32_t Hkv, int32_t d, int32_t window, float scale,
                     int32_t dtype, int32_t ring, void *workspace, size_t workspace_bytes,
                     int32_t *records, void *stream);

/* The kernel family gqa_prefill / gqa_decode would launch for these arguments
 * (GQA_KERNEL_NONE for a no-op or a refused call).  It depends on the
 * arguments only: a call whose pointers do not meet that kernel's alignment
 * is refused with GQA_ERR_ALIGN, so no other kernel ever runs in its place. */
int gqa_prefill_kernel(int32_t B, int32_t T, int32_t C, int32_t Hq, int32_t Hkv, int32_t d,
                       int32_t window, int32_t dtype);
int gqa_decode_kernel(int32_t B, int32_t C, int32_t Hq, int32_t Hkv, int32_t d, int32_t window,
                      int32_t dtype);

/*
 * Host helpers (no device work).
 *
 * gqa_kv_head_for_query: floor(h / (Hq / Hkv)), or -1 when Hkv <= 0, Hq <= 0,
 *   Hq % Hkv != 0 or h is outside 0..Hq-1 (kv_head_for_query in "Extend the
 *   existing full and cached attention paths").
 * gqa_window_start: max(s, t - (w - 1)) with the subtraction saturating at 0,
 *   or -1 when w == 0, s > t or an argument is negative (causal_window_start,
 *   same section).
 * gqa_kv_cache_bytes: 2 * L * B * T * Hkv * d * e, the K plus V payload of a
 *   cache ("GQA, FlashAttention and the KV cache", "Computing the cache
 *   requirement"); returns GQA_OK and writes *bytes, GQA_ERR_OVERFLOW if the
 *   product does not fit in 64 bits, GQA_ERR_NULL if bytes is NULL.
 * gqa_status_string: a static message for a status code.
 */
int32_t gqa_kv_head_for_query(int32_t h, int32_t Hq, int32_t Hkv);
int64_t gqa_window_start(int64_t t, int64_t seg_start, int64_t w);
int gqa_kv_cache_bytes(uint64_t L, uint64_t B, uint64_t T, uint64_t Hkv, uint64_t d, uint64_t e,
                       uint64_t *bytes);
const char *gqa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* GQA_H */
