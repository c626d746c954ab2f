/*
 * gqa_oracle.c -- plain, slow fp64 reference for grouped-query attention over
 * a KV cache (decode and causal prefill, optional inclusive-self window).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the HIP path is
 * checked against.  Only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark may load it.  It shares no code, header, table or helper
 * with the HIP library, and the product path never calls it.
 *
 * Every value is an IEEE double.  Callers widen their stored inputs (fp32 or
 * bf16 bits) to double exactly before calling, so the oracle sees the same
 * numbers the GPU sees.  Loops run in ascending index order; softmax subtracts
 * the maximum permitted score before exponentiating.
 *
 * Sources (the pages this follows):
 *  [HEADMAP]  "Share key/value heads and make context explicit", section
 *             "Give each query head an explicit shared KV head": r = Hq/Hkv,
 *             query head h reads shared KV head floor(h/r); and the function
 *             kv_head_for_query in "Extend the existing full and cached
 *             attention paths" (None for zero counts, non-divisible counts,
 *             out-of-range heads).
 *  [WINDOW]   same page, "Intersect the window with the context already
 *             permitted": an active query t < n_b reads keys s..t; a window
 *             w >= 1 counts the current cell and at most w-1 earlier cells;
 *             the lower bound is max(s, t saturating-minus (w-1)); w = 0 is
 *             refused; inactive padded queries have zero probabilities and
 *             zero output.  causal_window_start in "Extend the existing full
 *             and cached attention paths" gives None when w = 0 or s > t.
 *  [SOFTMAX]  same page, "Give each query head an explicit shared KV head":
 *             scaled dot product score, softmax over the permitted set only,
 *             excluded cells get probability zero, each query head
 *             normalises on its own, z = sum_j p_j v_j, head results are
 *             concatenated in head order.  Scale 1/sqrt(d) as in the
 *             incremental code of "Extend the existing full and cached
 *             attention paths" and in "How do you implement grouped query
 *             attention (GQA)?", section "Worked example".
 *  [DECODE]   "Extend the existing full and cached attention paths": the
 *             single new query sits at the cache's current length and reads
 *             every permitted earlier key plus its own (candidate) key.
 *  [MASKOFF]  "GQA, FlashAttention and the KV cache", section "The important
 *             mask bug with a cache", and the tril(s - t) offset mask in
 *             "How do you implement grouped query attention (GQA)?",
 *             section "Worked example": query i of t new ones sits at absolute
 *             position s - t + i (bottom-right alignment).
 *  [REPEAT]   "How do you implement grouped query attention (GQA)?", section
 *             "Grouped-query attention from first principles", Step 3:
 *             repeat_interleave along the head axis keeps the copies of one
 *             KV head adjacent; "Trade-offs and edge cases": a tiled repeat
 *             pairs heads with the wrong KV head.
 *  [BYTES]    "GQA, FlashAttention and the KV cache", section "Computing the
 *             cache requirement": M_KV = 2 L B T Hkv d e bytes.
 *  [SEGMENT]  "Share key/value heads and make context explicit", section
 *             "Intersect the window with the context already permitted": the
 *             query's own segment start s_{b,t} bounds its keys from below
 *             and is intersected with the window (six packed cells: at cell 4
 *             the segment starts at 2 and the window at 3; at cell 5 a new
 *             segment starts, leaving only self).
 *  [CANDIDATE] "Extend the existing full and cached attention paths": the
 *             incremental step reads the new (candidate) key and value from
 *             their own buffers at the new position and commits them to the
 *             cache as part of the same step.
 *  [ROLLING]  "Share key/value heads and make context explicit", the
 *             paragraph on the Mistral 7B report: sliding-window attention
 *             over a rolling buffer that overwrites the oldest entries; a
 *             buffer of capacity w holds every key a window of w reaches,
 *             cell j in slot j mod w.
 *
 * Layouts (d innermost, contiguous):
 *   prefill: q [B,Hq,T,d], k and v [B,Hkv,C,d], out [B,T,Hq,d] (the merged
 *            [B,T,Hq*d] row of the concatenated head vectors).
 *   decode:  q [B,Hq,d], k and v [B,Hkv,C,d], out [B,Hq,d]; seqlens n_b
 *            counts the cached cells including the new one, so the query is
 *            at position n_b - 1.
 *   window:  < 0 means no local window, 0 is refused, >= 1 is a window.
 *   records: per output row, five int32 values
 *            {kv head read, lowest key, highest key, key count, xor of keys};
 *            an inactive row records {g, -1, -1, 0, 0}.
 *
 * Return codes: 0 ok, 2 bad head counts, 3 zero window, 6 bad shape.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_ERR_HEADS 2
#define ORACLE_ERR_ZERO_WINDOW 3
#define ORACLE_ERR_SHAPE 6

/* [HEADMAP] floor(h / (Hq/Hkv)), or -1 for None. */
int64_t oracle_kv_head_for_query(int64_t h, int64_t hq, int64_t hkv)
{
    if (hkv <= 0 || hq <= 0 || hq % hkv != 0)
        return -1;
    if (h < 0 || h >= hq)
        return -1;
    return h / (hq / hkv);
}

/* [WINDOW] causal_window_start: None (-1) when w == 0 or s > t, else
 * max(s, t saturating-minus (w - 1)).  Arguments are cell indices >= 0 and a
 * window length >= 0. */
int64_t oracle_window_start(int64_t t, int64_t s, int64_t w)
{
    if (w == 0 || s > t)
        return -1;
    int64_t back = w - 1;
    int64_t sat = (t >= back) ? t - back : 0;
    return (s > sat) ? s : sat;
}

/* [BYTES] 2*L*B*T*Hkv*d*e with overflow refusal (returns 0 and writes the
 * product, or 1 on overflow). */
int oracle_kv_cache_bytes(uint64_t L, uint64_t B, uint64_t T, uint64_t hkv,
                          uint64_t d, uint64_t e, uint64_t *bytes)
{
    uint64_t f[7] = {2, L, B, T, hkv, d, e};
    uint64_t acc = 1;
    for (int i = 0; i < 7; ++i) {
        if (f[i] != 0 && acc > UINT64_MAX / f[i])
            return 1;
        acc *= f[i];
    }
    *bytes = acc;
    return 0;
}

static int check_heads(int hq, int hkv)
{
    if (hq <= 0 || hkv <= 0 || hq % hkv != 0)
        return ORACLE_ERR_HEADS;
    return ORACLE_OK;
}

/*
 * One attention row, straight from the definition [SOFTMAX]:
 *   scores s_j = scale * sum_c q_c k_{j,c} for j in lo..hi (ascending),
 *   m = max_j s_j, e_j = exp(s_j - m), Z = sum_j e_j, p_j = e_j / Z,
 *   z_c = sum_j p_j v_{j,c}.
 * krow/vrow point at key cell 0 of the shared KV lane; the permitted set is
 * the contiguous range lo..hi (non-empty).  probs (nullable) receives p_j at
 * index j.  scratch holds hi-lo+1 doubles.
 */
static void attend_row(const double *q, const double *krow, const double *vrow,
                       int64_t lo, int64_t hi, int d, double scale,
                       double *z, double *probs, double *scratch)
{
    int64_t n = hi - lo + 1;
    for (int64_t j = lo; j <= hi; ++j) {
        double dot = 0.0;
        for (int c = 0; c < d; ++c)
            dot += q[c] * krow[j * (int64_t)d + c];
        scratch[j - lo] = scale * dot;
    }
    double m = scratch[0];
    for (int64_t i = 1; i < n; ++i)
        if (scratch[i] > m)
            m = scratch[i];
    double sum = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        scratch[i] = exp(scratch[i] - m);
        sum += scratch[i];
    }
    for (int64_t i = 0; i < n; ++i)
        scratch[i] /= sum;
    for (int c = 0; c < d; ++c)
        z[c] = 0.0;
    for (int64_t j = lo; j <= hi; ++j) {
        double p = scratch[j - lo];
        if (probs)
            probs[j] = p;
        for (int c = 0; c < d; ++c)
            z[c] += p * vrow[j * (int64_t)d + c];
    }
}

static void write_record(int32_t *rec, int64_t g, int64_t lo, int64_t hi, int active)
{
    if (!rec)
        return;
    rec[0] = (int32_t)g;
    if (!active) {
        rec[1] = -1;
        rec[2] = -1;
        rec[3] = 0;
        rec[4] = 0;
        return;
    }
    int32_t x = 0;
    for (int64_t j = lo; j <= hi; ++j)
        x ^= (int32_t)j;
    rec[1] = (int32_t)lo;
    rec[2] = (int32_t)hi;
    rec[3] = (int32_t)(hi - lo + 1);
    rec[4] = x;
}

/*
 * Causal prefill [WINDOW][SOFTMAX].  seqlens (nullable => every n_b = T) holds
 * the active length n_b of each batch row, 0 <= n_b <= T.  Query t of batch
 * row b is active when t < n_b; it reads keys lo..t of KV head g(h) with
 * lo = 0 without a window and max(0, t - (w-1)) with one (segment start 0).
 * probs (nullable) is [B,Hq,T,C] and receives the probabilities (zero outside
 * the permitted set); rec (nullable) is [B,T,Hq,5].
 */
int oracle_prefill(const double *q, const double *k, const double *v, double *out,
                   double *probs, int32_t *rec, const int32_t *seqlens, int B, int T,
                   int C, int hq, int hkv, int d, int window, double scale)
{
    int rc = check_heads(hq, hkv);
    if (rc)
        return rc;
    if (window == 0)
        return ORACLE_ERR_ZERO_WINDOW;
    if (B < 0 || T < 0 || C < 0 || d <= 0 || T > C)
        return ORACLE_ERR_SHAPE;
    for (int b = 0; b < B; ++b) {
        int nb = seqlens ? seqlens[b] : T;
        if (nb < 0 || nb > T)
            return ORACLE_ERR_SHAPE;
    }
    if (probs)
        memset(probs, 0, sizeof(double) * (size_t)B * hq * T * C);
    const int64_t rows = (int64_t)B * hq;
#pragma omp parallel
    {
        double *scratch = (double *)malloc(sizeof(double) * (size_t)(C > 0 ? C : 1));
#pragma omp for schedule(dynamic)
        for (int64_t bh = 0; bh < rows; ++bh) {
            int b = (int)(bh / hq), h = (int)(bh % hq);
            int nb = seqlens ? seqlens[b] : T;
            int64_t g = oracle_kv_head_for_query(h, hq, hkv);
            const double *krow = k + ((int64_t)b * hkv + g) * C * d;
            const double *vrow = v + ((int64_t)b * hkv + g) * C * d;
            for (int t = 0; t < T; ++t) {
                double *z = out + (((int64_t)b * T + t) * hq + h) * d;
                int32_t *r = rec ? rec + (((int64_t)b * T + t) * hq + h) * 5 : NULL;
                if (t >= nb) {
                    for (int c = 0; c < d; ++c)
                        z[c] = 0.0;
                    write_record(r, g, 0, 0, 0);
                    continue;
                }
                int64_t lo = window < 0 ? 0 : oracle_window_start(t, 0, window);
                double *prow = probs ? probs + (((int64_t)b * hq + h) * T + t) * C : NULL;
                attend_row(q + (((int64_t)b * hq + h) * T + t) * d, krow, vrow, lo, t, d,
                           scale, z, prow, scratch);
                write_record(r, g, lo, t, 1);
            }
        }
        free(scratch);
    }
    return ORACLE_OK;
}

/*
 * Single-token decode [DECODE][WINDOW][SOFTMAX].  seqlens (nullable => every
 * n_b = C) counts the cached cells including the newly appended one,
 * 0 <= n_b <= C.  The query sits at t = n_b - 1 and reads keys
 * max(0, n_b - w)..n_b - 1 (all n_b keys without a window).  n_b = 0 gives a
 * zero row.  probs (nullable) is [B,Hq,C]; rec (nullable) is [B,Hq,5].
 */
int oracle_decode(const double *q, const double *k, const double *v, double *out,
                  double *probs, int32_t *rec, const int32_t *seqlens, int B, int C,
                  int hq, int hkv, int d, int window, double scale)
{
    int rc = check_heads(hq, hkv);
    if (rc)
        return rc;
    if (window == 0)
        return ORACLE_ERR_ZERO_WINDOW;
    if (B < 0 || C < 0 || d <= 0)
        return ORACLE_ERR_SHAPE;
    for (int b = 0; b < B; ++b) {
        int nb = seqlens ? seqlens[b] : C;
        if (nb < 0 || nb > C)
            return ORACLE_ERR_SHAPE;
    }
    if (probs)
        memset(probs, 0, sizeof(double) * (size_t)B * hq * C);
    const int64_t rows = (int64_t)B * hq;
#pragma omp parallel
    {
        double *scratch = (double *)malloc(sizeof(double) * (size_t)(C > 0 ? C : 1));
#pragma omp for schedule(dynamic)
        for (int64_t bh = 0; bh < rows; ++bh) {
            int b = (int)(bh / hq), h = (int)(bh % hq);
            int nb = seqlens ? seqlens[b] : C;
            int64_t g = oracle_kv_head_for_query(h, hq, hkv);
            double *z = out + bh * d;
            int32_t *r = rec ? rec + bh * 5 : NULL;
            if (nb == 0) {
                for (int c = 0; c < d; ++c)
                    z[c] = 0.0;
                write_record(r, g, 0, 0, 0);
                continue;
            }
            int64_t t = nb - 1;
            int64_t lo = window < 0 ? 0 : oracle_window_start(t, 0, window);
            const double *krow = k + ((int64_t)b * hkv + g) * C * d;
            const double *vrow = v + ((int64_t)b * hkv + g) * C * d;
            attend_row(q + bh * d, krow, vrow, lo, t, d, scale, z,
                       probs ? probs + bh * C : NULL, scratch);
            write_record(r, g, lo, t, 1);
        }
        free(scratch);
    }
    return ORACLE_OK;
}

/*
 * Second, independent formulation [REPEAT][MASKOFF]: materialise the KV heads
 * expanded to Hq lanes (repeat_interleave when tiled == 0; the wrong tiled
 * repeat when tiled != 0, as a negative control), build an explicit boolean
 * keep[i][j] matrix for the tq queries placed at absolute positions
 * s - tq + i over s = n_b keys (bottom-right alignment), intersect it with the
 * window and the active length, fill excluded scores with -infinity and run
 * per-head softmax attention over all C key cells.
 *
 * Used for prefill (tq = T queries, query i at position i, where s is the
 * row's n_b and the queries beyond n_b are inactive) and for decode
 * (tq = 1, the query at s - 1).  q is [B,Hq,tq,d]; out is [B,tq,Hq,d].
 */
int oracle_expanded(const double *q, const double *k, const double *v, double *out,
                    const int32_t *seqlens, int B, int tq, int C, int hq, int hkv, int d,
                    int window, double scale, int decode, int tiled)
{
    int rc = check_heads(hq, hkv);
    if (rc)
        return rc;
    if (window == 0)
        return ORACLE_ERR_ZERO_WINDOW;
    if (B < 0 || tq < 0 || C < 0 || d <= 0 || (!decode && tq > C) || (decode && tq != 1))
        return ORACLE_ERR_SHAPE;
    int r = hq / hkv;
    size_t lane = (size_t)C * d;
    double *kx = (double *)malloc(sizeof(double) * (size_t)B * hq * lane + 1);
    double *vx = (double *)malloc(sizeof(double) * (size_t)B * hq * lane + 1);
    unsigned char *keep = (unsigned char *)malloc((size_t)tq * C + 1);
    double *sc = (double *)malloc(sizeof(double) * (size_t)(C > 0 ? C : 1));
    if (!kx || !vx || !keep || !sc) {
        free(kx);
        free(vx);
        free(keep);
        free(sc);
        return ORACLE_ERR_SHAPE;
    }
    /* Expansion: lane (b, h) copies KV lane (b, src) where src follows the
     * adjacent repeat_interleave layout (copies of one head next to each
     * other) or, for the negative control, the tiled layout. */
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < hq; ++h) {
            int src = tiled ? (h % hkv) : (h / r);
            memcpy(kx + ((size_t)b * hq + h) * lane, k + ((size_t)b * hkv + src) * lane,
                   sizeof(double) * lane);
            memcpy(vx + ((size_t)b * hq + h) * lane, v + ((size_t)b * hkv + src) * lane,
                   sizeof(double) * lane);
        }
    for (int b = 0; b < B; ++b) {
        int nb = seqlens ? seqlens[b] : (decode ? C : tq);
        if (nb < 0 || nb > C || (!decode && nb > tq)) {
            free(kx);
            free(vx);
            free(keep);
            free(sc);
            return ORACLE_ERR_SHAPE;
        }
        /* keep[i][j]: the query's absolute position p = s - tq + i with
         * s = n_b for decode; for prefill the queries are the cells
         * themselves, p = i, active only when i < n_b. */
        for (int i = 0; i < tq; ++i) {
            long p = decode ? (long)nb - tq + i : i;
            int active = decode ? (nb > 0) : (i < nb);
            for (int j = 0; j < C; ++j) {
                int ok = active && j <= p && j < nb;
                if (window > 0 && (long)j < p - (window - 1))
                    ok = 0;
                keep[(size_t)i * C + j] = (unsigned char)ok;
            }
        }
        for (int h = 0; h < hq; ++h) {
            const double *kl = kx + ((size_t)b * hq + h) * lane;
            const double *vl = vx + ((size_t)b * hq + h) * lane;
            for (int i = 0; i < tq; ++i) {
                const double *qi = q + (((size_t)b * hq + h) * tq + i) * d;
                double *z = out + (((size_t)b * tq + i) * hq + h) * d;
                double m = -INFINITY;
                for (int j = 0; j < C; ++j) {
                    if (keep[(size_t)i * C + j]) {
                        double dot = 0.0;
                        for (int c = 0; c < d; ++c)
                            dot += qi[c] * kl[(size_t)j * d + c];
                        sc[j] = dot * scale;
                    } else {
                        sc[j] = -INFINITY;
                    }
                    if (sc[j] > m)
                        m = sc[j];
                }
                for (int c = 0; c < d; ++c)
                    z[c] = 0.0;
                if (m == -INFINITY)
                    continue; /* no permitted key: an inactive row, output 0 */
                double sum = 0.0;
                for (int j = 0; j < C; ++j) {
                    sc[j] = (sc[j] == -INFINITY) ? 0.0 : exp(sc[j] - m);
                    sum += sc[j];
                }
                for (int j = 0; j < C; ++j) {
                    double p = sc[j] / sum;
                    for (int c = 0; c < d; ++c)
                        z[c] += p * vl[(size_t)j * d + c];
                }
            }
        }
    }
    free(kx);
    free(vx);
    free(keep);
    free(sc);
    return ORACLE_OK;
}

/*
 * Queries against a cached prefix [MASKOFF][WINDOW][SEGMENT][SOFTMAX].
 * q is [B,Hq,Tq,d]; out is [B,Tq,Hq,d].  seqlens (nullable => every s_b = C)
 * is the number s_b of cells in the cache, the new ones included; qlens
 * (nullable => every t_b = Tq) is the number t_b <= Tq of new query rows of
 * batch row b.  Query row i < t_b sits at absolute position p = s_b - t_b + i
 * (bottom-right alignment) and reads keys lo..p, where lo is
 * causal_window_start(p, seg, w) with seg = segs[b,i] (nullable => 0), and
 * lo = seg without a window.  A row is inactive, with zero output and the
 * {g,-1,-1,0,0} record, when i >= t_b, when p < 0 (a query placed before the
 * first cell) or when its segment starts after it (seg > p, where the window
 * rule gives no start).  probs (nullable) is [B,Hq,Tq,C]; rec (nullable) is
 * [B,Tq,Hq,5].
 *
 * With t_b = s_b = n_b and no segments this is oracle_prefill; with Tq = 1
 * and t_b = 1 it is oracle_decode.
 */
int oracle_attend_prefix(const double *q, const double *k, const double *v, double *out,
                         double *probs, int32_t *rec, const int32_t *seqlens,
                         const int32_t *qlens, const int32_t *segs, int B, int Tq, int C,
                         int hq, int hkv, int d, int window, double scale)
{
    int rc = check_heads(hq, hkv);
    if (rc)
        return rc;
    if (window == 0)
        return ORACLE_ERR_ZERO_WINDOW;
    if (B < 0 || Tq < 0 || C < 0 || d <= 0 || Tq > C)
        return ORACLE_ERR_SHAPE;
    for (int b = 0; b < B; ++b) {
        int sb = seqlens ? seqlens[b] : C;
        int tb = qlens ? qlens[b] : Tq;
        if (sb < 0 || sb > C || tb < 0 || tb > Tq)
            return ORACLE_ERR_SHAPE;
    }
    if (probs)
        memset(probs, 0, sizeof(double) * (size_t)B * hq * Tq * C);
    const int64_t rows = (int64_t)B * hq;
#pragma omp parallel
    {
        double *scratch = (double *)malloc(sizeof(double) * (size_t)(C > 0 ? C : 1));
#pragma omp for schedule(dynamic)
        for (int64_t bh = 0; bh < rows; ++bh) {
            int b = (int)(bh / hq), h = (int)(bh % hq);
            int sb = seqlens ? seqlens[b] : C;
            int tb = qlens ? qlens[b] : Tq;
            int64_t g = oracle_kv_head_for_query(h, hq, hkv);
            const double *krow = k + ((int64_t)b * hkv + g) * C * d;
            const double *vrow = v + ((int64_t)b * hkv + g) * C * d;
            for (int i = 0; i < Tq; ++i) {
                double *z = out + (((int64_t)b * Tq + i) * hq + h) * d;
                int32_t *r = rec ? rec + (((int64_t)b * Tq + i) * hq + h) * 5 : NULL;
                int64_t p = (int64_t)sb - tb + i;
                int64_t seg = segs ? segs[(int64_t)b * Tq + i] : 0;
                int64_t lo = -1;
                if (i < tb && p >= 0)
                    lo = window < 0 ? (seg <= p ? seg : -1) : oracle_window_start(p, seg, window);
                if (lo < 0) {
                    for (int c = 0; c < d; ++c)
                        z[c] = 0.0;
                    write_record(r, g, 0, 0, 0);
                    continue;
                }
                double *prow = probs ? probs + (((int64_t)b * hq + h) * Tq + i) * C : NULL;
                attend_row(q + (((int64_t)b * hq + h) * Tq + i) * d, krow, vrow, lo, p, d,
                           scale, z, prow, scratch);
                write_record(r, g, lo, p, 1);
            }
        }
        free(scratch);
    }
    return ORACLE_OK;
}

/*
 * Decode with a candidate and/or a rolling cache [DECODE][CANDIDATE][ROLLING].
 * q is [B,Hq,d]; k and v are the caches [B,Hkv,C,d]; out is [B,Hq,d].
 * seqlens (nullable => every n_b = C) counts the cells of the sequence, the
 * new one included, so the query sits at n_b - 1.
 *
 * ring == 0: cell j is stored in slot j, and n_b <= C.
 * ring != 0: cell j is stored in slot j mod C; the window must satisfy
 *   1 <= w <= C so that every key the query may read is still held; n_b may
 *   exceed C.
 * knew/vnew (both or neither) are the candidate's key and value [B,Hkv,d]:
 * cell n_b - 1 is first committed to its slot (k and v are updated in
 * place), then the row attends over the committed cache.  Without a
 * candidate the cache already holds cell n_b - 1.
 *
 * The row reads keys max(0, n_b - w)..n_b - 1 (all of 0..n_b - 1 without a
 * window), gathered from their slots into a linear copy in ascending cell
 * order.  n_b = 0 gives a zero row and commits nothing.  rec (nullable) is
 * [B,Hq,5], in key cells (not slots).
 */
int oracle_decode_cache(const double *q, double *k, double *v, const double *knew,
                        const double *vnew, double *out, int32_t *rec,
                        const int32_t *seqlens, int B, int C, int hq, int hkv, int d,
                        int window, double scale, int ring)
{
    int rc = check_heads(hq, hkv);
    if (rc)
        return rc;
    if (window == 0)
        return ORACLE_ERR_ZERO_WINDOW;
    if (B < 0 || C < 0 || d <= 0 || ((knew == NULL) != (vnew == NULL)))
        return ORACLE_ERR_SHAPE;
    if (ring && (window < 1 || window > C))
        return ORACLE_ERR_SHAPE;
    int64_t span = 1;
    for (int b = 0; b < B; ++b) {
        int nb = seqlens ? seqlens[b] : C;
        if (nb < 0 || (!ring && nb > C))
            return ORACLE_ERR_SHAPE;
        if (nb > span)
            span = nb;
    }
    /* Commit each candidate (one per KV head of a batch row) to its slot. */
    if (knew)
        for (int b = 0; b < B; ++b) {
            int nb = seqlens ? seqlens[b] : C;
            if (nb == 0)
                continue;
            int64_t slot = ring ? (int64_t)(nb - 1) % C : nb - 1;
            for (int g = 0; g < hkv; ++g) {
                size_t dst = (((size_t)b * hkv + g) * C + slot) * d;
                size_t src = ((size_t)b * hkv + g) * d;
                memcpy(k + dst, knew + src, sizeof(double) * d);
                memcpy(v + dst, vnew + src, sizeof(double) * d);
            }
        }
    const int64_t rows = (int64_t)B * hq;
#pragma omp parallel
    {
        double *kl = (double *)malloc(sizeof(double) * (size_t)span * d);
        double *vl = (double *)malloc(sizeof(double) * (size_t)span * d);
        double *scratch = (double *)malloc(sizeof(double) * (size_t)span);
#pragma omp for schedule(dynamic)
        for (int64_t bh = 0; bh < rows; ++bh) {
            int b = (int)(bh / hq), h = (int)(bh % hq);
            int nb = seqlens ? seqlens[b] : C;
            int64_t g = oracle_kv_head_for_query(h, hq, hkv);
            double *z = out + bh * d;
            int32_t *r = rec ? rec + bh * 5 : NULL;
            if (nb == 0) {
                for (int c = 0; c < d; ++c)
                    z[c] = 0.0;
                write_record(r, g, 0, 0, 0);
                continue;
            }
            int64_t t = nb - 1;
            int64_t lo = window < 0 ? 0 : oracle_window_start(t, 0, window);
            const double *kc = k + ((int64_t)b * hkv + g) * C * d;
            const double *vc = v + ((int64_t)b * hkv + g) * C * d;
            /* Gather cells lo..t from their slots into a linear copy. */
            for (int64_t j = lo; j <= t; ++j) {
                int64_t slot = ring ? j % C : j;
                memcpy(kl + (j - lo) * d, kc + slot * d, sizeof(double) * d);
                memcpy(vl + (j - lo) * d, vc + slot * d, sizeof(double) * d);
            }
            attend_row(q + bh * d, kl, vl, 0, t - lo, d, scale, z, NULL, scratch);
            write_record(r, g, lo, t, 1);
        }
        free(kl);
        free(vl);
        free(scratch);
    }
    return ORACLE_OK;
}
