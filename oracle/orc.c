/*
 * orc.c -- plain, slow CPU reference for chunked-prefill causal attention
 * over a KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * bench's CPU-baseline leg load this library.  It shares no code, header or
 * constant with the GPU library and never calls it.
 *
 * Everything is fp64.  Stored elements (fp32, fp16, bf16) are widened to
 * double exactly before any arithmetic; nothing is rounded on the way out.
 *
 * What it computes (sources):
 *  - scaled dot-product attention, softmax(q k^T * scale) v with the
 *    default scale 1/sqrt(D): Ultralytics glossary "Chunked Prefill",
 *    section "how chunked prefill works" (the PyTorch demo);
 *  - a query at absolute position p sees keys [0, p] only, whether the
 *    prompt is run in one pass or in chunks: ONNX GenAI Wiki "Chunked
 *    Prefill", section 1.2 (causal mask);
 *  - the cache is appended strictly left to right and earlier bytes are
 *    never rewritten: same page, section 1.1 (append-only KV cache);
 *  - the rolling fixed-capacity cache new = cat(old, chunk)[c:] and the
 *    additive mask whose masked entries hold -32768: Horizon developer blog
 *    "Chunk Prefill", sections 3 and 4.
 *
 * Parity pins for every function live in tests/test_oracle_pins.py.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };

/* Threads the OpenMP loops use (reported beside the oracle's timings). */
int orc_num_threads(void) { return omp_get_max_threads(); }

/* Thread count of later OpenMP loops (timing runs at one thread and at all
   of them); n < 1 is ignored. */
void orc_set_num_threads(int n)
{
    if (n >= 1) omp_set_num_threads(n);
}

/* IEEE binary16 -> double, exact (subnormals, inf and NaN included). */
static double orc_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int mant = h & 0x3ff;
    double mag;
    if (expo == 0)
        mag = ldexp((double)mant, -24);               /* subnormal / zero */
    else if (expo == 31)
        mag = mant ? NAN : INFINITY;
    else
        mag = ldexp((double)(mant | 0x400), expo - 25); /* 1.m * 2^(e-15) */
    return sign ? -mag : mag;
}

/* bfloat16 is the top half of an fp32 bit pattern: widen exactly. */
static double orc_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Widen n stored elements of the given dtype to double.  Returns 0, or -1 on
 * an unknown dtype. */
int orc_widen(const void *src, int dtype, int64_t n, double *dst)
{
    int64_t i;
    if (dtype == ORC_F32) {
        const float *s = (const float *)src;
        for (i = 0; i < n; ++i) dst[i] = (double)s[i];
        return 0;
    }
    if (dtype == ORC_F16) {
        const uint16_t *s = (const uint16_t *)src;
        for (i = 0; i < n; ++i) dst[i] = orc_half_to_double(s[i]);
        return 0;
    }
    if (dtype == ORC_BF16) {
        const uint16_t *s = (const uint16_t *)src;
        for (i = 0; i < n; ++i) dst[i] = orc_bf16_to_double(s[i]);
        return 0;
    }
    return -1;
}

/*
 * Attention for n_q query rows of one sequence.
 *
 *   q      [n_q][Hq][D]    query rows (token-major)
 *   k, v   [Hkv][n_k][D]   one sequence's keys and values (head-major, the
 *                          same order as the cache)
 *   lo, hi [n_q]           row i sees keys j with lo[i] <= j <= hi[i]
 *   addmask [n_q][n_k] or NULL: added to every included score (the
 *                          additive-mask form of the Horizon blog, section 4)
 *   out    [n_q][Hq][D]
 *
 * Query head h reads KV head h / (Hq / Hkv): grouped-query attention with
 * contiguous groups (the pages name GQA without fixing the mapping; this is
 * the common reading, pinned against a library routine in the tests).
 *
 * For each (row, head):  s_j = scale * sum_d q_d k_jd (+ mask_j),
 * m = max_j s_j,  w_j = exp(s_j - m),  out_d = sum_j w_j v_jd / sum_j w_j.
 * A row whose visible set is empty has no defined result: it gets NaN.
 *
 * Returns 0, or -1 on inconsistent sizes.
 */
int orc_attention(const double *q, int n_q, int Hq,
                  const double *k, const double *v, int n_k, int Hkv, int D,
                  const int32_t *lo, const int32_t *hi,
                  const double *addmask, double scale, double *out)
{
    int i, h;
    if (n_q < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || n_k < 0 || Hq % Hkv != 0)
        return -1;
    for (i = 0; i < n_q; ++i)
        if (lo[i] < 0 || hi[i] >= n_k)
            return -1;

#pragma omp parallel for collapse(2) schedule(dynamic, 4)
    for (i = 0; i < n_q; ++i) {
        for (h = 0; h < Hq; ++h) {
            const int group = Hq / Hkv;
            const int g = h / group;
            const double *qi = q + ((int64_t)i * Hq + h) * D;
            const double *kg = k + (int64_t)g * n_k * D;
            const double *vg = v + (int64_t)g * n_k * D;
            double *oi = out + ((int64_t)i * Hq + h) * D;
            int j, d;
            int j0 = lo[i], j1 = hi[i];
            double m = -INFINITY, den = 0.0;
            double *s;

            if (j1 < j0) {
                for (d = 0; d < D; ++d) oi[d] = NAN;
                continue;
            }
            s = (double *)malloc(sizeof(double) * (size_t)(j1 - j0 + 1));
            for (j = j0; j <= j1; ++j) {
                double dot = 0.0;
                for (d = 0; d < D; ++d)
                    dot += qi[d] * kg[(int64_t)j * D + d];
                dot *= scale;
                if (addmask)
                    dot += addmask[(int64_t)i * n_k + j];
                s[j - j0] = dot;
                if (dot > m) m = dot;
            }
            for (d = 0; d < D; ++d) oi[d] = 0.0;
            for (j = j0; j <= j1; ++j) {
                double w = exp(s[j - j0] - m);
                den += w;
                for (d = 0; d < D; ++d)
                    oi[d] += w * vg[(int64_t)j * D + d];
            }
            for (d = 0; d < D; ++d) oi[d] /= den;
            free(s);
        }
    }
    return 0;
}

/*
 * Append `rows` token-major K/V rows to one sequence's cache at position
 * past_len: cache[h][past_len + r][:] = new[r][h][:].  A byte copy, so the
 * cache is bit-identical to its inputs (ONNX GenAI Wiki "Chunked Prefill",
 * section 1.1).  cache_* are [Hkv][cap][D] of elem_size bytes.
 * Returns 0, or -1 when the rows do not fit the capacity.
 */
int orc_kv_append(void *cache_k, void *cache_v, int Hkv, int cap, int D,
                  int elem_size, const void *k_new, const void *v_new,
                  int past_len, int rows)
{
    int h, r;
    const size_t row_bytes = (size_t)D * (size_t)elem_size;
    if (past_len < 0 || rows < 0 || past_len + rows > cap)
        return -1;
    for (r = 0; r < rows; ++r) {
        for (h = 0; h < Hkv; ++h) {
            size_t dst = ((size_t)h * cap + (size_t)(past_len + r)) * row_bytes;
            size_t src = ((size_t)r * Hkv + (size_t)h) * row_bytes;
            memcpy((char *)cache_k + dst, (const char *)k_new + src, row_bytes);
            memcpy((char *)cache_v + dst, (const char *)v_new + src, row_bytes);
        }
    }
    return 0;
}

/*
 * Rolling cache step, literally: tmp = cat(old, chunk) along the position
 * axis, then new = tmp[:, c:] (Horizon developer blog "Chunk Prefill",
 * section 3).  old/new are [H][C][D]; chunk is token-major [c][H][D].
 * Returns 0, or -1 if c > C.
 */
int orc_roll_append(const void *old, const void *chunk, void *out,
                    int H, int C, int c, int D, int elem_size)
{
    const size_t row = (size_t)D * (size_t)elem_size;
    char *tmp;
    int h, t;
    if (c < 0 || c > C)
        return -1;
    tmp = (char *)malloc((size_t)H * (size_t)(C + c) * row + 1);
    for (h = 0; h < H; ++h) {
        memcpy(tmp + (size_t)h * (C + c) * row,
               (const char *)old + (size_t)h * C * row, (size_t)C * row);
        for (t = 0; t < c; ++t)
            memcpy(tmp + ((size_t)h * (C + c) + (size_t)(C + t)) * row,
                   (const char *)chunk + ((size_t)t * H + h) * row, row);
    }
    for (h = 0; h < H; ++h)
        memcpy((char *)out + (size_t)h * C * row,
               tmp + ((size_t)h * (C + c) + (size_t)c) * row, (size_t)C * row);
    free(tmp);
    return 0;
}
