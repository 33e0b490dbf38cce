/*
 * pda_oracle.c -- fp64 CPU oracle for paged single-token decode attention.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path links, loads or calls
 * this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do. It shares no code, header, table or constant with the
 * GPU library: every decode, lookup and reduction below is written out here
 * from the definitions.
 *
 * What it computes (the plain definition: block paging only moves where a
 * token's key/value rows are stored and how they are found, the arithmetic
 * is ordinary attention -- "9 Decode and KV Cache", section 9.5,
 * PagedAttention):
 *
 *   for each sequence b and query head h, with g = n_q / n_kv and the KV head
 *   j = h / g (grouped-query attention: several query heads read one stored
 *   KV head -- GQA teaser on the kv-cache tag page; SoK paper section 1.1):
 *     n   = context_lens[b]                 (includes the token appended now)
 *     for t in [0, n):
 *        pb  = block_table[b][t / bs]        (logical block -> physical block,
 *        off = t % bs                         worked example "PagedAttention
 *                                             block lookup", section 9.5)
 *        k_t = K[pb][j][off][:],  v_t = V[pb][j][off][:]   (decoded to fp64;
 *              quantized caches: k_t = k_scale[pb][j] * dec(code))
 *        s_t = scale * sum_d q[b][h][d] * k_t[d]            (index order)
 *     m   = max_t s_t                        (pass 1)
 *     w_t = exp(s_t - m), Z = sum_t w_t      (pass 2)
 *     out = (sum_t w_t v_t) / Z
 *
 * A two-pass softmax, never an online one. n == 0 gives a zero row. A logical
 * block whose table entry is not a valid physical block id is an error, like
 * the failing dictionary lookup of the worked example: that row's output is
 * NaN and it is counted in the return value.
 *
 * An optional token window [t_begin, t_end) restricts the sum to a contiguous
 * range of logical positions; the partial result (normalised output, max
 * score m, and Z) is what a split-KV partition holds before the merge.
 *
 * Sliding window with attention sinks (long-context variants of "9 Decode and
 * KV Cache", section 9.7: a sliding window keeps only the most recent W
 * tokens; attention sinks keep the first few tokens as well; the sink and
 * sliding-window teasers on the kv-cache tag page): with window W > 0 and S
 * sink tokens, only positions t with t < S or t >= n - W enter the softmax;
 * the others are not looked up at all. W = 0 attends to every position.
 *
 * Element decodes (written from the format definitions, not from any library):
 *   f32  : IEEE binary32 as stored.
 *   bf16 : the upper 16 bits of a binary32.
 *   fp8  : OCP 8-bit E4M3 ("FN"): sign, 4 exponent bits with bias 7, 3 mantissa
 *          bits; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no inf.
 *   int8 : two's-complement integer value.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* cache element formats; OR_F64 holds values already decoded to fp64 (the
 * 4-bit cache is decoded on the Python side, see oracle/__init__.py) */
enum { OR_F32 = 0, OR_BF16 = 1, OR_FP8 = 2, OR_INT8 = 3, OR_F64 = 5 };

static double or_dec_f32(const void* p, int64_t i) {
    float f;
    memcpy(&f, (const char*)p + 4 * i, 4);
    return (double)f;
}

static double or_dec_bf16(const void* p, int64_t i) {
    uint16_t h;
    memcpy(&h, (const char*)p + 2 * i, 2);
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

double or_dec_fp8_code(unsigned code) {
    unsigned s = (code >> 7) & 1u, e = (code >> 3) & 15u, m = code & 7u;
    double v;
    if (e == 15u && m == 7u) return NAN;
    if (e == 0u) v = ldexp((double)m / 8.0, -6);
    else v = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return s ? -v : v;
}

static double or_dec_fp8(const void* p, int64_t i) {
    return or_dec_fp8_code(((const uint8_t*)p)[i]);
}

static double or_dec_int8(const void* p, int64_t i) {
    return (double)((const int8_t*)p)[i];
}

static double or_dec_f64(const void* p, int64_t i) {
    double d;
    memcpy(&d, (const char*)p + 8 * i, 8);
    return d;
}

typedef double (*or_dec_fn)(const void*, int64_t);

/* Is logical position t of an n-token row attended (window / sink rule)? */
static int or_attended(int64_t t, int64_t n, int64_t window, int64_t sinks) {
    return window <= 0 || t < sinks || t >= n - window;
}

static or_dec_fn or_decoder(int dtype) {
    switch (dtype) {
    case OR_F32: return or_dec_f32;
    case OR_BF16: return or_dec_bf16;
    case OR_FP8: return or_dec_fp8;
    case OR_INT8: return or_dec_int8;
    case OR_F64: return or_dec_f64;
    default: return NULL;
    }
}

/* Decode n elements of a raw buffer into fp64 (exposed for tests). */
int or_decode(const void* src, int dtype, int64_t n, double* dst) {
    or_dec_fn dec = or_decoder(dtype);
    if (!dec) return -1;
    for (int64_t i = 0; i < n; ++i) dst[i] = dec(src, i);
    return 0;
}

/*
 * Paged decode attention, fp64.
 *   q       [B][n_q][d_h]            (q_dtype f32 or bf16)
 *   k, v    [num_blocks][n_kv][bs][d_h] (kv_dtype)
 *   k_scale, v_scale [num_blocks][n_kv] fp32, used iff kv_dtype is fp8/int8
 *   block_table [B][max_blocks] int32, context_lens [B] int32
 *   rows    list of (b * n_q + h) to compute, or NULL for all B*n_q rows
 *   t_begin, t_end  token window (t_end < 0: to the end of each row)
 *   window, sinks   attend only to t < sinks or t >= n - window (window 0: all)
 *   out     [n_rows][d_h] fp64; m_out, z_out [n_rows] (either may be NULL)
 * Returns the number of rows that hit an unmapped block or an invalid
 * context length (their outputs are NaN), or -1 on a bad argument.
 */
int64_t or_paged_attn(int B, int n_q, int n_kv, int d_h, int bs, int num_blocks, int max_blocks,
                      const void* q, int q_dtype, const void* k, const void* v, int kv_dtype,
                      const float* k_scale, const float* v_scale,
                      const int32_t* block_table, const int32_t* context_lens, double scale,
                      const int64_t* rows, int64_t n_rows, int64_t t_begin, int64_t t_end,
                      int64_t window, int64_t sinks,
                      double* out, double* m_out, double* z_out, int nthreads) {
    if (B <= 0 || n_q <= 0 || n_kv <= 0 || d_h <= 0 || bs <= 0 || n_q % n_kv) return -1;
    if (window < 0 || sinks < 0) return -1;
    or_dec_fn dq = or_decoder(q_dtype), dkv = or_decoder(kv_dtype);
    if (!dq || !dkv) return -1;
    int quant = (kv_dtype == OR_FP8 || kv_dtype == OR_INT8);
    if (quant && (!k_scale || !v_scale)) return -1;
    const int g = n_q / n_kv;
    const int64_t total = rows ? n_rows : (int64_t)B * n_q;
    int64_t bad = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

#pragma omp parallel reduction(+ : bad)
    {
        int64_t cap = 0;
        double* s = NULL;
        double* qd = (double*)malloc(sizeof(double) * (size_t)d_h);
        double* acc = (double*)malloc(sizeof(double) * (size_t)d_h);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < total; ++r) {
            const int64_t row = rows ? rows[r] : r;
            const int b = (int)(row / n_q), h = (int)(row % n_q);
            const int j = h / g;
            double* o = out + r * d_h;
            const int64_t n = context_lens[b];
            int64_t lo = t_begin < 0 ? 0 : t_begin;
            int64_t hi = (t_end < 0 || t_end > n) ? n : t_end;
            if (n < 0 || n > (int64_t)max_blocks * bs) {
                for (int d = 0; d < d_h; ++d) o[d] = NAN;
                if (m_out) m_out[r] = NAN;
                if (z_out) z_out[r] = NAN;
                ++bad;
                continue;
            }
            if (hi <= lo) {
                for (int d = 0; d < d_h; ++d) o[d] = 0.0;
                if (m_out) m_out[r] = -INFINITY;
                if (z_out) z_out[r] = 0.0;
                continue;
            }
            if (hi - lo > cap) {
                cap = hi - lo;
                s = (double*)realloc(s, sizeof(double) * (size_t)cap);
            }
            for (int d = 0; d < d_h; ++d) qd[d] = dq(q, ((int64_t)b * n_q + h) * d_h + d);
            /* scores, checking every lookup */
            int unmapped = 0;
            for (int64_t t = lo; t < hi && !unmapped; ++t) {
                if (!or_attended(t, n, window, sinks)) continue;
                const int32_t pb = block_table[(int64_t)b * max_blocks + t / bs];
                if (pb < 0 || pb >= num_blocks) { unmapped = 1; break; }
                const int64_t base = (((int64_t)pb * n_kv + j) * bs + t % bs) * d_h;
                const double ks = quant ? (double)k_scale[(int64_t)pb * n_kv + j] : 1.0;
                double dot = 0.0;
                for (int d = 0; d < d_h; ++d) dot += qd[d] * (ks * dkv(k, base + d));
                s[t - lo] = scale * dot;
            }
            if (unmapped) {
                for (int d = 0; d < d_h; ++d) o[d] = NAN;
                if (m_out) m_out[r] = NAN;
                if (z_out) z_out[r] = NAN;
                ++bad;
                continue;
            }
            /* pass 1: maximum */
            double m = -INFINITY;
            for (int64_t t = lo; t < hi; ++t) {
                if (!or_attended(t, n, window, sinks)) continue;
                const double x = s[t - lo];
                if (isnan(x) || isnan(m)) m = NAN; /* a NaN key poisons the row */
                else if (x > m) m = x;
            }
            /* pass 2: weights, normaliser, weighted sum of values */
            double z = 0.0;
            for (int d = 0; d < d_h; ++d) acc[d] = 0.0;
            for (int64_t t = lo; t < hi; ++t) {
                if (!or_attended(t, n, window, sinks)) continue;
                const int32_t pb = block_table[(int64_t)b * max_blocks + t / bs];
                const int64_t base = (((int64_t)pb * n_kv + j) * bs + t % bs) * d_h;
                const double vs = quant ? (double)v_scale[(int64_t)pb * n_kv + j] : 1.0;
                const double w = exp(s[t - lo] - m);
                z += w;
                for (int d = 0; d < d_h; ++d) acc[d] += w * (vs * dkv(v, base + d));
            }
            if (z == 0.0) { /* no attended position in [lo, hi): an empty partial */
                for (int d = 0; d < d_h; ++d) o[d] = 0.0;
                if (m_out) m_out[r] = -INFINITY;
                if (z_out) z_out[r] = 0.0;
                continue;
            }
            for (int d = 0; d < d_h; ++d) o[d] = acc[d] / z;
            if (m_out) m_out[r] = m;
            if (z_out) z_out[r] = z;
        }
        free(s);
        free(qd);
        free(acc);
    }
    return bad;
}

int or_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
