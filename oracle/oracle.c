/*
 * oracle.c — plain, slow, f64 CPU oracle for paged grouped-query attention.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the bench's CPU-baseline leg
 * load this library.  It shares no code, header, table or helper with the HIP library; it
 * is written from the definitions on the source pages, not from the kernels.
 *
 * Everything is computed in IEEE double.  Inputs are widened exactly (f32, f16 and bf16 are
 * all subsets of f64); libm exp() is the only transcendental.  Single-threaded, no SIMD,
 * no reordering beyond what each definition states: sums run in ascending index order.
 *
 * Sources:
 *  - crucible, "Paged attention results": the reference attention order (full score vector,
 *    global maximum, exp(score - max), one sum, V accumulated in ascending history order);
 *    page translation physical_page = request_table[position >> 4], slot = position & 15;
 *    kv_head = query_head / (n_head / n_kv_head); a packed row at absolute P reads only its
 *    own request's positions 0..P; descriptors int4[packed_start, chunk_len, absolute_start,
 *    table_index].
 *  - crucible README, "Paged KV cache and continuous batching": pool layout and the offset
 *    formula (here per layer: [num_pages][page_size][Hkv][D]); "Split-position attention":
 *    per-chunk partial softmax merged by rescaling with exp(m_chunk - m_global), exact;
 *    "Validating the forward pass": the CPU path is scalar with f64 accumulation.
 *  - minfer 71 "D3-6 GQA q-head batched attention", 3.2 Excerpt A: chunk = ceil(nkv/splits),
 *    split sp covers [sp*chunk, min(nkv, sp*chunk + chunk)); Excerpt F: idle splits write
 *    max = -inf, sum = 0 and weigh zero in the merge.
 *
 * Pins: every function here is checked by the CPU tests against things other than itself —
 * closed forms, a library attention routine, exhaustive dtype decoding against numpy/torch,
 * brute-force causality, and the causal-position counts the crucible results page prints.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

/* Planted-mistake hooks, used only by the mutation test (tests/test_oracle_mutants.py):
 * building with -DORACLE_MUTANT=k compiles mistake k in, to show that some pin fails.
 * The normal build (ORACLE_MUTANT = 0) contains none of them. */
#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif
#define MUT(k) (ORACLE_MUTANT == (k))

/* ---------------------------------------------------------------- element decoding */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_f16_to_f64(uint16_t bits) {
    int sign = (bits >> 15) & 1;
    int expo = (bits >> 10) & 0x1f;
    int frac = bits & 0x3ff;
    double v;
    if (expo == 0) {
        v = ldexp((double)frac, MUT(1) ? -14 : -24);    /* subnormal: frac * 2^-24 */
    } else if (expo == 31) {
        v = frac ? NAN : INFINITY;
    } else {
        v = ldexp((double)(frac + 1024), expo - 25);    /* (1 + frac/2^10) * 2^(expo-15) */
    }
    return sign ? -v : v;
}

/* bfloat16: the upper 16 bits of an IEEE 754 binary32. */
double oracle_bf16_to_f64(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double load_elem(const void* base, int dtype, size_t idx) {
    switch (dtype) {
        case ORACLE_F32: return (double)((const float*)base)[idx];
        case ORACLE_F16: return oracle_f16_to_f64(((const uint16_t*)base)[idx]);
        default:         return oracle_bf16_to_f64(((const uint16_t*)base)[idx]);
    }
}

static int elem_size(int dtype) { return dtype == ORACLE_F32 ? 4 : 2; }

/* ---------------------------------------------------------------- paging */

/* Flat element index of K/V[position t][kv head][0] for one sequence's page-table row:
 * physical page = table_row[t / page_size], slot = t % page_size, pool [P][ps][Hkv][D]. */
static size_t row_index(const int32_t* table_row, int t, int kv_head, int num_kv_heads,
                        int head_dim, int page_size) {
    size_t page = (size_t)table_row[t / page_size];
    size_t slot = (size_t)((MUT(2) ? t + 1 : t) % page_size);
    return ((page * (size_t)page_size + slot) * (size_t)num_kv_heads + (size_t)kv_head) *
           (size_t)head_dim;
}

/* Contiguous gather of positions 0..n-1 of one KV head into dst[n][D] (f64). */
static void gather(const void* pages, int dtype, const int32_t* table_row, int n, int kv_head,
                   int num_kv_heads, int head_dim, int page_size, double* dst) {
    for (int t = 0; t < n; ++t) {
        size_t base = row_index(table_row, t, kv_head, num_kv_heads, head_dim, page_size);
        for (int d = 0; d < head_dim; ++d)
            dst[(size_t)t * head_dim + d] = load_elem(pages, dtype, base + (size_t)d);
    }
}

/* ---------------------------------------------------------------- attention of one row */

/* Exact two-pass softmax attention of one query row over the first n gathered positions:
 *   s[t]   = scale * sum_d q[d] * K[t][d]           (ascending d)
 *   m      = max_t s[t]
 *   p[t]   = exp(s[t] - m),  l = sum_t p[t]         (ascending t)
 *   out[d] = (sum_t p[t] * V[t][d]) / l             (ascending t)
 * s is caller scratch of at least n doubles.  n >= 1. */
static void attend(const float* q, const double* K, const double* V, int n, int head_dim,
                   double scale, double* s, double* out) {
    double m = -INFINITY;
    for (int t = 0; t < n; ++t) {
        double dot = 0.0;
        for (int d = 0; d < head_dim; ++d) dot += (double)q[d] * K[(size_t)t * head_dim + d];
        s[t] = MUT(3) ? dot : scale * dot;
        if (s[t] > m) m = s[t];
    }
    double l = 0.0;
    for (int t = 0; t < n; ++t) {
        s[t] = exp(s[t] - m);
        l += s[t];
    }
    for (int d = 0; d < head_dim; ++d) {
        double acc = 0.0;
        for (int t = 0; t < n; ++t) acc += s[t] * (MUT(4) ? K : V)[(size_t)t * head_dim + d];
        out[d] = acc / l;
    }
}

static int check_heads(int num_q_heads, int num_kv_heads, int head_dim, int page_size) {
    if (num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || page_size <= 0) return -1;
    if (num_q_heads % num_kv_heads != 0) return -1;
    return 0;
}

/* ---------------------------------------------------------------- decode */

/* First attended position of an n-token context under a sliding window of `window`
 * positions (vllm.cpp PR #383: the windowed arm of the decode kernel): the current token
 * and the window - 1 before it, [n - window, n); window <= 0 attends the whole context. */
static int window_start(int n, int window) {
    if (window <= 0 || n <= window) return 0;
    return MUT(14) ? n - window + 1 : n - window;
}

int oracle_decode(const float* q, const void* k_pages, const void* v_pages, int dtype,
                  const int32_t* page_table, const int32_t* context_lens, int num_seqs,
                  int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                  int max_pages_per_seq, float scale, int window, double* out) {
    if (check_heads(num_q_heads, num_kv_heads, head_dim, page_size)) return -1;
    const int group = num_q_heads / num_kv_heads;
    int max_ctx = 1;
    for (int b = 0; b < num_seqs; ++b) {
        int n = context_lens[b];
        if (n < 1 || n > max_pages_per_seq * page_size) return -2;
        if (n > max_ctx) max_ctx = n;
    }
    double* K = malloc(sizeof(double) * (size_t)max_ctx * head_dim);
    double* V = malloc(sizeof(double) * (size_t)max_ctx * head_dim);
    double* s = malloc(sizeof(double) * (size_t)max_ctx);
    if (!K || !V || !s) { free(K); free(V); free(s); return -3; }
    for (int b = 0; b < num_seqs; ++b) {
        const int n = context_lens[b];
        const int32_t* row = page_table + (size_t)b * max_pages_per_seq;
        for (int g = 0; g < num_kv_heads; ++g) {
            gather(k_pages, dtype, row, n, g, num_kv_heads, head_dim, page_size, K);
            gather(v_pages, dtype, row, n, g, num_kv_heads, head_dim, page_size, V);
            const int w0 = window_start(n, window);
            for (int j = 0; j < group; ++j) {
                const int h = MUT(5) ? j * num_kv_heads + g : g * group + j;
                attend(q + ((size_t)b * num_q_heads + h) * head_dim, K + (size_t)w0 * head_dim,
                       V + (size_t)w0 * head_dim, n - w0, head_dim, (double)scale, s,
                       out + ((size_t)b * num_q_heads + h) * head_dim);
            }
        }
    }
    free(K); free(V); free(s);
    return 0;
}

/* ---------------------------------------------------------------- split partials */

int oracle_split_range(int n, int num_splits, int split, int* lo, int* hi) {
    if (num_splits < 1 || split < 0 || split >= num_splits || n < 0) return -1;
    int chunk = MUT(6) ? n / num_splits : (n + num_splits - 1) / num_splits;
    int a = split * chunk;
    int e = a + chunk < n ? a + chunk : n;
    if (a > n) a = n;
    if (e < a) e = a;
    *lo = a;
    *hi = e;
    return 0;
}

int oracle_decode_partials(const float* q, const void* k_pages, const void* v_pages, int dtype,
                           const int32_t* page_table, const int32_t* context_lens,
                           int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                           int page_size, int max_pages_per_seq, float scale, int window,
                           int num_splits, double* partial_o, double* partial_m,
                           double* partial_l) {
    if (check_heads(num_q_heads, num_kv_heads, head_dim, page_size) || num_splits < 1)
        return -1;
    const int group = num_q_heads / num_kv_heads;
    int max_ctx = 1;
    for (int b = 0; b < num_seqs; ++b) {
        int n = context_lens[b];
        if (n < 0 || n > max_pages_per_seq * page_size) return -2;
        if (n > max_ctx) max_ctx = n;
    }
    double* K = malloc(sizeof(double) * (size_t)max_ctx * head_dim);
    double* V = malloc(sizeof(double) * (size_t)max_ctx * head_dim);
    double* s = malloc(sizeof(double) * (size_t)max_ctx);
    double* p = malloc(sizeof(double) * (size_t)max_ctx);
    if (!K || !V || !s || !p) { free(K); free(V); free(s); free(p); return -3; }
    for (int b = 0; b < num_seqs; ++b) {
        const int n = context_lens[b];
        const int32_t* row = page_table + (size_t)b * max_pages_per_seq;
        for (int g = 0; g < num_kv_heads; ++g) {
            gather(k_pages, dtype, row, n, g, num_kv_heads, head_dim, page_size, K);
            gather(v_pages, dtype, row, n, g, num_kv_heads, head_dim, page_size, V);
            for (int h = g * group; h < (g + 1) * group; ++h) {
                const float* qh = q + ((size_t)b * num_q_heads + h) * head_dim;
                for (int t = 0; t < n; ++t) {
                    double dot = 0.0;
                    for (int d = 0; d < head_dim; ++d)
                        dot += (double)qh[d] * K[(size_t)t * head_dim + d];
                    s[t] = (double)scale * dot;
                }
                /* The splits partition the attended positions [w0, n). */
                const int w0 = window_start(n, window);
                for (int sp = 0; sp < num_splits; ++sp) {
                    size_t slot = ((size_t)b * num_q_heads + h) * num_splits + sp;
                    double* o = partial_o + slot * head_dim;
                    int lo, hi;
                    oracle_split_range(n - w0, num_splits, sp, &lo, &hi);
                    lo += w0;
                    hi += w0;
                    if (lo >= hi) {                       /* idle split */
                        partial_m[slot] = -INFINITY;
                        partial_l[slot] = 0.0;
                        for (int d = 0; d < head_dim; ++d) o[d] = 0.0;
                        continue;
                    }
                    double m = -INFINITY;
                    for (int t = lo; t < hi; ++t) if (s[t] > m) m = s[t];
                    double l = 0.0;
                    for (int t = lo; t < hi; ++t) {
                        p[t] = exp(s[t] - m);
                        l += p[t];
                    }
                    for (int d = 0; d < head_dim; ++d) {
                        double acc = 0.0;
                        for (int t = lo; t < hi; ++t) acc += p[t] * V[(size_t)t * head_dim + d];
                        o[d] = acc;
                    }
                    partial_m[slot] = m;
                    partial_l[slot] = l;
                }
            }
        }
    }
    free(K); free(V); free(s); free(p);
    return 0;
}

/* ---------------------------------------------------------------- combine */

int oracle_combine(const double* partial_o, const double* partial_m, const double* partial_l,
                   int num_seqs, int num_q_heads, int head_dim, int num_splits, double* out) {
    if (num_splits < 1 || head_dim <= 0) return -1;
    for (size_t r = 0; r < (size_t)num_seqs * num_q_heads; ++r) {
        const double* m = partial_m + r * num_splits;
        const double* l = partial_l + r * num_splits;
        const double* o = partial_o + r * num_splits * head_dim;
        double* y = out + r * head_dim;
        double M = -INFINITY;
        for (int sp = 0; sp < num_splits; ++sp)
            if (l[sp] > 0.0 && m[sp] > M) M = m[sp];
        if (M == -INFINITY) {                             /* every split empty */
            for (int d = 0; d < head_dim; ++d) y[d] = 0.0;
            continue;
        }
        double L = 0.0;
        for (int sp = 0; sp < num_splits; ++sp)
            if (l[sp] > 0.0) L += (MUT(7) ? 1.0 : exp(m[sp] - M)) * l[sp];
        for (int d = 0; d < head_dim; ++d) {
            double acc = 0.0;
            for (int sp = 0; sp < num_splits; ++sp)
                if (l[sp] > 0.0)
                    acc += (MUT(7) ? 1.0 : exp(m[sp] - M)) * o[(size_t)sp * head_dim + d];
            y[d] = acc / L;
        }
    }
    return 0;
}

/* ---------------------------------------------------------------- prefill */

int oracle_prefill(const float* q, const void* k_pages, const void* v_pages, int dtype,
                   const int32_t* page_table, const int32_t* seg_desc, int num_segs,
                   int num_tables, int total_tokens, int num_q_heads, int num_kv_heads,
                   int head_dim, int page_size, int max_pages_per_seq, float scale,
                   double* out, int64_t* causal_positions) {
    if (check_heads(num_q_heads, num_kv_heads, head_dim, page_size)) return -1;
    const int group = num_q_heads / num_kv_heads;
    int max_hist = 1;
    for (int i = 0; i < num_segs; ++i) {
        const int32_t* dsc = seg_desc + 4 * (size_t)i;
        int start = dsc[0], len = dsc[1], abs0 = dsc[2], tbl = dsc[3];
        if (len < 0 || start < 0 || abs0 < 0 || start + len > total_tokens) return -2;
        if (tbl < 0 || tbl >= num_tables) return -2;
        if (len > 0 && abs0 + len > max_pages_per_seq * page_size) return -2;
        if (abs0 + len > max_hist) max_hist = abs0 + len;
    }
    double* K = malloc(sizeof(double) * (size_t)max_hist * head_dim);
    double* V = malloc(sizeof(double) * (size_t)max_hist * head_dim);
    double* s = malloc(sizeof(double) * (size_t)max_hist);
    if (!K || !V || !s) { free(K); free(V); free(s); return -3; }
    int64_t count = 0;
    for (int i = 0; i < num_segs; ++i) {
        const int32_t* dsc = seg_desc + 4 * (size_t)i;
        const int start = dsc[0], len = dsc[1], abs0 = dsc[2];
        const int32_t* row = page_table + (size_t)(MUT(11) ? 0 : dsc[3]) * max_pages_per_seq;
        if (len == 0) continue;
        const int hist = abs0 + len;                      /* positions 0 .. abs0+len-1 */
        for (int r = 0; r < len; ++r) count += (int64_t)(abs0 + r + 1);
        for (int g = 0; g < num_kv_heads; ++g) {
            gather(k_pages, dtype, row, hist, g, num_kv_heads, head_dim, page_size, K);
            gather(v_pages, dtype, row, hist, g, num_kv_heads, head_dim, page_size, V);
            for (int h = g * group; h < (g + 1) * group; ++h) {
                for (int r = 0; r < len; ++r) {
                    const int P = (MUT(9) ? 0 : abs0) + r;  /* absolute position of the row */
                    const size_t tok = (size_t)start + r;
                    attend(q + (tok * num_q_heads + h) * head_dim, K, V, MUT(8) ? P : P + 1,
                           head_dim,
                           (double)scale, s, out + (tok * num_q_heads + h) * head_dim);
                }
            }
        }
    }
    if (causal_positions) *causal_positions = count;
    free(K); free(V); free(s);
    return 0;
}

/* ---------------------------------------------------------------- page write */

int oracle_kv_write(const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                    int dtype, const int32_t* page_table, const int32_t* token_table_index,
                    const int32_t* token_position, int num_tokens, int num_tables,
                    int num_kv_heads, int head_dim, int page_size, int num_pages,
                    int max_pages_per_seq) {
    if (num_kv_heads <= 0 || head_dim <= 0 || page_size <= 0) return -1;
    const size_t row_bytes = (size_t)num_kv_heads * head_dim * elem_size(dtype);
    for (int i = 0; i < num_tokens; ++i) {
        int owner = token_table_index[i];
        int pos = token_position[i];
        if (owner < 0 || owner >= num_tables) continue;
        if (pos < 0 || pos >= max_pages_per_seq * page_size) continue;
        int page = page_table[(size_t)owner * max_pages_per_seq + pos / page_size];
        if (page < 0 || page >= num_pages) continue;
        size_t dst = ((size_t)page * page_size + (size_t)((MUT(10) ? pos + 1 : pos) % page_size)) *
                     row_bytes;
        memcpy((char*)k_pages + dst, (const char*)k_new + (size_t)i * row_bytes, row_bytes);
        memcpy((char*)v_pages + dst, (const char*)v_new + (size_t)i * row_bytes, row_bytes);
    }
    return 0;
}

/* ---------------------------------------------------------------- page write with RoPE */

/* Round x to the nearest value of a binary format with `digits` significant bits, smallest
 * normal exponent emin (fixed quantum below it: subnormals) and largest finite value
 * max_finite; ties to even; beyond the overflow threshold, infinity (IEEE 754 rounding).
 * x / quantum is exact (a power-of-two scaling), and rint rounds half to even. */
static double round_binary(double x, int digits, int emin, double max_finite) {
    if (x == 0.0 || isnan(x) || isinf(x)) return x;
    int e;
    frexp(x, &e);                       /* |x| in [2^(e-1), 2^e) */
    int ex = e - 1;
    if (ex < emin) ex = emin;
    const double quantum = ldexp(1.0, ex - (digits - 1));
    const double r = rint(x / quantum) * quantum;
    if (fabs(r) > max_finite) return copysign(INFINITY, x);
    return r;
}

/* Bit pattern of a value already representable in binary16 / bfloat16 (sign, biased
 * exponent, fraction; exponent 0 for zero and subnormals, all ones for infinity). */
static uint16_t encode_small(double r, int frac_bits, int bias) {
    uint16_t sign = signbit(r) ? (uint16_t)(1u << 15) : 0;
    const double a = fabs(r);
    const int exp_all_ones = (1 << (15 - frac_bits)) - 1;
    if (isinf(a)) return sign | (uint16_t)(exp_all_ones << frac_bits);
    if (a == 0.0) return sign;
    const double min_normal = ldexp(1.0, 1 - bias);
    if (a < min_normal) {   /* subnormal: a = frac * 2^(1 - bias - frac_bits) */
        return sign | (uint16_t)ldexp(a, bias - 1 + frac_bits);
    }
    int e;
    const double f = frexp(a, &e);      /* a = f * 2^e, f in [0.5, 1) */
    const int biased = e - 1 + bias;
    const uint32_t frac = (uint32_t)ldexp(2.0 * f - 1.0, frac_bits);
    return sign | (uint16_t)((biased << frac_bits) | frac);
}

/* Store f64 value y as element idx of a cache pool: rounded to f32 first (the arithmetic
 * precision of the kernels, so that both sides round the same f32 value to 16 bits), then
 * to binary16 or bfloat16, each time to nearest, ties to even. */
static void store_elem(void* base, int dtype, size_t idx, double y) {
    const double y32 = round_binary(y, 24, -126, 3.4028234663852886e38);
    if (dtype == ORACLE_F32) {
        ((float*)base)[idx] = (float)y32;
    } else if (dtype == ORACLE_F16) {
        ((uint16_t*)base)[idx] = encode_small(round_binary(y32, 11, -14, 65504.0), 10, 15);
    } else {
        ((uint16_t*)base)[idx] =
            encode_small(round_binary(y32, 8, -126, 3.3895313892515355e38), 7, 127);
    }
}

/* Rotary position embedding of one head row x[0..D) at position pos, in place, in f64.
 * Pair i (i < D/2) is (2i, 2i+1) for style 0 (adjacent dims) or (i, i + D/2) for style 1
 * (the two halves): the two pairing conventions the crucible README names as a silent
 * failure when swapped.  Its angle is the f32 product of f32(pos) and the caller's
 * frequency inv_freq[i] (the kernels' precision for the angle), and the pair turns by it:
 * (a, b) -> (a cos t - b sin t, a sin t + b cos t). */
static void rotate_row(double* x, int head_dim, int pos, const float* inv_freq, int style) {
    const int half = head_dim / 2;
    for (int i = 0; i < half; ++i) {
        const double t = round_binary((double)(float)pos * (double)inv_freq[i], 24, -126,
                                      3.4028234663852886e38);
        const double c = cos(t), sn = sin(MUT(12) ? -t : t);
        const int i0 = style == 0 ? 2 * i : i;
        const int i1 = style == 0 ? 2 * i + 1 : i + half;
        const double a = x[i0], b = x[i1];
        x[i0] = a * c - b * sn;
        x[i1] = a * sn + b * c;
    }
}

/* The page write with RoPE and conversion (crucible results: the K projection writes a
 * scratch slice, RoPE rotates it, K scatters to the paged pool, V scatters unrotated; the
 * query is rotated at the same positions before attention):
 *   q (optional, f32 [T][Hq][D]): rotated in place at token_position[i];
 *   K pages: rotate(k_new[i]) converted to the pool's dtype at (table[owner][pos / ps],
 *            pos % ps), as oracle_kv_write places rows;
 *   V pages: v_new[i] converted, same slot.
 * A token with a negative position is skipped altogether; one whose owner, position or page
 * is out of range keeps the pools untouched (its query is still rotated). */
int oracle_kv_write_rope(const float* k_new, const float* v_new, void* k_pages, void* v_pages,
                         int dtype, const int32_t* page_table, const int32_t* token_table_index,
                         const int32_t* token_position, const float* inv_freq, int style,
                         float* q, int num_q_heads, int num_tokens, int num_tables,
                         int num_kv_heads, int head_dim, int page_size, int num_pages,
                         int max_pages_per_seq) {
    if (num_kv_heads <= 0 || head_dim <= 0 || head_dim % 2 || page_size <= 0) return -1;
    if (style != 0 && style != 1) return -1;
    double* row = malloc(sizeof(double) * (size_t)head_dim);
    if (!row) return -2;
    for (int i = 0; i < num_tokens; ++i) {
        const int pos = token_position[i];
        if (pos < 0) continue;
        for (int h = 0; q && h < num_q_heads; ++h) {
            float* qr = q + ((size_t)i * num_q_heads + h) * head_dim;
            for (int d = 0; d < head_dim; ++d) row[d] = qr[d];
            rotate_row(row, head_dim, pos, inv_freq, style);
            for (int d = 0; d < head_dim; ++d) store_elem(qr, ORACLE_F32, (size_t)d, row[d]);
        }
        const int owner = token_table_index[i];
        if (owner < 0 || owner >= num_tables) continue;
        if (pos >= max_pages_per_seq * page_size) continue;
        const int page = page_table[(size_t)owner * max_pages_per_seq + pos / page_size];
        if (page < 0 || page >= num_pages) continue;
        const size_t slot = (size_t)page * page_size + (size_t)(pos % page_size);
        for (int h = 0; h < num_kv_heads; ++h) {
            const size_t src = ((size_t)i * num_kv_heads + h) * head_dim;
            const size_t dst = (slot * num_kv_heads + h) * head_dim;
            for (int d = 0; d < head_dim; ++d) row[d] = k_new[src + d];
            rotate_row(row, head_dim, MUT(13) ? pos + 1 : pos, inv_freq, style);
            for (int d = 0; d < head_dim; ++d) store_elem(k_pages, dtype, dst + d, row[d]);
            for (int d = 0; d < head_dim; ++d)
                store_elem(v_pages, dtype, dst + d, (double)v_new[src + d]);
        }
    }
    free(row);
    return 0;
}

/* f64 values rounded to a pool dtype as store_elem does (through f32), for the tests. */
void oracle_round_to(int dtype, const double* src, int64_t n, void* dst) {
    for (int64_t i = 0; i < n; ++i) store_elem(dst, dtype, (size_t)i, src[i]);
}

/* ---------------------------------------------------------------- helpers for the tests */

/* dst[i] = exact f64 value of element i of src (dtype f32, f16 or bf16). */
void oracle_widen(int dtype, const void* src, int64_t n, double* dst) {
    for (int64_t i = 0; i < n; ++i) dst[i] = load_elem(src, dtype, (size_t)i);
}
