/*
 * oracle.h — the f64 CPU oracle's own declarations (test infrastructure; see oracle.c).
 * Deliberately independent of the HIP library's header: nothing is shared.
 */
#ifndef PAGED_ATTN_ORACLE_H
#define PAGED_ATTN_ORACLE_H

#include <stdint.h>

#define ORACLE_F32 0
#define ORACLE_F16 1
#define ORACLE_BF16 2

double oracle_f16_to_f64(uint16_t bits);
double oracle_bf16_to_f64(uint16_t bits);

/* [lo, hi) token range of one split of an n-token context (chunk = ceil(n / num_splits)). */
int oracle_split_range(int n, int num_splits, int split, int* lo, int* hi);

/* out[b][h][d] = attention of q[b][h] over positions 0 .. context_lens[b]-1, or over the
 * last `window` of them when window > 0.  Returns 0. */
int oracle_decode(const float* q, const void* k_pages, const void* v_pages, int dtype,
                  const int32_t* page_table, const int32_t* context_lens, int num_seqs,
                  int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                  int max_pages_per_seq, float scale, int window, double* out);

/* Per-split (m, l, unnormalised O) in natural-log units; idle splits (-inf, 0, 0).  The
 * splits partition the attended positions (the last `window` when window > 0). */
int oracle_decode_partials(const float* q, const void* k_pages, const void* v_pages, int dtype,
                           const int32_t* page_table, const int32_t* context_lens,
                           int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                           int page_size, int max_pages_per_seq, float scale, int window,
                           int num_splits, double* partial_o, double* partial_m,
                           double* partial_l);

/* Log-sum-exp merge of split partials; all-empty rows give zeros. */
int oracle_combine(const double* partial_o, const double* partial_m, const double* partial_l,
                   int num_seqs, int num_q_heads, int head_dim, int num_splits, double* out);

/* Causal packed prefill over segment descriptors {packed_start, len, abs_start, table}.
 * *causal_positions receives sum over rows of (abs_start + r + 1), per head. */
int oracle_prefill(const float* q, const void* k_pages, const void* v_pages, int dtype,
                   const int32_t* page_table, const int32_t* seg_desc, int num_segs,
                   int num_tables, int total_tokens, int num_q_heads, int num_kv_heads,
                   int head_dim, int page_size, int max_pages_per_seq, float scale,
                   double* out, int64_t* causal_positions);

/* Byte copy of new K/V rows into their (page, slot); invalid tokens are skipped. */
int oracle_kv_write(const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                    int dtype, const int32_t* page_table, const int32_t* token_table_index,
                    const int32_t* token_position, int num_tokens, int num_tables,
                    int num_kv_heads, int head_dim, int page_size, int num_pages,
                    int max_pages_per_seq);



/* Page write with rotary position embedding: K rotated at its position, K and V converted
 * to the pool dtype (through f32, ties to even) and placed as oracle_kv_write places rows;
 * q (optional) rotated in place.  style 0 pairs dims (2i, 2i+1), style 1 pairs (i, i+D/2). */
int oracle_kv_write_rope(const float* k_new, const float* v_new, void* k_pages, void* v_pages,
                         int dtype, const int32_t* page_table, const int32_t* token_table_index,
                         const int32_t* token_position, const float* inv_freq, int style,
                         float* q, int num_q_heads, int num_tokens, int num_tables,
                         int num_kv_heads, int head_dim, int page_size, int num_pages,
                         int max_pages_per_seq);

/* dst[i] = src[i] rounded to dtype (through f32, to nearest, ties to even). */
void oracle_round_to(int dtype, const double* src, int64_t n, void* dst);

/* dst[i] = exact f64 value of element i of src. */
void oracle_widen(int dtype, const void* src, int64_t n, double* dst);
#endif
