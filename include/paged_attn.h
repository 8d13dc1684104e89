/*
 * paged_attn.h — C ABI of the MI355X (gfx950) paged grouped-query attention library.
 *
 * Operations over a block-paged KV cache:
 *   kv_page_write            scatter new K/V rows into their pages
 *   kv_page_write_rope       the same, from f32 rows: K (and the query) rotated by RoPE,
 *                            K and V rounded to the pool dtype
 *   paged_attn_decode        one query row per sequence, split-KV partial softmax
 *   paged_attn_combine       log-sum-exp merge of the split partials
 *   paged_attn_decode_fused  the three above for one decode step, in a single launch
 *   paged_attn_decode_fused_noalloc  the same step with a library-owned workspace
 *   paged_attn_prefill       causal attention for packed prompt segments
 *
 * Sources (the method these calls implement):
 *   [crucible-results] crucible, "Paged attention results" (docs/paged-attention-results.md):
 *       the descriptor, grid and causal-visibility description of the selected prefill kernel;
 *       the page translation physical_page = request_table[position >> 4], slot = position & 15;
 *       the GQA map kv_head = query_head / (n_head / n_kv_head).
 *   [crucible-readme] crucible README: "Paged KV cache and continuous batching" (pool layout,
 *       offset formula, power-of-two page size), "Split-position attention: implemented, exact,
 *       and it did not help" (per-chunk partial softmax merged by exp(m_chunk - m_global)),
 *       the scheduler section on chunked prefill (chunk row r attends to 0 ..= done + r),
 *       and "What actually runs" (owner and absolute-position arrays route the K/V writes).
 *   [minfer-d3-6] minfer step 71 "D3-6 GQA q-head batched attention", 3.2 Excerpts A and F:
 *       the split partition chunk = ceil(nkv / splits), split sp covers
 *       [sp*chunk, min(nkv, (sp+1)*chunk)); idle splits report max = -inf, sum = 0.
 *   [vllm-cpp-383] vllm.cpp PR #383, "head_dim-128 arm for the warp-split-KV decode kernel":
 *       the decode kernel's head_dim-256 instantiation and its windowed (HasWindow) arm.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The library allocates
 *     nothing, keeps no data between calls and is re-entrant (paged_attn_decode_fused keeps
 *     its per-call state in the caller's counter buffer; see there).  The one exception is
 *     paged_attn_decode_fused_noalloc, whose workspace is a fixed library-owned array per GPU
 *     shared by its calls (see there).
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL = the null stream).
 *     No call synchronises; ordering is stream order, so a kv_page_write enqueued before an
 *     attention call on the same stream is visible to it.
 *   - Host scalar arguments are validated before anything is enqueued.  On failure the call
 *     returns PA_EINVAL (malformed) or PA_EUNSUPPORTED (valid but not built) and enqueues
 *     nothing.  PA_ELAUNCH reports a HIP launch error.
 *   - Device-resident metadata (page tables, context lengths, descriptors, positions) is a
 *     caller contract: page ids in [0, num_pages), lengths and positions inside the table's
 *     capacity.  The kernels never read or write outside the buffers whose sizes the host
 *     arguments describe: out-of-range page ids are clamped (attention) or the row is
 *     skipped (write), and lengths are clamped to max_pages_per_seq * page_size; the
 *     numerical result for such input is unspecified.
 *   - Checked build (libpaged_attn_checked.so, compiled with -DPAGED_ATTN_CHECKED): the same
 *     entry points, whose kernels also record the device metadata they clamp or skip --
 *     a length outside [0, capacity], a page id outside [0, num_pages) among the positions
 *     a call reads or writes, a malformed prefill descriptor, a write to a missing table row
 *     or beyond the table's capacity (a negative owner or position remains an explicit
 *     skip).  Each call then synchronises its stream and returns PA_EDATA if anything was
 *     recorded.  It is a debugging aid: it synchronises, so it is not for graph capture,
 *     and its records are per library and device, so calls running at the same time from
 *     several host threads can see each other's reports.
 *   - Layouts are dense row-major with the innermost dimension last:
 *       q            [tokens][Hq][D]                    f32
 *       K/V pages    [num_pages][page_size][Hkv][D]     kv_dtype
 *       page_table   [rows][max_pages_per_seq]          int32, logical page -> physical page
 *     Query head h reads KV head h / (Hq / Hkv).
 *   - Supported: head_dim in {64, 128}, and 256 for decode, the merge and the page writes
 *     (decode at 256 with f16 or bf16 K/V: [vllm-cpp-383], the head_dim-256 decode arm);
 *     page_size a power of two in [1, 4096]; Hq a multiple of Hkv with Hq / Hkv <= 64;
 *     kv_dtype f32, f16 (IEEE binary16) or bf16.
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_dtype { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2 } pa_dtype;

typedef enum pa_status {
    PA_OK = 0,
    PA_EINVAL = -1,        /* malformed argument: null pointer, bad shape, overflow          */
    PA_EUNSUPPORTED = -2,  /* well-formed but not built: head_dim, dtype, group size          */
    PA_ELAUNCH = -3,       /* the HIP runtime rejected a launch (no device, bad stream, ...)  */
    PA_EDATA = -4,         /* checked build only: device metadata out of range (see below)    */
    PA_ESCRATCH = -5       /* paged_attn_decode_fused_noalloc: the call's split workspace does
                              not fit the library's fixed no-allocation workspace              */
} pa_status;

/* Short English text for a status code (static storage, never NULL). */
const char* paged_attn_status_string(int status);

/*
 * Bytes of split workspace that paged_attn_decode writes and paged_attn_combine reads:
 *   partial_o  [num_seqs][num_q_heads][num_splits][head_dim] f32
 *   partial_ml [num_seqs][num_q_heads][num_splits][2]        f32
 * Returns the sum of both sizes, or 0 if an argument is not positive or the size overflows.
 */
size_t paged_attn_decode_workspace_bytes(int num_seqs, int num_q_heads, int head_dim,
                                         int num_splits);

/*
 * Split-KV decode: the per-split partial softmax of [crucible-readme] "Split-position
 * attention" with the split partition of [minfer-d3-6] Excerpt A.
 *
 * Sequence b has ctx = context_lens[b] keys, positions 0 .. ctx-1 (ctx counts the current
 * token, whose K/V the caller has already written).  Its token t lives in physical page
 * page_table[b][t / page_size], slot t % page_size.  It attends to positions [w0, ctx):
 * w0 = 0, or with a sliding window (window > 0; [vllm-cpp-383], the windowed arm of the
 * decode kernel) w0 = max(0, ctx - window), the current token and the window - 1 before it.
 * With n = ctx - w0 and chunk = ceil(n / num_splits), split s covers tokens
 * [w0 + s*chunk, w0 + min(n, (s+1)*chunk)).  For every query head h and split s:
 *     score_t = scale * dot(q[b][h][:], K[t][h / (Hq/Hkv)][:])
 *     m       = max_t score_t                                  (natural-log units)
 *     l       = sum_t exp(score_t - m)
 *     O[:]    = sum_t exp(score_t - m) * V[t][h / (Hq/Hkv)][:] (not normalised)
 * written as partial_ml[b][h][s] = {m, l} and partial_o[b][h][s][:] = O.
 * An empty split writes m = -INFINITY, l = 0, O = 0.
 *
 *   q               [num_seqs][num_q_heads][head_dim] f32, device
 *   k_pages,v_pages [num_pages][page_size][num_kv_heads][head_dim] kv_dtype, device
 *   page_table      [num_seqs][max_pages_per_seq] int32, device
 *   context_lens    [num_seqs] int32, device; 1 <= ctx <= max_pages_per_seq * page_size
 *                   (ctx <= 0 makes every split empty)
 *   scale           normally 1/sqrt(head_dim), rounded to f32 by the caller
 *   window          sliding window in positions; <= 0 attends the whole context
 *   num_splits      S in [1, 4096]
 *   partial_o       [num_seqs][num_q_heads][S][head_dim] f32, device, written
 *   partial_ml      [num_seqs][num_q_heads][S][2] f32, device, written
 * num_seqs == 0 is a valid empty call: returns PA_OK and enqueues nothing.
 */
int paged_attn_decode(const float* q, const void* k_pages, const void* v_pages,
                      pa_dtype kv_dtype, const int32_t* page_table,
                      const int32_t* context_lens, int num_seqs, int num_q_heads,
                      int num_kv_heads, int head_dim, int page_size, int num_pages,
                      int max_pages_per_seq, float scale, int window, int num_splits,
                      float* partial_o, float* partial_ml, void* stream);

/*
 * Single-launch decode step: the page write of the current token, the split-KV partials and
 * their merge in ONE kernel (crucible README, "Split-position attention": the second
 * dispatch costs about what the split gains; minfer D3-6, section 3.3 and section 5: per-layer
 * dispatch and exposed latency are the residual).  The result equals
 *     kv_page_write(current token) ; paged_attn_decode ; paged_attn_combine
 * on the same arguments, to within f32 rounding (the merge is the same arithmetic).
 *
 *   k_new, v_new    [num_seqs][num_kv_heads][head_dim] kv_dtype, device: the K/V of each
 *                   sequence's current token, which sits at position context_lens[b] - 1;
 *                   it is stored into its page (bit-exact) and read from k_new/v_new here
 *   k_pages,v_pages written at that one slot per (sequence, KV head), read elsewhere
 *   partial_o, partial_ml  split workspace as for paged_attn_decode (left holding the
 *                   partials)
 *   counters        paged_attn_decode_fused_counters(...) uint32 words, device: zero before the
 *                   first call; every call leaves them zero again (the last split of a group
 *                   resets its counter; with num_splits = 1 they are not touched), so the
 *                   buffer is reused without clearing.  One counter per (sequence, KV
 *                   head, head group of the launch): a workgroup serves up to 16 query
 *                   heads (8 for f32 pools, 4 at head_dim 256), and the launch spreads a KV
 *                   head's heads over at most twice that many groups, never more than the
 *                   2 * ceil(G / 8) the buffer holds.
 *   out             [num_seqs][num_q_heads][head_dim] f32, device, written
 * All other arguments and rules as for paged_attn_decode.  Calls that share a counters
 * buffer must not overlap in time (enqueue them on one stream).
 */
int paged_attn_decode_fused(const float* q, const void* k_new, const void* v_new,
                            void* k_pages, void* v_pages, pa_dtype kv_dtype,
                            const int32_t* page_table, const int32_t* context_lens,
                            int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                            int page_size, int num_pages, int max_pages_per_seq, float scale,
                            int window, int num_splits, float* partial_o, float* partial_ml,
                            uint32_t* counters, float* out, void* stream);

/* Number of uint32 words of counters paged_attn_decode_fused needs at any head_dim, or 0 for
 * invalid arguments: num_seqs * num_kv_heads * 2 * ceil((Hq/Hkv) / 8) counters, each in a
 * 128-byte line of its own (32 words), so that the tickets of different groups do not queue
 * on one line.  The buffer's start must be 128-byte aligned for that (any device allocation
 * is); it is correct at any 4-byte alignment. */
size_t paged_attn_decode_fused_counters(int num_seqs, int num_q_heads, int num_kv_heads);

/*
 * paged_attn_decode_fused for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  The same step on the
 * same arguments, minus the caller's split workspace and counters, with the same result bit
 * for bit.  The partials and counters live in one library-owned device array per GPU of
 * paged_attn_noalloc_scratch_bytes() bytes (16 MiB), placed in that GPU's memory when the
 * library is first used on it and held until the process ends; the call itself allocates
 * nothing and frees nothing.
 *   Limits: the split workspace (paged_attn_decode_workspace_bytes(num_seqs, num_q_heads,
 *   head_dim, num_splits), e.g. 8.5 MB for 16 sequences x 64 heads x 16 splits at head_dim
 *   128) must fit in 15 MiB, and the counters (paged_attn_decode_fused_counters words) in
 *   1 MiB (8192 counters of 128 bytes); a larger call returns PA_ESCRATCH and enqueues
 *   nothing.
 *   Sharing: every call on one GPU uses that GPU's array, which keeps the last call's partials.
 *   Calls that overlap in time on one GPU (different streams or host threads) race and give
 *   undefined results: enqueue them on one stream.  The counters start at zero and every call
 *   leaves them at zero, so no clearing is needed between calls.
 * Arguments, rules and other errors as for paged_attn_decode_fused.
 */
int paged_attn_decode_fused_noalloc(const float* q, const void* k_new, const void* v_new,
                                    void* k_pages, void* v_pages, pa_dtype kv_dtype,
                                    const int32_t* page_table, const int32_t* context_lens,
                                    int num_seqs, int num_q_heads, int num_kv_heads,
                                    int head_dim, int page_size, int num_pages,
                                    int max_pages_per_seq, float scale, int window,
                                    int num_splits, float* out, void* stream);

/* Bytes of the fixed per-GPU workspace of paged_attn_decode_fused_noalloc. */
size_t paged_attn_noalloc_scratch_bytes(void);

/*
 * Merge of split partials ([crucible-readme] "Split-position attention": rescale each chunk
 * by exp(m_chunk - m_global) and merge; [minfer-d3-6] Excerpt F: idle splits weigh zero):
 *     M      = max over splits with l_s > 0 of m_s
 *     w_s    = exp(m_s - M) if l_s > 0, else 0
 *     out[:] = sum_s w_s * O_s[:] / sum_s w_s * l_s
 * A row whose splits are all empty is written as zeros.
 *   partial_o, partial_ml as written by paged_attn_decode (same num_seqs/heads/splits/dim)
 *   out  [num_seqs][num_q_heads][head_dim] f32, device, written
 */
int paged_attn_combine(const float* partial_o, const float* partial_ml, int num_seqs,
                       int num_q_heads, int head_dim, int num_splits, float* out,
                       void* stream);

/*
 * Causal packed prefill ([crucible-results] selected-kernel description; [crucible-readme]
 * scheduler section on chunked prefill).  Segment i is the int32 quadruple
 *     seg_desc[i] = {packed_start, chunk_len, absolute_start, table_index}
 * and its packed query row r (0 <= r < chunk_len), at q[packed_start + r], is the token at
 * absolute position P = absolute_start + r of the sequence whose pages are listed in
 * page_table[table_index].  It attends to that sequence's positions 0 .. P inclusive:
 *     out[packed_start + r][h][:] = softmax_t(scale * q.K[t]) . V[t],  t in [0, P]
 * The caller writes the K/V of every attended position (including the chunk itself) first,
 * with finite values at every position 0 .. absolute_start + chunk_len - 1: rows are
 * computed 16 at a time, and a masked position's weight is exactly 0, which does not cancel
 * an infinity or NaN held at a later position of the same chunk.
 * Segments must not overlap in the packed dimension; rows not covered by any segment are
 * left untouched.
 * Arithmetic: f32 products and sums for an f32 pool.  For an f16/bf16 pool the products run
 * on the 16-bit matrix units with f32 accumulation: K and V enter unchanged, while the
 * scaled q and the softmax weights are each carried as two 16-bit terms (hi + lo, residual
 * below 2^-16 of the value for bf16, 2^-22 for f16), so the result stays close to f32
 * rounding rather than to one 16-bit rounding of q and of the weights.
 *
 *   q               [total_tokens][num_q_heads][head_dim] f32, device
 *   k_pages,v_pages [num_pages][page_size][num_kv_heads][head_dim] kv_dtype, device
 *   page_table      [num_tables][max_pages_per_seq] int32, device
 *   seg_desc        [num_segs][4] int32, device
 *   max_chunk_len   host copy of max_i chunk_len (sizes the grid; rows past it are skipped)
 *   out             [total_tokens][num_q_heads][head_dim] f32, device, written
 * num_segs == 0 or max_chunk_len == 0 is a valid empty call.
 */
int paged_attn_prefill(const float* q, const void* k_pages, const void* v_pages,
                       pa_dtype kv_dtype, const int32_t* page_table, const int32_t* seg_desc,
                       int num_segs, int num_tables, int total_tokens, int max_chunk_len,
                       int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                       int num_pages, int max_pages_per_seq, float scale, float* out,
                       void* stream);

/*
 * Page write ([crucible-readme] "Paged KV cache and continuous batching" and "What actually
 * runs"): for token i with owner row o = token_table_index[i] and absolute position
 * p = token_position[i], copy the bytes of k_new[i][h][:] to
 * K[page_table[o][p / page_size]][p % page_size][h][:] for every KV head h, and the same
 * for V.  No conversion: the copy is bit-exact and every other byte of the pools is left
 * unchanged.  Tokens whose owner, position or page id is out of range are skipped.  Two
 * tokens mapping to the same slot in one call race (unspecified which one lands).
 *
 *   k_new, v_new        [num_tokens][num_kv_heads][head_dim] kv_dtype, device
 *   k_pages, v_pages    [num_pages][page_size][num_kv_heads][head_dim] kv_dtype, device
 *   page_table          [num_tables][max_pages_per_seq] int32, device
 *   token_table_index   [num_tokens] int32, device
 *   token_position      [num_tokens] int32, device
 * num_tokens == 0 is a valid empty call.
 */
int kv_page_write(const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                  pa_dtype kv_dtype, const int32_t* page_table,
                  const int32_t* token_table_index, const int32_t* token_position,
                  int num_tokens, int num_tables, int num_kv_heads, int head_dim,
                  int page_size, int num_pages, int max_pages_per_seq, void* stream);

/*
 * Page write with rotary position embedding (crucible, "Paged attention results": the K
 * projection output is rotated by RoPE and scattered to the paged pool, V is scattered
 * unrotated, and the query projection is rotated at the same positions before attention;
 * crucible README, "Validating the forward pass": the two RoPE pairing conventions).
 * For token i at position p = token_position[i] and each KV head h:
 *   K[slot][h][:] = rotate(k_new[i][h][:], p) and V[slot][h][:] = v_new[i][h][:], both
 *   rounded to kv_dtype (to nearest, ties to even), slot as for kv_page_write;
 *   q[i][hq][:] = rotate(q[i][hq][:], p) in place for every query head, if q is not NULL.
 * rotate turns pair i (i < head_dim / 2) — dims (2i, 2i+1) for PA_ROPE_ADJACENT, (i,
 * i + head_dim/2) for PA_ROPE_HALVES — by the angle t = f32(p) * inv_freq[i] (an f32
 * product): (a, b) -> (a cos t - b sin t, a sin t + b cos t), computed in f32.
 * A token with p < 0 is skipped altogether.  A token whose owner, position or page id is out
 * of range writes nothing (its query is still rotated).  Two tokens mapping to the same slot
 * in one call race (unspecified which one lands).
 *
 *   k_new, v_new        [num_tokens][num_kv_heads][head_dim] f32, device (K before RoPE)
 *   k_pages, v_pages    [num_pages][page_size][num_kv_heads][head_dim] kv_dtype, device
 *   page_table, token_table_index, token_position   as for kv_page_write
 *   inv_freq            [head_dim / 2] f32, device: the rotation frequency of each pair, e.g.
 *                       base^(-2i / head_dim) for a base of 10000
 *   q                   [num_tokens][num_q_heads][head_dim] f32, device, or NULL
 * num_tokens == 0 is a valid empty call.
 */
typedef enum pa_rope_style { PA_ROPE_ADJACENT = 0, PA_ROPE_HALVES = 1 } pa_rope_style;

int kv_page_write_rope(const float* k_new, const float* v_new, void* k_pages, void* v_pages,
                       pa_dtype kv_dtype, const int32_t* page_table,
                       const int32_t* token_table_index, const int32_t* token_position,
                       const float* inv_freq, pa_rope_style style, float* q, int num_q_heads,
                       int num_tokens, int num_tables, int num_kv_heads, int head_dim,
                       int page_size, int num_pages, int max_pages_per_seq, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */
