// api.hip — the C ABI of include/paged_attn.h: host-side validation, then one launch per
// kernel on the caller's stream.  No allocation and no synchronisation; the only state is
// read-once device facts (a device's CU count, a kernel's raised dynamic-LDS limit).
//
// Every host scalar is checked before anything is enqueued (crucible, "Paged attention
// results": malformed shapes, overflow and bad indices are rejected before device access).
// Device-resident metadata is not read here: that would need a device-to-host copy and a
// synchronisation.  The kernels instead keep every access inside the buffers the host
// arguments describe (clamped page ids, clamped lengths, skipped rows).  The checked build
// (-DPAGED_ATTN_CHECKED) is the exception: after each launch it synchronises the stream and
// reports the metadata its kernels found out of range as PA_EDATA.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

#include "../../include/paged_attn.h"
#include "common.h"

namespace {

constexpr int64_t kI32Max = 2147483647;
constexpr int kMaxGridYZ = 65535;
constexpr int kMaxSplits = 4096;
constexpr int kMaxGroup = 64;
// Query heads one decode workgroup serves: the 16 columns of a matrix-core block (16-bit
// pools at head_dim 64 and 128), or on the vector units (f32 pools, head_dim 256) 8, and 4 at
// head_dim 256, where every head holds D accumulators per lane group.
constexpr int kMaxHeadsPerWg = 16;
int max_heads_per_wg(int kv_dtype, int head_dim) {
    if (head_dim == 256) return 4;
    return kv_dtype == PA_F32 ? 8 : kMaxHeadsPerWg;
}
// The single-launch step's counter buffer holds 2 * ceil(group / 8) counters per KV head
// (paged_attn_decode_fused_counters), at least twice the head groups of any grid below,
// each in a 128-byte line of its own (kCounterStride words).
constexpr int kCounterHeads = 8;

// Compute units of the current device, read once per device (0 if the runtime cannot say).
int compute_units() {
    static std::atomic<int> cached[pa::kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= pa::kMaxDevices) return 0;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int ilog2(int x) {
    int s = 0;
    while ((1 << s) < x) ++s;
    return s;
}

bool valid_dtype(int d) { return d == PA_F32 || d == PA_F16 || d == PA_BF16; }

int elem_bytes(int d) { return d == PA_F32 ? 4 : 2; }

// Shape checks shared by the calls that read K/V pages.
int check_pages(int kv_dtype, int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                int num_pages, int max_pages_per_seq, bool allow_d256 = true) {
    if (!valid_dtype(kv_dtype)) return PA_EINVAL;
    if (num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads != 0)
        return PA_EINVAL;
    if (head_dim < 1 || page_size < 1 || num_pages < 1 || max_pages_per_seq < 1)
        return PA_EINVAL;
    if (head_dim != 64 && head_dim != 128 && !(allow_d256 && head_dim == 256))
        return PA_EUNSUPPORTED;
    if (!is_pow2(page_size) || page_size > 4096) return PA_EUNSUPPORTED;
    if (num_q_heads / num_kv_heads > kMaxGroup) return PA_EUNSUPPORTED;
    if ((int64_t)max_pages_per_seq * page_size > kI32Max) return PA_EINVAL;
    if ((int64_t)num_pages * page_size > kI32Max) return PA_EINVAL;
    return PA_OK;
}

// Status of an enqueued call.  The checked build then waits for the stream and reports
// device metadata that a kernel found out of range (and clamped or skipped) as PA_EDATA.
int launched(hipError_t e, void* stream) {
    if (e != hipSuccess) return PA_ELAUNCH;
    if constexpr (!pa::kChecked) {
        (void)stream;
        return PA_OK;
    } else {
        if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return PA_ELAUNCH;
        int any = 0;
        for (auto take : {pa::take_bad_metadata_decode, pa::take_bad_metadata_prefill,
                          pa::take_bad_metadata_kv_write, pa::take_bad_metadata_kv_write_rope}) {
            int bad = 0;
            if (take(&bad) != hipSuccess) return PA_ELAUNCH;
            any |= bad;
        }
        return any ? PA_EDATA : PA_OK;
    }
}

}  // namespace

extern "C" {

const char* paged_attn_status_string(int status) {
    switch (status) {
        case PA_OK: return "ok";
        case PA_EINVAL: return "invalid argument";
        case PA_EUNSUPPORTED: return "unsupported configuration";
        case PA_ELAUNCH: return "kernel launch failed";
        case PA_EDATA: return "device metadata out of range (checked build)";
        case PA_ESCRATCH: return "larger than the fixed no-allocation workspace";
        default: return "unknown status";
    }
}

size_t paged_attn_decode_workspace_bytes(int num_seqs, int num_q_heads, int head_dim,
                                         int num_splits) {
    if (num_seqs < 1 || num_q_heads < 1 || head_dim < 1 || num_splits < 1) return 0;
    const unsigned __int128 rows =
        (unsigned __int128)num_seqs * (unsigned __int128)num_q_heads * (unsigned)num_splits;
    const unsigned __int128 bytes = rows * (unsigned __int128)(head_dim + 2) * 4u;
    if (bytes > (unsigned __int128)SIZE_MAX / 2) return 0;
    return (size_t)bytes;
}

}  // extern "C"

namespace {

// Validation and argument packing shared by the two decode entry points.
int make_decode_args(const float* q, const void* k_pages, const void* v_pages, int kv_dtype,
                     const int32_t* page_table, const int32_t* context_lens, int num_seqs,
                     int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                     int num_pages, int max_pages_per_seq, float scale, int window,
                     int num_splits, float* partial_o, float* partial_ml, pa::DecodeArgs* out) {
    if (!q || !k_pages || !v_pages || !page_table || !context_lens || !partial_o || !partial_ml)
        return PA_EINVAL;
    int rc = check_pages(kv_dtype, num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                         max_pages_per_seq);
    if (rc != PA_OK) return rc;
    if (num_splits < 1) return PA_EINVAL;
    if (num_splits > kMaxSplits) return PA_EUNSUPPORTED;
    // head_dim 256 is built for 16-bit K/V (an f32 row slice would not fit the registers).
    if (head_dim == 256 && kv_dtype == PA_F32) return PA_EUNSUPPORTED;
    if (!isfinite(scale)) return PA_EINVAL;
    if (num_seqs > kMaxGridYZ) return PA_EUNSUPPORTED;
    if ((int64_t)num_seqs * max_pages_per_seq > kI32Max ||
        (int64_t)num_seqs * num_q_heads * num_splits * head_dim > kI32Max * 4LL)
        return PA_EINVAL;
    const int group = num_q_heads / num_kv_heads;
    const int max_heads = max_heads_per_wg(kv_dtype, head_dim);
    int head_groups = (group + max_heads - 1) / max_heads;
    // A grid with fewer workgroups than the device has CUs leaves CUs idle: then the query
    // heads of a KV head are spread over twice the workgroups.  Each reads that KV head's
    // rows; workgroups are dealt to the 8 XCDs in turn, so with a split count that is a
    // multiple of 8 the two workgroups of a split share an XCD and the second read mostly hits
    // its L2.  A head's column gives the same bits in any grouping, so the result is the same
    // to the bit.  Workgroups of fewer than 3 heads cost more in duplicated row reads than
    // they gain (measured: 8/2 heads at context 256 went 8.0 -> 8.4 us with groups of 2).
    if ((int64_t)num_seqs * num_kv_heads * head_groups * num_splits < compute_units() &&
        (group + 2 * head_groups - 1) / (2 * head_groups) >= 3)
        head_groups *= 2;
    const int heads_per_wg = (group + head_groups - 1) / head_groups;
    // Every head group serves at least one query head (9 heads in 4 groups would be 3, 3, 3
    // and an empty one): the count follows from the group size.
    head_groups = (group + heads_per_wg - 1) / heads_per_wg;
    if ((int64_t)num_kv_heads * head_groups > kMaxGridYZ) return PA_EUNSUPPORTED;
    // A batch whose sequences differ in length leaves the CUs that drew the long ones
    // streaming alone at the end.  On the matrix-core body (16-bit pools, head_dim 64 or 128),
    // a batch of up to kRankMax sequences whose table rows fit the staged table together, and
    // whose grid is resident at once (two workgroups per CU), is taken longest first, in
    // rounds of as many sequences as one workgroup per CU covers, every second round in
    // reverse: the two workgroups of a CU then hold a long and a short sequence.  The order
    // changes no bit of any sequence's result.  (A grid of several generations ranks nothing:
    // there the query, requested after the ranking, costs each workgroup a round trip.)
    int rank_round = 0;
    const int64_t per_seq = (int64_t)num_kv_heads * head_groups * num_splits;
    const int cus = compute_units();
    if (kv_dtype != PA_F32 && head_dim != 256 && num_seqs > 1 && num_seqs <= pa::kRankMax &&
        (int64_t)num_seqs * max_pages_per_seq <= pa::kDecodeTableCap && cus > 0 &&
        per_seq * num_seqs <= 2LL * cus)
        rank_round = (int)std::max<int64_t>(1, cus / per_seq);

    pa::DecodeArgs a = {};
    a.q = q;
    a.k_pages = k_pages;
    a.v_pages = v_pages;
    a.page_table = page_table;
    a.context_lens = context_lens;
    a.partial_o = partial_o;
    a.partial_ml = partial_ml;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.group = group;
    a.head_groups = head_groups;
    a.heads_per_wg = heads_per_wg;
    a.page_shift = ilog2(page_size);
    a.num_pages = num_pages;
    a.max_pages = max_pages_per_seq;
    a.num_splits = num_splits;
    a.window = window > 0 ? window : 0;
    a.qscale = scale * pa::kLog2e;
    a.rank_round = rank_round;
    *out = a;
    return PA_OK;
}

}  // namespace

extern "C" {

int paged_attn_decode(const float* q, const void* k_pages, const void* v_pages,
                      pa_dtype kv_dtype, const int32_t* page_table,
                      const int32_t* context_lens, int num_seqs, int num_q_heads,
                      int num_kv_heads, int head_dim, int page_size, int num_pages,
                      int max_pages_per_seq, float scale, int window, int num_splits,
                      float* partial_o, float* partial_ml, void* stream) {
    if (num_seqs < 0) return PA_EINVAL;
    if (num_seqs == 0) return PA_OK;
    pa::DecodeArgs a;
    int rc = make_decode_args(q, k_pages, v_pages, kv_dtype, page_table, context_lens, num_seqs,
                              num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                              max_pages_per_seq, scale, window, num_splits, partial_o, partial_ml, &a);
    if (rc != PA_OK) return rc;
    return launched(pa::launch_decode(a, kv_dtype, head_dim, false, (hipStream_t)stream),
                    stream);
}

size_t paged_attn_decode_fused_counters(int num_seqs, int num_q_heads, int num_kv_heads) {
    if (num_seqs < 1 || num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads)
        return 0;
    const int group = num_q_heads / num_kv_heads;
    const int head_groups = (group + kCounterHeads - 1) / kCounterHeads;
    return (size_t)num_seqs * num_kv_heads * head_groups * 2 * pa::kCounterStride;
}

int paged_attn_decode_fused(const float* q, const void* k_new, const void* v_new,
                            void* k_pages, void* v_pages, pa_dtype kv_dtype,
                            const int32_t* page_table, const int32_t* context_lens,
                            int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                            int page_size, int num_pages, int max_pages_per_seq, float scale,
                            int window, int num_splits, float* partial_o, float* partial_ml,
                            uint32_t* counters, float* out, void* stream) {
    if (num_seqs < 0) return PA_EINVAL;
    if (num_seqs == 0) return PA_OK;
    if (!k_new || !v_new || !counters || !out) return PA_EINVAL;
    pa::DecodeArgs a;
    int rc = make_decode_args(q, k_pages, v_pages, kv_dtype, page_table, context_lens, num_seqs,
                              num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                              max_pages_per_seq, scale, window, num_splits, partial_o, partial_ml, &a);
    if (rc != PA_OK) return rc;
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_pages_w = k_pages;
    a.v_pages_w = v_pages;
    a.counters = counters;
    a.out = out;
    return launched(pa::launch_decode(a, kv_dtype, head_dim, true, (hipStream_t)stream),
                    stream);
}

size_t paged_attn_noalloc_scratch_bytes(void) { return pa::kNoallocScratchBytes; }

int paged_attn_decode_fused_noalloc(const float* q, const void* k_new, const void* v_new,
                                    void* k_pages, void* v_pages, pa_dtype kv_dtype,
                                    const int32_t* page_table, const int32_t* context_lens,
                                    int num_seqs, int num_q_heads, int num_kv_heads,
                                    int head_dim, int page_size, int num_pages,
                                    int max_pages_per_seq, float scale, int window,
                                    int num_splits, float* out, void* stream) {
    if (num_seqs < 0) return PA_EINVAL;
    if (num_seqs == 0) return PA_OK;
    if (!k_new || !v_new || !out) return PA_EINVAL;
    if (num_q_heads < 1 || num_kv_heads < 1 || head_dim < 1 || num_splits < 1 ||
        num_q_heads % num_kv_heads != 0)
        return PA_EINVAL;
    // Workspace layout inside the fixed array: the counters in a region of their own at the
    // start (zero when the library is loaded, and every call leaves them zero, whatever the
    // sizes of earlier calls), then partial_o and partial_ml, each at a 256-byte boundary.
    // Sizes are checked before anything touches the device.
    const size_t po_bytes =
        paged_attn_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, num_splits);
    const size_t n_counters = paged_attn_decode_fused_counters(num_seqs, num_q_heads,
                                                               num_kv_heads);
    if (po_bytes == 0 || n_counters == 0) return PA_EINVAL;
    if (n_counters * sizeof(uint32_t) > pa::kNoallocCounterBytes) return PA_ESCRATCH;
    const size_t o_bytes = po_bytes / (size_t)(head_dim + 2) * (size_t)head_dim;
    const size_t ml_bytes = po_bytes - o_bytes;
    auto up256 = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t o_off = pa::kNoallocCounterBytes;
    const size_t ml_off = up256(o_off + o_bytes);
    if (ml_off + ml_bytes > pa::kNoallocScratchBytes) return PA_ESCRATCH;
    void* base = nullptr;
    if (pa::noalloc_scratch(&base) != hipSuccess) return PA_ELAUNCH;
    char* ws = static_cast<char*>(base);
    return paged_attn_decode_fused(q, k_new, v_new, k_pages, v_pages, kv_dtype, page_table,
                                   context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                   page_size, num_pages, max_pages_per_seq, scale, window,
                                   num_splits, reinterpret_cast<float*>(ws + o_off),
                                   reinterpret_cast<float*>(ws + ml_off),
                                   reinterpret_cast<uint32_t*>(ws), out, stream);
}

int paged_attn_combine(const float* partial_o, const float* partial_ml, int num_seqs,
                       int num_q_heads, int head_dim, int num_splits, float* out,
                       void* stream) {
    if (num_seqs < 0 || num_q_heads < 1 || num_splits < 1 || head_dim < 1) return PA_EINVAL;
    if (num_seqs == 0) return PA_OK;
    if (!partial_o || !partial_ml || !out) return PA_EINVAL;
    if (head_dim != 64 && head_dim != 128 && head_dim != 256) return PA_EUNSUPPORTED;
    if (num_splits > kMaxSplits) return PA_EUNSUPPORTED;
    if ((int64_t)num_seqs * num_q_heads > kI32Max / 32) return PA_EINVAL;
    pa::CombineArgs a;
    a.partial_o = partial_o;
    a.partial_ml = partial_ml;
    a.out = out;
    a.rows = num_seqs * num_q_heads;
    a.num_splits = num_splits;
    return launched(pa::launch_combine(a, head_dim, (hipStream_t)stream), stream);
}

int paged_attn_prefill(const float* q, const void* k_pages, const void* v_pages,
                       pa_dtype kv_dtype, const int32_t* page_table, const int32_t* seg_desc,
                       int num_segs, int num_tables, int total_tokens, int max_chunk_len,
                       int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                       int num_pages, int max_pages_per_seq, float scale, float* out,
                       void* stream) {
    if (num_segs < 0 || max_chunk_len < 0 || total_tokens < 0) return PA_EINVAL;
    if (num_segs == 0 || max_chunk_len == 0 || total_tokens == 0) return PA_OK;
    if (!q || !k_pages || !v_pages || !page_table || !seg_desc || !out) return PA_EINVAL;
    int rc = check_pages(kv_dtype, num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                         max_pages_per_seq,
                         /*allow_d256=*/false);
    if (rc != PA_OK) return rc;
    if (num_tables < 1) return PA_EINVAL;
    if (!isfinite(scale)) return PA_EINVAL;
    if (num_segs > kMaxGridYZ || num_q_heads > kMaxGridYZ) return PA_EUNSUPPORTED;
    if ((int64_t)num_tables * max_pages_per_seq > kI32Max ||
        (int64_t)total_tokens * num_q_heads * head_dim > kI32Max * 4LL)
        return PA_EINVAL;
    pa::PrefillArgs a;
    a.q = q;
    a.k_pages = k_pages;
    a.v_pages = v_pages;
    a.page_table = page_table;
    a.seg_desc = seg_desc;
    a.out = out;
    a.num_segs = num_segs;
    a.num_tables = num_tables;
    a.total_tokens = total_tokens;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.group = num_q_heads / num_kv_heads;
    a.page_shift = ilog2(page_size);
    a.num_pages = num_pages;
    a.max_pages = max_pages_per_seq;
    a.qscale = scale * pa::kLog2e;
    const int q_blocks = (max_chunk_len + 15) / 16;
    if ((int64_t)q_blocks * num_q_heads > kI32Max) return PA_EUNSUPPORTED;
    a.q_blocks = q_blocks;
    // One prompt at head_dim 64, two workgroups per CU: the order alternates direction every
    // CU-count workgroups, so each CU's second workgroup is one of the lightest blocks.
    const int cus = compute_units();
    a.round_wgs = (num_segs == 1 && head_dim == 64) ? cus : 0;
    a.rank_segs = (num_segs >= 2 && num_segs <= pa::kRankSegs) ? 1 : 0;
    // Query blocks that hold rows: at most ceil(len / 16) per segment, and the segments
    // share the total_tokens packed rows without overlap.
    const int64_t blocks = std::min<int64_t>((int64_t)q_blocks * num_segs,
                                             ((int64_t)total_tokens + 15) / 16 + num_segs - 1);
    const bool dense = blocks * num_q_heads > 2 * (int64_t)cus;
    return launched(
        pa::launch_prefill(a, kv_dtype, head_dim, q_blocks, dense, (hipStream_t)stream), stream);
}

int kv_page_write(const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                  pa_dtype kv_dtype, const int32_t* page_table,
                  const int32_t* token_table_index, const int32_t* token_position,
                  int num_tokens, int num_tables, int num_kv_heads, int head_dim,
                  int page_size, int num_pages, int max_pages_per_seq, void* stream) {
    if (num_tokens < 0) return PA_EINVAL;
    if (num_tokens == 0) return PA_OK;
    if (!k_new || !v_new || !k_pages || !v_pages || !page_table || !token_table_index ||
        !token_position)
        return PA_EINVAL;
    int rc = check_pages(kv_dtype, num_kv_heads, num_kv_heads, head_dim, page_size, num_pages,
                         max_pages_per_seq);
    if (rc != PA_OK) return rc;
    if (num_tables < 1) return PA_EINVAL;
    if ((int64_t)num_tables * max_pages_per_seq > kI32Max) return PA_EINVAL;
    const int64_t row_bytes = (int64_t)num_kv_heads * head_dim * elem_bytes(kv_dtype);
    if (row_bytes > kI32Max) return PA_EINVAL;
    const int row_vec16 = (int)(row_bytes / 16);
    if (((int64_t)num_tokens * row_vec16 + 255) / 256 > kI32Max) return PA_EINVAL;
    pa::KvWriteArgs a;
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_pages = k_pages;
    a.v_pages = v_pages;
    a.page_table = page_table;
    a.token_table_index = token_table_index;
    a.token_position = token_position;
    a.num_tokens = num_tokens;
    a.num_tables = num_tables;
    a.row_vec16 = row_vec16;
    a.page_shift = ilog2(page_size);
    a.num_pages = num_pages;
    a.max_pages = max_pages_per_seq;
    return launched(pa::launch_kv_write(a, (hipStream_t)stream), stream);
}

int kv_page_write_rope(const float* k_new, const float* v_new, void* k_pages, void* v_pages,
                       pa_dtype kv_dtype, const int32_t* page_table,
                       const int32_t* token_table_index, const int32_t* token_position,
                       const float* inv_freq, pa_rope_style style, float* q, int num_q_heads,
                       int num_tokens, int num_tables, int num_kv_heads, int head_dim,
                       int page_size, int num_pages, int max_pages_per_seq, void* stream) {
    if (num_tokens < 0) return PA_EINVAL;
    if (num_tokens == 0) return PA_OK;
    if (!k_new || !v_new || !k_pages || !v_pages || !page_table || !token_table_index ||
        !token_position || !inv_freq)
        return PA_EINVAL;
    if (style != PA_ROPE_ADJACENT && style != PA_ROPE_HALVES) return PA_EINVAL;
    int rc = check_pages(kv_dtype, num_kv_heads, num_kv_heads, head_dim, page_size, num_pages,
                         max_pages_per_seq);
    if (rc != PA_OK) return rc;
    if (num_tables < 1) return PA_EINVAL;
    if (q && num_q_heads < 1) return PA_EINVAL;
    if ((int64_t)num_tables * max_pages_per_seq > kI32Max) return PA_EINVAL;
    const int64_t heads = (int64_t)num_kv_heads + (q ? num_q_heads : 0);
    if ((int64_t)num_tokens * heads * head_dim > kI32Max * 8LL) return PA_EINVAL;
    pa::KvRopeArgs a;
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_pages = k_pages;
    a.v_pages = v_pages;
    a.page_table = page_table;
    a.token_table_index = token_table_index;
    a.token_position = token_position;
    a.inv_freq = inv_freq;
    a.q = q;
    a.num_tokens = num_tokens;
    a.num_tables = num_tables;
    a.num_kv_heads = num_kv_heads;
    a.num_q_heads = q ? num_q_heads : 0;
    a.head_dim = head_dim;
    a.style = (int)style;
    a.page_shift = ilog2(page_size);
    a.num_pages = num_pages;
    a.max_pages = max_pages_per_seq;
    return launched(pa::launch_kv_write_rope(a, kv_dtype, (hipStream_t)stream), stream);
}

}  // extern "C"
