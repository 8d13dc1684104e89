// kv_write.hip — scatter new K/V rows into their pages (a byte copy; no conversion).
//
// Method (crucible README, "Paged KV cache and continuous batching": page term from the page
// table, slot = position & (page_size - 1); "What actually runs": persistent owner and
// absolute-position arrays route the K/V writes).
//
// gfx950 mapping: the rows of all KV heads of one token are contiguous both in the input
// [T][Hkv][D] and in the destination slot [page][slot][Hkv][D], so each lane copies one
// 16-byte vector of K and the same vector of V: fully coalesced 128-bit loads and stores.
#include "common.h"

namespace pa {

// Checked build: set when a token to be written names no table row, a position past the
// table's capacity or a logical page without a valid id.  A negative owner or position is
// an explicit skip, not an error.
__device__ int g_bad_metadata_kv_write;

namespace {

__global__ void __launch_bounds__(256) kv_write_kernel(KvWriteArgs a) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)a.num_tokens * a.row_vec16;
    if (idx >= total) return;
    const int i = (int)(idx / a.row_vec16);
    const int c = (int)(idx - (int64_t)i * a.row_vec16);
    const int owner = a.token_table_index[i];
    const int pos = a.token_position[i];
    if (owner < 0 || pos < 0) return;
    if (owner >= a.num_tables || pos >= (a.max_pages << a.page_shift)) {
        if (c == 0) mark_bad(&g_bad_metadata_kv_write);
        return;
    }
    const int page = a.page_table[(size_t)owner * a.max_pages + (pos >> a.page_shift)];
    if (page < 0 || page >= a.num_pages) {
        if (c == 0) mark_bad(&g_bad_metadata_kv_write);
        return;
    }
    const size_t slot = ((size_t)page << a.page_shift) | (size_t)(pos & ((1 << a.page_shift) - 1));
    const size_t dst = slot * a.row_vec16 + c;
    reinterpret_cast<uint4*>(a.k_pages)[dst] = reinterpret_cast<const uint4*>(a.k_new)[idx];
    reinterpret_cast<uint4*>(a.v_pages)[dst] = reinterpret_cast<const uint4*>(a.v_new)[idx];
}

}  // namespace

PA_DEFINE_TAKE_BAD_METADATA(take_bad_metadata_kv_write, g_bad_metadata_kv_write)

hipError_t launch_kv_write(const KvWriteArgs& a, hipStream_t stream) {
    const int64_t total = (int64_t)a.num_tokens * a.row_vec16;
    const dim3 grid((unsigned)((total + 255) / 256));
    hipLaunchKernelGGL(kv_write_kernel, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pa
