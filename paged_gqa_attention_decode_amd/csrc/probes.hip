// probes.hip — measurement kernels for bench.py, built as libpaged_attn_probes.so beside the
// attention library and not part of its C ABI.  They bound what a decode launch can take:
//
//   pa_probe_read_walk   reads exactly the K/V rows a decode launch reads, in the same
//                        decomposition (one 4-wave workgroup per split, KV head and sequence;
//                        32-key tiles dealt to the waves in turn; 16-byte lane loads; the
//                        sequence's page ids staged in LDS; the split rule chunk = ceil(n / S)
//                        over the attended positions; with rank_round > 0 the batch taken in
//                        the decode's ranked order), with no arithmetic and no stores: the
//                        time of the bytes alone in that order.
//   pa_probe_read_plain  reads two contiguous regions of the same total size, front to back,
//                        from enough workgroups to fill the chip.
//   pa_probe_empty       an empty kernel over a given number of workgroups: the cost of a launch.
//
// The loaded values are XOR-folded and stored only if the fold equals a constant, so the
// loads stay live.  Every page id is clamped into [0, num_pages) and every key into the split,
// so each access stays inside the pools whatever the table holds.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kWalkThreads = 256;     // 4 waves
constexpr int kWalkTableCap = 4096;   // page ids of one sequence staged in LDS
constexpr uint32_t kNever = 0x9E3779B9u;

__device__ __forceinline__ uint32_t fold(uint4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

// P = 16-byte pieces of one K/V row of one KV head (row bytes / 16): 8, 16 or 32.
template <int P>
__global__ void __launch_bounds__(kWalkThreads) read_walk(
    const uint4* __restrict__ kp, const uint4* __restrict__ vp, const int32_t* __restrict__ table,
    const int32_t* __restrict__ ctxs, int S, int Hkv, int page_shift, int max_pages,
    int num_pages, int window, int rank_round, uint32_t* sink) {
    constexpr int RPI = 64 / P;         // rows per wave instruction
    constexpr int NI = 32 / RPI;        // instructions per 32-key tile, for K and for V
    __shared__ int s_tbl[kWalkTableCap];
    const int split = blockIdx.x;
    const int kvh = blockIdx.y;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int cap = max_pages << page_shift;
    int b = blockIdx.z;
    if (rank_round > 0) {
        // The decode's order: sequences ranked by attended length (longest first, ties by
        // index), slot z taking rank z within rounds of rank_round, every second one reversed.
        const int B = gridDim.z;
        int att = -1;
        if (lane < B) {
            att = min(max(ctxs[lane], 0), cap);
            if (window > 0) att = min(att, window);
        }
        int rank = 0;
        for (int j = 0; j < B; ++j) {
            const int other = __builtin_amdgcn_readlane(att, j);
            rank += (other > att || (other == att && j < lane)) ? 1 : 0;
        }
        const int z = blockIdx.z;
        const int rnd = z / rank_round;
        const int in_round = min(rank_round, B - rnd * rank_round);
        const int want = rnd * rank_round +
                         ((rnd & 1) ? in_round - 1 - (z - rnd * rank_round) : z - rnd * rank_round);
        const unsigned long long hit = __builtin_amdgcn_ballot_w64(lane < B && rank == want);
        b = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(hit));
    }
    const int32_t* trow = table + (size_t)b * max_pages;
    for (int i = tid; i < max_pages; i += kWalkThreads)
        s_tbl[i] = min(max(trow[i], 0), num_pages - 1);
    const int n = min(max(ctxs[b], 0), cap);
    __syncthreads();
    const int w0 = (window > 0 && n > window) ? n - window : 0;
    const int n_att = n - w0;
    const int chunk = (n_att + S - 1) / S;
    const int lo = w0 + min(split * chunk, n_att);
    const int hi = min(lo + chunk, n);
    const int ntiles = (hi - lo + 31) / 32;
    const int r = lane / P;
    const int piece = lane % P;
    const size_t slot = (size_t)Hkv * P;  // 16-byte pieces between consecutive slots
    const int pmask = (1 << page_shift) - 1;
    uint32_t acc = 0;
    for (int t = wave; t < ntiles; t += kWalkThreads / 64) {
        uint4 k[NI], v[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int key = min(lo + t * 32 + i * RPI + r, hi - 1);
            const size_t row = (((size_t)s_tbl[key >> page_shift] << page_shift) |
                                (size_t)(key & pmask)) * slot + (size_t)kvh * P + piece;
            k[i] = kp[row];
            v[i] = vp[row];
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) acc ^= fold(k[i]) ^ fold(v[i]);
    }
    if (acc == kNever) sink[0] = acc;
}

__global__ void __launch_bounds__(256) read_plain(const uint4* __restrict__ a,
                                                  const uint4* __restrict__ b, size_t n16,
                                                  uint32_t* sink) {
    uint32_t acc = 0;
    const size_t stride = (size_t)gridDim.x * 256 * 4;
    for (size_t i = (size_t)blockIdx.x * 1024 + threadIdx.x; i < n16; i += stride) {
        uint4 x[4], y[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const size_t j = i + 256 * u;
            x[u] = (j < n16) ? a[j] : make_uint4(0, 0, 0, 0);
            y[u] = (j < n16) ? b[j] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) acc ^= fold(x[u]) ^ fold(y[u]);
    }
    if (acc == kNever) sink[blockIdx.x] = acc;
}

__global__ void empty_kernel() {}

}  // namespace

extern "C" {

// K/V pools [num_pages][page_size][num_kv_heads][head_dim] of elt_bytes-byte elements, a
// page table [num_seqs][max_pages], lengths [num_seqs], a window (0: none) and a split count,
// as a decode launch takes them; rank_round as the decode sets it for the same call (0: grid
// order; > 0 needs at most 64 sequences); sink: one writable 32-bit word.  Returns a
// hipError_t, or hipErrorInvalidValue for a shape the probe does not cover (rows of 128, 256
// or 512 bytes, at most 4096 table entries per sequence).
int pa_probe_read_walk(const void* k_pages, const void* v_pages, int elt_bytes,
                       const int32_t* page_table, const int32_t* context_lens, int num_seqs,
                       int num_kv_heads, int head_dim, int page_size, int num_pages,
                       int max_pages, int num_splits, int window, int rank_round,
                       uint32_t* sink, void* stream) {
    if (rank_round < 0 || (rank_round > 0 && num_seqs > 64)) return (int)hipErrorInvalidValue;
    if (!k_pages || !v_pages || !page_table || !context_lens || !sink || num_seqs < 1 ||
        num_kv_heads < 1 || num_kv_heads > 65535 || num_seqs > 65535 || num_pages < 1 ||
        max_pages < 1 || max_pages > kWalkTableCap || num_splits < 1 || page_size < 1 ||
        (page_size & (page_size - 1)) != 0 || elt_bytes < 1)
        return (int)hipErrorInvalidValue;
    int shift = 0;
    while ((1 << shift) < page_size) ++shift;
    const int pieces = head_dim * elt_bytes / 16;
    if (head_dim * elt_bytes != pieces * 16) return (int)hipErrorInvalidValue;
    const dim3 grid(num_splits, num_kv_heads, num_seqs);
    const hipStream_t s = (hipStream_t)stream;
    const uint4* kp = (const uint4*)k_pages;
    const uint4* vp = (const uint4*)v_pages;
    if (pieces == 8)
        hipLaunchKernelGGL(read_walk<8>, grid, dim3(kWalkThreads), 0, s, kp, vp, page_table,
                           context_lens, num_splits, num_kv_heads, shift, max_pages, num_pages,
                           window, rank_round, sink);
    else if (pieces == 16)
        hipLaunchKernelGGL(read_walk<16>, grid, dim3(kWalkThreads), 0, s, kp, vp, page_table,
                           context_lens, num_splits, num_kv_heads, shift, max_pages, num_pages,
                           window, rank_round, sink);
    else if (pieces == 32)
        hipLaunchKernelGGL(read_walk<32>, grid, dim3(kWalkThreads), 0, s, kp, vp, page_table,
                           context_lens, num_splits, num_kv_heads, shift, max_pages, num_pages,
                           window, rank_round, sink);
    else
        return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}

// Reads bytes (a multiple of 16) from each of a and b; sink: workgroups writable words.
int pa_probe_read_plain(const void* a, const void* b, size_t bytes, int workgroups,
                        uint32_t* sink, void* stream) {
    if (!a || !b || !sink || bytes % 16 != 0 || workgroups < 1)
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(read_plain, dim3(workgroups), dim3(256), 0, (hipStream_t)stream,
                       (const uint4*)a, (const uint4*)b, bytes / 16, sink);
    return (int)hipGetLastError();
}

int pa_probe_empty(int workgroups, void* stream) {
    if (workgroups < 1) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(empty_kernel, dim3(workgroups), dim3(256), 0, (hipStream_t)stream);
    return (int)hipGetLastError();
}

}  // extern "C"
