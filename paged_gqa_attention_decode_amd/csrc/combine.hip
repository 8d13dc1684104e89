// combine.hip — log-sum-exp merge of the split partials into the decode output.
//
// Method (crucible README, "Split-position attention": a second kernel rescales every
// chunk by exp(m_chunk - m_global) and merges; minfer 71 "D3-6", 3.2 Excerpt F: idle splits
// carry max = -inf, sum = 0 and get zero weight).
//
// gfx950 mapping: D/4 lanes own one (sequence, head) row, one float4 of the output each;
// a 256-thread workgroup merges 256/(D/4) rows (merge_row in common.h: the splits are read
// in chunks of 32 whose loads are all in flight together; each split's weight is computed
// once, by the lane that loaded its (m, l), and shared with the row's other lanes through
// LDS; a running maximum rescales the accumulators when a later chunk raises it; one
// division at the end).  The partials come from the caller, so an idle split's O may hold
// anything: its terms are skipped by select.
#include "common.h"

namespace pa {
namespace {

template <int D>
__global__ void __launch_bounds__(256) combine_kernel(CombineArgs a) {
    constexpr int TPR = D / 4;        // threads per row
    constexpr int RPB = 256 / TPR;    // rows per workgroup
    __shared__ float2 s_w[RPB][kMergeChunk];
    const int rr = (int)threadIdx.x / TPR;
    const int row = blockIdx.x * RPB + rr;
    const int c = threadIdx.x % TPR;
    if (row >= a.rows) return;
    const int S = a.num_splits;
    const float2* ml = reinterpret_cast<const float2*>(a.partial_ml) + (size_t)row * S;
    const float4* po = reinterpret_cast<const float4*>(a.partial_o) + (size_t)row * S * TPR + c;
    const PlainPartials src{ml, po, TPR};
    reinterpret_cast<float4*>(a.out)[(size_t)row * TPR + c] =
        merge_row<TPR, false>(src, S, c, s_w[rr]);
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, int head_dim, hipStream_t stream) {
    const int rpb = 256 / (head_dim / 4);
    const dim3 grid((a.rows + rpb - 1) / rpb);
    if (head_dim == 64)
        hipLaunchKernelGGL(combine_kernel<64>, grid, dim3(256), 0, stream, a);
    else if (head_dim == 128)
        hipLaunchKernelGGL(combine_kernel<128>, grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(combine_kernel<256>, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pa
