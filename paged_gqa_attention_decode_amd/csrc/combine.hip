// combine.hip — log-sum-exp merge of the split partials into the decode output.
//
// Method (crucible README, "Split-position attention": a second kernel rescales every
// chunk by exp(m_chunk - m_global) and merges; minfer 71 "D3-6", 3.2 Excerpt F: idle splits
// carry max = -inf, sum = 0 and get zero weight).
//
// gfx950 mapping: D/4 lanes own one (sequence, head) row, one float4 of the output each;
// a 256-thread workgroup merges 256/(D/4) rows.  Pass 1 finds the largest m over the live
// splits, pass 2 accumulates exp(m_s - M) * {l_s, O_s} and divides once.
#include "common.h"

namespace pa {
namespace {

template <int D>
__global__ void __launch_bounds__(256) combine_kernel(CombineArgs a) {
    constexpr int TPR = D / 4;        // threads per row
    constexpr int RPB = 256 / TPR;    // rows per workgroup
    const int row = blockIdx.x * RPB + (int)threadIdx.x / TPR;
    const int c = threadIdx.x % TPR;
    if (row >= a.rows) return;
    const int S = a.num_splits;
    const float2* ml = reinterpret_cast<const float2*>(a.partial_ml) + (size_t)row * S;
    const float4* po = reinterpret_cast<const float4*>(a.partial_o) + (size_t)row * S * TPR + c;

    float M = -INFINITY;
    for (int s = 0; s < S; ++s) {
        const float2 v = ml[s];
        if (v.y > 0.f) M = fmaxf(M, v.x);
    }
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float L = 0.f;
    if (M != -INFINITY) {
#pragma unroll 4
        for (int s = 0; s < S; ++s) {
            const float2 v = ml[s];
            if (v.y > 0.f) {
                const float w = fast_exp2((v.x - M) * kLog2e);
                const float4 o = po[(size_t)s * TPR];
                L = fmaf(w, v.y, L);
                acc.x = fmaf(w, o.x, acc.x);
                acc.y = fmaf(w, o.y, acc.y);
                acc.z = fmaf(w, o.z, acc.z);
                acc.w = fmaf(w, o.w, acc.w);
            }
        }
    }
    float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
    if (L > 0.f) r = make_float4(acc.x / L, acc.y / L, acc.z / L, acc.w / L);
    reinterpret_cast<float4*>(a.out)[(size_t)row * TPR + c] = r;
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, int head_dim, hipStream_t stream) {
    const int rpb = 256 / (head_dim / 4);
    const dim3 grid((a.rows + rpb - 1) / rpb);
    if (head_dim == 64)
        hipLaunchKernelGGL(combine_kernel<64>, grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(combine_kernel<128>, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pa
