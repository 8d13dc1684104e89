// combine.hip — log-sum-exp merge of the split partials into the decode output.
//
// Method (crucible README, "Split-position attention": a second kernel rescales every
// chunk by exp(m_chunk - m_global) and merges; minfer 71 "D3-6", 3.2 Excerpt F: idle splits
// carry max = -inf, sum = 0 and get zero weight).
//
// gfx950 mapping: D/4 lanes own one (sequence, head) row, one float4 of the output each;
// a 256-thread workgroup merges 256/(D/4) rows.  The splits are read in chunks of 32 whose
// loads are all in flight together; a running maximum rescales the accumulators when a
// later chunk raises it, and the result is divided once at the end.
#include "common.h"

namespace pa {
namespace {

constexpr int kChunk = 32;  // splits whose partials are in flight at once

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

    // One pass with a running maximum: every load of a chunk is issued before any of its
    // values is used, so a chunk costs one memory round trip.
    float M = -INFINITY;  // natural-log units
    float L = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = 0; s0 < S; s0 += kChunk) {
        float2 v[kChunk];
        float4 o[kChunk];
#pragma unroll
        for (int k = 0; k < kChunk; ++k) {
            const int s = min(s0 + k, S - 1);
            v[k] = ml[s];
            o[k] = po[(size_t)s * TPR];
        }
        float cm = -INFINITY;
#pragma unroll
        for (int k = 0; k < kChunk; ++k) {
            const bool live = (s0 + k < S) && v[k].y > 0.f;
            cm = fmaxf(cm, live ? v[k].x : -INFINITY);
        }
        if (cm == -INFINITY) continue;             // nothing live in this chunk
        const float Mn = fmaxf(M, cm);
        const float r = fast_exp2((M - Mn) * kLog2e);  // 0 while M is still -inf
        L *= r;
        acc.x *= r;
        acc.y *= r;
        acc.z *= r;
        acc.w *= r;
#pragma unroll
        for (int k = 0; k < kChunk; ++k) {
            const bool live = (s0 + k < S) && v[k].y > 0.f;
            const float w = live ? fast_exp2((v[k].x - Mn) * kLog2e) : 0.f;
            // idle splits contribute nothing, whatever their O holds
            L = live ? fmaf(w, v[k].y, L) : L;
            acc.x = live ? fmaf(w, o[k].x, acc.x) : acc.x;
            acc.y = live ? fmaf(w, o[k].y, acc.y) : acc.y;
            acc.z = live ? fmaf(w, o[k].z, acc.z) : acc.z;
            acc.w = live ? fmaf(w, o[k].w, acc.w) : acc.w;
        }
        M = Mn;
    }
    float4 res = make_float4(0.f, 0.f, 0.f, 0.f);
    if (L > 0.f) res = make_float4(acc.x / L, acc.y / L, acc.z / L, acc.w / L);
    reinterpret_cast<float4*>(a.out)[(size_t)row * TPR + c] = res;
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
