// decode.hip — split-KV paged decode: per-split partial softmax for all query heads of one
// KV head.
//
// Method (crucible README, "Split-position attention": grid over heads and context chunks,
// each block reducing one chunk to a partial softmax; minfer 71 "D3-6 GQA q-head batched
// attention", 3.2 Excerpt A: chunk = ceil(nkv / splits) and the split's row range; section 2:
// one block per KV head serving all of its query heads reads each K/V row once).
//
// gfx950 mapping
//   grid  (num_splits, num_kv_heads * head_groups, num_seqs); one workgroup of `waves`
//         64-lane waves serves up to GH query heads of one KV head over one split.
//   rows  a K or V row is D * elt bytes (256 B for D=128 f16/bf16 and D=64 f32).  LPR lanes
//         cover one row with one 16-byte load each, so one wave-wide load fetches RPI = 64/LPR
//         rows.  Each lane group (LPR lanes) keeps its own online-softmax stream per head.
//   window each wave takes U rows per lane group (RPI*U rows) and issues every K and V load of
//         the window before the first dependent instruction (the whole-window staging of the
//         minfer 75 "D4-3" page, 3.2 Excerpt A/C); the window max gives one rescale per window
//         (minfer D3-6, 3.2 Excerpt B).
//   dots  each lane multiplies its slice for all GH heads; DPP row operations reduce the
//         partial dots inside the lane group; every lane reduces (the validity select comes
//         after the reduction, the D3-6 pitfall about divergent shuffles).
//   table the sequence's page-table row (or a slice of it) is staged in LDS once; page ids are
//         clamped into [0, num_pages) as they are staged.
//   merge lane groups merge by shuffles, waves through LDS; the workgroup writes the split's
//         (m, l) in natural-log units and the unnormalised O.
#include "common.h"

namespace pa {
namespace {

constexpr int kMaxWaves = 8;
constexpr int kTableCap = 1024;  // page-table entries staged in LDS at a time
constexpr int kWindowRows = 4;   // U: rows per lane group per window

template <typename KV, int D, int GH>
__global__ void __launch_bounds__(kMaxWaves * 64) decode_split_kernel(DecodeArgs a) {
    using T = typename KV::storage;
    constexpr int EPL = 16 / KV::kBytes;  // elements per lane load
    constexpr int LPR = D / EPL;          // lanes per row
    constexpr int RPI = 64 / LPR;         // rows per wave-wide load
    constexpr int U = kWindowRows;
    constexpr int WROWS = RPI * U;        // rows per wave per window
    static_assert(LPR >= 1 && LPR <= 64 && (64 % LPR) == 0, "row must map onto a wave");

    __shared__ int s_tbl[kTableCap];
    __shared__ float s_m[kMaxWaves][GH];
    __shared__ float s_l[kMaxWaves][GH];
    __shared__ float s_o[kMaxWaves][GH][D];

    const int nthreads = blockDim.x;
    const int nwaves = nthreads >> 6;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int lg = lane / LPR;  // row slot within a wave-wide load
    const int li = lane % LPR;  // 16-byte column within the row

    const int split = blockIdx.x;
    const int kvh = blockIdx.y / a.head_groups;
    const int hg = blockIdx.y % a.head_groups;
    const int b = blockIdx.z;
    const int h0 = kvh * a.group + hg * a.heads_per_wg;
    const int nh = min(GH, a.group - hg * a.heads_per_wg);

    // Stage the whole page-table row when it fits: independent of the context length, so
    // this load overlaps the length load instead of following it.
    const int32_t* trow = a.page_table + (size_t)b * a.max_pages;
    const bool whole_row = a.max_pages <= kTableCap;
    if (whole_row) {
        for (int i = tid; i < a.max_pages; i += nthreads)
            s_tbl[i] = clampi(trow[i], 0, a.num_pages - 1);
    }

    const int cap = a.max_pages << a.page_shift;
    const int ctx = clampi(a.context_lens[b], 0, cap);
    const int S = a.num_splits;
    const int chunk = (ctx + S - 1) / S;
    const int lo = min(split * chunk, ctx);
    const int hi = min(lo + chunk, ctx);

    // Query slices, pre-multiplied by scale*log2(e) so that scores are in base-2 units.
    float qv[GH][EPL];
#pragma unroll
    for (int j = 0; j < GH; ++j) {
        const int h = h0 + min(j, nh - 1);  // padded heads repeat the last real one
        const float* qp = a.q + ((size_t)b * a.num_q_heads + h) * D + li * EPL;
#pragma unroll
        for (int e = 0; e < EPL; e += 4) {
            const float4 t = *reinterpret_cast<const float4*>(qp + e);
            qv[j][e + 0] = t.x * a.qscale;
            qv[j][e + 1] = t.y * a.qscale;
            qv[j][e + 2] = t.z * a.qscale;
            qv[j][e + 3] = t.w * a.qscale;
        }
    }

    float m[GH], l[GH], o[GH][EPL];
#pragma unroll
    for (int j = 0; j < GH; ++j) {
        m[j] = -INFINITY;
        l[j] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[j][e] = 0.f;
    }

    const size_t slot_stride = (size_t)a.num_kv_heads * D;  // elements between slots
    const T* kbase = reinterpret_cast<const T*>(a.k_pages) + (size_t)kvh * D + li * EPL;
    const T* vbase = reinterpret_cast<const T*>(a.v_pages) + (size_t)kvh * D + li * EPL;
    const int pshift = a.page_shift;
    const int pmask = (1 << pshift) - 1;

    // Rows [r0, r1) of this split; page ids come from s_tbl[(t >> pshift) - pg0].
    auto process = [&](int r0, int r1, int pg0) {
        for (int w0 = r0 + wave * WROWS; w0 < r1; w0 += nwaves * WROWS) {
            uint4 kr[U], vr[U];
            bool ok[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int t = w0 + u * RPI + lg;
                ok[u] = t < r1;
                kr[u] = make_uint4(0, 0, 0, 0);
                vr[u] = make_uint4(0, 0, 0, 0);
                if (ok[u]) {
                    const size_t page = (size_t)s_tbl[(t >> pshift) - pg0];
                    const size_t row = ((page << pshift) | (size_t)(t & pmask)) * slot_stride;
                    kr[u] = *reinterpret_cast<const uint4*>(kbase + row);
                    vr[u] = *reinterpret_cast<const uint4*>(vbase + row);
                }
            }
            float sc[U][GH];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float kf[EPL];
                widen16<KV>(kr[u], kf);
#pragma unroll
                for (int j = 0; j < GH; ++j) {
                    float d = 0.f;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) d = fmaf(qv[j][e], kf[e], d);
                    d = group_sum<LPR>(d);
                    sc[u][j] = ok[u] ? d : -INFINITY;
                }
            }
            float p[U][GH];
#pragma unroll
            for (int j = 0; j < GH; ++j) {
                float mx = m[j];
#pragma unroll
                for (int u = 0; u < U; ++u) mx = fmaxf(mx, sc[u][j]);
                const float ms = (mx == -INFINITY) ? 0.f : mx;
                const float alpha = fast_exp2(m[j] - ms);
                float ps = 0.f;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    p[u][j] = fast_exp2(sc[u][j] - ms);
                    ps += p[u][j];
                }
                l[j] = fmaf(l[j], alpha, ps);
#pragma unroll
                for (int e = 0; e < EPL; ++e) o[j][e] *= alpha;
                m[j] = mx;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float vf[EPL];
                widen16<KV>(vr[u], vf);
#pragma unroll
                for (int j = 0; j < GH; ++j) {
#pragma unroll
                    for (int e = 0; e < EPL; ++e) o[j][e] = fmaf(p[u][j], vf[e], o[j][e]);
                }
            }
        }
    };

    if (whole_row) {
        __syncthreads();
        if (lo < hi) process(lo, hi, 0);
    } else if (lo < hi) {
        const int first = lo >> pshift;
        const int last = (hi - 1) >> pshift;
        for (int pg0 = first; pg0 <= last; pg0 += kTableCap) {
            const int n = min(kTableCap, last - pg0 + 1);
            __syncthreads();
            for (int i = tid; i < n; i += nthreads)
                s_tbl[i] = clampi(trow[pg0 + i], 0, a.num_pages - 1);
            __syncthreads();
            process(max(lo, pg0 << pshift), min(hi, (pg0 + n) << pshift), pg0);
        }
    }

    // Merge the lane groups of this wave (same rows' heads, different rows).
#pragma unroll
    for (int j = 0; j < GH; ++j) {
        float mw = m[j];
#pragma unroll
        for (int off = LPR; off < 64; off <<= 1) mw = fmaxf(mw, __shfl_xor(mw, off));
        const float ms = (mw == -INFINITY) ? 0.f : mw;
        const float f = fast_exp2(m[j] - ms);
        float lw = l[j] * f;
#pragma unroll
        for (int off = LPR; off < 64; off <<= 1) lw += __shfl_xor(lw, off);
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            float x = o[j][e] * f;
#pragma unroll
            for (int off = LPR; off < 64; off <<= 1) x += __shfl_xor(x, off);
            o[j][e] = x;
        }
        m[j] = mw;
        l[j] = lw;
    }
    if (lg == 0) {
#pragma unroll
        for (int j = 0; j < GH; ++j)
#pragma unroll
            for (int e = 0; e < EPL; ++e) s_o[wave][j][li * EPL + e] = o[j][e];
    }
    if (lane == 0) {
#pragma unroll
        for (int j = 0; j < GH; ++j) {
            s_m[wave][j] = m[j];
            s_l[wave][j] = l[j];
        }
    }
    __syncthreads();

    // Merge the waves and write the split's partial.
    for (int idx = tid; idx < GH * D; idx += nthreads) {
        const int j = idx / D;
        const int d = idx - j * D;
        if (j >= nh) continue;
        float M = -INFINITY;
        for (int w = 0; w < nwaves; ++w) M = fmaxf(M, s_m[w][j]);
        const float ms = (M == -INFINITY) ? 0.f : M;
        float L = 0.f, O = 0.f;
        for (int w = 0; w < nwaves; ++w) {
            const float f = fast_exp2(s_m[w][j] - ms);
            L = fmaf(s_l[w][j], f, L);
            O = fmaf(s_o[w][j][d], f, O);
        }
        const size_t slot = ((size_t)b * a.num_q_heads + h0 + j) * S + split;
        a.partial_o[slot * D + d] = O;
        if (d == 0) {
            a.partial_ml[2 * slot] = (L > 0.f) ? M * kLn2 : -INFINITY;
            a.partial_ml[2 * slot + 1] = L;
        }
    }
}

template <typename KV, int D>
hipError_t launch_typed(const DecodeArgs& a, int waves, hipStream_t stream) {
    const dim3 grid(a.num_splits, a.num_kv_heads * a.head_groups, a.num_seqs);
    const dim3 block(waves * 64);
    switch (a.heads_per_wg) {
#define PA_DECODE_CASE(GH)                                                         \
    case GH:                                                                       \
        hipLaunchKernelGGL((decode_split_kernel<KV, D, GH>), grid, block, 0, stream, a); \
        break;
        PA_DECODE_CASE(1)
        PA_DECODE_CASE(2)
        PA_DECODE_CASE(3)
        PA_DECODE_CASE(4)
        PA_DECODE_CASE(5)
        PA_DECODE_CASE(6)
        PA_DECODE_CASE(7)
        PA_DECODE_CASE(8)
#undef PA_DECODE_CASE
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int kv_dtype, int head_dim, int waves,
                         hipStream_t stream) {
    if (waves < 1 || waves > kMaxWaves) return hipErrorInvalidValue;
    if (head_dim == 64) {
        if (kv_dtype == 0) return launch_typed<F32, 64>(a, waves, stream);
        if (kv_dtype == 1) return launch_typed<F16, 64>(a, waves, stream);
        return launch_typed<BF16, 64>(a, waves, stream);
    }
    if (kv_dtype == 0) return launch_typed<F32, 128>(a, waves, stream);
    if (kv_dtype == 1) return launch_typed<F16, 128>(a, waves, stream);
    return launch_typed<BF16, 128>(a, waves, stream);
}

}  // namespace pa
