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
//   merge lane groups merge with a DPP row rotation and LDS-crossbar lane exchanges (no LDS
//         storage), waves through LDS; the workgroup writes the split's (m, l) in
//         natural-log units and the unnormalised O.
#include <algorithm>

#include "common.h"

namespace pa {
namespace {

constexpr int kMaxWaves = 8;
constexpr int kTableCap = 1024;  // page-table entries staged in LDS at a time
constexpr int kWindowRows = 4;   // U: rows per lane group per window

constexpr int kStreamLds = 64 * 1024;  // LDS for stream states at the largest head group

template <typename KV, int D>
struct DecodeGeom {
    static constexpr int EPL = 16 / KV::kBytes;  // elements per lane load
    static constexpr int LPR = D / EPL;          // lanes per row
    static constexpr int RPI = 64 / LPR;         // rows per wave-wide load = streams per wave
    // Most waves per workgroup: every stream keeps up to 8 heads x D floats in LDS.
    static constexpr int kWaves = (kStreamLds / (8 * D * 4) / RPI) < kMaxWaves
                                      ? (kStreamLds / (8 * D * 4) / RPI)
                                      : kMaxWaves;
};

// Dynamic LDS of one workgroup: staged page ids, then per stream (wave x lane group) and
// head the running max m, the sum l, the merge factor f, and the D-wide accumulator.
__host__ __device__ constexpr size_t decode_lds_bytes(int streams, int gh, int d) {
    return (size_t)kTableCap * 4 + (size_t)streams * gh * 4 * 4 + (size_t)streams * gh * d * 4;
}

// A split partial leaves the workgroup by a plain store, or, when another workgroup of the
// same launch merges it, by a device-scope one (written through this XCD's L2).
template <bool COHERENT>
__device__ __forceinline__ void store_partial(float* p, float v) {
    if constexpr (COHERENT)
        __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        *p = v;
}

template <typename KV, int D, int GH, bool FUSED>
__device__ __forceinline__ void decode_body(const DecodeArgs& a) {
    using T = typename KV::storage;
    using G = DecodeGeom<KV, D>;
    constexpr int EPL = G::EPL;
    constexpr int LPR = G::LPR;
    constexpr int RPI = G::RPI;
    constexpr int U = kWindowRows;
    constexpr int WROWS = RPI * U;        // rows per wave per window
    // Registers of q and of the accumulators (2 GH EPL) plus two windows of K/V (16 U).
    constexpr bool kPrefetch = 2 * GH * EPL + 16 * U < 192;
    constexpr int TPT = kTableCap / 64;   // table entries staged per thread (>= 64 threads)
    static_assert(LPR >= 8 && LPR <= 64 && (64 % LPR) == 0, "row must map onto a wave");

    extern __shared__ __align__(16) float lds[];
    __shared__ int s_last;  // single-launch step: this workgroup finished the group's last split
    const int nthreads = blockDim.x;
    const int nwaves = nthreads >> 6;
    const int streams = nwaves * RPI;
    int* s_tbl = reinterpret_cast<int*>(lds);
    float* s_m = lds + kTableCap;          // [streams][GH]
    float* s_l = s_m + streams * GH;       // [streams][GH]
    float* s_f = s_l + streams * GH;       // [streams][GH]
    float* s_o = s_f + 2 * streams * GH;   // [streams][GH][D] (16-byte aligned)

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

    // Nothing here depends on the context length, so the page-table row, the length and the
    // query are requested together, the table first: the K/V loads wait only for the table,
    // and the query's round trip overlaps them.
    const int32_t* trow = a.page_table + (size_t)b * a.max_pages;
    const bool whole_row = a.max_pages <= kTableCap;
    int tv[TPT];
    if (whole_row) {
#pragma unroll
        for (int k = 0; k < TPT; ++k) {
            const int i = tid + k * nthreads;
            tv[k] = (i < a.max_pages) ? trow[i] : 0;
        }
    }
    const int cap = a.max_pages << a.page_shift;
    const int ctx = clampi(a.context_lens[b], 0, cap);
    float qv[GH][EPL];
#pragma unroll
    for (int j = 0; j < GH; ++j) {
        const int h = h0 + min(j, nh - 1);  // padded heads repeat the last real one
        const float* qp = a.q + ((size_t)b * a.num_q_heads + h) * D + li * EPL;
#pragma unroll
        for (int e = 0; e < EPL; e += 4) {
            const float4 t = *reinterpret_cast<const float4*>(qp + e);
            qv[j][e + 0] = t.x;
            qv[j][e + 1] = t.y;
            qv[j][e + 2] = t.z;
            qv[j][e + 3] = t.w;
        }
    }
    const int S = a.num_splits;
    const int chunk = (ctx + S - 1) / S;
    const int lo = min(split * chunk, ctx);
    const int hi = min(lo + chunk, ctx);
    if (whole_row) {
#pragma unroll
        for (int k = 0; k < TPT; ++k) {
            const int i = tid + k * nthreads;
            if (i < a.max_pages) s_tbl[i] = clampi(tv[k], 0, a.num_pages - 1);
        }
    }
    // Scores in base-2 units: q is scaled once by scale * log2(e) (here, after the table
    // staging, so the preamble does not wait for q's round trip).
#pragma unroll
    for (int j = 0; j < GH; ++j)
#pragma unroll
        for (int e = 0; e < EPL; ++e) qv[j][e] *= a.qscale;

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
    // Single-launch step: the current token (position ctx - 1) is read from k_new / v_new;
    // its pool slot is written by this launch and read by none of its workgroups.
    const int t_new = FUSED ? ctx - 1 : -1;
    const T* knew = nullptr;
    const T* vnew = nullptr;
    if constexpr (FUSED) {
        const size_t off = ((size_t)b * a.num_kv_heads + kvh) * D + li * EPL;
        knew = reinterpret_cast<const T*>(a.k_new) + off;
        vnew = reinterpret_cast<const T*>(a.v_new) + off;
    }

    // One window: U rows per lane group starting at w0, rows past r1 clamped onto row
    // r1 - 1 (a valid address, cache hits) and flagged, so no branch guards the loads.
    struct Window {
        uint4 k[U], v[U];
        bool ok[U];
    };
    auto load_window = [&](Window& W, int w0, int r1, int pg0) {
        int t[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int tt = w0 + u * RPI + lg;
            W.ok[u] = tt < r1;
            t[u] = min(tt, r1 - 1);
        }
        int pg[U];
#pragma unroll
        for (int u = 0; u < U; ++u) pg[u] = s_tbl[(t[u] >> pshift) - pg0];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t row = (((size_t)pg[u] << pshift) | (size_t)(t[u] & pmask)) * slot_stride;
            const T* kp = kbase + row;
            const T* vp = vbase + row;
            if constexpr (FUSED) {
                kp = (t[u] == t_new) ? knew : kp;
                vp = (t[u] == t_new) ? vnew : vp;
            }
            W.k[u] = *reinterpret_cast<const uint4*>(kp);
            W.v[u] = *reinterpret_cast<const uint4*>(vp);
        }
    };
    auto compute_window = [&](const Window& W) {
        float sc[U][GH];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float kf[EPL];
            widen16<KV>(W.k[u], kf);
#pragma unroll
            for (int j = 0; j < GH; ++j) {
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) d = fmaf(qv[j][e], kf[e], d);
                d = group_sum<LPR>(d);
                sc[u][j] = W.ok[u] ? d : -INFINITY;
            }
        }
        float p[U][GH];
        float alpha[GH];
        bool moved = false;  // some running maximum of this lane changed
#pragma unroll
        for (int j = 0; j < GH; ++j) {
            float mx = m[j];
#pragma unroll
            for (int u = 0; u < U; ++u) mx = fmaxf(mx, sc[u][j]);
            const float ms = (mx == -INFINITY) ? 0.f : mx;
            alpha[j] = fast_exp2(m[j] - ms);
            moved |= mx != m[j];
            float ps = 0.f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                p[u][j] = fast_exp2(sc[u][j] - ms);
                ps += p[u][j];
            }
            l[j] = fmaf(l[j], alpha[j], ps);
            m[j] = mx;
        }
        // Where no running maximum of the wave moved, every alpha is exp2(0) = 1 (or the
        // accumulator is still all zeros), so the rescale is skipped without changing a bit.
        if (__builtin_amdgcn_ballot_w64(moved) != 0) {
#pragma unroll
            for (int j = 0; j < GH; ++j)
#pragma unroll
                for (int e = 0; e < EPL; ++e) o[j][e] *= alpha[j];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float vf[EPL];
            widen16<KV>(W.v[u], vf);
#pragma unroll
            for (int j = 0; j < GH; ++j) {
#pragma unroll
                for (int e = 0; e < EPL; ++e) o[j][e] = fmaf(p[u][j], vf[e], o[j][e]);
            }
        }
    };
    // Rows [r0, r1) of this split (r0 < r1).  Two register windows alternate: the next
    // window's loads are issued before the current window is computed.  Where q and the
    // accumulators already take most registers (8 heads of 16-bit K/V), one window is
    // loaded at a time and the second wave per SIMD that this frees room for hides the
    // latency instead; the windows, and so the arithmetic, are the same either way.
    auto process = [&](int r0, int r1, int pg0) {
        const int step = nwaves * WROWS;
        int w = r0 + wave * WROWS;
        if constexpr (!kPrefetch) {
            for (; w < r1; w += step) {
                Window A;
                load_window(A, w, r1, pg0);
                compute_window(A);
            }
            return;
        }
        Window A, B;
        if (w < r1) load_window(A, w, r1, pg0);
        while (w < r1) {
            int wn = w + step;
            if (wn < r1) load_window(B, wn, r1, pg0);
            compute_window(A);
            w = wn;
            if (w >= r1) break;
            wn = w + step;
            if (wn < r1) load_window(A, wn, r1, pg0);
            compute_window(B);
            w = wn;
        }
    };

    int pg0_last = 0;  // first table entry of the last staged slice
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
            pg0_last = pg0;
        }
    }

    // Single-launch step: the split holding the current token stores it into its page
    // (head group 0 only; one row per KV head).
    if constexpr (FUSED) {
        if (hg == 0 && wave == 0 && lg == 0 && t_new >= lo && t_new < hi) {
            const size_t page = (size_t)s_tbl[(t_new >> pshift) - pg0_last];
            const size_t row =
                (((page << pshift) | (size_t)(t_new & pmask)) * slot_stride) + (size_t)kvh * D +
                li * EPL;
            *reinterpret_cast<uint4*>(reinterpret_cast<T*>(a.k_pages_w) + row) =
                *reinterpret_cast<const uint4*>(knew);
            *reinterpret_cast<uint4*>(reinterpret_cast<T*>(a.v_pages_w) + row) =
                *reinterpret_cast<const uint4*>(vnew);
        }
    }

    // Every stream (wave, lane group) leaves its state in LDS; no cross-lane exchange.
    const int stream = wave * RPI + lg;
#pragma unroll
    for (int j = 0; j < GH; ++j) {
        float4* dst = reinterpret_cast<float4*>(s_o + ((size_t)stream * GH + j) * D + li * EPL);
#pragma unroll
        for (int e = 0; e < EPL; e += 4)
            dst[e / 4] = make_float4(o[j][e], o[j][e + 1], o[j][e + 2], o[j][e + 3]);
    }
    if (li == 0) {
#pragma unroll
        for (int j = 0; j < GH; ++j) {
            s_m[stream * GH + j] = m[j];
            s_l[stream * GH + j] = l[j];
        }
    }
    __syncthreads();

    // Merge, phase 1: per (stream, head) the factor f = exp(m_s - M), M the split's maximum.
    for (int idx = tid; idx < streams * GH; idx += nthreads) {
        const int j = idx % GH;
        float M = -INFINITY;
        for (int s2 = 0; s2 < streams; ++s2) M = fmaxf(M, s_m[s2 * GH + j]);
        const float ms = (M == -INFINITY) ? 0.f : M;
        s_f[idx] = fast_exp2(s_m[idx] - ms);
    }
    __syncthreads();

    // Merge, phase 2: one weighted sum per output element of the split's partial.
    for (int idx = tid; idx < GH * D; idx += nthreads) {
        const int j = idx / D;
        const int d = idx - j * D;
        if (j >= nh) continue;
        float O0 = 0.f, O1 = 0.f;
        int s2 = 0;
        for (; s2 + 1 < streams; s2 += 2) {
            O0 = fmaf(s_o[((size_t)s2 * GH + j) * D + d], s_f[s2 * GH + j], O0);
            O1 = fmaf(s_o[((size_t)(s2 + 1) * GH + j) * D + d], s_f[(s2 + 1) * GH + j], O1);
        }
        if (s2 < streams) O0 = fmaf(s_o[((size_t)s2 * GH + j) * D + d], s_f[s2 * GH + j], O0);
        const size_t slot = ((size_t)b * a.num_q_heads + h0 + j) * S + split;
        store_partial<FUSED>(a.partial_o + slot * D + d, O0 + O1);
        if (d == 0) {
            float L = 0.f, M = -INFINITY;
            for (int s3 = 0; s3 < streams; ++s3) {
                L = fmaf(s_l[s3 * GH + j], s_f[s3 * GH + j], L);
                M = fmaxf(M, s_m[s3 * GH + j]);
            }
            store_partial<FUSED>(a.partial_ml + 2 * slot, (L > 0.f) ? M * kLn2 : -INFINITY);
            store_partial<FUSED>(a.partial_ml + 2 * slot + 1, L);
        }
    }

    if constexpr (FUSED) {
        // The last of the group's S workgroups to finish merges their partials.  The partials
        // travel by device-scope stores and loads (written through to, and read from, the
        // device's coherence point), so no fence has to write back or invalidate a whole L2
        // (each XCD has its own, and that costs microseconds per workgroup).  Every wave waits
        // until its stores are acknowledged, the barrier gathers the waves, and only then is
        // the workgroup counted; the last one counted reads after its count returned.
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        uint32_t* counter = a.counters + ((size_t)b * a.num_kv_heads + kvh) * a.head_groups + hg;
        if (tid == 0) {
            const uint32_t prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
            s_last = (prev == (uint32_t)(S - 1)) ? 1 : 0;
        }
        __syncthreads();
        if (!s_last) return;
        constexpr int D4 = D / 4;
        // Buffer resources over this workgroup's rows of partials (bases uniform over the
        // workgroup; at most 8 heads x 4096 splits x D floats, far below 2^31 bytes).
        const size_t row0 = (size_t)b * a.num_q_heads + h0;
        CoherentPartials src;
        src.o_rsrc = __builtin_amdgcn_make_buffer_rsrc(a.partial_o + row0 * S * D, 0,
                                                       nh * S * D * 4, kRawBufferWord3);
        src.ml_rsrc = __builtin_amdgcn_make_buffer_rsrc(a.partial_ml + row0 * S * 2, 0,
                                                        nh * S * 8, kRawBufferWord3);
        src.o_stride = D * 4;
        for (int idx = tid; idx < nh * D4; idx += nthreads) {
            const int j = idx / D4;
            const int c = idx - j * D4;
            src.o_off = (uint32_t)((j * S * D + c * 4) * 4);
            src.ml_off = (uint32_t)(j * S * 8);
            reinterpret_cast<float4*>(a.out)[(row0 + j) * D4 + c] = merge_splits(src, S);
        }
        if (tid == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Split partials only (paged_attn_decode).
template <typename KV, int D, int GH>
__global__ void __launch_bounds__((DecodeGeom<KV, D>::kWaves * 64))
    __attribute__((amdgpu_waves_per_eu(2))) decode_split_kernel(DecodeArgs a) {
    decode_body<KV, D, GH, false>(a);
}

// The single-launch step (paged_attn_decode_fused): page write, partials, last-split merge.
template <typename KV, int D, int GH>
__global__ void __launch_bounds__((DecodeGeom<KV, D>::kWaves * 64))
    __attribute__((amdgpu_waves_per_eu(2))) decode_step_kernel(DecodeArgs a) {
    decode_body<KV, D, GH, true>(a);
}

template <typename KV, int D, int GH, bool FUSED>
const void* decode_kernel_ptr() {
    if constexpr (FUSED)
        return (const void*)decode_step_kernel<KV, D, GH>;
    else
        return (const void*)decode_split_kernel<KV, D, GH>;
}

template <typename KV, int D, int GH, bool FUSED>
hipError_t launch_gh(const DecodeArgs& a, int waves, hipStream_t stream) {
    using G = DecodeGeom<KV, D>;
    const size_t lds = decode_lds_bytes(waves * G::RPI, GH, D);
    // Workgroups asking for more than 64 KB of LDS opt in once per instantiation.
    static size_t opted = 64 * 1024;
    if (lds > opted) {
        hipError_t e = hipFuncSetAttribute(decode_kernel_ptr<KV, D, GH, FUSED>(),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        opted = lds;
    }
    const dim3 grid(a.num_splits, a.num_kv_heads * a.head_groups, a.num_seqs);
    if constexpr (FUSED)
        hipLaunchKernelGGL((decode_step_kernel<KV, D, GH>), grid, dim3(waves * 64), lds, stream, a);
    else
        hipLaunchKernelGGL((decode_split_kernel<KV, D, GH>), grid, dim3(waves * 64), lds, stream,
                           a);
    return hipGetLastError();
}

template <typename KV, int D, bool FUSED>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
    using G = DecodeGeom<KV, D>;
    // Waves per workgroup: enough for one window pass to cover a split of the table's
    // capacity (lengths live on the device), at most G::kWaves.  The choice depends only on
    // the split size, head_dim and dtype, never on the batch or the head grouping, so a
    // sequence's result is bit-identical whatever it is batched with, and a GQA group gives
    // the same bits as the equivalent MHA call.
    const int64_t cap = (int64_t)a.max_pages << a.page_shift;
    const int64_t chunk = (cap + a.num_splits - 1) / a.num_splits;
    const int64_t rows_per_pass = (int64_t)G::RPI * kWindowRows;
    int waves = (int)std::min<int64_t>(G::kWaves, (chunk + rows_per_pass - 1) / rows_per_pass);
    waves = std::max(waves, 1);
    switch (a.heads_per_wg) {
        case 1: return launch_gh<KV, D, 1, FUSED>(a, waves, stream);
        case 2: return launch_gh<KV, D, 2, FUSED>(a, waves, stream);
        case 3: return launch_gh<KV, D, 3, FUSED>(a, waves, stream);
        case 4: return launch_gh<KV, D, 4, FUSED>(a, waves, stream);
        case 5: return launch_gh<KV, D, 5, FUSED>(a, waves, stream);
        case 6: return launch_gh<KV, D, 6, FUSED>(a, waves, stream);
        case 7: return launch_gh<KV, D, 7, FUSED>(a, waves, stream);
        case 8: return launch_gh<KV, D, 8, FUSED>(a, waves, stream);
        default: return hipErrorInvalidValue;
    }
}

template <bool FUSED>
hipError_t launch_all(const DecodeArgs& a, int kv_dtype, int head_dim, hipStream_t stream) {
    if (head_dim == 64) {
        if (kv_dtype == 0) return launch_typed<F32, 64, FUSED>(a, stream);
        if (kv_dtype == 1) return launch_typed<F16, 64, FUSED>(a, stream);
        return launch_typed<BF16, 64, FUSED>(a, stream);
    }
    if (kv_dtype == 0) return launch_typed<F32, 128, FUSED>(a, stream);
    if (kv_dtype == 1) return launch_typed<F16, 128, FUSED>(a, stream);
    return launch_typed<BF16, 128, FUSED>(a, stream);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int kv_dtype, int head_dim, bool fused,
                         hipStream_t stream) {
    return fused ? launch_all<true>(a, kv_dtype, head_dim, stream)
                 : launch_all<false>(a, kv_dtype, head_dim, stream);
}

}  // namespace pa
