// decode_valu.h — the decode kernels on the vector ALUs, for f32 pools and for head_dim 256
// (included by decode.hip, in its translation unit).
//
// Why a second body: the f32 matrix-core instruction (v_mfma_f32_16x16x4_f32) has the same
// peak rate as the f32 vector units, so it saves issue slots but not time, and its 16-column
// blocks sit mostly idle at a few query heads per KV head; a 32-key tile of f32 scores is a
// chain of 32 such MFMAs.  At head_dim 256 the matrix-core operands of 16 columns need more
// than half a SIMD's registers, so that body runs one wave per SIMD, and the vector body
// with at most 4 heads per workgroup measured faster.  The other 16-bit pools use the
// matrix-core body in decode.hip.  Both bodies follow the same method, split rule, lazy
// rescale, partial layout and single-launch handoff, and give results within the f32 bar of
// the oracle; each is deterministic and batch- and grouping-invariant by itself.
//
// Method (crucible README, "Split-position attention": grid over heads and context chunks,
// each block reducing one chunk to a partial softmax; minfer 71 "D3-6 GQA q-head batched
// attention", 3.2 Excerpt A: chunk = ceil(nkv / splits) and the split's row range; section 2:
// one block per KV head serving all of its query heads reads each K/V row once).
//
// gfx950 mapping
//   grid  (num_splits, num_kv_heads * head_groups, num_seqs); one workgroup of `waves`
//         64-lane waves serves up to GH query heads (at most 8) of one KV head over one split.
//   rows  one K or V row (D elements) is spread over one 16-lane DPP row of a wave: each
//         lane holds D/16 elements (16 or 32 bytes, one or two vector loads), and one
//         wave-wide load fetches 4 rows.  Each 16-lane row keeps its own online-softmax
//         stream.
//   window each wave takes U rows per 16-lane row (4U rows) and issues every K and V load of
//         the window before the first dependent instruction (the whole-window staging of the
//         minfer 75 "D4-3" page, 3.2 Excerpt A/C).
//   dots  each lane multiplies its slice for all GH heads, then a reduce-scatter over the 16
//         lanes leaves every lane with the full score of one head.  The heads sit in the
//         lane's registers in a lane-dependent order (see slot_key), so each exchange step
//         is a single DPP add: 8 heads cost 8 adds per row instead of 32 for an all-reduce.
//         Every lane takes part in every step (the validity select comes after the
//         reduction, the D3-6 pitfall about divergent shuffles).
//   softmax each lane runs the online softmax of its own head only; the probabilities reach
//         the PV products by DPP row broadcasts.  The accumulator is rescaled only when a
//         head's maximum rises more than kLazyRescale above the reference it was scaled to;
//         the true maximum is tracked beside it and the split's partial is normalised to it.
//   table, merge, step, window, checks: as in decode.hip.
#pragma once

namespace pa {
namespace {
namespace valu {


// f(std::integral_constant<int, I>) for I in [I0, I1): a loop whose index is a constant.
template <int I0, int I1, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I0 < I1) {
        f(std::integral_constant<int, I0>{});
        static_for<I0 + 1, I1>(f);
    }
}

constexpr int kMaxWaves = 8;
constexpr int kTableCap = 1024;  // page-table entries staged in LDS at a time
constexpr int kWindowRows = 4;   // U: rows per 16-lane row per window
constexpr int kLanesPerRow = 16;
constexpr int kRowsPerLoad = 64 / kLanesPerRow;

// Base-2 headroom of the lazy rescale: probabilities are exp2(s - m_ref) <= 2^8.
constexpr float kLazyRescale = 8.f;

constexpr int kStreamLds = 64 * 1024;  // LDS for stream states at the largest head group

template <typename KV, int D>
struct DecodeGeom {
    static constexpr int EPL = D / kLanesPerRow;          // elements per lane and row
    static constexpr int WPL = EPL * KV::kBytes / 4;      // 32-bit words per lane and row
    static constexpr int kMaxGH = D > 128 ? 4 : 8;        // query heads per workgroup
    // Most waves per workgroup: every stream keeps up to kMaxGH heads x D floats in LDS.
    static constexpr int kWaves = (kStreamLds / (kMaxGH * D * 4) / kRowsPerLoad) < kMaxWaves
                                      ? (kStreamLds / (kMaxGH * D * 4) / kRowsPerLoad)
                                      : kMaxWaves;
};

// Dynamic LDS of one workgroup: staged page ids, then per head and stream (wave x 16-lane
// row) the reference maximum, the true maximum and the sum l, then per stream the GH x D
// accumulators (padded by 16 bytes).  The last-split merge reuses it from the start: 32
// float2 weight slots per row of D / 4 lanes (streams x 16 lanes in the workgroup).
__host__ __device__ constexpr size_t decode_lds_bytes(int streams, int gh, int d) {
    const size_t state = (size_t)kTableCap * 4 + (size_t)streams * gh * 3 * 4 +
                         (size_t)streams * (gh * d + 4) * 4;
    const size_t merge = (size_t)streams * 16 / (d / 4) * kMergeChunk * 8;
    return state > merge ? state : merge;
}

// ------------------------------------------------------------------ K/V row fragments

// One lane's slice of one K or V row: WPL 32-bit words, moved as one or two 16-byte loads
// (or one 8-byte load for 64 16-bit elements).
template <int WPL>
struct Frag {
    uint32_t w[WPL];
};

template <int WPL>
__device__ __forceinline__ void load_frag(Frag<WPL>& f, const void* p) {
    if constexpr (WPL == 2) {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        f.w[0] = v.x;
        f.w[1] = v.y;
    } else {
#pragma unroll
        for (int i = 0; i < WPL; i += 4) {
            const uint4 v = reinterpret_cast<const uint4*>(p)[i / 4];
            f.w[i] = v.x;
            f.w[i + 1] = v.y;
            f.w[i + 2] = v.z;
            f.w[i + 3] = v.w;
        }
    }
}

template <int WPL>
__device__ __forceinline__ void store_frag(void* p, const Frag<WPL>& f) {
    if constexpr (WPL == 2) {
        *reinterpret_cast<uint2*>(p) = make_uint2(f.w[0], f.w[1]);
    } else {
#pragma unroll
        for (int i = 0; i < WPL; i += 4)
            reinterpret_cast<uint4*>(p)[i / 4] = make_uint4(f.w[i], f.w[i + 1], f.w[i + 2],
                                                            f.w[i + 3]);
    }
}

template <typename KV, int WPL>
__device__ __forceinline__ void widen_frag(const Frag<WPL>& f, float* out) {
    constexpr int per = 4 / KV::kBytes;
#pragma unroll
    for (int i = 0; i < WPL; ++i) widen_word(KV{}, f.w[i], out + i * per);
}

// ------------------------------------------------------------------ head slots

// The GH heads of a workgroup are split into power-of-two groups of 8, 4, 2 and 1 (the
// binary digits of GH, largest first).  In group n (size N, first head B) lane li computes,
// in its register B + r, the partial dot of head B + (r ^ slot_key<N>(li)).  The exchange
// partners of the reduction are lane ^ 8 (row_ror:8), lane ^ 7 (row_half_mirror), lane ^ 2
// and lane ^ 1 (quad_perm), in that order; slot_key is the linear map of the lane bits
// under which the first log2(N) partners each flip exactly one key bit (from the high one
// down) and the later ones none.  So at every step a lane adds its register to the
// partner's register that holds the same head, and after the four steps the lane holds the
// full sum of head B + slot_key<N>(li).  The summation tree is the same for every N (and
// equal to the all-reduce used for N = 1), so a head's score has the same bits whatever
// companions it has.
template <int N>
__device__ __forceinline__ int slot_key(int li) {
    if constexpr (N == 8)
        return (((li >> 3) & 1) << 2) | (((li >> 2) & 1) << 1) | (((li >> 1) ^ (li >> 2)) & 1);
    if constexpr (N == 4) return (((li >> 3) & 1) << 1) | ((li >> 2) & 1);
    if constexpr (N == 2) return (li >> 3) & 1;
    return 0;
}

// The lowest lane of a 16-lane row whose key is H (inverse of slot_key with bit 0 clear).
template <int N>
__host__ __device__ constexpr int owner_lane(int H) {
    return N == 8   ? 8 * ((H >> 2) & 1) + 4 * ((H >> 1) & 1) + 2 * ((H ^ (H >> 1)) & 1)
           : N == 4 ? 8 * ((H >> 1) & 1) + 4 * (H & 1)
           : N == 2 ? 8 * (H & 1)
                    : 0;
}

// Lanes that store a group's softmax state (one per head; the others hold copies).
template <int N>
__device__ __forceinline__ bool is_owner(int li) {
    if constexpr (N == 8) return (li & 1) == 0;
    if constexpr (N == 4) return (li & 3) == 0;
    if constexpr (N == 2) return (li & 7) == 0;
    return li == 0;
}

template <int GH>
struct HeadGroups {
    static constexpr int count = ((GH >> 3) & 1) + ((GH >> 2) & 1) + ((GH >> 1) & 1) + (GH & 1);
    static constexpr int size(int g) {
        int k = 0;
        for (int n = 8; n >= 1; n >>= 1)
            if (GH & n) {
                if (k == g) return n;
                ++k;
            }
        return 0;
    }
    static constexpr int base(int g) {
        int b = 0;
        for (int k = 0; k < g; ++k) b += size(k);
        return b;
    }
};

constexpr int kDppRowRor8 = 0x128;      // lane i <- lane (i + 8) mod 16 (= i ^ 8)
constexpr int kDppRowHalfMirror = 0x141;  // lane i <- lane 7 - i within 8 (= i ^ 7)
constexpr int kDppQuadX2 = 0x4e;         // quad_perm [2,3,0,1] (= i ^ 2)
constexpr int kDppQuadX1 = 0xb1;         // quad_perm [1,0,3,2] (= i ^ 1)
template <int L>
__device__ __forceinline__ float row_bcast(float v) {  // row_newbcast: lane L of each row
    return dpp_mov<0x150 + L>(v);
}

// Reduce-scatter of one group's N partial dots (registers d[0..N)) over the 16 lanes.
template <int N>
__device__ __forceinline__ float reduce_scatter(const float* d) {
    float r;
    if constexpr (N == 8) {
        const float a0 = d[0] + dpp_mov<kDppRowRor8>(d[4]);
        const float a1 = d[1] + dpp_mov<kDppRowRor8>(d[5]);
        const float a2 = d[2] + dpp_mov<kDppRowRor8>(d[6]);
        const float a3 = d[3] + dpp_mov<kDppRowRor8>(d[7]);
        const float b0 = a0 + dpp_mov<kDppRowHalfMirror>(a2);
        const float b1 = a1 + dpp_mov<kDppRowHalfMirror>(a3);
        r = b0 + dpp_mov<kDppQuadX2>(b1);
    } else if constexpr (N == 4) {
        const float a0 = d[0] + dpp_mov<kDppRowRor8>(d[2]);
        const float a1 = d[1] + dpp_mov<kDppRowRor8>(d[3]);
        r = a0 + dpp_mov<kDppRowHalfMirror>(a1);
        r = r + dpp_mov<kDppQuadX2>(r);
    } else if constexpr (N == 2) {
        r = d[0] + dpp_mov<kDppRowRor8>(d[1]);
        r = r + dpp_mov<kDppRowHalfMirror>(r);
        r = r + dpp_mov<kDppQuadX2>(r);
    } else {
        r = d[0] + dpp_mov<kDppRowRor8>(d[0]);
        r = r + dpp_mov<kDppRowHalfMirror>(r);
        r = r + dpp_mov<kDppQuadX2>(r);
    }
    return r + dpp_mov<kDppQuadX1>(r);
}

// Value of head B + H of group (N, B) from the lane that owns it, in every lane of the row.
template <int N, int H>
__device__ __forceinline__ float from_owner(float v) {
    if constexpr (N == 1)
        return v;
    else
        return row_bcast<owner_lane<N>(H)>(v);
}

// A split partial leaves the workgroup by plain stores, or, when another workgroup of the
// same launch merges it, by device-scope ones (written through this XCD's L2): 16 bytes of
// O and 8 bytes of (m, l) per lane, through buffer resources over this workgroup's rows, so
// that a wave's store covers whole lines rather than a strided scatter of words.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
constexpr int kDeviceScopeStore = 16;  // buffer-instruction cache policy: device scope

struct PartialStore {
    __amdgpu_buffer_rsrc_t o_rsrc, ml_rsrc;  // over rows [row0, row0 + nh) of the partials
    __device__ __forceinline__ void o(uint32_t byte_off, float4 v) const {
        const u32x4 d = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z),
                         __float_as_uint(v.w)};
        __builtin_amdgcn_raw_buffer_store_b128(d, o_rsrc, byte_off, 0, kDeviceScopeStore);
    }
    __device__ __forceinline__ void ml(uint32_t byte_off, float m, float l) const {
        const u32x2 d = {__float_as_uint(m), __float_as_uint(l)};
        __builtin_amdgcn_raw_buffer_store_b64(d, ml_rsrc, byte_off, 0, kDeviceScopeStore);
    }
};

template <typename KV, int D, int GH, bool FUSED>
__device__ __forceinline__ void decode_body(const DecodeArgs& a) {
    using T = typename KV::storage;
    using G = DecodeGeom<KV, D>;
    using HG = HeadGroups<GH>;
    constexpr int NG = HG::count;
    constexpr int EPL = G::EPL;
    constexpr int WPL = G::WPL;
    constexpr int RPI = kRowsPerLoad;
    constexpr int U = kWindowRows;
    constexpr int WROWS = RPI * U;        // rows per wave per window
    // Registers of q and of the accumulators plus two windows of K/V.
    constexpr bool kPrefetch = 2 * GH * EPL + 4 * U * WPL <= 208;
    constexpr int TPT = kTableCap / 64;   // table entries staged per thread (>= 64 threads)

    extern __shared__ __align__(16) float lds[];
    __shared__ int s_last;  // single-launch step: this workgroup finished the group's last split
    const int nthreads = blockDim.x;
    const int nwaves = nthreads >> 6;
    const int streams = nwaves * RPI;
    int* s_tbl = reinterpret_cast<int*>(lds);
    float* s_m = lds + kTableCap;          // [GH][streams] reference maximum
    float* s_t = s_m + GH * streams;       // [GH][streams] true maximum
    float* s_l = s_t + GH * streams;       // [GH][streams] sum
    float* s_o = s_l + GH * streams;       // [streams][SOS]: per stream GH x D, then padding
    constexpr int SOS = GH * D + 4;        // padded so the 4 rows of a wave hit other banks

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int lg = lane / kLanesPerRow;  // row slot within a wave-wide load
    const int li = lane % kLanesPerRow;  // slice of the row

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
    if constexpr (kChecked) {
        // The length within [0, capacity], and (one workgroup per sequence and KV head) the
        // page ids of the attended positions within [0, num_pages).
        const int raw = a.context_lens[b];
        if (raw < 0 || raw > cap) mark_bad(&g_bad_metadata_decode);
        if (split == 0 && hg == 0) {
            const int first = (a.window > 0 && ctx > a.window) ? ctx - a.window : 0;
            const int p_end = (ctx + (1 << a.page_shift) - 1) >> a.page_shift;
            for (int p = (first >> a.page_shift) + tid; p < p_end; p += nthreads) {
                const int v = trow[p];
                if (v < 0 || v >= a.num_pages) mark_bad(&g_bad_metadata_decode);
            }
        }
    }
    // q in the lane's register order: register B + r of group (N, B) holds head
    // B + (r ^ slot_key<N>(li)); padded heads repeat the last real one.
    float qv[GH][EPL];
    static_for<0, NG>([&](auto gc) {
        constexpr int g = decltype(gc)::value;
        constexpr int N = HG::size(g);
        constexpr int B = HG::base(g);
        const int key = slot_key<N>(li);
#pragma unroll
        for (int r = 0; r < N; ++r) {
            const int h = h0 + min(B + (r ^ key), nh - 1);
            const float* qp = a.q + ((size_t)b * a.num_q_heads + h) * D + li * EPL;
#pragma unroll
            for (int e = 0; e < EPL; e += 4) {
                const float4 t = *reinterpret_cast<const float4*>(qp + e);
                qv[B + r][e + 0] = t.x;
                qv[B + r][e + 1] = t.y;
                qv[B + r][e + 2] = t.z;
                qv[B + r][e + 3] = t.w;
            }
        }
    });
    // The splits partition the attended positions [w0, ctx): the whole context, or with a
    // sliding window the current token and the window - 1 before it (vllm.cpp PR #383: the
    // windowed arm of the decode kernel).
    const int S = a.num_splits;
    const int w0 = (a.window > 0 && ctx > a.window) ? ctx - a.window : 0;
    const int n_att = ctx - w0;
    const int chunk = (n_att + S - 1) / S;
    const int lo = w0 + min(split * chunk, n_att);
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

    // Per group, for the lane's own head: the reference maximum the accumulator is scaled
    // to, the true running maximum and the running sum.  Accumulators in head order.
    float mr[NG], mt[NG], l[NG], o[GH][EPL];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        mr[g] = -INFINITY;
        mt[g] = -INFINITY;
        l[g] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < GH; ++j)
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[j][e] = 0.f;

    // Row addresses: one 32x32->64-bit multiply of the pool row by the bytes between slots
    // (Hkv * D * elt < 2^32), added to the lane's base.
    const uint32_t slot_bytes = (uint32_t)a.num_kv_heads * (uint32_t)(D * KV::kBytes);
    const size_t lane_off = ((size_t)kvh * D + li * EPL) * KV::kBytes;
    const char* kbase = reinterpret_cast<const char*>(a.k_pages) + lane_off;
    const char* vbase = reinterpret_cast<const char*>(a.v_pages) + lane_off;
    const int pshift = a.page_shift;
    const int pmask = (1 << pshift) - 1;
    // Single-launch step: the current token (position ctx - 1) is read from k_new / v_new;
    // its pool slot is written by this launch and read by none of its workgroups.  As in
    // kv_page_write, a token whose raw length lies outside [1, capacity] or whose raw page id
    // lies outside [0, num_pages) is neither written nor read from k_new / v_new.
    int t_new = -1;
    if constexpr (FUSED) {
        const int raw = a.context_lens[b];
        if (raw >= 1 && raw <= cap) {
            const int pid = trow[(raw - 1) >> a.page_shift];
            if (pid >= 0 && pid < a.num_pages) t_new = raw - 1;
        }
    }
    const T* knew = nullptr;
    const T* vnew = nullptr;
    if constexpr (FUSED) {
        const size_t off = ((size_t)b * a.num_kv_heads + kvh) * D + li * EPL;
        knew = reinterpret_cast<const T*>(a.k_new) + off;
        vnew = reinterpret_cast<const T*>(a.v_new) + off;
    }

    // One window: U rows per 16-lane row starting at w0, rows past r1 clamped onto row
    // r1 - 1 (a valid address, cache hits) and flagged, so no branch guards the loads.
    struct Window {
        Frag<WPL> k[U], v[U];
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
            const uint32_t row = ((uint32_t)pg[u] << pshift) | (uint32_t)(t[u] & pmask);
            const uint64_t off = (uint64_t)row * slot_bytes;
            const void* kp = kbase + off;
            const void* vp = vbase + off;
            if constexpr (FUSED) {
                kp = (t[u] == t_new) ? (const void*)knew : kp;
                vp = (t[u] == t_new) ? (const void*)vnew : vp;
            }
            load_frag(W.k[u], kp);
            load_frag(W.v[u], vp);
        }
    };
    auto compute_window = [&](const Window& W) {
        // Scores: every lane ends with its own head's score of each of the U rows.
        float s[NG][U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float kf[EPL];
            widen_frag<KV>(W.k[u], kf);
            float d[GH];
#pragma unroll
            for (int j = 0; j < GH; ++j) {
                float acc = qv[j][0] * kf[0];
#pragma unroll
                for (int e = 1; e < EPL; ++e) acc = fmaf(qv[j][e], kf[e], acc);
                d[j] = acc;
            }
            static_for<0, NG>([&](auto gc) {
                constexpr int g = decltype(gc)::value;
                const float r = reduce_scatter<HG::size(g)>(d + HG::base(g));
                s[g][u] = W.ok[u] ? r : -INFINITY;
            });
        }
        // Online softmax of the lane's heads, one rescale decision per window.
        float mx[NG];
        bool need = false;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            float v = s[g][0];
#pragma unroll
            for (int u = 1; u < U; ++u) v = fmaxf(v, s[g][u]);
            mx[g] = v;
            mt[g] = fmaxf(mt[g], v);
            need |= v > mr[g] + kLazyRescale;
        }
        // Rescale only where some head of the wave outgrew its reference by more than the
        // headroom; a head that did not keeps its reference and is multiplied by exactly 1,
        // so its bits do not depend on its companions.
        if (__builtin_amdgcn_ballot_w64(need) != 0) {
            float alpha[NG];
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const bool up = mx[g] > mr[g] + kLazyRescale;
                alpha[g] = up ? fast_exp2(mr[g] - mx[g]) : 1.f;  // a reference of -inf gives 0
                mr[g] = up ? mx[g] : mr[g];
                l[g] *= alpha[g];
            }
            static_for<0, NG>([&](auto gc) {
                constexpr int g = decltype(gc)::value;
                constexpr int N = HG::size(g);
                constexpr int B = HG::base(g);
                static_for<0, N>([&](auto hc) {
                    constexpr int h = decltype(hc)::value;
                    const float f = from_owner<N, h>(alpha[g]);
#pragma unroll
                    for (int e = 0; e < EPL; ++e) o[B + h][e] *= f;
                });
            });
        }
        float p[NG][U];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const float ms = (mr[g] == -INFINITY) ? 0.f : mr[g];
#pragma unroll
            for (int u = 0; u < U; ++u) p[g][u] = fast_exp2(s[g][u] - ms);
            float ps = p[g][0];
#pragma unroll
            for (int u = 1; u < U; ++u) ps += p[g][u];
            l[g] += ps;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float vf[EPL];
            widen_frag<KV>(W.v[u], vf);
            static_for<0, NG>([&](auto gc) {
                constexpr int g = decltype(gc)::value;
                constexpr int N = HG::size(g);
                constexpr int B = HG::base(g);
                static_for<0, N>([&](auto hc) {
                    constexpr int h = decltype(hc)::value;
                    const float pb = from_owner<N, h>(p[g][u]);
#pragma unroll
                    for (int e = 0; e < EPL; ++e) o[B + h][e] = fmaf(pb, vf[e], o[B + h][e]);
                });
            });
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
            const uint32_t page = (uint32_t)s_tbl[(t_new >> pshift) - pg0_last];
            const uint64_t off =
                (uint64_t)((page << pshift) | (uint32_t)(t_new & pmask)) * slot_bytes + lane_off;
            Frag<WPL> fk, fv;
            load_frag(fk, knew);
            load_frag(fv, vnew);
            store_frag(reinterpret_cast<char*>(a.k_pages_w) + off, fk);
            store_frag(reinterpret_cast<char*>(a.v_pages_w) + off, fv);
        }
    }

    // Every stream (wave, 16-lane row) leaves its state in LDS; no cross-lane exchange.
    const int stream = wave * RPI + lg;
#pragma unroll
    for (int j = 0; j < GH; ++j) {
        float4* dst = reinterpret_cast<float4*>(s_o + stream * SOS + j * D + li * EPL);
#pragma unroll
        for (int e = 0; e < EPL; e += 4)
            dst[e / 4] = make_float4(o[j][e], o[j][e + 1], o[j][e + 2], o[j][e + 3]);
    }
    static_for<0, NG>([&](auto gc) {
        constexpr int g = decltype(gc)::value;
        constexpr int N = HG::size(g);
        constexpr int B = HG::base(g);
        if (is_owner<N>(li)) {
            const int j = (B + slot_key<N>(li)) * streams + stream;
            s_m[j] = mr[g];
            s_t[j] = mt[g];
            s_l[j] = l[g];
        }
    });
    __syncthreads();

    // Merge of the streams: one thread per (head, 4 consecutive elements).  Stream s enters
    // with the factor exp(m_ref_s - M), M the split's true maximum (at least every stream's
    // reference, so the factor is at most 1; 0 for a stream that saw no row).  The per-stream
    // scalars are read four streams at a time.
    constexpr int D4 = D / 4;
    PartialStore pst;
    if constexpr (FUSED) {
        // Rows of partials of this workgroup's heads: at most 8 heads x 4096 splits x D
        // floats, far below 2^31 bytes; bases uniform over the workgroup.
        const size_t row0 = (size_t)b * a.num_q_heads + h0;
        pst.o_rsrc = __builtin_amdgcn_make_buffer_rsrc(a.partial_o + row0 * S * D, 0,
                                                       nh * S * D * 4, kRawBufferWord3);
        pst.ml_rsrc = __builtin_amdgcn_make_buffer_rsrc(a.partial_ml + row0 * S * 2, 0,
                                                        nh * S * 8, kRawBufferWord3);
    }
    auto merge_streams = [&](auto emit) {
        for (int idx = tid; idx < GH * D4; idx += nthreads) {
            const int j = idx / D4;
            const int c = idx - j * D4;
            if (j >= nh) continue;
            const float4* t4 = reinterpret_cast<const float4*>(s_t + j * streams);
            const float4* m4 = reinterpret_cast<const float4*>(s_m + j * streams);
            const float4* l4 = reinterpret_cast<const float4*>(s_l + j * streams);
            float M = -INFINITY;
            for (int q = 0; q < nwaves; ++q) {
                const float4 v = t4[q];
                M = fmaxf(M, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
            }
            const float ms = (M == -INFINITY) ? 0.f : M;
            float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
            float L = 0.f;
            for (int q = 0; q < nwaves; ++q) {
                const float4 mq = m4[q];
                const float4 lq = l4[q];
                const float f[4] = {fast_exp2(mq.x - ms), fast_exp2(mq.y - ms),
                                    fast_exp2(mq.z - ms), fast_exp2(mq.w - ms)};
                const float lv[4] = {lq.x, lq.y, lq.z, lq.w};
                float4 v[4];
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    v[k] = *reinterpret_cast<const float4*>(s_o + (4 * q + k) * SOS + j * D +
                                                            4 * c);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    O.x = fmaf(v[k].x, f[k], O.x);
                    O.y = fmaf(v[k].y, f[k], O.y);
                    O.z = fmaf(v[k].z, f[k], O.z);
                    O.w = fmaf(v[k].w, f[k], O.w);
                    L = fmaf(lv[k], f[k], L);
                }
            }
            const float mo = (L > 0.f) ? M * kLn2 : -INFINITY;
            emit(j, c, O, mo, L);
        }
    };

    if constexpr (!FUSED) {
        merge_streams([&](int j, int c, float4 O, float mo, float L) {
            const size_t slot = ((size_t)b * a.num_q_heads + h0 + j) * S + split;
            reinterpret_cast<float4*>(a.partial_o + slot * D)[c] = O;
            if (c == 0) reinterpret_cast<float2*>(a.partial_ml)[slot] = make_float2(mo, L);
        });
    } else {
        auto store_partial = [&](int j, int c, float4 O, float mo, float L) {
            const uint32_t js = (uint32_t)(j * S + split);
            pst.o(js * (uint32_t)(D * 4) + (uint32_t)c * 16u, O);
            if (c == 0) pst.ml(js * 8u, mo, L);
        };
        if (S == 1) {
            // One split: this partial is the whole row, and the merge's arithmetic applied to
            // it in registers gives the output the separate merge computes.  No ticket; the
            // counter stays at zero.
            merge_streams([&](int j, int c, float4 O, float mo, float L) {
                store_partial(j, c, O, mo, L);
                reinterpret_cast<float4*>(a.out)[((size_t)b * a.num_q_heads + h0 + j) * D4 + c] =
                    merge_splits(OwnPartial{make_float2(mo, L), O}, 1);
            });
            return;
        }
        merge_streams(store_partial);
        // The last of the group's S workgroups to finish merges their partials.  The partials
        // travel by device-scope stores and loads (written through to, and read from, the
        // device's coherence point), so no fence has to write back or invalidate a whole L2
        // (each XCD has its own, and that costs microseconds per workgroup).  Every wave waits
        // until its stores are acknowledged, the barrier gathers the waves, and only then is
        // the workgroup counted; the last one counted reads after its count returned.
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        uint32_t* counter =
            a.counters + (((size_t)b * a.num_kv_heads + kvh) * a.head_groups + hg) * kCounterStride;
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
        // The D4 lanes of a row merge it together, exchanging split weights through the
        // row's slots at the start of LDS (free once the streams' state is merged).
        float2* xw = reinterpret_cast<float2*>(lds) + (tid / D4) * kMergeChunk;
        for (int idx = tid; idx < nh * D4; idx += nthreads) {
            const int j = idx / D4;
            const int c = idx - j * D4;
            src.o_off = (uint32_t)((j * S * D + c * 4) * 4);
            src.ml_off = (uint32_t)(j * S * 8);
            reinterpret_cast<float4*>(a.out)[(row0 + j) * D4 + c] =
                merge_row<D4, true>(src, S, c, xw);
        }
        if (tid == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Split partials only (paged_attn_decode).
template <typename KV, int D, int GH>
__global__ void __launch_bounds__((DecodeGeom<KV, D>::kWaves * 64))
    __attribute__((amdgpu_waves_per_eu(2))) decode_valu_split_kernel(DecodeArgs a) {
    decode_body<KV, D, GH, false>(a);
}

// The single-launch step (paged_attn_decode_fused): page write, partials, last-split merge.
template <typename KV, int D, int GH>
__global__ void __launch_bounds__((DecodeGeom<KV, D>::kWaves * 64))
    __attribute__((amdgpu_waves_per_eu(2))) decode_valu_step_kernel(DecodeArgs a) {
    decode_body<KV, D, GH, true>(a);
}

template <typename KV, int D, int GH, bool FUSED>
const void* decode_kernel_ptr() {
    if constexpr (FUSED)
        return (const void*)decode_valu_step_kernel<KV, D, GH>;
    else
        return (const void*)decode_valu_split_kernel<KV, D, GH>;
}

template <typename KV, int D, int GH, bool FUSED>
hipError_t launch_gh(const DecodeArgs& a, int waves, hipStream_t stream) {
    const size_t lds = decode_lds_bytes(waves * kRowsPerLoad, GH, D);
    // Workgroups asking for more than 64 KB of LDS opt in, once per instantiation and device
    // (the largest size granted so far is kept per device; a repeated grant is harmless).
    if (lds > 64 * 1024) {
        static std::atomic<size_t> opted[kMaxDevices] = {};
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
            return hipErrorInvalidDevice;
        if (lds > opted[dev].load(std::memory_order_relaxed)) {
            hipError_t e = hipFuncSetAttribute(decode_kernel_ptr<KV, D, GH, FUSED>(),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)lds);
            if (e != hipSuccess) return e;
            size_t cur = opted[dev].load(std::memory_order_relaxed);
            while (cur < lds && !opted[dev].compare_exchange_weak(cur, lds)) {
            }
        }
    }
    const dim3 grid(a.num_splits, a.num_kv_heads * a.head_groups, a.num_seqs);
    if constexpr (FUSED)
        hipLaunchKernelGGL((decode_valu_step_kernel<KV, D, GH>), grid, dim3(waves * 64), lds, stream, a);
    else
        hipLaunchKernelGGL((decode_valu_split_kernel<KV, D, GH>), grid, dim3(waves * 64), lds, stream,
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
    int64_t cap = (int64_t)a.max_pages << a.page_shift;
    if (a.window > 0 && a.window < cap) cap = a.window;  // positions attended at most
    const int64_t chunk = (cap + a.num_splits - 1) / a.num_splits;
    const int64_t rows_per_pass = (int64_t)kRowsPerLoad * kWindowRows;
    int waves = (int)std::min<int64_t>(G::kWaves, (chunk + rows_per_pass - 1) / rows_per_pass);
    waves = std::max(waves, 1);
    switch (a.heads_per_wg) {
        case 1: return launch_gh<KV, D, 1, FUSED>(a, waves, stream);
        case 2: return launch_gh<KV, D, 2, FUSED>(a, waves, stream);
        case 3: return launch_gh<KV, D, 3, FUSED>(a, waves, stream);
        case 4: return launch_gh<KV, D, 4, FUSED>(a, waves, stream);
        default: break;
    }
    if constexpr (G::kMaxGH == 8) {
        switch (a.heads_per_wg) {
            case 5: return launch_gh<KV, D, 5, FUSED>(a, waves, stream);
            case 6: return launch_gh<KV, D, 6, FUSED>(a, waves, stream);
            case 7: return launch_gh<KV, D, 7, FUSED>(a, waves, stream);
            case 8: return launch_gh<KV, D, 8, FUSED>(a, waves, stream);
            default: break;
        }
    }
    return hipErrorInvalidValue;
}

template <bool FUSED>
hipError_t launch_all(const DecodeArgs& a, int kv_dtype, int head_dim, hipStream_t stream) {
    if (kv_dtype == 0) {
        if (head_dim == 64) return launch_typed<F32, 64, FUSED>(a, stream);
        if (head_dim == 128) return launch_typed<F32, 128, FUSED>(a, stream);
        return hipErrorInvalidValue;
    }
    if (head_dim != 256) return hipErrorInvalidValue;
    if (kv_dtype == 1) return launch_typed<F16, 256, FUSED>(a, stream);
    return launch_typed<BF16, 256, FUSED>(a, stream);
}

// f32 pools (head_dim 64, 128) and 16-bit pools at head_dim 256: the split kernel or the
// single-launch step.
hipError_t launch_decode_valu(const DecodeArgs& a, int kv_dtype, int head_dim, bool fused,
                              hipStream_t stream) {
    return fused ? launch_all<true>(a, kv_dtype, head_dim, stream)
                 : launch_all<false>(a, kv_dtype, head_dim, stream);
}

}  // namespace valu
}  // namespace
}  // namespace pa
