// decode.hip — split-KV paged decode: per-split partial softmax for the query heads of one
// KV head, on the matrix cores.
//
// Method (crucible README, "Split-position attention": grid over heads and context chunks,
// each block reducing one chunk to a partial softmax; minfer 71 "D3-6 GQA q-head batched
// attention", 3.2 Excerpt A: chunk = ceil(nkv / splits) and the split's row range; section 2:
// one block per KV head serving all of its query heads reads each K/V row once).
//
// gfx950 mapping
//   grid  (num_splits, num_kv_heads * head_groups, num_seqs); one workgroup of W 64-lane
//         waves serves up to 16 query heads of one KV head over one split, so each K/V row of
//         the split is read from HBM once for all of them.
//   tiles the split's rows are cut into 32-key tiles dealt round-robin to the waves.  A tile
//         is contracted against the workgroup's heads on the matrix cores with the operand
//         layouts of mfma_tiles.h: S^T = K Q^T with one query head per MFMA column, then
//         O^T += V^T P^T.  Every lane ends with 8 scores of ONE head (its column) and keeps
//         that head's online-softmax state, so the row maximum needs one exchange over the
//         four 16-lane groups per tile and nothing else crosses lanes.  (On the f32 vector
//         units the same contraction is 32 FMA instructions per K/V row for 8 heads at
//         D = 128 -- about the HBM time of the row's 512 bytes at the chip's rate -- plus the
//         widening and cross-lane reductions, which made that loop issue-bound; a tile costs
//         32 MFMAs of 16 cycles on one SIMD instead.)
//   loads each lane reads its K rows as 16-byte pieces of 16 keys x 32 dims per MFMA and its
//         V as NC consecutive dims of 8 keys.  The next tile's K and V are both requested as
//         soon as the scores have used this tile's K (V is double-buffered, K is not), so a
//         tile costs one memory round trip, overlapped with the softmax and PV product of
//         the tile before it.  Requests past a wave's last tile are clamped onto the split's
//         last row (cache hits).
//   pools f16 and bf16 at head_dim 64 and 128 here; f32 pools (whose MFMA has no rate
//         advantage over the vector units) and head_dim 256 run on the vector units
//         (decode_valu.h).
//   softmax base-2 scores (q pre-scaled by scale * log2 e).  The accumulator is rescaled only
//         when a head's maximum rises more than kLazyRescale above the reference it was scaled
//         to; the true maximum is tracked beside it and the partial is normalised to it.
//   table the sequence's page-table row (or a slice of it) is staged in LDS once; page ids
//         are clamped into [0, num_pages) as they are staged.
//   merge every wave leaves (m, l, O) of its heads in LDS; the workgroup writes the split's
//         (m, l) in natural-log units and the unnormalised O.
//   step  the single-launch step (paged_attn_decode_fused) also stores the current token's
//         K/V into its page and merges: the partials leave by device-scope stores, one
//         relaxed device-scope ticket per (sequence, KV head, head group) finds the last
//         workgroup, and that one reloads the group's partials and merges them with the
//         arithmetic of the separate merge kernel (the D/4 lanes of an output row sharing
//         each split's weight through LDS), so both paths give the same bits.  With
//         one split there is nothing to gather: each workgroup stores its partial, applies
//         that arithmetic to it in registers and writes the output, with no ticket.
//   heads the host spreads a KV head's query heads over twice the workgroups when the grid
//         would leave CUs idle; a head's column computes the same bits whatever the other
//         columns hold, so every grouping gives the same result.
//   order a batch of 2 .. kRankMax sequences whose grid is resident at once (at most two
//         workgroups per CU) runs the RANKED instantiation: every workgroup loads all lengths
//         and table rows, ranks the batch by attended length, and its grid slot takes the
//         sequence of that rank, in rounds of CU-count slots whose direction alternates, so
//         that the two workgroups of a CU hold a long and a short sequence.  A permutation of
//         the work: every sequence computes the same bits in either order.
//   window with a sliding window W the splits partition the attended positions
//         [ctx - W, ctx) (vllm.cpp PR #383 names the windowed arm of the decode kernel).
//   checks the checked build also marks a length or an attended page id out of range.
#include <algorithm>
#include <atomic>

#include "mfma_tiles.h"

namespace pa {

// Checked build: set when a length or an attended page id is outside its range.
__device__ int g_bad_metadata_decode;

namespace {

constexpr int kTableCap = 1024;  // page-table entries staged in LDS at a time
constexpr int kCols = 16;        // query heads per workgroup: the columns of an MFMA block

// Table entries staged by a workgroup: one sequence's row (or a slice of it), or with a
// ranked batch every sequence's row.
template <bool RANKED>
constexpr int table_cap() {
    return RANKED ? kDecodeTableCap : kTableCap;
}

// Base-2 headroom of the lazy rescale: probabilities are exp2(s - m_ref) <= 2^8.
constexpr float kLazyRescale = 8.f;

// Most waves per workgroup (two 4-wave workgroups share a CU at head_dim 128).
#ifndef PA_DECODE_MAX_WAVES
#define PA_DECODE_MAX_WAVES 4
#endif
template <int D>
constexpr int max_waves() {
    return PA_DECODE_MAX_WAVES;
}

__host__ __device__ constexpr int round4(int x) { return (x + 3) & ~3; }

// Dynamic LDS of one workgroup: tcap staged page ids; per (head, wave) the reference maximum, the
// true maximum and the sum l; per (wave, head) the D accumulators, padded by 16 bytes so the
// lanes' stores spread over the banks.  The last-split merge reuses it from the start: 32
// float2 weight slots per row of D / 4 lanes.
__host__ __device__ constexpr size_t decode_lds_bytes(int waves, int heads, int d, int tcap) {
    const size_t state = (size_t)tcap * 4 + (size_t)3 * round4(waves * heads) * 4 +
                         (size_t)waves * heads * (d + 4) * 4;
    const size_t merge = (size_t)waves * 64 / (d / 4) * kMergeChunk * 8;
    return state > merge ? state : merge;
}

// A split partial leaves the workgroup by plain stores, or, when another workgroup of the
// same launch merges it, by device-scope ones (written through this XCD's L2): 16 bytes of
// O and 8 bytes of (m, l) per lane, through buffer resources over this workgroup's rows.
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

template <typename KV, int D, bool FUSED, bool RANKED>
__device__ __forceinline__ void decode_body(const DecodeArgs& a) {
    using T = typename KV::storage;
    using Ops = TileOps<KV, D>;
    using Tile = typename Ops::Tile;
    constexpr int NC = D / 16;           // 16-dim blocks of the O^T accumulator
    constexpr int D4 = D / 4;            // float4 columns of an output row
    constexpr int SOH = D + 4;           // floats per (wave, head) accumulator row in LDS
    constexpr int TCAP = table_cap<RANKED>();
    constexpr int TPT = kTableCap / 64;  // table entries staged per thread (>= 64 threads)

    extern __shared__ __align__(16) float lds[];
    __shared__ int s_last;  // single-launch step: this workgroup finished the group's last split
    const int nthreads = blockDim.x;
    const int nwaves = nthreads >> 6;
    const int hpw = a.heads_per_wg;
    const int hw = round4(nwaves * hpw);
    int* s_tbl = reinterpret_cast<int*>(lds);
    float* s_m = lds + TCAP;       // [head][wave] reference maximum
    float* s_t = s_m + hw;         // [head][wave] true maximum
    float* s_l = s_t + hw;         // [head][wave] sum
    float* s_o = s_l + hw;         // [wave][head][SOH] accumulators

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int g = lane >> 4;    // MFMA k-group
    const int c16 = lane & 15;  // MFMA column: the lane's query head h0 + c16

    const int split = blockIdx.x;
    const int kvh = blockIdx.y / a.head_groups;
    const int hg = blockIdx.y % a.head_groups;
    const int h0 = kvh * a.group + hg * hpw;
    const int nh = min(hpw, a.group - hg * hpw);
    const int cap = a.max_pages << a.page_shift;

    // Nothing here depends on the context length, so the page-table row, the length and the
    // query are requested together, the table first: the K/V loads wait only for the table.
    // A ranked batch requests every sequence's length and table row (at most kRankMax
    // sequences, and entries within both the staged table and TPT per thread, which the host
    // checked), before it knows its own sequence.
    const int t_count = RANKED ? a.num_seqs * a.max_pages : a.max_pages;
    const int32_t* tsrc = a.page_table + (RANKED ? (size_t)0 : (size_t)blockIdx.z * a.max_pages);
    const bool whole_row = t_count <= TCAP && t_count <= TPT * nthreads;
    int tv[TPT];
    if (whole_row) {
#pragma unroll
        for (int k = 0; k < TPT; ++k) {
            const int i = tid + k * nthreads;
            tv[k] = (i < t_count) ? tsrc[i] : 0;
        }
    }
    int b = blockIdx.z;
    // In grid order the query is requested right after the table, ahead of the length and
    // the current token's page id (two dependent scalar round trips), so that its round trip
    // overlaps theirs; a ranked workgroup knows its sequence only after the ranking.  Columns
    // past the workgroup's heads get a zero query (their scores are computed and never
    // stored); it is scaled by scale * log2(e) after the table is staged.
    typename Ops::QRaw qraw;
    if constexpr (!RANKED)
        qraw = Ops::fetch_q(a.q + ((size_t)b * a.num_q_heads + h0 + min(c16, nh - 1)) * D, g);
    int raw_len;
    if constexpr (RANKED) {
        // Lane j holds sequence j's length; its rank orders the batch by attended length,
        // longest first, ties by index.  Grid slot z takes rank z within rounds of rank_round
        // slots, every second round reversed, so that the workgroups sharing a CU hold a long
        // and a short sequence.  Every wave computes the same permutation of the batch.
        const int B = a.num_seqs;
        const int len_j = (lane < B) ? a.context_lens[lane] : 0;
        int att = -1;
        if (lane < B) {
            att = clampi(len_j, 0, cap);
            if (a.window > 0) att = min(att, a.window);
        }
        int rank = 0;
        for (int j = 0; j < B; ++j) {
            const int other = __builtin_amdgcn_readlane(att, j);
            rank += (other > att || (other == att && j < lane)) ? 1 : 0;
        }
        const int z = blockIdx.z;
        const int R = a.rank_round;
        const int rnd = z / R;
        const int in_round = min(R, B - rnd * R);
        const int want = rnd * R + ((rnd & 1) ? in_round - 1 - (z - rnd * R) : z - rnd * R);
        const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < B && rank == want);
        b = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(hit));
        raw_len = __builtin_amdgcn_readlane(len_j, b);
    } else {
        raw_len = a.context_lens[b];
    }
    const int row_off = RANKED ? b * a.max_pages : 0;  // the sequence's row in the staged table
    const int32_t* trow = a.page_table + (size_t)b * a.max_pages;
    const int ctx = clampi(raw_len, 0, cap);
    if constexpr (kChecked) {
        // The length within [0, capacity], and (one workgroup per sequence and KV head) the
        // page ids of the attended positions within [0, num_pages).
        const int raw = raw_len;
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
    // Single-launch step: the current token (position ctx - 1) is read from k_new / v_new;
    // its pool slot is written by this launch and read by none of its workgroups.  As in
    // kv_page_write, a token whose raw length lies outside [1, capacity] or whose raw page id
    // lies outside [0, num_pages) is neither written nor read from k_new / v_new: attention
    // then reads the (clamped) pool like the split kernel, which keeps the step equal to
    // kv_page_write ; paged_attn_decode ; paged_attn_combine for such metadata too.
    int t_new = -1;
    if constexpr (FUSED) {
        const int raw = raw_len;
        if (raw >= 1 && raw <= cap) {
            const int pid = trow[(raw - 1) >> a.page_shift];
            if (pid >= 0 && pid < a.num_pages) t_new = raw - 1;
        }
    }
    if constexpr (RANKED)
        qraw = Ops::fetch_q(a.q + ((size_t)b * a.num_q_heads + h0 + min(c16, nh - 1)) * D, g);
    if (whole_row) {
#pragma unroll
        for (int k = 0; k < TPT; ++k) {
            const int i = tid + k * nthreads;
            if (i < t_count) s_tbl[i] = clampi(tv[k], 0, a.num_pages - 1);
        }
    }
    Ops ops;
    ops.set_q(qraw, c16 < nh ? a.qscale : 0.f);

    // The splits partition the attended positions [w0, ctx): the whole context, or with a
    // sliding window the current token and the window - 1 before it (vllm.cpp PR #383: the
    // windowed arm of the decode kernel).
    const int S = a.num_splits;
    const int w0 = (a.window > 0 && ctx > a.window) ? ctx - a.window : 0;
    const int n_att = ctx - w0;
    const int chunk = (n_att + S - 1) / S;
    const int lo = w0 + min(split * chunk, n_att);
    const int hi = min(lo + chunk, ctx);

    // Rows: pool row (page << shift | slot) times the elements between slots (Hkv * D), from
    // the KV head's dim 0; the current token's row comes from k_new / v_new.
    const uint32_t slot_elems = (uint32_t)a.num_kv_heads * D;
    const T* kpool = reinterpret_cast<const T*>(a.k_pages) + (size_t)kvh * D;
    const T* vpool = reinterpret_cast<const T*>(a.v_pages) + (size_t)kvh * D;
    const T* knew = nullptr;
    const T* vnew = nullptr;
    if constexpr (FUSED) {
        const size_t off = ((size_t)b * a.num_kv_heads + kvh) * D;
        knew = reinterpret_cast<const T*>(a.k_new) + off;
        vnew = reinterpret_cast<const T*>(a.v_new) + off;
    }
    const int pshift = a.page_shift;
    const int pmask = (1 << pshift) - 1;
    int pg0 = 0;  // first table entry of the staged slice
    auto pool_row = [&](int key) -> uint64_t {
        const uint32_t page = (uint32_t)s_tbl[row_off + (key >> pshift) - pg0];
        return (uint64_t)((page << pshift) | (uint32_t)(key & pmask)) * slot_elems;
    };
    auto krow = [&](int key) -> const T* {
        const T* p = kpool + pool_row(key);
        if constexpr (FUSED) p = (key == t_new) ? knew : p;
        return p;
    };
    auto vrow = [&](int key) -> const T* {
        const T* p = vpool + pool_row(key);
        if constexpr (FUSED) p = (key == t_new) ? vnew : p;
        return p;
    };

    // The lane's head: reference maximum the accumulator is scaled to, true running maximum,
    // and the lane's share of the sum (its 8 keys of every tile).
    float mr = -INFINITY, mt = -INFINITY, l = 0.f;
    floatx4 oacc[NC];
#pragma unroll
    for (int dt = 0; dt < NC; ++dt) oacc[dt] = floatx4{0.f, 0.f, 0.f, 0.f};

    // One tile of keys [j0, j0 + 32); keys at or past r1 are masked.
    auto compute_tile = [&](const Tile& tl, int j0, int r1, auto after_scores, auto after_pv) {
        floatx4 sacc[2];
        ops.scores(tl, sacc);
        after_scores();
        float s[2][4];
        float tmax = -INFINITY;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = j0 + 16 * st + 4 * g + i;
                s[st][i] = key < r1 ? sacc[st][i] : -INFINITY;
                tmax = fmaxf(tmax, s[st][i]);
            }
        tmax = across_groups_max<16>(tmax);  // over the 4 lane groups holding this head
        mt = fmaxf(mt, tmax);
        // Rescale only where some head of the wave outgrew its reference by more than the
        // headroom; a head that did not keeps its reference and is multiplied by exactly 1,
        // so its bits do not depend on its companions.
        const bool need = tmax > mr + kLazyRescale;
        if (__builtin_amdgcn_ballot_w64(need) != 0) {
            const float alpha = need ? fast_exp2(mr - tmax) : 1.f;  // a -inf reference gives 0
            mr = need ? tmax : mr;
            l *= alpha;
#pragma unroll
            for (int dt = 0; dt < NC; ++dt) oacc[dt] *= alpha;
        }
        const float ms = (mr == -INFINITY) ? 0.f : mr;
        float p[2][4];
        float ps = 0.f;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[st][i] = fast_exp2(s[st][i] - ms);
                ps += p[st][i];
            }
        l += ps;
        Ops::pv(tl, p, oacc);
        after_pv();
    };

    // Rows [r0, r1) of this split (r0 < r1): tiles r0 + 32 t, t = wave, wave + W, ...
    auto process = [&](int r0, int r1) {
        const int khi = r1 - 1;
        const int ntiles = (r1 - r0 + kTileKeys - 1) / kTileKeys;
        const int step = nwaves * kTileKeys;
        int t = wave;
        if (t >= ntiles) return;
        int j0 = r0 + t * kTileKeys;
        Tile A, B;
        Ops::load_k(A, krow, j0, khi, g, c16);
        Ops::load_v(A, vrow, j0, khi, g, c16);
        // The next tile's K and V, requested once this tile's scores have used its K.
        auto next = [&](Tile& N, int jn) {
            return [&N, jn, &krow, &vrow, khi, g, c16] {
                Ops::load_k(N, krow, jn, khi, g, c16);
                Ops::load_v(N, vrow, jn, khi, g, c16);
            };
        };
        for (;;) {
            int jn = j0 + step;
            compute_tile(A, j0, r1, next(B, jn), [] {});
            t += nwaves;
            j0 = jn;
            if (t >= ntiles) break;
            jn = j0 + step;
            compute_tile(B, j0, r1, next(A, jn), [] {});
            t += nwaves;
            j0 = jn;
            if (t >= ntiles) break;
        }
    };

    int pg0_last = 0;  // first table entry of the last staged slice
    if (whole_row) {
        __syncthreads();
        if (lo < hi) process(lo, hi);
    } else if (lo < hi) {
        const int first = lo >> pshift;
        const int last = (hi - 1) >> pshift;
        for (int p0 = first; p0 <= last; p0 += TCAP) {
            const int n = min(TCAP, last - p0 + 1);
            __syncthreads();
            for (int i = tid; i < n; i += nthreads)
                s_tbl[i] = clampi(trow[p0 + i], 0, a.num_pages - 1);
            __syncthreads();
            pg0 = p0;
            process(max(lo, p0 << pshift), min(hi, (p0 + n) << pshift));
            pg0_last = p0;
        }
    }

    // Single-launch step: the split holding the current token stores it into its page
    // (head group 0 only; one row per KV head, one 16-byte vector per lane of wave 0).
    if constexpr (FUSED) {
        constexpr int kVec = D * KV::kBytes / 16;
        if (hg == 0 && wave == 0 && lane < kVec && t_new >= lo && t_new < hi) {
            const uint32_t page = (uint32_t)s_tbl[row_off + (t_new >> pshift) - pg0_last];
            const size_t off =
                (size_t)((page << pshift) | (uint32_t)(t_new & pmask)) * slot_elems +
                (size_t)kvh * D;
            reinterpret_cast<uint4*>(reinterpret_cast<T*>(a.k_pages_w) + off)[lane] =
                reinterpret_cast<const uint4*>(knew)[lane];
            reinterpret_cast<uint4*>(reinterpret_cast<T*>(a.v_pages_w) + off)[lane] =
                reinterpret_cast<const uint4*>(vnew)[lane];
        }
    }

    // Every wave leaves its heads' state in LDS.  Lane (g, c16) holds dims
    // [4 g NC, 4 g NC + 4 NC) of head c16: element i of accumulator dt is dim NC (4g + i) + dt.
    l = across_groups_sum<16>(l);
    if (c16 < nh) {
        float* dst = s_o + (wave * hpw + c16) * SOH + 4 * g * NC;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int dt = 0; dt < NC; dt += 4)
                *reinterpret_cast<float4*>(dst + i * NC + dt) =
                    make_float4(oacc[dt][i], oacc[dt + 1][i], oacc[dt + 2][i], oacc[dt + 3][i]);
        if (g == 0) {
            const int j = c16 * nwaves + wave;
            s_m[j] = mr;
            s_t[j] = mt;
            s_l[j] = l;
        }
    }
    __syncthreads();

    // Merge of the waves: one thread per (head, 4 consecutive elements).  Wave w enters with
    // the factor exp(m_ref_w - M), M the split's true maximum (at least every wave's
    // reference, so the factor is at most 1; 0 for a wave that saw no row).
    PartialStore pst;
    if constexpr (FUSED) {
        // Rows of partials of this workgroup's heads: at most 16 heads x 4096 splits x 256
        // floats, far below 2^31 bytes; bases uniform over the workgroup.
        const size_t row0 = (size_t)b * a.num_q_heads + h0;
        pst.o_rsrc = __builtin_amdgcn_make_buffer_rsrc(a.partial_o + row0 * S * D, 0,
                                                       nh * S * D * 4, kRawBufferWord3);
        pst.ml_rsrc = __builtin_amdgcn_make_buffer_rsrc(a.partial_ml + row0 * S * 2, 0,
                                                        nh * S * 8, kRawBufferWord3);
    }
    auto merge_waves = [&](auto emit) {
        for (int idx = tid; idx < nh * D4; idx += nthreads) {
            const int j = idx / D4;
            const int c = idx - j * D4;
            float M = -INFINITY;
            for (int w = 0; w < nwaves; ++w) M = fmaxf(M, s_t[j * nwaves + w]);
            const float ms = (M == -INFINITY) ? 0.f : M;
            float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
            float L = 0.f;
            for (int w = 0; w < nwaves; ++w) {
                const float f = fast_exp2(s_m[j * nwaves + w] - ms);
                const float4 v = *reinterpret_cast<const float4*>(s_o + (w * hpw + j) * SOH + 4 * c);
                O.x = fmaf(v.x, f, O.x);
                O.y = fmaf(v.y, f, O.y);
                O.z = fmaf(v.z, f, O.z);
                O.w = fmaf(v.w, f, O.w);
                L = fmaf(s_l[j * nwaves + w], f, L);
            }
            const float mo = (L > 0.f) ? M * kLn2 : -INFINITY;
            emit(j, c, O, mo, L);
        }
    };

    if constexpr (!FUSED) {
        merge_waves([&](int j, int c, float4 O, float mo, float L) {
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
            merge_waves([&](int j, int c, float4 O, float mo, float L) {
                store_partial(j, c, O, mo, L);
                reinterpret_cast<float4*>(a.out)[((size_t)b * a.num_q_heads + h0 + j) * D4 + c] =
                    merge_splits(OwnPartial{make_float2(mo, L), O}, 1);
            });
            return;
        }
        merge_waves(store_partial);
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
        // Buffer resources over this workgroup's rows of partials (bases uniform over the
        // workgroup).
        const size_t row0 = (size_t)b * a.num_q_heads + h0;
        CoherentPartials src;
        src.o_rsrc = __builtin_amdgcn_make_buffer_rsrc(a.partial_o + row0 * S * D, 0,
                                                       nh * S * D * 4, kRawBufferWord3);
        src.ml_rsrc = __builtin_amdgcn_make_buffer_rsrc(a.partial_ml + row0 * S * 2, 0,
                                                        nh * S * 8, kRawBufferWord3);
        src.o_stride = D * 4;
        // The D4 lanes of a row merge it together, exchanging split weights through the
        // row's slots at the start of LDS (free once the waves' state is merged).
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

// Split partials only (paged_attn_decode).  RANKED: the batch taken longest first.
template <typename KV, int D, bool RANKED>
__global__ void __launch_bounds__(max_waves<D>() * 64)
    __attribute__((amdgpu_waves_per_eu(2))) decode_split_kernel(DecodeArgs a) {
    decode_body<KV, D, false, RANKED>(a);
}

// The single-launch step (paged_attn_decode_fused): page write, partials, last-split merge.
template <typename KV, int D, bool RANKED>
__global__ void __launch_bounds__(max_waves<D>() * 64)
    __attribute__((amdgpu_waves_per_eu(2))) decode_step_kernel(DecodeArgs a) {
    decode_body<KV, D, true, RANKED>(a);
}

template <typename KV, int D, bool FUSED, bool RANKED>
const void* decode_kernel_ptr() {
    if constexpr (FUSED)
        return (const void*)decode_step_kernel<KV, D, RANKED>;
    else
        return (const void*)decode_split_kernel<KV, D, RANKED>;
}

template <typename KV, int D, bool FUSED, bool RANKED>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
    // Waves per workgroup: enough for one pass of 32-key tiles to cover a split of the
    // table's capacity (lengths live on the device), at most max_waves<D>().  The choice
    // depends only on the split size, head_dim and dtype, never on the batch or the head
    // grouping, so a sequence's result is bit-identical whatever it is batched with, and a
    // GQA group gives the same bits as the equivalent MHA call.
    int64_t cap = (int64_t)a.max_pages << a.page_shift;
    if (a.window > 0 && a.window < cap) cap = a.window;  // positions attended at most
    const int64_t chunk = (cap + a.num_splits - 1) / a.num_splits;
    int waves = (int)std::min<int64_t>(max_waves<D>(), (chunk + kTileKeys - 1) / kTileKeys);
    waves = std::max(waves, 1);
    // A ranked batch stages every table row with kTableCap / 64 entries per thread; with too
    // few threads for that, the batch runs in grid order (the same results).
    if constexpr (RANKED) {
        if ((int64_t)a.num_seqs * a.max_pages > (int64_t)(kTableCap / 64) * waves * 64)
            return launch_typed<KV, D, FUSED, false>(a, stream);
    }
    const size_t lds = decode_lds_bytes(waves, a.heads_per_wg, D, table_cap<RANKED>());
    // Workgroups asking for more than 64 KB of LDS opt in, once per instantiation and device
    // (the largest size granted so far is kept per device; a repeated grant is harmless).
    if (lds > 64 * 1024) {
        static std::atomic<size_t> opted[kMaxDevices] = {};
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
            return hipErrorInvalidDevice;
        if (lds > opted[dev].load(std::memory_order_relaxed)) {
            hipError_t e = hipFuncSetAttribute(decode_kernel_ptr<KV, D, FUSED, RANKED>(),
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
        hipLaunchKernelGGL((decode_step_kernel<KV, D, RANKED>), grid, dim3(waves * 64), lds,
                           stream, a);
    else
        hipLaunchKernelGGL((decode_split_kernel<KV, D, RANKED>), grid, dim3(waves * 64), lds,
                           stream, a);
    return hipGetLastError();
}

template <bool FUSED, bool RANKED>
hipError_t launch_all(const DecodeArgs& a, int kv_dtype, int head_dim, hipStream_t stream) {
    if (head_dim == 64) {
        if (kv_dtype == 1) return launch_typed<F16, 64, FUSED, RANKED>(a, stream);
        if (kv_dtype == 2) return launch_typed<BF16, 64, FUSED, RANKED>(a, stream);
        return hipErrorInvalidValue;
    }
    if (kv_dtype == 1) return launch_typed<F16, 128, FUSED, RANKED>(a, stream);
    if (kv_dtype == 2) return launch_typed<BF16, 128, FUSED, RANKED>(a, stream);
    return hipErrorInvalidValue;
}

// A ranked batch (rank_round > 0) runs the instantiation that ranks it; the host sets
// rank_round only for 2 .. kRankMax sequences whose table rows fit kDecodeTableCap together.
template <bool FUSED>
hipError_t launch_mfma(const DecodeArgs& a, int kv_dtype, int head_dim, hipStream_t stream) {
    if (a.heads_per_wg < 1 || a.heads_per_wg > kCols) return hipErrorInvalidValue;
    if (a.rank_round > 0) {
        if (a.num_seqs < 2 || a.num_seqs > kRankMax ||
            (int64_t)a.num_seqs * a.max_pages > kDecodeTableCap)
            return hipErrorInvalidValue;
        return launch_all<FUSED, true>(a, kv_dtype, head_dim, stream);
    }
    return launch_all<FUSED, false>(a, kv_dtype, head_dim, stream);
}

}  // namespace

}  // namespace pa

#include "decode_valu.h"

namespace pa {

PA_DEFINE_TAKE_BAD_METADATA(take_bad_metadata_decode, g_bad_metadata_decode)

// f32 pools and head_dim 256 run on the vector units (decode_valu.h), the other 16-bit
// pools on the matrix cores.
hipError_t launch_decode(const DecodeArgs& a, int kv_dtype, int head_dim, bool fused,
                         hipStream_t stream) {
    if (kv_dtype == 0 || head_dim == 256)
        return valu::launch_decode_valu(a, kv_dtype, head_dim, fused, stream);
    return fused ? launch_mfma<true>(a, kv_dtype, head_dim, stream)
                 : launch_mfma<false>(a, kv_dtype, head_dim, stream);
}

}  // namespace pa
