// prefill.hip — causal packed prefill over segment descriptors on the MFMA units.
//
// Method (crucible, "Paged attention results": descriptors {packed_start, chunk_len,
// absolute_start, table_index}; a tile never crosses request ownership; a packed row at
// absolute P reads only its own request's positions 0..P; every logical page a tile crosses
// is translated separately.  The online softmax of the same page: m' = max(m, tile max),
// rescale by exp(m - m'), accumulate exp(score - m') and its weighted V, divide after the
// last visible tile.  crucible README scheduler section: chunk row r attends 0 ..= done + r).
//
// gfx950 mapping
//   grid  (ceil(max_chunk_len / 16) * Hq, 1, num_segs): x enumerates (query block, head)
//         with the last query blocks (longest causal history) of every head first, so the
//         heaviest blocks are dispatched before the light ones fill in behind them.  For one
//         prompt at D = 64 every second round of CU-count workgroups runs in reverse, so that
//         a CU's two workgroups are a heavy and a light block (they share its matrix cores
//         and memory pipeline, and a CU holding two heavy blocks set the end).  A call
//         with 2 .. kRankSegs segments takes them heaviest first (by last position), so
//         the longest histories are dispatched first whatever the descriptor order.  8 waves
//         per workgroup, all on the same 16 query rows of one head, held to 128 registers
//         for D = 64 so that two workgroups share a CU and a whole 512-token prefill is
//         resident at once (occupancy, not a second register set, hides the load latency);
//         an f32 grid of more than two workgroups per CU runs a build held to 85 registers,
//         three workgroups per CU.
//         The causal key range of the block is cut into 32-key tiles dealt round-robin to
//         the 8 waves, starting at a block-dependent wave; the 8 partial softmax states
//         merge through LDS at the end.  With a 16-bit pool a wave requests its next tile's
//         K once the scores have used the current K, and its V once the PV product has used
//         the current V.  The page ids of the block's key range are staged in
//         LDS, 1024 at a time.
//   math  Scores are computed transposed, S^T = K * Q^T (16 keys x 16 rows per MFMA), so
//         each lane ends with 4 keys of ONE query row (row = lane % 16).  That register
//         layout is the B operand P^T of O^T += V^T * P^T, so the probabilities never leave
//         registers, and the O^T accumulator also keeps one query row per lane: row max,
//         rescale and sum stay lane-local except for one max over the 4 lane groups per
//         tile.  Q is pre-scaled by scale*log2(e).  Two operand sets share this frame:
//         - f32 K/V: v_mfma_f32_16x16x4_f32.  K rows are read 4 consecutive dims per lane
//           (16 B).  The PV product takes its output dims in the order d = NC * c + dt (c
//           the accumulator row, dt the 16-dim block), so the V operands a lane needs for
//           one key are NC consecutive dims: one 16-byte load per key for D = 64.
//         - f16/bf16 K/V: v_mfma_f32_16x16x32_{f16,bf16}, K and V straight from the pool.
//           The f32 operands Q and P are each split into two terms of the pool's 16-bit
//           type, x = hi + lo, and both terms are multiplied (K q_hi + K q_lo, V p_hi +
//           V p_lo): the residual of the split is below 2^-16 |x| for bf16 and 2^-22 |x|
//           for f16, where one rounding of Q and P to bf16 alone (2^-9 |x|) can exceed the
//           16-bit tolerance on standard-normal inputs.  A lane's 8 K elements of one MFMA
//           are 8 consecutive dims (one 16-byte load).  For PV the contraction runs over
//           keys; the MFMA pairs A's and B's k index through the same (lane group, element)
//           slot, so the keys are assigned to slots as the score layout already holds them:
//           element e of lane group g is key 16 (e / 4) + 4 g + e % 4, and P^T is the lane's
//           own 8 probabilities.  V is loaded as NC consecutive dims of each of those 8 keys
//           (8 or 16 bytes per key) and regrouped into per-dim-block operands by byte
//           permutes.
//   keys  Keys past the block's last visible position are clamped onto it (no branch around
//         a load); keys past a row's own position are masked to -inf before the
//         exponential, so their weight is exactly zero.
//   checks The checked build also marks a malformed descriptor or a staged page id out of
//         range (every build clamps the page ids and skips the descriptor).
#include <type_traits>

#include "mfma_tiles.h"

namespace pa {

// Checked build: set when a descriptor or a page id of a segment's key range is out of range.
__device__ int g_bad_metadata_prefill;

namespace {

constexpr int kWaves = 8;
constexpr int kRows = 16;         // query rows per workgroup
constexpr int kTablePages = 1024; // page ids staged in LDS per slice of the key range

// Waves per SIMD the registers are budgeted for: 4 at D = 64 (two workgroups per CU), 2 at
// D = 128; the f32 pool at D = 64 also has a 6-wave build (three workgroups per CU, 77
// registers, no spills) for grids too large to be resident at two per CU.
template <typename KV, int D>
constexpr int default_occupancy() { return D <= 64 ? 4 : 2; }

template <typename KV, int D, int OCC>
__global__ void __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(OCC)))
    prefill_kernel(PrefillArgs a) {
    using T = typename KV::storage;
    using Ops = TileOps<KV, D>;
    constexpr int NC = D / 16;             // 16-wide dimension blocks

    __shared__ int s_tbl[kTablePages];
    __shared__ float s_m[kWaves][kRows];
    __shared__ float s_l[kWaves][kRows];
    // Per wave, row and dim; rows padded by one float, so that both the lanes' writes (16
    // rows x 4 dim groups) and the merge's reads (consecutive dims) hit distinct banks.
    __shared__ float s_o[kWaves][kRows][D + 1];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;    // MFMA k-group: 4 lane groups of 16
    const int c16 = lane & 15;  // query row within the block (B/D operand column)

    // The segment of this workgroup's z slot.  Ranked calls take the segments heaviest first
    // (by last position, absolute start + length; ties by index; a segment the checks below
    // skip last), so the blocks with the longest histories are dispatched first wherever
    // their segment sits in the descriptor array.  A permutation of the work: every segment
    // computes the same bits in any slot.  (The slot's descriptor is read once, after the
    // ranking: reading the slot's own first and another after a move measured slower.)
    int seg = (int)blockIdx.z;
    if (a.rank_segs) {
        const int cap0 = a.max_pages << a.page_shift;
        int wt = -1;  // lane i: segment i's last position + 1, -1 if it is skipped
        if (lane < a.num_segs) {
            const int32_t* d = a.seg_desc + 4 * lane;
            const int s0 = d[0], l0 = d[1], b0 = d[2], t0 = d[3];
            if (s0 >= 0 && s0 < a.total_tokens && l0 > 0 && b0 >= 0 && b0 < cap0 && t0 >= 0 &&
                t0 < a.num_tables)
                wt = b0 + min(min(l0, a.total_tokens - s0), cap0 - b0);
        }
        int rk = 0;
        for (int j = 0; j < a.num_segs; ++j) {
            const int other = __builtin_amdgcn_readlane(wt, j);
            rk += (other > wt || (other == wt && j < lane)) ? 1 : 0;
        }
        const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < a.num_segs && rk == seg);
        seg = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(hit));
    }
    const int32_t* dsc = a.seg_desc + 4 * (size_t)seg;
    const int start = dsc[0];
    int len = dsc[1];
    const int a0 = dsc[2];
    const int ti = dsc[3];
    const int cap = a.max_pages << a.page_shift;
    if constexpr (kChecked) {
        // A non-empty segment lies inside the packed rows, its positions inside the table's
        // capacity, and its table row exists; a negative length is malformed.
        if (threadIdx.x == 0 && blockIdx.x == 0 &&
            (len < 0 || (len > 0 && (start < 0 || len > a.total_tokens - start || a0 < 0 ||
                                     len > cap - a0 || ti < 0 || ti >= a.num_tables))))
            mark_bad(&g_bad_metadata_prefill);
    }
    if (start < 0 || start >= a.total_tokens || len <= 0 || a0 < 0 || a0 >= cap || ti < 0 ||
        ti >= a.num_tables)
        return;
    len = min(min(len, a.total_tokens - start), cap - a0);
    // The workgroup's rank in the heaviest-first order: blockIdx.x itself, or with rounds of
    // round_wgs workgroups (one per CU) every second round reversed, so that a CU's second
    // workgroup is one of the lightest blocks and its first one of the heaviest.
    int rank = (int)blockIdx.x;
    if (a.round_wgs > 0) {
        const int rnd = rank / a.round_wgs;
        const int in_round = min(a.round_wgs, (int)gridDim.x - rnd * a.round_wgs);
        if (rnd & 1) rank = rnd * a.round_wgs + in_round - 1 - (rank - rnd * a.round_wgs);
    }
    const int h = rank % a.num_q_heads;
    const int r0 = (a.q_blocks - 1 - rank / a.num_q_heads) * kRows;
    if (r0 >= len) return;

    const int kvh = h / a.group;
    const int kmax = a0 + min(r0 + kRows - 1, len - 1);  // last key any row here may see
    const int r = r0 + c16;
    const bool rvalid = r < len;
    const int qend = a0 + r;  // this lane's row sees keys 0..qend

    const int32_t* trow = a.page_table + (size_t)ti * a.max_pages;

    Ops ops;
    ops.load_q(a.q + ((size_t)(start + min(r, len - 1)) * a.num_q_heads + h) * D,
               rvalid ? a.qscale : 0.f, g);

    const T* kp = reinterpret_cast<const T*>(a.k_pages) + (size_t)kvh * D;
    const T* vp = reinterpret_cast<const T*>(a.v_pages) + (size_t)kvh * D;
    const size_t slot_stride = (size_t)a.num_kv_heads * D;
    const int pshift = a.page_shift;
    const int pmask = (1 << pshift) - 1;
    // The key range is walked in slices of kTablePages pages whose ids are staged in LDS
    // (one slice unless the history is longer than kTablePages pages); pg0 is the current
    // slice's first page and khi its last key.
    int pg0 = 0;
    int khi = kmax;
    auto row_off = [&](int key) -> size_t {
        const int page = s_tbl[(key >> pshift) - pg0];
        return (((size_t)page << pshift) | (size_t)(key & pmask)) * slot_stride;
    };
    auto krow = [&](int key) -> const T* { return kp + row_off(key); };
    auto vrow = [&](int key) -> const T* { return vp + row_off(key); };

    float m = -INFINITY;
    float lsum = 0.f;
    floatx4 oacc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) oacc[c] = floatx4{0.f, 0.f, 0.f, 0.f};

    // Keys past khi are clamped onto khi (a valid row, so no branch guards a load: the wait
    // for the current tile then never covers the loads of the next one).  Only the last
    // slice has such keys (khi = kmax there); their scores are masked for every row.
    auto compute_tile = [&](const typename Ops::Tile& tl, int t, auto after_scores,
                            auto after_pv) {
        const int j0 = t * kTileKeys;
        floatx4 sacc[2];
        ops.scores(tl, sacc);
        after_scores();

        float tmax = -INFINITY;
        float s[2][4];
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = j0 + 16 * st + 4 * g + i;
                s[st][i] = (rvalid && key <= qend) ? sacc[st][i] : -INFINITY;
                tmax = fmaxf(tmax, s[st][i]);
            }
        tmax = across_groups_max<16>(tmax);  // over the 4 lane groups holding this row
        const float mn = fmaxf(m, tmax);
        const float ms = (mn == -INFINITY) ? 0.f : mn;
        const float alpha = fast_exp2(m - ms);
        float p[2][4];
        float ps = 0.f;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[st][i] = fast_exp2(s[st][i] - ms);
                ps += p[st][i];
            }
        lsum = fmaf(lsum, alpha, ps);
        m = mn;
#pragma unroll
        for (int dt = 0; dt < NC; ++dt) oacc[dt] *= alpha;
        Ops::pv(tl, p, oacc);
        after_pv();
    };

    // This wave's tiles of a slice: t = t0 + w, t0 + w + 8, ... with w = (wave + block) % 8,
    // so the query blocks of a head, which all read the same K/V, start on different tiles
    // instead of all reading tile t0 at once.  The rotation depends only on the block's own
    // first row, so a segment computes the same bits wherever it sits in the packed batch.
    const int first = (wave + (r0 / kRows)) % kWaves;
    // 16-bit pools: the next tile's K is requested as soon as the scores have consumed this
    // tile's K, and its V once the PV product has consumed this tile's V, so the loads overlap
    // the softmax and the PV product without a second tile's worth of live registers.  Past
    // the wave's last tile the requests go on unguarded (keys clamp onto khi: cache hits,
    // never used), since a load guarded by a branch makes the compiler's wait counts assume
    // the path without it, and a counted, peeled schedule keeps two tiles live and spills.
    // The f32 pool keeps one tile in flight: its tiles are twice the bytes, its MFMA pipe is
    // already the shared resource, and the early requests measured slower there.
    auto run_tiles = [&](int t, int t_end) {
        if constexpr (std::is_same_v<KV, F32>) {
            for (; t < t_end; t += kWaves) {
                typename Ops::Tile tl;
                Ops::load_k(tl, krow, t * kTileKeys, khi, g, c16);
                Ops::load_v(tl, vrow, t * kTileKeys, khi, g, c16);
                compute_tile(tl, t, [] {}, [] {});
            }
        } else {
            if (t >= t_end) return;
            typename Ops::Tile A, B;
            Ops::load_k(A, krow, t * kTileKeys, khi, g, c16);
            Ops::load_v(A, vrow, t * kTileKeys, khi, g, c16);
            for (;;) {
                int jn = (t + kWaves) * kTileKeys;
                compute_tile(A, t, [&] { Ops::load_k(B, krow, jn, khi, g, c16); },
                             [&] { Ops::load_v(B, vrow, jn, khi, g, c16); });
                t += kWaves;
                if (t >= t_end) break;
                jn = (t + kWaves) * kTileKeys;
                compute_tile(B, t, [&] { Ops::load_k(A, krow, jn, khi, g, c16); },
                             [&] { Ops::load_v(A, vrow, jn, khi, g, c16); });
                t += kWaves;
                if (t >= t_end) break;
            }
        }
    };

    const int last_pg = kmax >> pshift;
    for (pg0 = 0; pg0 <= last_pg; pg0 += kTablePages) {
        const int n = min(kTablePages, last_pg - pg0 + 1);
        if (pg0 > 0) __syncthreads();  // every wave is done with the previous slice
        for (int i = threadIdx.x; i < n; i += kWaves * 64) {
            const int v = trow[pg0 + i];
            if (v < 0 || v >= a.num_pages) mark_bad(&g_bad_metadata_prefill);
            s_tbl[i] = clampi(v, 0, a.num_pages - 1);
        }
        __syncthreads();
        khi = min(kmax, ((pg0 + n) << pshift) - 1);
        // A slice starts on a tile boundary: kTablePages pages hold a multiple of 32 keys.
        run_tiles(((pg0 << pshift) / kTileKeys) + first, khi / kTileKeys + 1);
    }

    lsum = across_groups_sum<16>(lsum);
    if (g == 0) {
        s_m[wave][c16] = m;
        s_l[wave][c16] = lsum;
    }
#pragma unroll
    for (int dt = 0; dt < NC; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) s_o[wave][c16][NC * (4 * g + i) + dt] = oacc[dt][i];
    __syncthreads();

    for (int idx = threadIdx.x; idx < kRows * D; idx += kWaves * 64) {
        const int q = idx / D;
        const int d = idx - q * D;
        if (r0 + q >= len) continue;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][q]);
        const float ms = (M == -INFINITY) ? 0.f : M;
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = fast_exp2(s_m[w][q] - ms);
            L = fmaf(s_l[w][q], f, L);
            O = fmaf(s_o[w][q][d], f, O);
        }
        a.out[((size_t)(start + r0 + q) * a.num_q_heads + h) * D + d] = (L > 0.f) ? O / L : 0.f;
    }
}

// dense: more (query block, head) workgroups have rows than two per CU can hold at once
// (several prompts, or one long one).  Then the f32 D = 64 build at three workgroups per CU
// runs, so that more of the grid is resident at once; the blocks of a smaller grid are
// resident anyway and keep the larger register budget, whose schedule is faster per
// workgroup.  Both builds perform the same operations in the same order, so a segment's bits
// do not depend on which one ran.
template <typename KV, int D>
hipError_t launch_typed(const PrefillArgs& a, int q_blocks, bool dense, hipStream_t stream) {
    const dim3 grid(q_blocks * a.num_q_heads, 1, a.num_segs);
    constexpr int OCC = default_occupancy<KV, D>();
    if constexpr (std::is_same_v<KV, F32> && D == 64) {
        if (dense) {
            hipLaunchKernelGGL((prefill_kernel<KV, D, 6>), grid, dim3(kWaves * 64), 0, stream, a);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((prefill_kernel<KV, D, OCC>), grid, dim3(kWaves * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

PA_DEFINE_TAKE_BAD_METADATA(take_bad_metadata_prefill, g_bad_metadata_prefill)

hipError_t launch_prefill(const PrefillArgs& a, int kv_dtype, int head_dim, int q_blocks,
                          bool dense, hipStream_t stream) {
    if (head_dim == 64) {
        if (kv_dtype == 0) return launch_typed<F32, 64>(a, q_blocks, dense, stream);
        if (kv_dtype == 1) return launch_typed<F16, 64>(a, q_blocks, dense, stream);
        return launch_typed<BF16, 64>(a, q_blocks, dense, stream);
    }
    if (kv_dtype == 0) return launch_typed<F32, 128>(a, q_blocks, dense, stream);
    if (kv_dtype == 1) return launch_typed<F16, 128>(a, q_blocks, dense, stream);
    return launch_typed<BF16, 128>(a, q_blocks, dense, stream);
}

}  // namespace pa
