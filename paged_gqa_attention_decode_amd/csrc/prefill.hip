// prefill.hip — causal packed prefill over segment descriptors, f32 MFMA.
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
//         heaviest blocks are dispatched before the light ones fill in behind them.  8 waves
//         per workgroup, all on the same 16 query rows of one head, held to 128 registers
//         for D = 64 so that two workgroups share a CU and a whole 512-token prefill is
//         resident at once (occupancy, not a second register set, hides the load latency).
//         The causal key range of the block is cut into 32-key tiles dealt round-robin to
//         the 8 waves, starting at a block-dependent wave; the 8 partial softmax states
//         merge through LDS at the end.  The page ids of the block's key range are staged in
//         LDS, 1024 at a time.
//   math  v_mfma_f32_16x16x4_f32.  Scores are computed transposed, S^T = K * Q^T (16 keys x
//         16 rows per MFMA), so each lane ends with 4 keys of ONE query row (row = lane % 16).
//         That register layout is exactly the B operand P^T of O^T += V^T * P^T, so the
//         probabilities never leave registers, and the O^T accumulator also keeps one query
//         row per lane: row max, rescale and sum stay lane-local except for one max over the
//         4 lane groups per tile.
//   data  K rows are read 4 consecutive dims per lane (16 B for f32).  The PV product takes
//         its output dims in the order d = NC * c + dt (c the accumulator row, dt the
//         16-dim block), so the V operands a lane needs for one key are NC consecutive
//         dims: one 16-byte load per key for D = 64.  Keys past the block's last visible
//         position are clamped onto it (no branch around a load) and given zero V; keys past a
//         row's own position are masked to -inf before the exponential.  Q is pre-scaled by
//         scale*log2(e).
#include "common.h"

namespace pa {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4 mfma16(float a, float b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Four consecutive elements starting at p, widened to f32.
template <typename KV>
__device__ __forceinline__ void load4(const typename KV::storage* p, float* out) {
    if constexpr (KV::kBytes == 4) {
        const float4 t = *reinterpret_cast<const float4*>(p);
        out[0] = t.x;
        out[1] = t.y;
        out[2] = t.z;
        out[3] = t.w;
    } else {
        const uint2 t = *reinterpret_cast<const uint2*>(p);
        widen_word(KV{}, t.x, out);
        widen_word(KV{}, t.y, out + 2);
    }
}

constexpr int kWaves = 8;
constexpr int kRows = 16;         // query rows per workgroup
constexpr int kTileKeys = 32;     // keys per wave per step (two 16-key MFMA blocks)
constexpr int kTablePages = 1024; // page ids staged in LDS per slice of the key range

// One wave's operands for one 32-key tile.
template <int D>
struct PrefillTile {
    // K operand: lane (g, c16) of block st holds K[j0 + 16 st + c16][16c + 4g + kk].
    float kf[2][D / 16][4];
    // V^T operand of MFMA (st, i, dt): lane (g, c16) holds V[j0 + 16 st + 4g + i][NC c16 + dt].
    float vf[2][4][D / 16];
};

template <typename KV, int D>
__global__ void __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(D <= 64 ? 4 : 2)))
    prefill_kernel(PrefillArgs a) {
    using T = typename KV::storage;
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

    const int32_t* dsc = a.seg_desc + 4 * (size_t)blockIdx.z;
    const int start = dsc[0];
    int len = dsc[1];
    const int a0 = dsc[2];
    const int ti = dsc[3];
    const int cap = a.max_pages << a.page_shift;
    if (start < 0 || start >= a.total_tokens || len <= 0 || a0 < 0 || a0 >= cap || ti < 0 ||
        ti >= a.num_tables)
        return;
    len = min(min(len, a.total_tokens - start), cap - a0);
    const int h = (int)(blockIdx.x % (unsigned)a.num_q_heads);
    const int r0 = (a.q_blocks - 1 - (int)(blockIdx.x / (unsigned)a.num_q_heads)) * kRows;
    if (r0 >= len) return;

    const int kvh = h / a.group;
    const int kmax = a0 + min(r0 + kRows - 1, len - 1);  // last key any row here may see
    const int r = r0 + c16;
    const bool rvalid = r < len;
    const int qend = a0 + r;  // this lane's row sees keys 0..qend

    const int32_t* trow = a.page_table + (size_t)ti * a.max_pages;

    // Q^T operand: lane (g, c16) holds Q[row][16c + 4g + kk], kk = 0..3.
    float qr[NC][4];
    {
        const float* qp =
            a.q + ((size_t)(start + min(r, len - 1)) * a.num_q_heads + h) * D + 4 * g;
        const float qs = rvalid ? a.qscale : 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const float4 t = *reinterpret_cast<const float4*>(qp + 16 * c);
            qr[c][0] = t.x * qs;
            qr[c][1] = t.y * qs;
            qr[c][2] = t.z * qs;
            qr[c][3] = t.w * qs;
        }
    }

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

    // Keys past khi are clamped onto khi (a valid row, so no branch guards a load: the wait
    // for the current tile then never covers the loads of the next one).  Only the last
    // slice has such keys (khi = kmax there); their scores are masked for every row, and
    // their V rows are zeroed in compute_tile.
    auto load_tile = [&](PrefillTile<D>& tl, int t) {
        const int j0 = t * kTileKeys;
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const T* kr = kp + row_off(min(j0 + 16 * st + c16, khi)) + 4 * g;
#pragma unroll
            for (int c = 0; c < NC; ++c) load4<KV>(kr + 16 * c, tl.kf[st][c]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const T* vr = vp + row_off(min(j0 + 16 * st + 4 * g + i, khi)) + NC * c16;
#pragma unroll
                for (int d4 = 0; d4 < NC; d4 += 4) load4<KV>(vr + d4, &tl.vf[st][i][d4]);
            }
        }
    };

    float m = -INFINITY;
    float lsum = 0.f;
    floatx4 oacc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) oacc[c] = floatx4{0.f, 0.f, 0.f, 0.f};

    auto compute_tile = [&](const PrefillTile<D>& tl, int t) {
        const int j0 = t * kTileKeys;
        // S^T = K Q^T: lane (g, c16) gets scores of keys j0 + 16 st + 4g + i for row c16.
        floatx4 sacc[2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            sacc[st] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    sacc[st] = mfma16(tl.kf[st][c][kk], qr[c][kk], sacc[st]);
        }

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

        // O^T += V^T P^T (accumulator row c of block dt is output dim NC c + dt).  A key past
        // khi holds a copy of row khi: its V is zeroed so that its zero weight leaves O
        // unchanged whatever that row holds.
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool vok = j0 + 16 * st + 4 * g + i <= khi;
#pragma unroll
                for (int dt = 0; dt < NC; ++dt)
                    oacc[dt] = mfma16(vok ? tl.vf[st][i][dt] : 0.f, p[st][i], oacc[dt]);
            }
    };

    // This wave's tiles of a slice: t = t0 + w, t0 + w + 8, ... with w = (wave + block) % 8,
    // so the query blocks of a head, which all read the same K/V, start on different tiles
    // instead of all reading tile t0 at once.  The rotation depends only on the block's own
    // first row, so a segment computes the same bits wherever it sits in the packed batch.
    const int first = (wave + (r0 / kRows)) % kWaves;
    auto run_tiles = [&](int t, int t_end) {
        for (; t < t_end; t += kWaves) {
            PrefillTile<D> tl;
            load_tile(tl, t);
            compute_tile(tl, t);
        }
    };

    const int last_pg = kmax >> pshift;
    for (pg0 = 0; pg0 <= last_pg; pg0 += kTablePages) {
        const int n = min(kTablePages, last_pg - pg0 + 1);
        if (pg0 > 0) __syncthreads();  // every wave is done with the previous slice
        for (int i = threadIdx.x; i < n; i += kWaves * 64)
            s_tbl[i] = clampi(trow[pg0 + i], 0, a.num_pages - 1);
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

template <typename KV, int D>
hipError_t launch_typed(const PrefillArgs& a, int q_blocks, hipStream_t stream) {
    const dim3 grid(q_blocks * a.num_q_heads, 1, a.num_segs);
    hipLaunchKernelGGL((prefill_kernel<KV, D>), grid, dim3(kWaves * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int kv_dtype, int head_dim, int q_blocks,
                          hipStream_t stream) {
    (void)q_blocks;
    const int qb = q_blocks;
    if (head_dim == 64) {
        if (kv_dtype == 0) return launch_typed<F32, 64>(a, qb, stream);
        if (kv_dtype == 1) return launch_typed<F16, 64>(a, qb, stream);
        return launch_typed<BF16, 64>(a, qb, stream);
    }
    if (kv_dtype == 0) return launch_typed<F32, 128>(a, qb, stream);
    if (kv_dtype == 1) return launch_typed<F16, 128>(a, qb, stream);
    return launch_typed<BF16, 128>(a, qb, stream);
}

}  // namespace pa
