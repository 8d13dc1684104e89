// common.h — device helpers and launcher declarations shared by the gfx950 kernels.
//
// Element storage: K/V pages hold f32, IEEE binary16 or bfloat16 values.  Kernels move them
// in 16-byte (128-bit) lane loads and widen to f32 in registers; all arithmetic is f32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr float kLog2e = 1.4426950408889634f;  // log2(e): scores are kept in base-2 units
constexpr float kLn2 = 0.6931471805599453f;    // ln(2): back to natural-log units on store
constexpr int kMaxDevices = 64;  // devices whose host-side launch facts are cached

// ---------------------------------------------------------------- checked build

// Built with -DPAGED_ATTN_CHECKED, the kernels also record device metadata outside its
// documented range -- under the same conditions in which every build clamps or skips it --
// in a flag of their translation unit, which the entry points read after synchronising.
#ifdef PAGED_ATTN_CHECKED
constexpr bool kChecked = true;
#else
constexpr bool kChecked = false;
#endif

// Mark `flag` (a per-translation-unit device word) in the checked build; nothing otherwise.
__device__ __forceinline__ void mark_bad(int* flag) {
    if constexpr (kChecked) *reinterpret_cast<volatile int*>(flag) = 1;
}

// ---------------------------------------------------------------- cache element types

struct F32 {
    using storage = float;
    static constexpr int kBytes = 4;
};
struct F16 {
    using storage = uint16_t;
    static constexpr int kBytes = 2;
};
struct BF16 {
    using storage = uint16_t;
    static constexpr int kBytes = 2;
};

// Widen the elements packed in one 32-bit word.
__device__ __forceinline__ void widen_word(F32, uint32_t w, float* out) {
    out[0] = __builtin_bit_cast(float, w);
}
__device__ __forceinline__ void widen_word(F16, uint32_t w, float* out) {
    out[0] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
    out[1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
__device__ __forceinline__ void widen_word(BF16, uint32_t w, float* out) {
    out[0] = __builtin_bit_cast(float, w << 16);
    out[1] = __builtin_bit_cast(float, w & 0xffff0000u);
}

// ---------------------------------------------------------------- cross-lane reductions

// DPP move within 16-lane rows (the source lane always exists for these controls).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}

constexpr int kDppRor8 = 0x128;        // row_ror:8: lane i <- lane (i+8) mod 16 (= xor 8)
constexpr int kDppRor4 = 0x124;        // row_ror:4: lane i <- lane (i+4) mod 16
constexpr int kDppQuadXor1 = 0xb1;     // quad_perm [1,0,3,2]: lane i <- lane i ^ 1
constexpr int kDppQuadXor2 = 0x4e;     // quad_perm [2,3,0,1]: lane i <- lane i ^ 2

// Exchanges across 16-lane rows go through the LDS crossbar: ds_swizzle for xor 16 (inside
// each half-wave) and ds_bpermute for xor 32.  (The gfx950 permlane16/32 row swaps would
// stay in the VALU, but this compiler folds their two results as if they were equal, so
// they are not used.)
__device__ __forceinline__ float lane_xor16(float v) {
    // swizzle bitmask mode: and 0x1f, or 0, xor 0x10
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v),
                                                                 0x401f));
}
__device__ __forceinline__ float lane_xor32(float v) { return __shfl_xor(v, 32); }

// Reduction ACROSS the groups of N lanes of a wave: lanes with the same index within their
// group of N combine, and every lane ends with the same result for its index.
template <int N>
__device__ __forceinline__ float across_groups_sum(float v) {
    if constexpr (N <= 8) v += dpp_mov<kDppRor8>(v);
    if constexpr (N <= 16) v += lane_xor16(v);
    if constexpr (N <= 32) v += lane_xor32(v);
    return v;
}

template <int N>
__device__ __forceinline__ float across_groups_max(float v) {
    if constexpr (N <= 8) v = fmaxf(v, dpp_mov<kDppRor8>(v));
    if constexpr (N <= 16) v = fmaxf(v, lane_xor16(v));
    if constexpr (N <= 32) v = fmaxf(v, lane_xor32(v));
    return v;
}

// Maximum over each group of N consecutive lanes (N = 16, 32 or 64, groups aligned to N);
// every lane of a group ends with its group's maximum.  Within a 16-lane row: the quad's
// two xors, then rotations by 4 and 8 (after the quad steps a lane's quad holds one value,
// so the rotations cover the other three quads).
template <int N>
__device__ __forceinline__ float within_group_max(float v) {
    v = fmaxf(v, dpp_mov<kDppQuadXor1>(v));
    v = fmaxf(v, dpp_mov<kDppQuadXor2>(v));
    v = fmaxf(v, dpp_mov<kDppRor4>(v));
    v = fmaxf(v, dpp_mov<kDppRor8>(v));
    if constexpr (N >= 32) v = fmaxf(v, lane_xor16(v));
    if constexpr (N >= 64) v = fmaxf(v, lane_xor32(v));
    return v;
}

// Orders one wave's LDS accesses around it for the compiler: the LDS executes a wave's
// accesses in issue order, so a lane's read after this sees what other lanes of the same
// wave wrote before it, and a write after it cannot overtake an earlier read.
__device__ __forceinline__ void wave_lds_order() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return min(max(x, lo), hi); }

// ---------------------------------------------------------------- split merge

constexpr int kMergeChunk = 32;  // splits whose partials are in flight at once

// Where one row's split partials are read from, for one float4 column of the output:
// ml(s) = (m_s, l_s) in natural-log units and o(s) = that column of O_s, for s < S.
//
// Plain loads: the partials were written by an earlier launch.  A slot past S reads split
// S - 1 again (a cache hit), so no branch guards the loads.
struct PlainPartials {
    const float2* ml;
    const float4* po;
    int stride4;  // float4s between the column's entries of consecutive splits
    __device__ __forceinline__ float2 ml_at(int s, int S) const { return ml[min(s, S - 1)]; }
    __device__ __forceinline__ float4 o_at(int s, int S) const {
        return po[(size_t)min(s, S - 1) * stride4];
    }
};

// Device-scope loads: the partials were written by other workgroups of the running launch
// with device-scope stores, so each load has to be served by the device's coherence point,
// never by a stale line in this XCD's L2 (the cache-policy bit below; 16 bytes per access
// through a buffer resource whose base is uniform over the workgroup).  These loads are not
// cache hits, so a slot past S does not read split S - 1 again: its offset is moved past the
// resource's range (at most 2^31 bytes), where a buffer load returns zeros without a memory
// access, and no branch separates the loads.
constexpr int kDeviceScopeLoad = 16;  // buffer-instruction cache policy: device scope
constexpr uint32_t kRawBufferWord3 = 0x00020000;  // untyped 32-bit buffer, no swizzle
constexpr uint32_t kPastRange = 0x80000000u;      // a buffer offset beyond every resource here
struct CoherentPartials {
    __amdgpu_buffer_rsrc_t o_rsrc, ml_rsrc;
    uint32_t o_off;     // bytes from o_rsrc's base to this column of split 0
    uint32_t o_stride;  // bytes between consecutive splits
    uint32_t ml_off;    // bytes from ml_rsrc's base to (m, l) of split 0
    // (m, l) of split s, zeros past S (never live: l = 0)
    __device__ __forceinline__ float2 ml_at(int s, int S) const {
        const uint32_t off = (s < S) ? ml_off + (uint32_t)s * 8u : kPastRange;
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(ml_rsrc, off, 0, kDeviceScopeLoad);
        return make_float2(__uint_as_float(v[0]), __uint_as_float(v[1]));
    }
    // this column of O_s, zeros past S
    __device__ __forceinline__ float4 o_at(int s, int S) const {
        const uint32_t off = (s < S) ? o_off + (uint32_t)s * o_stride : kPastRange;
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(o_rsrc, off, 0, kDeviceScopeLoad);
        return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]),
                           __uint_as_float(v[3]));
    }
};

// A single split's partial held in registers: the source of the merge when a launch has one
// split, so that its output is the merge's arithmetic on that one partial.
struct OwnPartial {
    float2 ml;
    float4 o;
    __device__ __forceinline__ float2 ml_at(int s, int S) const {
        return (s < S) ? ml : make_float2(-INFINITY, 0.f);
    }
    __device__ __forceinline__ float4 o_at(int s, int S) const {
        return (s < S) ? o : make_float4(0.f, 0.f, 0.f, 0.f);
    }
};

// The merged column: acc / L, or zeros when no split saw a position.  Adding +0 makes a zero
// result +0 whatever the signs of the zero terms that formed it, so merges that skip an
// idle split and merges that add its zero product give the same bits.
__device__ __forceinline__ float4 merge_finish(float4 acc, float L) {
    if (!(L > 0.f)) return make_float4(0.f, 0.f, 0.f, 0.f);
    return make_float4(acc.x / L + 0.f, acc.y / L + 0.f, acc.z / L + 0.f, acc.w / L + 0.f);
}

// Merge of one (sequence, head) row's split partials for one float4 column of the output,
// by one lane on its own (the single-split step, whose one partial is in registers).  One
// pass with a running maximum; idle splits (l_s = 0) contribute nothing, whatever their O
// holds.  merge_row below is the same arithmetic shared over a row's lanes, and gives the
// same bits.
template <typename Src>
__device__ __forceinline__ float4 merge_splits(const Src& src, int S) {
    float M = -INFINITY;
    float L = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = 0; s0 < S; s0 += kMergeChunk) {
        float2 v[kMergeChunk];
        float4 o[kMergeChunk];
#pragma unroll
        for (int k = 0; k < kMergeChunk; ++k) {
            v[k] = src.ml_at(s0 + k, S);
            o[k] = src.o_at(s0 + k, S);
        }
        float cm = -INFINITY;
#pragma unroll
        for (int k = 0; k < kMergeChunk; ++k) {
            const bool live = (s0 + k < S) && v[k].y > 0.f;
            cm = fmaxf(cm, live ? v[k].x : -INFINITY);
        }
        if (cm == -INFINITY) continue;  // nothing live in this chunk
        const float Mn = fmaxf(M, cm);
        const float r = fast_exp2((M - Mn) * kLog2e);  // 0 while M is still -inf
        L *= r;
        acc.x *= r;
        acc.y *= r;
        acc.z *= r;
        acc.w *= r;
#pragma unroll
        for (int k = 0; k < kMergeChunk; ++k) {
            const bool live = (s0 + k < S) && v[k].y > 0.f;
            const float w = live ? fast_exp2((v[k].x - Mn) * kLog2e) : 0.f;
            L = live ? fmaf(w, v[k].y, L) : L;
            acc.x = live ? fmaf(w, o[k].x, acc.x) : acc.x;
            acc.y = live ? fmaf(w, o[k].y, acc.y) : acc.y;
            acc.z = live ? fmaf(w, o[k].z, acc.z) : acc.z;
            acc.w = live ? fmaf(w, o[k].w, acc.w) : acc.w;
        }
        M = Mn;
    }
    return merge_finish(acc, L);
}

// The same merge computed by the N consecutive lanes of one wave that own a row (N = D / 4;
// lane c of them produces float4 column c).  Per chunk of C splits, every lane requests its
// column's C O entries and the (m, l) of the chunk's splits it owns (c, c + N, ...), all
// before any is used (one memory round trip); one cross-lane maximum gives the chunk's
// maximum; the owning lane computes each split's weight exp(m_s - M) once and passes it with
// l_s through the row's LDS slots xw (float2, used by this row's lanes only), so the
// other lanes spend five FMAs per split instead of an exponential and a maximum.  The
// operations and their order are merge_splits's, so the results are the same bits.
// DEAD_FINITE: every O entry of an idle split is finite (partials written by the decode
// itself), so adding its zero-weighted product needs no select.
template <int N, bool DEAD_FINITE, int C, typename Src>
__device__ __forceinline__ float4 merge_row_chunks(const Src& src, int S, int c, float2* xw) {
    constexpr int PER = N <= C ? C / N : 1;  // splits owned per lane
    float M = -INFINITY;
    float L = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = 0; s0 < S; s0 += C) {
        float4 o[C];
#pragma unroll
        for (int k = 0; k < C; ++k) o[k] = src.o_at(s0 + k, S);
        float2 v[PER];
        bool live[PER];
        float cm = -INFINITY;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int k = c + i * N;
            const bool mine = k < C;  // lanes past the chunk own none
            v[i] = mine ? src.ml_at(s0 + k, S) : make_float2(-INFINITY, 0.f);
            live[i] = mine && (s0 + k < S) && v[i].y > 0.f;
            cm = fmaxf(cm, live[i] ? v[i].x : -INFINITY);
        }
        cm = within_group_max<N>(cm);
        // A chunk with nothing live leaves the state as it is (factor 1, zero weights).
        const bool any = cm != -INFINITY;
        const float Mn = any ? fmaxf(M, cm) : M;
        const float r = any ? fast_exp2((M - Mn) * kLog2e) : 1.f;  // 0 while M is still -inf
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int k = c + i * N;
            if (k < C)
                xw[k] = make_float2(live[i] ? fast_exp2((v[i].x - Mn) * kLog2e) : 0.f,
                                    live[i] ? v[i].y : 0.f);
        }
        wave_lds_order();
        L *= r;
        acc.x *= r;
        acc.y *= r;
        acc.z *= r;
        acc.w *= r;
#pragma unroll
        for (int k = 0; k < C; k += 2) {
            const float4 p = *reinterpret_cast<const float4*>(xw + k);  // (w, l) of k, k + 1
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const float w = h ? p.z : p.x;
                const float l = h ? p.w : p.y;  // 0 for an idle or absent split
                const float4 x = o[k + h];
                L = fmaf(w, l, L);
                if constexpr (DEAD_FINITE) {
                    acc.x = fmaf(w, x.x, acc.x);
                    acc.y = fmaf(w, x.y, acc.y);
                    acc.z = fmaf(w, x.z, acc.z);
                    acc.w = fmaf(w, x.w, acc.w);
                } else {
                    const bool lv = l > 0.f;
                    acc.x = lv ? fmaf(w, x.x, acc.x) : acc.x;
                    acc.y = lv ? fmaf(w, x.y, acc.y) : acc.y;
                    acc.z = lv ? fmaf(w, x.z, acc.z) : acc.z;
                    acc.w = lv ? fmaf(w, x.w, acc.w) : acc.w;
                }
            }
        }
        wave_lds_order();
        M = Mn;
    }
    return merge_finish(acc, L);
}

// The chunk a merge of S splits runs in: 8 for S <= 8 (one chunk, whose unused slots would
// only add zero terms), else 32.  Both sizes give the same bits for S <= 8, so the step and
// the merge kernel agree whatever they pick.  (A 4- and a 16-split chunk as well measured no
// faster, and the larger step kernel slowed the 32-split case.)
template <int N, bool DEAD_FINITE, typename Src>
__device__ __forceinline__ float4 merge_row(const Src& src, int S, int c, float2* xw) {
    if (S <= 8) return merge_row_chunks<N, DEAD_FINITE, 8>(src, S, c, xw);
    return merge_row_chunks<N, DEAD_FINITE, kMergeChunk>(src, S, c, xw);
}

// ---------------------------------------------------------------- launcher arguments

// The single-launch step's split counters sit kCounterStride uint32 words apart, one per
// 128-byte line: the tickets of a launch's groups then go to different lines.  Packed into
// one line, the 256 tickets of a 14B-shape step (eight counters) were served one after
// another and took ~2 us; spaced, the step runs 1.8 us faster.
constexpr int kCounterStride = 32;

struct DecodeArgs {
    const float* q;
    const void* k_pages;
    const void* v_pages;
    const int32_t* page_table;
    const int32_t* context_lens;
    float* partial_o;
    float* partial_ml;
    // single-launch step only (null otherwise)
    const void* k_new;       // [B][Hkv][D] current token's K and V
    const void* v_new;
    void* k_pages_w;         // the pools again, writable: the current token's slot
    void* v_pages_w;
    uint32_t* counters;      // [B][Hkv * head_groups] finished splits, kCounterStride words
                             // apart, reset by the last
    float* out;              // [B][Hq][D]
    int num_seqs, num_q_heads, num_kv_heads, group, head_groups, heads_per_wg;
    int page_shift, num_pages, max_pages, num_splits;
    int window;    // sliding window in positions (0: the whole context)
    float qscale;  // scale * log2(e)
    // > 0: the batch's sequences are taken longest first, in rounds of rank_round sequences
    // whose direction alternates (0: grid order).  Set only for batches of 2 .. kRankMax
    // sequences whose table rows fit the staged table together.
    int rank_round;
};

constexpr int kRankMax = 64;           // sequences a decode launch can rank (one per lane)
constexpr int kDecodeTableCap = 2048;  // page-table entries a decode workgroup stages in LDS

struct CombineArgs {
    const float* partial_o;
    const float* partial_ml;
    float* out;
    int rows;  // num_seqs * num_q_heads
    int num_splits;
};

struct PrefillArgs {
    const float* q;
    const void* k_pages;
    const void* v_pages;
    const int32_t* page_table;
    const int32_t* seg_desc;
    float* out;
    int num_segs, num_tables, total_tokens, num_q_heads, num_kv_heads, group;
    int page_shift, num_pages, max_pages;
    int q_blocks;  // 16-row query blocks of the longest segment
    float qscale;  // scale * log2(e)
    int round_wgs;  // workgroups dealt per round in alternating order (0: heaviest first only)
    int rank_segs;  // 1: segments taken heaviest first (2 .. kRankSegs segments), 0: in order
};
constexpr int kRankSegs = 16;  // most segments a prefill call ranks by their last position

struct KvWriteArgs {
    const void* k_new;
    const void* v_new;
    void* k_pages;
    void* v_pages;
    const int32_t* page_table;
    const int32_t* token_table_index;
    const int32_t* token_position;
    int num_tokens, num_tables, row_vec16;  // 16-byte vectors per token row (Hkv*D*elt/16)
    int page_shift, num_pages, max_pages;
};

struct KvRopeArgs {
    const float* k_new;       // [T][Hkv][D] f32, before the rotation
    const float* v_new;       // [T][Hkv][D] f32
    void* k_pages;
    void* v_pages;
    const int32_t* page_table;
    const int32_t* token_table_index;
    const int32_t* token_position;
    const float* inv_freq;    // [D/2] rotation frequency of each pair
    float* q;                 // [T][Hq][D] f32, rotated in place (null: none)
    int num_tokens, num_tables, num_kv_heads, num_q_heads, head_dim, style;
    int page_shift, num_pages, max_pages;
};

// Launchers (one translation unit each).  Return the hipError_t of the launch.
hipError_t launch_decode(const DecodeArgs& a, int kv_dtype, int head_dim, bool fused,
                         hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, int head_dim, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, int kv_dtype, int head_dim, int q_blocks,
                          bool dense, hipStream_t stream);
hipError_t launch_kv_write(const KvWriteArgs& a, hipStream_t stream);
hipError_t launch_kv_write_rope(const KvRopeArgs& a, int kv_dtype, hipStream_t stream);

// The no-allocation decode step's workspace: one fixed device array per GPU (noalloc.hip)
// of kNoallocScratchBytes bytes.  *ptr receives its device address on the current device
// (looked up once per device).
constexpr size_t kNoallocScratchBytes = size_t(16) << 20;
constexpr size_t kNoallocCounterBytes = size_t(1) << 20;  // at its start: counters only
hipError_t noalloc_scratch(void** ptr);

// Checked build: read and clear each kernel file's metadata flag (synchronous copies; call
// after the stream has been synchronised).  *bad is set when the flag was marked.
hipError_t take_bad_metadata_decode(int* bad);
hipError_t take_bad_metadata_prefill(int* bad);
hipError_t take_bad_metadata_kv_write(int* bad);
hipError_t take_bad_metadata_kv_write_rope(int* bad);

// The body of the four functions above, over one file's flag.
#define PA_DEFINE_TAKE_BAD_METADATA(NAME, FLAG)                                   \
    hipError_t NAME(int* bad) {                                                   \
        int v = 0;                                                                \
        hipError_t e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(FLAG), sizeof(int));    \
        if (e == hipSuccess && v != 0) {                                          \
            const int zero = 0;                                                   \
            e = hipMemcpyToSymbol(HIP_SYMBOL(FLAG), &zero, sizeof(int));          \
        }                                                                         \
        *bad = v;                                                                 \
        return e;                                                                 \
    }

}  // namespace pa
