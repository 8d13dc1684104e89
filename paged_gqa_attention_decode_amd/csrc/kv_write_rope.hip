// kv_write_rope.hip — page write with rotary position embedding and conversion to the pool
// dtype, and the query rotated at the same positions.
//
// Method (crucible, "Paged attention results": the K projection writes a scratch slice, RoPE
// rotates it, K scatters to the paged pool and V scatters unrotated; the query projection
// and its RoPE precede attention.  crucible README, "Validating the forward pass": the two
// RoPE pairing conventions, a silent failure when swapped; "What actually runs": owner and
// absolute-position arrays route the RoPE and the K/V writes).
//
// Pair i of a head row (i < D/2) is (2i, 2i+1) for PA_ROPE_ADJACENT or (i, i + D/2) for
// PA_ROPE_HALVES.  Its angle is the f32 product f32(pos) * inv_freq[i], and the pair turns
// by it: (a, b) -> (a cos t - b sin t, a sin t + b cos t), in f32 with the accurate sincos
// (range-reduced, so large positions keep their precision).  The result is rounded to the
// pool dtype to nearest, ties to even.
//
// gfx950 mapping: one thread per four pairs of kHeadsPerThread heads of one token (K/V heads
// or query heads; the four angles and their sines and cosines serve every head of the
// thread).  Per head, 8 elements: two 16-byte loads of the f32 row and one 16-byte
// (adjacent) or two 8-byte (halves) stores of a 16-bit row; all loads are issued before the
// first store.  Threads of one head group's units are consecutive, so each head's loads and
// stores are coalesced.  The K/V threads come first in the grid, then the query threads.
// Four heads per thread (a quarter of the sines and cosines) measured slower than one: the
// launch has a quarter of the threads, and at these sizes the parallelism counts for more.
#include "common.h"

namespace pa {

// Checked build: as for kv_page_write, a token to be written whose table row, position or
// page id is out of range (negative owner or position: an explicit skip).
__device__ int g_bad_metadata_kv_write_rope;

namespace {

// Two f32 values rounded to the pool dtype and packed into one 32-bit word.
__device__ __forceinline__ uint32_t pack2(F16, float x, float y) {
    const uint16_t a = __builtin_bit_cast(uint16_t, (_Float16)x);
    const uint16_t b = __builtin_bit_cast(uint16_t, (_Float16)y);
    return (uint32_t)a | ((uint32_t)b << 16);
}
__device__ __forceinline__ uint32_t pack2(BF16, float x, float y) {
    const uint16_t a = __builtin_bit_cast(uint16_t, (__bf16)x);
    const uint16_t b = __builtin_bit_cast(uint16_t, (__bf16)y);
    return (uint32_t)a | ((uint32_t)b << 16);
}

// Four consecutive elements of a pool row from f32 values.
template <typename KV>
__device__ __forceinline__ void store4(void* base, size_t elem, const float* v) {
    if constexpr (KV::kBytes == 4) {
        reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + elem)[0] =
            make_float4(v[0], v[1], v[2], v[3]);
    } else {
        reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(base) + elem)[0] =
            make_uint2(pack2(KV{}, v[0], v[1]), pack2(KV{}, v[2], v[3]));
    }
}

__device__ __forceinline__ void load4(const float* p, float* v) {
    const float4 t = *reinterpret_cast<const float4*>(p);
    v[0] = t.x;
    v[1] = t.y;
    v[2] = t.z;
    v[3] = t.w;
}

constexpr int kHeadsPerThread = 1;  // heads per thread (more heads per thread, fewer threads: slower)

template <typename KV>
__global__ void __launch_bounds__(256) kv_write_rope_kernel(KvRopeArgs a) {
    const int units = a.head_dim / 8;  // four pairs per thread
    const int kv_groups = (a.num_kv_heads + kHeadsPerThread - 1) / kHeadsPerThread;
    const int q_groups = a.q ? (a.num_q_heads + kHeadsPerThread - 1) / kHeadsPerThread : 0;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t kv_total = (int64_t)a.num_tokens * kv_groups * units;
    const int64_t q_total = (int64_t)a.num_tokens * q_groups * units;
    if (idx >= kv_total + q_total) return;
    const bool is_q = idx >= kv_total;
    const int64_t j = is_q ? idx - kv_total : idx;
    const int groups = is_q ? q_groups : kv_groups;
    const int heads = is_q ? a.num_q_heads : a.num_kv_heads;
    const int u = (int)(j % units);
    const int64_t tg = j / units;
    const int h0 = (int)(tg % groups) * kHeadsPerThread;
    const int tok = (int)(tg / groups);
    const int nh = min(kHeadsPerThread, heads - h0);
    const int pos = a.token_position[tok];
    if (pos < 0) return;

    // The unit's elements: e[0..4) at off0 and e[4..8) at off1; pair k (k < 4) is
    // (e[2k], e[2k+1]) for adjacent pairs, (e[k], e[k+4]) for halves.
    const int D = a.head_dim;
    const bool halves = a.style != 0;
    const int off0 = halves ? 4 * u : 8 * u;
    const int off1 = halves ? 4 * u + D / 2 : 8 * u + 4;
    float c[4], s[4];
    {
        const float4 f = *reinterpret_cast<const float4*>(a.inv_freq + 4 * u);
        const float fr[4] = {f.x, f.y, f.z, f.w};
        const float p = (float)pos;
#pragma unroll
        for (int k = 0; k < 4; ++k) sincosf(p * fr[k], &s[k], &c[k]);
    }
    auto rotate = [&](float* e) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int i0 = halves ? k : 2 * k;
            const int i1 = halves ? k + 4 : 2 * k + 1;
            const float x0 = e[i0], x1 = e[i1];
            e[i0] = x0 * c[k] - x1 * s[k];
            e[i1] = x0 * s[k] + x1 * c[k];
        }
    };

    // Every row of the thread's heads is loaded before any is stored.
    if (is_q) {
        float* row = a.q + ((size_t)tok * a.num_q_heads + h0) * D;
        float e[kHeadsPerThread][8];
#pragma unroll
        for (int hh = 0; hh < kHeadsPerThread; ++hh) {
            if (hh < nh) {
                load4(row + hh * D + off0, e[hh]);
                load4(row + hh * D + off1, e[hh] + 4);
            }
        }
#pragma unroll
        for (int hh = 0; hh < kHeadsPerThread; ++hh) {
            if (hh < nh) {
                rotate(e[hh]);
                *reinterpret_cast<float4*>(row + hh * D + off0) =
                    make_float4(e[hh][0], e[hh][1], e[hh][2], e[hh][3]);
                *reinterpret_cast<float4*>(row + hh * D + off1) =
                    make_float4(e[hh][4], e[hh][5], e[hh][6], e[hh][7]);
            }
        }
        return;
    }

    const int owner = a.token_table_index[tok];
    if (owner < 0) return;
    if (owner >= a.num_tables || pos >= (a.max_pages << a.page_shift)) {
        if (u == 0) mark_bad(&g_bad_metadata_kv_write_rope);
        return;
    }
    const int page = a.page_table[(size_t)owner * a.max_pages + (pos >> a.page_shift)];
    if (page < 0 || page >= a.num_pages) {
        if (u == 0) mark_bad(&g_bad_metadata_kv_write_rope);
        return;
    }
    const size_t slot = ((size_t)page << a.page_shift) | (size_t)(pos & ((1 << a.page_shift) - 1));
    const size_t dst = (slot * a.num_kv_heads + h0) * D;
    const size_t src = ((size_t)tok * a.num_kv_heads + h0) * D;

    float e[kHeadsPerThread][8], v[kHeadsPerThread][8];
#pragma unroll
    for (int hh = 0; hh < kHeadsPerThread; ++hh) {
        if (hh < nh) {
            load4(a.k_new + src + hh * D + off0, e[hh]);
            load4(a.k_new + src + hh * D + off1, e[hh] + 4);
            load4(a.v_new + src + hh * D + off0, v[hh]);
            load4(a.v_new + src + hh * D + off1, v[hh] + 4);
        }
    }
#pragma unroll
    for (int hh = 0; hh < kHeadsPerThread; ++hh) {
        if (hh < nh) {
            rotate(e[hh]);
            store4<KV>(a.k_pages, dst + hh * D + off0, e[hh]);
            store4<KV>(a.k_pages, dst + hh * D + off1, e[hh] + 4);
            store4<KV>(a.v_pages, dst + hh * D + off0, v[hh]);
            store4<KV>(a.v_pages, dst + hh * D + off1, v[hh] + 4);
        }
    }
}

}  // namespace

PA_DEFINE_TAKE_BAD_METADATA(take_bad_metadata_kv_write_rope, g_bad_metadata_kv_write_rope)

hipError_t launch_kv_write_rope(const KvRopeArgs& a, int kv_dtype, hipStream_t stream) {
    const int64_t units = a.head_dim / 8;
    const int64_t groups = (a.num_kv_heads + kHeadsPerThread - 1) / kHeadsPerThread +
                           (a.q ? (a.num_q_heads + kHeadsPerThread - 1) / kHeadsPerThread : 0);
    const int64_t total = (int64_t)a.num_tokens * units * groups;
    const dim3 grid((unsigned)((total + 255) / 256));
    if (kv_dtype == 0)
        hipLaunchKernelGGL(kv_write_rope_kernel<F32>, grid, dim3(256), 0, stream, a);
    else if (kv_dtype == 1)
        hipLaunchKernelGGL(kv_write_rope_kernel<F16>, grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(kv_write_rope_kernel<BF16>, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pa
