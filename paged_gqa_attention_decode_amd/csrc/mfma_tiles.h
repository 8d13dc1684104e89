// mfma_tiles.h — the matrix-core operand layouts shared by the decode and prefill kernels.
//
// Both kernels contract a 32-key tile of one KV head against up to 16 query columns with
// 16 x 16 MFMA blocks: scores are computed transposed, S^T = K Q^T (16 keys x 16 columns per
// block), so that lane (g, c16) -- g = lane / 16 the MFMA k-group, c16 = lane % 16 -- ends
// with 4 keys of ONE column (keys 16 st + 4 g + i of block st, i = 0..3).  That register
// layout is the B operand P^T of O^T += V^T P^T, so the probabilities never leave their lane,
// and the O^T accumulator keeps one column per lane as well: lane (g, c16) holds, in
// accumulator dt, element i, output dim NC (4 g + i) + dt of column c16 (NC = D / 16).
// A column is one query row in the prefill and one query head in the decode.
//
// Two operand sets share this frame:
//   - f32 K/V: v_mfma_f32_16x16x4_f32.  A lane reads 4 consecutive dims of a K row (16 B);
//     the PV product takes output dims in the order d = NC c16 + dt, so the V operands a
//     lane needs for one key are NC consecutive dims.
//   - f16/bf16 K/V: v_mfma_f32_16x16x32_{f16,bf16}, K and V straight from the pool.  The f32
//     operands (the scaled query and the probabilities) are each split into two terms of the
//     pool's 16-bit type, x = hi + lo, and both terms are multiplied: the residual of the
//     split is below 2^-16 |x| for bf16 and 2^-22 |x| for f16, where one rounding of q and p
//     to bf16 alone (2^-9 |x|) can exceed the 16-bit tolerance on standard-normal inputs.  A
//     lane's 8 K elements of one MFMA are 8 consecutive dims (one 16-byte load).  For PV the
//     contraction runs over keys; the MFMA pairs A's and B's k index through the same (lane
//     group, element) slot, so keys are assigned to slots as the score layout already holds
//     them: element e of lane group g is key 16 (e / 4) + 4 g + e % 4, and P^T is the lane's
//     own 8 probabilities.  V is loaded as NC consecutive dims of each of those 8 keys and
//     regrouped into per-dim-block operands by byte permutes.
// Every output element of an MFMA is one fixed-order dot product, independent of the other
// columns, so a column's bits do not depend on what the other columns hold.
//
// Rows are located by functors krow(key) / vrow(key) that return a pointer to dim 0 of the
// key's row for the tile's KV head (page translation, and in the decode step the current
// token's row taken from its own buffer).  Keys past khi are clamped onto khi: a valid row,
// so no branch guards a load; the caller masks their scores.
#pragma once

#include "common.h"

namespace pa {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kTileKeys = 32;  // keys per tile: two 16-key MFMA blocks

__device__ __forceinline__ floatx4 mfma4(float a, float b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma32(F16, uint4 a, uint4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(halfx8, a),
                                                   __builtin_bit_cast(halfx8, b), c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma32(BF16, uint4 a, uint4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// x and y each split into hi + lo terms of the 16-bit type (both rounded to nearest even):
// hi packs (hi(x), hi(y)) and lo packs (lo(x), lo(y)), x in the low half.
__device__ __forceinline__ void split_pair(F16, float x, float y, uint32_t& hi, uint32_t& lo) {
    const _Float16 hx = (_Float16)x, hy = (_Float16)y;
    const _Float16 lx = (_Float16)(x - (float)hx), ly = (_Float16)(y - (float)hy);
    hi = (uint32_t)__builtin_bit_cast(uint16_t, hx) |
         ((uint32_t)__builtin_bit_cast(uint16_t, hy) << 16);
    lo = (uint32_t)__builtin_bit_cast(uint16_t, lx) |
         ((uint32_t)__builtin_bit_cast(uint16_t, ly) << 16);
}
__device__ __forceinline__ void split_pair(BF16, float x, float y, uint32_t& hi, uint32_t& lo) {
    const __bf16 hx = (__bf16)x, hy = (__bf16)y;
    const __bf16 lx = (__bf16)(x - (float)hx), ly = (__bf16)(y - (float)hy);
    hi = (uint32_t)__builtin_bit_cast(uint16_t, hx) |
         ((uint32_t)__builtin_bit_cast(uint16_t, hy) << 16);
    lo = (uint32_t)__builtin_bit_cast(uint16_t, lx) |
         ((uint32_t)__builtin_bit_cast(uint16_t, ly) << 16);
}

// The 16-bit element sel of word a (low half) and of word b (high half), sel 0 or 1.
__device__ __forceinline__ uint32_t pair_halves(uint32_t a, uint32_t b, int sel) {
    return __builtin_amdgcn_perm(b, a, sel ? 0x07060302u : 0x05040100u);
}

template <typename KV, int D>
struct TileOps;

// f32 K/V on v_mfma_f32_16x16x4_f32.
template <int D>
struct TileOps<F32, D> {
    static constexpr int NC = D / 16;
    using T = float;
    // Q^T operand: lane (g, c16) holds Q[column][16c + 4g + kk], kk = 0..3.
    float q[NC][4];
    struct Tile {
        // K operand: lane (g, c16) of block st holds K[j0 + 16 st + c16][16c + 4g + kk].
        float kf[2][NC][4];
        // V^T operand of MFMA (st, i, dt): lane (g, c16) holds V[j0 + 16 st + 4g + i][NC c16 + dt].
        float vf[2][4][NC];
    };

    // The lane's part of the column's query row, as loaded (fetch_q), then times qs (set_q):
    // two steps, so that the loads can be issued before other waits.
    struct QRaw {
        float4 v[NC];
    };
    __device__ __forceinline__ static QRaw fetch_q(const float* row, int g) {
        QRaw r;
#pragma unroll
        for (int c = 0; c < NC; ++c) r.v[c] = *reinterpret_cast<const float4*>(row + 16 * c + 4 * g);
        return r;
    }
    __device__ __forceinline__ void set_q(const QRaw& r, float qs) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            q[c][0] = r.v[c].x * qs;
            q[c][1] = r.v[c].y * qs;
            q[c][2] = r.v[c].z * qs;
            q[c][3] = r.v[c].w * qs;
        }
    }
    __device__ __forceinline__ void load_q(const float* row, float qs, int g) {
        set_q(fetch_q(row, g), qs);
    }

    template <class Row>
    __device__ __forceinline__ static void load_k(Tile& tl, Row krow, int j0, int khi, int g,
                                                  int c16) {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const float* kr = krow(min(j0 + 16 * st + c16, khi)) + 4 * g;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const float4 t = *reinterpret_cast<const float4*>(kr + 16 * c);
                tl.kf[st][c][0] = t.x;
                tl.kf[st][c][1] = t.y;
                tl.kf[st][c][2] = t.z;
                tl.kf[st][c][3] = t.w;
            }
        }
    }
    template <class Row>
    __device__ __forceinline__ static void load_v(Tile& tl, Row vrow, int j0, int khi, int g,
                                                  int c16) {
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float* vr = vrow(min(j0 + 16 * st + 4 * g + i, khi)) + NC * c16;
#pragma unroll
                for (int d4 = 0; d4 < NC; d4 += 4) {
                    const float4 t = *reinterpret_cast<const float4*>(vr + d4);
                    tl.vf[st][i][d4 + 0] = t.x;
                    tl.vf[st][i][d4 + 1] = t.y;
                    tl.vf[st][i][d4 + 2] = t.z;
                    tl.vf[st][i][d4 + 3] = t.w;
                }
            }
    }

    // S^T = K Q^T: lane (g, c16) gets the scores of keys j0 + 16 st + 4g + i for column c16.
    __device__ __forceinline__ void scores(const Tile& tl, floatx4 (&sacc)[2]) const {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            sacc[st] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    sacc[st] = mfma4(tl.kf[st][c][kk], q[c][kk], sacc[st]);
        }
    }

    // O^T += V^T P^T (accumulator row c of block dt is output dim NC c + dt).
    __device__ __forceinline__ static void pv(const Tile& tl, const float (&p)[2][4],
                                              floatx4 (&oacc)[NC]) {
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int dt = 0; dt < NC; ++dt)
                    oacc[dt] = mfma4(tl.vf[st][i][dt], p[st][i], oacc[dt]);
    }
};

// f16 / bf16 K/V on v_mfma_f32_16x16x32_{f16,bf16}; the query and P as hi + lo terms.
template <typename KV, int D>
struct TileOps {
    static constexpr int NC = D / 16;
    static constexpr int NK = D / 32;  // 32-dim chunks of a row = 32-bit words of NC dims
    using T = uint16_t;
    // Q^T operand terms: lane (g, c16) holds Q[column][32c + 8g + e], e = 0..7.
    uint4 qh[NK], ql[NK];
    struct Tile {
        // K operand of block st: lane (g, c16) holds K[j0 + 16 st + c16][32c + 8g + e].
        uint4 k[2][NK];
        // Lane (g, c16): V[j0 + 16 st + 4g + i][NC c16 + 2w + (0, 1)] in word w.
        uint32_t v[2][4][NK];
    };

    struct QRaw {
        float4 v[2 * NK];
    };
    __device__ __forceinline__ static QRaw fetch_q(const float* row, int g) {
        QRaw r;
#pragma unroll
        for (int c = 0; c < NK; ++c) {
            r.v[2 * c] = *reinterpret_cast<const float4*>(row + 32 * c + 8 * g);
            r.v[2 * c + 1] = *reinterpret_cast<const float4*>(row + 32 * c + 8 * g + 4);
        }
        return r;
    }
    __device__ __forceinline__ void set_q(const QRaw& r, float qs) {
#pragma unroll
        for (int c = 0; c < NK; ++c) {
            const float4 a = r.v[2 * c], b = r.v[2 * c + 1];
            split_pair(KV{}, a.x * qs, a.y * qs, qh[c].x, ql[c].x);
            split_pair(KV{}, a.z * qs, a.w * qs, qh[c].y, ql[c].y);
            split_pair(KV{}, b.x * qs, b.y * qs, qh[c].z, ql[c].z);
            split_pair(KV{}, b.z * qs, b.w * qs, qh[c].w, ql[c].w);
        }
    }
    __device__ __forceinline__ void load_q(const float* row, float qs, int g) {
        set_q(fetch_q(row, g), qs);
    }

    template <class Row>
    __device__ __forceinline__ static void load_k(Tile& tl, Row krow, int j0, int khi, int g,
                                                  int c16) {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const T* kr = krow(min(j0 + 16 * st + c16, khi)) + 8 * g;
#pragma unroll
            for (int c = 0; c < NK; ++c) tl.k[st][c] = *reinterpret_cast<const uint4*>(kr + 32 * c);
        }
    }
    template <class Row>
    __device__ __forceinline__ static void load_v(Tile& tl, Row vrow, int j0, int khi, int g,
                                                  int c16) {
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const T* vr = vrow(min(j0 + 16 * st + 4 * g + i, khi)) + NC * c16;
                if constexpr (NK == 2) {
                    const uint2 t = *reinterpret_cast<const uint2*>(vr);
                    tl.v[st][i][0] = t.x;
                    tl.v[st][i][1] = t.y;
                } else {
#pragma unroll
                    for (int w = 0; w < NK; w += 4) {
                        const uint4 t = *reinterpret_cast<const uint4*>(vr + 2 * w);
                        tl.v[st][i][w + 0] = t.x;
                        tl.v[st][i][w + 1] = t.y;
                        tl.v[st][i][w + 2] = t.z;
                        tl.v[st][i][w + 3] = t.w;
                    }
                }
            }
    }

    __device__ __forceinline__ void scores(const Tile& tl, floatx4 (&sacc)[2]) const {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            sacc[st] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < NK; ++c) sacc[st] = mfma32(KV{}, tl.k[st][c], qh[c], sacc[st]);
#pragma unroll
            for (int c = 0; c < NK; ++c) sacc[st] = mfma32(KV{}, tl.k[st][c], ql[c], sacc[st]);
        }
    }

    __device__ __forceinline__ static void pv(const Tile& tl, const float (&p)[2][4],
                                              floatx4 (&oacc)[NC]) {
        // P^T operand: element e = p[e / 4][e % 4], as hi and lo terms.
        uint4 ph, pl;
        split_pair(KV{}, p[0][0], p[0][1], ph.x, pl.x);
        split_pair(KV{}, p[0][2], p[0][3], ph.y, pl.y);
        split_pair(KV{}, p[1][0], p[1][1], ph.z, pl.z);
        split_pair(KV{}, p[1][2], p[1][3], ph.w, pl.w);
#pragma unroll
        for (int dt = 0; dt < NC; ++dt) {
            // V^T operand of dim block dt: element e = V[key e][NC c16 + dt].
            const int w = dt >> 1, sel = dt & 1;
            uint4 va;
            va.x = pair_halves(tl.v[0][0][w], tl.v[0][1][w], sel);
            va.y = pair_halves(tl.v[0][2][w], tl.v[0][3][w], sel);
            va.z = pair_halves(tl.v[1][0][w], tl.v[1][1][w], sel);
            va.w = pair_halves(tl.v[1][2][w], tl.v[1][3][w], sel);
            oacc[dt] = mfma32(KV{}, va, ph, oacc[dt]);
            oacc[dt] = mfma32(KV{}, va, pl, oacc[dt]);
        }
    }
};

}  // namespace pa
