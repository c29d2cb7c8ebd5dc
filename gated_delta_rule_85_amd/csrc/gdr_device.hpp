// gdr_device.hpp -- device-side helpers shared by the gfx950 kernels:
// element types, vector loads/stores, wave reductions and the matrix-core
// (MFMA) fragment operations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdr_kernels.hpp"

namespace gdr {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// Gate activations of pre-activations (kRawGates).  softplus(x) = log(1 + e^x)
// evaluated as max(x, 0) + log1p(e^-|x|), without overflow; sigmoid(x) =
// 1 / (1 + e^-x), which saturates cleanly at 0 and 1.
__device__ __forceinline__ float softplus_f(float x) {
    return fmaxf(x, 0.f) + log1pf(__expf(-fabsf(x)));
}
__device__ __forceinline__ float sigmoid_f(float x) { return 1.f / (1.f + __expf(-x)); }
// log of the decay gate: log(alpha) for a stored alpha, -s softplus(x) for a
// pre-activation x (computed in the log domain, so strong decay cannot
// underflow to a zero whose log is -inf).
__device__ __forceinline__ float log_decay(float x, bool raw, float s) {
    return raw ? -s * softplus_f(x) : logf(x);
}

// Floor of a per-channel log decay inside the chunk form.  The chunk form
// splits a channel-wise decay e^{g_r - g_s} between the two operands of its
// Gram products around one reference per 16-row block, the midpoint of that
// block's log-decay range; with every token's log decay at least -F, each
// factor stays within e^{+-7.5 F} (15 decays per block), inside the fp32 and
// bf16 range for F = 10.  A decay below e^{-10} ~ 4.5e-5 is applied as
// e^{-10}: the part of a channel's state it lets through is then at most
// 4.5e-5 of that state instead of less.  Decays at or above e^{-10} are exact.
// The decode step applies every decay as given.
constexpr float kLogDecayFloor = -10.f;
// e^{kLogDecayFloor}: the smallest decay the chunk form applies.
constexpr float kDecayFloor = 4.53999297624848515e-5f;
// Middle factors of the off-diagonal 16x16 tiles of a 64-row chunk: pair p of
// the six strictly lower tile positions (R, S) = (1,0) (2,0) (2,1) (3,0) (3,1)
// (3,2), p = R (R - 1) / 2 + S.
__device__ __forceinline__ int pair_r(int p) { return 1 + (p >= 1) + (p >= 3); }
__device__ __forceinline__ int pair_s(int p) { const int r = pair_r(p); return p - r * (r - 1) / 2; }
__device__ __forceinline__ int pair_of(int R, int S) { return R * (R - 1) / 2 + S; }

// Sum over the 64 lanes of a wave; every lane gets the result.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, kWave);
    return x;
}

// ----------------------------------------------------------------------------
// Matrix-core tiles.  One wave computes a 16x16 fp32 tile D += A * B^T where
// A is 16 x K and B is 16 x K, both "K-contiguous" (row-major along K).  The
// accumulator fragment holds, in lane l, column (l % 16) and rows
// 4*(l / 16) + {0,1,2,3}.
//
// bf16: v_mfma_f32_16x16x32_bf16 consumes K = 32 per instruction; lane l
//   supplies row (l % 16) and K-elements 8*(l / 16) + {0..7} of each operand.
// fp32: v_mfma_f32_16x16x4_f32 consumes K = 4; lane l supplies row (l % 16)
//   and K-element (l / 16).
// ----------------------------------------------------------------------------
template <typename T> struct Mma;

template <> struct Mma<bf16> {
    static constexpr int kK = 32;          // K per instruction
    static constexpr int kPerLane = 8;     // operand elements per lane
    typedef bf16x8 frag;
    __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    // Fragment from a K-contiguous row: elements row[k0 + 8*(lane/16) + 0..7].
    __device__ __forceinline__ static frag load(const bf16 *row, int k0, int lane) {
        return *reinterpret_cast<const frag *>(row + k0 + 8 * (lane >> 4));
    }
    __device__ __forceinline__ static frag from_f32x8(const float *x) {
        frag f;
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = (bf16)x[i];
        return f;
    }
};

template <> struct Mma<float> {
    static constexpr int kK = 4;
    static constexpr int kPerLane = 1;
    typedef float frag;
    __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    __device__ __forceinline__ static frag load(const float *row, int k0, int lane) {
        return row[k0 + (lane >> 4)];
    }
    __device__ __forceinline__ static frag from_f32x8(const float *x) { return x[0]; }
};

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

constexpr int kChunk = 64;   // chunk length of the prefill

// ---- fragment-major workspace layout ------------------------------------------
// Each rows x K operand factor is stored as 16-row tiles by K-steps of the
// matrix-core instruction, and inside a tile in MFMA lane order, so that one
// wave's fragment load of a tile is one contiguous 1 KB (bf16) read: whole
// cache lines, no half-used lines.
template <typename TI> __device__ __forceinline__ long frag_off(int r, int k, int K) {
    using M = Mma<TI>;
    const int tile = (r >> 4) * (K / M::kK) + k / M::kK;
    const int ln = (r & 15) + 16 * ((k % M::kK) / M::kPerLane);
    return ((long)tile * kWave + ln) * M::kPerLane + (k % M::kPerLane);
}
// U~^T is consumed in accumulator layout: for value tile j/16 and row tile
// r/16, lane (j % 16) + 16 ((r % 16) / 4) holds rows r .. r+3 of column j.
__device__ __forceinline__ long ufrag_off(int j, int r) {
    return ((long)((j >> 4) * (kChunk / 16) + (r >> 4)) * kWave + (j & 15) + 16 * ((r & 15) >> 2)) * 4 +
           (r & 3);
}

// ---- vector loads and stores ---------------------------------------------------
__device__ __forceinline__ void store4(bf16 *dst, f32x4 x) {
    bf16x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (bf16)x[e];
    *reinterpret_cast<bf16x4 *>(dst) = v;
}
__device__ __forceinline__ void store4(float *dst, f32x4 x) {
    *reinterpret_cast<f32x4 *>(dst) = x;
}
__device__ __forceinline__ f32x4 load4(const bf16 *src) {
    bf16x4 v = *reinterpret_cast<const bf16x4 *>(src);
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ f32x4 load4(const float *src) {
    return *reinterpret_cast<const f32x4 *>(src);
}
__device__ __forceinline__ f32x4 to_f32x4(bf16x4 v) {
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ f32x4 to_f32x4(f32x4 v) { return v; }

// Copies an SW x n block kept transposed in LDS (src[j][r]: SW columns of n
// rows) to rows r < n_valid of a row-major destination (element (r, j) at
// dst[r * ld + j]), eight consecutive columns per thread and store.
template <typename TI, int SW, int P>
__device__ __forceinline__ void copy_transposed(TI *dst, long ld, const TI (*src)[P], int n,
                                                long n_valid, int tt, int nt) {
    static_assert(SW % 8 == 0, "eight columns per store");
    for (int qd = tt; qd < n * (SW / 8); qd += nt) {
        const int r = qd / (SW / 8), j0 = 8 * (qd % (SW / 8));
        if (r >= n_valid) continue;
        if constexpr (sizeof(TI) == 2) {
            bf16x8 x;
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = src[j0 + e][r];
            *reinterpret_cast<bf16x8 *>(dst + r * ld + j0) = x;
        } else {
            f32x4 x0, x1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x0[e] = src[j0 + e][r];
                x1[e] = src[j0 + 4 + e][r];
            }
            *reinterpret_cast<f32x4 *>(dst + r * ld + j0) = x0;
            *reinterpret_cast<f32x4 *>(dst + r * ld + j0 + 4) = x1;
        }
    }
}

// ---- buffer loads ------------------------------------------------------------
// The scan addresses each chunk's factors through a buffer descriptor built in
// scalar registers from the chunk's block address, plus a per-lane offset that
// never changes: the per-chunk address arithmetic stays scalar, so no vector
// register that may still be the target of a load in flight is rewritten.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, 0x7fffffff,
                                             0x00020000);
}
template <typename T> __device__ __forceinline__ T buf_load(__amdgpu_buffer_rsrc_t r, unsigned off) {
    if constexpr (sizeof(T) == 16) {
        typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
        u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
        return __builtin_bit_cast(T, v);
    } else if constexpr (sizeof(T) == 8) {
        typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
        u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
        return __builtin_bit_cast(T, v);
    } else {
        static_assert(sizeof(T) == 4, "4, 8 or 16 bytes");
        unsigned v = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
        return __builtin_bit_cast(T, v);
    }
}

}  // namespace gdr
