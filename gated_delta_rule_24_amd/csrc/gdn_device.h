// Device-side helpers shared by the gfx950 kernels: element types, loads and
// stores with conversion, and 16x16 matrix-core (MFMA) tile products.
//
// MFMA tile convention used everywhere in this library (wave64):
//   lane l, n = l % 16, j = l / 16.
//   A 16x16 fp32 accumulator tile C holds C[4j + i][n] in element i (i < 4).
//   One "k-tile" of an operand is 16 consecutive k indices.  For a k-tile kt
//   lane (m, j) supplies A[m][16kt + 4j + i] and B[16kt + 4j + i][n], i < 4.
// Because the product sums over k, any assignment of k indices to
// (lane group, slot) is correct as long as A and B use the same one.  The
// assignment above makes an accumulator tile of one product directly usable
// as the B operand of the next product (its k-tile is the tile's row block),
// so intermediate results never leave registers.
//   fp16 operands: v_mfma_f32_16x16x32_f16 consumes two k-tiles per issue
//                  (slots 0..3 = first k-tile, 4..7 = second).
//   fp32 operands: v_mfma_f32_16x16x4_f32 consumes one k index per lane
//                  group; a k-tile takes four issues (slot i on issue i).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint16_t ushort4_t __attribute__((ext_vector_type(4)));
typedef uint16_t ushort8_t __attribute__((ext_vector_type(8)));

struct bf16_t {
    uint16_t bits;
};

// ---- scalar conversions ------------------------------------------------------

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(_Float16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(bf16_t x) {
    return __uint_as_float(((uint32_t)x.bits) << 16);
}

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ _Float16 from_f32<_Float16>(float x) { return (_Float16)x; }
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
    uint32_t u = __float_as_uint(x);
    bf16_t r;
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) {
        r.bits = (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
    } else {
        r.bits = (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);  // round to nearest even
    }
    return r;
}

// ---- matrix-core tile products --------------------------------------------------

template <typename OP>
struct Mma;

template <>
struct Mma<_Float16> {
    using frag = half4_t;                 // 4 operand values of one k-tile
    static constexpr int KT_PER_ISSUE = 2;
    __device__ __forceinline__ static frag zero() { return frag{0, 0, 0, 0}; }
    __device__ __forceinline__ static frag cvt(float4_t x) {
        return frag{(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]};
    }
    // acc += A(k-tiles a0,a1) * B(k-tiles b0,b1)
    __device__ __forceinline__ static void issue(float4_t &acc, frag a0, frag a1, frag b0, frag b1) {
        half8_t a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
        half8_t b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
    }
};

template <>
struct Mma<float> {
    using frag = float4_t;
    static constexpr int KT_PER_ISSUE = 1;
    __device__ __forceinline__ static frag zero() { return frag{0.f, 0.f, 0.f, 0.f}; }
    __device__ __forceinline__ static frag cvt(float4_t x) { return x; }
    __device__ __forceinline__ static void issue(float4_t &acc, frag a, frag, frag b, frag) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
    }
};

// Four consecutive operand values from LDS (8-byte or 16-byte aligned read).
template <typename OP>
__device__ __forceinline__ typename Mma<OP>::frag lds_frag(const OP *p) {
    return *reinterpret_cast<const typename Mma<OP>::frag *>(p);
}

// ---- global loads of 8 consecutive input elements, converted to fp32 -----------

__device__ __forceinline__ void load8_f32(const float *p, float (&o)[8]) {
    float4_t a = *reinterpret_cast<const float4_t *>(p);
    float4_t b = *reinterpret_cast<const float4_t *>(p + 4);
    o[0] = a[0]; o[1] = a[1]; o[2] = a[2]; o[3] = a[3];
    o[4] = b[0]; o[5] = b[1]; o[6] = b[2]; o[7] = b[3];
}
__device__ __forceinline__ void load8_f32(const _Float16 *p, float (&o)[8]) {
    half8_t a = *reinterpret_cast<const half8_t *>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (float)a[i];
}
__device__ __forceinline__ void load8_f32(const bf16_t *p, float (&o)[8]) {
    ushort8_t a = *reinterpret_cast<const ushort8_t *>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = __uint_as_float(((uint32_t)a[i]) << 16);
}

// ---- wave-level helpers ---------------------------------------------------------

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ float wave_inclusive_scan(float x) {
    const int l = lane_id();
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        float y = __shfl_up(x, off, 64);
        if (l >= off) x += y;
    }
    return x;
}

}  // namespace gdn
