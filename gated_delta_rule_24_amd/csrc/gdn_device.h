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
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));   // raw 16 bytes, a native vector

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
// Round to nearest even with gfx950's conversion instruction (NaN stays NaN).
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
    return bf16_t{__builtin_bit_cast(uint16_t, (__bf16)x)};
}
// Two values rounded to bf16 by one instruction, the first in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), bf16x2_t));
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
    __device__ __forceinline__ static half8_t cvt8(float4_t x, float4_t y) {
        return half8_t{(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3],
                       (_Float16)y[0], (_Float16)y[1], (_Float16)y[2], (_Float16)y[3]};
    }
    __device__ __forceinline__ static void issue8(float4_t &acc, half8_t a, half8_t b) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
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

// 16-bit transposed LDS read (gfx950 ds_read_b64_tr_b16).  Within each group
// of 16 lanes, lane j receives as element e the (j mod 4)-th 16-bit value of
// the 8 bytes read by lane 4e + j/4 of its group.  So if lane s of the group
// points at row (R + s/4), columns (c0 + 4 (s mod 4)) .. +3 of a row-major
// 16-bit matrix, lane j receives rows R..R+3 of column c0 + j: a column
// fragment, i.e. a read of the transposed matrix.
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;
__device__ __forceinline__ uint2 lds_read_tr16(const void *p) {
    // generic -> LDS address: the low 32 bits of a shared-memory pointer
    const uint32_t a = (uint32_t)(uintptr_t)p;
    const short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t *)(uintptr_t)a);
    return __builtin_bit_cast(uint2, v);
}

// Column fragment of a row-major 16-bit matrix in LDS (`pitch` elements per
// row, a multiple of 4): lane (n, j) gets rows r0 + 8 j .. r0 + 8 j + 7 of
// column c0 + n, packed two rows per word in increasing row order, which is
// the operand of a 16x16x32 product with the matrix's transpose as a factor.
// Two transposing reads replace sixteen 16-bit reads.
__device__ __forceinline__ uint4 lds_col8_b16(const uint16_t *base, int pitch, int r0, int c0, int nn, int jj) {
    const uint16_t *p = base + (r0 + 8 * jj + (nn >> 2)) * pitch + c0 + 4 * (nn & 3);
    const uint2 lo = lds_read_tr16(p), hi = lds_read_tr16(p + 4 * pitch);
    return uint4{lo.x, lo.y, hi.x, hi.y};
}

// Operand fragment of a pair of k-tiles (32 consecutive k indices in the
// permuted order described at the top of this file): what one fp16 matrix
// instruction consumes per lane, or eight fp32 instructions.
template <typename OP>
struct Frag2;
template <>
struct Frag2<_Float16> {
    half8_t v;
    __device__ __forceinline__ static Frag2 make(half4_t lo, half4_t hi) {
        return Frag2{__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7)};
    }
    __device__ __forceinline__ static Frag2 zero() { return Frag2{half8_t{0, 0, 0, 0, 0, 0, 0, 0}}; }
    __device__ __forceinline__ static Frag2 cvt(float4_t lo, float4_t hi) {
        return Frag2{half8_t{(_Float16)lo[0], (_Float16)lo[1], (_Float16)lo[2], (_Float16)lo[3],
                             (_Float16)hi[0], (_Float16)hi[1], (_Float16)hi[2], (_Float16)hi[3]}};
    }
};
template <>
struct Frag2<float> {
    float4_t lo, hi;
    __device__ __forceinline__ static Frag2 make(float4_t a, float4_t b) { return Frag2{a, b}; }
    __device__ __forceinline__ static Frag2 zero() { return Frag2{float4_t{0.f, 0.f, 0.f, 0.f}, float4_t{0.f, 0.f, 0.f, 0.f}}; }
    __device__ __forceinline__ static Frag2 cvt(float4_t a, float4_t b) { return Frag2{a, b}; }
};

// acc += A * B over one pair of k-tiles.
__device__ __forceinline__ void mma2(float4_t &acc, const Frag2<_Float16> &a, const Frag2<_Float16> &b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma2(float4_t &acc, const Frag2<float> &a, const Frag2<float> &b) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[i], b.lo[i], acc, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[i], b.hi[i], acc, 0, 0, 0);
}

// Eight consecutive operand values of one LDS row: a k-tile pair fragment.
__device__ __forceinline__ Frag2<_Float16> row_frag2(const _Float16 *p) {
    return Frag2<_Float16>{*reinterpret_cast<const half8_t *>(p)};
}
__device__ __forceinline__ Frag2<float> row_frag2(const float *p) {
    return Frag2<float>{*reinterpret_cast<const float4_t *>(p), *reinterpret_cast<const float4_t *>(p + 4)};
}
// Eight values as the 16-byte LDS store of a row segment.
__device__ __forceinline__ void store_row8(_Float16 *p, half4_t lo, half4_t hi) {
    *reinterpret_cast<half8_t *>(p) = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ void store_row8(float *p, float4_t lo, float4_t hi) {
    reinterpret_cast<float4_t *>(p)[0] = lo;
    reinterpret_cast<float4_t *>(p)[1] = hi;
}

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

// ---- 8 consecutive input elements held as raw bits (for register prefetch) -------
// touch(): an empty asm that takes the registers as input and output.  Called
// right after a point where the loads filling them are known to be complete
// (an explicit wait for all vector memory), it makes the compiler treat the
// value as produced there, so it does not wait again, behind loads issued
// later, before the registers' first use.

template <typename in_t>
struct Raw8;

template <>
struct Raw8<bf16_t> {
    uint4 x;
    __device__ __forceinline__ void load(const bf16_t *p) { x = *reinterpret_cast<const uint4 *>(p); }
    // Re-issues the value as produced here (see Raw8 notes).
    __device__ __forceinline__ void touch() { asm volatile("" : "+v"(x.x), "+v"(x.y), "+v"(x.z), "+v"(x.w)); }
    __device__ __forceinline__ void zero() { x = make_uint4(0u, 0u, 0u, 0u); }
    __device__ __forceinline__ void store_lds(bf16_t *p) const { *reinterpret_cast<uint4 *>(p) = x; }
    __device__ __forceinline__ static void store_zero_lds(bf16_t *p) { *reinterpret_cast<uint4 *>(p) = make_uint4(0u, 0u, 0u, 0u); }
    __device__ __forceinline__ void to_f32(float (&o)[8]) const {
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            o[2 * e] = __uint_as_float(w[e] << 16);
            o[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
    }    // Element e of this vector and of `next` (the following row), packed as
    // one 32-bit LDS write; rows flagged false are written as zero.
    __device__ __forceinline__ void store_pair(const Raw8 &next, int e, bool k0, bool k1, bf16_t *dst) const {
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
        const uint32_t n[4] = {next.x.x, next.x.y, next.x.z, next.x.w};
        uint32_t a = k0 ? w[e >> 1] : 0u, b = k1 ? n[e >> 1] : 0u;
        *reinterpret_cast<uint32_t *>(dst) = __builtin_amdgcn_perm(b, a, (e & 1) ? 0x07060302u : 0x05040100u);
    }
};

template <>
struct Raw8<_Float16> {
    uint4 x;
    __device__ __forceinline__ void load(const _Float16 *p) { x = *reinterpret_cast<const uint4 *>(p); }
    __device__ __forceinline__ void touch() { asm volatile("" : "+v"(x.x), "+v"(x.y), "+v"(x.z), "+v"(x.w)); }
    __device__ __forceinline__ void zero() { x = make_uint4(0u, 0u, 0u, 0u); }
    __device__ __forceinline__ void store_lds(_Float16 *p) const { *reinterpret_cast<uint4 *>(p) = x; }
    __device__ __forceinline__ static void store_zero_lds(_Float16 *p) { *reinterpret_cast<uint4 *>(p) = make_uint4(0u, 0u, 0u, 0u); }
    __device__ __forceinline__ void to_f32(float (&o)[8]) const {
        const half8_t h = __builtin_bit_cast(half8_t, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (float)h[e];
    }    __device__ __forceinline__ void store_pair(const Raw8 &next, int e, bool k0, bool k1, _Float16 *dst) const {
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
        const uint32_t n[4] = {next.x.x, next.x.y, next.x.z, next.x.w};
        uint32_t a = k0 ? w[e >> 1] : 0u, b = k1 ? n[e >> 1] : 0u;
        *reinterpret_cast<uint32_t *>(dst) = __builtin_amdgcn_perm(b, a, (e & 1) ? 0x07060302u : 0x05040100u);
    }
};

template <>
struct Raw8<float> {
    uint4 x[2];
    __device__ __forceinline__ void load(const float *p) {
        x[0] = *reinterpret_cast<const uint4 *>(p);
        x[1] = *reinterpret_cast<const uint4 *>(p + 4);
    }
    __device__ __forceinline__ void zero() { x[0] = x[1] = make_uint4(0u, 0u, 0u, 0u); }
    __device__ __forceinline__ void touch() {
        asm volatile("" : "+v"(x[0].x), "+v"(x[0].y), "+v"(x[0].z), "+v"(x[0].w));
        asm volatile("" : "+v"(x[1].x), "+v"(x[1].y), "+v"(x[1].z), "+v"(x[1].w));
    }
    __device__ __forceinline__ void store_lds(float *p) const {
        reinterpret_cast<uint4 *>(p)[0] = x[0];
        reinterpret_cast<uint4 *>(p)[1] = x[1];
    }
    __device__ __forceinline__ static void store_zero_lds(float *p) {
        reinterpret_cast<uint4 *>(p)[0] = make_uint4(0u, 0u, 0u, 0u);
        reinterpret_cast<uint4 *>(p)[1] = make_uint4(0u, 0u, 0u, 0u);
    }
    __device__ __forceinline__ void to_f32(float (&o)[8]) const {
        o[0] = __uint_as_float(x[0].x); o[1] = __uint_as_float(x[0].y);
        o[2] = __uint_as_float(x[0].z); o[3] = __uint_as_float(x[0].w);
        o[4] = __uint_as_float(x[1].x); o[5] = __uint_as_float(x[1].y);
        o[6] = __uint_as_float(x[1].z); o[7] = __uint_as_float(x[1].w);
    }
    __device__ __forceinline__ void store_pair(const Raw8 &next, int e, bool k0, bool k1, float *dst) const {
        const uint32_t w[8] = {x[0].x, x[0].y, x[0].z, x[0].w, x[1].x, x[1].y, x[1].z, x[1].w};
        const uint32_t n[8] = {next.x[0].x, next.x[0].y, next.x[0].z, next.x[0].w,
                               next.x[1].x, next.x[1].y, next.x[1].z, next.x[1].w};
        *reinterpret_cast<uint2 *>(dst) = uint2{k0 ? w[e] : 0u, k1 ? n[e] : 0u};
    }
};

// acc += (row block X) (row block Y)^T over one k-tile pair of raw inputs.
// bf16 and fp16 rows use their own 16x16x32 instruction (exact products,
// fp32 sums); fp32 rows take eight 16x16x4 fp32 instructions.
__device__ __forceinline__ void gram_mma(float4_t &acc, const Raw8<bf16_t> &x, const Raw8<bf16_t> &y) {
    typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, x.x),
                                                 __builtin_bit_cast(bf16x8_t, y.x), acc, 0, 0, 0);
}
__device__ __forceinline__ void gram_mma(float4_t &acc, const Raw8<_Float16> &x, const Raw8<_Float16> &y) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, x.x),
                                                __builtin_bit_cast(half8_t, y.x), acc, 0, 0, 0);
}
__device__ __forceinline__ void gram_mma(float4_t &acc, const Raw8<float> &x, const Raw8<float> &y) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const float4_t a = __builtin_bit_cast(float4_t, x.x[hh]), b = __builtin_bit_cast(float4_t, y.x[hh]);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], acc, 0, 0, 0);
    }
}

template <typename in_t>
__device__ __forceinline__ in_t zero_elem() { return in_t{}; }

// Eight input values as two 4-element matrix-core operand fragments.  16-bit
// inputs become fp16 operands: fp16 inputs are copied bit for bit, bf16
// inputs are widened to fp32 and packed with one conversion per pair (the
// conversion rounds toward zero, which is exact for every bf16 value inside
// the fp16 normal range, the documented operand-range precondition).
__device__ __forceinline__ void to_op(const Raw8<bf16_t> &r, half4_t &lo, half4_t &hi) {
    const uint32_t w[4] = {r.x.x, r.x.y, r.x.z, r.x.w};
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    h2 p[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
        p[e] = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(w[e] << 16),
                                                                  __uint_as_float(w[e] & 0xffff0000u)));
    lo = half4_t{p[0][0], p[0][1], p[1][0], p[1][1]};
    hi = half4_t{p[2][0], p[2][1], p[3][0], p[3][1]};
}
__device__ __forceinline__ void to_op(const Raw8<_Float16> &r, half4_t &lo, half4_t &hi) {
    lo = __builtin_bit_cast(half4_t, uint2{r.x.x, r.x.y});
    hi = __builtin_bit_cast(half4_t, uint2{r.x.z, r.x.w});
}
__device__ __forceinline__ void to_op(const Raw8<float> &r, float4_t &lo, float4_t &hi) {
    lo = __builtin_bit_cast(float4_t, r.x[0]);
    hi = __builtin_bit_cast(float4_t, r.x[1]);
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

// ---- unit lower-triangular chunk matrices as 16 x 16 tiles ----------------------

// The lower tiles (a >= b) of a 64 x 64 chunk matrix, numbered row by row:
// tile t = a (a + 1) / 2 + b.
__host__ __device__ constexpr int tri_index(int a, int b) { return a * (a + 1) / 2 + b; }
__device__ __forceinline__ void tri_decode(int t, int &a, int &b) {
    a = t < 1 ? 0 : (t < 3 ? 1 : (t < 6 ? 2 : 3));
    b = t - a * (a + 1) / 2;
}

// acc + X Y for 16 x 16 fp32 blocks on four 16x16x4 instructions, x in the
// A-operand layout and y in the B-operand layout (x[s], y[s]: k = 4 j + s).
__device__ __forceinline__ float4_t mm16_f32(const float4_t &x, const float4_t &y, float4_t acc) {
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x[s], y[s], acc, 0, 0, 0);
    return acc;
}

// The inverses T_j = (I + N_j)^{-1} of the four unit lower-triangular 16 x 16
// diagonal blocks of a chunk matrix, by one wave.  On entry block j of `blk`
// (at j * BS floats, row pitch BP) holds N_j transposed: row c holds N_j[m][c]
// for m > c (other entries are not read).  Lane (n, j) solves row n of T_j,
//   x[c] = [c == n] - sum_{m > c} x[m] N_j[m][c],  c = 15 .. 0
// (row c of the transposed block is broadcast to the block's 16 lanes, the
// sum taken in increasing m), and writes it over row n of block j.  Only the
// wave itself touches `blk`: its LDS accesses are performed in program
// order, so the compiler alone has to be kept from moving them (the caller
// fences its writes of N before the call).  nn, jj: the lane's l mod 16 and
// l / 16, as the caller holds them.
template <int BP, int BS>
__device__ __forceinline__ void diag_block_inverse(float *blk, int nn, int jj) {
    const float *nt = blk + jj * BS;
    float x[16];
#pragma unroll
    for (int c = 15; c >= 0; --c) {
        float acc = (c == nn) ? 1.f : 0.f;
#pragma unroll
        for (int qd = (c + 1) / 4; qd < 4; ++qd) {
            const float4_t v = *reinterpret_cast<const float4_t *>(nt + c * BP + 4 * qd);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (4 * qd + e > c) acc -= x[4 * qd + e] * v[e];
        }
        x[c] = acc;
    }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int qd = 0; qd < 4; ++qd)
        *reinterpret_cast<float4_t *>(blk + jj * BS + nn * BP + 4 * qd) =
            float4_t{x[4 * qd], x[4 * qd + 1], x[4 * qd + 2], x[4 * qd + 3]};
    asm volatile("" ::: "memory");
}

}  // namespace gdn
