// Matrix-core (MFMA) helpers for gfx950, shared by the chunk-forward kernels.
//
// Every product in the library is built from 16x16 output tiles of one wave (64 lanes).
// Lane l = 16*g + c (g = l / 16 in 0..3, c = l % 16).
//
// Output / accumulator tile ("D layout", the hardware's layout of the 16x16 MFMA result):
//   lane (g, c), register r  <->  element [4g + r][c].
//
// Operands. A product over a 32-deep slice of the contraction index k uses one
// v_mfma_f32_16x16x32_bf16 (or eight v_mfma_f32_16x16x4_f32). Each lane supplies eight
// k-values for its row (A) or column (B). We fix which eight, once, for every operand:
//   lane group g holds k in {4g, 4g+1, 4g+2, 4g+3}        ("lo" half)
//                   and {16+4g, ..., 16+4g+3}              ("hi" half).
// Because A and B use the same assignment, the hardware's own k order inside the
// instruction does not matter: it pairs A[m][k] with B[k][n] for the same k.
// This assignment is chosen so that two stacked accumulator tiles (rows 0..15 and
// 16..31 of a result) ARE a B operand over those 32 rows, without a trip through LDS.
// A 16-deep product uses only the "lo" half (v_mfma_f32_16x16x16_bf16 / four
// v_mfma_f32_16x16x4_f32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short shortx4 __attribute__((ext_vector_type(4)));

template <typename E>
struct Vec4;
template <>
struct Vec4<float> {
    typedef floatx4 type;
};
template <>
struct Vec4<__bf16> {
    typedef bf16x4 type;
};

// Eight k-values of one operand: lo = k in 4g..4g+3, hi = k in 16+4g..16+4g+3.
template <typename E>
struct Frag {
    typename Vec4<E>::type lo, hi;
};

__device__ __forceinline__ floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }

template <typename E>
__device__ __forceinline__ typename Vec4<E>::type cvt4(floatx4 x);
template <>
__device__ __forceinline__ floatx4 cvt4<float>(floatx4 x) { return x; }
template <>
__device__ __forceinline__ bf16x4 cvt4<__bf16>(floatx4 x) {
    // two packed converts (round to nearest even), each materialised as one 32-bit word so
    // that the compiler does not split them into single-element converts and permutes
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    const b2 lo = __builtin_convertvector((f2){x[0], x[1]}, b2);
    const b2 hi = __builtin_convertvector((f2){x[2], x[3]}, b2);
    const unsigned w[2] = {__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
    return __builtin_bit_cast(bf16x4, w);
}

template <typename E, typename S>
__device__ __forceinline__ typename Vec4<E>::type cvt4_from(const S *p);

// ---------------------------------------------------------------- products

// acc += A(16 x 16) * B(16 x 16), lo halves only.
__device__ __forceinline__ floatx4 mma16(floatx4 acc, bf16x4 a, bf16x4 b) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(shortx4, a),
                                                     __builtin_bit_cast(shortx4, b), acc, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mma16(floatx4 acc, floatx4 a, floatx4 b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
    return acc;
}

// acc += A(16 x 32) * B(32 x 16).
__device__ __forceinline__ floatx4 mma32(floatx4 acc, const Frag<__bf16> &a, const Frag<__bf16> &b) {
    bf16x8 av = __builtin_shufflevector(a.lo, a.hi, 0, 1, 2, 3, 4, 5, 6, 7);
    bf16x8 bv = __builtin_shufflevector(b.lo, b.hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mma32(floatx4 acc, const Frag<float> &a, const Frag<float> &b) {
    acc = mma16(acc, a.lo, b.lo);
    return mma16(acc, a.hi, b.hi);
}

// ---------------------------------------------------------------- operand loads from LDS

// Operand whose k index runs along a row of a row-major matrix X (pitch ld elements):
// lane (g, c) reads X[row0 + c][k0 + 4g .. +3] and X[row0 + c][k0 + 16 + 4g .. +3].
// Serves as A for A[m][k] = X[m][k], or as B for B[k][n] = X[n][k].
template <typename E>
__device__ __forceinline__ Frag<E> frag_rows(const E *X, int ld, int row0, int k0) {
    const int lane = threadIdx.x & 63;
    const E *p = X + (row0 + (lane & 15)) * ld + k0 + 4 * (lane >> 4);
    typedef typename Vec4<E>::type V;
    Frag<E> f;
    f.lo = *reinterpret_cast<const V *>(p);
    f.hi = *reinterpret_cast<const V *>(p + 16);
    return f;
}
// lo half only (16-deep products).
template <typename E>
__device__ __forceinline__ typename Vec4<E>::type frag_rows_lo(const E *X, int ld, int row0, int k0) {
    const int lane = threadIdx.x & 63;
    const E *p = X + (row0 + (lane & 15)) * ld + k0 + 4 * (lane >> 4);
    return *reinterpret_cast<const typename Vec4<E>::type *>(p);
}
// Same, from an fp32 matrix, converted to E.
template <typename E>
__device__ __forceinline__ typename Vec4<E>::type frag_rows_lo_f32(const float *X, int ld, int row0, int k0) {
    const int lane = threadIdx.x & 63;
    const float *p = X + (row0 + (lane & 15)) * ld + k0 + 4 * (lane >> 4);
    return cvt4<E>(*reinterpret_cast<const floatx4 *>(p));
}
template <typename E>
__device__ __forceinline__ Frag<E> frag_rows_f32(const float *X, int ld, int row0, int k0) {
    const int lane = threadIdx.x & 63;
    const float *p = X + (row0 + (lane & 15)) * ld + k0 + 4 * (lane >> 4);
    Frag<E> f;
    f.lo = cvt4<E>(*reinterpret_cast<const floatx4 *>(p));
    f.hi = cvt4<E>(*reinterpret_cast<const floatx4 *>(p + 16));
    return f;
}

// Operand whose k index runs down a column of a row-major matrix X:
// lane (g, c) reads X[k0 + 4g + s][col0 + c] and X[k0 + 16 + 4g + s][col0 + c], s = 0..3.
// Serves as B for B[k][n] = X[k][n], or as A for A[m][k] = X[k][m].
template <typename E>
__device__ __forceinline__ Frag<E> frag_cols(const E *X, int ld, int col0, int k0) {
    const int lane = threadIdx.x & 63;
    const E *p = X + (k0 + 4 * (lane >> 4)) * ld + col0 + (lane & 15);
    Frag<E> f;
    typedef typename Vec4<E>::type V;
    V lo, hi;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        lo[s] = p[s * ld];
        hi[s] = p[(16 + s) * ld];
    }
    f.lo = lo;
    f.hi = hi;
    return f;
}
template <typename E>
__device__ __forceinline__ typename Vec4<E>::type frag_cols_lo(const E *X, int ld, int col0, int k0) {
    const int lane = threadIdx.x & 63;
    const E *p = X + (k0 + 4 * (lane >> 4)) * ld + col0 + (lane & 15);
    typename Vec4<E>::type lo;
#pragma unroll
    for (int s = 0; s < 4; ++s) lo[s] = p[s * ld];
    return lo;
}

// Two stacked accumulator tiles (rows 0..15 -> lo, rows 16..31 -> hi) as a B operand.
template <typename E>
__device__ __forceinline__ Frag<E> frag_from_acc(floatx4 top, floatx4 bottom) {
    Frag<E> f;
    f.lo = cvt4<E>(top);
    f.hi = cvt4<E>(bottom);
    return f;
}

// LDS ordering inside one wave: every earlier LDS access of this wave has completed.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0) (vmcnt/expcnt left at their maximum)
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace gdr
