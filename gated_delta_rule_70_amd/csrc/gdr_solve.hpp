// The unit lower-triangular inverse T = (I + A)^{-1} of one chunk, shared by the chunk kernels
// whose shared-memory struct holds the fp32 matrix A (pitch SM::AP) and the E-typed T (pitch
// SM::TP). A is strictly lower triangular (C x C, C = 16, 32 or 64), so T is unit lower
// triangular: T = I - A + A^2 - ..., which the chunk form of the delta rule applies to the
// right-hand sides of a chunk (the WY/UT form of `chunked_delta` on the "Prizma seq/delta.py"
// page, with the solve written as an explicit inverse so that it becomes a matrix-core product).
#pragma once

#include "gdr_mfma.hpp"

namespace gdr {

// By one wave. Diagonal 16x16 blocks by forward substitution (one lane per column), then
// T_10 = -T_11 A_10 T_00 (and T_32 for C = 64), then the lower-left 32x32 block
// T_BA = -T_BB A_BA T_AA (C = 64). Writes the lower triangle of sm.T; its strictly upper
// blocks must be zero (they are never written).
// kHoist: the block's rows of A (the same for the sixteen lanes of a group) are all read into
// registers before the substitution starts, so that its chain of multiply-adds does not wait on
// LDS row by row; it takes about 30 more registers, for kernels whose occupancy the LDS sets.
template <typename E, int C, typename SM, bool kHoist = false>
__device__ __forceinline__ void solve_unit_lower_inverse(SM &sm) {
    constexpr int NT = C / 16;
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, cc = lane & 15;
    if (g < NT) {
        const int base = 16 * g;
        float t[16];
        if constexpr (kHoist) {
            static_assert(SM::AP % 4 == 0, "16-byte rows of A");
            float4 ar[16][4];
#pragma unroll
            for (int i = 1; i < 16; ++i)
#pragma unroll
                for (int q = 0; q < (i + 3) / 4; ++q)
                    ar[i][q] = *reinterpret_cast<const float4 *>(sm.A + (base + i) * SM::AP + base + 4 * q);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float s = (i == cc) ? 1.f : 0.f;
#pragma unroll
                for (int j = 0; j < i; ++j) s -= ar[i][j / 4][j % 4] * t[j];
                t[i] = s;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float s = (i == cc) ? 1.f : 0.f;
                const float *arow = sm.A + (base + i) * SM::AP + base;
#pragma unroll
                for (int j = 0; j < i; ++j) s -= arow[j] * t[j];
                t[i] = s;
            }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sm.T[(base + i) * SM::TP + base + cc] = static_cast<E>(t[i]);
    }
    if (NT == 1) return;
    wave_lds_sync();
    // T_{2p+1, 2p} = -T_{2p+1,2p+1} A_{2p+1,2p} T_{2p,2p}
#pragma unroll
    for (int p = 0; p < NT / 2; ++p) {
        const int r1 = 2 * p + 1, c0 = 2 * p;
        floatx4 z = mma16(zero4(), frag_rows_lo_f32<E>(sm.A, SM::AP, 16 * r1, 16 * c0),
                          frag_cols_lo<E>(sm.T, SM::TP, 16 * c0, 16 * c0));
        floatx4 w = mma16(zero4(), frag_rows_lo<E>(sm.T, SM::TP, 16 * r1, 16 * r1), cvt4<E>(z));
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.T[(16 * r1 + 4 * g + r) * SM::TP + 16 * c0 + cc] = static_cast<E>(-w[r]);
    }
    if (NT == 2) return;
    wave_lds_sync();
    // lower-left 32x32 block: M = A_BA T_AA, T_BA = -T_BB M, one 16-column slice at a time
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
        floatx4 m0 = mma32(zero4(), frag_rows_f32<E>(sm.A, SM::AP, 32, 0), frag_cols<E>(sm.T, SM::TP, 16 * ct, 0));
        floatx4 m1 = mma32(zero4(), frag_rows_f32<E>(sm.A, SM::AP, 48, 0), frag_cols<E>(sm.T, SM::TP, 16 * ct, 0));
        const Frag<E> mb = frag_from_acc<E>(m0, m1);
        floatx4 l0 = mma32(zero4(), frag_rows<E>(sm.T, SM::TP, 32, 32), mb);
        floatx4 l1 = mma32(zero4(), frag_rows<E>(sm.T, SM::TP, 48, 32), mb);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            sm.T[(32 + 4 * g + r) * SM::TP + 16 * ct + cc] = static_cast<E>(-l0[r]);
            sm.T[(48 + 4 * g + r) * SM::TP + 16 * ct + cc] = static_cast<E>(-l1[r]);
        }
    }
}

}  // namespace gdr
