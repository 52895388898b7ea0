// Backward of the gated delta rule on gfx950, in chunk form: gradients of sum(out * dout) +
// sum(hT * dhT) with respect to q, k, v, log alpha, beta and h0.
//
// Forward of one chunk of C tokens (H = S^T [d_k][d_v] entry state, b the cumsum of log alpha in
// the chunk, gamma = e^b, w_j = e^{b_last - b_j}, r the read exponent: b for the post-write read,
// b - log alpha for the pre-write read):
//
//   G_ij = (k_i . k_j) e^{b_i - b_j} (j < i),  A = diag(beta) G,  T = (I + A)^{-1}
//   X = K H,  R = diag(beta) (V - diag(gamma) X),  U = T R
//   Pm_ij = (q_i . k_j) e^{r_i - b_j} (j <= i post, j < i pre),  O = diag(e^r) Q H + Pm U
//   H' = gamma_last H + K^T diag(w) U
//
// Its adjoint, given dO and dH' (the adjoint of the chunk's exit state):
//
//   dU = diag(w) K dH' + Pm^T dO,   dR = T^T dU,   dV = diag(beta) dR
//   dP = dO U^T,  M = dP * e^{r_i - b_j} (Pm's support),   dA = -dR U^T,  N = dA * e^{b_i - b_j} (j < i)
//   dQ = diag(e^r) dO H^T + M K
//   dK = diag(w) U dH'^T - diag(beta gamma) dR H^T + M^T Q + diag(beta) N K + (diag(beta) N)^T K
//   dbeta_i = dR_i . (V_i - gamma_i X_i) + sum_j dA_ij G_ij
//   dH = gamma_last dH' + Q^T diag(e^r) dO - K^T diag(beta gamma) dR
//   and the gradient of the exponents (b and r, then log alpha through the cumsum):
//     d b_last += gamma_last <dH', H> + sum_j w_j (K dH')_j . U_j,   d b_j -= w_j (K dH')_j . U_j
//     d r_i += e^{r_i} (dO H^T)_i . q_i + sum_j dP_ij Pm_ij,   d b_j -= sum_i dP_ij Pm_ij
//     d b_i -= beta_i gamma_i dR_i . X_i,   d b_i += sum_j dA_ij A_ij,   d b_j -= sum_i dA_ij A_ij
//     dlog alpha_s = sum_{i >= s} d b_i + sum_{i >= s} d r_i (post) or sum_{i > s} d r_i (pre)
//
// This is the derivative of the chunk form of `chunked_delta` on the "Prizma seq/delta.py" page
// (transposed to H = S^T), which equals the recurrence; the pages print no backward.
//
// One workgroup of 512 threads (eight waves) per (sequence, value head, 32 columns of d_v).
// Every quantity is per column or a sum over columns of per-column terms, so the column slices
// are independent. Each workgroup writes its share of dq, dk, dbeta and dlog alpha into its own
// partial buffer in the workspace, and a second kernel adds the partials of the column slices
// (and, for dq and dk, of the value heads that share a key head) in a fixed order, so the
// gradients are the same bits on every run; inside a workgroup every per-row sum likewise has
// one slot per contributing tile, added in a fixed order. Two sweeps: the chunk-form forward from
// h0, storing the slice of the state at each chunk start in the workspace; then the chunks from
// the last, each recomputing its forward quantities from its stored entry state and applying the
// adjoint above. All matrices of a chunk live in LDS in fp32; the products run on the matrix
// cores as split bf16 products with fp32 accumulation (16x16 output tiles shared out over the
// eight waves), the triangular inverse is the one the chunk forward kernels use, and the gate
// gradients are sums on the vector units.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "gdr_kernels.hpp"
#include "gdr_mfma.hpp"
#include "gdr_solve.hpp"

namespace gdr {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
// the rows of a CB x TV matrix are shared out 8 threads to a row (4 columns each) over the first
// CB * TV / 4 threads
constexpr int kRowThreads = kBwdBlock * kBwdCols / 4;
constexpr int CB = kBwdBlock;  // tokens per chunk
constexpr int TV = kBwdCols;   // value columns per workgroup

__device__ __forceinline__ float ld_f(const float *p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld_f(const __bf16 *p, int64_t i) { return (float)p[i]; }

struct Seq {
    int64_t t0, len;
    bool rev;
    __device__ __forceinline__ int64_t token(int64_t pos) const { return rev ? t0 + len - 1 - pos : t0 + pos; }
};

template <int DK>
struct alignas(16) Smem {
    static constexpr int KP = DK + 4, VP = TV + 4, AP = CB + 4, TP = CB + 4;
    float K[CB][KP], Q[CB][KP];
    float V[CB][VP], dO[CB][VP];
    float H[DK][VP], D[DK][VP];  // the chunk's entry state and the adjoint of its exit state
    float X[CB][VP], U[CB][VP], dU[CB][VP], dR[CB][VP], eO[CB][VP], bR[CB][VP];
    float A[CB * AP], T[CB * TP];  // flat: the shared triangular inverse reads them so
    float P[CB][TP], G[CB][TP], M[CB][TP], Nb[CB][TP];
    float la[CB], beta[CB], b[CB], r[CB];
    float dw[CB];
    // Per-row partial sums of the gate gradients, one slot per contributing tile or thread so
    // that they are added in a fixed order (no float atomics):
    //   pdr:    the read exponent r: the three dP tiles' row sums, then the DK / 16 dQ tiles'
    //   pdb:    the cumulative decay b: the dP tiles' column sums (3), the dA tiles' row sums (3)
    //           and column sums (3), and each row's own term from dR . X
    //   pdbeta: beta: the dA tiles' row sums (3), and each row's own term from dR . (V - gamma X)
    static constexpr int kPdr = 3 + DK / 16, kPdb = 10, kPdbeta = 4;
    float pdr[kPdr][CB], pdb[kPdb][CB], pdbeta[kPdbeta][CB];
    float hdp[kThreads / 64];  // <dH', H> of the chunk, per wave
};

// acc += A (16 x KD) B (KD x 16) with both operands in LDS. A is X[m0 + m][k] (or, with AT,
// X[k][m0 + m]); B is Y[k][n0 + n] (or, with BT, Y[n0 + n][k]). Output tile in the accumulator
// layout: lane (g, c), register r <-> [m0 + 4g + r][n0 + c].
//
// The products run as three bf16 products of split operands (x = hi + lo, hi = bf16(x),
// lo = bf16(x - hi)): hi*hi + hi*lo + lo*hi, accumulated in fp32. The dropped lo*lo term and the
// rounding of lo leave a relative error near 2^-16 per product, and three 16x16x32 bf16 products
// take a sixth of the matrix-core time of the eight 16x16x4 fp32 ones they replace. An operand
// known to hold bf16 values exactly (AX, BX: q, k, v or dout of a bf16 call, staged in LDS as
// fp32) has lo = 0, so its lo products are skipped: two products, or one when both are exact.
__device__ __forceinline__ void split_bf16(const floatx4 &x, bf16x4 &hi, bf16x4 &lo) {
    hi = cvt4<__bf16>(x);
    floatx4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = x[i] - (float)hi[i];
    lo = cvt4<__bf16>(r);
}
template <int KD, bool AT, bool BT, bool AX = false, bool BX = false>
__device__ __forceinline__ floatx4 mm(floatx4 acc, const float *X, int ldx, int m0, const float *Y, int ldy, int n0) {
#pragma unroll
    for (int k0 = 0; k0 < KD; k0 += 32) {
        const Frag<float> fa = AT ? frag_cols<float>(X, ldx, m0, k0) : frag_rows<float>(X, ldx, m0, k0);
        const Frag<float> fb = BT ? frag_rows<float>(Y, ldy, n0, k0) : frag_cols<float>(Y, ldy, n0, k0);
        Frag<__bf16> ah, al, bh, bl;
        if constexpr (AX) {
            ah.lo = cvt4<__bf16>(fa.lo);
            ah.hi = cvt4<__bf16>(fa.hi);
        } else {
            split_bf16(fa.lo, ah.lo, al.lo);
            split_bf16(fa.hi, ah.hi, al.hi);
        }
        if constexpr (BX) {
            bh.lo = cvt4<__bf16>(fb.lo);
            bh.hi = cvt4<__bf16>(fb.hi);
        } else {
            split_bf16(fb.lo, bh.lo, bl.lo);
            split_bf16(fb.hi, bh.hi, bl.hi);
        }
        if constexpr (!AX) acc = mma32(acc, al, bh);
        if constexpr (!BX) acc = mma32(acc, ah, bl);
        acc = mma32(acc, ah, bh);
    }
    return acc;
}

// sum of x over the 16 lanes of a lane group (the columns of a tile row)
__device__ __forceinline__ float row16(float x) {
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) x += __shfl_xor(x, off, 64);
    return x;
}
// sum of x over the 4 lane groups (the rows 4g + r of a tile column, for fixed r)
__device__ __forceinline__ float col4(float x) {
    x += __shfl_xor(x, 16, 64);
    x += __shfl_xor(x, 32, 64);
    return x;
}

template <typename E, int DK>
__global__ __launch_bounds__(kThreads) void bwd_kernel(BwdArgs a) {
    typedef Smem<DK> SM;
    __shared__ SM sm;
    // q, k, v and dout of a bf16 call are staged in LDS as fp32 but hold bf16 values exactly
    constexpr bool kX = std::is_same<E, __bf16>::value;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform across the wave
    const int g = lane >> 4, cc = lane & 15;
    const int64_t unit = blockIdx.x / a.ntiles;
    const int tile = (int)(blockIdx.x % a.ntiles);
    const int64_t seq = unit / a.Hv, head = unit % a.Hv;
    const int64_t kh = head / (a.Hv / a.Hk);
    const int64_t row = a.cu_seqlens ? 0 : seq;
    const bool pre = (a.flags & kFlagReadPre) != 0;
    const int64_t dvf = a.ntiles * TV;
    const int col0 = tile * TV;
    Seq sq;
    sq.t0 = 0;
    sq.len = a.T;
    int64_t slot0 = seq * ((a.T + CB - 1) / CB);
    if (a.cu_seqlens) {
        sq.t0 = a.cu_seqlens[seq];
        sq.len = a.cu_seqlens[seq + 1] - sq.t0;
        slot0 = sq.t0 / CB + seq;
    }
    sq.rev = (a.flags & kFlagReverse) != 0;
    const int64_t nch = (sq.len + CB - 1) / CB;

    const E *qb = reinterpret_cast<const E *>(a.q) + (row * a.Hk + kh) * a.T * DK;
    const E *kb = reinterpret_cast<const E *>(a.k) + (row * a.Hk + kh) * a.T * DK;
    const E *vb = reinterpret_cast<const E *>(a.v) + (row * a.Hv + head) * a.T * dvf + col0;
    const E *dob = reinterpret_cast<const E *>(a.dout) + (row * a.Hv + head) * a.T * dvf + col0;
    const float *lab = a.log_alpha + (row * a.Hv + head) * a.T;
    const float *beb = a.beta + (row * a.Hv + head) * a.T;
    // this workgroup's partial buffers: [B][Hv][ntiles][T][DK] for dq, dk; [B][Hv][ntiles][T]
    // for dlog alpha, dbeta (summed by bwd_reduce_kernel)
    const int64_t part = (row * a.Hv + head) * a.ntiles + tile;
    float *dqb = a.pq + part * a.T * DK;
    float *dkb = a.pk + part * a.T * DK;
    float *dvb = a.dv + (row * a.Hv + head) * a.T * dvf + col0;
    float *dlab = a.pla + part * a.T;
    float *dbeb = a.pbeta + part * a.T;
    // chunk-start states: [head][slot][tile] slices of DK x TV floats
    constexpr int64_t kSlice = (int64_t)DK * TV;
    float *ckpt = a.ws + ((head * a.nslots + slot0) * a.ntiles + tile) * kSlice;
    const int64_t cstride = a.ntiles * kSlice;
    // the full [dk][dv] state of this unit, at this slice's columns
    const int64_t sbase = (seq * a.Hv + head) * DK * dvf + col0;

    // the DK x TV elements of a state slice this thread handles: SR rows x 4 columns
    constexpr int SR = DK * TV / (kThreads * 4);
    const int sc0 = (tid % (TV / 4)) * 4, sr0 = (tid / (TV / 4)) * SR;
    // the 4 elements of a CB x TV matrix this thread handles (row ei, columns ej .. ej + 3)
    const int ei = tid / (TV / 4), ej = (tid % (TV / 4)) * 4;

    // matrices whose strictly upper 16x16 tiles are read as zeros and never written
    for (int i = tid; i < CB * SM::TP; i += kThreads) {
        sm.T[i] = 0.f;
        (&sm.P[0][0])[i] = 0.f;
        (&sm.G[0][0])[i] = 0.f;
        (&sm.M[0][0])[i] = 0.f;
        (&sm.Nb[0][0])[i] = 0.f;
    }
    for (int i = tid; i < CB * SM::AP; i += kThreads) sm.A[i] = 0.f;

    auto n_rows = [&](int64_t c) __attribute__((always_inline)) -> int { return (int)min((int64_t)CB, sq.len - c * CB); };

    constexpr int EPP = 16 / (int)sizeof(E);  // elements per piece
    constexpr int KPR = DK / EPP, VPR = TV / EPP;
    constexpr int NKP = CB * KPR, NVP = CB * VPR;
    constexpr int KPT = (NKP + kThreads - 1) / kThreads, VPT = (NVP + kThreads - 1) / kThreads;
    // a chunk's inputs in flight: 16-byte pieces of k, q, v, dout (rows past the end read row 0
    // and are zeroed when stored), and the gates of the thread's row
    struct StageRegs {
        uint4 kp[KPT], qp[KPT], vp[VPT], op[VPT];
        float lv, bv;
    };
    auto stage_issue = [&](int64_t c, bool adjoint, StageRegs &sr) __attribute__((always_inline)) {
        const int n = n_rows(c);
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            const int i = tid + e * kThreads, rr = i / KPR, p = i % KPR;
            sr.kp[e] = make_uint4(0, 0, 0, 0);
            sr.qp[e] = make_uint4(0, 0, 0, 0);
            if (i < NKP) {
                const int64_t off = sq.token(c * CB + (rr < n ? rr : 0)) * DK + p * EPP;
                sr.kp[e] = *reinterpret_cast<const uint4 *>(kb + off);
                if (adjoint) sr.qp[e] = *reinterpret_cast<const uint4 *>(qb + off);
            }
        }
#pragma unroll
        for (int e = 0; e < VPT; ++e) {
            const int i = tid + e * kThreads, rr = i / VPR, p = i % VPR;
            sr.vp[e] = make_uint4(0, 0, 0, 0);
            sr.op[e] = make_uint4(0, 0, 0, 0);
            if (i < NVP) {
                const int64_t off = sq.token(c * CB + (rr < n ? rr : 0)) * dvf + p * EPP;
                sr.vp[e] = *reinterpret_cast<const uint4 *>(vb + off);
                if (adjoint) sr.op[e] = *reinterpret_cast<const uint4 *>(dob + off);
            }
        }
        sr.lv = 0.f;
        sr.bv = 0.f;
        if (tid < CB && tid < n) {
            const int64_t t = sq.token(c * CB + tid);
            sr.lv = lab[t];
            sr.bv = beb[t];
        }
    };
    // piece -> EPP floats of row rr (zero past the end), into LDS as 16-byte stores
    auto put = [&](float *dst, const uint4 &piece, bool keep) __attribute__((always_inline)) {
        float f[EPP];
        if constexpr (sizeof(E) == 2) {
            const unsigned w[4] = {piece.x, piece.y, piece.z, piece.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f[2 * j] = __uint_as_float(w[j] << 16);
                f[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
            }
        } else {
            f[0] = __uint_as_float(piece.x);
            f[1] = __uint_as_float(piece.y);
            f[2] = __uint_as_float(piece.z);
            f[3] = __uint_as_float(piece.w);
        }
#pragma unroll
        for (int j = 0; j < EPP; j += 4)
            *reinterpret_cast<float4 *>(dst + j) =
                keep ? make_float4(f[j], f[j + 1], f[j + 2], f[j + 3]) : make_float4(0.f, 0.f, 0.f, 0.f);
    };
    auto stage_store = [&](int64_t c, const StageRegs &sr) __attribute__((always_inline)) {
        const int n = n_rows(c);
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            const int i = tid + e * kThreads, rr = i / KPR, p = i % KPR;
            if (i < NKP) {
                put(&sm.K[rr][p * EPP], sr.kp[e], rr < n);
                put(&sm.Q[rr][p * EPP], sr.qp[e], rr < n);
            }
        }
#pragma unroll
        for (int e = 0; e < VPT; ++e) {
            const int i = tid + e * kThreads, rr = i / VPR, p = i % VPR;
            if (i < NVP) {
                put(&sm.V[rr][p * EPP], sr.vp[e], rr < n);
                put(&sm.dO[rr][p * EPP], sr.op[e], rr < n);
            }
        }
        if (tid < CB) {
            sm.la[tid] = sr.lv;
            sm.beta[tid] = sr.bv;
            sm.dw[tid] = 0.f;
        }
        // the tiles leave some slots of the row partials untouched: they read as zero
        for (int i = tid; i < SM::kPdr * CB; i += kThreads) sm.pdr[i / CB][i % CB] = 0.f;
        for (int i = tid; i < SM::kPdb * CB; i += kThreads) sm.pdb[i / CB][i % CB] = 0.f;
        for (int i = tid; i < SM::kPdbeta * CB; i += kThreads) sm.pdbeta[i / CB][i % CB] = 0.f;
    };
    // inclusive cumsum of log alpha and the read exponents (one wave)
    auto gates = [&]() __attribute__((always_inline)) {
        if (tid < 64) {
            float x = tid < CB ? sm.la[tid] : 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(x, off, 64);
                if (tid >= off) x += y;
            }
            if (tid < CB) {
                sm.b[tid] = x;
                sm.r[tid] = pre ? x - sm.la[tid] : x;
            }
        }
    };
    // forward quantities of the chunk from its entry state in sm.H: X, G and A, P (adjoint only), T, U
    auto forward_parts = [&](bool adjoint) __attribute__((always_inline)) {
        // X = K H (tasks 0-3, one tile each); G = K K^T and P = Q K^T on the lower tiles (00, 10,
        // 11; tasks 4-6 and 7-9), shared out over the waves
        for (int task = wave; task < (adjoint ? 10 : 7); task += kWaves) {
            if (task < 4) {
                const int mt = task >> 1, nt = task & 1;
                const floatx4 x = mm<DK, false, false, kX>(zero4(), &sm.K[0][0], SM::KP, 16 * mt, &sm.H[0][0], SM::VP, 16 * nt);
#pragma unroll
                for (int r = 0; r < 4; ++r) sm.X[16 * mt + 4 * g + r][16 * nt + cc] = x[r];
                continue;
            }
            const int t = task - 4;
            const bool isp = t >= 3;
            const int tt = t % 3, mt = tt == 0 ? 0 : 1, nt = tt == 2 ? 1 : 0;
            const floatx4 v = mm<DK, false, true, kX, kX>(zero4(), isp ? &sm.Q[0][0] : &sm.K[0][0], SM::KP, 16 * mt,
                                                  &sm.K[0][0], SM::KP, 16 * nt);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * mt + 4 * g + r, j = 16 * nt + cc;
                if (isp) {
                    const bool keep = pre ? j < i : j <= i;
                    sm.P[i][j] = keep ? v[r] * __expf(fminf(sm.r[i] - sm.b[j], 0.f)) : 0.f;
                } else {
                    const float gg = j < i ? v[r] * __expf(fminf(sm.b[i] - sm.b[j], 0.f)) : 0.f;
                    sm.G[i][j] = gg;
                    sm.A[i * SM::AP + j] = sm.beta[i] * gg;
                }
            }
        }
        __syncthreads();
        // T = (I + A)^{-1} on wave 0; meanwhile R = diag(beta) (V - diag(gamma) X) into dR on
        // waves 4-7 and, in the adjoint, the parts of dU that do not need U on waves 1-3 and 5:
        // K D (kept in eO for dw), dU = diag(w) K D + P^T dO, and <D, H> on every thread
        if (wave == 0) solve_unit_lower_inverse<float, CB>(sm);
        const int rt = tid - (kThreads - kRowThreads);
        if (rt >= 0) {
            const int i = rt / (TV / 4), j0 = (rt % (TV / 4)) * 4;
            const float be = sm.beta[i], ga = __expf(sm.b[i]);
#pragma unroll
            for (int v = 0; v < 4; ++v) sm.dR[i][j0 + v] = be * (sm.V[i][j0 + v] - ga * sm.X[i][j0 + v]);
        }
        if (adjoint) {
            const int tile = wave == 5 ? 0 : (wave >= 1 && wave <= 3) ? wave : -1;
            if (tile >= 0) {
                const float blast = sm.b[CB - 1];
                const int mt = tile >> 1, nt = tile & 1;
                const floatx4 kd = mm<DK, false, false, kX>(zero4(), &sm.K[0][0], SM::KP, 16 * mt, &sm.D[0][0], SM::VP, 16 * nt);
                const floatx4 pd = mm<CB, true, false, false, kX>(zero4(), &sm.P[0][0], SM::TP, 16 * mt, &sm.dO[0][0], SM::VP, 16 * nt);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * mt + 4 * g + r, j = 16 * nt + cc;
                    const float wi = __expf(fminf(blast - sm.b[i], 0.f));
                    sm.dU[i][j] = wi * kd[r] + pd[r];
                    sm.eO[i][j] = kd[r];
                }
            }
            float s = 0.f;
            for (int u = 0; u < SR; ++u)
#pragma unroll
                for (int v = 0; v < 4; ++v) s += sm.D[sr0 + u][sc0 + v] * sm.H[sr0 + u][sc0 + v];
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
            if (lane == 0) sm.hdp[wave] = s;
        }
        __syncthreads();
        // U = T R
        if (wave < 4) {
            const int mt = wave >> 1, nt = wave & 1;
            const floatx4 u = mm<CB, false, false>(zero4(), sm.T, SM::TP, 16 * mt, &sm.dR[0][0], SM::VP, 16 * nt);
#pragma unroll
            for (int r = 0; r < 4; ++r) sm.U[16 * mt + 4 * g + r][16 * nt + cc] = u[r];
        }
        __syncthreads();
    };

    // A thread's part of a state slice: SR rows of 4 consecutive columns, moved as 16-byte pieces
    // (all loads issued before the stores).
    auto load_slice = [&](float (*dst)[SM::VP], const float *src, int64_t pitch) __attribute__((always_inline)) {
        float4 x[SR];
#pragma unroll
        for (int u = 0; u < SR; ++u)
            x[u] = src ? *reinterpret_cast<const float4 *>(src + (int64_t)(sr0 + u) * pitch + sc0) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int u = 0; u < SR; ++u) *reinterpret_cast<float4 *>(&dst[sr0 + u][sc0]) = x[u];
    };
    // ---- sweep 1: the chunk-form forward from h0, storing each chunk's entry state
    // (the inputs of chunk c + 1 are read into registers while chunk c is computed)
    load_slice(sm.H, a.h0 ? a.h0 + sbase : nullptr, dvf);
    StageRegs nx;
    if (nch > 0) stage_issue(0, false, nx);
    __syncthreads();
    for (int64_t c = 0; c < nch; ++c) {
#pragma unroll
        for (int u = 0; u < SR; ++u)
            *reinterpret_cast<float4 *>(ckpt + c * cstride + (sr0 + u) * TV + sc0) =
                *reinterpret_cast<const float4 *>(&sm.H[sr0 + u][sc0]);
        stage_store(c, nx);
        if (c + 1 < nch) stage_issue(c + 1, false, nx);
        __syncthreads();
        gates();
        __syncthreads();
        forward_parts(false);
        // H' = gamma_last H + K^T diag(w) U (wU into dU first)
        const float blast = sm.b[CB - 1], glast = __expf(blast);
        if (tid < kRowThreads) {
            const float wi = __expf(fminf(blast - sm.b[ei], 0.f));
#pragma unroll
            for (int v = 0; v < 4; ++v) sm.dU[ei][ej + v] = wi * sm.U[ei][ej + v];
        }
        __syncthreads();
        for (int t = wave; t < (DK / 16) * (TV / 16); t += kWaves) {
            const int mt = t / (TV / 16), nt = t % (TV / 16);
            floatx4 h;
#pragma unroll
            for (int r = 0; r < 4; ++r) h[r] = glast * sm.H[16 * mt + 4 * g + r][16 * nt + cc];
            h = mm<CB, true, false, kX>(h, &sm.K[0][0], SM::KP, 16 * mt, &sm.dU[0][0], SM::VP, 16 * nt);
#pragma unroll
            for (int r = 0; r < 4; ++r) sm.H[16 * mt + 4 * g + r][16 * nt + cc] = h[r];
        }
        __syncthreads();
    }

    // ---- sweep 2: the adjoint, chunk by chunk from the last (the inputs of chunk c - 1 are read
    // into registers while chunk c is computed)
    load_slice(sm.D, a.dhT ? a.dhT + sbase : nullptr, dvf);
    if (nch > 0) stage_issue(nch - 1, true, nx);
    // the entry state slice of the chunk after next is read into registers one chunk ahead
    float4 hpre[SR];
    auto slice_issue = [&](int64_t cc) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < SR; ++u) hpre[u] = *reinterpret_cast<const float4 *>(ckpt + cc * cstride + (int64_t)(sr0 + u) * TV + sc0);
    };
    if (nch > 0) slice_issue(nch - 1);
    for (int64_t c = nch - 1; c >= 0; --c) {
        const int n = n_rows(c);
#pragma unroll
        for (int u = 0; u < SR; ++u) *reinterpret_cast<float4 *>(&sm.H[sr0 + u][sc0]) = hpre[u];
        if (c > 0) slice_issue(c - 1);
        stage_store(c, nx);
        if (c > 0) stage_issue(c - 1, true, nx);
        __syncthreads();
        gates();
        __syncthreads();
        forward_parts(true);
        const float blast = sm.b[CB - 1], glast = __expf(blast);

        // dR = T^T dU on waves 0-3; dw_i = (K D)_i . U_i (K D in eO) on waves 4-7
        if (wave < 4) {
            const int mt = wave >> 1, nt = wave & 1;
            const floatx4 d = mm<CB, true, false>(zero4(), sm.T, SM::TP, 16 * mt, &sm.dU[0][0], SM::VP, 16 * nt);
#pragma unroll
            for (int r = 0; r < 4; ++r) sm.dR[16 * mt + 4 * g + r][16 * nt + cc] = d[r];
        } else {
            const int rt = tid - (kThreads - kRowThreads);
            const int i = rt / (TV / 4), j0 = (rt % (TV / 4)) * 4;
            float sw = 0.f;
#pragma unroll
            for (int v = 0; v < 4; ++v) sw += sm.eO[i][j0 + v] * sm.U[i][j0 + v];
            sw += __shfl_xor(sw, 1, 64);
            sw += __shfl_xor(sw, 2, 64);
            sw += __shfl_xor(sw, 4, 64);
            if ((rt % (TV / 4)) == 0) sm.dw[i] = sw;
        }
        __syncthreads();
        // dP = dO U^T -> M, dA = -dR U^T -> beta N on the lower tiles; their exponent and beta
        // gradients; then dV, R's gradients, and the scaled copies for the products below
        for (int t = wave; t < 6; t += kWaves) {
            const bool isa = t >= 3;
            const int tt = t % 3, mt = tt == 0 ? 0 : 1, nt = tt == 2 ? 1 : 0;
            floatx4 v = isa ? mm<TV, false, true>(zero4(), &sm.dR[0][0], SM::VP, 16 * mt, &sm.U[0][0], SM::VP, 16 * nt)
                            : mm<TV, false, true, kX>(zero4(), &sm.dO[0][0], SM::VP, 16 * mt, &sm.U[0][0], SM::VP, 16 * nt);
            if (isa) v = -v;
            float colsum[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * mt + 4 * g + r, j = 16 * nt + cc;
                float rs = 0.f, rb = 0.f;
                if (!isa) {
                    const bool keep = pre ? j < i : j <= i;
                    sm.M[i][j] = keep ? v[r] * __expf(fminf(sm.r[i] - sm.b[j], 0.f)) : 0.f;
                    rs = keep ? v[r] * sm.P[i][j] : 0.f;  // dP_ij Pm_ij
                } else {
                    const bool keep = j < i;
                    sm.Nb[i][j] = keep ? sm.beta[i] * v[r] * __expf(fminf(sm.b[i] - sm.b[j], 0.f)) : 0.f;
                    rs = keep ? v[r] * sm.A[i * SM::AP + j] : 0.f;  // dA_ij A_ij
                    rb = keep ? v[r] * sm.G[i][j] : 0.f;  // dA_ij G_ij
                }
                colsum[r] = rs;
                const float rsum = row16(rs), bsum = row16(rb);
                if (cc == 0) {
                    if (isa) {
                        sm.pdb[3 + tt][i] = rsum;
                        sm.pdbeta[tt][i] = bsum;
                    } else {
                        sm.pdr[tt][i] = rsum;
                    }
                }
            }
            // column sums (over the 16 rows of the tile) go to d b_j with a minus sign
            float cs = colsum[0] + colsum[1] + colsum[2] + colsum[3];
            cs = col4(cs);
            if (g == 0) sm.pdb[(isa ? 6 : 0) + tt][16 * nt + cc] = -cs;
        }
        if (tid < kRowThreads) {
            const int i = ei;
            const float be = sm.beta[i], ga = __expf(sm.b[i]), er = __expf(sm.r[i]);
            const float wi = __expf(fminf(blast - sm.b[i], 0.f));
            float sb = 0.f, sx = 0.f;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int j = ej + v;
                const float dr = sm.dR[i][j];
                sb += dr * (sm.V[i][j] - ga * sm.X[i][j]);
                sx += dr * sm.X[i][j];
                if (i < n) dvb[sq.token(c * CB + i) * dvf + j] = be * dr;
                sm.eO[i][j] = er * sm.dO[i][j];
                sm.bR[i][j] = -be * ga * dr;
                sm.dU[i][j] = wi * sm.U[i][j];
            }
            sb += __shfl_xor(sb, 1, 64); sb += __shfl_xor(sb, 2, 64); sb += __shfl_xor(sb, 4, 64);
            sx += __shfl_xor(sx, 1, 64); sx += __shfl_xor(sx, 2, 64); sx += __shfl_xor(sx, 4, 64);
            if ((tid % (TV / 4)) == 0) {
                sm.pdbeta[3][i] = sb;
                sm.pdb[9][i] = -be * ga * sx;
            }
        }
        __syncthreads();
        // dQ = diag(e^r) dO H^T + M K;  dK = wU D^T + bR H^T + M^T Q + Nb K + Nb^T K
        // (wU = diag(w) U in dU, bR = -diag(beta gamma) dR); the read's exponent gradient
        for (int t = wave; t < 2 * (DK / 16); t += kWaves) {
            const int mt = t / (DK / 16), nt = t % (DK / 16);
            floatx4 oh = mm<TV, false, true, kX>(zero4(), &sm.dO[0][0], SM::VP, 16 * mt, &sm.H[0][0], SM::VP, 16 * nt);
            floatx4 dq;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * mt + 4 * g + r;
                const float er = __expf(sm.r[i]);
                dq[r] = er * oh[r];
                const float rq = row16(dq[r] * sm.Q[i][16 * nt + cc]);
                if (cc == 0) sm.pdr[3 + nt][i] = rq;
            }
            dq = mm<CB, false, false, false, kX>(dq, &sm.M[0][0], SM::TP, 16 * mt, &sm.K[0][0], SM::KP, 16 * nt);
            // three independent partial sums, so that the products do not wait on each other
            floatx4 dk = mm<TV, false, true>(zero4(), &sm.dU[0][0], SM::VP, 16 * mt, &sm.D[0][0], SM::VP, 16 * nt);
            floatx4 dk2 = mm<TV, false, true>(zero4(), &sm.bR[0][0], SM::VP, 16 * mt, &sm.H[0][0], SM::VP, 16 * nt);
            floatx4 dk3 = mm<CB, true, false, false, kX>(zero4(), &sm.M[0][0], SM::TP, 16 * mt, &sm.Q[0][0], SM::KP, 16 * nt);
            dk = mm<CB, false, false, false, kX>(dk, &sm.Nb[0][0], SM::TP, 16 * mt, &sm.K[0][0], SM::KP, 16 * nt);
            dk2 = mm<CB, true, false, false, kX>(dk2, &sm.Nb[0][0], SM::TP, 16 * mt, &sm.K[0][0], SM::KP, 16 * nt);
            dk += dk2 + dk3;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * mt + 4 * g + r;
                if (i < n) {
                    const int64_t tk = sq.token(c * CB + i);
                    dqb[tk * DK + 16 * nt + cc] = dq[r];
                    dkb[tk * DK + 16 * nt + cc] = dk[r];
                }
            }
        }
        // dH = gamma_last D + Q^T eO + K^T bR
        constexpr int NDH = ((DK / 16) * (TV / 16) + kWaves - 1) / kWaves;
        floatx4 dh[NDH];
        for (int t = wave, s = 0; t < (DK / 16) * (TV / 16); t += kWaves, ++s) {
            const int mt = t / (TV / 16), nt = t % (TV / 16);
            floatx4 h;
#pragma unroll
            for (int r = 0; r < 4; ++r) h[r] = glast * sm.D[16 * mt + 4 * g + r][16 * nt + cc];
            h = mm<CB, true, false, kX>(h, &sm.Q[0][0], SM::KP, 16 * mt, &sm.eO[0][0], SM::VP, 16 * nt);
            h = mm<CB, true, false, kX>(h, &sm.K[0][0], SM::KP, 16 * mt, &sm.bR[0][0], SM::VP, 16 * nt);
            dh[s] = h;
        }
        __syncthreads();
        for (int t = wave, s = 0; t < (DK / 16) * (TV / 16); t += kWaves, ++s) {
            const int mt = t / (TV / 16), nt = t % (TV / 16);
#pragma unroll
            for (int r = 0; r < 4; ++r) sm.D[16 * mt + 4 * g + r][16 * nt + cc] = dh[s][r];
        }
        // gate gradients of the chunk: the exit decay terms on the last row, then suffix sums
        if (tid < 64) {
            const int i = tid;
            float x = 0.f, z = 0.f;
            float dbeta_i = 0.f;
            if (i < CB) {
                const float wi = __expf(fminf(blast - sm.b[i], 0.f));
                float dbi = 0.f, dri = 0.f;
#pragma unroll
                for (int p = 0; p < SM::kPdb; ++p) dbi += sm.pdb[p][i];
#pragma unroll
                for (int p = 0; p < SM::kPdr; ++p) dri += sm.pdr[p][i];
#pragma unroll
                for (int p = 0; p < SM::kPdbeta; ++p) dbeta_i += sm.pdbeta[p][i];
                dbi -= wi * sm.dw[i];
                // the last row also takes glast <D, H> + sum_j w_j dw_j (a sum over the wave)
                float s = __expf(fminf(blast - sm.b[i], 0.f)) * sm.dw[i];
#pragma unroll
                for (int off = 16; off > 0; off >>= 1) s += __shfl_xor(s, off, 32);
                if (i == CB - 1) {
                    float hd = 0.f;
#pragma unroll
                    for (int w = 0; w < kWaves; ++w) hd += sm.hdp[w];
                    dbi += glast * hd + s;
                }
                // post: the read exponent is b itself; pre: b - log alpha leaves out row i's own
                // log alpha, so its gradient enters the sums of the rows after it only
                x = dbi + (pre ? 0.f : dri);
                z = pre ? dri : 0.f;
            }
            const float zi = z;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float x2 = __shfl_down(x, off, 64), z2 = __shfl_down(z, off, 64);
                if (i + off < 64) {
                    x += x2;
                    z += z2;
                }
            }
            if (i < n) {
                const int64_t t = sq.token(c * CB + i);
                dlab[t] = x + z - zi;
                dbeb[t] = dbeta_i;
            }
        }
        __syncthreads();
    }
    if (a.dh0) {
#pragma unroll
        for (int u = 0; u < SR; ++u)
            *reinterpret_cast<float4 *>(a.dh0 + sbase + (int64_t)(sr0 + u) * dvf + sc0) =
                *reinterpret_cast<const float4 *>(&sm.D[sr0 + u][sc0]);
    }
}

// dq, dk: the sum over the value heads of a key head and over the column slices of the
// partials, 4 consecutive d_k elements per thread; dlog alpha, dbeta: the sum over the column
// slices. Every sum runs in the same order on every call.
__global__ void bwd_reduce_kernel(BwdArgs a, int dk) {
    const int64_t grp = a.Hv / a.Hk;
    const int64_t nq4 = a.B * a.Hk * a.T * dk / 4, ng = a.B * a.Hv * a.T;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < nq4 + ng; e += stride) {
        if (e < nq4) {
            const int64_t i = 4 * e;                    // element of [B][Hk][T][dk]
            const int64_t td = i % (a.T * dk), bk = i / (a.T * dk);
            const int64_t b = bk / a.Hk, kh = bk % a.Hk;
            float4 sq = make_float4(0.f, 0.f, 0.f, 0.f), sk = sq;
            for (int64_t j = 0; j < grp; ++j)
                for (int64_t t = 0; t < a.ntiles; ++t) {
                    const int64_t src = ((b * a.Hv + kh * grp + j) * a.ntiles + t) * a.T * dk + td;
                    const float4 x = *reinterpret_cast<const float4 *>(a.pq + src);
                    const float4 y = *reinterpret_cast<const float4 *>(a.pk + src);
                    sq.x += x.x; sq.y += x.y; sq.z += x.z; sq.w += x.w;
                    sk.x += y.x; sk.y += y.y; sk.z += y.z; sk.w += y.w;
                }
            *reinterpret_cast<float4 *>(a.dq + i) = sq;
            *reinterpret_cast<float4 *>(a.dk + i) = sk;
        } else {
            const int64_t i = e - nq4;                  // element of [B][Hv][T]
            const int64_t tt = i % a.T, bh = i / a.T;
            float sl = 0.f, sb = 0.f;
            for (int64_t t = 0; t < a.ntiles; ++t) {
                sl += a.pla[(bh * a.ntiles + t) * a.T + tt];
                sb += a.pbeta[(bh * a.ntiles + t) * a.T + tt];
            }
            a.dlog_alpha[i] = sl;
            a.dbeta[i] = sb;
        }
    }
}

template <typename E, int DK>
hipError_t launch_t(const BwdArgs &a, hipStream_t s) {
    hipLaunchKernelGGL((bwd_kernel<E, DK>), dim3((unsigned)(a.units * a.ntiles)), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs &a, int dtype, int dk, int dv, hipStream_t stream) {
    (void)dv;
    hipError_t e = hipSuccess;
    if (a.units > 0) {
        if (dtype == kDtypeBf16) e = dk == 64 ? launch_t<__bf16, 64>(a, stream) : launch_t<__bf16, 128>(a, stream);
        else e = dk == 64 ? launch_t<float, 64>(a, stream) : launch_t<float, 128>(a, stream);
        if (e != hipSuccess) return e;
    }
    // every element of dq, dk, dlog alpha and dbeta is written by the reduction (zero where no
    // partial exists: no value heads or no column slices cannot happen, T = 0 has no elements)
    const int64_t work = a.B * a.Hk * a.T * dk / 4 + a.B * a.Hv * a.T;
    if (work <= 0) return hipSuccess;
    const int64_t blocks = (work + 255) / 256;
    hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(256), 0, stream, a, dk);
    return hipGetLastError();
}

}  // namespace gdr
