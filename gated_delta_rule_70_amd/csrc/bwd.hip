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
// One workgroup of 256 threads per (sequence, value head, 32 columns of d_v). Every quantity is
// per column or a sum over columns of per-column terms, so the column slices are independent:
// dq, dk, dbeta and dlog alpha are added with float atomics into buffers a fill kernel clears
// first (this also sums dq and dk over the value heads that share a key head). Two sweeps: the
// chunk-form forward from h0, storing the slice of the state at each chunk start in the
// workspace; then the chunks from the last, each recomputing its forward quantities from its
// stored entry state and applying the adjoint above. All matrices of a chunk live in LDS in
// fp32; the products are register-blocked fp32 FMAs spread over the 256 threads.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "gdr_kernels.hpp"

namespace gdr {

namespace {

constexpr int kThreads = 256;
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
struct Smem {
    // odd pitches: a column read across the lanes of a wave hits distinct banks
    static constexpr int KP = DK + 1, VP = TV + 1, CP = CB + 1;
    float K[CB][KP], Q[CB][KP];
    float V[CB][VP], dO[CB][VP];
    float H[DK][VP], D[DK][VP];  // the chunk's entry state and the adjoint of its exit state
    float X[CB][VP], U[CB][VP], dU[CB][VP], dR[CB][VP];
    float T[CB][CP], P[CB][CP], G[CB][CP], M[CB][CP], N[CB][CP];
    float la[CB], beta[CB], b[CB], r[CB];
    float db[CB], dr[CB], dbeta[CB], dw[CB];
    float hd;  // <dH', H> of the chunk
};

template <typename E, int DK>
__global__ __launch_bounds__(kThreads) void bwd_kernel(BwdArgs a) {
    __shared__ Smem<DK> sm;
    const int tid = threadIdx.x;
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
    float *dqb = a.dq + (row * a.Hk + kh) * a.T * DK;
    float *dkb = a.dk + (row * a.Hk + kh) * a.T * DK;
    float *dvb = a.dv + (row * a.Hv + head) * a.T * dvf + col0;
    float *dlab = a.dlog_alpha + (row * a.Hv + head) * a.T;
    float *dbeb = a.dbeta + (row * a.Hv + head) * a.T;
    // chunk-start states: [head][slot][tile] slices of DK x TV floats
    constexpr int64_t kSlice = (int64_t)DK * TV;
    float *ckpt = a.ws + ((head * a.nslots + slot0) * a.ntiles + tile) * kSlice;
    const int64_t cstride = a.ntiles * kSlice;
    // the full [dk][dv] state of this unit, at this slice's columns
    const int64_t sbase = (seq * a.Hv + head) * DK * dvf + col0;

    // the DK x TV elements of a state slice this thread handles: SR rows x 4 columns
    constexpr int SR = DK * TV / (kThreads * 4);
    const int sc0 = (tid % (TV / 4)) * 4, sr0 = (tid / (TV / 4)) * SR;
    // the 2 x 2 block of a CB x TV or CB x CB matrix this thread handles
    const int bi0 = (tid / 16) * 2, bj0 = (tid % 16) * 2;

    auto n_rows = [&](int64_t c) __attribute__((always_inline)) -> int { return (int)min((int64_t)CB, sq.len - c * CB); };

    // load chunk c's inputs into LDS (rows past the end are zero: no decay, no write)
    auto stage = [&](int64_t c, bool adjoint) __attribute__((always_inline)) {
        const int n = n_rows(c);
        for (int i = tid; i < CB * DK; i += kThreads) {
            const int rr = i / DK, cc = i % DK;
            const int64_t t = rr < n ? sq.token(c * CB + rr) : 0;
            sm.K[rr][cc] = rr < n ? ld_f(kb, t * DK + cc) : 0.f;
            if (adjoint) sm.Q[rr][cc] = rr < n ? ld_f(qb, t * DK + cc) : 0.f;
        }
        for (int i = tid; i < CB * TV; i += kThreads) {
            const int rr = i / TV, cc = i % TV;
            const int64_t t = rr < n ? sq.token(c * CB + rr) : 0;
            sm.V[rr][cc] = rr < n ? ld_f(vb, t * dvf + cc) : 0.f;
            if (adjoint) sm.dO[rr][cc] = rr < n ? ld_f(dob, t * dvf + cc) : 0.f;
        }
        if (tid < CB) {
            const int64_t t = tid < n ? sq.token(c * CB + tid) : 0;
            sm.la[tid] = tid < n ? lab[t] : 0.f;
            sm.beta[tid] = tid < n ? beb[t] : 0.f;
            sm.db[tid] = 0.f;
            sm.dr[tid] = 0.f;
            sm.dbeta[tid] = 0.f;
            sm.dw[tid] = 0.f;
        }
        if (tid == 0) sm.hd = 0.f;
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
    // forward quantities of the chunk from its entry state in sm.H: X, G, P (adjoint only), T, U
    auto forward_parts = [&](bool adjoint) __attribute__((always_inline)) {
        {
            float x[2][2] = {{0.f, 0.f}, {0.f, 0.f}}, g[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
            float p[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
            #pragma unroll 4
            for (int n = 0; n < DK; ++n) {
                const float k0 = sm.K[bi0][n], k1 = sm.K[bi0 + 1][n];
                const float h0 = sm.H[n][bj0], h1 = sm.H[n][bj0 + 1];
                const float kj0 = sm.K[bj0][n], kj1 = sm.K[bj0 + 1][n];
                x[0][0] += k0 * h0; x[0][1] += k0 * h1; x[1][0] += k1 * h0; x[1][1] += k1 * h1;
                g[0][0] += k0 * kj0; g[0][1] += k0 * kj1; g[1][0] += k1 * kj0; g[1][1] += k1 * kj1;
                if (adjoint) {
                    const float q0 = sm.Q[bi0][n], q1 = sm.Q[bi0 + 1][n];
                    p[0][0] += q0 * kj0; p[0][1] += q0 * kj1; p[1][0] += q1 * kj0; p[1][1] += q1 * kj1;
                }
            }
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int v = 0; v < 2; ++v) {
                    const int i = bi0 + u, j = bj0 + v;
                    sm.X[i][j] = x[u][v];
                    sm.G[i][j] = j < i ? g[u][v] * __expf(fminf(sm.b[i] - sm.b[j], 0.f)) : 0.f;
                    if (adjoint) {
                        const bool keep = pre ? j < i : j <= i;
                        sm.P[i][j] = keep ? p[u][v] * __expf(fminf(sm.r[i] - sm.b[j], 0.f)) : 0.f;
                    }
                }
        }
        __syncthreads();
        // T = (I + diag(beta) G)^{-1}: one lane per column, forward substitution down the column
        // (in place in LDS: each lane reads back only what it wrote)
        if (tid < CB) {
            const int c = tid;
            for (int i = 0; i < CB; ++i) {
                float s = 0.f;
                #pragma unroll 4
                for (int j = c; j < i; ++j) s += sm.G[i][j] * sm.T[j][c];
                sm.T[i][c] = i < c ? 0.f : ((i == c ? 1.f : 0.f) - sm.beta[i] * s);
            }
        }
        __syncthreads();
        // U = T R, R = diag(beta) (V - diag(gamma) X)
        {
            float u[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
            #pragma unroll 4
            for (int m = 0; m <= bi0 + 1; ++m) {
                const float be = sm.beta[m], ga = __expf(sm.b[m]);
                const float r0 = be * (sm.V[m][bj0] - ga * sm.X[m][bj0]);
                const float r1 = be * (sm.V[m][bj0 + 1] - ga * sm.X[m][bj0 + 1]);
                const float t0 = sm.T[bi0][m], t1 = sm.T[bi0 + 1][m];
                u[0][0] += t0 * r0; u[0][1] += t0 * r1; u[1][0] += t1 * r0; u[1][1] += t1 * r1;
            }
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                sm.U[bi0][bj0 + v] = u[0][v];
                sm.U[bi0 + 1][bj0 + v] = u[1][v];
            }
        }
        __syncthreads();
    };

    // ---- sweep 1: the chunk-form forward from h0, storing each chunk's entry state
    for (int u = 0; u < SR; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int n = sr0 + u, cc = sc0 + v;
            sm.H[n][cc] = a.h0 ? a.h0[sbase + (int64_t)n * dvf + cc] : 0.f;
        }
    __syncthreads();
    for (int64_t c = 0; c < nch; ++c) {
        for (int u = 0; u < SR; ++u)
#pragma unroll
            for (int v = 0; v < 4; ++v) ckpt[c * cstride + (sr0 + u) * TV + sc0 + v] = sm.H[sr0 + u][sc0 + v];
        stage(c, false);
        __syncthreads();
        gates();
        __syncthreads();
        forward_parts(false);
        // H' = gamma_last H + K^T diag(w) U
        const float blast = sm.b[CB - 1];
        float hn[SR][4];
        for (int u = 0; u < SR; ++u)
#pragma unroll
            for (int v = 0; v < 4; ++v) hn[u][v] = __expf(blast) * sm.H[sr0 + u][sc0 + v];
        #pragma unroll 4
        for (int j = 0; j < CB; ++j) {
            const float wj = __expf(fminf(blast - sm.b[j], 0.f));
            for (int u = 0; u < SR; ++u) {
                const float kw = sm.K[j][sr0 + u] * wj;
#pragma unroll
                for (int v = 0; v < 4; ++v) hn[u][v] += kw * sm.U[j][sc0 + v];
            }
        }
        __syncthreads();
        for (int u = 0; u < SR; ++u)
#pragma unroll
            for (int v = 0; v < 4; ++v) sm.H[sr0 + u][sc0 + v] = hn[u][v];
        __syncthreads();
    }

    // ---- sweep 2: the adjoint, chunk by chunk from the last
    for (int u = 0; u < SR; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int n = sr0 + u, cc = sc0 + v;
            sm.D[n][cc] = a.dhT ? a.dhT[sbase + (int64_t)n * dvf + cc] : 0.f;
        }
    for (int64_t c = nch - 1; c >= 0; --c) {
        const int n = n_rows(c);
        for (int u = 0; u < SR; ++u)
#pragma unroll
            for (int v = 0; v < 4; ++v) sm.H[sr0 + u][sc0 + v] = ckpt[c * cstride + (sr0 + u) * TV + sc0 + v];
        stage(c, true);
        __syncthreads();
        gates();
        __syncthreads();
        forward_parts(true);
        const float blast = sm.b[CB - 1], glast = __expf(blast);

        // dU = diag(w) K D + P^T dO, and dw_i = (K D)_i . U_i
        {
            float kd[2][2] = {{0.f, 0.f}, {0.f, 0.f}}, pd[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
            #pragma unroll 4
            for (int m = 0; m < DK; ++m) {
                const float k0 = sm.K[bi0][m], k1 = sm.K[bi0 + 1][m];
                const float d0 = sm.D[m][bj0], d1 = sm.D[m][bj0 + 1];
                kd[0][0] += k0 * d0; kd[0][1] += k0 * d1; kd[1][0] += k1 * d0; kd[1][1] += k1 * d1;
            }
            #pragma unroll 4
            for (int m = bi0; m < CB; ++m) {
                const float p0 = sm.P[m][bi0], p1 = sm.P[m][bi0 + 1];
                const float o0 = sm.dO[m][bj0], o1 = sm.dO[m][bj0 + 1];
                pd[0][0] += p0 * o0; pd[0][1] += p0 * o1; pd[1][0] += p1 * o0; pd[1][1] += p1 * o1;
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int i = bi0 + u;
                const float wi = __expf(fminf(blast - sm.b[i], 0.f));
                float dwp = 0.f;
#pragma unroll
                for (int v = 0; v < 2; ++v) {
                    sm.dU[i][bj0 + v] = wi * kd[u][v] + pd[u][v];
                    dwp += kd[u][v] * sm.U[i][bj0 + v];
                }
                atomicAdd(&sm.dw[i], dwp);
            }
        }
        // <D, H> of the chunk (for the exit decay)
        {
            float s = 0.f;
            for (int u = 0; u < SR; ++u)
#pragma unroll
                for (int v = 0; v < 4; ++v) s += sm.D[sr0 + u][sc0 + v] * sm.H[sr0 + u][sc0 + v];
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
            if ((tid & 63) == 0) atomicAdd(&sm.hd, s);
        }
        __syncthreads();
        // dR = T^T dU
        {
            float d[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
            #pragma unroll 4
            for (int m = bi0; m < CB; ++m) {
                const float t0 = sm.T[m][bi0], t1 = sm.T[m][bi0 + 1];
                const float u0 = sm.dU[m][bj0], u1 = sm.dU[m][bj0 + 1];
                d[0][0] += t0 * u0; d[0][1] += t0 * u1; d[1][0] += t1 * u0; d[1][1] += t1 * u1;
            }
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int v = 0; v < 2; ++v) sm.dR[bi0 + u][bj0 + v] = d[u][v];
        }
        __syncthreads();
        // dP = dO U^T -> M; dA = -dR U^T -> N; the exponent gradients of P and A; dbeta from A
        {
            float dp[2][2] = {{0.f, 0.f}, {0.f, 0.f}}, da[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
            #pragma unroll 4
            for (int cc = 0; cc < TV; ++cc) {
                const float o0 = sm.dO[bi0][cc], o1 = sm.dO[bi0 + 1][cc];
                const float r0 = sm.dR[bi0][cc], r1 = sm.dR[bi0 + 1][cc];
                const float u0 = sm.U[bj0][cc], u1 = sm.U[bj0 + 1][cc];
                dp[0][0] += o0 * u0; dp[0][1] += o0 * u1; dp[1][0] += o1 * u0; dp[1][1] += o1 * u1;
                da[0][0] -= r0 * u0; da[0][1] -= r0 * u1; da[1][0] -= r1 * u0; da[1][1] -= r1 * u1;
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int i = bi0 + u;
                float rrow = 0.f, brow = 0.f, bet = 0.f;
#pragma unroll
                for (int v = 0; v < 2; ++v) {
                    const int j = bj0 + v;
                    const bool pk = pre ? j < i : j <= i;
                    sm.M[i][j] = pk ? dp[u][v] * __expf(fminf(sm.r[i] - sm.b[j], 0.f)) : 0.f;
                    sm.N[i][j] = j < i ? da[u][v] * __expf(fminf(sm.b[i] - sm.b[j], 0.f)) : 0.f;
                    const float pp = pk ? dp[u][v] * sm.P[i][j] : 0.f;                 // dP_ij Pm_ij
                    const float gg = j < i ? da[u][v] * sm.G[i][j] : 0.f;              // dA_ij G_ij
                    rrow += pp;
                    brow += sm.beta[i] * gg;                                           // dA_ij A_ij
                    bet += gg;
                    atomicAdd(&sm.db[j], -(pp + sm.beta[i] * gg));
                }
                atomicAdd(&sm.dr[i], rrow);
                atomicAdd(&sm.db[i], brow);
                atomicAdd(&sm.dbeta[i], bet);
            }
        }
        // dV, and dbeta and the exponent gradient from R
        {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int i = bi0 + u;
                const float be = sm.beta[i], ga = __expf(sm.b[i]);
                float sb = 0.f, sx = 0.f;
#pragma unroll
                for (int v = 0; v < 2; ++v) {
                    const int j = bj0 + v;
                    const float dr = sm.dR[i][j];
                    sb += dr * (sm.V[i][j] - ga * sm.X[i][j]);
                    sx += dr * sm.X[i][j];
                    if (i < n) dvb[sq.token(c * CB + i) * dvf + j] = be * dr;
                }
                atomicAdd(&sm.dbeta[i], sb);
                atomicAdd(&sm.db[i], -be * ga * sx);
            }
        }
        __syncthreads();
        // dQ, dK (CB x DK; QI rows x NV columns per thread, columns n0 + 32 v so that the lanes of a
        // wave read 32 consecutive rows of H and D) and the exponent gradient of the read
        {
            constexpr int NV = DK / 32, QI = CB / 8;
            const int n0 = tid % 32, i0 = (tid / 32) * QI;
            for (int u = 0; u < QI; ++u) {
                const int i = i0 + u;
                const float er = __expf(sm.r[i]);
                const float wi = __expf(fminf(blast - sm.b[i], 0.f));
                const float bg = sm.beta[i] * __expf(sm.b[i]);
                float dq[NV], dk[NV], oh[NV];
#pragma unroll
                for (int v = 0; v < NV; ++v) dq[v] = dk[v] = oh[v] = 0.f;
                #pragma unroll 4
                for (int cc = 0; cc < TV; ++cc) {
                    const float o = sm.dO[i][cc], uu = sm.U[i][cc], dr = sm.dR[i][cc];
#pragma unroll
                    for (int v = 0; v < NV; ++v) {
                        const float h = sm.H[n0 + 32 * v][cc], d = sm.D[n0 + 32 * v][cc];
                        oh[v] += o * h;
                        dk[v] += wi * uu * d - bg * dr * h;
                    }
                }
                #pragma unroll 4
                for (int j = 0; j < CB; ++j) {
                    const float mij = sm.M[i][j], mji = sm.M[j][i];
                    const float nn = sm.beta[i] * sm.N[i][j] + sm.beta[j] * sm.N[j][i];
#pragma unroll
                    for (int v = 0; v < NV; ++v) {
                        const float kj = sm.K[j][n0 + 32 * v], qj = sm.Q[j][n0 + 32 * v];
                        dq[v] += mij * kj;
                        dk[v] += mji * qj + nn * kj;
                    }
                }
                float rq = 0.f;
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    dq[v] += er * oh[v];
                    rq += er * oh[v] * sm.Q[i][n0 + 32 * v];
                }
                atomicAdd(&sm.dr[i], rq);
                if (i < n) {
                    const int64_t t = sq.token(c * CB + i);
#pragma unroll
                    for (int v = 0; v < NV; ++v) {
                        atomicAdd(dqb + t * DK + n0 + 32 * v, dq[v]);
                        atomicAdd(dkb + t * DK + n0 + 32 * v, dk[v]);
                    }
                }
            }
        }
        // dH = gamma_last D + Q^T diag(e^r) dO - K^T diag(beta gamma) dR
        float dh[SR][4];
        for (int u = 0; u < SR; ++u)
#pragma unroll
            for (int v = 0; v < 4; ++v) dh[u][v] = glast * sm.D[sr0 + u][sc0 + v];
        #pragma unroll 4
        for (int j = 0; j < CB; ++j) {
            const float er = __expf(sm.r[j]), bg = sm.beta[j] * __expf(sm.b[j]);
            for (int u = 0; u < SR; ++u) {
                const float qe = sm.Q[j][sr0 + u] * er, kg = sm.K[j][sr0 + u] * bg;
#pragma unroll
                for (int v = 0; v < 4; ++v) dh[u][v] += qe * sm.dO[j][sc0 + v] - kg * sm.dR[j][sc0 + v];
            }
        }
        __syncthreads();
        for (int u = 0; u < SR; ++u)
#pragma unroll
            for (int v = 0; v < 4; ++v) sm.D[sr0 + u][sc0 + v] = dh[u][v];
        // gate gradients of the chunk: the exit decay terms on the last row, then suffix sums
        if (tid < 64) {
            const int i = tid;
            float x = 0.f, z = 0.f;
            if (i < CB) {
                const float wi = __expf(fminf(blast - sm.b[i], 0.f));
                float dbi = sm.db[i] - wi * sm.dw[i];
                if (i == CB - 1) {
                    float s = glast * sm.hd;
                    for (int j = 0; j < CB; ++j) s += __expf(fminf(blast - sm.b[j], 0.f)) * sm.dw[j];
                    dbi += s;
                }
                // post: the read exponent is b itself; pre: b - log alpha leaves out row i's own
                // log alpha, so its gradient enters the sums of the rows after it only
                x = dbi + (pre ? 0.f : sm.dr[i]);
                z = pre ? sm.dr[i] : 0.f;
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
                atomicAdd(dlab + t, x + z - zi);
                atomicAdd(dbeb + t, sm.dbeta[i]);
            }
        }
        __syncthreads();
    }
    if (a.dh0) {
        for (int u = 0; u < SR; ++u)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int nn = sr0 + u, cc = sc0 + v;
                a.dh0[sbase + (int64_t)nn * dvf + cc] = sm.D[nn][cc];
            }
    }
}

__global__ void zero_kernel(float *p, int64_t n) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0.f;
}

// clear n floats with a kernel (not a memset node, so the call stays safe to capture in a graph)
hipError_t clear(float *p, int64_t n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = (n + 255) / 256;
    const unsigned grid = (unsigned)(blocks < 4096 ? blocks : 4096);
    hipLaunchKernelGGL(zero_kernel, dim3(grid), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

template <typename E, int DK>
hipError_t launch_t(const BwdArgs &a, hipStream_t s) {
    hipLaunchKernelGGL((bwd_kernel<E, DK>), dim3((unsigned)(a.units * a.ntiles)), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs &a, int dtype, int dk, int dv, hipStream_t stream) {
    (void)dv;
    // the sums over columns and value heads start from zero
    hipError_t e;
    if ((e = clear(a.dq, a.B * a.Hk * a.T * dk, stream)) != hipSuccess) return e;
    if ((e = clear(a.dk, a.B * a.Hk * a.T * dk, stream)) != hipSuccess) return e;
    if ((e = clear(a.dlog_alpha, a.B * a.Hv * a.T, stream)) != hipSuccess) return e;
    if ((e = clear(a.dbeta, a.B * a.Hv * a.T, stream)) != hipSuccess) return e;
    if (a.units == 0) return hipSuccess;
    if (dtype == kDtypeBf16) return dk == 64 ? launch_t<__bf16, 64>(a, stream) : launch_t<__bf16, 128>(a, stream);
    return dk == 64 ? launch_t<float, 64>(a, stream) : launch_t<float, 128>(a, stream);
}

}  // namespace gdr
