// Chunk-parallel forward of the gated delta rule on gfx950.
//
// Per (sequence, value head, 32-wide slice of d_v) one workgroup of 4 waves walks the
// chunks of its sequence in scan order. Per chunk of C tokens with local log-decay
// cumsum b_i (b'_i = b_i - a_i for the pre-write read) and entry state H ([d_k][d_v]):
//
//   A   = strict_lower(beta_i (k_i . k_j) e^{b_i - b_j})            (C x C, fp32)
//   T   = (I + A)^{-1}                                              (unit lower solve)
//   R   = diag(beta) V - diag(beta e^{b}) K H
//   U   = T R                          (the rows of U are the u_t of the recurrence)
//   O   = diag(e^{b}) Q H + [(q_i . k_j) e^{b_i - b_j}]_{j<=i} U     (post-write read)
//       = diag(e^{b'}) Q H + [(q_i . k_j) e^{b'_i - b_j}]_{j<i} U    (pre-write read)
//   H  <- e^{b_C} H + K^T diag(e^{b_C - b}) U
//
// This is the WY/UT chunk form of `chunked_delta` (gated branch) on the "Prizma
// seq/delta.py" page, transposed to H = S^T and with the solve applied as an explicit
// inverse T so that it becomes a matrix-core product; the decay ratios are formed as
// exponentials of log differences that are never positive (that page's underflow note).
//
// Work split inside the workgroup, per chunk:
//   all waves   Gram tiles K K^T and Q K^T (lower triangle only) -> A (fp32) and P (E) in LDS
//   wave 0      T = (I + A)^{-1}: 16x16 diagonal blocks by forward substitution (one lane
//               per column), off-diagonal blocks by block merges on the matrix cores
//   waves 0, 1  the state-dependent chain for one 16-column tile of d_v each; the state
//               tile lives in accumulator registers and is fed back as a B operand
//               directly (see gdr_mfma.hpp), so the chain needs no LDS round trip
//   all threads prefetch the next chunk's q/k/v/gates into registers during the chunk
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "gdr_kernels.hpp"
#include "gdr_mfma.hpp"
#include "gdr_solve.hpp"

namespace gdr {

namespace {

constexpr int kThreads = 256;
constexpr int kDvTile = 32;

template <typename E>
struct Pad {
    static constexpr int v = 16 / sizeof(E);  // one 16-byte pad per row
};

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(__bf16 x) { return (float)x; }
template <typename E>
__device__ __forceinline__ E from_f(float x) { return (E)x; }

template <typename E, int C, int DK>
struct Smem {
    static constexpr int KP = DK + Pad<E>::v;       // pitch of K/Q rows (elements)
    static constexpr int VP = kDvTile + Pad<E>::v;  // pitch of V rows
    static constexpr int AP = C + 4;                // pitch of the fp32 A matrix
    static constexpr int TP = C + Pad<E>::v;        // pitch of T and P
    E K[C * KP];
    E Q[C * KP];
    E V[C * VP];
    E T[C * TP];
    E P[C * TP];
    float A[C * AP];
    float la[C];    // raw log alpha of the chunk (0 past the end)
    float beta[C];  // beta (0 past the end)
    float b[C];     // inclusive cumsum of la
};

// Registers holding the next chunk while the current one is processed.
template <typename E, int C, int DK>
struct Prefetch {
    static constexpr int KPIECES = C * DK * (int)sizeof(E) / 16;      // 16-byte pieces
    static constexpr int KPER = (KPIECES + kThreads - 1) / kThreads;
    static constexpr int VPIECES = C * kDvTile * (int)sizeof(E) / 16;
    static constexpr int VPER = (VPIECES + kThreads - 1) / kThreads;
    static constexpr int KROW = DK * (int)sizeof(E) / 16;             // pieces per K row
    static constexpr int VROW = kDvTile * (int)sizeof(E) / 16;
    uint4 k[KPER], q[KPER], v[VPER];
    float la, beta;
};

// One sequence as the kernel walks it. With ns delta sub-steps per token (DeltaProduct) the
// walk is over the ns * tokens sub-steps of the sequence in order; k, v and beta are stored per
// sub-step, q, the decay and the output per token: sub-step pos belongs to token tok0 + pos / ns,
// the decay enters on its first sub-step and the read happens on sub-step jread of each token.
struct SeqView {
    int64_t t0, len;  // first step (token, or sub-step) and length of the sequence in its row
    int64_t tok0;     // first token of the sequence (= t0 when ns == 1)
    bool rev;         // only with ns == 1
    int ns, jread;
    __device__ __forceinline__ int64_t token(int64_t pos) const { return rev ? t0 + len - 1 - pos : t0 + pos; }
    // token of step pos and whether that step is the one its token reads at / decays at
    __device__ __forceinline__ int64_t owner(int64_t pos, bool &read_step, bool &first_step) const {
        if (ns == 1) {
            read_step = first_step = true;
            return token(pos);
        }
        const int p = (int)pos, j = p % ns;
        read_step = j == jread;
        first_step = j == 0;
        return tok0 + p / ns;
    }
};

template <typename E, int C, int DK>
__device__ __forceinline__ void prefetch_chunk(Prefetch<E, C, DK> &pf, const SeqView &sv, int64_t c,
                                               const char *kb, const char *qb, const char *vb,
                                               const float *ab, const float *bb, int64_t dv, int dcol0,
                                               const float *A_log, const float *dt_bias, int64_t head) {
    typedef Prefetch<E, C, DK> PF;
    const int tid = threadIdx.x;
    const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < PF::KPER; ++i) {
        const int piece = tid + i * kThreads;
        pf.k[i] = z;
        pf.q[i] = z;
        if (piece < PF::KPIECES) {
            const int r = piece / PF::KROW, cp = piece % PF::KROW;
            const int64_t pos = c * C + r;
            if (pos < sv.len) {
                const int64_t off = sv.token(pos) * (int64_t)(DK * sizeof(E)) + cp * 16;
                pf.k[i] = *reinterpret_cast<const uint4 *>(kb + off);
                bool rd, first;
                const int64_t t = sv.owner(pos, rd, first);
                if (rd) pf.q[i] = *reinterpret_cast<const uint4 *>(qb + t * (int64_t)(DK * sizeof(E)) + cp * 16);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < PF::VPER; ++i) {
        const int piece = tid + i * kThreads;
        pf.v[i] = z;
        if (piece < PF::VPIECES) {
            const int r = piece / PF::VROW, cp = piece % PF::VROW;
            const int64_t pos = c * C + r;
            if (pos < sv.len) {
                const int64_t off = (sv.token(pos) * dv + dcol0) * (int64_t)sizeof(E) + cp * 16;
                pf.v[i] = *reinterpret_cast<const uint4 *>(vb + off);
            }
        }
    }
    pf.la = 0.f;
    pf.beta = 0.f;
    if (tid < C) {
        const int64_t pos = c * C + tid;
        if (pos < sv.len) {
            const int64_t e = sv.token(pos);
            bool rd, first;
            const int64_t t = sv.owner(pos, rd, first);
            // raw gate inputs become log alpha and beta here when A_log is given
            if (first) pf.la = A_log ? gate_log_alpha(ab[t], A_log, dt_bias, head) : ab[t];
            pf.beta = A_log ? gate_beta(bb[e]) : bb[e];
        }
    }
}

template <typename E, int C, int DK>
__device__ __forceinline__ void store_chunk(const Prefetch<E, C, DK> &pf, Smem<E, C, DK> &sm) {
    typedef Prefetch<E, C, DK> PF;
    typedef Smem<E, C, DK> SM;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < PF::KPER; ++i) {
        const int piece = tid + i * kThreads;
        if (piece < PF::KPIECES) {
            const int r = piece / PF::KROW, cp = piece % PF::KROW;
            *reinterpret_cast<uint4 *>(reinterpret_cast<char *>(sm.K + r * SM::KP) + cp * 16) = pf.k[i];
            *reinterpret_cast<uint4 *>(reinterpret_cast<char *>(sm.Q + r * SM::KP) + cp * 16) = pf.q[i];
        }
    }
#pragma unroll
    for (int i = 0; i < PF::VPER; ++i) {
        const int piece = tid + i * kThreads;
        if (piece < PF::VPIECES) {
            const int r = piece / PF::VROW, cp = piece % PF::VROW;
            *reinterpret_cast<uint4 *>(reinterpret_cast<char *>(sm.V + r * SM::VP) + cp * 16) = pf.v[i];
        }
    }
    if (tid < C) {
        sm.la[tid] = pf.la;
        sm.beta[tid] = pf.beta;
    }
}

// Unit-norm rows: every row of K and Q in LDS divided by max(||row||, eps) (rows past the
// end are zero and stay zero). One wave per row at a time; each lane holds DK / 64 elements.
template <typename E, int C, int DK>
__device__ __forceinline__ void normalize_rows(Smem<E, C, DK> &sm) {
    typedef Smem<E, C, DK> SM;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    constexpr int PER = DK / 64;
    for (int row = wave; row < 2 * C; row += kThreads / 64) {
        E *p = (row < C ? sm.K : sm.Q) + (row % C) * SM::KP;
        float x[PER], s = 0.f;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            x[e] = to_f(p[lane + 64 * e]);
            s += x[e] * x[e];
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
        const float r = 1.f / fmaxf(sqrtf(s), kL2Eps);
#pragma unroll
        for (int e = 0; e < PER; ++e) p[lane + 64 * e] = from_f<E>(x[e] * r);
    }
}

// Inclusive prefix sum of la over the chunk (wave 0, lane i = token i).
template <typename E, int C, int DK>
__device__ __forceinline__ void gate_cumsum(Smem<E, C, DK> &sm) {
    const int lane = threadIdx.x & 63;
    float x = lane < C ? sm.la[lane] : 0.f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane < C) sm.b[lane] = x;
}

// Lower-triangular 16x16 tiles of K K^T (-> A) and Q K^T (-> P), spread over the waves.
template <typename E, int C, int DK>
__device__ __forceinline__ void gram_tiles(Smem<E, C, DK> &sm, bool pre) {
    typedef Smem<E, C, DK> SM;
    constexpr int NT = C / 16;
    constexpr int NTRI = NT * (NT + 1) / 2;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, cc = lane & 15;
    for (int t = wave; t < 2 * NTRI; t += kThreads / 64) {
        const int which = t / NTRI;  // 0: K K^T, 1: Q K^T
        int idx = t % NTRI, i = 0;
        while (idx > i) {
            idx -= i + 1;
            ++i;
        }
        const int j = idx;
        const E *X = which ? sm.Q : sm.K;
        floatx4 acc = zero4();
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks)
            acc = mma32(acc, frag_rows<E>(X, SM::KP, 16 * i, 32 * ks), frag_rows<E>(sm.K, SM::KP, 16 * j, 32 * ks));
        const int col = 16 * j + cc;
        const float bcol = sm.b[col];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * i + 4 * g + r;
            const float brow = sm.b[row];
            if (which == 0) {
                const float e = __expf(fminf(brow - bcol, 0.f));
                sm.A[row * SM::AP + col] = (col < row) ? sm.beta[row] * acc[r] * e : 0.f;
            } else {
                const float bread = pre ? brow - sm.la[row] : brow;
                const float e = __expf(fminf(bread - bcol, 0.f));
                const bool keep = pre ? (col < row) : (col <= row);
                sm.P[row * SM::TP + col] = from_f<E>(keep ? acc[r] * e : 0.f);
            }
        }
    }
}

template <typename E, int C, int DK>
__global__ __launch_bounds__(kThreads) void chunk_fwd_kernel(ChunkArgs a) {
    typedef Smem<E, C, DK> SM;
    constexpr int NT = C / 16;
    constexpr int HT = DK / 16;
    __shared__ SM sm;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, cc = lane & 15;

    // block -> (unit, d_v tile); the d_v tiles of one unit land on the same XCD
    // (workgroups are dealt to the 8 XCDs round-robin), so they share K/Q in its L2
    const int64_t blk = blockIdx.x;
    const int64_t xcd = blk & 7, slot = blk >> 3;
    const int64_t unit = (slot / a.ntiles) * 8 + xcd;
    const int tile = (int)(slot % a.ntiles);
    if (unit >= a.units) return;
    const int64_t seq = unit / a.Hv, head = unit % a.Hv;
    const int64_t kh = head / (a.Hv / a.Hk);
    const int64_t row = a.cu_seqlens ? 0 : seq;
    SeqView sv;
    const int ns = a.n_sub;
    sv.ns = ns;
    sv.jread = (a.flags & kFlagReadPre) ? 0 : ns - 1;
    sv.tok0 = 0;
    int64_t ntok = a.T;
    if (a.cu_seqlens) {
        sv.tok0 = a.cu_seqlens[seq];
        ntok = a.cu_seqlens[seq + 1] - sv.tok0;
    }
    sv.t0 = sv.tok0 * ns;
    sv.len = ntok * ns;
    sv.rev = (a.flags & kFlagReverse) != 0;
    const bool pre = (a.flags & kFlagReadPre) != 0;
    const bool acc_out = (a.flags & kFlagAccumulate) != 0;
    const bool l2 = (a.flags & kFlagL2Norm) != 0;
    const int64_t nchunks = (sv.len + C - 1) / C;
    const int dcol0 = tile * kDvTile;

    const int64_t Ts = a.T * ns;  // steps per row
    const char *kb = reinterpret_cast<const char *>(a.k) + (row * a.Hk + kh) * Ts * DK * (int64_t)sizeof(E);
    const char *qb = reinterpret_cast<const char *>(a.q) + (row * a.Hk + kh) * a.T * DK * (int64_t)sizeof(E);
    const char *vb = reinterpret_cast<const char *>(a.v) + (row * a.Hv + head) * Ts * a.dv * (int64_t)sizeof(E);
    const float *ab = a.log_alpha + (row * a.Hv + head) * a.T;
    const float *bb = a.beta + (row * a.Hv + head) * Ts;
    E *ob = reinterpret_cast<E *>(a.out) + (row * a.Hv + head) * a.T * a.dv;

    // zero T and P once: their strictly upper blocks are never written again
    for (int i = tid; i < C * SM::TP; i += kThreads) {
        sm.T[i] = from_f<E>(0.f);
        sm.P[i] = from_f<E>(0.f);
    }

    // the chain waves hold their 16-column state tile: rows 16t + 4g + r, column dcol + cc
    const bool chain = wave < 2;
    const int lcol = wave * 16;           // column inside the 32-wide tile
    const int dcol = dcol0 + lcol + cc;   // column of d_v this lane owns in the chain
    floatx4 H[HT];
#pragma unroll
    for (int t = 0; t < HT; ++t) H[t] = zero4();
    if (chain && a.h0) {
        const float *hb = a.h0 + (seq * a.Hv + head) * DK * a.dv;
#pragma unroll
        for (int t = 0; t < HT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) H[t][r] = hb[(16 * t + 4 * g + r) * a.dv + dcol];
    }

    Prefetch<E, C, DK> pf;
    if (nchunks > 0) {
        prefetch_chunk<E, C, DK>(pf, sv, 0, kb, qb, vb, ab, bb, a.dv, dcol0, a.A_log, a.dt_bias, head);
        store_chunk<E, C, DK>(pf, sm);
    }
    __syncthreads();
    if (l2 && nchunks > 0) {
        normalize_rows<E, C, DK>(sm);
        __syncthreads();
    }

    for (int64_t c = 0; c < nchunks; ++c) {
        if (c + 1 < nchunks) prefetch_chunk<E, C, DK>(pf, sv, c + 1, kb, qb, vb, ab, bb, a.dv, dcol0, a.A_log, a.dt_bias, head);

        if (wave == 0) gate_cumsum<E, C, DK>(sm);
        __syncthreads();
        gram_tiles<E, C, DK>(sm, pre);
        __syncthreads();
        if (wave == 0) solve_unit_lower_inverse<E, C>(sm);
        __syncthreads();

        if (chain) {
            // X_K = K H, X_Q = Q H
            floatx4 XK[NT], XQ[NT];
#pragma unroll
            for (int mi = 0; mi < NT; ++mi) {
                XK[mi] = zero4();
                XQ[mi] = zero4();
            }
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks) {
                const Frag<E> hb = frag_from_acc<E>(H[2 * ks], H[2 * ks + 1]);
#pragma unroll
                for (int mi = 0; mi < NT; ++mi) {
                    XK[mi] = mma32(XK[mi], frag_rows<E>(sm.K, SM::KP, 16 * mi, 32 * ks), hb);
                    XQ[mi] = mma32(XQ[mi], frag_rows<E>(sm.Q, SM::KP, 16 * mi, 32 * ks), hb);
                }
            }
            // R = beta V - beta e^{b} X_K
            floatx4 R[NT];
#pragma unroll
            for (int mi = 0; mi < NT; ++mi)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int rr = 16 * mi + 4 * g + r;
                    const float be = sm.beta[rr];
                    R[mi][r] = be * to_f(sm.V[rr * SM::VP + lcol + cc]) - be * __expf(sm.b[rr]) * XK[mi][r];
                }
            // U = T R (T lower triangular: row tile mi needs k tiles <= mi)
            floatx4 U[NT];
#pragma unroll
            for (int mi = 0; mi < NT; ++mi) {
                U[mi] = zero4();
#pragma unroll
                for (int kt = 0; kt <= mi; kt += 2) {
                    if (kt + 1 < NT)
                        U[mi] = mma32(U[mi], frag_rows<E>(sm.T, SM::TP, 16 * mi, 16 * kt), frag_from_acc<E>(R[kt], R[kt + 1]));
                    else
                        U[mi] = mma16(U[mi], frag_rows_lo<E>(sm.T, SM::TP, 16 * mi, 16 * kt), cvt4<E>(R[kt]));
                }
            }
            // O = e^{b or b'} X_Q + P U ; stored per row
            const float blast = sm.b[C - 1];
#pragma unroll
            for (int mi = 0; mi < NT; ++mi) {
                floatx4 o;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int rr = 16 * mi + 4 * g + r;
                    const float bread = pre ? sm.b[rr] - sm.la[rr] : sm.b[rr];
                    o[r] = __expf(bread) * XQ[mi][r];
                }
#pragma unroll
                for (int kt = 0; kt <= mi; kt += 2) {
                    if (kt + 1 < NT)
                        o = mma32(o, frag_rows<E>(sm.P, SM::TP, 16 * mi, 16 * kt), frag_from_acc<E>(U[kt], U[kt + 1]));
                    else
                        o = mma16(o, frag_rows_lo<E>(sm.P, SM::TP, 16 * mi, 16 * kt), cvt4<E>(U[kt]));
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t pos = c * C + 16 * mi + 4 * g + r;
                    bool rd, first;
                    const int64_t t = pos < sv.len ? sv.owner(pos, rd, first) : 0;
                    if (pos < sv.len && rd) {
                        E *dst = ob + t * a.dv + dcol;
                        const float prev = acc_out ? to_f(*dst) : 0.f;
                        *dst = from_f<E>(prev + o[r]);
                    }
                }
            }
            // H <- e^{b_C} H + K^T diag(e^{b_C - b}) U
            floatx4 W[NT];
#pragma unroll
            for (int mi = 0; mi < NT; ++mi)
#pragma unroll
                for (int r = 0; r < 4; ++r) W[mi][r] = __expf(fminf(blast - sm.b[16 * mi + 4 * g + r], 0.f)) * U[mi][r];
            const float gC = __expf(blast);
#pragma unroll
            for (int t = 0; t < HT; ++t) {
                H[t] = H[t] * gC;
#pragma unroll
                for (int kt = 0; kt < NT; kt += 2) {
                    if (kt + 1 < NT)
                        H[t] = mma32(H[t], frag_cols<E>(sm.K, SM::KP, 16 * t, 16 * kt), frag_from_acc<E>(W[kt], W[kt + 1]));
                    else
                        H[t] = mma16(H[t], frag_cols_lo<E>(sm.K, SM::KP, 16 * t, 16 * kt), cvt4<E>(W[kt]));
                }
            }
        }
        __syncthreads();
        if (c + 1 < nchunks) {
            store_chunk<E, C, DK>(pf, sm);
            __syncthreads();
            if (l2) {
                normalize_rows<E, C, DK>(sm);
                __syncthreads();
            }
        }
    }

    if (chain && a.hT) {
        float *hb = a.hT + (seq * a.Hv + head) * DK * a.dv;
#pragma unroll
        for (int t = 0; t < HT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) hb[(16 * t + 4 * g + r) * a.dv + dcol] = H[t][r];
    }
}

template <typename E, int C, int DK>
hipError_t launch_typed(const ChunkArgs &a, hipStream_t stream) {
    const int64_t groups = (a.units + 7) / 8;
    const int64_t blocks = groups * 8 * a.ntiles;
    hipLaunchKernelGGL((chunk_fwd_kernel<E, C, DK>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template <typename E>
hipError_t launch_dk(const ChunkArgs &a, int chunk, int dk, hipStream_t s) {
    if (dk == 64) {
        if (chunk == 16) return launch_typed<E, 16, 64>(a, s);
        if (chunk == 32) return launch_typed<E, 32, 64>(a, s);
        return launch_typed<E, 64, 64>(a, s);
    }
    if (chunk == 16) return launch_typed<E, 16, 128>(a, s);
    if (chunk == 32) return launch_typed<E, 32, 128>(a, s);
    return launch_typed<E, 64, 128>(a, s);
}

}  // namespace

hipError_t launch_chunk_fwd(const ChunkArgs &a, int dtype, int chunk, int dk, hipStream_t stream) {
    if (a.units == 0 || a.ntiles == 0) return hipSuccess;
    // The fast kernel takes 1, 2, 4, 8 or 16 delta sub-steps per token (they divide its chunk,
    // so a chunk starts on a token) and head slabs whose byte offsets fit its 32-bit copies.
    const bool pow2 = (a.n_sub & (a.n_sub - 1)) == 0;
    const int64_t slab_rows = a.T * (int64_t)a.n_sub;
    const int64_t row_bytes = a.dv * 2 > 256 ? a.dv * 2 : 256;
    if (pow2 && slab_rows * row_bytes < INT32_MAX && chunk_fwd_fast_supported(dtype, chunk, dk))
        return launch_chunk_fwd_fast(a, stream);
    if (dtype == kDtypeBf16) return launch_dk<__bf16>(a, chunk, dk, stream);
    return launch_dk<float>(a, chunk, dk, stream);
}

// ---------------------------------------------------------------- diagnostic

__global__ void selftest_mfma_kernel(const float *A, const float *B, float *D) {
    // A [16][32], B [32][16] row-major; D[3][16][16]
    const int lane = threadIdx.x & 63, g = lane >> 4, cc = lane & 15;
    __shared__ float sa[16 * 32], sb[32 * 16];
    __shared__ __bf16 ha[16 * 32], hb[32 * 16];
    for (int i = threadIdx.x; i < 512; i += 64) {
        sa[i] = A[i];
        sb[i] = B[i];
        ha[i] = (__bf16)A[i];
        hb[i] = (__bf16)B[i];
    }
    __syncthreads();
    floatx4 d0 = mma32(zero4(), frag_rows<__bf16>(ha, 32, 0, 0), frag_cols<__bf16>(hb, 16, 0, 0));
    floatx4 d1 = mma32(zero4(), frag_rows<float>(sa, 32, 0, 0), frag_cols<float>(sb, 16, 0, 0));
    floatx4 d2 = mma16(zero4(), frag_rows_lo<__bf16>(ha, 32, 0, 0), frag_cols_lo<__bf16>(hb, 16, 0, 0));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        D[(4 * g + r) * 16 + cc] = d0[r];
        D[256 + (4 * g + r) * 16 + cc] = d1[r];
        D[512 + (4 * g + r) * 16 + cc] = d2[r];
    }
}

hipError_t launch_selftest_mfma(const float *a, const float *b, float *d, hipStream_t stream) {
    hipLaunchKernelGGL(selftest_mfma_kernel, dim3(1), dim3(64), 0, stream, a, b, d);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return hipStreamSynchronize(stream);
}

}  // namespace gdr
