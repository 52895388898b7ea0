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
// Only two of these quantities are carried from chunk to chunk: the state H (forward) and its
// adjoint dH (backward). Everything else is local to a chunk once H and dH' are known. So the
// backward runs as three kernels on one stream, 64-token chunks:
//
//   1. prep, one workgroup per (value head, chunk): the gate cumsums b and r, G, Pm and
//      T = (I + A)^{-1}; T, T^T and Pm^T go to the workspace as ready matrix-core operands.
//   2. sweeps, one workgroup per (sequence, value head, 32 value columns) and direction, the
//      two directions in one launch: the forward sweep keeps H and per chunk forms X, R, U (U is
//      stored) and the next H, storing each chunk's entry state; the adjoint sweep keeps dH and
//      per chunk forms dU, dR (stored; dV = diag(beta) dR is written) and the previous dH,
//      storing each chunk's exit adjoint. Neither needs the other.
//   3. gradients, one workgroup per (key head, chunk): for each value head of the key head
//      (in order) and each 32-column slice (in order) it reads H, dH', U and dR of the chunk and
//      accumulates X, K dH', dP, dA, dO H^T and the dK terms over the slices; then M, N, the rest
//      of dQ and dK, and the gate gradients. dq and dk are summed over the value heads in the
//      workgroup's registers, so every gradient is written once, by one workgroup, in a fixed
//      order: the same bits on every call, with no float atomics and no second reduction.
//
// All products run on the matrix cores as split bf16 products with fp32 accumulation: an fp32
// operand x is split into hi = bf16(x) and lo = bf16(x - hi) and a 32-deep product is
// hi*hi + hi*lo + lo*hi (relative error near 2^-16 per product); q, k, v and dout of a bf16 call
// hold bf16 values exactly, so their lo parts are zero and those products are skipped.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "gdr_kernels.hpp"
#include "gdr_mfma.hpp"
#include "gdr_solve.hpp"

namespace gdr {

namespace {

constexpr int CB = kBwdBlock;  // tokens per chunk
constexpr int TV = kBwdCols;   // value columns per slice
constexpr int NMT = CB / 16;   // 16-row tiles of a chunk
constexpr int kWaves = 8, kThreads = 64 * kWaves;
constexpr int kPrepThreads = 256;
static_assert(CB == 64 && TV == 32, "the tile assignments are written for 64-token chunks and 32-column slices");
constexpr int SP = CB + 4;  // pitch of fp32 [CB][CB] matrices
template <typename E>
constexpr int pad_of() { return 16 / (int)sizeof(E); }  // one 16-byte piece of padding per row

// The record of one (value head, chunk slot): A-operand fragments of T, T^T and Pm^T as split
// bf16 ([16-row tile][32-deep slice][lane] of a 16-byte hi part and a 16-byte lo part, in the
// register layout mma32 takes), then b[CB] and r[CB].
constexpr int kSlabBytes = 64 * 32;
constexpr int kSlices = CB / 32;
constexpr int kMatBytes = NMT * kSlices * kSlabBytes;
constexpr int kRecT = 0, kRecTt = kMatBytes, kRecPt = 2 * kMatBytes;
template <int DK>
struct Rec {
    static constexpr int64_t kBytes = kBwdRecBytes;
    static constexpr int kGates = 3 * kMatBytes;
    static_assert(kGates + 2 * CB * 4 == kBytes, "record layout");
};

// the lower 16x16 tiles (mt >= nt) of a CB x CB matrix, in a fixed order
__device__ __forceinline__ void lower_tile(int idx, int &mt, int &nt) {
    mt = idx >= 6 ? 3 : idx >= 3 ? 2 : idx >= 1 ? 1 : 0;
    nt = idx - mt * (mt + 1) / 2;
}

struct Seq {
    int64_t t0, len;
    bool rev;
    __device__ __forceinline__ int64_t token(int64_t pos) const { return rev ? t0 + len - 1 - pos : t0 + pos; }
    // the lowest token of chunk c (n rows), and row r's distance from it: per-lane addresses are a
    // uniform base plus a small unsigned offset, which the loads take in scalar-base form
    __device__ __forceinline__ int64_t low(int64_t c, int n) const { return rev ? token(c * CB + n - 1) : token(c * CB); }
    __device__ __forceinline__ int off(int r, int n) const { return rev ? n - 1 - r : r; }
};
struct Loc {
    int64_t seq, row, slot0;  // row: the batch row of q, k, v (0 when packed)
    Seq sq;
};
__device__ __forceinline__ Loc locate_seq(const BwdArgs &a, int64_t seq) {
    Loc L;
    L.seq = seq;
    L.row = a.cu_seqlens ? 0 : seq;
    L.sq.t0 = 0;
    L.sq.len = a.T;
    L.slot0 = seq * ((a.T + CB - 1) / CB);
    if (a.cu_seqlens) {
        L.sq.t0 = a.cu_seqlens[seq];
        L.sq.len = a.cu_seqlens[seq + 1] - L.sq.t0;
        L.slot0 = L.sq.t0 / CB + seq;
    }
    L.sq.rev = (a.flags & kFlagReverse) != 0;
    return L;
}
// the sequence and chunk of a chunk slot; false for a slot that holds no chunk (packed inputs
// leave gaps). Slots of sequence s start at cu[s] / CB + s, which increases with s.
__device__ __forceinline__ bool locate_slot(const BwdArgs &a, int64_t slot, Loc &L, int64_t &c) {
    if (!a.cu_seqlens) {
        const int64_t nch = (a.T + CB - 1) / CB;
        if (nch == 0) return false;
        L = locate_seq(a, slot / nch);
        c = slot % nch;
        return L.seq < a.B;
    }
    int64_t lo = 0, hi = a.nseq - 1;
    while (lo < hi) {
        const int64_t mid = (lo + hi + 1) >> 1;
        if ((int64_t)a.cu_seqlens[mid] / CB + mid <= slot) lo = mid;
        else hi = mid - 1;
    }
    L = locate_seq(a, lo);
    c = slot - L.slot0;
    return c >= 0 && c * CB < L.sq.len;
}

// ---------------------------------------------------------------- operands

// An operand fragment split once (hi, lo); for an operand that holds bf16 values exactly only hi
// is set, and the products below skip its lo part.
struct Split {
    Frag<__bf16> h, l;
};
__device__ __forceinline__ void split_bf16(const floatx4 &x, bf16x4 &hi, bf16x4 &lo) {
    hi = cvt4<__bf16>(x);
    floatx4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = x[i] - (float)hi[i];
    lo = cvt4<__bf16>(r);
}
__device__ __forceinline__ Split split_frag(const Frag<float> &f) {
    Split s;
    split_bf16(f.lo, s.h.lo, s.l.lo);
    split_bf16(f.hi, s.h.hi, s.l.hi);
    return s;
}
// acc += a b; AX / BX: the operand is exactly bf16 (lo = 0)
template <bool AX, bool BX>
__device__ __forceinline__ floatx4 mms(floatx4 acc, const Split &a, const Split &b) {
    if constexpr (!AX) acc = mma32(acc, a.l, b.h);
    if constexpr (!BX) acc = mma32(acc, a.h, b.l);
    return mma32(acc, a.h, b.h);
}
// gfx950 transpose read: in each 16-lane group, lane i receives element i % 4 of the 8-byte
// pieces addressed by lanes 4v + i / 4 (v = 0..3)
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
__device__ __forceinline__ bf16x4 tr16(const __bf16 *p) {
    return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(p)));
}
// columns of a row-major bf16 matrix (as frag_cols): lane j of group g addresses row
// k0 + 4g + j / 4, columns col0 + 4 (j % 4) .. + 3, so that lane c receives X[k0 + 4g + v][col0 + c]
__device__ __forceinline__ Frag<__bf16> cols_tr(const __bf16 *X, int ld, int col0, int k0) {
    const int lane = threadIdx.x & 63, g = lane >> 4, j = lane & 15;
    const __bf16 *p = X + (k0 + 4 * g + (j >> 2)) * ld + col0 + 4 * (j & 3);
    Frag<__bf16> f;
    f.lo = tr16(p);
    f.hi = tr16(p + 16 * ld);
    return f;
}
// from an E-typed matrix in LDS: rows (A[m][k] = X[m][k] or B[k][n] = X[n][k]) or columns
template <typename E>
__device__ __forceinline__ Split ldr(const E *X, int ld, int row0, int k0) {
    if constexpr (std::is_same<E, __bf16>::value) {
        Split s{};
        s.h = frag_rows<__bf16>(X, ld, row0, k0);
        return s;
    } else {
        return split_frag(frag_rows<float>(X, ld, row0, k0));
    }
}
template <typename E>
__device__ __forceinline__ Split ldc(const E *X, int ld, int col0, int k0) {
    if constexpr (std::is_same<E, __bf16>::value) {
        Split s{};
        s.h = cols_tr(X, ld, col0, k0);
        return s;
    } else {
        return split_frag(frag_cols<float>(X, ld, col0, k0));
    }
}
// rows of an fp32 matrix, each lane's row scaled by sc
__device__ __forceinline__ Split ldr_scaled(const float *X, int ld, int row0, int k0, float sc) {
    Frag<float> f = frag_rows<float>(X, ld, row0, k0);
    f.lo *= sc;
    f.hi *= sc;
    return split_frag(f);
}
// An fp32 matrix held in LDS already split: planes h (bf16(x)) and l (bf16(x - h)), R x C each.
// Split once where a value is produced instead of at every read: a row fragment is then two 8-byte
// reads per plane and a column fragment two transposed reads per plane, with no conversions.
template <int R, int C>
struct SplitMat {
    static constexpr int P = C + 8;  // pitch in bf16: one 16-byte piece of padding per row
    __bf16 h[R][P], l[R][P];
};
template <int R, int C>
__device__ __forceinline__ Split sm_rows(const SplitMat<R, C> &X, int row0, int k0) {
    Split s;
    s.h = frag_rows<__bf16>(&X.h[0][0], SplitMat<R, C>::P, row0, k0);
    s.l = frag_rows<__bf16>(&X.l[0][0], SplitMat<R, C>::P, row0, k0);
    return s;
}
template <int R, int C>
__device__ __forceinline__ Split sm_cols(const SplitMat<R, C> &X, int col0, int k0) {
    Split s;
    s.h = cols_tr(&X.h[0][0], SplitMat<R, C>::P, col0, k0);
    s.l = cols_tr(&X.l[0][0], SplitMat<R, C>::P, col0, k0);
    return s;
}
// element (r, c) as fp32 (h + l)
template <int R, int C>
__device__ __forceinline__ float sm_get(const SplitMat<R, C> &X, int r, int c) {
    return (float)X.h[r][c] + (float)X.l[r][c];
}
// the accumulator tile v of lane (g, c) (rows m0 + 4g .. + 3, column n0 + c) stored transposed:
// Xt[n0 + c][m0 + 4g .. + 3], one 8-byte write per plane
template <int R, int C>
__device__ __forceinline__ void sm_put_t(SplitMat<R, C> &Xt, int m0, int n0, const floatx4 &v) {
    const int lane = threadIdx.x & 63;
    bf16x4 hi, lo;
    split_bf16(v, hi, lo);
    const int rr = n0 + (lane & 15), cc = m0 + 4 * (lane >> 4);
    *reinterpret_cast<bf16x4 *>(&Xt.h[rr][cc]) = hi;
    *reinterpret_cast<bf16x4 *>(&Xt.l[rr][cc]) = lo;
}
// columns of a row-major E-typed matrix in LDS (as frag_cols), row k scaled by sk[k], split
template <typename E>
__device__ __forceinline__ Split cols_kscaled(const E *X, int ld, int col0, int k0, const float *sk) {
    const int lane = threadIdx.x & 63;
    const int kb = k0 + 4 * (lane >> 4);
    Frag<float> f;
    if constexpr (std::is_same<E, __bf16>::value) {
        const Frag<__bf16> x = cols_tr(X, ld, col0, k0);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            f.lo[s] = (float)x.lo[s] * sk[kb + s];
            f.hi[s] = (float)x.hi[s] * sk[kb + 16 + s];
        }
    } else {
        const Frag<float> x = frag_cols<float>(X, ld, col0, k0);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            f.lo[s] = x.lo[s] * sk[kb + s];
            f.hi[s] = x.hi[s] * sk[kb + 16 + s];
        }
    }
    return split_frag(f);
}
// rows of a split matrix (the 32 columns from column 0), each lane's row scaled by sc and split again
template <int R, int C>
__device__ __forceinline__ Split sm_scaled_rows(const SplitMat<R, C> &X, int row0, float sc) {
    const Split a = sm_rows(X, row0, 0);
    Frag<float> f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f.lo[i] = sc * ((float)a.h.lo[i] + (float)a.l.lo[i]);
        f.hi[i] = sc * ((float)a.h.hi[i] + (float)a.l.hi[i]);
    }
    return split_frag(f);
}
// four consecutive elements of a row
template <int R, int C>
__device__ __forceinline__ void sm_put4(SplitMat<R, C> &X, int r, int c, const float4 &v) {
    bf16x4 hi, lo;
    split_bf16(floatx4{v.x, v.y, v.z, v.w}, hi, lo);
    *reinterpret_cast<bf16x4 *>(&X.h[r][c]) = hi;
    *reinterpret_cast<bf16x4 *>(&X.l[r][c]) = lo;
}

// a fragment slab of a record, as loaded (two 16-byte pieces per lane)
struct Slab {
    uint4 h, l;
};
__device__ __forceinline__ Slab ld_slab(const uint8_t *rec, int off, int mt, int ks) {
    const uint4 *p = reinterpret_cast<const uint4 *>(rec + off + (mt * kSlices + ks) * kSlabBytes + (threadIdx.x & 63) * 32);
    Slab s;
    s.h = p[0];
    s.l = p[1];
    return s;
}
__device__ __forceinline__ Split slab_split(const Slab &s) {
    Split r;
    r.h = __builtin_bit_cast(Frag<__bf16>, s.h);
    r.l = __builtin_bit_cast(Frag<__bf16>, s.l);
    return r;
}

// no instruction is moved across this point by the compiler's scheduler: keeps a phase's loads
// from being hoisted all at once (which costs more registers than the latency it hides)
__device__ __forceinline__ void fence_sched() { __builtin_amdgcn_sched_barrier(0); }

// The address of an LDS object, hidden from the optimizer (it is uniform and stays in a scalar
// register): addresses derived from it are then formed where they are used instead of being
// hoisted out of a loop and kept live across it, which with a large LDS layout (offsets beyond
// the 64 KiB the instructions' immediates reach) costs a vector register per access pattern.
typedef __attribute__((address_space(3))) char lds_char;
template <typename T>
__device__ __forceinline__ T *lds_opaque(T *p) {
    uint32_t off = (uint32_t)(uintptr_t)(lds_char *)(char *)p;
    asm volatile("" : "+s"(off));
    return reinterpret_cast<T *>((char *)(lds_char *)(uintptr_t)off);
}

// x moved between the lanes of each 16-lane row by the DPP control CTRL (a VALU operation)
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
// sum of x over the 16 lanes of a lane group (the columns of a tile row): swaps within quads
// (quad_perm [1,0,3,2], [2,3,0,1]), then the row rotated by 4 and by 8 lanes; every lane ends
// with the sum (in the same order on every run)
__device__ __forceinline__ float row16(float x) {
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x124>(x);
    x += dpp<0x128>(x);
    return x;
}
// sum of x over the 4 lane groups (the rows 4g + r of a tile column, for fixed r)
__device__ __forceinline__ float col4(float x) {
    x += __shfl_xor(x, 16, 64);
    x += __shfl_xor(x, 32, 64);
    return x;
}

// The rows of one chunk of an E-typed [token][stride] matrix, W elements from the row start, as
// 16-byte pieces shared out over NT threads: issued into registers, then stored into LDS (rows
// past the chunk end read the chunk's first row and are stored as zeros). Every thread issues the
// same number of loads (a thread past the last piece reads one again and does not store it), so
// that the compiler can count the loads in flight exactly instead of waiting for all of them.
template <typename E, int W, int NT>
struct Rows {
    static constexpr int EPP = 16 / (int)sizeof(E), PR = W / EPP, N = CB * PR, PT = (N + NT - 1) / NT;
    uint4 p[PT];
    __device__ __forceinline__ void issue(const E *src, int64_t stride, const Seq &sq, int64_t c, int n, int tid) {
        const E *base = src + sq.low(c, n) * stride;
#pragma unroll
        for (int e = 0; e < PT; ++e) {
            const int i = (tid + e * NT) % N, rr = i / PR, pc = i % PR;
            const uint32_t o = (uint32_t)(sq.off(rr < n ? rr : 0, n) * (int)stride + pc * EPP);
            p[e] = *reinterpret_cast<const uint4 *>(base + o);
        }
    }
    __device__ __forceinline__ void store(E *dst, int pitch, int n, int tid) const {
#pragma unroll
        for (int e = 0; e < PT; ++e) {
            const int i = tid + e * NT, rr = i / PR, pc = i % PR;
            if (i < N) *reinterpret_cast<uint4 *>(dst + rr * pitch + pc * EPP) = rr < n ? p[e] : make_uint4(0, 0, 0, 0);
        }
    }
};

// inclusive prefix sum over the 64 lanes of a wave
__device__ __forceinline__ float wave_scan(float x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    return x;
}

// ---------------------------------------------------------------- 1. prep

template <typename E, int DK>
struct PrepSmem {
    static constexpr int KP = DK + pad_of<E>(), AP = SP, TP = SP;
    // Once the products that read K and Q are done, T (zeroed, then written by the solve) takes
    // the place of K and A that of Q (Pm never enters the LDS). With bf16 inputs four workgroups
    // fit on a compute unit.
    union {
        E K[CB][KP];
        float T[CB * SP];  // flat: the shared triangular inverse reads T and A so
    };
    union {
        E Q[CB][KP];
        float A[CB * SP];
    };
    float la[CB], beta[CB], b[CB], r[CB];
};
static_assert(sizeof(PrepSmem<__bf16, 128>) * 4 <= 160 * 1024, "four prep workgroups per compute unit");

// The prep's products: five 16x16 tiles per wave, the ten lower tiles of G and the ten of Pm.
// A Pm^T operand slab (mt, ks) of the record holds Pm tiles (2 ks, mt) and (2 ks + 1, mt) in the
// same lanes (lo and hi halves of the fragment), so the Pm tiles are dealt in those pairs and each
// slab is written from the registers of one wave; a slab whose (2 ks, mt) tile lies above the
// diagonal has only its hi tile. Wave 0, which solves, takes G tiles only. A job is 12 bits,
// kind | tm << 4 | tn << 8 for tile (tm, tn); five per wave.
enum : int { kJobG = 0, kJobPLo = 1, kJobPHi = 2, kJobPOnly = 3 };
constexpr uint64_t prep_job(int kind, int tm, int tn) { return (uint64_t)(kind | tm << 4 | tn << 8); }
constexpr uint64_t prep_jobs(uint64_t j0, uint64_t j1, uint64_t j2, uint64_t j3, uint64_t j4) {
    return j0 | j1 << 12 | j2 << 24 | j3 << 36 | j4 << 48;
}
constexpr uint64_t kPrepJobs[4] = {
    prep_jobs(prep_job(kJobG, 0, 0), prep_job(kJobG, 1, 0), prep_job(kJobG, 1, 1), prep_job(kJobG, 2, 0),
              prep_job(kJobG, 2, 1)),
    prep_jobs(prep_job(kJobPLo, 0, 0), prep_job(kJobPHi, 1, 0), prep_job(kJobPLo, 2, 0), prep_job(kJobPHi, 3, 0),
              prep_job(kJobG, 2, 2)),
    prep_jobs(prep_job(kJobPLo, 2, 1), prep_job(kJobPHi, 3, 1), prep_job(kJobPLo, 2, 2), prep_job(kJobPHi, 3, 2),
              prep_job(kJobG, 3, 0)),
    prep_jobs(prep_job(kJobPOnly, 1, 1), prep_job(kJobPOnly, 3, 3), prep_job(kJobG, 3, 1), prep_job(kJobG, 3, 2),
              prep_job(kJobG, 3, 3)),
};
// Pm^T slabs with no lower tile, written as zeros by wave 0: (mt, ks) = (2, 0) and (3, 0)

template <typename E, int DK>
__device__ __forceinline__ void prep_body(const BwdArgs &a) {
    typedef PrepSmem<E, DK> SM;
    __shared__ __align__(16) SM sm;
    constexpr bool kX = std::is_same<E, __bf16>::value;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, cc = lane & 15;
    const int64_t head = blockIdx.x / a.nslots, slot = blockIdx.x % a.nslots;
    Loc L;
    int64_t c;
    if (!locate_slot(a, slot, L, c)) return;
    const int n = (int)min((int64_t)CB, L.sq.len - c * CB);
    const int64_t kh = head / (a.Hv / a.Hk);
    const bool pre = (a.flags & kFlagReadPre) != 0;
    const E *qb = reinterpret_cast<const E *>(a.q) + (L.row * a.Hk + kh) * a.T * DK;
    const E *kb = reinterpret_cast<const E *>(a.k) + (L.row * a.Hk + kh) * a.T * DK;
    const float *lab = a.log_alpha + (L.row * a.Hv + head) * a.T;
    const float *beb = a.beta + (L.row * a.Hv + head) * a.T;
    {
        Rows<E, DK, kPrepThreads> kp, qp;
        kp.issue(kb, DK, L.sq, c, n, tid);
        qp.issue(qb, DK, L.sq, c, n, tid);
        float lv = 0.f, bv = 0.f;
        if (tid < n) {
            const int64_t t = L.sq.token(c * CB + tid);
            lv = lab[t];
            bv = beb[t];
        }
        kp.store(&sm.K[0][0], SM::KP, n, tid);
        qp.store(&sm.Q[0][0], SM::KP, n, tid);
        if (tid < CB) {
            sm.la[tid] = lv;
            sm.beta[tid] = bv;
        }
    }
    __syncthreads();
    if (wave == 0) {
        const float x = wave_scan(sm.la[lane]);
        sm.b[lane] = x;
        sm.r[lane] = pre ? x - sm.la[lane] : x;
    }
    __syncthreads();
    uint8_t *rec = a.rec + (head * a.nslots + slot) * Rec<DK>::kBytes;
    static_assert(kPrepThreads == 256 && NMT == 4 && kSlices == 2, "the job table is written for 4 waves and 64-token chunks");
    const uint64_t jobs = wave == 0 ? kPrepJobs[0] : wave == 1 ? kPrepJobs[1] : wave == 2 ? kPrepJobs[2] : kPrepJobs[3];
    auto job = [&](int s, int &kind, int &tm, int &tn) __attribute__((always_inline)) {
        const int j = (int)((jobs >> (12 * s)) & 0xfff);
        kind = j & 15;
        tm = (j >> 4) & 15;
        tn = j >> 8;
    };
    floatx4 acc[5];
#pragma unroll
    for (int s = 0; s < 5; ++s) {
        int kind, tm, tn;
        job(s, kind, tm, tn);
        acc[s] = zero4();
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks)
            acc[s] = mms<kX, kX>(acc[s], ldr<E>(kind == kJobG ? &sm.K[0][0] : &sm.Q[0][0], SM::KP, 16 * tm, 32 * ks),
                                 ldr<E>(&sm.K[0][0], SM::KP, 16 * tn, 32 * ks));
    }
    // Pm^T slab (mt, ks) from its tiles' registers: Pm_ij = (Q K^T)_ij e^{r_i - b_j} on the kept
    // entries (j <= i, or j < i for the pre-write read)
    auto put_pt = [&](int mt, int ks, const floatx4 &lo, const floatx4 &hi) __attribute__((always_inline)) {
        Frag<float> f;
        f.lo = lo;
        f.hi = hi;
        const Split sp = split_frag(f);
        uint4 *dst = reinterpret_cast<uint4 *>(rec + kRecPt + (mt * kSlices + ks) * kSlabBytes + lane * 32);
        dst[0] = __builtin_bit_cast(uint4, sp.h);
        dst[1] = __builtin_bit_cast(uint4, sp.l);
    };
    {
        floatx4 plo = zero4();
#pragma unroll
        for (int s = 0; s < 5; ++s) {
            int kind, tm, tn;
            job(s, kind, tm, tn);
            if (kind == kJobG) continue;
            floatx4 pv;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * tm + 4 * g + r, j = 16 * tn + cc;
                const bool keep = pre ? j < i : j <= i;
                pv[r] = keep ? acc[s][r] * __expf(fminf(sm.r[i] - sm.b[j], 0.f)) : 0.f;
            }
            if (kind == kJobPLo) plo = pv;
            else put_pt(tn, tm >> 1, kind == kJobPHi ? plo : zero4(), pv);
        }
        if (wave == 0) {
            put_pt(2, 0, zero4(), zero4());
            put_pt(3, 0, zero4(), zero4());
        }
    }
    __syncthreads();
    for (int i = tid; i < CB * SP; i += kPrepThreads) sm.T[i] = 0.f;
    // the G tiles into A (over Q), each with its mirrored upper tile of zeros
#pragma unroll
    for (int s = 0; s < 5; ++s) {
        int kind, tm, tn;
        job(s, kind, tm, tn);
        if (kind != kJobG) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * tm + 4 * g + r, j = 16 * tn + cc;
            sm.A[i * SP + j] = j < i ? sm.beta[i] * acc[s][r] * __expf(fminf(sm.b[i] - sm.b[j], 0.f)) : 0.f;
            if (tm > tn) sm.A[(16 * tn + 4 * g + r) * SP + 16 * tm + cc] = 0.f;
        }
    }
    __syncthreads();
    if (wave == 0) solve_unit_lower_inverse<float, CB>(sm);
    __syncthreads();
    // T and T^T as A-operand fragments: lane (g, c) of slab (mt, ks) holds row 16 mt + c,
    // columns 32 ks + 4g + s and 32 ks + 16 + 4g + s (s = 0..3)
    for (int it = tid; it < 2 * NMT * kSlices * 64; it += kPrepThreads) {
        const int mat = it / (NMT * kSlices * 64), sl = (it / 64) % (NMT * kSlices), ln = it % 64;
        const int mt = sl / kSlices, ks = sl % kSlices;
        const int row = 16 * mt + (ln & 15), kb0 = 32 * ks + 4 * (ln >> 4);
        Frag<float> f;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int k = kb0 + (s < 4 ? s : 12 + s);
            const float x = mat == 0 ? sm.T[row * SP + k] : sm.T[k * SP + row];
            if (s < 4) f.lo[s] = x;
            else f.hi[s - 4] = x;
        }
        const Split sp = split_frag(f);
        uint4 *dst = reinterpret_cast<uint4 *>(rec + mat * kMatBytes + sl * kSlabBytes + ln * 32);
        dst[0] = __builtin_bit_cast(uint4, sp.h);
        dst[1] = __builtin_bit_cast(uint4, sp.l);
    }
    if (tid < CB) {
        float *rb = reinterpret_cast<float *>(rec + Rec<DK>::kGates);
        rb[tid] = sm.b[tid];
        rb[CB + tid] = sm.r[tid];
    }
}

template <typename E, int DK>
__global__ __launch_bounds__(kPrepThreads) void bwd_prep_kernel(BwdArgs a) {
    prep_body<E, DK>(a);
}
// bf16: at most 128 registers, so that four workgroups (4 waves each) fit on a compute unit
template <int DK>
__global__ __launch_bounds__(kPrepThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void bwd_prep_kernel_bf16(BwdArgs a) {
    prep_body<__bf16, DK>(a);
}

// ---------------------------------------------------------------- 2. sweeps

// The sweeps keep the running state (H, or its adjoint D) in the MFMA accumulators of the waves
// that update it, each wave its own 16x16 tiles, in fp32 for the whole unit. What the products read
// is held in LDS split and transposed, so that every B operand is a row fragment: Ht[col][d]
// (the state slice), Rt, wUt, dUt, bRt [col][token].
template <typename E, int DK>
struct FwdSmem {
    static constexpr int KP = DK + pad_of<E>(), VP = TV + pad_of<E>();
    float b[2][CB], beta[2][CB];
    SplitMat<TV, CB> Rt, wUt;
    SplitMat<TV, DK> Ht;
    E V[CB][VP];
    E K[2][CB][KP];  // this chunk's k and the next chunk's
};
template <typename E, int DK>
struct AdjSmem {
    static constexpr int KP = DK + pad_of<E>(), VP = TV + pad_of<E>();
    // one buffer of k, q and dout: the next chunk's are stored after an extra barrier, which
    // keeps a workgroup under 80 KB of LDS (with bf16 inputs), so that a forward and an adjoint
    // workgroup share a compute unit
    float b[CB], er[CB], beta[CB];
    SplitMat<TV, CB> dUt, bRt;
    SplitMat<TV, DK> Dt;
    E dO[CB][VP];
    E K[CB][KP], Q[CB][KP];
};
template <typename E, int DK>
constexpr size_t sweep_smem_bytes() {
    return sizeof(FwdSmem<E, DK>) > sizeof(AdjSmem<E, DK>) ? sizeof(FwdSmem<E, DK>) : sizeof(AdjSmem<E, DK>);
}

// The state tiles of a wave: tile s is (row tile (wave + 8 s) / 2 of d_k, column tile (wave + 8 s) % 2).
template <int DK>
struct StateTiles {
    static constexpr int N = (DK / 16) * (TV / 16) / kWaves;
    static_assert(N * kWaves == (DK / 16) * (TV / 16), "whole state tiles per wave");
    floatx4 v[N];
    __device__ __forceinline__ static int hm(int wave, int s) { return (wave + kWaves * s) / (TV / 16); }
    __device__ __forceinline__ static int hn(int wave, int s) { return (wave + kWaves * s) % (TV / 16); }
    // from / to a [dk][dv] state in global memory (the slice starting at column col0 of row p)
    __device__ __forceinline__ void load(const float *p, int64_t dvf, int wave) {
        const int lane = threadIdx.x & 63, g = lane >> 4, cc = lane & 15;
#pragma unroll
        for (int s = 0; s < N; ++s)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                v[s][r] = p ? p[(int64_t)(16 * hm(wave, s) + 4 * g + r) * dvf + 16 * hn(wave, s) + cc] : 0.f;
    }
    __device__ __forceinline__ void save(float *p, int64_t dvf, int wave) const {
        const int lane = threadIdx.x & 63, g = lane >> 4, cc = lane & 15;
#pragma unroll
        for (int s = 0; s < N; ++s)
#pragma unroll
            for (int r = 0; r < 4; ++r) p[(int64_t)(16 * hm(wave, s) + 4 * g + r) * dvf + 16 * hn(wave, s) + cc] = v[s][r];
    }
    // to a transposed TV x DK slice in the workspace: lane (g, c) holds 4 consecutive d of column c
    __device__ __forceinline__ void save_t(float *p, int wave) const {
        const int lane = threadIdx.x & 63, g = lane >> 4, cc = lane & 15;
#pragma unroll
        for (int s = 0; s < N; ++s)
            *reinterpret_cast<floatx4 *>(p + (16 * hn(wave, s) + cc) * DK + 16 * hm(wave, s) + 4 * g) = v[s];
    }
    __device__ __forceinline__ void put(SplitMat<TV, DK> &Xt, int wave) const {
#pragma unroll
        for (int s = 0; s < N; ++s) sm_put_t(Xt, 16 * hm(wave, s), 16 * hn(wave, s), v[s]);
    }
};

// Forward sweep of one (sequence, value head, column slice): per chunk, the entry state to the
// workspace, X = K H, R = diag(beta) (V - diag(gamma) X), U = T R (U to the workspace) and
// H' = gamma_last H + K^T diag(w) U. The next chunk's k, v and gates are read while the state
// is updated and stored into the other buffer, so a chunk takes three barriers.
template <typename E, int DK>
__device__ __forceinline__ void fwd_sweep(const BwdArgs &a, int64_t unit, int tile, char *smraw) {
    typedef FwdSmem<E, DK> SM;
    SM &sm = *reinterpret_cast<SM *>(smraw);
    constexpr bool kX = std::is_same<E, __bf16>::value;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, cc = lane & 15;
    const int64_t seq = unit / a.Hv, head = unit % a.Hv, kh = head / (a.Hv / a.Hk);
    const Loc L = locate_seq(a, seq);
    const int64_t nch = (L.sq.len + CB - 1) / CB;
    const int64_t dvf = a.ntiles * TV;
    const int col0 = tile * TV;
    const E *kb = reinterpret_cast<const E *>(a.k) + (L.row * a.Hk + kh) * a.T * DK;
    const E *vb = reinterpret_cast<const E *>(a.v) + (L.row * a.Hv + head) * a.T * dvf + col0;
    const float *beb = a.beta + (L.row * a.Hv + head) * a.T;
    float *ub = a.us + (head * a.nslots + L.slot0) * CB * dvf + col0;
    constexpr int64_t kSlice = (int64_t)DK * TV;
    float *hs = a.hs + ((head * a.nslots + L.slot0) * a.ntiles + tile) * kSlice;
    const int64_t hstride = a.ntiles * kSlice;
    const uint8_t *rec0 = a.rec + (head * a.nslots + L.slot0) * Rec<DK>::kBytes;
    StateTiles<DK> H;
    H.load(a.h0 ? a.h0 + (seq * a.Hv + head) * DK * dvf + col0 : nullptr, dvf, wave);
    H.put(sm.Ht, wave);
    // this wave's output tile of X, R and U
    const int mt = wave >> 1, nt = wave & 1;
    Rows<E, DK, kThreads> kp;
    Rows<E, TV, kThreads> vp;
    float bv = 0.f, betav = 0.f;
    // (every thread issues the same loads; only the first CB threads keep the gates)
    auto issue = [&](int64_t c) __attribute__((always_inline)) {
        const int n = (int)min((int64_t)CB, L.sq.len - c * CB);
        kp.issue(kb, DK, L.sq, c, n, tid);
        vp.issue(vb, dvf, L.sq, c, n, tid);
        const int gr = tid & (CB - 1);
        bv = reinterpret_cast<const float *>(rec0 + c * Rec<DK>::kBytes + Rec<DK>::kGates)[gr];
        betav = (beb + L.sq.low(c, n))[(uint32_t)L.sq.off(gr < n ? gr : 0, n)];
    };
    auto store = [&](int64_t c, int buf) __attribute__((always_inline)) {
        const int n = (int)min((int64_t)CB, L.sq.len - c * CB);
        kp.store(&sm.K[buf][0][0], SM::KP, n, tid);
        vp.store(&sm.V[0][0], SM::VP, n, tid);
        if (tid < CB) {
            sm.b[buf][tid] = bv;
            sm.beta[buf][tid] = tid < n ? betav : 0.f;
        }
    };
    // T's rows 16 mt .. 16 mt + 15 are zero past column 16 mt + 15 (the zero slab is read too:
    // the same loads in every wave); a chunk's slabs are read during the previous chunk
    Slab tr[kSlices];
    auto issue_t = [&](int64_t c) __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < kSlices; ++ks) tr[ks] = ld_slab(rec0 + c * Rec<DK>::kBytes, kRecT, mt, ks);
    };
    if (nch > 0) {
        issue(0);
        issue_t(0);
        store(0, 0);
    }
    __syncthreads();
    for (int64_t c = 0; c < nch; ++c) {
        SM &sm = *lds_opaque(reinterpret_cast<SM *>(smraw));
        const int cur = (int)(c & 1);
        const E *Kc = &sm.K[cur][0][0];
        const float *bc = sm.b[cur];
        H.save_t(hs + c * hstride, wave);
        // X = K H, R = diag(beta) (V - diag(gamma) X)
        {
            floatx4 x = zero4();
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks)
                x = mms<kX, false>(x, ldr<E>(Kc, SM::KP, 16 * mt, 32 * ks), sm_rows(sm.Ht, 16 * nt, 32 * ks));
            floatx4 rv;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * mt + 4 * g + r, j = 16 * nt + cc;
                rv[r] = sm.beta[cur][i] * ((float)sm.V[i][j] - __expf(bc[i]) * x[r]);
            }
            sm_put_t(sm.Rt, 16 * mt, 16 * nt, rv);
        }
        __syncthreads();
        issue(c + 1 < nch ? c + 1 : c);
        // U = T R (to the workspace), diag(w) U
        {
            floatx4 u = zero4();
#pragma unroll
            for (int ks = 0; ks < kSlices; ++ks)
                if (32 * ks <= 16 * mt + 15) u = mms<false, false>(u, slab_split(tr[ks]), sm_rows(sm.Rt, 16 * nt, 32 * ks));
            const float blast = bc[CB - 1];
            float *ubc = ub + c * CB * dvf;  // (a uniform base and a 32-bit lane offset)
            floatx4 wu;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * mt + 4 * g + r, j = 16 * nt + cc;
                ubc[(uint32_t)(i * (int)dvf + j)] = u[r];
                wu[r] = __expf(fminf(blast - bc[i], 0.f)) * u[r];
            }
            sm_put_t(sm.wUt, 16 * mt, 16 * nt, wu);
        }
        __syncthreads();
        // the next chunk's T slabs (T is done with once U is formed) queue while the update runs
        issue_t(c + 1 < nch ? c + 1 : c);
        // H' = gamma_last H + K^T diag(w) U, each wave on its own tiles
        {
            const float glast = __expf(bc[CB - 1]);
#pragma unroll
            for (int s = 0; s < StateTiles<DK>::N; ++s) {
                const int hm = StateTiles<DK>::hm(wave, s), hn = StateTiles<DK>::hn(wave, s);
                floatx4 h = glast * H.v[s];
#pragma unroll
                for (int ks = 0; ks < kSlices; ++ks)
                    h = mms<kX, false>(h, ldc<E>(Kc, SM::KP, 16 * hm, 32 * ks), sm_rows(sm.wUt, 16 * hn, 32 * ks));
                H.v[s] = h;
            }
            H.put(sm.Ht, wave);
        }
        if (c + 1 < nch) store(c + 1, cur ^ 1);
        __syncthreads();
    }
}

// Adjoint sweep of one (sequence, value head, column slice), from the last chunk: per chunk, the
// exit adjoint D to the workspace, dU = diag(w) K D + Pm^T dO, dR = T^T dU (to the workspace)
// and D <- gamma_last D + Q^T diag(e^r) dO - K^T diag(beta gamma) dR.
template <typename E, int DK>
__device__ __forceinline__ void adj_sweep(const BwdArgs &a, int64_t unit, int tile, char *smraw) {
    typedef AdjSmem<E, DK> SM;
    SM &sm = *reinterpret_cast<SM *>(smraw);
    constexpr bool kX = std::is_same<E, __bf16>::value;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, cc = lane & 15;
    const int64_t seq = unit / a.Hv, head = unit % a.Hv, kh = head / (a.Hv / a.Hk);
    const Loc L = locate_seq(a, seq);
    const int64_t nch = (L.sq.len + CB - 1) / CB;
    const int64_t dvf = a.ntiles * TV;
    const int col0 = tile * TV;
    const E *kb = reinterpret_cast<const E *>(a.k) + (L.row * a.Hk + kh) * a.T * DK;
    const E *qb = reinterpret_cast<const E *>(a.q) + (L.row * a.Hk + kh) * a.T * DK;
    const E *ob = reinterpret_cast<const E *>(a.dout) + (L.row * a.Hv + head) * a.T * dvf + col0;
    const float *beb = a.beta + (L.row * a.Hv + head) * a.T;
    float *drb = a.drs + (head * a.nslots + L.slot0) * CB * dvf + col0;
    constexpr int64_t kSlice = (int64_t)DK * TV;
    float *ds = a.ds + ((head * a.nslots + L.slot0) * a.ntiles + tile) * kSlice;
    const int64_t dstride = a.ntiles * kSlice;
    const uint8_t *rec0 = a.rec + (head * a.nslots + L.slot0) * Rec<DK>::kBytes;
    const int64_t sbase = (seq * a.Hv + head) * DK * dvf + col0;
    StateTiles<DK> D;
    D.load(a.dhT ? a.dhT + sbase : nullptr, dvf, wave);
    D.put(sm.Dt, wave);
    const int mt = wave >> 1, nt = wave & 1;
    Rows<E, DK, kThreads> kp, qp;
    Rows<E, TV, kThreads> op;
    float bv = 0.f, rv = 0.f, betav = 0.f;
    auto issue = [&](int64_t c) __attribute__((always_inline)) {
        const int n = (int)min((int64_t)CB, L.sq.len - c * CB);
        kp.issue(kb, DK, L.sq, c, n, tid);
        qp.issue(qb, DK, L.sq, c, n, tid);
        op.issue(ob, dvf, L.sq, c, n, tid);
        const int gr = tid & (CB - 1);
        const float *rb = reinterpret_cast<const float *>(rec0 + c * Rec<DK>::kBytes + Rec<DK>::kGates);
        bv = rb[gr];
        rv = rb[CB + gr];
        betav = (beb + L.sq.low(c, n))[(uint32_t)L.sq.off(gr < n ? gr : 0, n)];
    };
    // The store addresses are formed at each call from a thread index the compiler cannot
    // hoist (the lane from v_mbcnt in volatile asm) and a laundered LDS base. Kept across the
    // loop, they were spilled under the 128-register cap, and the reloads, which share the
    // vector-memory counter with global loads, each waited for the T^T and Pm^T slab loads
    // issued just before.
    auto store = [&](int64_t c) __attribute__((always_inline)) {
        const int n = (int)min((int64_t)CB, L.sq.len - c * CB);
        int t;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(t));
        t += wave << 6;
        SM &sl = *lds_opaque(reinterpret_cast<SM *>(smraw));
        kp.store(&sl.K[0][0], SM::KP, n, t);
        qp.store(&sl.Q[0][0], SM::KP, n, t);
        op.store(&sl.dO[0][0], SM::VP, n, t);
        if (t < CB) {
            sl.b[t] = bv;
            sl.er[t] = __expf(rv);
            sl.beta[t] = t < n ? betav : 0.f;
        }
    };
    // T^T and Pm^T (rows 16 mt .. 16 mt + 15 are zero before column 16 mt; the zero slabs are read
    // too), read during the previous chunk
    Slab tt[kSlices], pt[kSlices];
    constexpr int NDT = StateTiles<DK>::N;
    auto issue_f = [&](int64_t c) __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < kSlices; ++ks) {
            pt[ks] = ld_slab(rec0 + c * Rec<DK>::kBytes, kRecPt, mt, ks);
            tt[ks] = ld_slab(rec0 + c * Rec<DK>::kBytes, kRecTt, mt, ks);
        }
    };
    if (nch > 0) {
        issue(nch - 1);
        issue_f(nch - 1);
        store(nch - 1);
    }
    __syncthreads();
    for (int64_t c = nch - 1; c >= 0; --c) {
        SM &sm = *lds_opaque(reinterpret_cast<SM *>(smraw));
        const E *Kc = &sm.K[0][0];
        const E *Qc = &sm.Q[0][0];
        const E *Oc = &sm.dO[0][0];
        const float *bc = sm.b;
        D.save_t(ds + c * dstride, wave);
        // dU = diag(w) K D + Pm^T dO
        {
            floatx4 y = zero4(), p = zero4();
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks)
                y = mms<kX, false>(y, ldr<E>(Kc, SM::KP, 16 * mt, 32 * ks), sm_rows(sm.Dt, 16 * nt, 32 * ks));
#pragma unroll
            for (int ks = 0; ks < kSlices; ++ks)
                if (32 * ks + 31 >= 16 * mt) p = mms<false, kX>(p, slab_split(pt[ks]), ldc<E>(Oc, SM::VP, 16 * nt, 32 * ks));
            const float blast = bc[CB - 1];
            floatx4 du;
#pragma unroll
            for (int r = 0; r < 4; ++r) du[r] = __expf(fminf(blast - bc[16 * mt + 4 * g + r], 0.f)) * y[r] + p[r];
            sm_put_t(sm.dUt, 16 * mt, 16 * nt, du);
        }
        __syncthreads();
        issue(c > 0 ? c - 1 : 0);
        // dR = T^T dU (to the workspace), -diag(beta gamma) dR
        {
            floatx4 d = zero4();
#pragma unroll
            for (int ks = 0; ks < kSlices; ++ks)
                if (32 * ks + 31 >= 16 * mt) d = mms<false, false>(d, slab_split(tt[ks]), sm_rows(sm.dUt, 16 * nt, 32 * ks));
            float *drc = drb + c * CB * dvf;
            floatx4 br;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * mt + 4 * g + r, j = 16 * nt + cc;
                drc[(uint32_t)(i * (int)dvf + j)] = d[r];
                br[r] = -sm.beta[i] * __expf(bc[i]) * d[r];
            }
            sm_put_t(sm.bRt, 16 * mt, 16 * nt, br);
        }
        __syncthreads();
        // D <- gamma_last D + Q^T diag(e^r) dO + K^T bR, each wave on its own tiles
        {
            const float glast = __expf(bc[CB - 1]);
#pragma unroll
            for (int s = 0; s < NDT; ++s) {
                const int hm = StateTiles<DK>::hm(wave, s), hn = StateTiles<DK>::hn(wave, s);
                floatx4 h = glast * D.v[s];
#pragma unroll
                for (int ks = 0; ks < kSlices; ++ks) {
                    h = mms<false, kX>(h, cols_kscaled<E>(Qc, SM::KP, 16 * hm, 32 * ks, sm.er), ldc<E>(Oc, SM::VP, 16 * hn, 32 * ks));
                    h = mms<kX, false>(h, ldc<E>(Kc, SM::KP, 16 * hm, 32 * ks), sm_rows(sm.bRt, 16 * hn, 32 * ks));
                }
                D.v[s] = h;
            }
            D.put(sm.Dt, wave);
        }
        issue_f(c > 0 ? c - 1 : 0);
        __syncthreads();
        if (c > 0) store(c - 1);
        __syncthreads();
    }
    if (a.dh0) D.save(a.dh0 + sbase, dvf, wave);
}

// Both sweeps in one launch: workgroups [0, n) run the forward sweep, [n, 2n) the adjoint sweep
// (n = units x column slices), so that as the first n fill one slot of every compute unit the
// second n pair each forward workgroup with an adjoint one. Within each half the ids are spread
// so that the column slices of a unit run on the same XCD (workgroups go to the XCDs round
// robin) and share its L2.
template <typename E, int DK>
__device__ __forceinline__ void sweep_body(const BwdArgs &a) {
    __shared__ __attribute__((aligned(16))) char smraw[sweep_smem_bytes<E, DK>()];
    const int64_t n = a.units * a.ntiles;
    const bool adjoint = blockIdx.x >= n;
    int64_t w = adjoint ? blockIdx.x - n : blockIdx.x;
    if (n % 8 == 0) w = (w % 8) * (n / 8) + w / 8;
    if (adjoint) adj_sweep<E, DK>(a, w / a.ntiles, (int)(w % a.ntiles), smraw);
    else fwd_sweep<E, DK>(a, w / a.ntiles, (int)(w % a.ntiles), smraw);
}
template <typename E, int DK>
__global__ __launch_bounds__(kThreads) void bwd_sweep_kernel(BwdArgs a) {
    sweep_body<E, DK>(a);
}
// bf16: at most 128 registers, so that two workgroups (8 waves each) fit on a compute unit
template <int DK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void bwd_sweep_kernel_bf16(BwdArgs a) {
    sweep_body<__bf16, DK>(a);
}

// ---------------------------------------------------------------- 3. gradients

template <typename E, int DK>
struct GradSmem {
    // (ordered so that the arrays indexed in many different ways lie in the first 64 KiB, within
    // reach of the LDS instructions' immediate offsets)
    static constexpr int KP = DK + pad_of<E>(), VP = TV + pad_of<E>(), HP = DK + 4;
    // Per-row partial sums, one slot per contributing tile, added in a fixed order:
    //   sx, sb, sw: dR . X, dR . (V - gamma X) and (K D) . U over the two 16-column halves
    //   pr, ar, gr: row sums of dP Pm, dA A and dA G per column tile; pc, ac: their column sums
    //   (negated) per row tile; rq: e^r (dO H^T) . q per 16-column tile of d_k
    float sx[2][CB], sb[2][CB], sw[2][CB];
    float pr[NMT][CB], pc[NMT][CB], ar[NMT][CB], ac[NMT][CB], gr[NMT][CB];
    float rq[DK / 16][CB];
    float hd[kWaves];
    float b[CB], r[CB], beta[CB];
    // a column slice of U and dR (token-major) and, with bf16 inputs, of diag(w) U and
    // -diag(beta gamma) dR, the A operands of the dK terms (with fp32 inputs they are scaled at
    // each read, to stay within the LDS)
    static constexpr bool kPre = sizeof(E) == 2;
    SplitMat<CB, TV> U, dR;
    SplitMat<kPre ? CB : 1, kPre ? TV : 8> wU, bR;
    union {
        struct {
            // a column slice of the entry state and the exit adjoint, transposed
            SplitMat<TV, DK> Ht, Dt;
        } t;
        struct {
            // M and diag(beta) N, transposed and split, once every slice is done
            SplitMat<CB, CB> Mt, Nt;
        } m;
    } u;
    E dO[CB][VP], V[CB][VP];
    E K[CB][KP], Q[CB][KP];
};

template <typename E, int DK>
__global__ __launch_bounds__(kThreads) void bwd_grad_kernel(BwdArgs a) {
    typedef GradSmem<E, DK> SM;
    __shared__ SM smem;
    SM &sm = smem;
    constexpr bool kX = std::is_same<E, __bf16>::value;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, cc = lane & 15;
    const int64_t kh = blockIdx.x / a.nslots, slot = blockIdx.x % a.nslots;
    Loc L;
    int64_t c;
    if (!locate_slot(a, slot, L, c)) return;
    const int n = (int)min((int64_t)CB, L.sq.len - c * CB);
    const bool pre = (a.flags & kFlagReadPre) != 0;
    const int64_t grp = a.Hv / a.Hk, dvf = a.ntiles * TV;
    const int64_t nit = grp * a.ntiles;
    constexpr int64_t kSlice = (int64_t)DK * TV;
    const E *qb = reinterpret_cast<const E *>(a.q) + (L.row * a.Hk + kh) * a.T * DK;
    const E *kb = reinterpret_cast<const E *>(a.k) + (L.row * a.Hk + kh) * a.T * DK;
    {
        Rows<E, DK, kThreads> kp, qp;
        kp.issue(kb, DK, L.sq, c, n, tid);
        qp.issue(qb, DK, L.sq, c, n, tid);
        kp.store(&sm.K[0][0], SM::KP, n, tid);
        qp.store(&sm.Q[0][0], SM::KP, n, tid);
    }
    // staged inputs of one (value head, column slice) step
    // this thread's part of a transposed TV x DK state slice: NF4 runs of 4 floats of one row
    constexpr int NF4 = DK * TV / (kThreads * 4), TPR = DK / (4 * NF4);
    const int tcol = tid / TPR, td0 = (tid % TPR) * 4 * NF4;
    float4 hpre[NF4], dpre[NF4], upre, rpre;
    Rows<E, TV, kThreads> op, vp;
    float gb = 0.f, gr_ = 0.f, gbeta = 0.f;
    const int ur = tid / (TV / 4), uc = (tid % (TV / 4)) * 4;  // the thread's 4 elements of U and dR
    static_assert(CB * TV / 4 == kThreads, "one 16-byte piece of U and of dR per thread");
    auto issue = [&](int64_t it) __attribute__((always_inline)) {
        const int64_t head = kh * grp + it / a.ntiles;
        const int tile = (int)(it % a.ntiles);
        const int64_t sidx = ((head * a.nslots + slot) * a.ntiles + tile) * kSlice;
        const float *hsb = a.hs + sidx, *dsb = a.ds + sidx;
#pragma unroll
        for (int u = 0; u < NF4; ++u) {
            const uint32_t o = (uint32_t)(tcol * DK + td0 + 4 * u);
            hpre[u] = *reinterpret_cast<const float4 *>(hsb + o);
            dpre[u] = *reinterpret_cast<const float4 *>(dsb + o);
        }
        const int64_t vbase = (L.row * a.Hv + head) * a.T * dvf + tile * TV;
        const int64_t cbase = (head * a.nslots + slot) * CB * dvf + tile * TV;
        const uint32_t uo = (uint32_t)(ur * (int)dvf + uc);
        upre = *reinterpret_cast<const float4 *>(a.us + cbase + uo);
        rpre = *reinterpret_cast<const float4 *>(a.drs + cbase + uo);
        op.issue(reinterpret_cast<const E *>(a.dout) + vbase, dvf, L.sq, c, n, tid);
        vp.issue(reinterpret_cast<const E *>(a.v) + vbase, dvf, L.sq, c, n, tid);
        const int gi = tid & (CB - 1);
        const float *rb = reinterpret_cast<const float *>(a.rec + (head * a.nslots + slot) * Rec<DK>::kBytes + Rec<DK>::kGates);
        gb = rb[gi];
        gr_ = rb[CB + gi];
        gbeta = (a.beta + (L.row * a.Hv + head) * a.T + L.sq.low(c, n))[(uint32_t)L.sq.off(gi < n ? gi : 0, n)];
    };

    // tile assignments: X and K D: tile (xm, xn) of the CB x TV slice; dP, dA: lower tiles
    // wave, wave + 8, wave + 16 of the twenty; dQ, dK: d_k tile qn, row tiles qm(s)
    const int xm = wave >> 1, xn = wave & 1;
    constexpr int NQ = DK / 16, NQT = NMT * NQ / kWaves;
    const int qn = wave % NQ;
    auto qm = [&](int s) __attribute__((always_inline)) -> int { return wave / NQ + s * (kWaves / NQ); };
    floatx4 dQ[NQT], dK[NQT], dQH[NQT], pa[3];
#pragma unroll
    for (int s = 0; s < NQT; ++s) {
        dQ[s] = zero4();
        dK[s] = zero4();
    }
    float ax[4], bx[4], wy[4], hsum = 0.f;

    if (nit > 0) issue(0);
    for (int64_t it = 0; it < nit; ++it) {
        SM &sm = *lds_opaque(&smem);
        const int64_t v = it / a.ntiles;
        const int tile = (int)(it % a.ntiles);
        __syncthreads();
        if (tile == 0) hsum = 0.f;
#pragma unroll
        for (int u = 0; u < NF4; ++u) {
            const float4 h = hpre[u], d = dpre[u];
            sm_put4(sm.u.t.Ht, tcol, td0 + 4 * u, h);
            sm_put4(sm.u.t.Dt, tcol, td0 + 4 * u, d);
            hsum += h.x * d.x + h.y * d.y + h.z * d.z + h.w * d.w;
        }
        // (rows past the chunk end hold zeros in U and dR); lane l of every wave holds the gates
        // of row l of this step's value head
        sm_put4(sm.U, ur, uc, upre);
        sm_put4(sm.dR, ur, uc, rpre);
        const float be = __shfl(gbeta, ur, 64);
        if constexpr (SM::kPre) {
            const float bu = __shfl(gb, ur, 64), bl = __shfl(gb, CB - 1, 64);
            const float wr = __expf(fminf(bl - bu, 0.f)), br = -be * __expf(bu);
            sm_put4(sm.wU, ur, uc, make_float4(wr * upre.x, wr * upre.y, wr * upre.z, wr * upre.w));
            sm_put4(sm.bR, ur, uc, make_float4(br * rpre.x, br * rpre.y, br * rpre.z, br * rpre.w));
        }
        // dV = diag(beta) dR
        if (ur < n) {
            const int64_t head = kh * grp + v;
            *reinterpret_cast<float4 *>(a.dv + ((L.row * a.Hv + head) * a.T + L.sq.token(c * CB + ur)) * dvf + tile * TV + uc) =
                make_float4(be * rpre.x, be * rpre.y, be * rpre.z, be * rpre.w);
        }
        op.store(&sm.dO[0][0], SM::VP, n, tid);
        vp.store(&sm.V[0][0], SM::VP, n, tid);
        if (tile == 0) {
            if (tid < CB) {
                sm.b[tid] = gb;
                sm.r[tid] = gr_;
                sm.beta[tid] = tid < n ? gbeta : 0.f;
            }
#pragma unroll
            for (int s = 0; s < NQT; ++s) dQH[s] = zero4();
#pragma unroll
            for (int s = 0; s < 3; ++s) pa[s] = zero4();
#pragma unroll
            for (int r = 0; r < 4; ++r) ax[r] = bx[r] = wy[r] = 0.f;
        }
        __syncthreads();
        const float blast = sm.b[CB - 1];
        // X = K H and Y = K D on this wave's tile: dR . X, dR . (V - gamma X), Y . U per row
        {
            floatx4 x = zero4(), y = zero4();
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks) {
                const Split ka = ldr<E>(&sm.K[0][0], SM::KP, 16 * xm, 32 * ks);
                x = mms<kX, false>(x, ka, sm_rows(sm.u.t.Ht, 16 * xn, 32 * ks));
                y = mms<kX, false>(y, ka, sm_rows(sm.u.t.Dt, 16 * xn, 32 * ks));
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * xm + 4 * g + r, j = 16 * xn + cc;
                const float dr = sm_get(sm.dR, i, j);
                ax[r] += dr * x[r];
                bx[r] += dr * ((float)sm.V[i][j] - __expf(sm.b[i]) * x[r]);
                wy[r] += y[r] * sm_get(sm.U, i, j);
            }
        }
        // The next slice of this value head is read during this one's products (the first slice
        // of the next value head after this one's gate gradients). Its loads are issued here,
        // after the first products, not before the barrier: the ~56 KB of every wave's loads
        // queue in the vector memory path for 1-2k cycles, which before the barrier every wave
        // waited out.
        if (tile + 1 < a.ntiles) issue(it + 1);
        fence_sched();
        // dP = dO U^T and -dA = dR U^T on the lower tiles
#pragma unroll
        for (int s = 0; s < 3; ++s) {
            const int task = wave + kWaves * s;
            if (task < 20) {
                int pm, pn;
                lower_tile(task % 10, pm, pn);
                const Split ub = sm_rows(sm.U, 16 * pn, 0);
                if (task >= 10) pa[s] = mms<false, false>(pa[s], sm_rows(sm.dR, 16 * pm, 0), ub);
                else pa[s] = mms<kX, false>(pa[s], ldr<E>(&sm.dO[0][0], SM::VP, 16 * pm, 0), ub);
            }
        }
        fence_sched();
        // dO H^T, and diag(w) U dH'^T - diag(beta gamma) dR H^T into dK
        {
            const Split hB = sm_cols(sm.u.t.Ht, 16 * qn, 0);
            const Split dB = sm_cols(sm.u.t.Dt, 16 * qn, 0);
#pragma unroll
            for (int s = 0; s < NQT; ++s) {
                const int m = qm(s);
                dQH[s] = mms<kX, false>(dQH[s], ldr<E>(&sm.dO[0][0], SM::VP, 16 * m, 0), hB);
                if constexpr (SM::kPre) {
                    dK[s] = mms<false, false>(dK[s], sm_rows(sm.wU, 16 * m, 0), dB);
                    dK[s] = mms<false, false>(dK[s], sm_rows(sm.bR, 16 * m, 0), hB);
                } else {
                    const int row = 16 * m + cc;
                    const float wr = __expf(fminf(blast - sm.b[row], 0.f));
                    const float br = -sm.beta[row] * __expf(sm.b[row]);
                    dK[s] = mms<false, false>(dK[s], sm_scaled_rows(sm.U, 16 * m, wr), dB);
                    dK[s] = mms<false, false>(dK[s], sm_scaled_rows(sm.dR, 16 * m, br), hB);
                }
                fence_sched();
            }
        }
        if (tile + 1 < a.ntiles) continue;

        // ---- every slice of value head v is in: M, N, the rest of dQ and dK, the gates
        __syncthreads();
        {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * xm + 4 * g + r;
                const float s1 = row16(ax[r]), s2 = row16(bx[r]), s3 = row16(wy[r]);
                if (cc == 0) {
                    sm.sx[xn][i] = s1;
                    sm.sb[xn][i] = s2;
                    sm.sw[xn][i] = s3;
                }
            }
            float h = hsum;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) h += __shfl_xor(h, off, 64);
            if (lane == 0) sm.hd[wave] = h;
            // dQ += diag(e^r) dO H^T, and the read's exponent gradient e^r (dO H^T) . q
#pragma unroll
            for (int s = 0; s < NQT; ++s) {
                const int m = qm(s);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * m + 4 * g + r;
                    const float qh = __expf(sm.r[i]) * dQH[s][r];
                    const float rqv = row16(qh * (float)sm.Q[i][16 * qn + cc]);
                    if (cc == 0) sm.rq[qn][i] = rqv;
                    dQ[s][r] += qh;
                }
            }
        }
        fence_sched();
#pragma unroll
        for (int s = 0; s < 3; ++s) {
            const int task = wave + kWaves * s;
            if (task >= 20) continue;
            const bool isa = task >= 10;
            int pm, pn;
            lower_tile(task % 10, pm, pn);
            // the tile of G (isa) or Pm, again
            floatx4 gv = zero4();
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks)
                gv = mms<kX, kX>(gv, ldr<E>(isa ? &sm.K[0][0] : &sm.Q[0][0], SM::KP, 16 * pm, 32 * ks),
                                 ldr<E>(&sm.K[0][0], SM::KP, 16 * pn, 32 * ks));
            float csum = 0.f;
            floatx4 mv;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * pm + 4 * g + r, j = 16 * pn + cc;
                float rs, rb = 0.f;
                if (!isa) {
                    const bool keep = pre ? j < i : j <= i;
                    const float e = __expf(fminf(sm.r[i] - sm.b[j], 0.f));
                    const float dp = pa[s][r];
                    mv[r] = keep ? dp * e : 0.f;
                    rs = keep ? dp * gv[r] * e : 0.f;  // dP_ij Pm_ij
                } else {
                    const bool keep = j < i;
                    const float e = __expf(fminf(sm.b[i] - sm.b[j], 0.f));
                    const float da = -pa[s][r], gij = keep ? gv[r] * e : 0.f;
                    mv[r] = keep ? sm.beta[i] * da * e : 0.f;
                    rs = da * sm.beta[i] * gij;  // dA_ij A_ij
                    rb = da * gij;               // dA_ij G_ij
                }
                csum += rs;
                const float rsum = row16(rs);
                if (isa) {
                    const float bsum = row16(rb);
                    if (cc == 0) {
                        sm.ar[pn][i] = rsum;
                        sm.gr[pn][i] = bsum;
                    }
                } else if (cc == 0) {
                    sm.pr[pn][i] = rsum;
                }
            }
            // the tile of M (or N), and the zero tile mirrored above the diagonal
            SplitMat<CB, CB> &Xt = isa ? sm.u.m.Nt : sm.u.m.Mt;
            sm_put_t(Xt, 16 * pm, 16 * pn, mv);
            if (pm > pn) sm_put_t(Xt, 16 * pn, 16 * pm, zero4());
            // column sums over the tile's 16 rows enter d b_j with a minus sign
            csum = col4(csum);
            if (g == 0) {
                if (isa) sm.ac[pm][16 * pn + cc] = -csum;
                else sm.pc[pm][16 * pn + cc] = -csum;
            }
            fence_sched();
        }
        __syncthreads();
        // dQ += M K;  dK += M^T Q + N K + N^T K (N holds diag(beta) N)
#pragma unroll
        for (int s = 0; s < NQT; ++s) {
            const int m = qm(s);
#pragma unroll
            for (int ks = 0; ks < kSlices; ++ks) {
                const Split kB = ldc<E>(&sm.K[0][0], SM::KP, 16 * qn, 32 * ks);
                if (32 * ks <= 16 * m + 15) {  // rows of M and N: zero past column 16 m + 15
                    dQ[s] = mms<false, kX>(dQ[s], sm_cols(sm.u.m.Mt, 16 * m, 32 * ks), kB);
                    dK[s] = mms<false, kX>(dK[s], sm_cols(sm.u.m.Nt, 16 * m, 32 * ks), kB);
                }
                if (32 * ks + 31 >= 16 * m) {  // columns of M and N: zero above row 16 m
                    dK[s] = mms<false, kX>(dK[s], sm_rows(sm.u.m.Mt, 16 * m, 32 * ks), ldc<E>(&sm.Q[0][0], SM::KP, 16 * qn, 32 * ks));
                    dK[s] = mms<false, kX>(dK[s], sm_rows(sm.u.m.Nt, 16 * m, 32 * ks), kB);
                }
                fence_sched();
            }
        }
        __syncthreads();
        // gate gradients of value head v: per-row sums, then suffix sums through the cumsum
        if (wave == 0) {
            const int i = lane, mi = i / 16;
            const float wi = __expf(fminf(blast - sm.b[i], 0.f)), gi = __expf(sm.b[i]);
            const float dwi = sm.sw[0][i] + sm.sw[1][i];
            float db = 0.f, dr = 0.f, dbeta = sm.sb[0][i] + sm.sb[1][i];
            for (int t = 0; t <= mi; ++t) {
                db += sm.ar[t][i];
                dr += sm.pr[t][i];
                dbeta += sm.gr[t][i];
            }
            for (int t = mi; t < NMT; ++t) db += sm.pc[t][i] + sm.ac[t][i];
#pragma unroll
            for (int t = 0; t < DK / 16; ++t) dr += sm.rq[t][i];
            db -= sm.beta[i] * gi * (sm.sx[0][i] + sm.sx[1][i]);
            db -= wi * dwi;
            // the last row also takes gamma_last <D, H> + sum_j w_j (K D)_j . U_j
            float s = wi * dwi;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
            if (i == CB - 1) {
                float hd = 0.f;
#pragma unroll
                for (int w = 0; w < kWaves; ++w) hd += sm.hd[w];
                db += __expf(blast) * hd + s;
            }
            // post: the read exponent is b itself; pre: b - log alpha leaves out row i's own
            // log alpha, so its gradient enters the sums of the rows after it only
            float x = db + (pre ? 0.f : dr), z = pre ? dr : 0.f;
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
                const int64_t head = kh * grp + v;
                const int64_t t = (L.row * a.Hv + head) * a.T + L.sq.token(c * CB + i);
                a.dlog_alpha[t] = x + z - zi;
                a.dbeta[t] = dbeta;
            }
        }
        if (it + 1 < nit) issue(it + 1);
    }
    // dq, dk of the key head: the sum over its value heads, in order
    const int64_t qbase = (L.row * a.Hk + kh) * a.T * DK;
#pragma unroll
    for (int s = 0; s < NQT; ++s) {
        const int m = qm(s);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * m + 4 * g + r;
            if (i < n) {
                const int64_t o = qbase + L.sq.token(c * CB + i) * DK + 16 * qn + cc;
                a.dq[o] = dQ[s][r];
                a.dk[o] = dK[s][r];
            }
        }
    }
}

template <typename E, int DK>
hipError_t launch_t(const BwdArgs &a, hipStream_t s) {
    const int64_t np = a.Hv * a.nslots, nsw = 2 * a.units * a.ntiles, ng = a.Hk * a.nslots;
    if (np > 0) {
        if constexpr (std::is_same<E, __bf16>::value)
            hipLaunchKernelGGL((bwd_prep_kernel_bf16<DK>), dim3((unsigned)np), dim3(kPrepThreads), 0, s, a);
        else
            hipLaunchKernelGGL((bwd_prep_kernel<E, DK>), dim3((unsigned)np), dim3(kPrepThreads), 0, s, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (nsw > 0) {
        if constexpr (std::is_same<E, __bf16>::value)
            hipLaunchKernelGGL((bwd_sweep_kernel_bf16<DK>), dim3((unsigned)nsw), dim3(kThreads), 0, s, a);
        else
            hipLaunchKernelGGL((bwd_sweep_kernel<E, DK>), dim3((unsigned)nsw), dim3(kThreads), 0, s, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (ng > 0) {
        hipLaunchKernelGGL((bwd_grad_kernel<E, DK>), dim3((unsigned)ng), dim3(kThreads), 0, s, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_bwd(const BwdArgs &a, int dtype, int dk, int dv, hipStream_t stream) {
    (void)dv;
    if (dtype == kDtypeBf16) return dk == 64 ? launch_t<__bf16, 64>(a, stream) : launch_t<__bf16, 128>(a, stream);
    return dk == 64 ? launch_t<float, 64>(a, stream) : launch_t<float, 128>(a, stream);
}

}  // namespace gdr
