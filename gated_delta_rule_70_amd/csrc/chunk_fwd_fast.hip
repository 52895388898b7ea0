// Fast chunked forward for the common shape: bf16 q/k/v, chunk 64, d_k = 128, fp32 state.
//
// Same chunk algebra as chunk_fwd.hip (the WY/UT form of `chunked_delta` on the "Prizma
// seq/delta.py" page, with H = S^T), organised for the matrix cores of gfx950:
//
//   A   = strict_lower(beta_i (k_i . k_j) e^{b_i - b_j})        T_ii = (I + A_ii)^{-1}
//   R   = diag(beta) (V - diag(e^{b}) K H)
//   U   by block forward substitution over the four 16-row blocks:
//         U_i = T_ii (R_i - sum_{j<i} A_ij U_j)                 (U = (I + A)^{-1} R exactly)
//   O   = diag(e^{b} | e^{b'}) Q H + P U,   P = [(q_i . k_j) e^{b_i - b_j}]_{j<=i} (post)
//                                              [(q_i . k_j) e^{b'_i - b_j}]_{j<i}  (pre)
//   H  <- e^{b_C} H + K^T diag(e^{b_C - b}) U
//
// One workgroup = 4 waves per (sequence, value head, 32 columns of d_v), walking the chunks:
//   waves 0, 1  "chain": the state-dependent part for chunk c, one 16-column tile each. The
//               state tile stays in accumulator registers and is the B operand of K H and
//               Q H directly; every other operand is one 16-byte LDS read.
//   wave 2      "diagonal prep" for chunk c+1: diagonal tiles of K K^T and Q K^T, the four
//               16x16 inverses T_ii by forward substitution (one lane per column), the gate
//               scalars, and K in the operand layout of K H.
//   wave 3      "off-diagonal prep" for chunk c+1: off-diagonal tiles of K K^T (-> -A_ij)
//               and Q K^T (-> P), Q in operand layout, K^T in operand layout, V transposed.
// The prep waves load q/k/gates straight from global memory into operand registers; what
// the chain needs is written into one of two LDS buffers, so a single barrier per chunk
// separates producer and consumer.
//
// Operand convention (see gdr_mfma.hpp): a 32-deep fragment gives lane (g, c) the k-values
// {4g..4g+3} ("lo") and {16+4g..16+4g+3} ("hi"); LDS fragment buffers store the 64 lanes'
// 16 bytes contiguously ("fragment-native"), so every chain read is conflict-free.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "gdr_kernels.hpp"
#include "gdr_mfma.hpp"

namespace gdr {

namespace {

constexpr int kC = 64, kDK = 128, kDVT = 32;
constexpr int kVtPitch = kC + 4;  // bf16 elements per transposed V row (padding against conflicts)

// byte offsets inside one of the two chunk buffers
constexpr int kOffKf = 0;                          // 16 frags (i, ks) x 64 lanes x 16 B
constexpr int kOffQf = kOffKf + 16 * 1024;         // same for Q
constexpr int kOffKtf = kOffQf + 16 * 1024;        // 16 frags (t, kp): K^T as A operand
constexpr int kOffPf = kOffKtf + 16 * 1024;        // 6 frags: P row tiles x 32-deep k slices
constexpr int kOffNA = kOffPf + 6 * 1024;          // -A: A10 (lo, 512 B), A2x (1 KB), A3x (1 KB), A32 (lo)
constexpr int kOffTd = kOffNA + 3 * 1024;          // T_ii, 4 lo-only frags of 512 B
constexpr int kOffVt = kOffTd + 2 * 1024;          // V^T [32][kVtPitch] bf16
constexpr int kOffSc = kOffVt + kDVT * kVtPitch * 2;  // scalars: beta, e^b, read scale, e^{bC-b} [64] each, e^{bC}
constexpr int kBufBytes = kOffSc + 4 * 256 + 16;
// private areas
constexpr int kOffAd = 2 * kBufBytes;              // wave 2: A_ii^T blocks, fp32 [4][16][16]
constexpr int kOffG2 = kOffAd + 4 * 1024;          // wave 2: b, beta, la [64] fp32
constexpr int kOffG3 = kOffG2 + 3 * 256;           // wave 3: b, beta, la [64] fp32
constexpr int kOffStage = kOffG3 + 3 * 256;        // chain: output staging, 2 x [64][16] bf16
constexpr int kSmemBytes = kOffStage + 2 * 2048;
static_assert(kSmemBytes <= 160 * 1024, "LDS budget");

// index of the P fragment for row tile mi and 32-deep k slice kp (kp <= mi / 2)
__device__ __forceinline__ int pf_index(int mi, int kp) { return mi < 2 ? mi : 2 + 2 * (mi - 2) + kp; }

struct SeqView {
    int64_t t0, len;
    bool rev;
    __device__ __forceinline__ int64_t token(int64_t pos) const { return rev ? t0 + len - 1 - pos : t0 + pos; }
};

struct PrepRegs {
    uint4 k[4][4];  // K row fragments (tile row i, 32-deep slice ks)
    uint4 q[4][4];  // Q row fragments
    float la, beta; // lane i: token i of the chunk
};

// Row fragments straight from global memory: lane (g, c) gets row 16i + c, columns
// 32ks + 4g..+3 and 32ks + 16 + 4g..+3. Rows past the end of the sequence are zero.
__device__ __forceinline__ void load_prep(PrepRegs &p, const SeqView &sv, int64_t chunk, const __bf16 *kb,
                                          const __bf16 *qb, const float *ab, const float *bb, bool want_q) {
    const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t pos = chunk * kC + 16 * i + c;
        const bool ok = pos < sv.len;
        const int64_t tok = ok ? sv.token(pos) : 0;
        const uint2 *kr = reinterpret_cast<const uint2 *>(kb + tok * kDK + 4 * g);
        const uint2 *qr = reinterpret_cast<const uint2 *>(qb + tok * kDK + 4 * g);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            uint2 lo = make_uint2(0, 0), hi = lo, qlo = lo, qhi = lo;
            if (ok) {
                lo = kr[ks * 8];       // +32 elements = 8 uint2
                hi = kr[ks * 8 + 4];   // +16 elements
                if (want_q) {
                    qlo = qr[ks * 8];
                    qhi = qr[ks * 8 + 4];
                }
            }
            p.k[i][ks] = make_uint4(lo.x, lo.y, hi.x, hi.y);
            p.q[i][ks] = make_uint4(qlo.x, qlo.y, qhi.x, qhi.y);
        }
    }
    const int64_t pos = chunk * kC + lane;
    p.la = 0.f;
    p.beta = 0.f;
    if (pos < sv.len) {
        const int64_t t = sv.token(pos);
        p.la = ab[t];
        p.beta = bb[t];
    }
}

__device__ __forceinline__ Frag<__bf16> as_frag(uint4 u) {
    Frag<__bf16> f;
    f.lo = __builtin_bit_cast(bf16x4, make_uint2(u.x, u.y));
    f.hi = __builtin_bit_cast(bf16x4, make_uint2(u.z, u.w));
    return f;
}

__device__ __forceinline__ Frag<__bf16> lds_frag(const char *base, int idx) {
    const int lane = threadIdx.x & 63;
    return as_frag(*reinterpret_cast<const uint4 *>(base + (idx * 64 + lane) * 16));
}
__device__ __forceinline__ bf16x4 lds_frag_lo(const char *base, int idx) {
    const int lane = threadIdx.x & 63;
    return *reinterpret_cast<const bf16x4 *>(base + (idx * 64 + lane) * 8);
}

// Inclusive prefix sum over the 64 lanes (token order of the chunk).
__device__ __forceinline__ float wave_cumsum(float x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    return x;
}

// Gate values of the chunk into a private LDS area: b (cumsum), beta, la.
__device__ __forceinline__ void stage_gates(char *smem, int off, const PrepRegs &p, float &b_lane) {
    const int lane = threadIdx.x & 63;
    b_lane = wave_cumsum(p.la);
    float *gb = reinterpret_cast<float *>(smem + off);
    gb[lane] = b_lane;
    gb[64 + lane] = p.beta;
    gb[128 + lane] = p.la;
    wave_lds_sync();
}

// 16x16 Gram tile from register fragments: acc = X_i Y_j^T over d_k = 128.
__device__ __forceinline__ floatx4 gram(const uint4 (&x)[4], const uint4 (&y)[4]) {
    floatx4 acc = zero4();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) acc = mma32(acc, as_frag(x[ks]), as_frag(y[ks]));
    return acc;
}

// Location of element (row rr within a 16-row tile, k' within a 32-deep slice) in a
// fragment-native bf16 buffer: returns the element index relative to the fragment base.
__device__ __forceinline__ int frag32_elem(int rr, int kk) {
    const int gg = (kk & 15) >> 2, s = (kk & 3) + 4 * (kk >> 4);
    return ((gg << 4) | rr) * 8 + s;
}
__device__ __forceinline__ int frag16_elem(int rr, int kk) {
    return (((kk >> 2) << 4) | rr) * 4 + (kk & 3);
}

// ------------------------------------------------------------------ wave 2: diagonal prep
__device__ __forceinline__ void prep_diag(char *smem, char *buf, const PrepRegs &p, bool pre) {
    const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
    float b_lane;
    stage_gates(smem, kOffG2, p, b_lane);
    const float *gb = reinterpret_cast<const float *>(smem + kOffG2);

    // gate scalars for the chain
    {
        float *sc = reinterpret_cast<float *>(buf + kOffSc);
        const float bC = __shfl(b_lane, 63, 64);
        sc[lane] = p.beta;
        sc[64 + lane] = __expf(b_lane);
        sc[128 + lane] = __expf(pre ? b_lane - p.la : b_lane);
        sc[192 + lane] = __expf(fminf(bC - b_lane, 0.f));
        if (lane == 0) sc[256] = __expf(bC);
    }
    // K in the operand layout of K H
    {
        uint4 *kf = reinterpret_cast<uint4 *>(buf + kOffKf);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) kf[(i * 4 + ks) * 64 + lane] = p.k[i][ks];
    }
    // diagonal tiles of K K^T and Q K^T
    floatx4 gk[4], gq[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        gk[i] = gram(p.k[i], p.k[i]);
        gq[i] = gram(p.q[i], p.k[i]);
    }
    float *adt = reinterpret_cast<float *>(smem + kOffAd);
    __bf16 *pf = reinterpret_cast<__bf16 *>(buf + kOffPf);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int col = 16 * i + c;
        const float bcol = gb[col];
        const floatx4 brow = *reinterpret_cast<const floatx4 *>(gb + 16 * i + 4 * g);
        const floatx4 betar = *reinterpret_cast<const floatx4 *>(gb + 64 + 16 * i + 4 * g);
        const floatx4 lar = *reinterpret_cast<const floatx4 *>(gb + 128 + 16 * i + 4 * g);
        floatx4 a;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rr = 4 * g + r;
            a[r] = (c < rr) ? betar[r] * gk[i][r] * __expf(fminf(brow[r] - bcol, 0.f)) : 0.f;
            const float bread = pre ? brow[r] - lar[r] : brow[r];
            const bool keep = pre ? (c < rr) : (c <= rr);
            const float pv = keep ? gq[i][r] * __expf(fminf(bread - bcol, 0.f)) : 0.f;
            pf[pf_index(i, i >> 1) * 512 + frag32_elem(rr, 16 * (i & 1) + c)] = (__bf16)pv;
        }
        // A_ii^T: column c of A_ii holds rows 4g..4g+3 here
        *reinterpret_cast<floatx4 *>(adt + (i * 16 + c) * 16 + 4 * g) = a;
    }
    wave_lds_sync();
    // T_ii = (I + A_ii)^{-1}: lane (i = g, c) computes column c, eliminating column j of A
    // into every later row as soon as t_j is known
    float acc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = (r == c) ? 1.f : 0.f;
    const float *ablk = adt + g * 256;
#pragma unroll
    for (int j = 0; j < 15; ++j) {
        const float tj = acc[j];
        const floatx4 *colj = reinterpret_cast<const floatx4 *>(ablk + j * 16);
#pragma unroll
        for (int q4 = (j + 1) >> 2; q4 < 4; ++q4) {
            const floatx4 v = colj[q4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * q4 + e;
                if (r > j) acc[r] -= v[e] * tj;
            }
        }
    }
    __bf16 *td = reinterpret_cast<__bf16 *>(buf + kOffTd) + g * 256;
#pragma unroll
    for (int r = 0; r < 16; ++r) td[frag16_elem(r, c)] = (__bf16)acc[r];
}

// ------------------------------------------------------------------ wave 3: off-diagonal prep
__device__ __forceinline__ void prep_off(char *smem, char *buf, const PrepRegs &p, bool pre,
                                         const SeqView &sv, int64_t chunk, const __bf16 *vb, int64_t dv,
                                         int dcol0) {
    const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
    // V tile of the chunk, transposed: lane = row
    uint4 vrow[4];
    {
        const int64_t pos = chunk * kC + lane;
        const bool ok = pos < sv.len;
        const uint4 *src = reinterpret_cast<const uint4 *>(vb + (ok ? sv.token(pos) : 0) * dv + dcol0);
#pragma unroll
        for (int x = 0; x < 4; ++x) vrow[x] = ok ? src[x] : make_uint4(0, 0, 0, 0);
    }
    float b_lane;
    stage_gates(smem, kOffG3, p, b_lane);
    const float *gb = reinterpret_cast<const float *>(smem + kOffG3);

    // Q in the operand layout of Q H
    {
        uint4 *qf = reinterpret_cast<uint4 *>(buf + kOffQf);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) qf[(i * 4 + ks) * 64 + lane] = p.q[i][ks];
    }
    // off-diagonal tiles (i > j) of K K^T and Q K^T
    floatx4 gk[6], gq[6];
    {
        int n = 0;
#pragma unroll
        for (int i = 1; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < i; ++j, ++n) {
                gk[n] = gram(p.k[i], p.k[j]);
                gq[n] = gram(p.q[i], p.k[j]);
            }
    }
    // K^T in the operand layout of K^T W: element K[tok][d] goes to fragment (t = d/16,
    // kp = tok/32), lane ((tok%32 % 16)/4, d%16), slot (tok%4) + 4*((tok%32)/16)
    {
        __bf16 *ktf = reinterpret_cast<__bf16 *>(buf + kOffKtf);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const uint4 u = p.k[i][ks];
                const bf16x8 v = __builtin_bit_cast(bf16x8, u);
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const int t = 2 * ks + (s >> 2);
                    const int cc = 4 * g + (s & 3);
                    const int kp = i >> 1;
                    const int gg = c >> 2, ss = (c & 3) + 4 * (i & 1);
                    ktf[((t * 2 + kp) * 64 + ((gg << 4) | cc)) * 8 + ss] = v[s];
                }
            }
    }
    // V^T
    {
        __bf16 *vt = reinterpret_cast<__bf16 *>(buf + kOffVt);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const bf16x8 v = __builtin_bit_cast(bf16x8, vrow[x]);
#pragma unroll
            for (int e = 0; e < 8; ++e) vt[(8 * x + e) * kVtPitch + lane] = v[e];
        }
    }
    // epilogues: -A_ij (j < i) for the block substitution, P_ij
    __bf16 *na = reinterpret_cast<__bf16 *>(buf + kOffNA);
    __bf16 *pf = reinterpret_cast<__bf16 *>(buf + kOffPf);
    {
        int n = 0;
#pragma unroll
        for (int i = 1; i < 4; ++i) {
            const floatx4 brow = *reinterpret_cast<const floatx4 *>(gb + 16 * i + 4 * g);
            const floatx4 betar = *reinterpret_cast<const floatx4 *>(gb + 64 + 16 * i + 4 * g);
            const floatx4 lar = *reinterpret_cast<const floatx4 *>(gb + 128 + 16 * i + 4 * g);
#pragma unroll
            for (int j = 0; j < i; ++j, ++n) {
                const float bcol = gb[16 * j + c];
                // -A block destination
                __bf16 *dst;
                int kk;
                bool lo_only;
                if (i == 1) { dst = na; kk = c; lo_only = true; }
                else if (i == 2) { dst = na + 256; kk = 16 * j + c; lo_only = false; }
                else if (j < 2) { dst = na + 768; kk = 16 * j + c; lo_only = false; }
                else { dst = na + 1280; kk = c; lo_only = true; }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int rr = 4 * g + r;
                    const float e = __expf(fminf(brow[r] - bcol, 0.f));
                    const float av = -betar[r] * gk[n][r] * e;
                    dst[lo_only ? frag16_elem(rr, kk) : frag32_elem(rr, kk)] = (__bf16)av;
                    const float bread = pre ? brow[r] - lar[r] : brow[r];
                    const float pv = gq[n][r] * __expf(fminf(bread - bcol, 0.f));
                    pf[pf_index(i, j >> 1) * 512 + frag32_elem(rr, 16 * (j & 1) + c)] = (__bf16)pv;
                }
            }
        }
    }
}

__global__ __launch_bounds__(256) void chunk_fwd_fast_kernel(ChunkArgs a) {
    extern __shared__ __align__(16) char smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c = lane & 15;

    const int64_t blk = blockIdx.x;
    const int64_t xcd = blk & 7, slot = blk >> 3;
    const int64_t unit = (slot / a.ntiles) * 8 + xcd;
    const int tile = (int)(slot % a.ntiles);
    if (unit >= a.units) return;
    const int64_t seq = unit / a.Hv, head = unit % a.Hv;
    const int64_t kh = head / (a.Hv / a.Hk);
    const int64_t row = a.cu_seqlens ? 0 : seq;
    SeqView sv;
    sv.t0 = 0;
    sv.len = a.T;
    if (a.cu_seqlens) {
        sv.t0 = a.cu_seqlens[seq];
        sv.len = a.cu_seqlens[seq + 1] - sv.t0;
    }
    sv.rev = (a.flags & kFlagReverse) != 0;
    const bool pre = (a.flags & kFlagReadPre) != 0;
    const bool acc_out = (a.flags & kFlagAccumulate) != 0;
    const int64_t nchunks = (sv.len + kC - 1) / kC;
    const int dcol0 = tile * kDVT;

    const __bf16 *kb = reinterpret_cast<const __bf16 *>(a.k) + (row * a.Hk + kh) * a.T * kDK;
    const __bf16 *qb = reinterpret_cast<const __bf16 *>(a.q) + (row * a.Hk + kh) * a.T * kDK;
    const __bf16 *vb = reinterpret_cast<const __bf16 *>(a.v) + (row * a.Hv + head) * a.T * a.dv;
    const float *ab = a.log_alpha + (row * a.Hv + head) * a.T;
    const float *bb = a.beta + (row * a.Hv + head) * a.T;
    __bf16 *ob = reinterpret_cast<__bf16 *>(a.out) + (row * a.Hv + head) * a.T * a.dv;

    // the upper 16x16 tiles inside the P fragments (0,1) and (2,3) are never written: zero them
    for (int b = 0; b < 2; ++b) {
        __bf16 *pf = reinterpret_cast<__bf16 *>(smem + b * kBufBytes + kOffPf);
        for (int e = tid; e < 2 * 512; e += 256) {
            const int fr = e < 512 ? 0 : 3;
            const int el = e & 511;
            const int ln = el >> 3, s = el & 7;
            if (s >= 4) pf[fr * 512 + ln * 8 + s] = (__bf16)0.f;
            (void)ln;
        }
    }

    // The two roles run separate loops with the same barrier sequence (one barrier after the
    // prologue, one per chunk), so each role's registers are live only in its own loop.
    if (wave >= 2) {
        if (nchunks == 0) return;
        PrepRegs pr;
        load_prep(pr, sv, 0, kb, qb, ab, bb, true);
        if (wave == 2) prep_diag(smem, smem, pr, pre);
        else prep_off(smem, smem, pr, pre, sv, 0, vb, a.dv, dcol0);
        if (nchunks > 1) load_prep(pr, sv, 1, kb, qb, ab, bb, true);
        __syncthreads();
        for (int64_t ch = 0; ch < nchunks; ++ch) {
            if (ch + 1 < nchunks) {
                char *nxt = smem + (int)((ch + 1) & 1) * kBufBytes;
                if (wave == 2) prep_diag(smem, nxt, pr, pre);
                else prep_off(smem, nxt, pr, pre, sv, ch + 1, vb, a.dv, dcol0);
                if (ch + 2 < nchunks) load_prep(pr, sv, ch + 2, kb, qb, ab, bb, true);
            }
            __syncthreads();
        }
        return;
    }

    // chain waves: state rows 16t + 4g + r, column dcol of d_v
    const int dcol = dcol0 + wave * 16 + c;
    floatx4 H[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) H[t] = zero4();
    if (a.h0) {
        const float *hb = a.h0 + (seq * a.Hv + head) * kDK * a.dv;
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) H[t][r] = hb[(16 * t + 4 * g + r) * a.dv + dcol];
    }
    if (nchunks > 0) __syncthreads();

    for (int64_t ch = 0; ch < nchunks; ++ch) {
        char *cur = smem + (int)(ch & 1) * kBufBytes;
        {
            const float *sc = reinterpret_cast<const float *>(cur + kOffSc);
            // X_K = K H, X_Q = Q H
            floatx4 XK[4], XQ[4];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                XK[mi] = zero4();
                XQ[mi] = zero4();
            }
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const Frag<__bf16> hb = frag_from_acc<__bf16>(H[2 * ks], H[2 * ks + 1]);
#pragma unroll
                for (int mi = 0; mi < 4; ++mi) {
                    XK[mi] = mma32(XK[mi], lds_frag(cur + kOffKf, mi * 4 + ks), hb);
                    XQ[mi] = mma32(XQ[mi], lds_frag(cur + kOffQf, mi * 4 + ks), hb);
                }
            }
            // R = beta (V - e^{b} X_K)
            floatx4 R[4];
            const __bf16 *vt = reinterpret_cast<const __bf16 *>(cur + kOffVt) + (wave * 16 + c) * kVtPitch;
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                const bf16x4 v4 = *reinterpret_cast<const bf16x4 *>(vt + 16 * mi + 4 * g);
                const floatx4 be = *reinterpret_cast<const floatx4 *>(sc + 16 * mi + 4 * g);
                const floatx4 eb = *reinterpret_cast<const floatx4 *>(sc + 64 + 16 * mi + 4 * g);
#pragma unroll
                for (int r = 0; r < 4; ++r) R[mi][r] = be[r] * ((float)v4[r] - eb[r] * XK[mi][r]);
            }
            // U_i = T_ii (R_i - sum_{j<i} A_ij U_j)
            const char *na = cur + kOffNA;
            const char *td = cur + kOffTd;
            floatx4 U[4];
            U[0] = mma16(zero4(), lds_frag_lo(td, 0), cvt4<__bf16>(R[0]));
            floatx4 S = mma16(R[1], lds_frag_lo(na, 0), cvt4<__bf16>(U[0]));
            U[1] = mma16(zero4(), lds_frag_lo(td, 1), cvt4<__bf16>(S));
            const Frag<__bf16> u01 = frag_from_acc<__bf16>(U[0], U[1]);
            S = mma32(R[2], lds_frag(na + 512, 0), u01);
            floatx4 S3 = mma32(R[3], lds_frag(na + 1536, 0), u01);
            U[2] = mma16(zero4(), lds_frag_lo(td, 2), cvt4<__bf16>(S));
            S3 = mma16(S3, lds_frag_lo(na + 2560, 0), cvt4<__bf16>(U[2]));
            U[3] = mma16(zero4(), lds_frag_lo(td, 3), cvt4<__bf16>(S3));
            const Frag<__bf16> u23 = frag_from_acc<__bf16>(U[2], U[3]);
            // O = e^{b | b'} X_Q + P U
            floatx4 O[4];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                const floatx4 er = *reinterpret_cast<const floatx4 *>(sc + 128 + 16 * mi + 4 * g);
                O[mi] = er * XQ[mi];
                O[mi] = mma32(O[mi], lds_frag(cur + kOffPf, pf_index(mi, 0)), u01);
                if (mi >= 2) O[mi] = mma32(O[mi], lds_frag(cur + kOffPf, pf_index(mi, 1)), u23);
            }
            // H <- e^{b_C} H + K^T diag(e^{b_C - b}) U
            floatx4 W[4];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                const floatx4 ec = *reinterpret_cast<const floatx4 *>(sc + 192 + 16 * mi + 4 * g);
                W[mi] = ec * U[mi];
            }
            const float gC = sc[256];
            const Frag<__bf16> w01 = frag_from_acc<__bf16>(W[0], W[1]);
            const Frag<__bf16> w23 = frag_from_acc<__bf16>(W[2], W[3]);
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                H[t] = H[t] * gC;
                H[t] = mma32(H[t], lds_frag(cur + kOffKtf, t * 2 + 0), w01);
                H[t] = mma32(H[t], lds_frag(cur + kOffKtf, t * 2 + 1), w23);
            }
            // outputs through a per-wave staging tile for 16-byte stores
            __bf16 *stg = reinterpret_cast<__bf16 *>(smem + kOffStage + wave * 2048);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int r = 0; r < 4; ++r) stg[(16 * mi + 4 * g + r) * 16 + c] = (__bf16)O[mi][r];
            wave_lds_sync();
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int piece = lane + 64 * q;
                const int rrow = piece >> 1, half = piece & 1;
                const int64_t pos = ch * kC + rrow;
                if (pos < sv.len) {
                    uint4 val = *reinterpret_cast<const uint4 *>(stg + rrow * 16 + 8 * half);
                    uint4 *dst = reinterpret_cast<uint4 *>(ob + sv.token(pos) * a.dv + dcol0 + wave * 16 + 8 * half);
                    if (acc_out) {
                        const bf16x8 o8 = __builtin_bit_cast(bf16x8, val);
                        const bf16x8 p8 = __builtin_bit_cast(bf16x8, *dst);
                        bf16x8 s8;
#pragma unroll
                        for (int e = 0; e < 8; ++e) s8[e] = (__bf16)((float)o8[e] + (float)p8[e]);
                        val = __builtin_bit_cast(uint4, s8);
                    }
                    *dst = val;
                }
            }
        }
        __syncthreads();
    }

    if (a.hT) {
        float *hb = a.hT + (seq * a.Hv + head) * kDK * a.dv;
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) hb[(16 * t + 4 * g + r) * a.dv + dcol] = H[t][r];
    }
}

}  // namespace

bool chunk_fwd_fast_supported(int dtype, int chunk, int dk) {
    return dtype == kDtypeBf16 && chunk == kC && dk == kDK;
}

hipError_t launch_chunk_fwd_fast(const ChunkArgs &a, hipStream_t stream) {
    static bool configured = false;
    if (!configured) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&chunk_fwd_fast_kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, kSmemBytes);
        if (e != hipSuccess) return e;
        configured = true;
    }
    const int64_t blocks = (a.units + 7) / 8 * 8 * a.ntiles;
    hipLaunchKernelGGL(chunk_fwd_fast_kernel, dim3((unsigned)blocks), dim3(256), kSmemBytes, stream, a);
    return hipGetLastError();
}

}  // namespace gdr
