// Chunk-parallel forward of GDN-2 on gfx950: the delta rule with a decay per key channel and
// separate erase and write gates (BidirectionalGatedDeltaNet2 on the "tiny_gdn/fugue.py" page),
// in the layout H = S^T [d_k][d_v]:
//
//   H_t = (I - k_t (b_t * k_t)^T) Diag(e^{g_t}) H_{t-1} + k_t (w_t * v_t)^T
//
// Per chunk of C tokens with entry state H0 and G the per-channel cumsum of g inside the chunk
// (G_{-1} = 0, Gr_t = G_t for the post-write read, G_{t-1} for the pre-write read):
//
//   A_ts = sum_c b_tc k_tc k_sc e^{G_tc - G_sc}     (s < t)       T = (I + A)^{-1}
//   P_ts = sum_c q_tc k_sc e^{Gr_tc - G_sc}         (s <= t post, s < t pre)
//   U    = T (W * V - (B * K * e^{G}) H0)            (the rows of U are the u_t of the recurrence)
//   O    = (Q * e^{Gr}) H0 + P U
//   H   <- Diag(e^{G_C}) H0 + (K * e^{G_C - G})^T U
//
// This is the chunk form of the scalar kernels with the decay ratios moved inside the
// contractions, so they must be formed per channel. Every ratio is kept at most 1 by measuring
// decay from a reference row per 16-token block I of the chunk (ref_I = 16 I - 1; row -1 is
// the chunk entry), with f_t = e^{G_t - G_ref} (t in I), r_s = e^{G_end(I) - G_s} (s in I) and
// the block decay D_I = e^{G_end(I) - G_ref(I)}:
//
//   LA_t = b_t k_t f_t,   LP_t = q_t f(r)_t,   R_s = k_s r_s      (stored in place of b, q, k)
//   tile (I, J < I):  sum_c LA_tc R_sc prod_{J < J' < I} D_J'c   (every factor <= 1)
//   tile (I, I):      sum_c LA_tc R_sc / D_Ic                    (exact while D_Ic >= e^-60)
//
// A diagonal block whose decay over some channel is stronger than that (log decay sum below
// -60 over 16 tokens) takes an exact path instead: running products of e^{g} along the block,
// on the vector units. The chain uses the same operands: B K e^{G} and Q e^{Gr} of block I are
// LA_I and LP_I against Diag(e^{G_ref(I)}) H0, and the state update runs block by block,
// H <- Diag(D_J) H + R_J^T U_J.
//
// Work split inside the workgroup of 4 waves (one per (sequence, value head, 32 columns of
// d_v)), per chunk: all threads load the chunk and form the per-channel products (one thread
// per pair of channels and block); the waves share the Gram tiles on the matrix cores (and the
// exact diagonal blocks, one wave per block); wave 0 inverts I + A; waves 0 and 1 run the
// state-dependent chain for 16 columns each, with the state in accumulator registers; all
// threads prefetch the next chunk into registers meanwhile.
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
constexpr float kSafeLogDecay = -60.f;  // block decay (natural log) below which the exact path runs

template <typename E>
struct Pad {
    static constexpr int v = 16 / sizeof(E);
};
template <typename E>
constexpr bool kIsBf16 = sizeof(E) == 2;
// the chain's output staging (bf16 outputs only): two waves x up to 32 rows x 16 columns, fp32
template <typename E, int C>
struct OutStage {
    static constexpr int kPitch = 20, kRows = C < 32 ? C : 32;
    static constexpr int kFloats = kIsBf16<E> ? 2 * kRows * kPitch : 4;
};

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(__bf16 x) { return (float)x; }

// two adjacent elements as floats, and back
__device__ __forceinline__ void ld2(const float *p, float &x, float &y) {
    const float2 t = *reinterpret_cast<const float2 *>(p);
    x = t.x;
    y = t.y;
}
__device__ __forceinline__ void ld2(const __bf16 *p, float &x, float &y) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    const b2 t = *reinterpret_cast<const b2 *>(p);
    x = (float)t[0];
    y = (float)t[1];
}
__device__ __forceinline__ void st2(float *p, float x, float y) { *reinterpret_cast<float2 *>(p) = make_float2(x, y); }
__device__ __forceinline__ void st2(__bf16 *p, float x, float y) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    *reinterpret_cast<b2 *>(p) = __builtin_convertvector((f2){x, y}, b2);
}

template <typename E, int C, int DK>
struct alignas(16) Smem {
    static constexpr int NT = C / 16;
    static constexpr int KP = DK + Pad<E>::v;       // pitch of the C x DK matrices (elements)
    static constexpr int VP = kDvTile + Pad<E>::v;  // pitch of the V and W tiles
    static constexpr int AP = C + 4;                // pitch of the fp32 A matrix
    static constexpr int TP = C + Pad<E>::v;        // pitch of T and P
    static constexpr int GP = DK + 4;               // pitch of the fp32 gate matrix
    E K[C * KP];   // k, then R
    E Q[C * KP];   // q, then LP
    E Bk[C * KP];  // b, then LA
    E V[C * VP];
    E W[C * VP];
    E T[C * TP];
    E P[C * TP];
    float A[C * AP];
    float G[C * GP];                              // g, then e^{g}
    float dec[NT * DK] __attribute__((aligned(16)));   // D_I per channel
    float inv[NT * DK] __attribute__((aligned(16)));   // 1 / D_I (0 for a block on the exact path)
    float eref[NT * DK] __attribute__((aligned(16)));  // e^{G_ref(I)} per channel
    int unsafe[NT];
};

template <typename E, int C, int DK>
struct Prefetch {
    static constexpr int KROW = DK * (int)sizeof(E) / 16;  // 16-byte pieces per row of k, q, b
    static constexpr int KPIECES = C * KROW;
    static constexpr int KPER = (KPIECES + kThreads - 1) / kThreads;
    static constexpr int GROW = DK * 4 / 16;
    static constexpr int GPIECES = C * GROW;
    static constexpr int GPER = (GPIECES + kThreads - 1) / kThreads;
    static constexpr int VROW = kDvTile * (int)sizeof(E) / 16;
    static constexpr int VPIECES = C * VROW;
    static constexpr int VPER = (VPIECES + kThreads - 1) / kThreads;
    uint4 k[KPER], q[KPER], b[KPER], g[GPER], v[VPER], w[VPER];
};

struct SeqView {
    int64_t t0, len;
    bool rev;
    __device__ __forceinline__ int64_t token(int64_t pos) const { return rev ? t0 + len - 1 - pos : t0 + pos; }
};

struct Bases {
    const char *k, *q, *b, *g, *v, *w;
    int64_t dv;
    int dcol0;
};

template <typename E, int C, int DK>
__device__ __forceinline__ void prefetch_chunk(Prefetch<E, C, DK> &pf, const SeqView &sv, int64_t c, const Bases &bs) {
    typedef Prefetch<E, C, DK> PF;
    const int tid = threadIdx.x;
    const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < PF::KPER; ++i) {
        const int piece = tid + i * kThreads;
        pf.k[i] = z;
        pf.q[i] = z;
        pf.b[i] = z;
        if (piece < PF::KPIECES) {
            const int r = piece / PF::KROW, cp = piece % PF::KROW;
            const int64_t pos = c * C + r;
            if (pos < sv.len) {
                const int64_t off = sv.token(pos) * (int64_t)(DK * sizeof(E)) + cp * 16;
                pf.k[i] = *reinterpret_cast<const uint4 *>(bs.k + off);
                pf.q[i] = *reinterpret_cast<const uint4 *>(bs.q + off);
                pf.b[i] = *reinterpret_cast<const uint4 *>(bs.b + off);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < PF::GPER; ++i) {
        const int piece = tid + i * kThreads;
        pf.g[i] = z;  // zero log decay (no decay) past the end
        if (piece < PF::GPIECES) {
            const int r = piece / PF::GROW, cp = piece % PF::GROW;
            const int64_t pos = c * C + r;
            if (pos < sv.len) pf.g[i] = *reinterpret_cast<const uint4 *>(bs.g + sv.token(pos) * (int64_t)(DK * 4) + cp * 16);
        }
    }
#pragma unroll
    for (int i = 0; i < PF::VPER; ++i) {
        const int piece = tid + i * kThreads;
        pf.v[i] = z;
        pf.w[i] = z;
        if (piece < PF::VPIECES) {
            const int r = piece / PF::VROW, cp = piece % PF::VROW;
            const int64_t pos = c * C + r;
            if (pos < sv.len && bs.v) {
                const int64_t off = (sv.token(pos) * bs.dv + bs.dcol0) * (int64_t)sizeof(E) + cp * 16;
                pf.v[i] = *reinterpret_cast<const uint4 *>(bs.v + off);
                pf.w[i] = *reinterpret_cast<const uint4 *>(bs.w + off);
            }
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
            const int o = r * SM::KP * (int)sizeof(E) + cp * 16;
            *reinterpret_cast<uint4 *>(reinterpret_cast<char *>(sm.K) + o) = pf.k[i];
            *reinterpret_cast<uint4 *>(reinterpret_cast<char *>(sm.Q) + o) = pf.q[i];
            *reinterpret_cast<uint4 *>(reinterpret_cast<char *>(sm.Bk) + o) = pf.b[i];
        }
    }
#pragma unroll
    for (int i = 0; i < PF::GPER; ++i) {
        const int piece = tid + i * kThreads;
        if (piece < PF::GPIECES) {
            const int r = piece / PF::GROW, cp = piece % PF::GROW;
            *reinterpret_cast<uint4 *>(reinterpret_cast<char *>(sm.G) + r * SM::GP * 4 + cp * 16) = pf.g[i];
        }
    }
#pragma unroll
    for (int i = 0; i < PF::VPER; ++i) {
        const int piece = tid + i * kThreads;
        if (piece < PF::VPIECES) {
            const int r = piece / PF::VROW, cp = piece % PF::VROW;
            const int o = r * SM::VP * (int)sizeof(E) + cp * 16;
            *reinterpret_cast<uint4 *>(reinterpret_cast<char *>(sm.V) + o) = pf.v[i];
            *reinterpret_cast<uint4 *>(reinterpret_cast<char *>(sm.W) + o) = pf.w[i];
        }
    }
    if (tid < SM::NT) sm.unsafe[tid] = 0;
}

// Unit-norm rows of K and Q (rows past the end are zero and stay zero).
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
        for (int e = 0; e < PER; ++e) p[lane + 64 * e] = static_cast<E>(x[e] * r);
    }
}

// Per (channel, block): e^{g} in place of g, the block decay D, its inverse where the block is
// on the matrix-core path, and the flag of a block that needs the exact path.
template <typename E, int C, int DK>
__device__ __forceinline__ void block_decays(Smem<E, C, DK> &sm) {
    typedef Smem<E, C, DK> SM;
    for (int pi = threadIdx.x; pi < DK * SM::NT; pi += kThreads) {
        const int c = pi % DK, blk = pi / DK;
        float *p = sm.G + 16 * blk * SM::GP + c;
        float gv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) gv[i] = p[i * SM::GP];
        float s = 0.f, d = 1.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            s += gv[i];
            const float a = __expf(gv[i]);
            d *= a;
            p[i * SM::GP] = a;
        }
        const bool safe = s >= kSafeLogDecay;
        sm.dec[blk * DK + c] = d;
        sm.inv[blk * DK + c] = safe ? 1.f / d : 0.f;
        if (!safe) atomicOr(&sm.unsafe[blk], 1);
    }
}

// The operands in place: LA = b k f, LP = q f (f of the previous row for the pre-write read),
// R = k r, and e^{G_ref} per block; one (channel, block) per thread.
template <typename E, int C, int DK>
__device__ __forceinline__ void form_operands(Smem<E, C, DK> &sm, bool pre) {
    typedef Smem<E, C, DK> SM;
    for (int pi = threadIdx.x; pi < DK * SM::NT; pi += kThreads) {
        const int c = pi % DK, blk = pi / DK;
        float e = 1.f;
        for (int j = 0; j < blk; ++j) e *= sm.dec[j * DK + c];
        sm.eref[blk * DK + c] = e;
        const int r0 = 16 * blk;
        float a[16], kv[16], qv[16], bv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            a[i] = sm.G[(r0 + i) * SM::GP + c];
            kv[i] = to_f(sm.K[(r0 + i) * SM::KP + c]);
            qv[i] = to_f(sm.Q[(r0 + i) * SM::KP + c]);
            bv[i] = to_f(sm.Bk[(r0 + i) * SM::KP + c]);
        }
        float f = 1.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float prev = f;
            f *= a[i];
            sm.Bk[(r0 + i) * SM::KP + c] = static_cast<E>(bv[i] * kv[i] * f);
            sm.Q[(r0 + i) * SM::KP + c] = static_cast<E>(qv[i] * (pre ? prev : f));
        }
        float r = 1.f;
#pragma unroll
        for (int i = 15; i >= 0; --i) {
            sm.K[(r0 + i) * SM::KP + c] = static_cast<E>(kv[i] * r);
            r *= a[i];
        }
    }
}

// One diagonal block on the exact path, by one wave, from the raw b, k, q and e^{g} (called
// before form_operands). Lane (p, cg) = (lane & 7, lane >> 3) owns the columns s = p and
// s = 15 - p and channels [cg * DK/8, (cg + 1) * DK/8); it carries y_c = k_sc prod_{s<u<=t} e^{g_uc}
// down the rows t and sums its channels; the eight channel groups are then added across lanes.
template <typename E, int C, int DK>
__device__ __forceinline__ void exact_diag_block(Smem<E, C, DK> &sm, int blk, bool pre) {
    typedef Smem<E, C, DK> SM;
    constexpr int NCH = DK / 8;
    const int lane = threadIdx.x & 63;
    const int p = lane & 7, cg = lane >> 3;
    const int c0 = cg * NCH, r0 = 16 * blk;
    const int sa = p, sb = 15 - p;
    float ya[NCH], yb[NCH];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        ya[j] = to_f(sm.K[(r0 + sa) * SM::KP + c0 + j]);
        yb[j] = to_f(sm.K[(r0 + sb) * SM::KP + c0 + j]);
    }
    for (int t = 0; t < 16; ++t) {
        const int row = r0 + t;
        float av[NCH], kb[NCH], qv[NCH];
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            av[j] = sm.G[row * SM::GP + c0 + j];
            kb[j] = to_f(sm.Bk[row * SM::KP + c0 + j]) * to_f(sm.K[row * SM::KP + c0 + j]);
            qv[j] = to_f(sm.Q[row * SM::KP + c0 + j]);
        }
        float res[4];  // A(t, sa), P(t, sa), A(t, sb), P(t, sb)
#pragma unroll
        for (int side = 0; side < 2; ++side) {
            float *y = side ? yb : ya;
            const int s = side ? sb : sa;
            float pa = 0.f, pp = 0.f;
            if (t > s) {
                if (pre) {
#pragma unroll
                    for (int j = 0; j < NCH; ++j) pp += qv[j] * y[j];
                }
#pragma unroll
                for (int j = 0; j < NCH; ++j) {
                    y[j] *= av[j];
                    pa += kb[j] * y[j];
                }
                if (!pre) {
#pragma unroll
                    for (int j = 0; j < NCH; ++j) pp += qv[j] * y[j];
                }
            } else if (t == s && !pre) {
#pragma unroll
                for (int j = 0; j < NCH; ++j) pp += qv[j] * y[j];
            }
            res[2 * side] = pa;
            res[2 * side + 1] = pp;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int off = 8; off < 64; off <<= 1) res[i] += __shfl_xor(res[i], off, 64);
        }
        if (cg == 0) {
            sm.A[row * SM::AP + r0 + sa] = res[0];
            sm.P[row * SM::TP + r0 + sa] = static_cast<E>(res[1]);
            sm.A[row * SM::AP + r0 + sb] = res[2];
            sm.P[row * SM::TP + r0 + sb] = static_cast<E>(res[3]);
        }
    }
}

// Fragment times a per-k factor: lo covers k = k0 + 4g + 0..3, hi k = k0 + 16 + 4g + 0..3.
template <typename E>
__device__ __forceinline__ Frag<E> scale_frag(const Frag<E> &f, floatx4 lo, floatx4 hi);
template <>
__device__ __forceinline__ Frag<float> scale_frag<float>(const Frag<float> &f, floatx4 lo, floatx4 hi) {
    Frag<float> r;
    r.lo = f.lo * lo;
    r.hi = f.hi * hi;
    return r;
}
template <>
__device__ __forceinline__ Frag<__bf16> scale_frag<__bf16>(const Frag<__bf16> &f, floatx4 lo, floatx4 hi) {
    floatx4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = (float)f.lo[i] * lo[i];
        b[i] = (float)f.hi[i] * hi[i];
    }
    Frag<__bf16> r;
    r.lo = cvt4<__bf16>(a);
    r.hi = cvt4<__bf16>(b);
    return r;
}

// The lower-triangular 16x16 tiles of A and P on the matrix cores, shared by the waves.
template <typename E, int C, int DK>
__device__ __forceinline__ void gram_tiles(Smem<E, C, DK> &sm, bool pre) {
    typedef Smem<E, C, DK> SM;
    constexpr int NT = SM::NT;
    constexpr int NTRI = NT * (NT + 1) / 2;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, cc = lane & 15;
    for (int t = wave; t < NTRI; t += kThreads / 64) {
        int idx = t, i = 0;
        while (idx > i) {
            idx -= i + 1;
            ++i;
        }
        const int j = idx;
        if (i == j && sm.unsafe[i]) continue;  // written by the exact path
        floatx4 acc_a = zero4(), acc_p = zero4();
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks) {
            Frag<E> la = frag_rows<E>(sm.Bk, SM::KP, 16 * i, 32 * ks);
            Frag<E> lp = frag_rows<E>(sm.Q, SM::KP, 16 * i, 32 * ks);
            const Frag<E> r = frag_rows<E>(sm.K, SM::KP, 16 * j, 32 * ks);
            if (j != i - 1) {
                const int k0 = 32 * ks + 4 * g;
                floatx4 flo, fhi;
                if (j == i) {
                    flo = *reinterpret_cast<const floatx4 *>(sm.inv + i * DK + k0);
                    fhi = *reinterpret_cast<const floatx4 *>(sm.inv + i * DK + k0 + 16);
                } else {
                    flo = *reinterpret_cast<const floatx4 *>(sm.dec + (j + 1) * DK + k0);
                    fhi = *reinterpret_cast<const floatx4 *>(sm.dec + (j + 1) * DK + k0 + 16);
                    for (int jj = j + 2; jj < i; ++jj) {
                        flo *= *reinterpret_cast<const floatx4 *>(sm.dec + jj * DK + k0);
                        fhi *= *reinterpret_cast<const floatx4 *>(sm.dec + jj * DK + k0 + 16);
                    }
                }
                la = scale_frag<E>(la, flo, fhi);
                lp = scale_frag<E>(lp, flo, fhi);
            }
            acc_a = mma32(acc_a, la, r);
            acc_p = mma32(acc_p, lp, r);
        }
        const int col = 16 * j + cc;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int row = 16 * i + 4 * g + rr;
            const bool keep_a = col < row;
            const bool keep_p = pre ? col < row : col <= row;
            sm.A[row * SM::AP + col] = keep_a ? acc_a[rr] : 0.f;
            sm.P[row * SM::TP + col] = static_cast<E>(keep_p ? acc_p[rr] : 0.f);
        }
    }
}

template <typename E, int C, int DK>
__global__ __launch_bounds__(kThreads) void gdn2_chunk_kernel(Gdn2Args a) {
    typedef Smem<E, C, DK> SM;
    constexpr int NT = SM::NT;
    constexpr int HT = DK / 16;
    __shared__ SM sm;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform across the wave
    const int g = lane >> 4, cc = lane & 15;

    // block -> (unit, d_v tile); the tiles of one unit land on one XCD and share K/Q in its L2
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
    const bool l2 = (a.flags & kFlagL2Norm) != 0;
    const int64_t nchunks = (sv.len + C - 1) / C;
    const int dcol0 = tile * kDvTile;

    Bases bs;
    const int64_t kq_off = (row * a.Hk + kh) * a.T * DK;
    const int64_t v_off = (row * a.Hv + head) * a.T * a.dv;
    bs.k = reinterpret_cast<const char *>(a.k) + kq_off * (int64_t)sizeof(E);
    bs.q = reinterpret_cast<const char *>(a.q) + kq_off * (int64_t)sizeof(E);
    bs.b = reinterpret_cast<const char *>(a.b) + kq_off * (int64_t)sizeof(E);
    bs.g = reinterpret_cast<const char *>(a.g) + kq_off * 4;
    bs.v = reinterpret_cast<const char *>(a.v) + v_off * (int64_t)sizeof(E);
    bs.w = reinterpret_cast<const char *>(a.w) + v_off * (int64_t)sizeof(E);
    bs.dv = a.dv;
    bs.dcol0 = dcol0;
    E *ob = reinterpret_cast<E *>(a.out) + v_off;

    // strictly upper blocks of T and P are never written again
    for (int i = tid; i < C * SM::TP; i += kThreads) {
        sm.T[i] = static_cast<E>(0.f);
        sm.P[i] = static_cast<E>(0.f);
    }

    const bool chain = wave < 2;
    const int lcol = wave * 16;
    const int dcol = dcol0 + lcol + cc;
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
        prefetch_chunk<E, C, DK>(pf, sv, 0, bs);
        store_chunk<E, C, DK>(pf, sm);
    }
    __syncthreads();

    for (int64_t c = 0; c < nchunks; ++c) {
        if (c + 1 < nchunks) prefetch_chunk<E, C, DK>(pf, sv, c + 1, bs);

        if (l2) normalize_rows<E, C, DK>(sm);
        block_decays<E, C, DK>(sm);
        __syncthreads();
        bool any_unsafe = false;
#pragma unroll
        for (int i = 0; i < NT; ++i) any_unsafe |= sm.unsafe[i] != 0;
        if (any_unsafe) {
            for (int i = wave; i < NT; i += kThreads / 64)
                if (sm.unsafe[i]) exact_diag_block<E, C, DK>(sm, i, pre);
            __syncthreads();
        }
        form_operands<E, C, DK>(sm, pre);
        __syncthreads();
        gram_tiles<E, C, DK>(sm, pre);
        __syncthreads();
        if (wave == 0) solve_unit_lower_inverse<E, C>(sm);
        __syncthreads();

        if (chain) {
            // X_K = (B K e^G) H, X_Q = (Q e^{Gr}) H, block by block against Diag(e^{G_ref}) H
            floatx4 XK[NT], XQ[NT];
#pragma unroll
            for (int mi = 0; mi < NT; ++mi) {
                XK[mi] = zero4();
                XQ[mi] = zero4();
            }
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks) {
#pragma unroll
                for (int mi = 0; mi < NT; ++mi) {
                    floatx4 h0 = H[2 * ks], h1 = H[2 * ks + 1];
                    if (mi > 0) {
                        h0 *= *reinterpret_cast<const floatx4 *>(sm.eref + mi * DK + 32 * ks + 4 * g);
                        h1 *= *reinterpret_cast<const floatx4 *>(sm.eref + mi * DK + 32 * ks + 16 + 4 * g);
                    }
                    const Frag<E> hb = frag_from_acc<E>(h0, h1);
                    XK[mi] = mma32(XK[mi], frag_rows<E>(sm.Bk, SM::KP, 16 * mi, 32 * ks), hb);
                    XQ[mi] = mma32(XQ[mi], frag_rows<E>(sm.Q, SM::KP, 16 * mi, 32 * ks), hb);
                }
            }
            // right-hand sides W * V - X_K, then U = T R
            floatx4 R[NT];
#pragma unroll
            for (int mi = 0; mi < NT; ++mi)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int rr = 16 * mi + 4 * g + r;
                    R[mi][r] = to_f(sm.W[rr * SM::VP + lcol + cc]) * to_f(sm.V[rr * SM::VP + lcol + cc]) - XK[mi][r];
                }
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
            // O = X_Q + P U
#pragma unroll
            for (int mi = 0; mi < NT; ++mi) {
                floatx4 o = XQ[mi];
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
                    if (pos < sv.len) {
                        E *dst = ob + sv.token(pos) * a.dv + dcol;
                        const float prev = acc_out ? to_f(*dst) : 0.f;
                        *dst = static_cast<E>(prev + o[r]);
                    }
                }
            }
            // H <- Diag(D_J) H + R_J^T U_J, block by block
#pragma unroll
            for (int J = 0; J < NT; ++J) {
#pragma unroll
                for (int t = 0; t < HT; ++t) {
                    H[t] *= *reinterpret_cast<const floatx4 *>(sm.dec + J * DK + 16 * t + 4 * g);
                    H[t] = mma16(H[t], frag_cols_lo<E>(sm.K, SM::KP, 16 * t, 16 * J), cvt4<E>(U[J]));
                }
            }
        }
        __syncthreads();
        if (c + 1 < nchunks) {
            store_chunk<E, C, DK>(pf, sm);
            __syncthreads();
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

// ============================================================ two-pass form
// With a workspace the forward runs in two passes. The first computes, for every chunk at once
// (one workgroup per chunk and key head), what depends on the chunk's keys and gates alone:
//
//   Wc = T (B * K * e^{G})        [C][d_k]   (the WY form: U = T (W * V) - Wc H0)
//   Qc = Q * e^{Gr}               [C][d_k]
//   Kt = (K * e^{G_C - G})^T      [d_k][C]
//   P, T                          [C][C]
//   e^{G_C}                       [d_k] fp32
//
// from the per-block operands above (LA, LP and R times the products of block decays that make
// them relative to the chunk start or end; every factor <= 1). The second walks the chunks of
// each (sequence, value head, 32 columns of d_v) with the state in registers:
//
//   U = T (W * V) - Wc H,   O = Qc H + P U,   H <- Diag(e^{G_C}) H + Kt U
//
// so that its serial part holds only the products against the state.
template <typename E, int C, int DK>
struct WsKey {  // bytes of one (chunk, key head) block, every part 16-byte aligned
    static constexpr int64_t kW = 0;
    static constexpr int64_t kQ = kW + (int64_t)C * DK * sizeof(E);
    static constexpr int64_t kKt = kQ + (int64_t)C * DK * sizeof(E);
    static constexpr int64_t kP = kKt + (int64_t)C * DK * sizeof(E);
    static constexpr int64_t kT = kP + (int64_t)C * C * sizeof(E);
    static constexpr int64_t kEgc = kT + (int64_t)C * C * sizeof(E);
    static constexpr int64_t kBytes = kEgc + DK * 4;
};

// workspace slot of chunk c of sequence seq (packed: cu[seq] / C + seq + c, which keeps the
// slots of consecutive sequences apart; else seq * ceil(T / C) + c)
template <int C>
__device__ __forceinline__ int64_t ws_slot(const Gdn2Args &a, int64_t seq, int64_t c) {
    if (a.cu_seqlens) return a.cu_seqlens[seq] / C + seq + c;
    return seq * ((a.T + C - 1) / C) + c;
}

// 16-byte pieces from a padded LDS matrix (rows of RB bytes) to a dense global one
template <int ROWS, int RB>
__device__ __forceinline__ void lds_to_global(char *dst, const char *src, int src_pitch) {
    constexpr int PR = RB / 16, N = ROWS * PR;
    for (int i = threadIdx.x; i < N; i += kThreads) {
        const int r = i / PR, p = i % PR;
        *reinterpret_cast<uint4 *>(dst + r * RB + p * 16) = *reinterpret_cast<const uint4 *>(src + r * src_pitch + p * 16);
    }
}

template <typename E, int C, int DK>
__global__ __launch_bounds__(kThreads) void gdn2_prep_kernel(Gdn2Args a) {
    typedef Smem<E, C, DK> SM;
    typedef WsKey<E, C, DK> WK;
    constexpr int NT = SM::NT;
    __shared__ SM sm;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform across the wave
    const int g = lane >> 4, cc = lane & 15;

    // workgroup -> (slot, key head) -> (sequence, chunk); slots between sequences are idle
    const int64_t slot = blockIdx.x / a.Hk, kh = blockIdx.x % a.Hk;
    int64_t seq, c;
    if (a.cu_seqlens) {
        // the last sequence whose first slot is <= slot
        int64_t lo = 0, hi = a.units / a.Hv - 1;
        while (lo < hi) {
            const int64_t mid = (lo + hi + 1) / 2;
            if (a.cu_seqlens[mid] / C + mid <= slot) lo = mid;
            else hi = mid - 1;
        }
        seq = lo;
        c = slot - (a.cu_seqlens[seq] / C + seq);
    } else {
        const int64_t per = (a.T + C - 1) / C;
        seq = slot / per;
        c = slot % per;
    }
    SeqView sv;
    sv.t0 = 0;
    sv.len = a.T;
    if (a.cu_seqlens) {
        sv.t0 = a.cu_seqlens[seq];
        sv.len = a.cu_seqlens[seq + 1] - sv.t0;
    }
    sv.rev = (a.flags & kFlagReverse) != 0;
    if (c < 0 || c * C >= sv.len) return;
    const bool pre = (a.flags & kFlagReadPre) != 0;
    const bool l2 = (a.flags & kFlagL2Norm) != 0;
    const int64_t row = a.cu_seqlens ? 0 : seq;

    Bases bs;
    const int64_t kq_off = (row * a.Hk + kh) * a.T * DK;
    bs.k = reinterpret_cast<const char *>(a.k) + kq_off * (int64_t)sizeof(E);
    bs.q = reinterpret_cast<const char *>(a.q) + kq_off * (int64_t)sizeof(E);
    bs.b = reinterpret_cast<const char *>(a.b) + kq_off * (int64_t)sizeof(E);
    bs.g = reinterpret_cast<const char *>(a.g) + kq_off * 4;
    bs.v = nullptr;  // the value side is the second pass's
    bs.w = nullptr;
    bs.dv = a.dv;
    bs.dcol0 = 0;

    for (int i = tid; i < C * SM::TP; i += kThreads) {
        sm.T[i] = static_cast<E>(0.f);
        sm.P[i] = static_cast<E>(0.f);
    }
    {
        Prefetch<E, C, DK> pf;
        prefetch_chunk<E, C, DK>(pf, sv, c, bs);
        store_chunk<E, C, DK>(pf, sm);
    }
    __syncthreads();
    if (l2) {
        normalize_rows<E, C, DK>(sm);
        __syncthreads();
    }
    block_decays<E, C, DK>(sm);
    __syncthreads();
    bool any_unsafe = false;
#pragma unroll
    for (int i = 0; i < NT; ++i) any_unsafe |= sm.unsafe[i] != 0;
    if (any_unsafe) {
        for (int i = wave; i < NT; i += kThreads / 64)
            if (sm.unsafe[i]) exact_diag_block<E, C, DK>(sm, i, pre);
        __syncthreads();
    }
    form_operands<E, C, DK>(sm, pre);
    __syncthreads();
    gram_tiles<E, C, DK>(sm, pre);
    __syncthreads();
    if (wave == 0) solve_unit_lower_inverse<E, C, SM, true>(sm);

    char *kb = reinterpret_cast<char *>(a.ws) + (ws_slot<C>(a, seq, c) * a.Hk + kh) * WK::kBytes;
    // chunk-relative operands in place (while wave 0 solves): LA and LP times e^{G_ref} of their
    // block, R times the decay of the blocks after its own; e^{G_C} = the product of all block
    // decays
    for (int i = tid; i < NT * DK; i += kThreads) {
        const int blk = i / DK, ch = i % DK;
        const float er = sm.eref[blk * DK + ch];
        float tail = 1.f;
        for (int j = blk + 1; j < NT; ++j) tail *= sm.dec[j * DK + ch];
#pragma unroll 4
        for (int r = 16 * blk; r < 16 * blk + 16; ++r) {
            sm.Bk[r * SM::KP + ch] = static_cast<E>(to_f(sm.Bk[r * SM::KP + ch]) * er);
            sm.Q[r * SM::KP + ch] = static_cast<E>(to_f(sm.Q[r * SM::KP + ch]) * er);
            sm.K[r * SM::KP + ch] = static_cast<E>(to_f(sm.K[r * SM::KP + ch]) * tail);
        }
        if (blk == 0) {
            float e = 1.f;
            for (int j = 0; j < NT; ++j) e *= sm.dec[j * DK + ch];
            reinterpret_cast<float *>(kb + WK::kEgc)[ch] = e;
        }
    }
    __syncthreads();
    // Wc = T LAe on the matrix cores: NT x DK/16 output tiles over the waves
    constexpr int NWT = NT * (DK / 16);
    constexpr int PER = (NWT + 3) / 4;
    floatx4 wt[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int t = wave + 4 * j;
        wt[j] = zero4();
        if (t < NWT) {
            const int mi = t / (DK / 16), nj = t % (DK / 16);
            if constexpr (C == 16) {
                wt[j] = mma16(wt[j], frag_rows_lo<E>(sm.T, SM::TP, 0, 0), frag_cols_lo<E>(sm.Bk, SM::KP, 16 * nj, 0));
            } else {
#pragma unroll
                for (int k0 = 0; k0 < C; k0 += 32)
                    wt[j] = mma32(wt[j], frag_rows<E>(sm.T, SM::TP, 16 * mi, k0), frag_cols<E>(sm.Bk, SM::KP, 16 * nj, k0));
            }
        }
    }
    // the rest of the block while the products are in registers: Qc, Kt (transposed), P, T
    lds_to_global<C, DK * sizeof(E)>(kb + WK::kQ, reinterpret_cast<const char *>(sm.Q), SM::KP * sizeof(E));
    lds_to_global<C, C * sizeof(E)>(kb + WK::kP, reinterpret_cast<const char *>(sm.P), SM::TP * sizeof(E));
    lds_to_global<C, C * sizeof(E)>(kb + WK::kT, reinterpret_cast<const char *>(sm.T), SM::TP * sizeof(E));
    {
        constexpr int EPP = 16 / sizeof(E);  // elements per 16-byte piece
        constexpr int PR = C / EPP, N = DK * PR;
        for (int i = tid; i < N; i += kThreads) {
            const int d = i / PR, t0 = (i % PR) * EPP;
            uint4 piece;
            E *v = reinterpret_cast<E *>(&piece);
#pragma unroll
            for (int e = 0; e < EPP; ++e) v[e] = sm.K[(t0 + e) * SM::KP + d];
            *reinterpret_cast<uint4 *>(kb + WK::kKt + ((int64_t)d * C + t0) * sizeof(E)) = piece;
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int t = wave + 4 * j;
        if (t < NWT) {
            const int mi = t / (DK / 16), nj = t % (DK / 16);
#pragma unroll
            for (int r = 0; r < 4; ++r) sm.Bk[(16 * mi + 4 * g + r) * SM::KP + 16 * nj + cc] = static_cast<E>(wt[j][r]);
        }
    }
    __syncthreads();
    lds_to_global<C, DK * sizeof(E)>(kb + WK::kW, reinterpret_cast<const char *>(sm.Bk), SM::KP * sizeof(E));
}

// Chain buffers: one chunk's operands, padded rows (E elements unless noted); WV = W * V of
// the workgroup's 32 columns
template <typename E, int C, int DK>
struct alignas(16) ChainBuf {
    static constexpr int KP = DK + Pad<E>::v;        // Wc, Qc
    static constexpr int CP = C + Pad<E>::v;         // Kt, P, T
    static constexpr int UP = kDvTile + Pad<E>::v;   // WV
    E W[C * KP];
    E Q[C * KP];
    E Kt[DK * CP];
    E P[C * CP];
    E T[C * CP];
    E WV[C * UP];
    float egc[DK];
};
// The copy of one chunk by a pair of loader waves (128 threads): the key block is contiguous
// in the workspace (piece i at byte 16 i); v and w pieces come in pairs and are multiplied on
// the way into LDS. R pairs of loader waves take every R-th chunk, each pair with one set of
// registers, so that R copies are in flight and each has R chain steps to arrive.
template <typename E, int C, int DK>
struct ChainCopy {
    static constexpr int EPP = 16 / sizeof(E);
    static constexpr int NW = C * DK / EPP, NP = C * C / EPP, NE = DK / 4;
    static constexpr int NKEY = 3 * NW + 2 * NP + NE;
    static constexpr int NV = C * kDvTile / EPP;
    static constexpr int kLoaders = kThreads / 2;
    static constexpr int PK = (NKEY + kLoaders - 1) / kLoaders;
    static constexpr int PV = (NV + kLoaders - 1) / kLoaders;
    static constexpr int kRegs = 4 * (PK + 2 * PV);  // VGPRs of one set
    static constexpr int R = kRegs <= 72 ? 3 : kRegs <= 100 ? 2 : 1;
    static constexpr int kWaves = 2 + 2 * R;  // two chain waves, R loader pairs
    // double-buffered operands and the output staging must fit in the 160 KB of LDS
    static constexpr bool kFits = 2 * sizeof(ChainBuf<E, C, DK>) + 4 * OutStage<E, C>::kFloats <= 160 * 1024;
};

// LDS byte offset inside ChainBuf of key piece i
template <typename E, int C, int DK>
__device__ __forceinline__ int key_piece_dst(int i) {
    typedef ChainCopy<E, C, DK> CC;
    typedef ChainBuf<E, C, DK> CB;
    constexpr int es = sizeof(E), EPP = CC::EPP;
    if (i < 2 * CC::NW) {
        const int m = i < CC::NW ? 0 : 1, j = i - m * CC::NW;
        return (m ? offsetof(CB, Q) : offsetof(CB, W)) + (j / (DK / EPP)) * CB::KP * es + (j % (DK / EPP)) * 16;
    }
    i -= 2 * CC::NW;
    if (i < CC::NW) return offsetof(CB, Kt) + (i / (C / EPP)) * CB::CP * es + (i % (C / EPP)) * 16;
    i -= CC::NW;
    if (i < 2 * CC::NP) {
        const int m = i < CC::NP ? 0 : 1, j = i - m * CC::NP;
        return (m ? offsetof(CB, T) : offsetof(CB, P)) + (j / (C / EPP)) * CB::CP * es + (j % (C / EPP)) * 16;
    }
    i -= 2 * CC::NP;
    return offsetof(CB, egc) + i * 16;
}

template <typename E, int C, int DK>
__global__ __launch_bounds__((64 * ChainCopy<E, C, DK>::kWaves)) void gdn2_chain_kernel(Gdn2Args a) {
    typedef ChainBuf<E, C, DK> CB;
    typedef ChainCopy<E, C, DK> CC;
    typedef WsKey<E, C, DK> WK;
    constexpr int NT = C / 16;
    constexpr int HT = DK / 16;
    constexpr int R = CC::R;
    __shared__ CB buf[2];
    // each chain wave's output of a chunk, 32 rows at a time, fp32 [rows][16 columns]: written in
    // the accumulator layout, read back as 8 consecutive columns of a row per lane, so that a
    // bf16 output row piece goes out as one 16-byte store
    constexpr int kOutP = OutStage<E, C>::kPitch, kOutRows = OutStage<E, C>::kRows;
    __shared__ __align__(16) float ostage[OutStage<E, C>::kFloats];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform across the wave
    const int g = lane >> 4, cc = lane & 15;
    const int64_t blk = blockIdx.x;
    const int64_t xcd = blk & 7, sl = blk >> 3;
    const int64_t unit = (sl / a.ntiles) * 8 + xcd;
    const int tile = (int)(sl % a.ntiles);
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
    const bool acc_out = (a.flags & kFlagAccumulate) != 0;
    const int64_t nchunks = (sv.len + C - 1) / C;
    const int dcol0 = tile * kDvTile;
    const int64_t v_off = (row * a.Hv + head) * a.T * a.dv + dcol0;
    E *ob = reinterpret_cast<E *>(a.out) + (row * a.Hv + head) * a.T * a.dv;

    if (wave >= 2) {
        // loader pair G = (wave - 2) / 2 copies the chunks j with j % R == G; the same barrier
        // sequence as the chain waves (one after the first copy, one per chunk)
        const int G = (wave - 2) >> 1;
        const int lt = tid - 128 * (G + 1);
        const char *wsk = reinterpret_cast<const char *>(a.ws);
        const E *vb = reinterpret_cast<const E *>(a.v) + v_off;
        const E *wb = reinterpret_cast<const E *>(a.w) + v_off;
        int kdst[CC::PK];
#pragma unroll
        for (int j = 0; j < CC::PK; ++j) {
            const int i = lt + j * CC::kLoaders;
            kdst[j] = i < CC::NKEY ? key_piece_dst<E, C, DK>(i) : -1;
        }
        uint4 rk[CC::PK], rv[CC::PV], rw[CC::PV];
        auto issue = [&](int64_t ch) __attribute__((always_inline)) {
            const char *kb = wsk + (ws_slot<C>(a, seq, ch) * a.Hk + kh) * WK::kBytes;
#pragma unroll
            for (int j = 0; j < CC::PK; ++j) {
                const int i = lt + j * CC::kLoaders;
                rk[j] = make_uint4(0, 0, 0, 0);
                if (i < CC::NKEY) rk[j] = *reinterpret_cast<const uint4 *>(kb + (int64_t)i * 16);
            }
#pragma unroll
            for (int j = 0; j < CC::PV; ++j) {
                const int i = lt + j * CC::kLoaders;
                rv[j] = make_uint4(0, 0, 0, 0);
                rw[j] = make_uint4(0, 0, 0, 0);
                if (i < CC::NV) {
                    const int r = i / (kDvTile / CC::EPP), p = i % (kDvTile / CC::EPP);
                    const int64_t pos = ch * C + r;
                    if (pos < sv.len) {
                        const int64_t off = sv.token(pos) * a.dv + p * CC::EPP;
                        rv[j] = *reinterpret_cast<const uint4 *>(vb + off);
                        rw[j] = *reinterpret_cast<const uint4 *>(wb + off);
                    }
                }
            }
        };
        auto store = [&](int64_t ch) __attribute__((always_inline)) {
            char *base = reinterpret_cast<char *>(&buf[ch & 1]);
#pragma unroll
            for (int j = 0; j < CC::PK; ++j)
                if (kdst[j] >= 0) *reinterpret_cast<uint4 *>(base + kdst[j]) = rk[j];
#pragma unroll
            for (int j = 0; j < CC::PV; ++j) {
                const int i = lt + j * CC::kLoaders;
                if (i < CC::NV) {
                    const int r = i / (kDvTile / CC::EPP), p = i % (kDvTile / CC::EPP);
                    uint4 piece;
                    const uint4 vv = rv[j], ww = rw[j];
                    E *pr = reinterpret_cast<E *>(&piece);
                    const E *ve = reinterpret_cast<const E *>(&vv);
                    const E *we = reinterpret_cast<const E *>(&ww);
#pragma unroll
                    for (int e = 0; e < CC::EPP; ++e) pr[e] = static_cast<E>(to_f(ve[e]) * to_f(we[e]));
                    *reinterpret_cast<uint4 *>(base + offsetof(CB, WV) + r * CB::UP * sizeof(E) + p * 16) = piece;
                }
            }
        };
        // chunk j is issued R steps before it is stored (at step j - 1, into buffer j & 1)
        if (G < nchunks) issue(G);
        if (G == 0 && nchunks > 0) {
            store(0);
            if (R < nchunks) issue(R);
        }
        __syncthreads();
        int turn = 1 % R;  // the pair whose chunk is stored in this step: (c + 1) % R
        for (int64_t c = 0; c < nchunks; ++c) {
            if (turn == G && c + 1 < nchunks) {
                store(c + 1);
                if (c + 1 + R < nchunks) issue(c + 1 + R);
            }
            turn = turn + 1 == R ? 0 : turn + 1;
            __syncthreads();
        }
        return;
    }

    // chain waves: 16 columns each
    const int lcol = wave * 16;
    const int dcol = dcol0 + lcol + cc;
    floatx4 H[HT];
#pragma unroll
    for (int t = 0; t < HT; ++t) H[t] = zero4();
    if (a.h0) {
        const float *hb = a.h0 + (seq * a.Hv + head) * DK * a.dv;
#pragma unroll
        for (int t = 0; t < HT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) H[t][r] = hb[(16 * t + 4 * g + r) * a.dv + dcol];
    }
    // The state's loads complete here. Otherwise the compiler's wait for them stays at the top
    // of the chunk loop, where on later chunks it would wait for the previous chunk's output
    // stores (loads and stores share one counter).
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    // output rows: token t0 + pos (t0 + len - 1 - pos reversed); a lane writes rows 4g + r of
    // each 16-row tile, column dcol
    const int64_t ostep = sv.rev ? -a.dv : a.dv;
    E *const ofirst = ob + (sv.rev ? sv.t0 + sv.len - 1 : sv.t0) * a.dv + dcol + 4 * g * ostep;
    __syncthreads();
    for (int64_t c = 0; c < nchunks; ++c) {
        const CB &cb = buf[c & 1];
        // every operand of the step read from LDS up front, so that the reads overlap each other
        // and the products below wait on them once rather than one at a time
        constexpr int NK = DK / 32;
        Frag<E> fw[NT][NK], fq[NT][NK];
#pragma unroll
        for (int ks = 0; ks < NK; ++ks)
#pragma unroll
            for (int mi = 0; mi < NT; ++mi) {
                fw[mi][ks] = frag_rows<E>(cb.W, CB::KP, 16 * mi, 32 * ks);
                fq[mi][ks] = frag_rows<E>(cb.Q, CB::KP, 16 * mi, 32 * ks);
            }
        floatx4 U[NT];
        // T (W * V): independent of the state
        if constexpr (C == 16) {
            U[0] = mma16(zero4(), frag_rows_lo<E>(cb.T, CB::CP, 0, 0), frag_cols_lo<E>(cb.WV, CB::UP, lcol, 0));
        } else {
            Frag<E> wv[NT / 2];
#pragma unroll
            for (int kc = 0; kc < NT / 2; ++kc) wv[kc] = frag_cols<E>(cb.WV, CB::UP, lcol, 32 * kc);
#pragma unroll
            for (int mi = 0; mi < NT; ++mi) {
                U[mi] = zero4();
#pragma unroll
                for (int kc = 0; kc <= mi / 2; ++kc) U[mi] = mma32(U[mi], frag_rows<E>(cb.T, CB::CP, 16 * mi, 32 * kc), wv[kc]);
            }
        }
        floatx4 XW[NT], XQ[NT];
#pragma unroll
        for (int mi = 0; mi < NT; ++mi) {
            XW[mi] = zero4();
            XQ[mi] = zero4();
        }
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) {
            const Frag<E> hb = frag_from_acc<E>(H[2 * ks], H[2 * ks + 1]);
#pragma unroll
            for (int mi = 0; mi < NT; ++mi) {
                XW[mi] = mma32(XW[mi], fw[mi][ks], hb);
                XQ[mi] = mma32(XQ[mi], fq[mi][ks], hb);
            }
        }
        // operands of the state update and the output, read while the products above run
        Frag<E> fk[HT][C >= 32 ? C / 32 : 1];
        typename Vec4<E>::type fk16[C == 16 ? HT : 1];
        floatx4 eg[HT];
#pragma unroll
        for (int t = 0; t < HT; ++t) {
            eg[t] = *reinterpret_cast<const floatx4 *>(cb.egc + 16 * t + 4 * g);
            if constexpr (C == 16) {
                fk16[t] = frag_rows_lo<E>(cb.Kt, CB::CP, 16 * t, 0);
            } else {
#pragma unroll
                for (int kc = 0; kc < C / 32; ++kc) fk[t][kc] = frag_rows<E>(cb.Kt, CB::CP, 16 * t, 32 * kc);
            }
        }
#pragma unroll
        for (int mi = 0; mi < NT; ++mi) U[mi] -= XW[mi];
        // H <- Diag(e^{G_C}) H + Kt U
#pragma unroll
        for (int t = 0; t < HT; ++t) {
            H[t] *= eg[t];
            if constexpr (C == 16) {
                H[t] = mma16(H[t], fk16[t], cvt4<E>(U[0]));
            } else {
#pragma unroll
                for (int kc = 0; kc < C / 32; ++kc) H[t] = mma32(H[t], fk[t][kc], frag_from_acc<E>(U[2 * kc], U[2 * kc + 1]));
            }
        }
        // O = Qc H + P U, stored (with accumulation, the previous values are read first, all
        // at once)
        E *orow = ofirst + c * C * ostep;
        floatx4 O[NT];
#pragma unroll
        for (int mi = 0; mi < NT; ++mi) {
            O[mi] = XQ[mi];
#pragma unroll
            for (int kt = 0; kt <= mi; kt += 2) {
                if (kt + 1 < NT)
                    O[mi] = mma32(O[mi], frag_rows<E>(cb.P, CB::CP, 16 * mi, 16 * kt), frag_from_acc<E>(U[kt], U[kt + 1]));
                else
                    O[mi] = mma16(O[mi], frag_rows_lo<E>(cb.P, CB::CP, 16 * mi, 16 * kt), cvt4<E>(U[kt]));
            }
        }
        if constexpr (kIsBf16<E>) {
            float *st = ostage + wave * kOutRows * kOutP;
#pragma unroll
            for (int rb = 0; rb < C; rb += kOutRows) {
#pragma unroll
            for (int mi = rb / 16; mi < (rb + kOutRows) / 16; ++mi)
#pragma unroll
                for (int r = 0; r < 4; ++r) st[(16 * mi - rb + 4 * g + r) * kOutP + cc] = O[mi][r];
            // two 8-column pieces per row; rows past the end of the sequence are not written
#pragma unroll
            for (int pi = lane; pi < 2 * kOutRows; pi += 64) {
                const int rr = pi >> 1, half = pi & 1;
                const int64_t pos = c * C + rb + rr;
                const float4 x0 = *reinterpret_cast<const float4 *>(st + rr * kOutP + 8 * half);
                const float4 x1 = *reinterpret_cast<const float4 *>(st + rr * kOutP + 8 * half + 4);
                if (pos < sv.len) {
                    bf16x8 *dst = reinterpret_cast<bf16x8 *>(ob + sv.token(pos) * a.dv + dcol0 + lcol + 8 * half);
                    float f[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
                    if (acc_out) {
                        const bf16x8 old = *dst;
#pragma unroll
                        for (int e = 0; e < 8; ++e) f[e] += (float)old[e];
                    }
                    bf16x8 val;
#pragma unroll
                    for (int e = 0; e < 8; ++e) val[e] = (__bf16)f[e];
                    *dst = val;
                }
            }
            }
        } else {
            const int64_t left = sv.len - c * C - 4 * g;  // rows 16 mi + r of this lane exist below left
            if (acc_out) {
#pragma unroll
                for (int mi = 0; mi < NT; ++mi)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (16 * mi + r < left) O[mi][r] += to_f(orow[(16 * mi + r) * ostep]);
            }
#pragma unroll
            for (int mi = 0; mi < NT; ++mi)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (16 * mi + r < left) orow[(16 * mi + r) * ostep] = static_cast<E>(O[mi][r]);
        }
        __syncthreads();
    }
    if (a.hT) {
        float *hb = a.hT + (seq * a.Hv + head) * DK * a.dv;
#pragma unroll
        for (int t = 0; t < HT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) hb[(16 * t + 4 * g + r) * a.dv + dcol] = H[t][r];
    }
}

template <typename E, int C, int DK>
hipError_t launch_two_pass(const Gdn2Args &a, hipStream_t stream) {
    const int64_t prep_blocks = a.nslots * a.Hk;
    if (prep_blocks > 0) {
        hipLaunchKernelGGL((gdn2_prep_kernel<E, C, DK>), dim3((unsigned)prep_blocks), dim3(kThreads), 0, stream, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t blocks = (a.units + 7) / 8 * 8 * a.ntiles;
    hipLaunchKernelGGL((gdn2_chain_kernel<E, C, DK>), dim3((unsigned)blocks), dim3(64 * ChainCopy<E, C, DK>::kWaves), 0,
                       stream, a);
    return hipGetLastError();
}

template <typename E, int C, int DK>
hipError_t launch_typed(const Gdn2Args &a, hipStream_t stream) {
    const int64_t groups = (a.units + 7) / 8;
    const int64_t blocks = groups * 8 * a.ntiles;
    hipLaunchKernelGGL((gdn2_chunk_kernel<E, C, DK>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

// without a workspace the fused one-pass kernel, with one the two passes
template <typename E, int C, int DK>
hipError_t launch_form(const Gdn2Args &a, hipStream_t stream) {
    static_assert(WsKey<E, C, DK>::kBytes % 16 == 0, "workspace blocks keep 16-byte alignment");
    // fp32 with 64-token chunks: the chain's two operand buffers do not fit in LDS; the one-pass
    // kernel serves it whether or not a workspace is given
    if constexpr (ChainCopy<E, C, DK>::kFits) {
        if (a.ws) return launch_two_pass<E, C, DK>(a, stream);
    }
    return launch_typed<E, C, DK>(a, stream);
}

}  // namespace

bool gdn2_chunk_supported(int dtype, int chunk, int dk) {
    if (chunk != 16 && chunk != 32 && chunk != 64) return false;
    if (dk != 64 && dk != 128) return false;
    return !(dtype == kDtypeF32 && dk == 128 && chunk == 64);  // does not fit in LDS
}

hipError_t launch_gdn2_chunk_fwd(const Gdn2Args &a, int dtype, int chunk, int dk, hipStream_t s) {
    if (a.units == 0 || a.ntiles == 0) return hipSuccess;
    if (!gdn2_chunk_supported(dtype, chunk, dk)) return hipErrorInvalidValue;
    if (dtype == kDtypeBf16) {
        if (dk == 64) {
            if (chunk == 16) return launch_form<__bf16, 16, 64>(a, s);
            if (chunk == 32) return launch_form<__bf16, 32, 64>(a, s);
            return launch_form<__bf16, 64, 64>(a, s);
        }
        if (chunk == 16) return launch_form<__bf16, 16, 128>(a, s);
        if (chunk == 32) return launch_form<__bf16, 32, 128>(a, s);
        return launch_form<__bf16, 64, 128>(a, s);
    }
    if (dk == 64) {
        if (chunk == 16) return launch_form<float, 16, 64>(a, s);
        if (chunk == 32) return launch_form<float, 32, 64>(a, s);
        return launch_form<float, 64, 64>(a, s);
    }
    if (chunk == 16) return launch_form<float, 16, 128>(a, s);
    return launch_form<float, 32, 128>(a, s);
}

int64_t gdn2_ws_key_bytes(int dtype, int chunk, int dk) {
    const int64_t es = dtype == kDtypeBf16 ? 2 : 4;
    return es * (3 * (int64_t)chunk * dk + 2 * (int64_t)chunk * chunk) + 4 * (int64_t)dk;
}

}  // namespace gdr
