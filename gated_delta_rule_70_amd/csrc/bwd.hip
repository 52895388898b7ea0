// Backward of the gated delta rule on gfx950: gradients of the outputs and final state with
// respect to q, k, v, log alpha, beta and h0, by the adjoint of the per-token recurrence
// (H = S^T [d_k][d_v], alpha = e^{log alpha}):
//
//   forward   x = H^T k,  u = beta (v - alpha x),  H' = alpha H + k u^T,  o = H'^T q (or H^T q)
//   adjoint   (dH' += q do^T for the post-write read)
//             du = dH'^T k,  dv = beta du,  dbeta = du . (v - alpha x),  dx = -alpha beta du
//             dk = dH' u + H dx,  dq = H' do (post) or H do (pre)
//             dlog alpha = alpha (<dH', H> - beta du . x)
//             dH = alpha dH' + k dx^T   (+ q do^T for the pre-write read)
//
// The pages print no backward; this is the derivative of the recurrence they define (the
// "Prizma seq/delta.py" page requires forward and gradient agreement with it).
//
// One workgroup of 256 threads per (sequence, value head, 32 columns of d_v), with the state
// layout of the decode step: each thread holds 4 adjacent columns of a band of rows of its slice
// of the state H and of the adjoint dH in registers. Every quantity of the recurrence is either
// per column (x, u, du, dv) or a sum over columns of per-column terms (dq, dk, the scalars of
// dbeta and dlog alpha), so the column slices run independently and add their partial sums with
// float atomics into buffers a fill kernel clears first (this also sums dq and dk over the value
// heads that share a key head). Reductions over rows go through LDS (one barrier per token, the
// partials double-buffered: each wave first adds its bands with lane shuffles); reductions over
// the slice's columns stay inside a row band (8 lanes) as lane shuffles. Three sweeps per sequence: a forward sweep that stores the slice of
// the state at the start of every 32-token block in the workspace; then, block by block from the
// last, a forward recompute that stores the slice before each token of the block (workspace),
// and the reverse adjoint sweep over the block.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "gdr_kernels.hpp"

namespace gdr {

namespace {

constexpr int kThreads = 256;
typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float ld_f(const float *p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld_f(const __bf16 *p, int64_t i) { return (float)p[i]; }

struct Seq {
    int64_t t0, len;
    bool rev;
    __device__ __forceinline__ int64_t token(int64_t pos) const { return rev ? t0 + len - 1 - pos : t0 + pos; }
};

// sum over the `width` lanes of a row band (width a power of two, bands aligned)
template <int W>
__device__ __forceinline__ float band_sum(float x) {
#pragma unroll
    for (int off = 1; off < W; off <<= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// sum over the row bands of one wave: the lanes with the same lane % W (W lanes per band)
template <int W>
__device__ __forceinline__ f4 wave_bands_sum(f4 v) {
#pragma unroll
    for (int off = W; off < 64; off <<= 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += __shfl_xor(v[e], off, 64);
    }
    return v;
}

template <typename E, int DK>
__global__ __launch_bounds__(kThreads) void bwd_kernel(BwdArgs a) {
    constexpr int DV = kBwdCols;       // columns of the slice
    constexpr int CG = DV / 4;         // threads per row band (4 columns each)
    constexpr int RG = kThreads / CG;  // row bands
    constexpr int RPT = DK / RG;       // rows per thread
    constexpr int CB = kBwdBlock;
    static_assert(RPT * RG == DK && CG * RG == kThreads && CG <= 64, "tile shape");

    __shared__ float sk[CB][DK], sq[CB][DK], sv[CB][DV], sdo[CB][DV];
    __shared__ float sal[CB], sbe[CB];
    constexpr int NW = kThreads / 64;  // waves; row sums are reduced per wave first, then over waves
    __shared__ f4 px[2][NW][CG], pd[2][NW][CG];
    __shared__ float pw[2][NW];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cg = tid % CG, rg = tid / CG;
    const int64_t unit = blockIdx.x / a.ntiles;
    const int tile = (int)(blockIdx.x % a.ntiles);
    const int64_t dvf = a.ntiles * DV;  // full d_v
    const int col0 = tile * DV;
    const int64_t seq = unit / a.Hv, head = unit % a.Hv;
    const int64_t kh = head / (a.Hv / a.Hk);
    const int64_t row = a.cu_seqlens ? 0 : seq;
    const bool pre = (a.flags & kFlagReadPre) != 0;
    Seq span;
    span.t0 = 0;
    span.len = a.T;
    int64_t slot0 = seq * ((a.T + CB - 1) / CB);
    if (a.cu_seqlens) {
        span.t0 = a.cu_seqlens[seq];
        span.len = a.cu_seqlens[seq + 1] - span.t0;
        slot0 = span.t0 / CB + seq;
    }
    span.rev = (a.flags & kFlagReverse) != 0;
    const int64_t nblk = (span.len + CB - 1) / CB;

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
    // states in the workspace: [head][slot][tile] and [unit][token of the block][tile] slices
    const int64_t st = DK * DV / 4;  // f4 per slice
    f4 *ckpt = reinterpret_cast<f4 *>(a.ws) + ((head * a.nslots + slot0) * a.ntiles + tile) * st;
    f4 *cbuf = reinterpret_cast<f4 *>(a.ws) + ((a.Hv * a.nslots + unit * CB) * a.ntiles + tile) * st;
    const int64_t sstride = a.ntiles * st;  // from one slot (or token) to the next

    // stage block b of the scan into LDS (the inputs the sweeps read token by token)
    auto stage = [&](int64_t blk, bool adjoint) {
        const int64_t n = min((int64_t)CB, span.len - blk * CB);
        for (int i = tid; i < CB * DK; i += kThreads) {
            const int r = i / DK, c = i % DK;
            const int64_t t = r < n ? span.token(blk * CB + r) : 0;
            sk[r][c] = r < n ? ld_f(kb, t * DK + c) : 0.f;
            if (adjoint) sq[r][c] = r < n ? ld_f(qb, t * DK + c) : 0.f;
        }
        for (int i = tid; i < CB * DV; i += kThreads) {
            const int r = i / DV, c = i % DV;
            const int64_t t = r < n ? span.token(blk * CB + r) : 0;
            sv[r][c] = r < n ? ld_f(vb, t * dvf + c) : 0.f;
            if (adjoint) sdo[r][c] = r < n ? ld_f(dob, t * dvf + c) : 0.f;
        }
        if (tid < CB) {
            const int64_t t = tid < n ? span.token(blk * CB + tid) : 0;
            sal[tid] = tid < n ? __expf(lab[t]) : 1.f;
            sbe[tid] = tid < n ? beb[t] : 0.f;
        }
    };

    int buf = 0;
    // one token of the forward recurrence on the registers h (token i of the staged block)
    auto forward_step = [&](f4 *h, int i) {
        f4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < RPT; ++r) x += h[r] * sk[i][rg * RPT + r];
        x = wave_bands_sum<CG>(x);
        if (lane < CG) px[buf][wave][cg] = x;
        __syncthreads();
        x = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < NW; ++j) x += px[buf][j][cg];
        buf ^= 1;
        const float al = sal[i], be = sbe[i];
        const f4 v4 = {sv[i][4 * cg], sv[i][4 * cg + 1], sv[i][4 * cg + 2], sv[i][4 * cg + 3]};
        const f4 u = be * (v4 - al * x);
#pragma unroll
        for (int r = 0; r < RPT; ++r) h[r] = al * h[r] + sk[i][rg * RPT + r] * u;
    };

    f4 h[RPT];
    // element (row, col0 + 4 cg) of this unit's full [dk][dv] state, in f4 units
    const int64_t sbase = (seq * a.Hv + head) * (DK * dvf / 4) + col0 / 4 + cg;
    const int64_t srow = dvf / 4;
#pragma unroll
    for (int r = 0; r < RPT; ++r)
        h[r] = a.h0 ? reinterpret_cast<const f4 *>(a.h0)[sbase + (rg * RPT + r) * srow] : f4{0.f, 0.f, 0.f, 0.f};

    // sweep 1: states at the block starts
    for (int64_t blk = 0; blk < nblk; ++blk) {
#pragma unroll
        for (int r = 0; r < RPT; ++r) ckpt[blk * sstride + (rg * RPT + r) * CG + cg] = h[r];
        stage(blk, false);
        __syncthreads();
        const int n = (int)min((int64_t)CB, span.len - blk * CB);
        for (int i = 0; i < n; ++i) forward_step(h, i);
        __syncthreads();
    }

    // sweeps 2 and 3, block by block from the last
    f4 g[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r)
        g[r] = a.dhT ? reinterpret_cast<const f4 *>(a.dhT)[sbase + (rg * RPT + r) * srow] : f4{0.f, 0.f, 0.f, 0.f};
    for (int64_t blk = nblk - 1; blk >= 0; --blk) {
        stage(blk, true);
        __syncthreads();
        const int n = (int)min((int64_t)CB, span.len - blk * CB);
#pragma unroll
        for (int r = 0; r < RPT; ++r) h[r] = ckpt[blk * sstride + (rg * RPT + r) * CG + cg];
        for (int i = 0; i < n; ++i) {
#pragma unroll
            for (int r = 0; r < RPT; ++r) cbuf[i * sstride + (rg * RPT + r) * CG + cg] = h[r];
            forward_step(h, i);
        }
        for (int i = n - 1; i >= 0; --i) {
#pragma unroll
            for (int r = 0; r < RPT; ++r) h[r] = cbuf[i * sstride + (rg * RPT + r) * CG + cg];  // state before token i
            const float al = sal[i], be = sbe[i];
            const f4 do4 = {sdo[i][4 * cg], sdo[i][4 * cg + 1], sdo[i][4 * cg + 2], sdo[i][4 * cg + 3]};
            const f4 v4 = {sv[i][4 * cg], sv[i][4 * cg + 1], sv[i][4 * cg + 2], sv[i][4 * cg + 3]};
            if (!pre) {
#pragma unroll
                for (int r = 0; r < RPT; ++r) g[r] += sq[i][rg * RPT + r] * do4;
            }
            // row reductions: x = H^T k, du = dH'^T k; and <dH', H>
            f4 xp = {0.f, 0.f, 0.f, 0.f}, dp = xp;
            float hd = 0.f;
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
                const float kr = sk[i][rg * RPT + r];
                xp += h[r] * kr;
                dp += g[r] * kr;
                const f4 m = g[r] * h[r];
                hd += m[0] + m[1] + m[2] + m[3];
            }
            xp = wave_bands_sum<CG>(xp);
            dp = wave_bands_sum<CG>(dp);
            if (lane < CG) {
                px[buf][wave][cg] = xp;
                pd[buf][wave][cg] = dp;
            }
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) hd += __shfl_xor(hd, off, 64);
            if (lane == 0) pw[buf][wave] = hd;
            __syncthreads();
            f4 x = {0.f, 0.f, 0.f, 0.f}, du = x;
#pragma unroll
            for (int j = 0; j < NW; ++j) {
                x += px[buf][j][cg];
                du += pd[buf][j][cg];
            }
            hd = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) hd += pw[buf][w];
            buf ^= 1;
            const f4 e = v4 - al * x;
            const f4 u = be * e;
            const f4 dx = -al * be * du;
            // scalars over the columns of the row band (the same in every band)
            const f4 m1 = u * do4, m2 = du * e, m3 = du * x;
            const float s_udo = band_sum<CG>(m1[0] + m1[1] + m1[2] + m1[3]);
            const float s_due = band_sum<CG>(m2[0] + m2[1] + m2[2] + m2[3]);
            const float s_dux = band_sum<CG>(m3[0] + m3[1] + m3[2] + m3[3]);
            const int64_t t = span.token(blk * CB + i);
            // per row: dq = H' do (post) or H do (pre); dk = dH' u + H dx
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
                const f4 mq = h[r] * do4;
                const f4 mk = g[r] * u + h[r] * dx;
                float q_r = band_sum<CG>(mq[0] + mq[1] + mq[2] + mq[3]);
                const float k_r = band_sum<CG>(mk[0] + mk[1] + mk[2] + mk[3]);
                const int rr = rg * RPT + r;
                if (!pre) q_r = al * q_r + sk[i][rr] * s_udo;
                if (cg == 0) {
                    atomicAdd(dqb + t * DK + rr, q_r);
                    atomicAdd(dkb + t * DK + rr, k_r);
                }
            }
            if (rg == 0) {
                const f4 dvv = be * du;
#pragma unroll
                for (int c = 0; c < 4; ++c) dvb[t * dvf + 4 * cg + c] = dvv[c];
            }
            if (tid == 0) {  // this slice's share of the sums over columns
                atomicAdd(dbeb + t, s_due);
                atomicAdd(dlab + t, al * (hd - be * s_dux));
            }
            // dH = alpha dH' + k dx^T (+ q do^T for the pre-write read)
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
                const int rr = rg * RPT + r;
                g[r] = al * g[r] + sk[i][rr] * dx;
                if (pre) g[r] += sq[i][rr] * do4;
            }
        }
        __syncthreads();
    }
    if (a.dh0) {
#pragma unroll
        for (int r = 0; r < RPT; ++r) reinterpret_cast<f4 *>(a.dh0)[sbase + (rg * RPT + r) * srow] = g[r];
    }
}

__global__ void zero_kernel(float *p, int64_t n) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0.f;
}

template <typename E, int DK>
hipError_t launch_t(const BwdArgs &a, hipStream_t s) {
    hipLaunchKernelGGL((bwd_kernel<E, DK>), dim3((unsigned)(a.units * a.ntiles)), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <typename E>
hipError_t launch_e(const BwdArgs &a, int dk, hipStream_t s) {
    return dk == 64 ? launch_t<E, 64>(a, s) : launch_t<E, 128>(a, s);
}

}  // namespace

// clear n floats with a kernel (not a memset node, so the call stays safe to capture in a graph)
hipError_t clear(float *p, int64_t n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = (n + 255) / 256;
    const unsigned grid = (unsigned)(blocks < 4096 ? blocks : 4096);
    hipLaunchKernelGGL(zero_kernel, dim3(grid), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs &a, int dtype, int dk, int dv, hipStream_t stream) {
    (void)dv;
    // the sums over columns and value heads start from zero
    hipError_t e;
    if ((e = clear(a.dq, a.B * a.Hk * a.T * dk, stream)) != hipSuccess) return e;
    if ((e = clear(a.dk, a.B * a.Hk * a.T * dk, stream)) != hipSuccess) return e;
    if ((e = clear(a.dlog_alpha, a.B * a.Hv * a.T, stream)) != hipSuccess) return e;
    if ((e = clear(a.dbeta, a.B * a.Hv * a.T, stream)) != hipSuccess) return e;
    if (a.units == 0) return hipSuccess;
    if (dtype == kDtypeBf16) return launch_e<__bf16>(a, dk, stream);
    return launch_e<float>(a, dk, stream);
}

}  // namespace gdr
