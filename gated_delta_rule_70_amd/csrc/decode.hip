// One-token recurrent decode step on gfx950.
//
// One workgroup of 256 threads per (sequence, value head) state H [d_k][d_v] (fp32).
// From the old state, in one pass over its elements (the algebra of the recurrence
// in the "Prizma seq/delta.py" module docstring, rearranged so that H is touched once):
//
//   x = H^T k,  y = H^T q,  u = beta (v - alpha x),  H' = alpha H + k u^T
//   o = alpha y + (k . q) u   (post-write read: H'^T q),   o = y  (pre-write read)
//
// Each thread owns 4 adjacent columns of a band of rows and keeps its elements in
// registers between the read and the write, so state_out may equal state_in. The
// state is streamed once in and once out with 16-byte non-temporal accesses: the
// kernel is bound by HBM bandwidth, and the reductions over d_k go through LDS.
//
// With unit-norm rows requested, q and k enter as r_q q and r_k k (r = 1 / max(||row||,
// eps)); the scales are applied to the reduced x, y and k.q and to u in the update, so the
// raw vectors are never rewritten. With raw gates, log alpha and beta are formed here.
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
__device__ __forceinline__ void st_f(float *p, int64_t i, float x) { p[i] = x; }
__device__ __forceinline__ void st_f(__bf16 *p, int64_t i, float x) { p[i] = (__bf16)x; }

template <typename E, int DK, int DV>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
    constexpr int CG = DV / 4;          // column groups of 4 (threads per row band)
    constexpr int RG = kThreads / CG;   // row bands
    constexpr int RPT = DK / RG;        // rows per thread
    static_assert(RPT * RG == DK && CG * RG == kThreads, "tile shape");

    __shared__ float sk[DK], sq[DK], sv[DV];
    __shared__ f4 px[RG][CG], py[RG][CG];
    __shared__ float skq, srk, srq;

    const int tid = threadIdx.x;
    const int cg = tid % CG, rg = tid / CG;
    const int64_t w = blockIdx.x;  // (sequence, value head)
    const int64_t n = w / a.Hv, head = w % a.Hv;
    const int64_t kh = head / (a.Hv / a.Hk);

    const f4 *sin = reinterpret_cast<const f4 *>(a.state_in + w * DK * DV);
    f4 *sout = reinterpret_cast<f4 *>(a.state_out + w * DK * DV);

    // issue the state loads first: they are the bulk of the traffic
    f4 h[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) h[i] = __builtin_nontemporal_load(sin + (rg * RPT + i) * CG + cg);

    const E *qp = reinterpret_cast<const E *>(a.q) + (n * a.Hk + kh) * DK;
    const E *kp = reinterpret_cast<const E *>(a.k) + (n * a.Hk + kh) * DK;
    const E *vp = reinterpret_cast<const E *>(a.v) + w * DV;
    for (int i = tid; i < DK; i += kThreads) {
        sk[i] = ld_f(kp, i);
        sq[i] = ld_f(qp, i);
    }
    for (int i = tid; i < DV; i += kThreads) sv[i] = ld_f(vp, i);
    const float alpha = __expf(a.A_log ? gate_log_alpha(a.log_alpha[w], a.A_log, a.dt_bias, head) : a.log_alpha[w]);
    const float beta = a.A_log ? gate_beta(a.beta[w]) : a.beta[w];
    const bool l2 = (a.flags & kFlagL2Norm) != 0;
    __syncthreads();

    if (tid < 64) {  // k . q, and the row norms, by wave 0
        float s = 0.f, skk = 0.f, sqq = 0.f;
        for (int i = tid; i < DK; i += 64) {
            s += sk[i] * sq[i];
            skk += sk[i] * sk[i];
            sqq += sq[i] * sq[i];
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            s += __shfl_xor(s, off, 64);
            skk += __shfl_xor(skk, off, 64);
            sqq += __shfl_xor(sqq, off, 64);
        }
        if (tid == 0) {
            const float rk = l2 ? 1.f / fmaxf(sqrtf(skk), kL2Eps) : 1.f;
            const float rq = l2 ? 1.f / fmaxf(sqrtf(sqq), kL2Eps) : 1.f;
            skq = s * rk * rq;
            srk = rk;
            srq = rq;
        }
    }

    f4 x = {0.f, 0.f, 0.f, 0.f}, y = x;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        x += h[i] * sk[rg * RPT + i];
        y += h[i] * sq[rg * RPT + i];
    }
    px[rg][cg] = x;
    py[rg][cg] = y;
    __syncthreads();
    x = f4{0.f, 0.f, 0.f, 0.f};
    y = x;
#pragma unroll
    for (int j = 0; j < RG; ++j) {
        x += px[j][cg];
        y += py[j][cg];
    }
    const float rk = srk, rq = srq;
    x *= rk;  // x = H^T k with the normalised k
    y *= rq;
    const f4 v4 = {sv[4 * cg], sv[4 * cg + 1], sv[4 * cg + 2], sv[4 * cg + 3]};
    const f4 u = beta * (v4 - alpha * x);
    const f4 uk = rk * u;  // the normalised k's scale, moved onto u for the update

#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const f4 r = alpha * h[i] + sk[rg * RPT + i] * uk;
        __builtin_nontemporal_store(r, sout + (rg * RPT + i) * CG + cg);
    }
    if (rg == 0) {
        E *op = reinterpret_cast<E *>(a.out) + w * DV + 4 * cg;
        const bool pre = (a.flags & kFlagReadPre) != 0;
        const float kq = skq;
        const f4 o = pre ? y : alpha * y + kq * u;
#pragma unroll
        for (int c = 0; c < 4; ++c) st_f(op, c, o[c]);
    }
}

template <typename E, int DK, int DV>
hipError_t launch_t(const DecodeArgs &a, hipStream_t s) {
    const int64_t blocks = a.N * a.Hv;
    hipLaunchKernelGGL((decode_kernel<E, DK, DV>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <typename E>
hipError_t launch_e(const DecodeArgs &a, int dk, int dv, hipStream_t s) {
    if (dk == 64) return dv == 64 ? launch_t<E, 64, 64>(a, s) : launch_t<E, 64, 128>(a, s);
    return dv == 64 ? launch_t<E, 128, 64>(a, s) : launch_t<E, 128, 128>(a, s);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, int dtype, int dk, int dv, hipStream_t stream) {
    if (a.N == 0) return hipSuccess;
    if (dtype == kDtypeBf16) return launch_e<__bf16>(a, dk, dv, stream);
    return launch_e<float>(a, dk, dv, stream);
}

}  // namespace gdr
