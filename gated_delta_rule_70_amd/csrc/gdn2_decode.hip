// One-token GDN-2 decode step on gfx950 (the update of BidirectionalGatedDeltaNet2 on the
// "tiny_gdn/fugue.py" page for a single token, state H = S^T [d_k][d_v] in fp32).
//
// With a_c = e^{g_c} per key channel, the erase gate b and the write gate w, in one pass over
// the old state:
//
//   x = H^T (a * b * k),   u = w * v - x,   H' = Diag(a) H + k u^T
//   o = H^T (a * q) + (k . q) u   (post-write read: H'^T q),   o = H^T q   (pre-write read)
//
// The thread layout follows the scalar decode step: one workgroup of 256 threads per
// (sequence, value head); each thread keeps 4 adjacent columns of a band of rows in registers
// between the read and the write, so state_out may equal state_in, and the state streams once
// in and once out with 16-byte non-temporal accesses (the step is bound by HBM bandwidth).
// With unit-norm rows requested, the scales of q and k are applied to the reduced sums and to
// u in the update, as in the scalar step.
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
__global__ __launch_bounds__(kThreads) void gdn2_decode_kernel(Gdn2DecodeArgs a) {
    constexpr int CG = DV / 4;
    constexpr int RG = kThreads / CG;
    constexpr int RPT = DK / RG;
    static_assert(RPT * RG == DK && CG * RG == kThreads, "tile shape");

    __shared__ float sk[DK], sx[DK], sy[DK], sa[DK], su[DV];
    __shared__ f4 px[RG][CG], py[RG][CG];
    __shared__ float skq, srk, srq;

    const int tid = threadIdx.x;
    const int cg = tid % CG, rg = tid / CG;
    const int64_t w = blockIdx.x;  // (sequence, value head)
    const int64_t n = w / a.Hv, head = w % a.Hv;
    const int64_t kh = head / (a.Hv / a.Hk);
    const bool pre = (a.flags & kFlagReadPre) != 0;
    const bool l2 = (a.flags & kFlagL2Norm) != 0;

    const f4 *sin = reinterpret_cast<const f4 *>(a.state_in + w * DK * DV);
    f4 *sout = reinterpret_cast<f4 *>(a.state_out + w * DK * DV);
    f4 h[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) h[i] = __builtin_nontemporal_load(sin + (rg * RPT + i) * CG + cg);

    const int64_t kq = (n * a.Hk + kh) * DK;
    const E *qp = reinterpret_cast<const E *>(a.q) + kq;
    const E *kp = reinterpret_cast<const E *>(a.k) + kq;
    const E *bp = reinterpret_cast<const E *>(a.b) + kq;
    const float *gp = a.g + kq;
    const E *vp = reinterpret_cast<const E *>(a.v) + w * DV;
    const E *wp = reinterpret_cast<const E *>(a.w) + w * DV;
    // per key channel: the read vectors a*b*k (x) and a*q or q (y), and a for the update
    for (int i = tid; i < DK; i += kThreads) {
        const float kk = ld_f(kp, i), qq = ld_f(qp, i), ai = __expf(gp[i]);
        sk[i] = kk;
        sa[i] = ai;
        sx[i] = ai * ld_f(bp, i) * kk;
        sy[i] = pre ? qq : ai * qq;
    }
    for (int i = tid; i < DV; i += kThreads) su[i] = ld_f(wp, i) * ld_f(vp, i);
    __syncthreads();

    if (tid < 64) {  // k . q and the row norms, by wave 0 (q is recovered from y where needed)
        float s = 0.f, skk = 0.f, sqq = 0.f;
        for (int i = tid; i < DK; i += 64) {
            const float qq = ld_f(qp, i);
            s += sk[i] * qq;
            skk += sk[i] * sk[i];
            sqq += qq * qq;
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
        x += h[i] * sx[rg * RPT + i];
        y += h[i] * sy[rg * RPT + i];
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
    x *= rk;
    y *= rq;
    const f4 wv = {su[4 * cg], su[4 * cg + 1], su[4 * cg + 2], su[4 * cg + 3]};
    const f4 u = wv - x;
    const f4 uk = rk * u;

#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg * RPT + i;
        const f4 nh = sa[r] * h[i] + sk[r] * uk;
        __builtin_nontemporal_store(nh, sout + r * CG + cg);
    }
    if (rg == 0) {
        E *op = reinterpret_cast<E *>(a.out) + w * DV + 4 * cg;
        const f4 o = pre ? y : y + skq * u;
#pragma unroll
        for (int c = 0; c < 4; ++c) st_f(op, c, o[c]);
    }
}

template <typename E, int DK, int DV>
hipError_t launch_t(const Gdn2DecodeArgs &a, hipStream_t s) {
    hipLaunchKernelGGL((gdn2_decode_kernel<E, DK, DV>), dim3((unsigned)(a.N * a.Hv)), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <typename E>
hipError_t launch_e(const Gdn2DecodeArgs &a, int dk, int dv, hipStream_t s) {
    if (dk == 64) return dv == 64 ? launch_t<E, 64, 64>(a, s) : launch_t<E, 64, 128>(a, s);
    return dv == 64 ? launch_t<E, 128, 64>(a, s) : launch_t<E, 128, 128>(a, s);
}

}  // namespace

hipError_t launch_gdn2_decode(const Gdn2DecodeArgs &a, int dtype, int dk, int dv, hipStream_t stream) {
    if (a.N == 0) return hipSuccess;
    if (dtype == kDtypeBf16) return launch_e<__bf16>(a, dk, dv, stream);
    return launch_e<float>(a, dk, dv, stream);
}

}  // namespace gdr
