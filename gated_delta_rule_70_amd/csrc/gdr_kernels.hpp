// Host-side launch interface between the C ABI (gdr_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

constexpr uint32_t kFlagReadPre = 1u;
constexpr uint32_t kFlagReverse = 2u;
constexpr uint32_t kFlagAccumulate = 4u;
constexpr uint32_t kFlagL2Norm = 8u;  // q and k rows divided by max(||row||, kL2Eps) first
constexpr float kL2Eps = 1e-6f;
constexpr int kDtypeF32 = 0;
constexpr int kDtypeBf16 = 1;

// With A_log (and dt_bias) set, log_alpha and beta hold the raw gate inputs a and b and the
// kernels form log alpha = -exp(A_log[h]) softplus(a + dt_bias[h]) and beta = sigmoid(b).
struct ChunkArgs {
    const void *q, *k, *v;
    const float *log_alpha, *beta, *h0;
    const float *A_log, *dt_bias;
    const int32_t *cu_seqlens;
    void *out;
    float *hT;
    int64_t B, T, Hk, Hv, dv;
    int64_t units;   // sequences x value heads
    int64_t ntiles;  // dv / 32
    uint32_t flags;
    // delta sub-steps per token (DeltaProduct; 1 for the plain rule): k, v and beta hold n_sub
    // rows per token ([..][T][n_sub][..]); the fast kernel serves powers of two, the generic
    // kernel any count
    int32_t n_sub;
};

struct DecodeArgs {
    const void *q, *k, *v;
    const float *log_alpha, *beta;
    const float *A_log, *dt_bias;  // as in ChunkArgs
    const float *state_in;
    float *state_out;
    void *out;
    int64_t N, Hk, Hv;
    uint32_t flags;
};

// GDN-2: g [B][Hk][T][dk] fp32 log decay per key channel, b [B][Hk][T][dk] erase gate and
// w [B][Hv][T][dv] write gate in the element type of q, k, v.
struct Gdn2Args {
    const void *q, *k, *v, *b, *w;
    const float *g, *h0;
    const int32_t *cu_seqlens;
    void *out;
    float *hT;
    int64_t B, T, Hk, Hv, dv;
    int64_t units;   // sequences x value heads
    int64_t ntiles;  // dv / 32
    uint32_t flags;
    // two-pass form (ws non-null): a block per (chunk slot, key head)
    void *ws;
    int64_t nslots;
};

// GDN-2 decode: g, b [N][Hk][dk] (g fp32), w [N][Hv][dv].
struct Gdn2DecodeArgs {
    const void *q, *k, *v, *b, *w;
    const float *g;
    const float *state_in;
    float *state_out;
    void *out;
    int64_t N, Hk, Hv;
    uint32_t flags;
};

// Backward of the scalar rule. Gradient buffers are fp32: dq, dk [B][Hk][T][dk] (summed over the
// value heads of a key head), dv [B][Hv][T][dv], dlog_alpha, dbeta [B][Hv][T], dh0 like h0.
// The workspace holds, per chunk slot of every value head (nslots per head, kBwdBlock tokens per
// chunk): a record of kBwdRecBytes (the chunk's inverse and read matrix as matrix-core
// operands, and its gate cumsums), the entry state hs and the exit-state adjoint ds
// of the chunk (per kBwdCols-column slice, kBwdCols x dk fp32 each, transposed); and us, drs
// [Hv][nslots][kBwdBlock][dv] fp32, the chunk form's U and dR of every chunk (rows past a
// segment's end hold zeros).
constexpr int kBwdBlock = 64;
constexpr int kBwdCols = 32;  // value columns per workgroup of the state sweeps
constexpr int64_t kBwdRecBytes = 3 * 16384 + 2 * kBwdBlock * 4;
struct BwdArgs {
    const void *q, *k, *v, *dout;
    const float *log_alpha, *beta, *h0, *dhT;
    const int32_t *cu_seqlens;
    float *dq, *dk, *dv, *dlog_alpha, *dbeta, *dh0;
    uint8_t *rec;
    float *hs, *ds, *us, *drs;
    int64_t B, T, Hk, Hv;
    int64_t nseq;    // sequences (B, or the packed segments)
    int64_t units;   // sequences x value heads
    int64_t nslots;  // chunk slots per value head
    int64_t ntiles;  // dv / kBwdCols
    uint32_t flags;
};

hipError_t launch_chunk_fwd(const ChunkArgs &a, int dtype, int chunk, int dk, hipStream_t stream);
bool chunk_fwd_fast_supported(int dtype, int chunk, int dk);
hipError_t launch_chunk_fwd_fast(const ChunkArgs &a, hipStream_t stream);
bool gdn2_chunk_supported(int dtype, int chunk, int dk);
hipError_t launch_gdn2_chunk_fwd(const Gdn2Args &a, int dtype, int chunk, int dk, hipStream_t stream);
// bytes of one (chunk, key head) block of the two-pass workspace
int64_t gdn2_ws_key_bytes(int dtype, int chunk, int dk);
hipError_t launch_gdn2_decode(const Gdn2DecodeArgs &a, int dtype, int dk, int dv, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs &a, int dtype, int dk, int dv, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &a, int dtype, int dk, int dv, hipStream_t stream);
// softplus without overflow: max(x, 0) + log(1 + e^{-|x|}); the second term is below 2^-24
// (and lost next to 1) only where it is negligible against the first or is itself < 6e-8
__device__ __forceinline__ float softplus_f(float x) { return fmaxf(x, 0.f) + __logf(1.f + __expf(-fabsf(x))); }
// the gates of one token of value head h from their raw inputs (see ChunkArgs)
__device__ __forceinline__ float gate_log_alpha(float a, const float *A_log, const float *dt_bias, int64_t h) {
    const float x = a + dt_bias[h];
    return -__expf(A_log[h]) * softplus_f(x);
}
__device__ __forceinline__ float gate_beta(float b) { return __builtin_amdgcn_rcpf(1.f + __expf(-b)); }

hipError_t launch_selftest_mfma(const float *a, const float *b, float *d, hipStream_t stream);

// Size of the fixed device scratch of the allocation-free entry points (one copy per GPU).
constexpr int64_t kScratchBytes = INT64_C(64) << 20;
// Its device address on the current device (looked up on the first call per device).
hipError_t scratch_region(void **ptr);

}  // namespace gdr
