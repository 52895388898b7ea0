// Host-side launch interface between the C ABI (gdr_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

constexpr uint32_t kFlagReadPre = 1u;
constexpr uint32_t kFlagReverse = 2u;
constexpr uint32_t kFlagAccumulate = 4u;
constexpr int kDtypeF32 = 0;
constexpr int kDtypeBf16 = 1;

struct ChunkArgs {
    const void *q, *k, *v;
    const float *log_alpha, *beta, *h0;
    const int32_t *cu_seqlens;
    void *out;
    float *hT;
    int64_t B, T, Hk, Hv, dv;
    int64_t units;   // sequences x value heads
    int64_t ntiles;  // dv / 32
    uint32_t flags;
};

struct DecodeArgs {
    const void *q, *k, *v;
    const float *log_alpha, *beta;
    const float *state_in;
    float *state_out;
    void *out;
    int64_t N, Hk, Hv;
    uint32_t flags;
};

hipError_t launch_chunk_fwd(const ChunkArgs &a, int dtype, int chunk, int dk, hipStream_t stream);
bool chunk_fwd_fast_supported(int dtype, int chunk, int dk);
hipError_t launch_chunk_fwd_fast(const ChunkArgs &a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &a, int dtype, int dk, int dv, hipStream_t stream);
hipError_t launch_selftest_mfma(const float *a, const float *b, float *d, hipStream_t stream);

}  // namespace gdr
