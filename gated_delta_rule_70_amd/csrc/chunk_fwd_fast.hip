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
//   wave 0  "chain": the state-dependent part for chunk c over all 32 columns. The state
//           tiles stay in accumulator registers and are the B operands of K H and Q H
//           directly; each operand fragment read from LDS feeds both 16-column tiles.
//   wave 1  "diagonal" prep for chunk c+1: gate scalars, diagonal tiles of K K^T and the four
//           16x16 inverses T_ii by forward substitution; copies K of chunk c+2.
//   wave 2  "P" prep for chunk c+1: the ten lower tiles of Q K^T with their decay factors;
//           copies Q of chunk c+2.
//   wave 3  "A" prep for chunk c+1: the six off-diagonal tiles of K K^T (-> -A_ij); copies V
//           and the gates of chunk c+2.
// Raw q/k/v of a chunk are copied once per workgroup, global -> LDS directly (16 bytes per
// lane, no registers), into a ring of three buffers: while the chain reads chunk c and the
// prep waves read chunk c+1, the loads for chunk c+2 are in flight. Rows are XOR-swizzled by
// 16-byte piece so that operand reads hit distinct banks. The products the prep waves hand
// to the chain go through a second, double-buffered area. One barrier per chunk.
//
// Operand order. Products whose two operands are both read from LDS use the hardware's
// contiguous k order (one 16-byte read per lane). The state tile is fed back from its
// accumulator layout, where a lane holds rows 4g..4g+3 of two stacked 16-row tiles; to make
// that coincide with the contiguous order, the state's d_k rows are kept permuted inside
// each 32-row block: stored row 16h + 4g + e holds true row 8g + 4h + e. Only the K^T operand
// of the state update and the h0/hT accesses see the permutation. Off-diagonal Gram tiles
// are computed transposed (K_j Q_i^T), which leaves each lane holding 4 consecutive columns
// of one row: exactly its slice of the chain's A operand. K^T and V are read by the chain
// with the gfx950 transpose read (ds_read_b64_tr_b16): in each 16-lane group, lane i
// receives element i%4 of the 8-byte chunks addressed by lanes 4v + i/4.
//
// Decays are carried as base-2 logarithms (b2 = log2(e) * b) and exponentiated with exp2.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "gdr_kernels.hpp"
#include "gdr_mfma.hpp"

namespace gdr {

namespace {

constexpr int kC = 64, kDK = 128, kDVT = 32;
constexpr float kLog2e = 1.4426950408889634f;

// raw buffer (one of three): K, Q [64 rows][256 B] and V [64 rows][64 B], swizzled; gates
constexpr int kRawK = 0, kRawQ = 16384, kRawV = 32768, kRawLa = 36864, kRawBeta = 37120;
constexpr int kRawBytes = 37376;
// derived buffer (one of two)
constexpr int kDerP = 0;      // 6 P fragments (row tile, 32-deep slice) x 1 KB
constexpr int kDerNA = 6144;  // -A: A10 (16-deep, 512 B), A2x (1 KB), A3x (1 KB), A32 (16-deep, 512 B)
constexpr int kDerTd = 9216;  // T_ii: four 16-deep fragments of 512 B
constexpr int kDerSc = 11264; // beta, e^b, read scale, e^{bC-b} [64] each, then e^{bC}
constexpr int kDerBytes = 12320;
constexpr int kOffRaw = 0;
constexpr int kOffDer = kOffRaw + 3 * kRawBytes;
constexpr int kOffAd = kOffDer + 2 * kDerBytes;   // wave 1: A_ii^T blocks fp32 [4][16][16]
constexpr int kOffG1 = kOffAd + 4096;             // wave 1: b2, beta [64]
constexpr int kOffG2 = kOffG1 + 512;              // wave 2: rowfP [64], colfP [3][64]
constexpr int kOffG3 = kOffG2 + 1024;             // wave 3: beta*rowfA [64], colfA [3][64]
constexpr int kOffStage = kOffG3 + 1024;         // output staging, two of [32 cols][64 rows] bf16
constexpr int kStageBytes = 4096;
constexpr int kSmemBytes = kOffStage + 2 * kStageBytes;
static_assert(kSmemBytes <= 160 * 1024, "LDS budget");

typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

__device__ __forceinline__ int pf_index(int mi, int kp) { return mi < 2 ? mi : 2 + 2 * (mi - 2) + kp; }
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Rows of one chunk: scan row r (0..rmax valid) is token lo + (fwd ? r : rmax - r); rows past
// rmax repeat the last valid token (finite data, zero gates).
struct ChunkRows {
    int64_t lo;
    int rmax;
    bool fwd;
    __device__ __forceinline__ int off(int r) const {
        const int rr = r < rmax ? r : rmax;
        return fwd ? rr : rmax - rr;
    }
};
__device__ __forceinline__ ChunkRows chunk_rows(int64_t t0, int64_t len, bool fwd, int64_t ch) {
    ChunkRows cr;
    const int64_t p0 = ch * kC;
    const int64_t left = len - 1 - p0;
    cr.rmax = (int)(left < kC - 1 ? left : kC - 1);
    cr.fwd = fwd;
    cr.lo = fwd ? t0 + p0 : t0 + len - 1 - p0 - cr.rmax;
    return cr;
}

// ------------------------------------------------------------------ global -> LDS copies
// Buffer loads straight into LDS: lane l of copy instruction n writes LDS bytes
// [n*1024 + 16 l, +16); we choose the 16-byte piece it reads, so the LDS image is
// row-major and XOR-swizzled by piece. The buffer resource covers one head's slab (reads at
// or past its end return zero); the chunk's first token goes into the scalar offset, the
// lane's row and piece into the 32-bit vector offset.
//
// The copies are issued from inline assembly. The compiler cannot tell which LDS bytes a
// copy writes, so for the intrinsic it waits for every outstanding copy before the next LDS
// read of the wave, which here would put the whole global-memory latency of the next chunk's
// copies in front of the current chunk's prep work. The copies target a ring slot that no
// wave reads until after the next barrier, and each wave waits for its own copies (vmcnt)
// before that barrier, so no other wait is needed.
constexpr unsigned kRsrcWord3 = 0x00020000;  // raw (untyped) buffer access
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 slab_rsrc(const void *base, int64_t bytes) {
    const unsigned n = bytes > 0x7fffffff ? 0x7fffffffu : (unsigned)bytes;
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    u32x4 r;
    r.x = __builtin_amdgcn_readfirstlane((unsigned)p);
    r.y = __builtin_amdgcn_readfirstlane((unsigned)(p >> 32) & 0xffffu);  // stride 0
    r.z = __builtin_amdgcn_readfirstlane(n);
    r.w = kRsrcWord3;
    return r;
}
__device__ __forceinline__ unsigned lds_addr(const void *p) {
    return __builtin_amdgcn_readfirstlane(
        (unsigned)reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char *)p));
}
// 16 bytes per lane into LDS at m0 + 16 lane (one wait state after the write of m0)
__device__ __forceinline__ void dma_b128(unsigned lds, u32x4 rsrc, int voff, int soff) {
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds)
                 : "memory");
}
// 4 bytes per lane into LDS at m0 + 4 lane
__device__ __forceinline__ void dma_b32(unsigned lds, u32x4 rsrc, int voff, int soff) {
    asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds)
                 : "memory");
}
// Per-lane vector offsets of the copies. They are the same for every full chunk (the chunk's
// first token goes into the scalar offset); only a ragged last chunk needs its own, clamped
// ones. Both sets are computed before the chunk loop and never rewritten: the compiler
// waits for all outstanding copies before it reuses a register that one of them addresses
// with, so offsets computed inside the loop would serialise the copies with the prep work.
struct CopyOffsets {
    int kq[16], v[4], gate;
    __device__ __forceinline__ void init(const ChunkRows &cr, int64_t dv) {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int n = 0; n < 16; ++n) {
            const int row = 4 * n + (lane >> 4);
            kq[n] = cr.off(row) * 256 + (((lane & 15) ^ (row & 15)) << 4);
        }
        const int rowb = (int)(dv * 2);
        const int piece = (lane & 3) ^ (lane >> 4);
#pragma unroll
        for (int n = 0; n < 4; ++n) v[n] = cr.off(16 * n + (lane >> 2)) * rowb + piece * 16;
        // rows past the end get an offset beyond the buffer, which reads as zero
        gate = lane <= cr.rmax ? cr.off(lane) * 4 : 0x40000000;
        // opaque to the optimiser, so they stay in their registers instead of being
        // recomputed into temporaries next to each copy
#pragma unroll
        for (int n = 0; n < 16; ++n) asm volatile("" : "+v"(kq[n]));
#pragma unroll
        for (int n = 0; n < 4; ++n) asm volatile("" : "+v"(v[n]));
        asm volatile("" : "+v"(gate));
    }
};
__device__ __forceinline__ void copy_kq(char *dst, u32x4 rsrc, const CopyOffsets &co, int64_t lo) {
    const int soff = __builtin_amdgcn_readfirstlane((int)(lo * 256));
    const unsigned base = lds_addr(dst);
#pragma unroll
    for (int n = 0; n < 16; ++n) dma_b128(base + n * 1024, rsrc, co.kq[n], soff);
}
__device__ __forceinline__ void copy_v(char *dst, u32x4 rsrc, const CopyOffsets &co, int64_t lo, int64_t dv) {
    const int soff = __builtin_amdgcn_readfirstlane((int)(lo * dv * 2));
    const unsigned base = lds_addr(dst);
#pragma unroll
    for (int n = 0; n < 4; ++n) dma_b128(base + n * 1024, rsrc, co.v[n], soff);
}
// Gates of the chunk (log alpha, beta) straight into the raw buffer: lane r loads row r.
__device__ __forceinline__ void copy_gates(char *raw, u32x4 ra, u32x4 rb, const CopyOffsets &co, int64_t lo) {
    const int soff = __builtin_amdgcn_readfirstlane((int)(lo * 4));
    dma_b32(lds_addr(raw + kRawLa), ra, co.gate, soff);
    dma_b32(lds_addr(raw + kRawBeta), rb, co.gate, soff);
}
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Workgroup barrier that orders LDS only: this wave's LDS accesses complete, then s_barrier.
// (The plain __syncthreads() would also wait for outstanding global stores, which nobody
// in the workgroup reads; global->LDS copies are waited for explicitly before it.)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ------------------------------------------------------------------ operand reads
__device__ __forceinline__ Frag<__bf16> u4_frag(uint4 u) {
    Frag<__bf16> f;
    f.lo = __builtin_bit_cast(bf16x4, make_uint2(u.x, u.y));
    f.hi = __builtin_bit_cast(bf16x4, make_uint2(u.z, u.w));
    return f;
}
// Per-lane LDS offsets of the contiguous-order operand (row 16i + c, columns 32ks + 8g..+7):
// byte 4096 i + (256 c + 16 (g ^ c)) ^ (ks << 6).
struct RowFragOffsets {
    int o[4];
    __device__ __forceinline__ void init() {
        const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
        const int base = 256 * c + ((g ^ c) << 4);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) o[ks] = base ^ (ks << 6);
    }
};
__device__ __forceinline__ uint4 row_frag(const char *buf, const RowFragOffsets &ro, int i, int ks) {
    return *reinterpret_cast<const uint4 *>(buf + ro.o[ks] + 4096 * i);
}
__device__ __forceinline__ bf16x4 tr16(const char *p) {
    return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(p)));
}
// K^T operand of the state update for stored state tile t: lane (g, i) gets
// K[32kp + 4g + v][pi(16t + i)] (lo) and the rows 16 further (hi), v = 0..3, where
// pi(16t + 4q + e) = 32(t/2) + 8q + 4(t%2) + e. Lane j of group g addresses row
// 32kp + 4g + j/4 (+16), columns pi(16t + 4(j%4)) .. +3.
struct KtOffsets {
    int o[4];  // per t/2
    __device__ __forceinline__ void init() {
        const int lane = threadIdx.x & 63, g = lane >> 4, j = lane & 15;
        const int r16 = 4 * g + (j >> 2);
        const int z = (j & 3) ^ r16;
        const int base = r16 * 256 + (z << 4);
#pragma unroll
        for (int th = 0; th < 4; ++th) o[th] = base ^ (th << 6);
    }
};
__device__ __forceinline__ Frag<__bf16> kt_frag(const char *kbuf, const KtOffsets &ko, int t, int kp) {
    const char *p = kbuf + ko.o[t >> 1] + 8192 * kp + 8 * (t & 1);
    Frag<__bf16> f;
    f.lo = tr16(p);
    f.hi = tr16(p + 4096);
    return f;
}
// V rows 16mi + 4g + v, column 16w + i, as an accumulator-layout tile: lane j of group g
// addresses row 16mi + 4g + j/4, columns 16w + 4(j%4)..+3.
__device__ __forceinline__ int v_lane_offset(int w) {
    const int lane = threadIdx.x & 63, g = lane >> 4, j = lane & 15;
    const int slot = (2 * w + ((j >> 1) & 1)) ^ g;
    return (4 * g + (j >> 2)) * 64 + (slot << 4) + 8 * (j & 1);
}
__device__ __forceinline__ Frag<__bf16> der_frag(const char *base, int idx) {
    const int lane = threadIdx.x & 63;
    return u4_frag(*reinterpret_cast<const uint4 *>(base + (idx * 64 + lane) * 16));
}
__device__ __forceinline__ bf16x4 der_frag_lo(const char *base, int idx) {
    const int lane = threadIdx.x & 63;
    return *reinterpret_cast<const bf16x4 *>(base + (idx * 64 + lane) * 8);
}
// Output staging tile, column-major: column col (0..31) is 128 bytes of 16 row quads, quad
// position XOR-swizzled by col % 16. The chain writes a lane's four rows of one column as
// one 8-byte store; the write-back reads it with the transpose read, which hands each lane
// four consecutive columns of one row.
__device__ __forceinline__ int stage_off(int col, int quad) { return col * 128 + ((quad ^ (col & 15)) << 3); }

// Inclusive prefix sum over the 64 lanes: shifts within each 16-lane row, then the row
// totals are broadcast forward (DPP row_bcast:15 into rows 1 and 3, row_bcast:31 into
// rows 2 and 3). Lanes whose source is outside the row read 0.
#define GDR_DPP_STEP(ctrl, rmask, bz)                                                                \
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), ctrl, \
                                                               rmask, 0xf, bz))
__device__ __forceinline__ float wave_cumsum(float x) {
    GDR_DPP_STEP(0x111, 0xf, true);   // row_shr:1
    GDR_DPP_STEP(0x112, 0xf, true);   // row_shr:2
    GDR_DPP_STEP(0x114, 0xf, true);   // row_shr:4
    GDR_DPP_STEP(0x118, 0xf, true);   // row_shr:8
    GDR_DPP_STEP(0x142, 0xa, false);  // row_bcast:15
    GDR_DPP_STEP(0x143, 0xc, false);  // row_bcast:31
    return x;
}
#undef GDR_DPP_STEP
__device__ __forceinline__ float lane_value(float x, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

__device__ __forceinline__ floatx4 gram_u4(const uint4 (&x)[4], const uint4 (&y)[4]) {
    floatx4 acc = zero4();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) acc = mma32(acc, u4_frag(x[ks]), u4_frag(y[ks]));
    return acc;
}

__device__ __forceinline__ uint2 pack4(floatx4 v) { return __builtin_bit_cast(uint2, cvt4<__bf16>(v)); }

// ------------------------------------------------------------------ gate scalars
// Every prep wave starts from the chunk's gates in the raw buffer (lane = token row).
struct Gates {
    float la2, beta, b2;  // log2-scaled log alpha, beta, inclusive log2 cumsum
};
__device__ __forceinline__ Gates read_gates(const char *raw) {
    const int lane = threadIdx.x & 63;
    Gates gt;
    gt.la2 = reinterpret_cast<const float *>(raw + kRawLa)[lane] * kLog2e;
    gt.beta = reinterpret_cast<const float *>(raw + kRawBeta)[lane];
    gt.b2 = wave_cumsum(gt.la2);
    return gt;
}

// ------------------------------------------------------------------ wave 1: diagonal prep
__device__ __forceinline__ void prep_diag(char *smem, const char *raw, char *der, bool pre, const RowFragOffsets &ro) {
    const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
    const Gates gt = read_gates(raw);
    float *gb = reinterpret_cast<float *>(smem + kOffG1);
    gb[lane] = gt.b2;
    gb[64 + lane] = gt.beta;
    {
        float *sc = reinterpret_cast<float *>(der + kDerSc);
        const float bC = lane_value(gt.b2, 63);
        sc[lane] = gt.beta;
        sc[64 + lane] = ex2(gt.b2);
        sc[128 + lane] = ex2(pre ? gt.b2 - gt.la2 : gt.b2);
        sc[192 + lane] = ex2(bC - gt.b2);
        if (lane == 0) sc[256] = ex2(bC);
    }
    uint4 kf[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kf[i][ks] = row_frag(raw + kRawK, ro, i, ks);
    wave_lds_sync();
    float *adt = reinterpret_cast<float *>(smem + kOffAd);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // A_ii in standard orientation: lane holds rows 16i + 4g + r, column 16i + c
        const floatx4 gk = gram_u4(kf[i], kf[i]);
        const floatx4 b4 = *reinterpret_cast<const floatx4 *>(gb + 16 * i + 4 * g);
        const floatx4 beta4 = *reinterpret_cast<const floatx4 *>(gb + 64 + 16 * i + 4 * g);
        const float bc = gb[16 * i + c];
        floatx4 a;
#pragma unroll
        for (int r = 0; r < 4; ++r) a[r] = (c < 4 * g + r) ? beta4[r] * gk[r] * ex2(b4[r] - bc) : 0.f;
        *reinterpret_cast<floatx4 *>(adt + (i * 16 + c) * 16 + 4 * g) = a;
    }
    wave_lds_sync();
    // T_ii = (I + A_ii)^{-1}: lane (i = g, c) computes column c. The column of A it needs is
    // read into registers first; then each solved t_j is eliminated from every later row.
    const float *ablk = adt + g * 256;
    floatx4 acol[15][4];
#pragma unroll
    for (int j = 0; j < 15; ++j)
#pragma unroll
        for (int q4 = (j + 1) >> 2; q4 < 4; ++q4) acol[j][q4] = reinterpret_cast<const floatx4 *>(ablk + j * 16)[q4];
    float acc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = (r == c) ? 1.f : 0.f;
#pragma unroll
    for (int j = 0; j < 15; ++j) {
        const float tj = acc[j];
#pragma unroll
        for (int r = j + 1; r < 16; ++r) acc[r] -= acol[j][r >> 2][r & 3] * tj;
    }
    // 16-deep A-operand fragment of T_ii: element (r, c) -> lane (c/4, r), slot c%4
    char *td = der + kDerTd + g * 512 + ((c >> 2) << 7) + 2 * (c & 3);
#pragma unroll
    for (int r = 0; r < 16; ++r) *reinterpret_cast<__bf16 *>(td + 8 * r) = (__bf16)acc[r];
}

// Decay factors of off-diagonal tiles are split at each 16-row tile: for rows in tile i and
// columns before it, e^{x_row - b_col} = e^{x_row - ref_i} * e^{ref_i - b_col} with both
// exponents <= 0 (ref_i = b_{16i} for A and the post-write read, b_{16i-1} = b'_{16i} for
// the pre-write read).
__device__ __forceinline__ void tile_refs(float b2, float &s0, float &s16, float &s32, float &s48, float &e15,
                                          float &e31, float &e47) {
    s0 = lane_value(b2, 0);
    s16 = lane_value(b2, 16);
    s32 = lane_value(b2, 32);
    s48 = lane_value(b2, 48);
    e15 = lane_value(b2, 15);
    e31 = lane_value(b2, 31);
    e47 = lane_value(b2, 47);
}

// ------------------------------------------------------------------ wave 2: P prep
__device__ __forceinline__ void prep_p(char *smem, const char *raw, char *der, bool pre, const RowFragOffsets &ro) {
    const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
    const Gates gt = read_gates(raw);
    float *gw = reinterpret_cast<float *>(smem + kOffG2);
    float s0, s16, s32, s48, e15, e31, e47;
    tile_refs(gt.b2, s0, s16, s32, s48, e15, e31, e47);
    {
        const int tile = lane >> 4;
        const float ref = tile == 0 ? s0 : tile == 1 ? s16 : tile == 2 ? s32 : s48;
        const float refp = tile == 1 ? e15 : tile == 2 ? e31 : e47;
        // row factor of row = lane, for tiles i >= 1
        gw[lane] = pre ? ex2(fminf(gt.b2 - gt.la2 - refp, 0.f)) : ex2(fminf(gt.b2 - ref, 0.f));
        gw[64 + lane] = lane < 16 ? ex2((pre ? e15 : s16) - gt.b2) : 0.f;
        gw[128 + lane] = lane < 32 ? ex2((pre ? e31 : s32) - gt.b2) : 0.f;
        gw[192 + lane] = lane < 48 ? ex2((pre ? e47 : s48) - gt.b2) : 0.f;
    }
    // read-side log decay of the row and log decay of the column, for the diagonal tiles
    const float bread = pre ? gt.b2 - gt.la2 : gt.b2;
    uint4 kf[4][4], qf[4][4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            kf[i][ks] = row_frag(raw + kRawK, ro, i, ks);
            qf[i][ks] = row_frag(raw + kRawQ, ro, i, ks);
        }
    wave_lds_sync();
    char *pf = der + kDerP;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // row 16i + c of this lane: its read decay, from lane 16i + c
        const float br = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * (16 * i + c), __builtin_bit_cast(int, bread)));
        const float rowf = gw[16 * i + c];
#pragma unroll
        for (int j = 0; j <= i; ++j) {
            // transposed tile: lane holds row 16i + c, columns 16j + 4g + r
            const floatx4 gq = gram_u4(kf[j], qf[i]);
            floatx4 pv;
            if (j < i) {
                const floatx4 cf = *reinterpret_cast<const floatx4 *>(gw + 64 * i + 16 * j + 4 * g);
                pv = rowf * cf * gq;
            } else {
                // diagonal tile: columns 16i + 4g + r against row 16i + c
                const floatx4 bcol = {__builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * (16 * i + 4 * g + 0), __builtin_bit_cast(int, gt.b2))),
                                      __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * (16 * i + 4 * g + 1), __builtin_bit_cast(int, gt.b2))),
                                      __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * (16 * i + 4 * g + 2), __builtin_bit_cast(int, gt.b2))),
                                      __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * (16 * i + 4 * g + 3), __builtin_bit_cast(int, gt.b2)))};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int cc = 4 * g + r;
                    const bool keep = pre ? (cc < c) : (cc <= c);
                    pv[r] = keep ? gq[r] * ex2(br - bcol[r]) : 0.f;
                }
            }
            *reinterpret_cast<uint2 *>(pf + pf_index(i, j >> 1) * 1024 + lane * 16 + 8 * (j & 1)) = pack4(pv);
        }
    }
}

// ------------------------------------------------------------------ wave 3: A prep
__device__ __forceinline__ void prep_a(char *smem, const char *raw, char *der, const RowFragOffsets &ro) {
    const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
    const Gates gt = read_gates(raw);
    float *gw = reinterpret_cast<float *>(smem + kOffG3);
    float s0, s16, s32, s48, e15, e31, e47;
    tile_refs(gt.b2, s0, s16, s32, s48, e15, e31, e47);
    {
        const int tile = lane >> 4;
        const float ref = tile == 0 ? s0 : tile == 1 ? s16 : tile == 2 ? s32 : s48;
        gw[lane] = gt.beta * ex2(fminf(gt.b2 - ref, 0.f));
        gw[64 + lane] = lane < 16 ? ex2(s16 - gt.b2) : 0.f;
        gw[128 + lane] = lane < 32 ? ex2(s32 - gt.b2) : 0.f;
        gw[192 + lane] = lane < 48 ? ex2(s48 - gt.b2) : 0.f;
    }
    uint4 kf[4][4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int i = 0; i < 4; ++i) kf[i][ks] = row_frag(raw + kRawK, ro, i, ks);
    wave_lds_sync();
    char *na = der + kDerNA;
#pragma unroll
    for (int i = 1; i < 4; ++i) {
        const float ar = gw[16 * i + c];  // beta * row factor of row 16i + c
#pragma unroll
        for (int j = 0; j < i; ++j) {
            // transposed tile: lane holds row 16i + c, columns 16j + 4g + r
            const floatx4 gk = gram_u4(kf[j], kf[i]);
            const floatx4 cf = *reinterpret_cast<const floatx4 *>(gw + 64 * i + 16 * j + 4 * g);
            const floatx4 av = (-ar) * cf * gk;
            int aoff;
            if (i == 1) aoff = lane * 8;                           // A10, 16-deep
            else if (i == 2) aoff = 512 + lane * 16 + 8 * j;       // A20 | A21
            else if (j < 2) aoff = 1536 + lane * 16 + 8 * j;       // A30 | A31
            else aoff = 2560 + lane * 8;                           // A32, 16-deep
            *reinterpret_cast<uint2 *>(na + aoff) = pack4(av);
        }
    }
}

// Write-back of one chunk's output from its staging tile: transpose read r covers rows
// 16(r/2) .. +15 and columns 16(r%2) .. +15; lane (g, i) gets row 16(r/2) + i, columns
// 16(r%2) + 4g .. +3 and stores them as 8 bytes.
__device__ __forceinline__ void write_back(const char *stg, __bf16 *obase, const ChunkRows &cr, int64_t dv,
                                           bool acc_out) {
    const int lane = threadIdx.x & 63, g = lane >> 4, j = lane & 15;
    bf16x4 val[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int col = 16 * (r & 1) + 4 * g + (j >> 2);
        val[r] = tr16(stg + stage_off(col, 4 * (r >> 1) + (j & 3)));
    }
    wave_lds_sync();
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int row = 16 * (r >> 1) + j;
        if (row <= cr.rmax) {
            bf16x4 *dst = reinterpret_cast<bf16x4 *>(obase + (int64_t)cr.off(row) * dv + 16 * (r & 1) + 4 * g);
            bf16x4 v = val[r];
            if (acc_out) {
                const bf16x4 prev = *dst;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = (__bf16)((float)v[e] + (float)prev[e]);
            }
            *dst = v;
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
    int64_t t0 = 0, len = a.T;
    if (a.cu_seqlens) {
        t0 = a.cu_seqlens[seq];
        len = a.cu_seqlens[seq + 1] - t0;
    }
    const bool fwd = (a.flags & kFlagReverse) == 0;
    const bool pre = (a.flags & kFlagReadPre) != 0;
    const bool acc_out = (a.flags & kFlagAccumulate) != 0;
    const int64_t nchunks = (len + kC - 1) / kC;
    const int dcol0 = tile * kDVT;

    const __bf16 *kb = reinterpret_cast<const __bf16 *>(a.k) + (row * a.Hk + kh) * a.T * kDK;
    const __bf16 *qb = reinterpret_cast<const __bf16 *>(a.q) + (row * a.Hk + kh) * a.T * kDK;
    const __bf16 *vb = reinterpret_cast<const __bf16 *>(a.v) + (row * a.Hv + head) * a.T * a.dv;
    const float *ab = a.log_alpha + (row * a.Hv + head) * a.T;
    const float *bb = a.beta + (row * a.Hv + head) * a.T;
    __bf16 *ob = reinterpret_cast<__bf16 *>(a.out) + (row * a.Hv + head) * a.T * a.dv;

    // The two roles run separate loops with the same barrier sequence (two barriers in
    // the prologue, one per chunk), so each role's registers are live only in its own loop.
    if (wave >= 1) {
        if (nchunks == 0) return;
        RowFragOffsets ro;
        ro.init();
        // the upper 16x16 tiles inside P fragments 0 and 3 are never written: zero them
        if (wave == 2) {
            for (int d = 0; d < 2; ++d) {
                char *pf = smem + kOffDer + d * kDerBytes + kDerP;
                *reinterpret_cast<uint2 *>(pf + lane * 16 + 8) = make_uint2(0, 0);
                *reinterpret_cast<uint2 *>(pf + 3 * 1024 + lane * 16 + 8) = make_uint2(0, 0);
            }
        }
        // one loop per role, so that each keeps only its own loop-invariant registers
        auto run = [&](auto role) {
            constexpr int R = decltype(role)::value;
            u32x4 rsrc0, rsrc1;
            if constexpr (R == 1) {
                rsrc0 = slab_rsrc(kb, a.T * kDK * 2);
                rsrc1 = rsrc0;
            } else if constexpr (R == 2) {
                rsrc0 = slab_rsrc(qb, a.T * kDK * 2);
                rsrc1 = rsrc0;
            } else {
                rsrc0 = slab_rsrc(vb + dcol0, a.T * a.dv * 2 - dcol0 * 2);
                rsrc1 = slab_rsrc(ab, (t0 + len) * 4);
            }
            const u32x4 rbeta = slab_rsrc(bb, (t0 + len) * 4);
            // lane offsets of a full chunk (rmax = 63) and of the last chunk
            CopyOffsets cfull, clast;
            {
                ChunkRows full;
                full.lo = 0;
                full.rmax = kC - 1;
                full.fwd = fwd;
                cfull.init(full, a.dv);
                clast.init(chunk_rows(t0, len, fwd, nchunks - 1), a.dv);
            }
            auto copy = [&](char *rawn, const CopyOffsets &co, int64_t lo) {
                if constexpr (R == 1) copy_kq(rawn + kRawK, rsrc0, co, lo);
                else if constexpr (R == 2) copy_kq(rawn + kRawQ, rsrc0, co, lo);
                else {
                    copy_v(rawn + kRawV, rsrc0, co, lo, a.dv);
                    copy_gates(rawn, rsrc1, rbeta, co, lo);
                }
            };
            // two explicit paths, so that each copy addresses with one of the fixed sets
            auto issue = [&](int64_t ch, const CopyOffsets &co) {
                char *rawn = smem + kOffRaw + (int)(ch % 3) * kRawBytes;
                copy(rawn, co, chunk_rows(t0, len, fwd, ch).lo);
            };
            auto prep = [&](int64_t ch) {
                const char *rawp = smem + kOffRaw + (int)(ch % 3) * kRawBytes;
                char *derp = smem + kOffDer + (int)(ch & 1) * kDerBytes;
                if constexpr (R == 1) prep_diag(smem, rawp, derp, pre, ro);
                else if constexpr (R == 2) prep_p(smem, rawp, derp, pre, ro);
                else prep_a(smem, rawp, derp, ro);
            };
            auto store = [&](int64_t ch) {
                const ChunkRows cr = chunk_rows(t0, len, fwd, ch);
                write_back(smem + kOffStage + (int)(ch & 1) * kStageBytes, ob + cr.lo * a.dv + dcol0, cr, a.dv,
                           acc_out);
            };
            auto step = [&](int64_t ch) {
                if constexpr (R == 3) {
                    if (ch >= 1) store(ch - 1);
                }
                if (ch + 1 < nchunks) prep(ch + 1);
                wait_vmem();
                lds_barrier();
            };
            if (nchunks == 1) issue(0, clast);
            else issue(0, cfull);
            wait_vmem();
            lds_barrier();
            if (nchunks == 2) issue(1, clast);
            else if (nchunks > 2) issue(1, cfull);
            prep(0);
            wait_vmem();
            lds_barrier();
            // The loop that copies full chunks and the tail that copies the last chunk are
            // separate code, so that no copy's offset register is chosen at run time.
            int64_t ch = 0;
            for (; ch + 3 < nchunks; ++ch) {
                issue(ch + 2, cfull);
                step(ch);
            }
            for (; ch < nchunks; ++ch) {
                if (ch + 2 < nchunks) issue(ch + 2, clast);
                step(ch);
            }
            if constexpr (R == 3) store(nchunks - 1);
        };
        if (wave == 1) run(std::integral_constant<int, 1>{});
        else if (wave == 2) run(std::integral_constant<int, 2>{});
        else run(std::integral_constant<int, 3>{});
        return;
    }

    // chain wave: stored state rows 16t + 4g + r (true row 32(t/2) + 8g + 4(t%2) + r) of
    // the two 16-column tiles ct, column dcol0 + 16 ct + c
    floatx4 H[2][8];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int t = 0; t < 8; ++t) H[ct][t] = zero4();
    if (a.h0) {
        const float *hb = a.h0 + (seq * a.Hv + head) * kDK * a.dv + dcol0 + c;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) H[ct][t][r] = hb[(32 * (t >> 1) + 8 * g + 4 * (t & 1) + r) * a.dv + 16 * ct];
    }
    RowFragOffsets ro;
    ro.init();
    KtOffsets ko;
    ko.init();
    const int voff0 = v_lane_offset(0), voff1 = v_lane_offset(1);
    const int scoff = 16 * g;  // bytes: rows 4g..4g+3 of a 16-row tile
    if (nchunks > 0) {
        lds_barrier();
        lds_barrier();
    }

    // Each phase issues the LDS reads of the next one before its own arithmetic, and
    // scheduling fences keep the compiler from sinking them back to their uses.
    for (int64_t ch = 0; ch < nchunks; ++ch) {
        const char *raw = smem + kOffRaw + (int)(ch % 3) * kRawBytes;
        const char *der = smem + kOffDer + (int)(ch & 1) * kDerBytes;
        const char *sc = der + kDerSc + scoff;
        const char *na = der + kDerNA;
        const char *td = der + kDerTd;
        // X_K = K H, X_Q = Q H for both column tiles; each operand fragment feeds two products
        floatx4 XK[2][4], XQ[2][4];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                XK[ct][mi] = zero4();
                XQ[ct][mi] = zero4();
            }
        uint4 fk[2][4], fq[2][4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            fk[0][mi] = row_frag(raw + kRawK, ro, mi, 0);
            fq[0][mi] = row_frag(raw + kRawQ, ro, mi, 0);
        }
        bf16x4 vv[2][4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks < 3) {
#pragma unroll
                for (int mi = 0; mi < 4; ++mi) {
                    fk[(ks + 1) & 1][mi] = row_frag(raw + kRawK, ro, mi, ks + 1);
                    fq[(ks + 1) & 1][mi] = row_frag(raw + kRawQ, ro, mi, ks + 1);
                }
            } else {
#pragma unroll
                for (int mi = 0; mi < 4; ++mi) {
                    vv[0][mi] = tr16(raw + kRawV + voff0 + 1024 * mi);
                    vv[1][mi] = tr16(raw + kRawV + voff1 + 1024 * mi);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            const Frag<__bf16> h0f = frag_from_acc<__bf16>(H[0][2 * ks], H[0][2 * ks + 1]);
            const Frag<__bf16> h1f = frag_from_acc<__bf16>(H[1][2 * ks], H[1][2 * ks + 1]);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                const Frag<__bf16> kf = u4_frag(fk[ks & 1][mi]);
                const Frag<__bf16> qf = u4_frag(fq[ks & 1][mi]);
                XK[0][mi] = mma32(XK[0][mi], kf, h0f);
                XK[1][mi] = mma32(XK[1][mi], kf, h1f);
                XQ[0][mi] = mma32(XQ[0][mi], qf, h0f);
                XQ[1][mi] = mma32(XQ[1][mi], qf, h1f);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // R = beta (V - e^{b} X_K); the substitution's operands are read meanwhile
        floatx4 be[4], eb[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            be[mi] = *reinterpret_cast<const floatx4 *>(sc + 64 * mi);
            eb[mi] = *reinterpret_cast<const floatx4 *>(sc + 256 + 64 * mi);
        }
        const bf16x4 t0f = der_frag_lo(td, 0), t1f = der_frag_lo(td, 1), t2f = der_frag_lo(td, 2), t3f = der_frag_lo(td, 3);
        const bf16x4 a10 = der_frag_lo(na, 0), a32 = der_frag_lo(na + 2560, 0);
        const Frag<__bf16> a2x = der_frag(na + 512, 0), a3x = der_frag(na + 1536, 0);
        __builtin_amdgcn_sched_barrier(0);
        floatx4 U[2][4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                U[0][mi][r] = be[mi][r] * ((float)vv[0][mi][r] - eb[mi][r] * XK[0][mi][r]);
                U[1][mi][r] = be[mi][r] * ((float)vv[1][mi][r] - eb[mi][r] * XK[1][mi][r]);
            }
        // U_i = T_ii (R_i - sum_{j<i} A_ij U_j), both column tiles interleaved; the output
        // operands are read meanwhile
        const Frag<__bf16> p0 = der_frag(der + kDerP, 0), p1 = der_frag(der + kDerP, 1);
        const Frag<__bf16> p20 = der_frag(der + kDerP, 2), p21 = der_frag(der + kDerP, 3);
        const Frag<__bf16> p30 = der_frag(der + kDerP, 4), p31 = der_frag(der + kDerP, 5);
        floatx4 er[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) er[mi] = *reinterpret_cast<const floatx4 *>(sc + 512 + 64 * mi);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) U[ct][0] = mma16(zero4(), t0f, cvt4<__bf16>(U[ct][0]));
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) U[ct][1] = mma16(U[ct][1], a10, cvt4<__bf16>(U[ct][0]));
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) U[ct][1] = mma16(zero4(), t1f, cvt4<__bf16>(U[ct][1]));
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            const Frag<__bf16> u01 = frag_from_acc<__bf16>(U[ct][0], U[ct][1]);
            U[ct][2] = mma32(U[ct][2], a2x, u01);
            U[ct][3] = mma32(U[ct][3], a3x, u01);
        }
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) U[ct][2] = mma16(zero4(), t2f, cvt4<__bf16>(U[ct][2]));
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) U[ct][3] = mma16(U[ct][3], a32, cvt4<__bf16>(U[ct][2]));
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) U[ct][3] = mma16(zero4(), t3f, cvt4<__bf16>(U[ct][3]));
        // O = e^{b | b'} X_Q + P U into the staging tile; the state-update operands are read
        // meanwhile
        floatx4 ec[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) ec[mi] = *reinterpret_cast<const floatx4 *>(sc + 768 + 64 * mi);
        const float gC = *reinterpret_cast<const float *>(der + kDerSc + 1024);
        Frag<__bf16> kt[2][2];
        kt[0][0] = kt_frag(raw + kRawK, ko, 0, 0);
        kt[0][1] = kt_frag(raw + kRawK, ko, 0, 1);
        __builtin_amdgcn_sched_barrier(0);
        {
            char *stg = smem + kOffStage + (int)(ch & 1) * kStageBytes;
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const Frag<__bf16> u01 = frag_from_acc<__bf16>(U[ct][0], U[ct][1]);
                const Frag<__bf16> u23 = frag_from_acc<__bf16>(U[ct][2], U[ct][3]);
                floatx4 O[4];
#pragma unroll
                for (int mi = 0; mi < 4; ++mi) O[mi] = er[mi] * XQ[ct][mi];
                O[0] = mma32(O[0], p0, u01);
                O[1] = mma32(O[1], p1, u01);
                O[2] = mma32(O[2], p20, u01);
                O[2] = mma32(O[2], p21, u23);
                O[3] = mma32(O[3], p30, u01);
                O[3] = mma32(O[3], p31, u23);
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
                    *reinterpret_cast<uint2 *>(stg + stage_off(16 * ct + c, 4 * mi + g)) = pack4(O[mi]);
            }
        }
        // H <- e^{b_C} H + K^T diag(e^{b_C - b}) U
        {
            floatx4 W[2][4];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                W[0][mi] = ec[mi] * U[0][mi];
                W[1][mi] = ec[mi] * U[1][mi];
            }
            const Frag<__bf16> w001 = frag_from_acc<__bf16>(W[0][0], W[0][1]), w023 = frag_from_acc<__bf16>(W[0][2], W[0][3]);
            const Frag<__bf16> w101 = frag_from_acc<__bf16>(W[1][0], W[1][1]), w123 = frag_from_acc<__bf16>(W[1][2], W[1][3]);
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                if (t < 7) {
                    kt[(t + 1) & 1][0] = kt_frag(raw + kRawK, ko, t + 1, 0);
                    kt[(t + 1) & 1][1] = kt_frag(raw + kRawK, ko, t + 1, 1);
                }
                __builtin_amdgcn_sched_barrier(0);
                H[0][t] = H[0][t] * gC;
                H[1][t] = H[1][t] * gC;
                H[0][t] = mma32(H[0][t], kt[t & 1][0], w001);
                H[1][t] = mma32(H[1][t], kt[t & 1][0], w101);
                H[0][t] = mma32(H[0][t], kt[t & 1][1], w023);
                H[1][t] = mma32(H[1][t], kt[t & 1][1], w123);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        lds_barrier();
    }

    if (a.hT) {
        float *hb = a.hT + (seq * a.Hv + head) * kDK * a.dv + dcol0 + c;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) hb[(32 * (t >> 1) + 8 * g + 4 * (t & 1) + r) * a.dv + 16 * ct] = H[ct][t][r];
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
