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
//               Q H directly.
//   wave 2      "diagonal prep" for chunk c+1: gate scalars, diagonal tiles of K K^T and
//               Q K^T, the four 16x16 inverses T_ii by forward substitution.
//   wave 3      "off-diagonal prep" for chunk c+1: off-diagonal tiles of K K^T (-> -A_ij)
//               and Q K^T (-> P).
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
constexpr int kOffAd = kOffDer + 2 * kDerBytes;   // wave 2: A_ii^T blocks fp32 [4][16][16]
constexpr int kOffG2 = kOffAd + 4096;             // wave 2: b2, beta, la2 [64]
constexpr int kOffG3 = kOffG2 + 768;              // wave 3: beta*rowfA, rowfP [64]; colfA, colfP [3][64]
constexpr int kOffStage = kOffG3 + 8 * 256;
constexpr int kSmemBytes = kOffStage + 2 * 2048;  // chain output staging [2][64][16] bf16
static_assert(kSmemBytes <= 160 * 1024, "LDS budget");

typedef __attribute__((address_space(3))) void lds_void;
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
// row-major and XOR-swizzled by piece. The buffer resource covers one head's slab; the
// chunk's first token goes into the scalar offset, the lane's row and piece into the
// 32-bit vector offset.
constexpr int kRsrcWord3 = 0x00020000;  // raw (untyped) buffer access
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slab_rsrc(const void *base, int64_t bytes) {
    const int n = bytes > 0x7fffffff ? 0x7fffffff : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, kRsrcWord3);
}
// Per-lane vector offsets of the copies. For every full chunk they are the same (the chunk's
// first token goes into the scalar offset), so they are computed once and kept in registers
// that are never rewritten while copies are in flight; only a ragged last chunk computes
// clamped offsets.
struct CopyOffsets {
    int kq[16], v[4];
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
    }
};
__device__ __forceinline__ void copy_kq(char *dst, __amdgpu_buffer_rsrc_t rsrc, const CopyOffsets &co, int64_t lo) {
    const int soff = __builtin_amdgcn_readfirstlane((int)(lo * 256));
#pragma unroll
    for (int n = 0; n < 16; ++n)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void *)(dst + n * 1024), 16, co.kq[n], soff, 0, 0);
}
__device__ __forceinline__ void copy_v(char *dst, __amdgpu_buffer_rsrc_t rsrc, const CopyOffsets &co, int64_t lo,
                                       int64_t dv) {
    const int soff = __builtin_amdgcn_readfirstlane((int)(lo * dv * 2));
#pragma unroll
    for (int n = 0; n < 4; ++n)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void *)(dst + n * 1024), 16, co.v[n], soff, 0, 0);
}
// Gates of the chunk (log alpha, beta) straight into the raw buffer: lane r loads row r.
// Rows past the end get an offset beyond the buffer, which reads as zero.
__device__ __forceinline__ void copy_gates(char *raw, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                           const ChunkRows &cr) {
    const int lane = threadIdx.x & 63;
    const int voff = lane <= cr.rmax ? cr.off(lane) * 4 : 0x40000000;
    const int soff = __builtin_amdgcn_readfirstlane((int)(cr.lo * 4));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(raw + kRawLa), 4, voff, soff, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(raw + kRawBeta), 4, voff, soff, 0, 0);
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

// ------------------------------------------------------------------ wave 2: diagonal prep
__device__ __forceinline__ void prep_diag(char *smem, const char *raw, char *der, bool pre, const RowFragOffsets &ro) {
    const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
    const float la2 = reinterpret_cast<const float *>(raw + kRawLa)[lane] * kLog2e;
    const float beta = reinterpret_cast<const float *>(raw + kRawBeta)[lane];
    const float b2 = wave_cumsum(la2);
    float *gb = reinterpret_cast<float *>(smem + kOffG2);
    gb[lane] = b2;
    gb[64 + lane] = beta;
    gb[128 + lane] = la2;
    {
        float *sc = reinterpret_cast<float *>(der + kDerSc);
        const float bC = lane_value(b2, 63);
        sc[lane] = beta;
        sc[64 + lane] = ex2(b2);
        sc[128 + lane] = ex2(pre ? b2 - la2 : b2);
        sc[192 + lane] = ex2(bC - b2);
        if (lane == 0) sc[256] = ex2(bC);
    }
    uint4 kf[4][4], qf[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            kf[i][ks] = row_frag(raw + kRawK, ro, i, ks);
            qf[i][ks] = row_frag(raw + kRawQ, ro, i, ks);
        }
    wave_lds_sync();
    float *adt = reinterpret_cast<float *>(smem + kOffAd);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // A_ii in standard orientation: lane holds rows 4g+r, column c
        const floatx4 gk = gram_u4(kf[i], kf[i]);
        // P_ii transposed: lane holds row 16i + c, columns 16i + 4g + r
        const floatx4 gq = gram_u4(kf[i], qf[i]);
        const floatx4 b4 = *reinterpret_cast<const floatx4 *>(gb + 16 * i + 4 * g);
        const floatx4 beta4 = *reinterpret_cast<const floatx4 *>(gb + 64 + 16 * i + 4 * g);
        const float bc = gb[16 * i + c];
        const float bread = pre ? bc - gb[128 + 16 * i + c] : bc;
        floatx4 a, p;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rr = 4 * g + r;
            const float ea = ex2(b4[r] - bc);      // exponent <= 0 where kept
            a[r] = (c < rr) ? beta4[r] * gk[r] * ea : 0.f;
            const float ep = ex2(bread - b4[r]);   // exponent <= 0 where kept
            const bool keep = pre ? (rr < c) : (rr <= c);
            p[r] = keep ? gq[r] * ep : 0.f;
        }
        *reinterpret_cast<floatx4 *>(adt + (i * 16 + c) * 16 + 4 * g) = a;
        *reinterpret_cast<uint2 *>(der + kDerP + pf_index(i, i >> 1) * 1024 + lane * 16 + 8 * (i & 1)) = pack4(p);
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
    // 16-deep A-operand fragment of T_ii: element (r, c) -> lane (c/4, r), slot c%4
    char *td = der + kDerTd + g * 512 + ((c >> 2) << 7) + 2 * (c & 3);
#pragma unroll
    for (int r = 0; r < 16; ++r) *reinterpret_cast<__bf16 *>(td + 8 * r) = (__bf16)acc[r];
}

// ------------------------------------------------------------------ wave 3: off-diagonal prep
// Decay factors are split at each 16-row tile: for rows in tile i and columns before it,
// e^{x_row - b_col} = e^{x_row - ref_i} * e^{ref_i - b_col} with both exponents <= 0
// (ref_i = b_{16i} for A and the post-write read, b_{16i-1} = b'_{16i} for the pre-write read).
__device__ __forceinline__ void prep_off(char *smem, const char *raw, char *der, bool pre, const RowFragOffsets &ro) {
    const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
    const float la2 = reinterpret_cast<const float *>(raw + kRawLa)[lane] * kLog2e;
    const float beta = reinterpret_cast<const float *>(raw + kRawBeta)[lane];
    const float b2 = wave_cumsum(la2);
    float *gw = reinterpret_cast<float *>(smem + kOffG3);
    {
        const int tile = lane >> 4;
        const float s0 = lane_value(b2, 0), s16 = lane_value(b2, 16), s32 = lane_value(b2, 32), s48 = lane_value(b2, 48);
        const float e15 = lane_value(b2, 15), e31 = lane_value(b2, 31), e47 = lane_value(b2, 47);
        const float ref = tile == 0 ? s0 : tile == 1 ? s16 : tile == 2 ? s32 : s48;
        const float refp_any = tile == 1 ? e15 : tile == 2 ? e31 : e47;
        gw[lane] = beta * ex2(fminf(b2 - ref, 0.f));
        gw[64 + lane] = pre ? ex2(fminf(b2 - la2 - refp_any, 0.f)) : ex2(fminf(b2 - ref, 0.f));
#pragma unroll
        for (int i = 1; i < 4; ++i) {
            const float r1 = lane_value(b2, 16 * i);
            const float r2 = lane_value(b2, 16 * i - 1);
            const bool before = lane < 16 * i;
            gw[128 + (i - 1) * 64 + lane] = before ? ex2(r1 - b2) : 0.f;
            gw[320 + (i - 1) * 64 + lane] = before ? ex2((pre ? r2 : r1) - b2) : 0.f;
        }
    }
    uint4 kf[4][4], qf[3][4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int i = 0; i < 4; ++i) kf[i][ks] = row_frag(raw + kRawK, ro, i, ks);
#pragma unroll
        for (int i = 1; i < 4; ++i) qf[i - 1][ks] = row_frag(raw + kRawQ, ro, i, ks);
    }
    wave_lds_sync();
    char *na = der + kDerNA;
#pragma unroll
    for (int i = 1; i < 4; ++i) {
        const float ar = gw[16 * i + c];          // beta * rowfA of row 16i + c
        const float pr = gw[64 + 16 * i + c];     // rowfP of row 16i + c
#pragma unroll
        for (int j = 0; j < i; ++j) {
            // transposed tiles: lane holds row 16i + c, columns 16j + 4g + r
            const floatx4 gk = gram_u4(kf[j], kf[i]);
            const floatx4 gq = gram_u4(kf[j], qf[i - 1]);
            const floatx4 cA = *reinterpret_cast<const floatx4 *>(gw + 128 + (i - 1) * 64 + 16 * j + 4 * g);
            const floatx4 cP = *reinterpret_cast<const floatx4 *>(gw + 320 + (i - 1) * 64 + 16 * j + 4 * g);
            const floatx4 av = (-ar) * cA * gk;
            const floatx4 pv = pr * cP * gq;
            int aoff;
            if (i == 1) aoff = lane * 8;                           // A10, 16-deep
            else if (i == 2) aoff = 512 + lane * 16 + 8 * j;       // A20 | A21
            else if (j < 2) aoff = 1536 + lane * 16 + 8 * j;       // A30 | A31
            else aoff = 2560 + lane * 8;                           // A32, 16-deep
            *reinterpret_cast<uint2 *>(na + aoff) = pack4(av);
            *reinterpret_cast<uint2 *>(der + kDerP + pf_index(i, j >> 1) * 1024 + lane * 16 + 8 * (j & 1)) = pack4(pv);
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
    if (wave >= 2) {
        if (nchunks == 0) return;
        RowFragOffsets ro;
        ro.init();
        // the upper 16x16 tiles inside P fragments 0 and 3 are never written: zero them
        for (int d = 0; d < 2; ++d) {
            char *pf = smem + kOffDer + d * kDerBytes + kDerP;
            *reinterpret_cast<uint2 *>(pf + (wave == 2 ? 0 : 3) * 1024 + lane * 16 + 8) = make_uint2(0, 0);
        }
        const __amdgpu_buffer_rsrc_t ra = slab_rsrc(ab, (t0 + len) * 4);
        const __amdgpu_buffer_rsrc_t rb = slab_rsrc(bb, (t0 + len) * 4);
        const __amdgpu_buffer_rsrc_t rk = slab_rsrc(kb, a.T * kDK * 2);
        const __amdgpu_buffer_rsrc_t rq = slab_rsrc(qb, a.T * kDK * 2);
        const __amdgpu_buffer_rsrc_t rv = slab_rsrc(vb + dcol0, a.T * a.dv * 2 - dcol0 * 2);
        // offsets of a full chunk (rmax = 63): the same for every full chunk
        CopyOffsets cfull;
        {
            ChunkRows full;
            full.lo = 0;
            full.rmax = kC - 1;
            full.fwd = fwd;
            cfull.init(full, a.dv);
        }
        auto issue = [&](int64_t ch) {
            char *rawn = smem + kOffRaw + (int)(ch % 3) * kRawBytes;
            const ChunkRows cr = chunk_rows(t0, len, fwd, ch);
            if (cr.rmax == kC - 1) {
                if (wave == 2) {
                    copy_kq(rawn + kRawK, rk, cfull, cr.lo);
                } else {
                    copy_kq(rawn + kRawQ, rq, cfull, cr.lo);
                    copy_v(rawn + kRawV, rv, cfull, cr.lo, a.dv);
                }
            } else {
                CopyOffsets cpart;
                cpart.init(cr, a.dv);
                if (wave == 2) {
                    copy_kq(rawn + kRawK, rk, cpart, cr.lo);
                } else {
                    copy_kq(rawn + kRawQ, rq, cpart, cr.lo);
                    copy_v(rawn + kRawV, rv, cpart, cr.lo, a.dv);
                }
            }
            if (wave == 3) copy_gates(rawn, ra, rb, cr);
        };
        auto finish = [&](int64_t) { wait_vmem(); };
        auto prep = [&](int64_t ch) {
            const char *rawp = smem + kOffRaw + (int)(ch % 3) * kRawBytes;
            char *derp = smem + kOffDer + (int)(ch & 1) * kDerBytes;
            if (wave == 2) prep_diag(smem, rawp, derp, pre, ro);
            else prep_off(smem, rawp, derp, pre, ro);
        };
        issue(0);
        finish(0);
        lds_barrier();
        if (nchunks > 1) issue(1);
        prep(0);
        if (nchunks > 1) finish(1);
        lds_barrier();
        for (int64_t ch = 0; ch < nchunks; ++ch) {
            if (ch + 2 < nchunks) issue(ch + 2);
            if (ch + 1 < nchunks) prep(ch + 1);
            if (ch + 2 < nchunks) finish(ch + 2);
            lds_barrier();
        }
        return;
    }

    // chain waves: stored state rows 16t + 4g + r (true row 32(t/2) + 8g + 4(t%2) + r),
    // column dcol of d_v
    const int dcol = dcol0 + wave * 16 + c;
    floatx4 H[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) H[t] = zero4();
    if (a.h0) {
        const float *hb = a.h0 + (seq * a.Hv + head) * kDK * a.dv + dcol;
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) H[t][r] = hb[(32 * (t >> 1) + 8 * g + 4 * (t & 1) + r) * a.dv];
    }
    RowFragOffsets ro;
    ro.init();
    KtOffsets ko;
    ko.init();
    const int voff = v_lane_offset(wave);
    const int scoff = 16 * g;  // bytes: rows 4g..4g+3 of a 16-row tile
    char *stg = smem + kOffStage + wave * 2048;
    char *stg_w = stg + 128 * g + 2 * c;
    if (nchunks > 0) {
        lds_barrier();
        lds_barrier();
    }

    for (int64_t ch = 0; ch < nchunks; ++ch) {
        const char *raw = smem + kOffRaw + (int)(ch % 3) * kRawBytes;
        const char *der = smem + kOffDer + (int)(ch & 1) * kDerBytes;
        const char *sc = der + kDerSc + scoff;
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
                XK[mi] = mma32(XK[mi], u4_frag(row_frag(raw + kRawK, ro, mi, ks)), hb);
                XQ[mi] = mma32(XQ[mi], u4_frag(row_frag(raw + kRawQ, ro, mi, ks)), hb);
            }
        }
        // R = beta (V - e^{b} X_K)
        floatx4 R[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const bf16x4 v4 = tr16(raw + kRawV + voff + 1024 * mi);
            const floatx4 be = *reinterpret_cast<const floatx4 *>(sc + 64 * mi);
            const floatx4 eb = *reinterpret_cast<const floatx4 *>(sc + 256 + 64 * mi);
#pragma unroll
            for (int r = 0; r < 4; ++r) R[mi][r] = be[r] * ((float)v4[r] - eb[r] * XK[mi][r]);
        }
        // U_i = T_ii (R_i - sum_{j<i} A_ij U_j)
        const char *na = der + kDerNA;
        const char *td = der + kDerTd;
        floatx4 U[4];
        U[0] = mma16(zero4(), der_frag_lo(td, 0), cvt4<__bf16>(R[0]));
        floatx4 S = mma16(R[1], der_frag_lo(na, 0), cvt4<__bf16>(U[0]));
        U[1] = mma16(zero4(), der_frag_lo(td, 1), cvt4<__bf16>(S));
        const Frag<__bf16> u01 = frag_from_acc<__bf16>(U[0], U[1]);
        S = mma32(R[2], der_frag(na + 512, 0), u01);
        floatx4 S3 = mma32(R[3], der_frag(na + 1536, 0), u01);
        U[2] = mma16(zero4(), der_frag_lo(td, 2), cvt4<__bf16>(S));
        S3 = mma16(S3, der_frag_lo(na + 2560, 0), cvt4<__bf16>(U[2]));
        U[3] = mma16(zero4(), der_frag_lo(td, 3), cvt4<__bf16>(S3));
        const Frag<__bf16> u23 = frag_from_acc<__bf16>(U[2], U[3]);
        // O = e^{b | b'} X_Q + P U
        floatx4 O[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const floatx4 er = *reinterpret_cast<const floatx4 *>(sc + 512 + 64 * mi);
            O[mi] = er * XQ[mi];
            O[mi] = mma32(O[mi], der_frag(der + kDerP, pf_index(mi, 0)), u01);
            if (mi >= 2) O[mi] = mma32(O[mi], der_frag(der + kDerP, pf_index(mi, 1)), u23);
        }
        // H <- e^{b_C} H + K^T diag(e^{b_C - b}) U
        floatx4 W[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const floatx4 ec = *reinterpret_cast<const floatx4 *>(sc + 768 + 64 * mi);
            W[mi] = ec * U[mi];
        }
        const float gC = *reinterpret_cast<const float *>(der + kDerSc + 1024);
        const Frag<__bf16> w01 = frag_from_acc<__bf16>(W[0], W[1]);
        const Frag<__bf16> w23 = frag_from_acc<__bf16>(W[2], W[3]);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            H[t] = H[t] * gC;
            H[t] = mma32(H[t], kt_frag(raw + kRawK, ko, t, 0), w01);
            H[t] = mma32(H[t], kt_frag(raw + kRawK, ko, t, 1), w23);
        }
        // outputs through a per-wave staging tile for 16-byte stores
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int r = 0; r < 4; ++r) *reinterpret_cast<__bf16 *>(stg_w + 512 * mi + 32 * r) = (__bf16)O[mi][r];
        wave_lds_sync();
        {
            const ChunkRows cr = chunk_rows(t0, len, fwd, ch);
            char *obase = reinterpret_cast<char *>(ob + cr.lo * a.dv + dcol0 + wave * 16);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int rrow = 32 * q + (lane >> 1);
                if (rrow <= cr.rmax) {
                    uint4 val = *reinterpret_cast<const uint4 *>(stg + 1024 * q + 16 * lane);
                    uint4 *dst = reinterpret_cast<uint4 *>(obase + (int64_t)cr.off(rrow) * (a.dv * 2) + 16 * (lane & 1));
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
        lds_barrier();
    }

    if (a.hT) {
        float *hb = a.hT + (seq * a.Hv + head) * kDK * a.dv + dcol;
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) hb[(32 * (t >> 1) + 8 * g + 4 * (t & 1) + r) * a.dv] = H[t][r];
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
