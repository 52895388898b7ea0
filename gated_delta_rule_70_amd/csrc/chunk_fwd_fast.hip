// Fast chunked forward for the common shape: bf16 q/k/v, chunk 64, d_k = 128, fp32 state.
//
// Same chunk algebra as chunk_fwd.hip (the WY/UT form of `chunked_delta` on the "Prizma
// seq/delta.py" page, with H = S^T), organised for the matrix cores of gfx950:
//
//   A   = diag(beta) Ah,  Ah = strict_lower((k_i . k_j) e^{b_i - b_j}),
//   T_ii = (I + A_ii)^{-1} = (I - A_ii)(I + A_ii^2)(I + A_ii^4)(I + A_ii^8)   (A_ii^16 = 0)
//   R   = V - diag(e^{b}) K H
//   U   by block forward substitution over the four 16-row blocks, with beta folded into the
//       diagonal inverses (U = (I + A)^{-1} diag(beta) R exactly):
//         U_i = (T_ii diag(beta_i)) (R_i - sum_{j<i} Ah_ij U_j)
//   O   = diag(e^{b} | e^{b'}) Q H + P U,   P = [(q_i . k_j) e^{b_i - b_j}]_{j<=i} (post)
//                                              [(q_i . k_j) e^{b'_i - b_j}]_{j<i}  (pre)
//   H  <- e^{b_C} H + K^T diag(e^{b_C - b}) U
//
// One workgroup = 8 waves per (sequence, value head, 32 columns of d_v), walking the chunks.
// Waves w and w + 4 share a SIMD.
//   waves 0, 1  "chain": the state-dependent part for chunk c, one 16-column tile each. The
//               state tiles stay in accumulator registers and are the B operands of K H and
//               Q H directly.
//   wave 2      diagonal prep for chunk c+1: gate scalars, diagonal tiles of K K^T and the
//               four 16x16 inverses T_ii as products of matrix-core squarings.
//   wave 3      off-diagonal tiles of K K^T (-> -A_ij) for chunk c+1, and the write-back of
//               the output of chunk c-1 from its staging tile.
//   waves 5, 7  the ten lower tiles of Q K^T with their decay factors (P) for chunk c+1.
//   waves 4, 6  copies for chunk c+2 (K; Q, V and gates) and L2 touches of chunk c+3; they
//               issue little.
// Raw q/k/v of a chunk are copied once per workgroup, global -> LDS directly (16 bytes per
// lane, no registers), into a ring of three buffers: while the chain reads chunk c and the
// prep waves read chunk c+1, the loads for chunk c+2 are in flight, and chunk c+3 is being
// brought into L2 so that those loads hit there. In K and Q the 16-byte
// pieces of a row are XOR-swizzled by a function of the row (row_swz) so that the
// row-fragment reads and the transposed K reads spread over the banks. The products the prep waves hand
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

#include <mutex>
#include <type_traits>

#include "gdr_kernels.hpp"
#include "gdr_mfma.hpp"

namespace gdr {

namespace {

constexpr int kC = 64, kDK = 128, kDVT = 32;
constexpr int kMaxDevices = 64;
// Wave roles. Waves w and w + 4 share a SIMD: each chain wave (0, 1) shares its SIMD with a
// copy wave, which issues little; the four prep waves take the other two SIMDs.
constexpr int kThreads = 512;
constexpr int kWaveCopyK = 4, kWaveCopyQ = 6, kWaveDiag = 2, kWaveP3 = 5, kWaveA = 3, kWaveP012 = 7;
constexpr int kWaveStore = kWaveA;  // the wave that writes the output back
constexpr float kLog2e = 1.4426950408889634f;

// raw buffer (one of three): K, Q [64 rows][256 B] and V [64 rows][64 B], swizzled; gates
constexpr int kRawK = 0, kRawQ = 16384, kRawV = 32768, kRawLa = 36864, kRawBeta = 37120;
// gate tables of the chunk, written into its raw buffer by the copy waves once their copies
// have arrived: inclusive log2 cumsum b [64]; read-side log decay [64]; P and -A decay
// factors (row factors [64], column factors [3][64] each); e^b, read scale, e^{bC-b} [64]
// each; e^{bC}; beta [64]; the row scales of k and q (1 / max(||row||, eps), or 1 without
// normalisation) [64] each
constexpr int kTabB2 = 37376, kTabBread = 37632, kTabGP = 37888, kTabGA = 38912;
constexpr int kTabEb = 39936, kTabEr = 40192, kTabEc = 40448, kTabGC = 40704;
constexpr int kTabBeta = 40720, kTabRk = 40976, kTabRq = 41232;
constexpr int kRawBytes = 41488;
// derived buffer (one of two)
constexpr int kDerP = 0;      // 6 P fragments (row tile, 32-deep slice) x 1 KB
constexpr int kDerNA = 6144;  // -A: A10 (16-deep, 512 B), A2x (1 KB), A3x (1 KB), A32 (16-deep, 512 B)
constexpr int kDerTd = 9216;  // T_ii: four 16-deep fragments of 512 B
constexpr int kDerBytes = 11264;
constexpr int kOffRaw = 0;
constexpr int kOffDer = kOffRaw + 3 * kRawBytes;
constexpr int kOffStage = kOffDer + 2 * kDerBytes;  // output staging, two of [32 cols][64 rows] bf16
constexpr int kStageBytes = 4096;
constexpr int kSortMax = 128;  // packed segments ranked by length (beyond, the order is kept)
// with accumulation, the output's previous values of a chunk, copied in like the V slice
constexpr int kOffPrev = kOffStage + 2 * kStageBytes;
constexpr int kPrevBytes = 4096;
// a word per lane that the L2 prefetch touches land in; nothing reads it
constexpr int kOffTouch = kOffPrev + 2 * kPrevBytes;
constexpr int kSmemBytes = kOffTouch + 256;
// L2 prefetch: how many steps ahead of its copies a chunk is touched, and the bytes one
// touch brings in (the L2 fills a miss by 32-byte sectors)
constexpr int kPfDist = 1;
constexpr int kPfSector = 32;
constexpr int kTouchPerQuarter = 4096 / kPfSector / 64;  // per quarter of a 16 KB K or Q chunk
static_assert(kSmemBytes <= 160 * 1024, "LDS budget");
static_assert((kSortMax + 2) * 4 <= kRawBytes, "segment offsets fit in a raw slot");

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
// Swizzle of the 16-byte pieces of K and Q row r: piece p is stored at p ^ row_swz(r). A
// 16-byte LDS read is served in four passes of sixteen lanes; on gfx950 a pass takes the
// lanes with equal bit 5 and equal parity of bits 4, 3 and 2 (measured), and is free of
// bank conflicts when its lanes address sixteen different pieces modulo 256 bytes. With
// r = 4a + b (a, b = 0..3), row_swz(r) = 4b + h(a), h = (0, 2, 3, 1): every pass of the
// row-fragment read (lane (g, c) reads row c, piece (4ks + g) ^ row_swz(c)) meets all sixteen
// pieces, and the sixteen lanes of a transposed K read that share g (rows 4g..4g+3, four
// neighbouring pieces each) also meet sixteen different pieces. A plain XOR with r % 16
// leaves the transposed read four lanes to a piece, which costs it 1.7x in LDS time.
__device__ __forceinline__ int row_swz(int r) {
    const int a = (r >> 2) & 3;
    return ((r & 3) << 2) | ((((a ^ (a >> 1)) & 1) << 1) | (a >> 1));
}
// With 2^sh delta sub-steps per token (scan rows), k, v and beta have a row per sub-step and
// q, log alpha and the output a row per token: scan row r of a chunk reads q row r >> sh
// (relative to the chunk's first token, lo >> sh; chunks start on a token since 2^sh divides
// the chunk), takes log alpha on the token's first sub-step only and gives the output of its
// token on one sub-step. With sh = 0 the two sets of offsets coincide.
struct CopyOffsets {
    int kq[16], q[16], v[4], o[4], gate, gate_la;
    __device__ __forceinline__ void init(const ChunkRows &cr, int64_t dv, int sh) {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int n = 0; n < 16; ++n) {
            const int row = 4 * n + (lane >> 4);
            const int piece = ((lane & 15) ^ row_swz(row)) << 4;
            kq[n] = cr.off(row) * 256 + piece;
            q[n] = (cr.off(row) >> sh) * 256 + piece;
        }
        const int rowb = (int)(dv * 2);
        const int piece = (lane & 3) ^ (lane >> 4);
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            v[n] = cr.off(16 * n + (lane >> 2)) * rowb + piece * 16;
            o[n] = (cr.off(16 * n + (lane >> 2)) >> sh) * rowb + piece * 16;
        }
        // rows past the end get an offset beyond the buffer, which reads as zero
        gate = lane <= cr.rmax ? cr.off(lane) * 4 : 0x40000000;
        gate_la = (lane <= cr.rmax && (lane & ((1 << sh) - 1)) == 0) ? (cr.off(lane) >> sh) * 4 : 0x40000000;
        // opaque to the optimiser, so they stay in their registers instead of being
        // recomputed into temporaries next to each copy
#pragma unroll
        for (int n = 0; n < 16; ++n) asm volatile("" : "+v"(kq[n]));
#pragma unroll
        for (int n = 0; n < 16; ++n) asm volatile("" : "+v"(q[n]));
#pragma unroll
        for (int n = 0; n < 4; ++n) asm volatile("" : "+v"(v[n]));
#pragma unroll
        for (int n = 0; n < 4; ++n) asm volatile("" : "+v"(o[n]));
        asm volatile("" : "+v"(gate));
        asm volatile("" : "+v"(gate_la));
    }
};
__device__ __forceinline__ void copy_kq(char *dst, u32x4 rsrc, const int (&offs)[16], int64_t lo) {
    const int soff = __builtin_amdgcn_readfirstlane((int)(lo * 256));
    const unsigned base = lds_addr(dst);
#pragma unroll
    for (int n = 0; n < 16; ++n) dma_b128(base + n * 1024, rsrc, offs[n], soff);
}
__device__ __forceinline__ void copy_v(char *dst, u32x4 rsrc, const int (&offs)[4], int64_t lo, int64_t dv) {
    const int soff = __builtin_amdgcn_readfirstlane((int)(lo * dv * 2));
    const unsigned base = lds_addr(dst);
#pragma unroll
    for (int n = 0; n < 4; ++n) dma_b128(base + n * 1024, rsrc, offs[n], soff);
}
// Gates of the chunk (log alpha, beta) straight into the raw buffer: lane r loads row r.
__device__ __forceinline__ void copy_gates(char *raw, u32x4 ra, u32x4 rb, const CopyOffsets &co, int64_t lo, int sh) {
    const int soff_la = __builtin_amdgcn_readfirstlane((int)((lo >> sh) * 4));
    const int soff = __builtin_amdgcn_readfirstlane((int)(lo * 4));
    dma_b32(lds_addr(raw + kRawLa), ra, co.gate_la, soff_la);
    dma_b32(lds_addr(raw + kRawBeta), rb, co.gate, soff);
}

// L2 prefetch of a later chunk. The ring holds three chunks, so a chunk's copies are issued
// one step before the step that needs them, and a step is shorter than a global-memory miss
// under full load. Touches issued kPfDist steps before the copies bring the chunk into L2,
// where its copies then hit. A touch is a one-dword load per lane into a scratch word of
// LDS: it has no destination register, and vector loads complete in issue order, so a wave
// waits for its copies with the count of touches issued after them still outstanding.
// The value tiles of a unit read the same K and Q chunk; tile t touches the quarters t,
// t + ntiles, ... of it (a tile takes nq quarter slots; a slot past the fourth quarter touches
// quarter slot mod 4 again). The chunk offset is clamped so that the touched range ends inside
// the slab; every lane addresses inside that range, so no touch depends on the buffer's range
// check (which a slab shorter than the range still gets).
struct TouchOffsets {
    int kq[4][kTouchPerQuarter], v[2], gate;
    __device__ __forceinline__ void init(int tile, int ntiles, int64_t dv) {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int q = tile + j * ntiles;
#pragma unroll
            for (int i = 0; i < kTouchPerQuarter; ++i) {
                kq[j][i] = (q & 3) * 4096 + (i * 64 + lane) * kPfSector;
                asm volatile("" : "+v"(kq[j][i]));
            }
        }
        // V: the tile's 64-byte slice of row `lane`; gates: the eight sectors of 32 bytes of
        // a chunk's 64 rows, each taken by eight lanes
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            v[i] = lane * (int)(dv * 2) + i * 32;
            asm volatile("" : "+v"(v[i]));
        }
        gate = (lane & 7) * 32;
        asm volatile("" : "+v"(gate));
    }
};
// quarter slots per tile: every quarter of K and Q is taken by one tile
__device__ __forceinline__ int touch_slots(int ntiles) { return ntiles >= 4 ? 1 : ntiles == 1 ? 4 : 2; }
// the chunk's byte offset in a slab, clamped so that [soff, soff + span) ends inside it
__device__ __forceinline__ int touch_soff(int64_t off, int64_t span, int64_t slab) {
    int64_t hi = slab - span;
    if (hi < 0) hi = 0;
    return __builtin_amdgcn_readfirstlane((int)(off < hi ? off : hi));
}
// lds: the scratch word's LDS address
__device__ __forceinline__ void touch_kq(unsigned lds, u32x4 rsrc, const TouchOffsets &to, int nq, int64_t row0, int64_t slab) {
    const int soff = touch_soff(row0 * 256, 16384, slab);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (j < nq) {
#pragma unroll
            for (int i = 0; i < kTouchPerQuarter; ++i) dma_b32(lds, rsrc, to.kq[j][i], soff);
        }
    }
}
__device__ __forceinline__ void touch_v(unsigned lds, u32x4 rsrc, const TouchOffsets &to, int64_t row0, int64_t dv, int64_t slab) {
    const int soff = touch_soff(row0 * dv * 2, 64 * dv * 2, slab);
    dma_b32(lds, rsrc, to.v[0], soff);
    dma_b32(lds, rsrc, to.v[1], soff);
}
__device__ __forceinline__ void touch_gate(unsigned lds, u32x4 rsrc, const TouchOffsets &to, int64_t row0, int64_t slab) {
    dma_b32(lds, rsrc, to.gate, touch_soff(row0 * 4, 256, slab));
}
// Waits until at most N vector loads of the wave are outstanding: with loads completing in
// issue order, all but the last N issued have landed.
template <int N>
__device__ __forceinline__ void vm_wait() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// the same with N = Base + PerSlot * nq, nq one of the quarter slot counts 1, 2, 4 (a count
// past the counter's range is cut to its maximum, which only waits for more)
constexpr int vm_cap(int n) { return n < 63 ? n : 63; }
template <int Base, int PerSlot>
__device__ __forceinline__ void vm_wait_slots(int nq) {
    if (nq >= 4) vm_wait<vm_cap(Base + 4 * PerSlot)>();
    else if (nq >= 2) vm_wait<vm_cap(Base + 2 * PerSlot)>();
    else vm_wait<vm_cap(Base + PerSlot)>();
}
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
// byte 4096 i + (256 c + 16 (g ^ row_swz(c))) ^ (ks << 6).
struct RowFragOffsets {
    int o[4];
    __device__ __forceinline__ void init() {
        const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
        const int base = 256 * c + ((g ^ row_swz(c)) << 4);
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
        const int z = (j & 3) ^ row_swz(r16);
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


// Gram tiles x_a . y_b for a list of (a, b) pairs, slice-outer so that consecutive products
// go to different accumulators and none waits for the previous one's result.
template <int N>
__device__ __forceinline__ void grams(floatx4 (&acc)[N], const uint4 (*x)[4], const uint4 (*y)[4], const int (&xa)[N],
                                      const int (&yb)[N]) {
#pragma unroll
    for (int n = 0; n < N; ++n) acc[n] = zero4();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int n = 0; n < N; ++n) acc[n] = mma32(acc[n], u4_frag(x[xa[n]][ks]), u4_frag(y[yb[n]][ks]));
}

__device__ __forceinline__ uint2 pack4(floatx4 v) { return __builtin_bit_cast(uint2, cvt4<__bf16>(v)); }

// ------------------------------------------------------------------ gate scalars
// The chunk's gates per token row (lane = row).
struct Gates {
    float la2, beta, b2;  // log2-scaled log alpha, beta, inclusive log2 cumsum
};

// ------------------------------------------------------------------ diagonal prep
// kL2: the k rows are scaled to unit length (their scales are in the chunk's table)
template <bool kL2, bool kPro>
__device__ __forceinline__ void prep_diag(char *smem, const char *raw, char *der, bool pre, const RowFragOffsets &ro) {
    const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
    (void)smem;
    (void)pre;
    const float *tb = reinterpret_cast<const float *>(raw + kTabB2);
    // beta: the table's (formed from a raw input) in the prologue form, else the copied input
    const float *rb = reinterpret_cast<const float *>(raw + (kPro ? kTabBeta : kRawBeta));
    const float *rk = reinterpret_cast<const float *>(raw + kTabRk);
    uint4 kf[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kf[i][ks] = row_frag(raw + kRawK, ro, i, ks);
    __builtin_amdgcn_sched_barrier(0);
    floatx4 gkk[4];
    grams<4>(gkk, kf, kf, {0, 1, 2, 3}, {0, 1, 2, 3});
    // B_i = A_ii^T in accumulator layout: lane (g, c) holds A_ii[c][4g + r] (row 16i + c of
    // the chunk, column 16i + 4g + r), from the symmetric Gram tile; the k row scales (1
    // without normalisation) multiply row and column.
    floatx4 bt[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const floatx4 gk = gkk[i];
        const floatx4 bcol = *reinterpret_cast<const floatx4 *>(tb + 16 * i + 4 * g);
        floatx4 rcol = {1.f, 1.f, 1.f, 1.f};
        float betarow = rb[16 * i + c];
        if constexpr (kL2) {
            rcol = *reinterpret_cast<const floatx4 *>(rk + 16 * i + 4 * g);
            betarow *= rk[16 * i + c];
        }
        const float brow = tb[16 * i + c];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            bt[i][r] = (4 * g + r < c) ? betarow * rcol[r] * gk[r] * ex2(brow - bcol[r]) : 0.f;
    }
    // T_ii = (I + A_ii)^{-1} = (I - A)(I + A^2)(I + A^4)(I + A^8), exact because the strictly
    // lower 16x16 A has A^16 = 0; all factors are polynomials in A, so they commute. On the
    // matrix cores: an accumulator-layout tile D(M) serves as the B operand M or as the A
    // operand M^T, and D(M^T) is D(M) multiplied by I with the operands swapped. Products
    // accumulate in fp32; operands are rounded to bf16. The four blocks run interleaved.
    floatx4 eye;
#pragma unroll
    for (int r = 0; r < 4; ++r) eye[r] = (4 * g + r == c) ? 1.f : 0.f;
    const bf16x4 eyeb = cvt4<__bf16>(eye);
    floatx4 da[4], a2[4], a2t[4], a4[4], a4t[4], a8[4], p1t[4], p2t[4], tt[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) da[i] = mma16(zero4(), cvt4<__bf16>(bt[i]), eyeb);              // D(A)
#pragma unroll
    for (int i = 0; i < 4; ++i) a2[i] = mma16(zero4(), cvt4<__bf16>(bt[i]), cvt4<__bf16>(da[i])); // D(A^2)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a2t[i] = mma16(zero4(), cvt4<__bf16>(a2[i]), eyeb);                                    // D(A^2T)
        const floatx4 imb = eye - bt[i];                                                       // D(I - A^T)
        p1t[i] = mma16(imb, cvt4<__bf16>(a2[i]), cvt4<__bf16>(imb));                           // (I + A^2T)(I - A^T)
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) a4[i] = mma16(zero4(), cvt4<__bf16>(a2t[i]), cvt4<__bf16>(a2[i])); // D(A^4)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a4t[i] = mma16(zero4(), cvt4<__bf16>(a4[i]), eyeb);                                    // D(A^4T)
        p2t[i] = mma16(p1t[i], cvt4<__bf16>(a4[i]), cvt4<__bf16>(p1t[i]));                     // (I + A^4T) P1^T
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) a8[i] = mma16(zero4(), cvt4<__bf16>(a4t[i]), cvt4<__bf16>(a4[i])); // D(A^8)
#pragma unroll
    for (int i = 0; i < 4; ++i) tt[i] = mma16(p2t[i], cvt4<__bf16>(a8[i]), cvt4<__bf16>(p2t[i]));  // D(T^T)
    // 16-deep A-operand fragment of T_ii diag(beta_i): lane (g, c) holds T[c][4g + r] (from
    // D(T^T)), scaled by the beta of column token 16i + 4g + r
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const floatx4 b4 = *reinterpret_cast<const floatx4 *>(rb + 16 * i + 4 * g);
        *reinterpret_cast<uint2 *>(der + kDerTd + i * 512 + lane * 8) = pack4(tt[i] * b4);
    }
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

// Gate tables of one chunk (raw buffer raw, gates already in LDS), for the prep waves and
// the chain: b = inclusive cumsum of log2 alpha over the chunk, the read-side log decay, the
// decay factors of the P and -A tiles split at 16-row references (no exponent is positive),
// and the chain's scalars.
// Row scales of a K or Q buffer ([64 rows][256 B], pieces swizzled within each row, which
// does not matter for a sum of squares): lane = row, 1 / max(||row||, eps), or 1 when the
// rows are used as given. Lane l reads the pieces of its row starting at piece l % 16, so
// that the sixteen lanes of each LDS pass address sixteen different pieces.
__device__ __forceinline__ float row_scales(const char *buf, float *dst, bool l2) {
    const int lane = threadIdx.x & 63;
    float r = 1.f;
    if (l2) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const char *row = buf + lane * 256;
        // all sixteen reads issued before the first use, so that their latencies overlap
        uint4 w[16];
#pragma unroll
        for (int p = 0; p < 16; ++p) w[p] = *reinterpret_cast<const uint4 *>(row + (((p + lane) & 15) << 4));
        __builtin_amdgcn_sched_barrier(0);
        float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < 16; ++p) {
            const unsigned u[4] = {w[p].x, w[p].y, w[p].z, w[p].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // two squares per instruction, accumulated in fp32 (four independent sums)
                const bf16x2 x = __builtin_bit_cast(bf16x2, u[e]);
                s[e] = __builtin_amdgcn_fdot2_f32_bf16(x, x, s[e], false);
            }
        }
        const float ss = (s[0] + s[1]) + (s[2] + s[3]);
        r = 1.f / fmaxf(sqrtf(ss), kL2Eps);
    }
    dst[lane] = r;
    return r;
}
// With row scales, the chain's scalars of the chunk take them (the chain then needs no extra
// product): e^b and e^{bC-b} those of k, the read scale those of q. The prep waves apply
// them where they read K and to the rows of P.
__device__ __forceinline__ void fold_row_scales(char *raw) {
    const int lane = threadIdx.x & 63;
    const float rk = reinterpret_cast<const float *>(raw + kTabRk)[lane];
    const float rq = reinterpret_cast<const float *>(raw + kTabRq)[lane];
    reinterpret_cast<float *>(raw + kTabEb)[lane] *= rk;
    reinterpret_cast<float *>(raw + kTabEc)[lane] *= rk;
    reinterpret_cast<float *>(raw + kTabEr)[lane] *= rq;
}

// Raw gate inputs of a gated call: the per-head parameters and the chunk's last valid row
// (rows past it are padding, with no decay and no write).
struct RawGates {
    bool raw;        // false: the gates arrive as log alpha and beta
    float nea, dtb;  // -exp(A_log[h]) and dt_bias[h] of the workgroup's value head
    int rmax;
};
template <bool kPro>
__device__ __forceinline__ void gate_tables(char *raw, bool pre, const RawGates &rg) {
    const int lane = threadIdx.x & 63;
    Gates gt;
    {
        const float x = reinterpret_cast<const float *>(raw + kRawLa)[lane];
        const float y = reinterpret_cast<const float *>(raw + kRawBeta)[lane];
        const bool valid = lane <= rg.rmax;
        float la = x, beta = y;
        if (rg.raw) {
            la = valid ? rg.nea * softplus_f(x + rg.dtb) : 0.f;
            beta = valid ? gate_beta(y) : 0.f;
        }
        gt.la2 = la * kLog2e;
        gt.beta = beta;
        gt.b2 = wave_cumsum(gt.la2);
    }
    if constexpr (kPro) reinterpret_cast<float *>(raw + kTabBeta)[lane] = gt.beta;
    float *tb = reinterpret_cast<float *>(raw + kTabB2);
    float *tr = reinterpret_cast<float *>(raw + kTabBread);
    float *gp = reinterpret_cast<float *>(raw + kTabGP);
    float *ga = reinterpret_cast<float *>(raw + kTabGA);
    float s0, s16, s32, s48, e15, e31, e47;
    tile_refs(gt.b2, s0, s16, s32, s48, e15, e31, e47);
    tb[lane] = gt.b2;
    tr[lane] = pre ? gt.b2 - gt.la2 : gt.b2;
    const int tile = lane >> 4;
    const float ref = tile == 0 ? s0 : tile == 1 ? s16 : tile == 2 ? s32 : s48;
    const float refp = tile == 1 ? e15 : tile == 2 ? e31 : e47;
    // P: row factor of row = lane (used for row tiles >= 1), column factors against the
    // reference of row tiles 1, 2, 3
    gp[lane] = pre ? ex2(fminf(gt.b2 - gt.la2 - refp, 0.f)) : ex2(fminf(gt.b2 - ref, 0.f));
    gp[64 + lane] = lane < 16 ? ex2((pre ? e15 : s16) - gt.b2) : 0.f;
    gp[128 + lane] = lane < 32 ? ex2((pre ? e31 : s32) - gt.b2) : 0.f;
    gp[192 + lane] = lane < 48 ? ex2((pre ? e47 : s48) - gt.b2) : 0.f;
    // -A: the same split for the write-side decays
    ga[lane] = ex2(fminf(gt.b2 - ref, 0.f));
    ga[64 + lane] = lane < 16 ? ex2(s16 - gt.b2) : 0.f;
    ga[128 + lane] = lane < 32 ? ex2(s32 - gt.b2) : 0.f;
    ga[192 + lane] = lane < 48 ? ex2(s48 - gt.b2) : 0.f;
    const float bC = lane_value(gt.b2, 63);
    reinterpret_cast<float *>(raw + kTabEb)[lane] = ex2(gt.b2);
    reinterpret_cast<float *>(raw + kTabEr)[lane] = ex2(pre ? gt.b2 - gt.la2 : gt.b2);
    reinterpret_cast<float *>(raw + kTabEc)[lane] = ex2(bC - gt.b2);
    if (lane == 0) reinterpret_cast<float *>(raw + kTabGC)[0] = ex2(bC);
}

// ------------------------------------------------------------------ P prep (row tiles I0 .. I1-1)
template <int I0, int I1, bool kL2>
__device__ __forceinline__ void prep_p(const char *raw, char *der, bool pre, const RowFragOffsets &ro) {
    const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
    const float *gw = reinterpret_cast<const float *>(raw + kTabGP);
    // log decay of the columns and read-side log decay of the rows, for the diagonal tiles
    const float *tb = reinterpret_cast<const float *>(raw + kTabB2);
    const float *tr = reinterpret_cast<const float *>(raw + kTabBread);
    // with unit-norm rows, the k row scales multiply the columns and the q row scales the rows
    const float *rk = reinterpret_cast<const float *>(raw + kTabRk);
    const float *rq = reinterpret_cast<const float *>(raw + kTabRq);
    uint4 kf[I1][4], qf[I1][4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int i = 0; i < I1; ++i) {
            kf[i][ks] = row_frag(raw + kRawK, ro, i, ks);
            if (i >= I0) qf[i][ks] = row_frag(raw + kRawQ, ro, i, ks);
        }
    __builtin_amdgcn_sched_barrier(0);
    char *pf = der + kDerP;
    // tiles (i, j), j <= i, in row order
    constexpr int NT = (I1 * (I1 + 1) - I0 * (I0 + 1)) / 2;
    int ti[NT], tj[NT];
    {
        int n = 0;
#pragma unroll
        for (int i = I0; i < I1; ++i)
#pragma unroll
            for (int j = 0; j <= i; ++j) {
                ti[n] = i;
                tj[n] = j;
                ++n;
            }
    }
    floatx4 gqk[NT];
    grams<NT>(gqk, kf, qf, tj, ti);
#pragma unroll
    for (int i = I0; i < I1; ++i) {
        // row 16i + c of this lane: its read decay and its row factor
        const float br = tr[16 * i + c];
        const float rqrow = kL2 ? rq[16 * i + c] : 1.f;
        const float rowf = gw[16 * i + c] * rqrow;
#pragma unroll
        for (int j = 0; j <= i; ++j) {
            // transposed tile: lane holds row 16i + c, columns 16j + 4g + r
            const floatx4 gq = gqk[(i * (i + 1) - I0 * (I0 + 1)) / 2 + j];
            floatx4 pv;
            floatx4 rcol = {1.f, 1.f, 1.f, 1.f};
            if constexpr (kL2) rcol = *reinterpret_cast<const floatx4 *>(rk + 16 * j + 4 * g);
            if (j < i) {
                const floatx4 cf = *reinterpret_cast<const floatx4 *>(gw + 64 * i + 16 * j + 4 * g);
                pv = rowf * cf * rcol * gq;
            } else {
                // diagonal tile: columns 16i + 4g + r against row 16i + c
                const floatx4 bcol = *reinterpret_cast<const floatx4 *>(tb + 16 * i + 4 * g);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int cc = 4 * g + r;
                    const bool keep = pre ? (cc < c) : (cc <= c);
                    pv[r] = keep ? rqrow * rcol[r] * gq[r] * ex2(br - bcol[r]) : 0.f;
                }
            }
            *reinterpret_cast<uint2 *>(pf + pf_index(i, j >> 1) * 1024 + lane * 16 + 8 * (j & 1)) = pack4(pv);
        }
    }
}

// ------------------------------------------------------------------ A prep
template <bool kL2>
__device__ __forceinline__ void prep_a(const char *raw, char *der, const RowFragOffsets &ro) {
    const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
    const float *gw = reinterpret_cast<const float *>(raw + kTabGA);
    const float *rk = reinterpret_cast<const float *>(raw + kTabRk);  // k row scales (1 without normalisation)
    uint4 kf[4][4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int i = 0; i < 4; ++i) kf[i][ks] = row_frag(raw + kRawK, ro, i, ks);
    __builtin_amdgcn_sched_barrier(0);
    char *na = der + kDerNA;
    floatx4 gkk[6];
    grams<6>(gkk, kf, kf, {0, 0, 1, 0, 1, 2}, {1, 2, 2, 3, 3, 3});
#pragma unroll
    for (int i = 1; i < 4; ++i) {
        const float ar = kL2 ? gw[16 * i + c] * rk[16 * i + c] : gw[16 * i + c];  // row factor of row 16i + c
#pragma unroll
        for (int j = 0; j < i; ++j) {
            // transposed tile: lane holds row 16i + c, columns 16j + 4g + r
            const floatx4 gk = gkk[(i * (i - 1)) / 2 + j];
            const floatx4 cf = *reinterpret_cast<const floatx4 *>(gw + 64 * i + 16 * j + 4 * g);
            floatx4 av = (-ar) * cf * gk;
            if constexpr (kL2) av *= *reinterpret_cast<const floatx4 *>(rk + 16 * j + 4 * g);
            int aoff;
            if (i == 1) aoff = lane * 8;                           // A10, 16-deep
            else if (i == 2) aoff = 512 + lane * 16 + 8 * j;       // A20 | A21
            else if (j < 2) aoff = 1536 + lane * 16 + 8 * j;       // A30 | A31
            else aoff = 2560 + lane * 8;                           // A32, 16-deep
            *reinterpret_cast<uint2 *>(na + aoff) = pack4(av);
        }
    }
}

// Write-back of one chunk's output from its staging tile. Transpose reads 2r and 2r+1 cover
// rows 16r .. 16r+15; in 16-lane group g, lane i addresses column 8g + 4h + i/4 (h = read
// parity) and rows 16r + 4(i%4) .. +3, so that lane i receives row 16r + i, columns 8g + 4h
// .. +3: the two reads give it 16 contiguous bytes of the output row.
// With acc_out, prv holds the output's previous values of the chunk in the V-slice layout
// (row R at 64 R bytes, 16-byte piece p at p ^ ((R % 16) / 4)). With 2^sh sub-steps per
// token, obase is the chunk's first token and row R is the output of token R >> sh when
// R % 2^sh = jread (the reading sub-step), and is dropped otherwise.
__device__ __forceinline__ void write_back(const char *stg, const char *prv, __bf16 *obase, const ChunkRows &cr,
                                           int64_t dv, bool acc_out, int sh, int jread) {
    const int lane = threadIdx.x & 63, g = lane >> 4, j = lane & 15;
    bf16x8 val[4], prev[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const bf16x4 lo = tr16(stg + stage_off(8 * g + (j >> 2), 4 * r + (j & 3)));
        const bf16x4 hi = tr16(stg + stage_off(8 * g + 4 + (j >> 2), 4 * r + (j & 3)));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            val[r][e] = lo[e];
            val[r][4 + e] = hi[e];
        }
        if (acc_out) prev[r] = *reinterpret_cast<const bf16x8 *>(prv + (16 * r + j) * 64 + ((g ^ (j >> 2)) << 4));
    }
    wave_lds_sync();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = 16 * r + j;
        if (row <= cr.rmax && (row & ((1 << sh) - 1)) == jread) {
            bf16x8 *dst = reinterpret_cast<bf16x8 *>(obase + (int64_t)(cr.off(row) >> sh) * dv + 8 * g);
            bf16x8 v = val[r];
            if (acc_out) {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = (__bf16)((float)v[e] + (float)prev[r][e]);
            }
            // streaming store: nothing in this kernel reads the output back, and with
            // ordinary stores the concurrent copies into LDS run measurably slower
            __builtin_nontemporal_store(v, dst);
        }
    }
}

// kPro: the form that takes the fused prologue (unit-norm q/k rows, gates from raw inputs);
// the plain form carries none of its code.
template <bool kPro>
__global__ __launch_bounds__(kThreads) void chunk_fwd_fast_kernel(ChunkArgs a) {
    extern __shared__ __align__(16) char smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c = lane & 15;

    const int64_t blk = blockIdx.x;
    const int64_t xcd = blk & 7, slot = blk >> 3;
    const int64_t unit = (slot / a.ntiles) * 8 + xcd;
    const int tile = (int)(slot % a.ntiles);
    if (unit >= a.units) return;
    int64_t seq = unit / a.Hv;
    const int64_t head = unit % a.Hv;
    const int64_t kh = head / (a.Hv / a.Hk);
    // Packed segments are taken longest first: unit ranks are dispatched in order, so the
    // workgroups of long segments start early and short ones fill in at the end (this is what
    // balances a few long segments of unequal length). Rank r goes to the segment with r longer
    // segments before it (ties by index), counted by the first nseq threads over all segments in
    // LDS: nseq^2 / 512 steps per thread, well under a microsecond up to kSortMax segments. With
    // more segments every workgroup is short and the order is kept as given.
    if (a.cu_seqlens) {
        const int nseq = (int)(a.units / a.Hv);
        if (nseq <= kSortMax) {
            int *cu = reinterpret_cast<int *>(smem + kOffRaw + 2 * kRawBytes);  // unused until chunk 2 is copied
            for (int i = tid; i <= nseq; i += kThreads) cu[i] = a.cu_seqlens[i];
            __syncthreads();
            const int rank = (int)seq;
            for (int s0 = tid; s0 < nseq; s0 += kThreads) {
                const int l0 = cu[s0 + 1] - cu[s0];
                int r = 0;
                for (int s1 = 0; s1 < nseq; ++s1) {
                    const int l1 = cu[s1 + 1] - cu[s1];
                    r += (l1 > l0) || (l1 == l0 && s1 < s0);
                }
                if (r == rank) cu[nseq + 1] = s0;
            }
            __syncthreads();
            seq = cu[nseq + 1];
            __syncthreads();
        }
    }
    const int64_t row = a.cu_seqlens ? 0 : seq;
    // scan rows: 2^sh delta sub-steps per token (sh = 0 for the plain rule); t0 and len count
    // scan rows, Ts is the scan length of a row of the batch
    const int sh = __builtin_ctz((unsigned)a.n_sub);
    const int64_t Ts = a.T << sh;
    int64_t t0 = 0, len = Ts;
    if (a.cu_seqlens) {
        t0 = (int64_t)a.cu_seqlens[seq] << sh;
        len = ((int64_t)a.cu_seqlens[seq + 1] << sh) - t0;
    }
    const bool fwd = (a.flags & kFlagReverse) == 0;
    const bool pre = (a.flags & kFlagReadPre) != 0;
    const bool acc_out = (a.flags & kFlagAccumulate) != 0;
    const bool l2 = kPro && (a.flags & kFlagL2Norm) != 0;
    const int64_t nchunks = (len + kC - 1) / kC;
    const int dcol0 = tile * kDVT;

    const __bf16 *kb = reinterpret_cast<const __bf16 *>(a.k) + (row * a.Hk + kh) * Ts * kDK;
    const __bf16 *qb = reinterpret_cast<const __bf16 *>(a.q) + (row * a.Hk + kh) * a.T * kDK;
    const __bf16 *vb = reinterpret_cast<const __bf16 *>(a.v) + (row * a.Hv + head) * Ts * a.dv;
    const float *ab = a.log_alpha + (row * a.Hv + head) * a.T;
    const float *bb = a.beta + (row * a.Hv + head) * Ts;
    __bf16 *ob = reinterpret_cast<__bf16 *>(a.out) + (row * a.Hv + head) * a.T * a.dv;
    // the sub-step whose row gives a token's output: its first (pre-write read) or last
    const int jread = pre ? 0 : (1 << sh) - 1;

    // The roles run separate loops with the same barrier sequence (two barriers in the
    // prologue, one per chunk), so each role's registers are live only in its own loop.
    if (wave >= 2) {
        if (nchunks == 0) return;
        RowFragOffsets ro;
        ro.init();
        // the upper 16x16 tiles inside P fragments 0 and 3 are never written: zero them
        if (wave == kWaveP012) {
            for (int d = 0; d < 2; ++d) {
                char *pf = smem + kOffDer + d * kDerBytes + kDerP;
                *reinterpret_cast<uint2 *>(pf + lane * 16 + 8) = make_uint2(0, 0);
                *reinterpret_cast<uint2 *>(pf + 3 * 1024 + lane * 16 + 8) = make_uint2(0, 0);
            }
        }
        // one loop per role, so that each keeps only its own loop-invariant registers
        auto run = [&](auto role) __attribute__((always_inline)) {
            constexpr int R = decltype(role)::value;
            constexpr bool kCopies = R == kWaveCopyK || R == kWaveCopyQ;
            // The K wave copies K (and Q in the prologue form) and computes the row norms; the G
            // wave copies the gates and V (and Q in the plain form), builds the gate tables and
            // folds the norms into them. The prologue form puts the norms on the wave that shares
            // its SIMD with the diagonal prep rather than with a chain wave.
            constexpr int kKW = kPro ? kWaveCopyQ : kWaveCopyK;
            constexpr int kGW = kPro ? kWaveCopyK : kWaveCopyQ;
            // the value head's gate parameters, read once (raw gate inputs only)
            bool raw_gates = false;
            float nea = 0.f, dtb = 0.f;
            if constexpr (kPro && R == kGW) {
                if (a.A_log) {
                    raw_gates = true;
                    nea = -__expf(a.A_log[head]);
                    dtb = a.dt_bias[head];
                }
            }
            u32x4 rsrc0, rsrc1, rsrc2, rsrc3, rsrc4;
            if constexpr (R == kKW) {
                rsrc0 = slab_rsrc(kb, Ts * kDK * 2);
                // the prologue form copies Q here too: this wave then owns both operands whose
                // row norms it computes
                if constexpr (kPro) rsrc1 = slab_rsrc(qb, a.T * kDK * 2);
            } else if constexpr (R == kGW) {
                rsrc0 = slab_rsrc(qb, a.T * kDK * 2);
                rsrc1 = slab_rsrc(vb + dcol0, Ts * a.dv * 2 - dcol0 * 2);
                rsrc4 = slab_rsrc(ob + dcol0, a.T * a.dv * 2 - dcol0 * 2);
                rsrc2 = slab_rsrc(ab, ((t0 + len) >> sh) * 4);
                rsrc3 = slab_rsrc(bb, (t0 + len) * 4);
            }
            // lane offsets of a full chunk (rmax = 63) and of the last chunk
            CopyOffsets cfull, clast;
            if constexpr (kCopies) {
                ChunkRows full;
                full.lo = 0;
                full.rmax = kC - 1;
                full.fwd = fwd;
                cfull.init(full, a.dv, sh);
                clast.init(chunk_rows(t0, len, fwd, nchunks - 1), a.dv, sh);
            }
            TouchOffsets to;
            const int nq = touch_slots((int)a.ntiles);
            const unsigned tl = lds_addr(smem + kOffTouch);
            if constexpr (kCopies) to.init(tile, (int)a.ntiles, a.dv);
            // L2 touches of chunk ch by this copy wave: kTouchBase + kTouchSlot * nq loads
            constexpr int kTouchBase = R == kKW ? 0 : 4;
            constexpr int kTouchSlot = (R == kKW ? (kPro ? 2 : 1) : (kPro ? 0 : 1)) * kTouchPerQuarter;
            // loads of one chunk's copies (K, Q, V slice, two gate rows)
            constexpr int kIssued = R == kKW ? (kPro ? 32 : 16) : (kPro ? 6 : 22);
            auto touch = [&](int64_t ch) __attribute__((always_inline)) {
                const int64_t lo = chunk_rows(t0, len, fwd, ch).lo;
                if constexpr (R == kKW) {
                    touch_kq(tl, rsrc0, to, nq, lo, Ts * kDK * 2);
                    if constexpr (kPro) touch_kq(tl, rsrc1, to, nq, lo >> sh, a.T * kDK * 2);
                } else {
                    if constexpr (!kPro) touch_kq(tl, rsrc0, to, nq, lo >> sh, a.T * kDK * 2);
                    touch_v(tl, rsrc1, to, lo, a.dv, Ts * a.dv * 2 - dcol0 * 2);
                    touch_gate(tl, rsrc2, to, lo >> sh, ((t0 + len) >> sh) * 4);
                    touch_gate(tl, rsrc3, to, lo, (t0 + len) * 4);
                }
            };
            // two explicit paths, so that each copy addresses with one of the fixed sets
            auto issue = [&](int64_t ch, const CopyOffsets &co) __attribute__((always_inline)) {
                char *rawn = smem + kOffRaw + (int)(ch % 3) * kRawBytes;
                const int64_t lo = chunk_rows(t0, len, fwd, ch).lo;
                if constexpr (R == kKW) {
                    copy_kq(rawn + kRawK, rsrc0, co.kq, lo);
                    if constexpr (kPro) copy_kq(rawn + kRawQ, rsrc1, co.q, lo >> sh);
                } else if constexpr (R == kGW) {
                    if constexpr (!kPro) copy_kq(rawn + kRawQ, rsrc0, co.q, lo >> sh);
                    copy_v(rawn + kRawV, rsrc1, co.v, lo, a.dv);
                    copy_gates(rawn, rsrc2, rsrc3, co, lo, sh);
                }
            };
            auto prep = [&](int64_t ch) __attribute__((always_inline)) {
                const char *rawp = smem + kOffRaw + (int)(ch % 3) * kRawBytes;
                char *derp = smem + kOffDer + (int)(ch & 1) * kDerBytes;
                // the two forms of each prep, with and without the k row scales
                if constexpr (R == kWaveDiag) {
                    if (l2) prep_diag<true, kPro>(smem, rawp, derp, pre, ro);
                    else prep_diag<false, kPro>(smem, rawp, derp, pre, ro);
                } else if constexpr (R == kWaveA) {
                    if (l2) prep_a<true>(rawp, derp, ro);
                    else prep_a<false>(rawp, derp, ro);
                } else if constexpr (R == kWaveP012) {
                    if (l2) prep_p<0, 3, true>(rawp, derp, pre, ro);
                    else prep_p<0, 3, false>(rawp, derp, pre, ro);
                } else if constexpr (R == kWaveP3) {
                    if (l2) prep_p<3, 4, true>(rawp, derp, pre, ro);
                    else prep_p<3, 4, false>(rawp, derp, pre, ro);
                }
            };
            auto store = [&](int64_t ch) __attribute__((always_inline)) {
                const ChunkRows cr = chunk_rows(t0, len, fwd, ch);
                write_back(smem + kOffStage + (int)(ch & 1) * kStageBytes, smem + kOffPrev + (int)(ch & 1) * kPrevBytes,
                           ob + (cr.lo >> sh) * a.dv + dcol0, cr, a.dv, acc_out, sh, jread);
            };
            // the wave that copies the gates builds the chunk's gate tables as soon as its copies
            // have landed, one chunk ahead of the prep waves that read them
            auto tables = [&](int64_t ch) __attribute__((always_inline)) {
                char *rawc = smem + kOffRaw + (int)(ch % 3) * kRawBytes;
                if constexpr (R == kGW) {
                    const RawGates rg{raw_gates, nea, dtb, chunk_rows(t0, len, fwd, ch).rmax};
                    gate_tables<kPro>(rawc, pre, rg);
                }
                // the k and q row scales, by the wave that copies K and Q in the prologue form
                if constexpr (R == kKW && kPro) {
                    if (l2) {
                        row_scales(rawc + kRawK, reinterpret_cast<float *>(rawc + kTabRk), true);
                        row_scales(rawc + kRawQ, reinterpret_cast<float *>(rawc + kTabRq), true);
                    }
                }
            };
            // One step later (the tables and the row scales of the chunk are complete then): the
            // row scales folded into the chain's scalars.
            auto qstage = [&](int64_t ch) __attribute__((always_inline)) {
                if constexpr (R == kGW) {
                    if (l2) fold_row_scales(smem + kOffRaw + (int)(ch % 3) * kRawBytes);
                }
            };
            auto step = [&](int64_t ch) __attribute__((always_inline)) {
                if (ch + 1 < nchunks) qstage(ch + 1);
                if constexpr (R == kGW) {
                    // with accumulation, the output's previous values of chunk ch, which the
                    // write-back adds in the next step
                    if (acc_out) {
                        char *prv = smem + kOffPrev + (int)(ch & 1) * kPrevBytes;
                        const int64_t lo = chunk_rows(t0, len, fwd, ch).lo;
                        if (ch == nchunks - 1) copy_v(prv, rsrc4, clast.o, lo >> sh, a.dv);
                        else copy_v(prv, rsrc4, cfull.o, lo >> sh, a.dv);
                    }
                }
                if constexpr (R == kWaveStore) {
                    if (ch >= 1) store(ch - 1);
                }
                // touches go after every copy that this step's wait must see land
                const bool touched = ch + 2 + kPfDist < nchunks;
                if constexpr (kCopies) {
                    if (touched) touch(ch + 2 + kPfDist);
                }
                if (ch + 1 < nchunks) prep(ch + 1);
                // the copy waves wait for their copies; the store wave's streaming stores
                // are not waited for (nothing reads them), and no other wave loads
                if constexpr (kCopies) {
                    if (touched) vm_wait_slots<kTouchBase, kTouchSlot>(nq);
                    else vm_wait<0>();
                }
                if (ch + 2 < nchunks) tables(ch + 2);
                lds_barrier();
            };
            // The first two chunks are copied together (ring slot 1 is not read before the
            // second barrier), then the touches of the next kPfDist chunks are issued.
            const bool touched = nchunks >= 2 + kPfDist;
            if constexpr (kCopies) {
                if (nchunks == 1) issue(0, clast);
                else issue(0, cfull);
                if (nchunks == 2) issue(1, clast);
                else if (nchunks > 2) issue(1, cfull);
                if (touched) {
                    for (int c2 = 2; c2 < 2 + kPfDist; ++c2) touch(c2);
                    vm_wait_slots<kIssued + kPfDist * kTouchBase, kPfDist * kTouchSlot>(nq);
                } else {
                    vm_wait<0>();
                }
            }
            tables(0);
            lds_barrier();
            qstage(0);
            prep(0);
            if constexpr (kCopies) {
                if (touched) vm_wait_slots<kPfDist * kTouchBase, kPfDist * kTouchSlot>(nq);
                else vm_wait<0>();
            }
            if (nchunks > 1) tables(1);
            lds_barrier();
            // The loop that copies full chunks and the tail that copies the last chunk are
            // separate code, so that no copy's offset register is chosen at run time.
            int64_t ch = 0;
            for (; ch + 3 < nchunks; ++ch) {
                if constexpr (kCopies) issue(ch + 2, cfull);
                step(ch);
            }
            for (; ch < nchunks; ++ch) {
                if constexpr (kCopies) {
                    if (ch + 2 < nchunks) issue(ch + 2, clast);
                }
                step(ch);
            }
            if constexpr (R == kWaveStore) store(nchunks - 1);
        };
        if (wave == kWaveDiag) run(std::integral_constant<int, kWaveDiag>{});
        else if (wave == kWaveA) run(std::integral_constant<int, kWaveA>{});
        else if (wave == kWaveP012) run(std::integral_constant<int, kWaveP012>{});
        else if (wave == kWaveP3) run(std::integral_constant<int, kWaveP3>{});
        else if (wave == kWaveCopyK) run(std::integral_constant<int, kWaveCopyK>{});
        else run(std::integral_constant<int, kWaveCopyQ>{});
        return;
    }

    // chain wave ct: stored state rows 16t + 4g + r (true row 32(t/2) + 8g + 4(t%2) + r) of
    // the 16-column tile ct, column dcol0 + 16 ct + c
    const int ct = wave;
    const int col = dcol0 + 16 * ct + c;
    floatx4 H[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) H[t] = zero4();
    if (a.h0) {
        const float *hb = a.h0 + (seq * a.Hv + head) * kDK * a.dv + col;
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) H[t][r] = hb[(32 * (t >> 1) + 8 * g + 4 * (t & 1) + r) * a.dv];
    }
    RowFragOffsets ro;
    ro.init();
    KtOffsets ko;
    ko.init();
    const int voff = v_lane_offset(ct);
    const int scoff = 16 * g;  // bytes: rows 4g..4g+3 of a 16-row tile
    if (nchunks > 0) {
        lds_barrier();
        lds_barrier();
    }
    // the first slice of K for X_K of the next chunk is read before each barrier (the raw
    // buffer of chunk c+1 is complete while chunk c runs)
    uint4 fk_next[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) fk_next[mi] = row_frag(smem + kOffRaw + kRawK, ro, mi, 0);

    // Per chunk: X_K = K H, then R, then the block substitution for U (a chain of dependent
    // small products) with the independent X_Q = Q H products interleaved into its gaps,
    // then the state update with the output products interleaved. Operands of a step are
    // read from LDS one step ahead, and scheduling fences keep that order.
    // The step is instantiated for the six phases of (ring slot, derived buffer) so that every
    // LDS address is a per-lane register plus a constant.
    auto step = [&](int64_t ch, auto phase) __attribute__((always_inline)) {
        constexpr int P = decltype(phase)::value;
        const char *raw = smem + kOffRaw + (P % 3) * kRawBytes;
        const char *der = smem + kOffDer + (P & 1) * kDerBytes;
        const char *sc = raw + kTabEb + scoff;  // e^b, then read scale and e^{bC-b} 256 B apart
        const char *na = der + kDerNA;
        const char *td = der + kDerTd;
        // ---- X_K = K H
        floatx4 XK[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) XK[mi] = zero4();
        uint4 fk[2][4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) fk[0][mi] = fk_next[mi];
        Frag<__bf16> hf[4];
        bf16x4 vv[4];
        floatx4 eb[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks < 3) {
#pragma unroll
                for (int mi = 0; mi < 4; ++mi) fk[(ks + 1) & 1][mi] = row_frag(raw + kRawK, ro, mi, ks + 1);
            } else {
#pragma unroll
                for (int mi = 0; mi < 4; ++mi) {
                    vv[mi] = tr16(raw + kRawV + voff + 1024 * mi);
                    eb[mi] = *reinterpret_cast<const floatx4 *>(sc + 64 * mi);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            hf[ks] = frag_from_acc<__bf16>(H[2 * ks], H[2 * ks + 1]);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) XK[mi] = mma32(XK[mi], u4_frag(fk[ks & 1][mi]), hf[ks]);
            __builtin_amdgcn_sched_barrier(0);
        }
        // ---- R = beta (V - e^{b} X_K); operands of the substitution and the first Q slice
        const bf16x4 t0f = der_frag_lo(td, 0), t1f = der_frag_lo(td, 1), t2f = der_frag_lo(td, 2), t3f = der_frag_lo(td, 3);
        const bf16x4 a10 = der_frag_lo(na, 0), a32 = der_frag_lo(na + 2560, 0);
        const Frag<__bf16> a2x = der_frag(na + 512, 0), a3x = der_frag(na + 1536, 0);
        uint4 fq[2][4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) fq[0][mi] = row_frag(raw + kRawQ, ro, mi, 0);
        __builtin_amdgcn_sched_barrier(0);
        floatx4 U[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int r = 0; r < 4; ++r) U[mi][r] = (float)vv[mi][r] - eb[mi][r] * XK[mi][r];
        __builtin_amdgcn_sched_barrier(0);
        // ---- U_i = T_ii (R_i - sum_{j<i} A_ij U_j) with X_Q = Q H interleaved: the sixteen
        // X_Q products (slice ks, row tile mi) fill the latency of each level
        floatx4 XQ[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) XQ[mi] = zero4();
        floatx4 er[4], ec[4];
        Frag<__bf16> kt[3][2];
        auto xq_items = [&](int first, int last) __attribute__((always_inline)) {
#pragma unroll
            for (int it = first; it < last; ++it) {
                const int ks = it >> 2, mi = it & 3;
                if (mi == 0) {
                    if (ks < 3) {
#pragma unroll
                        for (int m = 0; m < 4; ++m) fq[(ks + 1) & 1][m] = row_frag(raw + kRawQ, ro, m, ks + 1);
                    } else {
                        // operands of the state update and the output
#pragma unroll
                        for (int m = 0; m < 4; ++m) {
                            // the post-write read scale e^{b} is eb itself, unless eb carries the
                            // k row scales
                            er[m] = (pre || l2) ? *reinterpret_cast<const floatx4 *>(sc + 256 + 64 * m) : eb[m];
                            ec[m] = *reinterpret_cast<const floatx4 *>(sc + 512 + 64 * m);
                        }
                        kt[0][0] = kt_frag(raw + kRawK, ko, 0, 0);
                        kt[0][1] = kt_frag(raw + kRawK, ko, 0, 1);
                        kt[1][0] = kt_frag(raw + kRawK, ko, 1, 0);
                        kt[1][1] = kt_frag(raw + kRawK, ko, 1, 1);
                    }
                }
                XQ[mi] = mma32(XQ[mi], u4_frag(fq[ks & 1][mi]), hf[ks]);
            }
        };
        U[0] = mma16(zero4(), t0f, cvt4<__bf16>(U[0]));
        xq_items(0, 2);
        __builtin_amdgcn_sched_barrier(0);
        U[1] = mma16(U[1], a10, cvt4<__bf16>(U[0]));
        xq_items(2, 4);
        __builtin_amdgcn_sched_barrier(0);
        U[1] = mma16(zero4(), t1f, cvt4<__bf16>(U[1]));
        xq_items(4, 6);
        __builtin_amdgcn_sched_barrier(0);
        {
            const Frag<__bf16> u01 = frag_from_acc<__bf16>(U[0], U[1]);
            U[2] = mma32(U[2], a2x, u01);
            U[3] = mma32(U[3], a3x, u01);
        }
        xq_items(6, 9);
        __builtin_amdgcn_sched_barrier(0);
        U[2] = mma16(zero4(), t2f, cvt4<__bf16>(U[2]));
        xq_items(9, 11);
        __builtin_amdgcn_sched_barrier(0);
        U[3] = mma16(U[3], a32, cvt4<__bf16>(U[2]));
        xq_items(11, 13);
        __builtin_amdgcn_sched_barrier(0);
        U[3] = mma16(zero4(), t3f, cvt4<__bf16>(U[3]));
        xq_items(13, 16);
        __builtin_amdgcn_sched_barrier(0);
        // ---- H <- e^{b_C} H + K^T diag(e^{b_C - b}) U, with O = e^{b | b'} X_Q + P U
        // interleaved (output row tile t/2 after state tile t, for odd t)
        const float gC = *reinterpret_cast<const float *>(raw + kTabGC);
        Frag<__bf16> p[6];
#pragma unroll
        for (int f = 0; f < 6; ++f) p[f] = der_frag(der + kDerP, f);
        Frag<__bf16> w01, w23, u01, u23;
        {
            floatx4 W[4];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) W[mi] = ec[mi] * U[mi];
            w01 = frag_from_acc<__bf16>(W[0], W[1]);
            w23 = frag_from_acc<__bf16>(W[2], W[3]);
            u01 = frag_from_acc<__bf16>(U[0], U[1]);
            u23 = frag_from_acc<__bf16>(U[2], U[3]);
        }
        char *stg = smem + kOffStage + (P & 1) * kStageBytes;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            if (t < 6) {
                kt[(t + 2) % 3][0] = kt_frag(raw + kRawK, ko, t + 2, 0);
                kt[(t + 2) % 3][1] = kt_frag(raw + kRawK, ko, t + 2, 1);
            }
            __builtin_amdgcn_sched_barrier(0);
            H[t] = H[t] * gC;
            H[t] = mma32(H[t], kt[t % 3][0], w01);
            H[t] = mma32(H[t], kt[t % 3][1], w23);
            if (t & 1) {
                const int mi = t >> 1;
                floatx4 O = er[mi] * XQ[mi];
                if (mi < 2) {
                    O = mma32(O, p[mi], u01);
                } else {
                    O = mma32(O, p[2 * mi - 2], u01);
                    O = mma32(O, p[2 * mi - 1], u23);
                }
                *reinterpret_cast<uint2 *>(stg + stage_off(16 * ct + c, 4 * mi + g)) = pack4(O);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (ch + 1 < nchunks) {
            const char *raw_next = smem + kOffRaw + ((P + 1) % 3) * kRawBytes;
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) fk_next[mi] = row_frag(raw_next + kRawK, ro, mi, 0);
        }
        lds_barrier();
    };
    for (int64_t ch = 0; ch < nchunks; ch += 6) {
        step(ch, std::integral_constant<int, 0>{});
        if (ch + 1 >= nchunks) break;
        step(ch + 1, std::integral_constant<int, 1>{});
        if (ch + 2 >= nchunks) break;
        step(ch + 2, std::integral_constant<int, 2>{});
        if (ch + 3 >= nchunks) break;
        step(ch + 3, std::integral_constant<int, 3>{});
        if (ch + 4 >= nchunks) break;
        step(ch + 4, std::integral_constant<int, 4>{});
        if (ch + 5 >= nchunks) break;
        step(ch + 5, std::integral_constant<int, 5>{});
    }

    if (a.hT) {
        float *hb = a.hT + (seq * a.Hv + head) * kDK * a.dv + col;
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

// The LDS size attribute is set once per device and form; concurrent first launches from
// several host threads are serialised by the mutex.
template <bool kPro>
hipError_t configure_form() {
    static std::mutex mu;
    static bool done[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (done[dev]) return hipSuccess;
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&chunk_fwd_fast_kernel<kPro>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kSmemBytes);
    if (e == hipSuccess) done[dev] = true;
    return e;
}

template <bool kPro>
hipError_t launch_form(const ChunkArgs &a, hipStream_t stream) {
    const hipError_t ce = configure_form<kPro>();
    if (ce != hipSuccess) return ce;
    const int64_t blocks = (a.units + 7) / 8 * 8 * a.ntiles;
    hipLaunchKernelGGL(chunk_fwd_fast_kernel<kPro>, dim3((unsigned)blocks), dim3(kThreads), kSmemBytes, stream, a);
    return hipGetLastError();
}

hipError_t launch_chunk_fwd_fast(const ChunkArgs &a, hipStream_t stream) {
    if (a.A_log || (a.flags & kFlagL2Norm)) return launch_form<true>(a, stream);
    return launch_form<false>(a, stream);
}

}  // namespace gdr
