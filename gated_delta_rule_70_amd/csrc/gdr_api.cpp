// C ABI of the gated delta rule library: host-side argument validation and dispatch.
// Every check happens before anything is enqueued; see include/gdr.h for the contract.
#include "../../include/gdr.h"

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "gdr_kernels.hpp"

namespace {

thread_local char g_last_error[512] = "";

gdr_status_t fail(gdr_status_t s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

struct Range {
    const char *name;
    uintptr_t lo, hi;  // [lo, hi)
    bool present() const { return lo != 0 && hi > lo; }
};

Range rng(const char *name, const void *p, int64_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{name, lo, lo + (uintptr_t)(bytes > 0 ? bytes : 0)};
}

bool overlap(const Range &a, const Range &b) {
    return a.present() && b.present() && a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// product of non-negative sizes, or -1 on overflow past 2^62
int64_t prod(std::initializer_list<int64_t> xs) {
    int64_t r = 1;
    for (int64_t x : xs) {
        if (x < 0) return -1;
        if (x != 0 && r > (INT64_C(1) << 62) / x) return -1;
        r *= x;
    }
    return r;
}

int64_t elem_size(int32_t dtype) { return dtype == GDR_BF16 ? 2 : 4; }

// The names the two gate arguments carry in messages.
struct GateNames {
    const char *a, *b;
};

// A validated chunked-forward launch: everything the kernel needs, checked on the host.
struct ChunkCall {
    gdr::ChunkArgs a;
    int32_t dtype, chunk, dk;
};

gdr_status_t chunk_prepare(const void *q, const void *k, const void *v, const float *log_alpha,
                           const float *beta, const float *A_log, const float *dt_bias, bool gated,
                           const float *h0, const int32_t *cu_seqlens, int32_t chunk, void *out, float *hT,
                           const gdr_chunk_dims_t *dims, int32_t n_sub, ChunkCall *call);
gdr_status_t chunk_launch(const ChunkCall &call, void *stream);
gdr_status_t chunk_impl(const void *q, const void *k, const void *v, const float *log_alpha,
                        const float *beta, const float *A_log, const float *dt_bias, bool gated,
                        const float *h0, const int32_t *cu_seqlens, int32_t chunk, void *out, float *hT,
                        const gdr_chunk_dims_t *dims, void *stream, int32_t n_sub = 1);
gdr_status_t bidir_impl(const void *q, const void *k, const void *v, const float *la_f, const float *beta_f,
                        const float *la_r, const float *beta_r, const float *h0_f, const float *h0_r,
                        const int32_t *cu_seqlens, int32_t chunk, void *out, float *hT_f, float *hT_r,
                        const gdr_chunk_dims_t *dims, void *stream);
gdr_status_t decode_impl(const void *q, const void *k, const void *v, const float *log_alpha,
                         const float *beta, const float *A_log, const float *dt_bias, bool gated,
                         const float *state_in, float *state_out, void *out, const gdr_decode_dims_t *dims,
                         void *stream);

}  // namespace

extern "C" {

int32_t gdr_abi_version(void) { return 1; }

const char *gdr_last_error(void) { return g_last_error; }

const char *gdr_status_string(gdr_status_t s) {
    switch (s) {
    case GDR_OK: return "ok";
    case GDR_ERR_NULL: return "a required pointer is NULL";
    case GDR_ERR_DIMS: return "invalid or inconsistent sizes";
    case GDR_ERR_DTYPE: return "unknown dtype";
    case GDR_ERR_CHUNK: return "chunk must be 16, 32 or 64";
    case GDR_ERR_ALIGN: return "pointer not 16-byte aligned";
    case GDR_ERR_ALIAS: return "buffers overlap";
    case GDR_ERR_UNSUPPORTED: return "unsupported head size";
    case GDR_ERR_FLAGS: return "unknown flag bits";
    case GDR_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

gdr_status_t gdr_chunk_fwd(const void *q, const void *k, const void *v, const float *log_alpha,
                           const float *beta, const float *h0, const int32_t *cu_seqlens,
                           int32_t chunk, void *out, float *hT, const gdr_chunk_dims_t *dims,
                           void *stream) {
    return chunk_impl(q, k, v, log_alpha, beta, nullptr, nullptr, false, h0, cu_seqlens, chunk, out, hT, dims,
                      stream);
}

gdr_status_t gdr_chunk_fwd_gated(const void *q, const void *k, const void *v, const float *a, const float *b,
                                 const float *A_log, const float *dt_bias, const float *h0,
                                 const int32_t *cu_seqlens, int32_t chunk, void *out, float *hT,
                                 const gdr_chunk_dims_t *dims, void *stream) {
    return chunk_impl(q, k, v, a, b, A_log, dt_bias, true, h0, cu_seqlens, chunk, out, hT, dims, stream);
}

gdr_status_t gdr_chunk_fwd_bidir(const void *q, const void *k, const void *v, const float *log_alpha_fwd,
                                 const float *beta_fwd, const float *log_alpha_rev, const float *beta_rev,
                                 const float *h0_fwd, const float *h0_rev, const int32_t *cu_seqlens, int32_t chunk,
                                 void *out, float *hT_fwd, float *hT_rev, const gdr_chunk_dims_t *dims,
                                 void *stream) {
    return bidir_impl(q, k, v, log_alpha_fwd, beta_fwd, log_alpha_rev, beta_rev, h0_fwd, h0_rev, cu_seqlens, chunk,
                      out, hT_fwd, hT_rev, dims, stream);
}

gdr_status_t gdr_delta_product_fwd(const void *q, const void *k, const void *v, const float *log_alpha,
                                   const float *beta, const float *h0, const int32_t *cu_seqlens, int32_t n_delta,
                                   int32_t chunk, void *out, float *hT, const gdr_chunk_dims_t *dims, void *stream) {
    return chunk_impl(q, k, v, log_alpha, beta, nullptr, nullptr, false, h0, cu_seqlens, chunk, out, hT, dims,
                      stream, n_delta);
}

gdr_status_t gdr_decode_step(const void *q, const void *k, const void *v, const float *log_alpha,
                             const float *beta, const float *state_in, float *state_out, void *out,
                             const gdr_decode_dims_t *dims, void *stream) {
    return decode_impl(q, k, v, log_alpha, beta, nullptr, nullptr, false, state_in, state_out, out, dims, stream);
}

gdr_status_t gdr_decode_step_gated(const void *q, const void *k, const void *v, const float *a, const float *b,
                                   const float *A_log, const float *dt_bias, const float *state_in,
                                   float *state_out, void *out, const gdr_decode_dims_t *dims, void *stream) {
    return decode_impl(q, k, v, a, b, A_log, dt_bias, true, state_in, state_out, out, dims, stream);
}

}  // extern "C"

namespace {

gdr_status_t chunk_prepare(const void *q, const void *k, const void *v, const float *log_alpha,
                           const float *beta, const float *A_log, const float *dt_bias, bool gated,
                           const float *h0, const int32_t *cu_seqlens, int32_t chunk, void *out, float *hT,
                           const gdr_chunk_dims_t *dims, int32_t n_sub, ChunkCall *call) {
    const GateNames gn = gated ? GateNames{"a", "b"} : GateNames{"log_alpha", "beta"};
    if (!dims) return fail(GDR_ERR_NULL, "dims is NULL");
    const gdr_chunk_dims_t d = *dims;
    if (d.dtype != GDR_F32 && d.dtype != GDR_BF16) return fail(GDR_ERR_DTYPE, "dtype %d is not GDR_F32 or GDR_BF16", d.dtype);
    if (d.flags & ~(GDR_READ_PRE | GDR_REVERSE | GDR_ACCUMULATE | GDR_QK_L2NORM))
        return fail(GDR_ERR_FLAGS, "flags 0x%x has unknown bits", d.flags);
    if (chunk != 16 && chunk != 32 && chunk != 64) return fail(GDR_ERR_CHUNK, "chunk %d is not 16, 32 or 64", chunk);
    if (d.B < 0 || d.T < 0) return fail(GDR_ERR_DIMS, "B (%lld) and T (%lld) must be >= 0", (long long)d.B, (long long)d.T);
    if (d.Hk < 1 || d.Hv < 1 || d.Hv % d.Hk) return fail(GDR_ERR_DIMS, "Hv (%lld) must be a positive multiple of Hk (%lld)", (long long)d.Hv, (long long)d.Hk);
    if (d.dk != 64 && d.dk != 128) return fail(GDR_ERR_UNSUPPORTED, "dk %lld is not 64 or 128", (long long)d.dk);
    if (d.dv < 32 || d.dv > 256 || d.dv % 32) return fail(GDR_ERR_UNSUPPORTED, "dv %lld is not a multiple of 32 in [32, 256]", (long long)d.dv);
    if (n_sub < 1 || n_sub > 16) return fail(GDR_ERR_DIMS, "n_delta %d is not in [1, 16]", n_sub);
    if (n_sub > 1 && (d.flags & GDR_REVERSE))
        return fail(GDR_ERR_FLAGS, "GDR_REVERSE is not supported with n_delta > 1");
    if (d.T > INT32_MAX / n_sub) return fail(GDR_ERR_DIMS, "T * n_delta must be below 2^31");
    int64_t nseq = d.B;
    if (cu_seqlens) {
        if (d.B != 1) return fail(GDR_ERR_DIMS, "cu_seqlens needs B == 1 (got %lld)", (long long)d.B);
        if (d.num_seqs < 1) return fail(GDR_ERR_DIMS, "num_seqs (%lld) must be >= 1 with cu_seqlens", (long long)d.num_seqs);
        nseq = d.num_seqs;
    }
    const int64_t es = elem_size(d.dtype);
    const int64_t nq = prod({d.B, d.Hk, d.T, d.dk}), nv = prod({d.B, d.Hv, d.T, d.dv});
    const int64_t ng = prod({d.B, d.Hv, d.T}), ns = prod({nseq, d.Hv, d.dk, d.dv});
    // k, v and beta carry n_sub rows per token
    const int64_t nk = prod({nq, n_sub}), nvs = prod({nv, n_sub}), ngs = prod({ng, n_sub});
    if (nq < 0 || nv < 0 || ng < 0 || ns < 0 || nk < 0 || nvs < 0 || ngs < 0 || nk > (INT64_C(1) << 60) / es)
        return fail(GDR_ERR_DIMS, "sizes overflow");
    if (nq > 0 && (!q || !k)) return fail(GDR_ERR_NULL, "q or k is NULL");
    if (nv > 0 && (!v || !out)) return fail(GDR_ERR_NULL, "v or out is NULL");
    if (ng > 0 && (!log_alpha || !beta)) return fail(GDR_ERR_NULL, "%s or %s is NULL", gn.a, gn.b);
    if (gated && (!A_log || !dt_bias)) return fail(GDR_ERR_NULL, "A_log or dt_bias is NULL");
    if ((A_log && !aligned(A_log, 4)) || (dt_bias && !aligned(dt_bias, 4)))
        return fail(GDR_ERR_ALIGN, "A_log or dt_bias is not 4-byte aligned");
    const void *al16[] = {q, k, v, out, h0, hT};
    const char *al16n[] = {"q", "k", "v", "out", "h0", "hT"};
    for (int i = 0; i < 6; ++i)
        if (al16[i] && !aligned(al16[i], 16)) return fail(GDR_ERR_ALIGN, "%s is not 16-byte aligned", al16n[i]);
    if ((log_alpha && !aligned(log_alpha, 4)) || (beta && !aligned(beta, 4)) || (cu_seqlens && !aligned(cu_seqlens, 4)))
        return fail(GDR_ERR_ALIGN, "%s, %s or cu_seqlens is not 4-byte aligned", gn.a, gn.b);

    const Range rq = rng("q", q, nq * es), rk = rng("k", k, nk * es), rv = rng("v", v, nvs * es);
    const Range ra = rng(gn.a, log_alpha, ng * 4), rb = rng(gn.b, beta, ngs * 4);
    const Range rh0 = rng("h0", h0, ns * 4), rhT = rng("hT", hT, ns * 4);
    const Range rcu = rng("cu_seqlens", cu_seqlens, cu_seqlens ? (nseq + 1) * 4 : 0);
    const Range ro = rng("out", out, nv * es);
    const Range rA = rng("A_log", A_log, gated ? d.Hv * 4 : 0), rdt = rng("dt_bias", dt_bias, gated ? d.Hv * 4 : 0);
    const Range ins[] = {rq, rk, rv, ra, rb, rh0, rcu, rA, rdt};
    for (const Range &r : ins) {
        if (overlap(ro, r)) return fail(GDR_ERR_ALIAS, "out overlaps %s", r.name);
        if (&r != &ins[5] && overlap(rhT, r)) return fail(GDR_ERR_ALIAS, "hT overlaps %s", r.name);
    }
    if (overlap(ro, rhT)) return fail(GDR_ERR_ALIAS, "out overlaps hT");
    if (overlap(rhT, rh0) && rhT.lo != rh0.lo) return fail(GDR_ERR_ALIAS, "hT partially overlaps h0");

    gdr::ChunkArgs a;
    a.q = q; a.k = k; a.v = v;
    a.log_alpha = log_alpha; a.beta = beta; a.h0 = h0;
    a.A_log = gated ? A_log : nullptr;
    a.dt_bias = gated ? dt_bias : nullptr;
    a.cu_seqlens = cu_seqlens;
    a.out = out; a.hT = hT;
    a.B = d.B; a.T = d.T; a.Hk = d.Hk; a.Hv = d.Hv; a.dv = d.dv;
    a.units = nseq * d.Hv;
    a.ntiles = d.dv / 32;
    a.flags = d.flags;
    a.n_sub = n_sub;
    const int64_t blocks = (a.units + 7) / 8 * 8 * a.ntiles;
    if (blocks > INT32_MAX) return fail(GDR_ERR_DIMS, "too many (sequence, head) units: %lld", (long long)a.units);
    call->a = a;
    call->dtype = d.dtype;
    call->chunk = chunk;
    call->dk = (int32_t)d.dk;
    return GDR_OK;
}

gdr_status_t chunk_launch(const ChunkCall &c, void *stream) {
    const hipError_t e = gdr::launch_chunk_fwd(c.a, c.dtype, c.chunk, c.dk, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GDR_ERR_HIP, "chunk forward launch: %s", hipGetErrorString(e));
    return GDR_OK;
}

gdr_status_t chunk_impl(const void *q, const void *k, const void *v, const float *log_alpha,
                        const float *beta, const float *A_log, const float *dt_bias, bool gated,
                        const float *h0, const int32_t *cu_seqlens, int32_t chunk, void *out, float *hT,
                        const gdr_chunk_dims_t *dims, void *stream, int32_t n_sub) {
    g_last_error[0] = '\0';
    ChunkCall call;
    const gdr_status_t s = chunk_prepare(q, k, v, log_alpha, beta, A_log, dt_bias, gated, h0, cu_seqlens, chunk,
                                         out, hT, dims, n_sub, &call);
    return s != GDR_OK ? s : chunk_launch(call, stream);
}

// Both scans of a bidirectional layer: the forward scan writes (or accumulates into) out, then
// the reverse scan accumulates into it. Both are validated before either is enqueued.
gdr_status_t bidir_impl(const void *q, const void *k, const void *v, const float *la_f, const float *beta_f,
                        const float *la_r, const float *beta_r, const float *h0_f, const float *h0_r,
                        const int32_t *cu_seqlens, int32_t chunk, void *out, float *hT_f, float *hT_r,
                        const gdr_chunk_dims_t *dims, void *stream) {
    g_last_error[0] = '\0';
    if (!dims) return fail(GDR_ERR_NULL, "dims is NULL");
    if (dims->flags & GDR_REVERSE)
        return fail(GDR_ERR_FLAGS, "GDR_REVERSE is not a flag of the bidirectional call (it runs both directions)");
    gdr_chunk_dims_t df = *dims, dr = *dims;
    dr.flags |= GDR_REVERSE | GDR_ACCUMULATE;
    ChunkCall cf, cr;
    char msg[sizeof(g_last_error)];
    gdr_status_t s = chunk_prepare(q, k, v, la_f, beta_f, nullptr, nullptr, false, h0_f, cu_seqlens, chunk, out,
                                   hT_f, &df, 1, &cf);
    if (s != GDR_OK) {
        snprintf(msg, sizeof(msg), "forward scan: %s", g_last_error);
        return fail(s, "%s", msg);
    }
    s = chunk_prepare(q, k, v, la_r, beta_r, nullptr, nullptr, false, h0_r, cu_seqlens, chunk, out, hT_r, &dr, 1,
                      &cr);
    if (s != GDR_OK) {
        snprintf(msg, sizeof(msg), "reverse scan: %s", g_last_error);
        return fail(s, "%s", msg);
    }
    // the forward scan's final state is written before the reverse scan reads its inputs, so it
    // must not overlap them; the reverse scan's final state is held to the same rule against the
    // forward scan's inputs (stream order alone would allow that overlap), and the two final
    // states must not overlap each other
    const int64_t ns = prod({cf.a.units, dims->dk, dims->dv}) * 4, ng = prod({dims->B, dims->Hv, dims->T}) * 4;
    const Range rhf = rng("hT_fwd", hT_f, ns), rhr = rng("hT_rev", hT_r, ns);
    const Range others_f[] = {rng("log_alpha_rev", la_r, ng), rng("beta_rev", beta_r, ng), rng("h0_rev", h0_r, ns),
                              rhr};
    const Range others_r[] = {rng("log_alpha_fwd", la_f, ng), rng("beta_fwd", beta_f, ng), rng("h0_fwd", h0_f, ns)};
    for (const Range &r : others_f)
        if (overlap(rhf, r)) return fail(GDR_ERR_ALIAS, "hT_fwd overlaps %s", r.name);
    for (const Range &r : others_r)
        if (overlap(rhr, r)) return fail(GDR_ERR_ALIAS, "hT_rev overlaps %s", r.name);
    s = chunk_launch(cf, stream);
    return s != GDR_OK ? s : chunk_launch(cr, stream);
}

gdr_status_t decode_impl(const void *q, const void *k, const void *v, const float *log_alpha,
                         const float *beta, const float *A_log, const float *dt_bias, bool gated,
                         const float *state_in, float *state_out, void *out, const gdr_decode_dims_t *dims,
                         void *stream) {
    g_last_error[0] = '\0';
    const GateNames gn = gated ? GateNames{"a", "b"} : GateNames{"log_alpha", "beta"};
    if (!dims) return fail(GDR_ERR_NULL, "dims is NULL");
    const gdr_decode_dims_t d = *dims;
    if (d.dtype != GDR_F32 && d.dtype != GDR_BF16) return fail(GDR_ERR_DTYPE, "dtype %d is not GDR_F32 or GDR_BF16", d.dtype);
    if (d.flags & ~(GDR_READ_PRE | GDR_QK_L2NORM))
        return fail(GDR_ERR_FLAGS, "flags 0x%x: decode takes GDR_READ_PRE and GDR_QK_L2NORM only", d.flags);
    if (d.N < 0) return fail(GDR_ERR_DIMS, "N (%lld) must be >= 0", (long long)d.N);
    if (d.Hk < 1 || d.Hv < 1 || d.Hv % d.Hk) return fail(GDR_ERR_DIMS, "Hv (%lld) must be a positive multiple of Hk (%lld)", (long long)d.Hv, (long long)d.Hk);
    if ((d.dk != 64 && d.dk != 128) || (d.dv != 64 && d.dv != 128))
        return fail(GDR_ERR_UNSUPPORTED, "dk (%lld) and dv (%lld) must be 64 or 128", (long long)d.dk, (long long)d.dv);
    const int64_t es = elem_size(d.dtype);
    const int64_t nq = prod({d.N, d.Hk, d.dk}), nv = prod({d.N, d.Hv, d.dv}), ng = prod({d.N, d.Hv});
    const int64_t ns = prod({d.N, d.Hv, d.dk, d.dv});
    if (nq < 0 || nv < 0 || ng < 0 || ns < 0 || ns > (INT64_C(1) << 60)) return fail(GDR_ERR_DIMS, "sizes overflow");
    if (d.N * d.Hv > INT32_MAX) return fail(GDR_ERR_DIMS, "N * Hv too large");
    if (d.N > 0 && (!q || !k || !v || !log_alpha || !beta || !state_in || !state_out || !out))
        return fail(GDR_ERR_NULL, "a tensor pointer is NULL");
    if (gated && (!A_log || !dt_bias)) return fail(GDR_ERR_NULL, "A_log or dt_bias is NULL");
    if ((A_log && !aligned(A_log, 4)) || (dt_bias && !aligned(dt_bias, 4)))
        return fail(GDR_ERR_ALIGN, "A_log or dt_bias is not 4-byte aligned");
    const void *al16[] = {q, k, v, out, state_in, state_out};
    const char *al16n[] = {"q", "k", "v", "out", "state_in", "state_out"};
    for (int i = 0; i < 6; ++i)
        if (al16[i] && !aligned(al16[i], 16)) return fail(GDR_ERR_ALIGN, "%s is not 16-byte aligned", al16n[i]);
    if ((log_alpha && !aligned(log_alpha, 4)) || (beta && !aligned(beta, 4)))
        return fail(GDR_ERR_ALIGN, "%s or %s is not 4-byte aligned", gn.a, gn.b);
    const Range rq = rng("q", q, nq * es), rk = rng("k", k, nq * es), rv = rng("v", v, nv * es);
    const Range ra = rng(gn.a, log_alpha, ng * 4), rb = rng(gn.b, beta, ng * 4);
    const Range rsi = rng("state_in", state_in, ns * 4), rso = rng("state_out", state_out, ns * 4);
    const Range ro = rng("out", out, nv * es);
    const Range rA = rng("A_log", A_log, gated ? d.Hv * 4 : 0), rdt = rng("dt_bias", dt_bias, gated ? d.Hv * 4 : 0);
    const Range ins[] = {rq, rk, rv, ra, rb, rsi, rA, rdt};
    for (const Range &r : ins) {
        if (overlap(ro, r)) return fail(GDR_ERR_ALIAS, "out overlaps %s", r.name);
        if (&r != &ins[5] && overlap(rso, r)) return fail(GDR_ERR_ALIAS, "state_out overlaps %s", r.name);
    }
    if (overlap(ro, rso)) return fail(GDR_ERR_ALIAS, "out overlaps state_out");
    if (overlap(rso, rsi) && rso.lo != rsi.lo) return fail(GDR_ERR_ALIAS, "state_out partially overlaps state_in");

    gdr::DecodeArgs a;
    a.q = q; a.k = k; a.v = v;
    a.log_alpha = log_alpha; a.beta = beta;
    a.A_log = gated ? A_log : nullptr;
    a.dt_bias = gated ? dt_bias : nullptr;
    a.state_in = state_in; a.state_out = state_out; a.out = out;
    a.N = d.N; a.Hk = d.Hk; a.Hv = d.Hv;
    a.flags = d.flags;
    const hipError_t e = gdr::launch_decode(a, d.dtype, (int)d.dk, (int)d.dv, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GDR_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
    return GDR_OK;
}

}  // namespace

namespace {

// Two-pass GDN-2 workspace: one slot per chunk of every sequence (packed: T / C + S + 1, which
// covers the slots cu[s] / C + s + c the kernels use), each holding a block per key head.
// Returns -1 for sizes that do not make sense.
int64_t gdn2_slots(const gdr_chunk_dims_t &d, int64_t chunk, bool packed) {
    if (packed) return d.T / chunk + d.num_seqs + 1;
    return d.B * ((d.T + chunk - 1) / chunk);
}
int64_t gdn2_ws_bytes(const gdr_chunk_dims_t &d, int32_t chunk, bool packed) {
    if ((d.dtype != GDR_F32 && d.dtype != GDR_BF16) || (chunk != 16 && chunk != 32 && chunk != 64) ||
        (d.dk != 64 && d.dk != 128) || d.T < 0 || d.B < 0 || d.Hk < 1 || d.Hv < 1 || d.dv < 0 ||
        (packed && d.num_seqs < 1))
        return -1;
    const int dt = d.dtype == GDR_BF16 ? gdr::kDtypeBf16 : gdr::kDtypeF32;
    const int64_t slots = gdn2_slots(d, chunk, packed);
    return prod({slots, d.Hk, gdr::gdn2_ws_key_bytes(dt, chunk, (int)d.dk)});
}

// A validated GDN-2 chunked-forward launch.
struct Gdn2Call {
    gdr::Gdn2Args a;
    int dtype, chunk, dk;
};

gdr_status_t gdn2_prepare(const void *q, const void *k, const void *v, const float *g, const void *b,
                          const void *w, const float *h0, const int32_t *cu_seqlens, int32_t chunk, void *out,
                          float *hT, void *workspace, int64_t workspace_bytes, const gdr_chunk_dims_t *dims,
                          Gdn2Call *call) {
    if (!dims) return fail(GDR_ERR_NULL, "dims is NULL");
    const gdr_chunk_dims_t d = *dims;
    if (d.dtype != GDR_F32 && d.dtype != GDR_BF16) return fail(GDR_ERR_DTYPE, "dtype %d is not GDR_F32 or GDR_BF16", d.dtype);
    if (d.flags & ~(GDR_READ_PRE | GDR_REVERSE | GDR_ACCUMULATE | GDR_QK_L2NORM))
        return fail(GDR_ERR_FLAGS, "flags 0x%x has unknown bits", d.flags);
    if (chunk != 16 && chunk != 32 && chunk != 64) return fail(GDR_ERR_CHUNK, "chunk %d is not 16, 32 or 64", chunk);
    if (d.B < 0 || d.T < 0) return fail(GDR_ERR_DIMS, "B (%lld) and T (%lld) must be >= 0", (long long)d.B, (long long)d.T);
    if (d.Hk < 1 || d.Hv < 1 || d.Hv % d.Hk) return fail(GDR_ERR_DIMS, "Hv (%lld) must be a positive multiple of Hk (%lld)", (long long)d.Hv, (long long)d.Hk);
    if (d.dk != 64 && d.dk != 128) return fail(GDR_ERR_UNSUPPORTED, "dk %lld is not 64 or 128", (long long)d.dk);
    if (d.dv < 32 || d.dv > 256 || d.dv % 32) return fail(GDR_ERR_UNSUPPORTED, "dv %lld is not a multiple of 32 in [32, 256]", (long long)d.dv);
    if (!gdr::gdn2_chunk_supported(d.dtype == GDR_BF16 ? gdr::kDtypeBf16 : gdr::kDtypeF32, chunk, (int)d.dk))
        return fail(GDR_ERR_CHUNK, "chunk 64 with fp32 and dk 128 does not fit in shared memory (use 16 or 32)");
    int64_t nseq = d.B;
    if (cu_seqlens) {
        if (d.B != 1) return fail(GDR_ERR_DIMS, "cu_seqlens needs B == 1 (got %lld)", (long long)d.B);
        if (d.num_seqs < 1) return fail(GDR_ERR_DIMS, "num_seqs (%lld) must be >= 1 with cu_seqlens", (long long)d.num_seqs);
        nseq = d.num_seqs;
    }
    const int64_t es = elem_size(d.dtype);
    const int64_t nq = prod({d.B, d.Hk, d.T, d.dk}), nv = prod({d.B, d.Hv, d.T, d.dv});
    const int64_t ns = prod({nseq, d.Hv, d.dk, d.dv});
    if (nq < 0 || nv < 0 || ns < 0 || nq > (INT64_C(1) << 59)) return fail(GDR_ERR_DIMS, "sizes overflow");
    if (nq > 0 && (!q || !k || !g || !b)) return fail(GDR_ERR_NULL, "q, k, g or b is NULL");
    if (nv > 0 && (!v || !w || !out)) return fail(GDR_ERR_NULL, "v, w or out is NULL");
    const void *al16[] = {q, k, v, g, b, w, out, h0, hT};
    const char *al16n[] = {"q", "k", "v", "g", "b", "w", "out", "h0", "hT"};
    for (int i = 0; i < 9; ++i)
        if (al16[i] && !aligned(al16[i], 16)) return fail(GDR_ERR_ALIGN, "%s is not 16-byte aligned", al16n[i]);
    if (cu_seqlens && !aligned(cu_seqlens, 4)) return fail(GDR_ERR_ALIGN, "cu_seqlens is not 4-byte aligned");

    const Range rq = rng("q", q, nq * es), rk = rng("k", k, nq * es), rv = rng("v", v, nv * es);
    const Range rg = rng("g", g, nq * 4), rb = rng("b", b, nq * es), rw = rng("w", w, nv * es);
    const Range rh0 = rng("h0", h0, ns * 4), rhT = rng("hT", hT, ns * 4);
    const Range rcu = rng("cu_seqlens", cu_seqlens, cu_seqlens ? (nseq + 1) * 4 : 0);
    const Range ro = rng("out", out, nv * es);
    const Range ins[] = {rq, rk, rv, rg, rb, rw, rh0, rcu};
    for (const Range &r : ins) {
        if (overlap(ro, r)) return fail(GDR_ERR_ALIAS, "out overlaps %s", r.name);
        if (&r != &ins[6] && overlap(rhT, r)) return fail(GDR_ERR_ALIAS, "hT overlaps %s", r.name);
    }
    if (overlap(ro, rhT)) return fail(GDR_ERR_ALIAS, "out overlaps hT");
    if (overlap(rhT, rh0) && rhT.lo != rh0.lo) return fail(GDR_ERR_ALIAS, "hT partially overlaps h0");
    int64_t nslots = 0;
    if (workspace) {
        const int64_t need = gdn2_ws_bytes(d, chunk, cu_seqlens != nullptr);
        if (need < 0) return fail(GDR_ERR_DIMS, "workspace size overflows");
        if (workspace_bytes < need)
            return fail(GDR_ERR_DIMS, "workspace_bytes %lld is below the %lld bytes needed", (long long)workspace_bytes,
                        (long long)need);
        if (!aligned(workspace, 16)) return fail(GDR_ERR_ALIGN, "workspace is not 16-byte aligned");
        const Range rws = rng("workspace", workspace, need);
        for (const Range &r : ins)
            if (overlap(rws, r)) return fail(GDR_ERR_ALIAS, "workspace overlaps %s", r.name);
        if (overlap(rws, ro) || overlap(rws, rhT)) return fail(GDR_ERR_ALIAS, "workspace overlaps out or hT");
        nslots = gdn2_slots(d, chunk, cu_seqlens != nullptr);
        if (nslots * d.Hk > INT32_MAX) return fail(GDR_ERR_DIMS, "too many chunks for the workspace pass");
    }

    gdr::Gdn2Args a;
    a.q = q; a.k = k; a.v = v; a.b = b; a.w = w;
    a.g = g; a.h0 = h0;
    a.cu_seqlens = cu_seqlens;
    a.out = out; a.hT = hT;
    a.B = d.B; a.T = d.T; a.Hk = d.Hk; a.Hv = d.Hv; a.dv = d.dv;
    a.units = nseq * d.Hv;
    a.ntiles = d.dv / 32;
    a.flags = d.flags;
    a.ws = workspace;
    a.nslots = nslots;
    const int64_t blocks = (a.units + 7) / 8 * 8 * a.ntiles;
    if (blocks > INT32_MAX) return fail(GDR_ERR_DIMS, "too many (sequence, head) units: %lld", (long long)a.units);
    call->a = a;
    call->dtype = d.dtype == GDR_BF16 ? gdr::kDtypeBf16 : gdr::kDtypeF32;
    call->chunk = chunk;
    call->dk = (int)d.dk;
    return GDR_OK;
}

gdr_status_t gdn2_launch(const Gdn2Call &c, void *stream) {
    const hipError_t e = gdr::launch_gdn2_chunk_fwd(c.a, c.dtype, c.chunk, c.dk, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GDR_ERR_HIP, "GDN-2 chunk forward launch: %s", hipGetErrorString(e));
    return GDR_OK;
}

gdr_status_t gdn2_chunk_impl(const void *q, const void *k, const void *v, const float *g, const void *b,
                             const void *w, const float *h0, const int32_t *cu_seqlens, int32_t chunk, void *out,
                             float *hT, void *workspace, int64_t workspace_bytes, const gdr_chunk_dims_t *dims,
                             void *stream) {
    g_last_error[0] = '\0';
    Gdn2Call call;
    const gdr_status_t s = gdn2_prepare(q, k, v, g, b, w, h0, cu_seqlens, chunk, out, hT, workspace, workspace_bytes,
                                        dims, &call);
    return s != GDR_OK ? s : gdn2_launch(call, stream);
}

// Both GDN-2 scans of a bidirectional layer: the forward scan writes (or accumulates into) out,
// then the reverse scan accumulates into it; both are validated before either is enqueued, and the
// two passes share the workspace one after the other.
gdr_status_t gdn2_bidir_impl(const void *q, const void *k, const void *v, const float *g_f, const void *b_f,
                             const void *w_f, const float *g_r, const void *b_r, const void *w_r, const float *h0_f,
                             const float *h0_r, const int32_t *cu_seqlens, int32_t chunk, void *out, float *hT_f,
                             float *hT_r, void *workspace, int64_t workspace_bytes, const gdr_chunk_dims_t *dims,
                             void *stream) {
    g_last_error[0] = '\0';
    if (!dims) return fail(GDR_ERR_NULL, "dims is NULL");
    if (dims->flags & GDR_REVERSE)
        return fail(GDR_ERR_FLAGS, "GDR_REVERSE is not a flag of the bidirectional call (it runs both directions)");
    gdr_chunk_dims_t df = *dims, dr = *dims;
    dr.flags |= GDR_REVERSE | GDR_ACCUMULATE;
    Gdn2Call cf, cr;
    char msg[sizeof(g_last_error)];
    gdr_status_t s = gdn2_prepare(q, k, v, g_f, b_f, w_f, h0_f, cu_seqlens, chunk, out, hT_f, workspace,
                                  workspace_bytes, &df, &cf);
    if (s != GDR_OK) {
        snprintf(msg, sizeof(msg), "forward scan: %s", g_last_error);
        return fail(s, "%s", msg);
    }
    s = gdn2_prepare(q, k, v, g_r, b_r, w_r, h0_r, cu_seqlens, chunk, out, hT_r, workspace, workspace_bytes, &dr,
                     &cr);
    if (s != GDR_OK) {
        snprintf(msg, sizeof(msg), "reverse scan: %s", g_last_error);
        return fail(s, "%s", msg);
    }
    // the forward scan's final state must not overlap an input of the reverse scan, which reads
    // them after it is written; the reverse scan's final state is held to the same rule against
    // the forward scan's inputs, and the two final states must not overlap each other (each
    // scan's own check already keeps the workspace off its inputs)
    const gdr_chunk_dims_t &d = *dims;
    const int64_t es = elem_size(d.dtype);
    const int64_t nk = prod({d.B, d.Hk, d.T, d.dk}), nvv = prod({d.B, d.Hv, d.T, d.dv});
    const int64_t ns = prod({cf.a.units, d.dk, d.dv}) * 4;
    const Range rhf = rng("hT_fwd", hT_f, ns), rhr = rng("hT_rev", hT_r, ns);
    const Range ins_r[] = {rng("g_rev", g_r, nk * 4), rng("b_rev", b_r, nk * es), rng("w_rev", w_r, nvv * es),
                           rng("h0_rev", h0_r, ns), rhr};
    const Range ins_f[] = {rng("g_fwd", g_f, nk * 4), rng("b_fwd", b_f, nk * es), rng("w_fwd", w_f, nvv * es),
                           rng("h0_fwd", h0_f, ns)};
    for (const Range &r : ins_r)
        if (overlap(rhf, r)) return fail(GDR_ERR_ALIAS, "hT_fwd overlaps %s", r.name);
    for (const Range &r : ins_f)
        if (overlap(rhr, r)) return fail(GDR_ERR_ALIAS, "hT_rev overlaps %s", r.name);
    s = gdn2_launch(cf, stream);
    return s != GDR_OK ? s : gdn2_launch(cr, stream);
}

gdr_status_t gdn2_decode_impl(const void *q, const void *k, const void *v, const float *g, const void *b,
                              const void *w, const float *state_in, float *state_out, void *out,
                              const gdr_decode_dims_t *dims, void *stream) {
    g_last_error[0] = '\0';
    if (!dims) return fail(GDR_ERR_NULL, "dims is NULL");
    const gdr_decode_dims_t d = *dims;
    if (d.dtype != GDR_F32 && d.dtype != GDR_BF16) return fail(GDR_ERR_DTYPE, "dtype %d is not GDR_F32 or GDR_BF16", d.dtype);
    if (d.flags & ~(GDR_READ_PRE | GDR_QK_L2NORM))
        return fail(GDR_ERR_FLAGS, "flags 0x%x: decode takes GDR_READ_PRE and GDR_QK_L2NORM only", d.flags);
    if (d.N < 0) return fail(GDR_ERR_DIMS, "N (%lld) must be >= 0", (long long)d.N);
    if (d.Hk < 1 || d.Hv < 1 || d.Hv % d.Hk) return fail(GDR_ERR_DIMS, "Hv (%lld) must be a positive multiple of Hk (%lld)", (long long)d.Hv, (long long)d.Hk);
    if ((d.dk != 64 && d.dk != 128) || (d.dv != 64 && d.dv != 128))
        return fail(GDR_ERR_UNSUPPORTED, "dk (%lld) and dv (%lld) must be 64 or 128", (long long)d.dk, (long long)d.dv);
    const int64_t es = elem_size(d.dtype);
    const int64_t nq = prod({d.N, d.Hk, d.dk}), nv = prod({d.N, d.Hv, d.dv});
    const int64_t ns = prod({d.N, d.Hv, d.dk, d.dv});
    if (nq < 0 || nv < 0 || ns < 0 || ns > (INT64_C(1) << 60)) return fail(GDR_ERR_DIMS, "sizes overflow");
    if (d.N * d.Hv > INT32_MAX) return fail(GDR_ERR_DIMS, "N * Hv too large");
    if (d.N > 0 && (!q || !k || !v || !g || !b || !w || !state_in || !state_out || !out))
        return fail(GDR_ERR_NULL, "a tensor pointer is NULL");
    const void *al16[] = {q, k, v, g, b, w, out, state_in, state_out};
    const char *al16n[] = {"q", "k", "v", "g", "b", "w", "out", "state_in", "state_out"};
    for (int i = 0; i < 9; ++i)
        if (al16[i] && !aligned(al16[i], 16)) return fail(GDR_ERR_ALIGN, "%s is not 16-byte aligned", al16n[i]);
    const Range rq = rng("q", q, nq * es), rk = rng("k", k, nq * es), rv = rng("v", v, nv * es);
    const Range rg = rng("g", g, nq * 4), rb = rng("b", b, nq * es), rw = rng("w", w, nv * es);
    const Range rsi = rng("state_in", state_in, ns * 4), rso = rng("state_out", state_out, ns * 4);
    const Range ro = rng("out", out, nv * es);
    const Range ins[] = {rq, rk, rv, rg, rb, rw, rsi};
    for (const Range &r : ins) {
        if (overlap(ro, r)) return fail(GDR_ERR_ALIAS, "out overlaps %s", r.name);
        if (&r != &ins[6] && overlap(rso, r)) return fail(GDR_ERR_ALIAS, "state_out overlaps %s", r.name);
    }
    if (overlap(ro, rso)) return fail(GDR_ERR_ALIAS, "out overlaps state_out");
    if (overlap(rso, rsi) && rso.lo != rsi.lo) return fail(GDR_ERR_ALIAS, "state_out partially overlaps state_in");

    gdr::Gdn2DecodeArgs a;
    a.q = q; a.k = k; a.v = v; a.b = b; a.w = w;
    a.g = g;
    a.state_in = state_in; a.state_out = state_out; a.out = out;
    a.N = d.N; a.Hk = d.Hk; a.Hv = d.Hv;
    a.flags = d.flags;
    const hipError_t e = gdr::launch_gdn2_decode(a, d.dtype == GDR_BF16 ? gdr::kDtypeBf16 : gdr::kDtypeF32, (int)d.dk,
                                                 (int)d.dv, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GDR_ERR_HIP, "GDN-2 decode launch: %s", hipGetErrorString(e));
    return GDR_OK;
}

}  // namespace

extern "C" {

gdr_status_t gdr_gdn2_chunk_fwd(const void *q, const void *k, const void *v, const float *g, const void *b,
                                const void *w, const float *h0, const int32_t *cu_seqlens, int32_t chunk,
                                void *out, float *hT, void *workspace, int64_t workspace_bytes,
                                const gdr_chunk_dims_t *dims, void *stream) {
    return gdn2_chunk_impl(q, k, v, g, b, w, h0, cu_seqlens, chunk, out, hT, workspace, workspace_bytes, dims,
                           stream);
}

gdr_status_t gdr_gdn2_chunk_fwd_bidir(const void *q, const void *k, const void *v, const float *g_fwd,
                                      const void *b_fwd, const void *w_fwd, const float *g_rev, const void *b_rev,
                                      const void *w_rev, const float *h0_fwd, const float *h0_rev,
                                      const int32_t *cu_seqlens, int32_t chunk, void *out, float *hT_fwd, float *hT_rev,
                                      void *workspace, int64_t workspace_bytes, const gdr_chunk_dims_t *dims,
                                      void *stream) {
    return gdn2_bidir_impl(q, k, v, g_fwd, b_fwd, w_fwd, g_rev, b_rev, w_rev, h0_fwd, h0_rev, cu_seqlens, chunk, out,
                           hT_fwd, hT_rev, workspace, workspace_bytes, dims, stream);
}

gdr_status_t gdr_gdn2_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const float *g, const void *b,
                                        const void *w, const float *h0, const int32_t *cu_seqlens, int32_t chunk,
                                        void *out, float *hT, const gdr_chunk_dims_t *dims, void *stream) {
    g_last_error[0] = '\0';
    if (!dims) return fail(GDR_ERR_NULL, "dims is NULL");
    const int64_t need = gdn2_ws_bytes(*dims, chunk, cu_seqlens != nullptr);
    if (need > gdr::kScratchBytes)
        return fail(GDR_ERR_DIMS, "these sizes need %lld bytes of workspace; the allocation-free entry point holds "
                    "%lld (GDR_NOALLOC_SCRATCH_BYTES): call gdr_gdn2_chunk_fwd with a workspace instead",
                    (long long)need, (long long)gdr::kScratchBytes);
    // need < 0 (unsupported dtype, chunk, dk or sizes) is reported by the checks of the call itself
    void *ws = nullptr;
    if (need > 0) {
        const hipError_t e = gdr::scratch_region(&ws);
        if (e != hipSuccess) return fail(GDR_ERR_HIP, "device scratch: %s", hipGetErrorString(e));
    }
    return gdn2_chunk_impl(q, k, v, g, b, w, h0, cu_seqlens, chunk, out, hT, ws, gdr::kScratchBytes, dims, stream);
}

int64_t gdr_gdn2_chunk_fwd_workspace_bytes(const gdr_chunk_dims_t *dims, int32_t chunk, int32_t packed) {
    if (!dims) return -1;
    return gdn2_ws_bytes(*dims, chunk, packed != 0);
}

gdr_status_t gdr_gdn2_decode_step(const void *q, const void *k, const void *v, const float *g, const void *b,
                                  const void *w, const float *state_in, float *state_out, void *out,
                                  const gdr_decode_dims_t *dims, void *stream) {
    return gdn2_decode_impl(q, k, v, g, b, w, state_in, state_out, out, dims, stream);
}

}  // extern "C"

namespace {

// chunk slots per value head: one per 64-token chunk of every sequence (packed: the slots of
// segment s start at cu[s] / 64 + s, so that no two segments share one)
int64_t bwd_slots(const gdr_chunk_dims_t &d, bool packed) {
    const int64_t CB = gdr::kBwdBlock;
    if (packed) return d.T / CB + d.num_seqs + 1;
    return d.B * ((d.T + CB - 1) / CB);
}

// Workspace of the backward, in this order: a record per (value head, slot) (the chunk's
// triangular inverse and read matrix as matrix-core operands, and its gate cumsums); the
// entry state and the exit-state adjoint of every chunk (dk x dv fp32 each); U and dR of every
// chunk (64 x dv fp32 each, rows past a segment's end included).
struct BwdLayout {
    int64_t rec, states, tokens, total;
};
BwdLayout bwd_layout(const gdr_chunk_dims_t &d, bool packed) {
    BwdLayout l;
    const int64_t slots = bwd_slots(d, packed);
    l.rec = prod({d.Hv, slots, gdr::kBwdRecBytes});
    l.states = prod({d.Hv, slots, d.dk, d.dv, 4});
    l.tokens = prod({d.Hv, slots, gdr::kBwdBlock, d.dv, 4});
    l.total = (l.rec < 0 || l.states < 0 || l.tokens < 0) ? -1 : l.rec + 2 * l.states + 2 * l.tokens;
    return l;
}
int64_t bwd_workspace_bytes(const gdr_chunk_dims_t &d, bool packed) { return bwd_layout(d, packed).total; }

gdr_status_t bwd_impl(const void *q, const void *k, const void *v, const float *log_alpha, const float *beta,
                      const float *h0, const int32_t *cu_seqlens, const void *dout, const float *dhT, float *dq,
                      float *dk, float *dv, float *dlog_alpha, float *dbeta, float *dh0, void *workspace,
                      int64_t workspace_bytes, const gdr_chunk_dims_t *dims, void *stream) {
    g_last_error[0] = '\0';
    if (!dims) return fail(GDR_ERR_NULL, "dims is NULL");
    const gdr_chunk_dims_t d = *dims;
    if (d.dtype != GDR_F32 && d.dtype != GDR_BF16) return fail(GDR_ERR_DTYPE, "dtype %d is not GDR_F32 or GDR_BF16", d.dtype);
    if (d.flags & ~(GDR_READ_PRE | GDR_REVERSE | GDR_ACCUMULATE))
        return fail(GDR_ERR_FLAGS, "flags 0x%x: the backward takes GDR_READ_PRE, GDR_REVERSE and GDR_ACCUMULATE", d.flags);
    if (d.B < 0 || d.T < 0) return fail(GDR_ERR_DIMS, "B (%lld) and T (%lld) must be >= 0", (long long)d.B, (long long)d.T);
    if (d.Hk < 1 || d.Hv < 1 || d.Hv % d.Hk) return fail(GDR_ERR_DIMS, "Hv (%lld) must be a positive multiple of Hk (%lld)", (long long)d.Hv, (long long)d.Hk);
    if (d.dk != 64 && d.dk != 128) return fail(GDR_ERR_UNSUPPORTED, "dk %lld is not 64 or 128", (long long)d.dk);
    if (d.dv < 32 || d.dv > 256 || d.dv % 32) return fail(GDR_ERR_UNSUPPORTED, "dv %lld is not a multiple of 32 in [32, 256]", (long long)d.dv);
    int64_t nseq = d.B;
    if (cu_seqlens) {
        if (d.B != 1) return fail(GDR_ERR_DIMS, "cu_seqlens needs B == 1 (got %lld)", (long long)d.B);
        if (d.num_seqs < 1) return fail(GDR_ERR_DIMS, "num_seqs (%lld) must be >= 1 with cu_seqlens", (long long)d.num_seqs);
        nseq = d.num_seqs;
    }
    const int64_t es = elem_size(d.dtype);
    const int64_t nq = prod({d.B, d.Hk, d.T, d.dk}), nv = prod({d.B, d.Hv, d.T, d.dv});
    const int64_t ng = prod({d.B, d.Hv, d.T}), ns = prod({nseq, d.Hv, d.dk, d.dv});
    const int64_t need = bwd_workspace_bytes(d, cu_seqlens != nullptr);
    if (nq < 0 || nv < 0 || ng < 0 || ns < 0 || need < 0 || nq > (INT64_C(1) << 59))
        return fail(GDR_ERR_DIMS, "sizes overflow");
    if (nq > 0 && (!q || !k || !dq || !dk)) return fail(GDR_ERR_NULL, "q, k, dq or dk is NULL");
    if (nv > 0 && (!v || !dout || !dv)) return fail(GDR_ERR_NULL, "v, dout or dv is NULL");
    if (ng > 0 && (!log_alpha || !beta || !dlog_alpha || !dbeta))
        return fail(GDR_ERR_NULL, "log_alpha, beta, dlog_alpha or dbeta is NULL");
    if (nseq * d.Hv > 0 && !workspace) return fail(GDR_ERR_NULL, "workspace is NULL");
    if (workspace_bytes < need)
        return fail(GDR_ERR_DIMS, "workspace_bytes %lld is below the %lld bytes this call needs", (long long)workspace_bytes, (long long)need);
    const void *al16[] = {q, k, v, dout, h0, dhT, dq, dk, dv, dh0, workspace};
    const char *al16n[] = {"q", "k", "v", "dout", "h0", "dhT", "dq", "dk", "dv", "dh0", "workspace"};
    for (int i = 0; i < 11; ++i)
        if (al16[i] && !aligned(al16[i], 16)) return fail(GDR_ERR_ALIGN, "%s is not 16-byte aligned", al16n[i]);
    if ((log_alpha && !aligned(log_alpha, 4)) || (beta && !aligned(beta, 4)) || (dlog_alpha && !aligned(dlog_alpha, 4)) ||
        (dbeta && !aligned(dbeta, 4)) || (cu_seqlens && !aligned(cu_seqlens, 4)))
        return fail(GDR_ERR_ALIGN, "a gate, gate gradient or cu_seqlens pointer is not 4-byte aligned");
    const Range ins[] = {rng("q", q, nq * es), rng("k", k, nq * es), rng("v", v, nv * es),
                         rng("log_alpha", log_alpha, ng * 4), rng("beta", beta, ng * 4), rng("h0", h0, ns * 4),
                         rng("cu_seqlens", cu_seqlens, cu_seqlens ? (nseq + 1) * 4 : 0), rng("dout", dout, nv * es),
                         rng("dhT", dhT, ns * 4)};
    const Range outs[] = {rng("dq", dq, nq * 4), rng("dk", dk, nq * 4), rng("dv", dv, nv * 4),
                          rng("dlog_alpha", dlog_alpha, ng * 4), rng("dbeta", dbeta, ng * 4), rng("dh0", dh0, ns * 4),
                          rng("workspace", workspace, need)};
    for (const Range &o : outs) {
        for (const Range &r : ins)
            if (overlap(o, r)) return fail(GDR_ERR_ALIAS, "%s overlaps %s", o.name, r.name);
        for (const Range &o2 : outs)
            if (&o2 != &o && overlap(o, o2)) return fail(GDR_ERR_ALIAS, "%s overlaps %s", o.name, o2.name);
    }
    gdr::BwdArgs a;
    a.q = q; a.k = k; a.v = v; a.dout = dout;
    a.log_alpha = log_alpha; a.beta = beta; a.h0 = h0; a.dhT = dhT;
    a.cu_seqlens = cu_seqlens;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dlog_alpha = dlog_alpha; a.dbeta = dbeta; a.dh0 = dh0;
    {
        const BwdLayout l = bwd_layout(d, cu_seqlens != nullptr);
        char *p = static_cast<char *>(workspace);
        a.rec = reinterpret_cast<uint8_t *>(p);
        a.hs = reinterpret_cast<float *>(p + l.rec);
        a.ds = reinterpret_cast<float *>(p + l.rec + l.states);
        a.us = reinterpret_cast<float *>(p + l.rec + 2 * l.states);
        a.drs = reinterpret_cast<float *>(p + l.rec + 2 * l.states + l.tokens);
    }
    a.B = d.B; a.T = d.T; a.Hk = d.Hk; a.Hv = d.Hv;
    a.nseq = nseq;
    a.units = nseq * d.Hv;
    a.nslots = bwd_slots(d, cu_seqlens != nullptr);
    a.ntiles = d.dv / gdr::kBwdCols;
    a.flags = d.flags;
    if (2 * a.units * a.ntiles > INT32_MAX || a.Hv * a.nslots > INT32_MAX)
        return fail(GDR_ERR_DIMS, "too many (sequence, head) units or chunks");
    const hipError_t e = gdr::launch_bwd(a, d.dtype, (int)d.dk, (int)d.dv, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GDR_ERR_HIP, "backward launch: %s", hipGetErrorString(e));
    return GDR_OK;
}

}  // namespace

extern "C" {

int64_t gdr_chunk_bwd_workspace_bytes(const gdr_chunk_dims_t *dims, int32_t packed) {
    if (!dims || dims->T < 0 || dims->B < 0 || dims->Hv < 1 || (packed && dims->num_seqs < 1)) return -1;
    return bwd_workspace_bytes(*dims, packed != 0);
}

gdr_status_t gdr_chunk_bwd(const void *q, const void *k, const void *v, const float *log_alpha, const float *beta,
                           const float *h0, const int32_t *cu_seqlens, const void *dout, const float *dhT, float *dq,
                           float *dk, float *dv, float *dlog_alpha, float *dbeta, float *dh0, void *workspace,
                           int64_t workspace_bytes, const gdr_chunk_dims_t *dims, void *stream) {
    return bwd_impl(q, k, v, log_alpha, beta, h0, cu_seqlens, dout, dhT, dq, dk, dv, dlog_alpha, dbeta, dh0,
                    workspace, workspace_bytes, dims, stream);
}

}  // extern "C"

extern "C" {

gdr_status_t gdr_selftest_mfma(const float *a, const float *b, float *d, void *stream) {
    g_last_error[0] = '\0';
    if (!a || !b || !d) return fail(GDR_ERR_NULL, "a, b and d must be device pointers");
    const hipError_t e = gdr::launch_selftest_mfma(a, b, d, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GDR_ERR_HIP, "selftest: %s", hipGetErrorString(e));
    return GDR_OK;
}

}  // extern "C"
