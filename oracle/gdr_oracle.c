/*
 * Gated delta rule: plain fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the reference the HIP library is
 * checked against. Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load it; the product path never does. It shares no
 * code, header or constant with the GPU library.
 *
 * What it computes (per token, no blocking, no reordering):
 *
 *   H_t = alpha_t * H_{t-1} + k_t u_t^T,   u_t = beta_t * (v_t - alpha_t * H_{t-1}^T k_t)
 *   post-write read:  o_t = H_t^T q_t
 *   pre-write read:   o_t = H_{t-1}^T q_t
 *
 * with alpha_t = exp(log_alpha_t). Sources:
 *   - "Prizma seq/delta.py" page, module docstring: S_t = alpha_t S_{t-1} + u_t k_t^T,
 *     u_t = beta_t (v_t - alpha_t S_{t-1} k_t), pre-write read o_t = S_{t-1} q_t;
 *     `_delta_reference`: per token, read first, then the erase term from the
 *     pre-update state, then decay and write.
 *   - "sparse-delta-memory layer.py" page, SparseDeltaMemory docstring: decay the
 *     memory by exp(g) and add beta*k(v - M k)^T (same update, post-write read).
 *   - "flashrt-structures fused_layer.py" page, `_decode_one`: the one-token core
 *     reads state_in and writes a separate state_out.
 *   - "tiny_gdn/fugue.py" page, `segment_layout` and `BidirectionalGatedDeltaNet2.scan`:
 *     packed segments given by cu_seqlens, state reset at each segment start, the
 *     backward direction scanning each segment reversed in place; `heads`: value
 *     head j uses key head floor(j / (Hv/Hk)).
 *
 * Layout (our reading): the page stores S as [d_v x d_k]; we store H = S^T as
 * row-major [d_k][d_v], so the read is o = H^T q.
 *
 * Tensors (all fp64, contiguous, row-major):
 *   q, k       [B][Hk][T][dk]
 *   v          [B][Hv][T][dv]
 *   log_alpha  [B][Hv][T]
 *   beta       [B][Hv][T]
 *   h0, hT     [nseq][Hv][dk][dv]     (h0 may be NULL: zero state; hT may be NULL)
 *   out        [B][Hv][T][dv]
 * Sequences: without cu_seqlens, sequence n is batch row n over tokens [0, T)
 * (nseq == B). With cu_seqlens (B == 1), sequence n covers tokens
 * [cu[n], cu[n+1]) of row 0.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define GDR_ORACLE_READ_PRE 1u
#define GDR_ORACLE_REVERSE 2u
#define GDR_ORACLE_ACCUMULATE 4u

int gdr_oracle_version(void) { return 1; }

/* One (sequence, value head) unit of the scan. H is dk*dv scratch. */
static void scan_unit(const double *q, const double *k, const double *v,
                      const double *log_alpha, const double *beta,
                      const double *h0, double *out, double *hT,
                      int64_t Hk, int64_t Hv, int64_t T, int64_t dk, int64_t dv,
                      int64_t row, int64_t head, int64_t t_begin, int64_t t_end,
                      int64_t seq, unsigned flags, double *H, double *x, double *o)
{
    const int64_t group = Hv / Hk;
    const int64_t khead = head / group;
    const double *qh = q + (row * Hk + khead) * T * dk;
    const double *kh = k + (row * Hk + khead) * T * dk;
    const double *vh = v + (row * Hv + head) * T * dv;
    const double *ah = log_alpha + (row * Hv + head) * T;
    const double *bh = beta + (row * Hv + head) * T;
    double *oh = out + (row * Hv + head) * T * dv;
    const int pre = (flags & GDR_ORACLE_READ_PRE) != 0;
    const int rev = (flags & GDR_ORACLE_REVERSE) != 0;
    const int acc = (flags & GDR_ORACLE_ACCUMULATE) != 0;

    /* step 1: H = h0 or 0 */
    if (h0) {
        memcpy(H, h0 + (seq * Hv + head) * dk * dv, (size_t)(dk * dv) * sizeof(double));
    } else {
        memset(H, 0, (size_t)(dk * dv) * sizeof(double));
    }

    const int64_t n = t_end - t_begin;
    for (int64_t s = 0; s < n; ++s) {
        /* scan position s visits token t (forward) or the mirror token (reverse) */
        const int64_t t = rev ? (t_end - 1 - s) : (t_begin + s);
        const double *qt = qh + t * dk;
        const double *kt = kh + t * dk;
        const double *vt = vh + t * dv;
        const double alpha = exp(ah[t]);
        const double b = bh[t];

        /* pre-write read: o = H_{t-1}^T q */
        if (pre) {
            for (int64_t c = 0; c < dv; ++c) o[c] = 0.0;
            for (int64_t r = 0; r < dk; ++r) {
                const double qr = qt[r];
                const double *Hr = H + r * dv;
                for (int64_t c = 0; c < dv; ++c) o[c] += Hr[c] * qr;
            }
        }
        /* erase term from the pre-update state: x = H_{t-1}^T k */
        for (int64_t c = 0; c < dv; ++c) x[c] = 0.0;
        for (int64_t r = 0; r < dk; ++r) {
            const double kr = kt[r];
            const double *Hr = H + r * dv;
            for (int64_t c = 0; c < dv; ++c) x[c] += Hr[c] * kr;
        }
        /* u = beta (v - alpha x), stored back into x */
        for (int64_t c = 0; c < dv; ++c) x[c] = b * (vt[c] - alpha * x[c]);
        /* H = alpha H + k u^T */
        for (int64_t r = 0; r < dk; ++r) {
            const double kr = kt[r];
            double *Hr = H + r * dv;
            for (int64_t c = 0; c < dv; ++c) Hr[c] = alpha * Hr[c] + kr * x[c];
        }
        /* post-write read: o = H_t^T q */
        if (!pre) {
            for (int64_t c = 0; c < dv; ++c) o[c] = 0.0;
            for (int64_t r = 0; r < dk; ++r) {
                const double qr = qt[r];
                const double *Hr = H + r * dv;
                for (int64_t c = 0; c < dv; ++c) o[c] += Hr[c] * qr;
            }
        }
        double *ot = oh + t * dv;
        if (acc) {
            for (int64_t c = 0; c < dv; ++c) ot[c] += o[c];
        } else {
            for (int64_t c = 0; c < dv; ++c) ot[c] = o[c];
        }
    }
    if (hT) memcpy(hT + (seq * Hv + head) * dk * dv, H, (size_t)(dk * dv) * sizeof(double));
}

/*
 * Full scan over every (sequence, value head) unit.
 * cu_seqlens: NULL, or nseq+1 int64 offsets (then B must be 1).
 * nthreads <= 0 uses the OpenMP default. Returns 0 on success, -1 on bad
 * arguments, -2 on allocation failure.
 */
int gdr_oracle_scan(const double *q, const double *k, const double *v,
                    const double *log_alpha, const double *beta, const double *h0,
                    const int64_t *cu_seqlens, int64_t nseq,
                    int64_t B, int64_t T, int64_t Hk, int64_t Hv, int64_t dk, int64_t dv,
                    unsigned flags, double *out, double *hT, int nthreads)
{
    if (!q || !k || !v || !log_alpha || !beta || !out) return -1;
    if (B < 0 || T < 0 || Hk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0 || Hv % Hk) return -1;
    if (cu_seqlens) {
        if (B != 1 || nseq < 0) return -1;
        if (cu_seqlens[0] != 0 || cu_seqlens[nseq] != T) return -1;
        for (int64_t n = 0; n < nseq; ++n)
            if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
    } else {
        nseq = B;
    }
    const int64_t units = nseq * Hv;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel reduction(|| : failed)
    {
        /* every thread reaches the worksharing loop, even if its malloc failed */
        double *H = (double *)malloc((size_t)(dk * dv + 2 * dv) * sizeof(double));
        double *x = H ? H + dk * dv : NULL;
        double *o = H ? x + dv : NULL;
#pragma omp for schedule(dynamic, 1)
        for (int64_t u = 0; u < units; ++u) {
            if (!H) { failed = 1; continue; }
            const int64_t seq = u / Hv;
            const int64_t head = u % Hv;
            const int64_t row = cu_seqlens ? 0 : seq;
            const int64_t tb = cu_seqlens ? cu_seqlens[seq] : 0;
            const int64_t te = cu_seqlens ? cu_seqlens[seq + 1] : T;
            scan_unit(q, k, v, log_alpha, beta, h0, out, hT, Hk, Hv, T, dk, dv,
                      row, head, tb, te, seq, flags, H, x, o);
        }
        free(H);
    }
    return failed ? -2 : 0;
}

/*
 * One recurrent decode step for N independent sequences.
 *   q, k [N][Hk][dk]; v [N][Hv][dv]; log_alpha, beta [N][Hv];
 *   state_in, state_out [N][Hv][dk][dv] (may be the same buffer); out [N][Hv][dv].
 * Written independently of the scan above, so that the two can be checked
 * against each other.
 */
int gdr_oracle_decode(const double *q, const double *k, const double *v,
                      const double *log_alpha, const double *beta,
                      const double *state_in, double *state_out, double *out,
                      int64_t N, int64_t Hk, int64_t Hv, int64_t dk, int64_t dv,
                      unsigned flags, int nthreads)
{
    if (!q || !k || !v || !log_alpha || !beta || !state_in || !state_out || !out) return -1;
    if (N < 0 || Hk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0 || Hv % Hk) return -1;
    const int pre = (flags & GDR_ORACLE_READ_PRE) != 0;
    const int64_t group = Hv / Hk;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel reduction(|| : failed)
    {
        /* every thread reaches the worksharing loop, even if its malloc failed */
        double *buf = (double *)malloc((size_t)(dk * dv + 3 * dv) * sizeof(double));
        double *Hn = buf;                    /* new state, built before any store */
        double *x = buf ? Hn + dk * dv : NULL; /* H^T k */
        double *y = buf ? x + dv : NULL;       /* H^T q */
        double *u = buf ? y + dv : NULL;
#pragma omp for schedule(dynamic, 16)
            for (int64_t w = 0; w < N * Hv; ++w) {
                if (!buf) { failed = 1; continue; }
                const int64_t nidx = w / Hv, head = w % Hv, kh = head / group;
                const double *S = state_in + w * dk * dv;
                const double *qv = q + (nidx * Hk + kh) * dk;
                const double *kv = k + (nidx * Hk + kh) * dk;
                const double *vv = v + w * dv;
                const double alpha = exp(log_alpha[w]);
                const double b = beta[w];
                for (int64_t c = 0; c < dv; ++c) { x[c] = 0.0; y[c] = 0.0; }
                for (int64_t r = 0; r < dk; ++r)
                    for (int64_t c = 0; c < dv; ++c) {
                        x[c] += S[r * dv + c] * kv[r];
                        y[c] += S[r * dv + c] * qv[r];
                    }
                for (int64_t c = 0; c < dv; ++c) u[c] = b * (vv[c] - alpha * x[c]);
                for (int64_t r = 0; r < dk; ++r)
                    for (int64_t c = 0; c < dv; ++c)
                        Hn[r * dv + c] = alpha * S[r * dv + c] + kv[r] * u[c];
                double *ov = out + w * dv;
                if (pre) {
                    for (int64_t c = 0; c < dv; ++c) ov[c] = y[c];
                } else {
                    /* read of the new state, computed directly: H_new^T q */
                    for (int64_t c = 0; c < dv; ++c) ov[c] = 0.0;
                    for (int64_t r = 0; r < dk; ++r)
                        for (int64_t c = 0; c < dv; ++c) ov[c] += Hn[r * dv + c] * qv[r];
                }
                memcpy(state_out + w * dk * dv, Hn, (size_t)(dk * dv) * sizeof(double));
            }
        free(buf);
    }
    return failed ? -2 : 0;
}
