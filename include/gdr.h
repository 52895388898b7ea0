/*
 * gdr.h - C ABI of the gated delta rule library for AMD Instinct MI355X (gfx950).
 *
 * The operation (state H = S^T stored row-major [d_k][d_v] per sequence and value head):
 *
 *   H_t = alpha_t * H_{t-1} + k_t u_t^T,     u_t = beta_t * (v_t - alpha_t * H_{t-1}^T k_t)
 *   post-write read   o_t = H_t^T q_t        pre-write read   o_t = H_{t-1}^T q_t
 *
 * with alpha_t = exp(log_alpha_t). This is the update defined in the module docstring
 * of the "Prizma seq/delta.py" page (which stores S = H^T and reads before the write)
 * and in the SparseDeltaMemory docstring of the "sparse-delta-memory layer.py" page
 * (decay by exp(g), then the beta-weighted erase-and-write, read after the write).
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer to contiguous row-major memory, 16-byte
 *     aligned; the `dims` structs are HOST pointers. The caller owns all memory: the
 *     library allocates nothing on the device and keeps no state between calls.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream) and the call
 *     returns without synchronising. No host read of device data happens, so calls can
 *     be captured into a HIP graph.
 *   - Arguments are validated on the host before anything is launched. A non-GDR_OK
 *     status means nothing was enqueued; gdr_last_error() then names the offending
 *     argument (thread-local text, valid until the next call on that thread).
 *   - Value head j reads query/key head j / (Hv / Hk) (key heads shared by groups of
 *     value heads, as in `heads` of BidirectionalGatedDeltaNet2 on the "tiny_gdn/fugue.py"
 *     page and the head-profile checks on the "flashrt-structures fused_layer.py" page).
 *   - log_alpha must be <= 0 and finite (a decay); q and k are used as given unless
 *     GDR_QK_L2NORM is set.
 *
 * The fused prologue (the steps the pages run just before the recurrence):
 *   - GDR_QK_L2NORM: each row of q and of k (one token of one key head) is first divided by
 *     max(||row||_2, 1e-6), as F.normalize(x, dim=-1, eps=1e-6) does on the
 *     "nested-learning self_modifying.py" page, and as the kernels of the "flashrt-structures
 *     fused_layer.py" page (use_qk_l2norm) and the "tiny_gdn/fugue.py" page
 *     (use_qk_l2norm_in_kernel) do inside the core.
 *   - the *_gated entry points take the raw gate inputs a, b [..][Hv] and per-value-head
 *     parameters A_log, dt_bias [Hv] and form
 *         log_alpha = -exp(A_log[h]) * softplus(a + dt_bias[h]),   beta = sigmoid(b)
 *     (compute_gates on the "sparse-delta-memory layer.py" page; the gating step before the
 *     core on the "flashrt-structures fused_layer.py" page).
 */
#ifndef GDR_H_
#define GDR_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdr_status {
    GDR_OK = 0,
    GDR_ERR_NULL = 1,        /* a required pointer is NULL */
    GDR_ERR_DIMS = 2,        /* a size is out of range or sizes disagree */
    GDR_ERR_DTYPE = 3,       /* unknown dtype code */
    GDR_ERR_CHUNK = 4,       /* chunk is not 16, 32 or 64 */
    GDR_ERR_ALIGN = 5,       /* a pointer is not 16-byte aligned */
    GDR_ERR_ALIAS = 6,       /* two buffers overlap in a way the operation forbids */
    GDR_ERR_UNSUPPORTED = 7, /* a head size the kernels do not cover */
    GDR_ERR_FLAGS = 8,       /* unknown flag bits */
    GDR_ERR_HIP = 9          /* the HIP runtime reported an error */
} gdr_status_t;

typedef enum gdr_dtype {
    GDR_F32 = 0,  /* IEEE binary32 */
    GDR_BF16 = 1  /* bfloat16 */
} gdr_dtype_t;

/* flag bits */
#define GDR_READ_PRE 1u   /* o_t = H_{t-1}^T q_t instead of H_t^T q_t */
#define GDR_REVERSE 2u    /* scan each sequence from its last token to its first */
#define GDR_ACCUMULATE 4u /* out += o instead of out = o */
#define GDR_QK_L2NORM 8u  /* normalise each row of q and k to unit L2 norm first */

typedef struct gdr_chunk_dims {
    int64_t B;        /* batch rows; must be 1 when cu_seqlens is given */
    int64_t T;        /* tokens per row (the packed total when cu_seqlens is given) */
    int64_t Hk;       /* query/key heads, >= 1 */
    int64_t Hv;       /* value heads, a positive multiple of Hk */
    int64_t dk;       /* key size: 64 or 128 */
    int64_t dv;       /* value size: a multiple of 32, at most 256 */
    int64_t num_seqs; /* segments described by cu_seqlens (ignored when it is NULL) */
    int32_t dtype;    /* gdr_dtype_t of q, k, v and out */
    uint32_t flags;   /* GDR_READ_PRE | GDR_REVERSE | GDR_ACCUMULATE | GDR_QK_L2NORM */
} gdr_chunk_dims_t;

typedef struct gdr_decode_dims {
    int64_t N;      /* independent sequences */
    int64_t Hk;     /* query/key heads */
    int64_t Hv;     /* value heads, a positive multiple of Hk */
    int64_t dk;     /* 64 or 128 */
    int64_t dv;     /* 64 or 128 */
    int32_t dtype;  /* gdr_dtype_t of q, k, v and out */
    uint32_t flags; /* GDR_READ_PRE | GDR_QK_L2NORM */
} gdr_decode_dims_t;

/*
 * gdr_chunk_fwd - the chunk-parallel forward over whole sequences.
 *
 * Computes, for every sequence and value head, the outputs o_t of every token and the
 * final state, exactly as the per-token recurrence above would (up to rounding): the
 * WY/UT chunk form of `chunked_delta` on the "Prizma seq/delta.py" page, where a unit
 * lower-triangular solve per chunk makes the intra-chunk recurrence exact, so `chunk`
 * changes the result only through rounding (the same page and the module docstring of
 * the "sparse-delta-memory layer.py" page). Packed segments (cu_seqlens) restart the
 * state at each segment start, and GDR_REVERSE scans each segment from its end, as
 * `segment_layout` and `BidirectionalGatedDeltaNet2.scan` on the "tiny_gdn/fugue.py"
 * page do.
 *
 *   q, k        [B][Hk][T][dk]  dtype
 *   v           [B][Hv][T][dv]  dtype
 *   log_alpha   [B][Hv][T]      fp32, <= 0
 *   beta        [B][Hv][T]      fp32
 *   h0          [S][Hv][dk][dv] fp32 initial state per sequence, or NULL for zeros;
 *               S = B, or num_seqs with cu_seqlens. Read only.
 *   cu_seqlens  NULL, or DEVICE int32 [num_seqs + 1] segment offsets into row 0 with
 *               cu[0] = 0, non-decreasing, cu[num_seqs] = T (a precondition: it is not
 *               read on the host). Empty segments are allowed (their hT is h0).
 *   chunk       16, 32 or 64 tokens per chunk.
 *   out         [B][Hv][T][dv]  dtype; written (or accumulated into with GDR_ACCUMULATE).
 *               Must not overlap any input.
 *   hT          [S][Hv][dk][dv] fp32 final state, or NULL when not wanted. It may be
 *               exactly h0 (updated in place); any other overlap is GDR_ERR_ALIAS.
 *
 * Errors: GDR_ERR_NULL (q, k, v, log_alpha, beta, out or dims NULL, or num_seqs < 1 with
 * cu_seqlens), GDR_ERR_DIMS, GDR_ERR_DTYPE, GDR_ERR_CHUNK, GDR_ERR_ALIGN, GDR_ERR_ALIAS,
 * GDR_ERR_UNSUPPORTED (dk not 64/128, dv not a multiple of 32 up to 256), GDR_ERR_FLAGS,
 * GDR_ERR_HIP (launch failure). T == 0 is valid: only hT is written.
 */
gdr_status_t gdr_chunk_fwd(const void *q, const void *k, const void *v,
                           const float *log_alpha, const float *beta,
                           const float *h0, const int32_t *cu_seqlens, int32_t chunk,
                           void *out, float *hT,
                           const gdr_chunk_dims_t *dims, void *stream);

/*
 * gdr_chunk_fwd_bidir - both scans of a bidirectional layer over shared q, k, v, summed per
 * token: the forward scan of every sequence or packed segment, plus the scan of each segment
 * run from its last token to its first, each with its own gate set, initial and final state,
 * and the same read (GDR_READ_PRE for the pre-write read both scans of the bidirectional
 * layer on the "tiny_gdn/fugue.py" page use: `BidirectionalGatedDeltaNet2.scan` reverses each
 * segment in place, and its `forward` adds the two directions). The page scales the sum by
 * 1/2; that factor belongs to the caller (fold it into v, or scale out).
 *
 *   out[t] = o_fwd[t] + o_rev[t]   (out += both with GDR_ACCUMULATE)
 *
 *   q, k, v, cu_seqlens, chunk, out, dims, stream: as gdr_chunk_fwd; dims->flags may hold
 *       GDR_READ_PRE, GDR_ACCUMULATE and GDR_QK_L2NORM (the latter for both scans).
 *   log_alpha_fwd, beta_fwd  [B][Hv][T] fp32 gates of the forward scan
 *   log_alpha_rev, beta_rev  [B][Hv][T] fp32 gates of the reverse scan, indexed by token as
 *       the forward ones (not by scan position)
 *   h0_fwd, h0_rev           [S][Hv][dk][dv] fp32 initial states, or NULL for zeros. For the
 *       reverse scan this is the state before the segment's last token is read.
 *   hT_fwd, hT_rev           [S][Hv][dk][dv] fp32 final states, or NULL; each may be exactly its
 *       own direction's h0 (in place). A final state may not overlap any input of the other
 *       direction or the other final state (GDR_ERR_ALIAS).
 *
 * The two scans are enqueued one after the other on the stream (the forward scan writes out,
 * the reverse scan adds to it); both are validated before either is enqueued. No single
 * sweep can produce the sum with one read of q, k, v: the reverse read at token t depends on
 * every later token of the segment. The second read of q, k, v comes one scan after the first.
 *
 * Errors: as gdr_chunk_fwd, the message naming the scan; GDR_ERR_FLAGS for GDR_REVERSE.
 */
gdr_status_t gdr_chunk_fwd_bidir(const void *q, const void *k, const void *v,
                                 const float *log_alpha_fwd, const float *beta_fwd,
                                 const float *log_alpha_rev, const float *beta_rev,
                                 const float *h0_fwd, const float *h0_rev,
                                 const int32_t *cu_seqlens, int32_t chunk, void *out,
                                 float *hT_fwd, float *hT_rev,
                                 const gdr_chunk_dims_t *dims, void *stream);

/*
 * gdr_chunk_fwd_gated - gdr_chunk_fwd with the gates formed from their raw inputs in the
 * kernel (see the fused prologue above), typically together with GDR_QK_L2NORM:
 *
 *   a, b        [B][Hv][T] fp32 raw decay input and raw write-gate logit (any sign)
 *   A_log       [Hv] fp32, dt_bias [Hv] fp32: per value head
 *
 * Every other argument, flag and error as gdr_chunk_fwd; GDR_ERR_NULL also when A_log or
 * dt_bias is NULL.
 */
gdr_status_t gdr_chunk_fwd_gated(const void *q, const void *k, const void *v,
                                 const float *a, const float *b,
                                 const float *A_log, const float *dt_bias,
                                 const float *h0, const int32_t *cu_seqlens, int32_t chunk,
                                 void *out, float *hT,
                                 const gdr_chunk_dims_t *dims, void *stream);

/*
 * gdr_decode_step - one token of the recurrence for N independent sequences.
 *
 * The one-token recurrent core of `_decode_one` on the "flashrt-structures
 * fused_layer.py" page: it reads state_in and writes state_out and the read o.
 *
 *   q, k        [N][Hk][dk]      dtype
 *   v           [N][Hv][dv]      dtype
 *   log_alpha   [N][Hv]          fp32, <= 0
 *   beta        [N][Hv]          fp32
 *   state_in    [N][Hv][dk][dv]  fp32
 *   state_out   [N][Hv][dk][dv]  fp32; may be exactly state_in (in place), any other
 *               overlap is GDR_ERR_ALIAS.
 *   out         [N][Hv][dv]      dtype; must not overlap any other argument.
 *
 * Each state element is read once and written once.
 * Errors: as gdr_chunk_fwd (no chunk); dk, dv must be 64 or 128.
 */
gdr_status_t gdr_decode_step(const void *q, const void *k, const void *v,
                             const float *log_alpha, const float *beta,
                             const float *state_in, float *state_out, void *out,
                             const gdr_decode_dims_t *dims, void *stream);

/*
 * gdr_decode_step_gated - gdr_decode_step with the gates formed from their raw inputs
 * (see the fused prologue above):
 *
 *   a, b        [N][Hv] fp32 raw decay input and raw write-gate logit
 *   A_log       [Hv] fp32, dt_bias [Hv] fp32: per value head
 *
 * Every other argument, flag and error as gdr_decode_step; GDR_ERR_NULL also when A_log or
 * dt_bias is NULL.
 */
gdr_status_t gdr_decode_step_gated(const void *q, const void *k, const void *v,
                                   const float *a, const float *b,
                                   const float *A_log, const float *dt_bias,
                                   const float *state_in, float *state_out, void *out,
                                   const gdr_decode_dims_t *dims, void *stream);

/*
 * gdr_chunk_bwd - gradients of gdr_chunk_fwd (the backward pass for training through it).
 *
 * Given the upstream gradients dout (of out) and dhT (of the final state), computes the
 * gradients of sum(out * dout) + sum(hT * dhT) with respect to every input: the derivative of
 * the per-token recurrence (the pages print no backward; the "Prizma seq/delta.py" page requires
 * the chunked form to agree with the recurrence in gradient, and the other pages train through
 * the operation). Same flags, layouts and segments as gdr_chunk_fwd (GDR_ACCUMULATE does not
 * change the gradients; GDR_QK_L2NORM is not taken: pass q, k as the forward saw them).
 *
 *   q, k, v, log_alpha, beta, h0, cu_seqlens, dims: exactly as given to gdr_chunk_fwd
 *   dout        [B][Hv][T][dv]  dtype
 *   dhT         [S][Hv][dk][dv] fp32, or NULL for zero
 *   dq, dk      [B][Hk][T][dk]  fp32 (a key head receives the sum over its value heads)
 *   dv          [B][Hv][T][dv]  fp32
 *   dlog_alpha, dbeta [B][Hv][T] fp32
 *   dh0         [S][Hv][dk][dv] fp32, or NULL when not wanted
 *   workspace   DEVICE scratch of at least gdr_chunk_bwd_workspace_bytes(dims, cu_seqlens != NULL)
 *               bytes, 16-byte aligned, owned by the caller; its contents are not needed
 *               before or after the call. Calls that share a workspace must not overlap.
 *
 * dk must be 64 or 128, dv a multiple of 32 up to 256. Every output is fully written. Outputs
 * and workspace must not overlap inputs or each other (GDR_ERR_ALIAS).
 * Errors as gdr_chunk_fwd, plus GDR_ERR_DIMS when workspace_bytes is too small.
 * The backward runs the chunk form over 64-token chunks as three kernels on `stream`: a
 * chunk-parallel pass forms each chunk's gate cumsums, read matrix and triangular inverse; two
 * sweeps (one launch) carry the state forward and its adjoint backward through the chunks,
 * keeping every chunk's entry state, exit-state adjoint, U and dR in the workspace (each a
 * dk x dv or 64 x dv fp32 block per chunk and value head, plus a 49,664-byte record); a second
 * chunk-parallel pass forms every gradient of a chunk from those. Its products run on the bf16
 * matrix cores with each fp32 operand split in two bf16 parts (hi*hi + hi*lo + lo*hi, fp32
 * accumulation): a relative error near 2^-16 per product.
 * Deterministic: the same inputs give the same bits on every call. Every gradient element is
 * written once, by one workgroup, which adds the contributions of the column slices (and, for
 * dq and dk, of the value heads of a key head) in a fixed order; no float atomics are used.
 */
int64_t gdr_chunk_bwd_workspace_bytes(const gdr_chunk_dims_t *dims, int32_t packed);
gdr_status_t gdr_chunk_bwd(const void *q, const void *k, const void *v,
                           const float *log_alpha, const float *beta,
                           const float *h0, const int32_t *cu_seqlens,
                           const void *dout, const float *dhT,
                           float *dq, float *dk, float *dv, float *dlog_alpha, float *dbeta, float *dh0,
                           void *workspace, int64_t workspace_bytes,
                           const gdr_chunk_dims_t *dims, void *stream);

/*
 * gdr_delta_product_fwd - DeltaProduct: n_delta delta sub-steps per token (the n_delta branch of
 * `_delta_reference` and `chunked_delta` on the "Prizma seq/delta.py" page). For token t and
 * sub-step j = 0 .. n_delta-1, with alpha_tj = exp(log_alpha_t) for j = 0 and 1 otherwise (the
 * decay applies once per token, on its first sub-step):
 *
 *   u_tj = beta_tj (v_tj - alpha_tj H^T k_tj),   H <- alpha_tj H + k_tj u_tj^T
 *
 * GDR_READ_PRE reads o_t = H^T q_t before the token's first sub-step (the page's read); without
 * it the read comes after the token's last sub-step. This is gdr_chunk_fwd over the sequence of
 * T * n_delta sub-steps, and is computed that way (chunks of sub-steps).
 *
 *   q           [B][Hk][T][dk]           dtype
 *   k           [B][Hk][T][n_delta][dk]  dtype
 *   v           [B][Hv][T][n_delta][dv]  dtype
 *   log_alpha   [B][Hv][T]               fp32, <= 0 (one decay per token)
 *   beta        [B][Hv][T][n_delta]      fp32
 *   h0, cu_seqlens (in tokens), chunk (in sub-steps), out [B][Hv][T][dv], hT, dims, stream:
 *   as gdr_chunk_fwd.
 *
 * n_delta in [1, 16] (GDR_ERR_DIMS otherwise, and when T * n_delta >= 2^31); GDR_REVERSE with
 * n_delta > 1 is GDR_ERR_FLAGS; GDR_QK_L2NORM normalises q and every sub-step's key.
 * Errors otherwise as gdr_chunk_fwd.
 */
gdr_status_t gdr_delta_product_fwd(const void *q, const void *k, const void *v,
                                   const float *log_alpha, const float *beta,
                                   const float *h0, const int32_t *cu_seqlens, int32_t n_delta,
                                   int32_t chunk, void *out, float *hT,
                                   const gdr_chunk_dims_t *dims, void *stream);

/*
 * GDN-2: the delta rule with a decay per key channel and separate erase and write gates, the
 * update stated in the BidirectionalGatedDeltaNet2 docstring on the "tiny_gdn/fugue.py" page
 * (which also forms g = -exp(A_log) softplus(f + dt_bias) per key channel, b = sigmoid(.) or
 * twice that with negative eigenvalues allowed, w = sigmoid(.), in its `heads` and `project`):
 *
 *   H_t = (I - k_t (b_t * k_t)^T) Diag(exp g_t) H_{t-1} + k_t (w_t * v_t)^T
 *       = Diag(e^{g_t}) H_{t-1} + k_t u_t^T,   u_t = w_t * v_t - (Diag(e^{g_t}) H_{t-1})^T (b_t * k_t)
 *
 * (* is the element-wise product). g and b belong to the key head (one value per key channel),
 * w to the value head (one value per value channel); the reads are those of the scalar rule.
 * With g_t = log(alpha_t), b_t = w_t = beta_t on every channel this is gdr_chunk_fwd's update.
 * g must be finite and <= 0; b and w may take any finite value (b in (0, 2) allows the negative
 * eigenvalues of the page's allow_neg_eigval option).
 *
 * gdr_gdn2_chunk_fwd - the chunk-parallel forward of GDN-2 over whole sequences (the per-channel
 * form of the chunk algebra of gdr_chunk_fwd; `chunk_gdn2` as the page calls it).
 *
 *   q, k        [B][Hk][T][dk]  dtype
 *   v           [B][Hv][T][dv]  dtype
 *   g           [B][Hk][T][dk]  fp32 log decay per key channel, <= 0
 *   b           [B][Hk][T][dk]  dtype erase gate per key channel
 *   w           [B][Hv][T][dv]  dtype write gate per value channel
 *   h0, cu_seqlens, out, hT, dims, stream: as gdr_chunk_fwd (all four flags apply).
 *   workspace   DEVICE scratch of at least gdr_gdn2_chunk_fwd_workspace_bytes(dims, chunk,
 *               cu_seqlens != NULL) bytes, or NULL. Owned by the caller; its contents do not
 *               matter before or after the call; calls that share a workspace must not
 *               overlap. With a workspace the forward runs in two passes: the first computes
 *               the key side of every chunk at once (for each chunk and key head: the WY-form
 *               factor T (b * k * e^G), q * e^{Gr}, (k * e^{G_C - G})^T, the intra-chunk read
 *               matrix, T = (I + A)^{-1} and e^{G_C}), the second walks the chunks with the
 *               state. Without one a single fused pass does both (allocation-free, slower); fp32
 *               with chunk 64 always takes the fused pass. The results agree up to rounding.
 *   workspace_bytes  its size in bytes.
 *
 * Every tensor pointer 16-byte aligned. chunk 16, 32 or 64, except that fp32 with dk = 128
 * takes 16 or 32 only (GDR_ERR_CHUNK): the fp32 operands of a 64-token chunk do not fit in the
 * 160 KB of shared memory of a compute unit. A 16-token block whose decay summed over the block
 * is below -60 on some channel is computed exactly on a slower path (see gdn2_fwd.hip);
 * results do not depend on which path a block takes beyond rounding.
 * Errors: as gdr_chunk_fwd; GDR_ERR_NULL also when g, b or w is NULL with T > 0; with a
 * workspace, GDR_ERR_DIMS when workspace_bytes is too small, GDR_ERR_ALIGN when it is not
 * 16-byte aligned and GDR_ERR_ALIAS when it overlaps an input or output.
 */
gdr_status_t gdr_gdn2_chunk_fwd(const void *q, const void *k, const void *v,
                                const float *g, const void *b, const void *w,
                                const float *h0, const int32_t *cu_seqlens, int32_t chunk,
                                void *out, float *hT, void *workspace, int64_t workspace_bytes,
                                const gdr_chunk_dims_t *dims, void *stream);

/*
 * gdr_gdn2_chunk_fwd_bidir - both GDN-2 scans of the bidirectional layer on the "tiny_gdn/fugue.py"
 * page (`BidirectionalGatedDeltaNet2`: `scan` runs each packed segment forward and reversed in
 * place, each direction with its own decay and gates; `forward` adds the two), over shared q, k,
 * v, summed per token into out (out += both with GDR_ACCUMULATE). The page scales the sum by 1/2
 * and reads before the write on its reverse scan; the scale is the caller's, and dims->flags
 * (GDR_READ_PRE, GDR_ACCUMULATE, GDR_QK_L2NORM) apply to both scans.
 *
 *   q, k, v, cu_seqlens, chunk, out, workspace, workspace_bytes, dims, stream: as
 *       gdr_gdn2_chunk_fwd; the two passes use the workspace one after the other, so one of
 *       gdr_gdn2_chunk_fwd_workspace_bytes bytes serves both (NULL: the one-pass kernel).
 *   g_fwd, b_fwd, w_fwd / g_rev, b_rev, w_rev   the forward and the reverse scan's log decay,
 *       erase and write gates, in gdr_gdn2_chunk_fwd's layouts, indexed by token
 *   h0_fwd, h0_rev, hT_fwd, hT_rev   per direction, as in gdr_chunk_fwd_bidir
 *
 * Both scans are validated before either is enqueued. Errors: as gdr_gdn2_chunk_fwd, the message
 * naming the scan; GDR_ERR_FLAGS for GDR_REVERSE; GDR_ERR_ALIAS when a final state or the
 * workspace overlaps an input of the other direction, or the two final states overlap.
 */
gdr_status_t gdr_gdn2_chunk_fwd_bidir(const void *q, const void *k, const void *v,
                                      const float *g_fwd, const void *b_fwd, const void *w_fwd,
                                      const float *g_rev, const void *b_rev, const void *w_rev,
                                      const float *h0_fwd, const float *h0_rev,
                                      const int32_t *cu_seqlens, int32_t chunk, void *out,
                                      float *hT_fwd, float *hT_rev, void *workspace,
                                      int64_t workspace_bytes, const gdr_chunk_dims_t *dims,
                                      void *stream);

/*
 * gdr_gdn2_chunk_fwd_noalloc - gdr_gdn2_chunk_fwd in its two-pass form without a caller
 * workspace and without allocating: for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Arguments, results and errors as gdr_gdn2_chunk_fwd with workspace = NULL replaced by the
 * library's fixed device scratch of GDR_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU: a static array of
 * the library's code object, held by each GPU from the library's first launch there until the
 * process ends. Sizes whose workspace (gdr_gdn2_chunk_fwd_workspace_bytes) exceeds it are
 * rejected with GDR_ERR_DIMS before anything runs (for bf16, d_k = 128 and chunk 32 that is about
 * 2,300 (chunk, key head) blocks, e.g. B = 1, Hk = 16, T = 4096). The call allocates nothing and
 * keeps the scratch's device address per device. All calls on one GPU share the scratch: calls
 * that overlap in time on the same GPU (other streams or host threads) race on it and must be
 * serialised by the caller. The scratch needs no clearing (the first pass writes every byte the
 * second reads). The device is the current HIP device, which must own the stream.
 */
#define GDR_NOALLOC_SCRATCH_BYTES (INT64_C(64) << 20)
gdr_status_t gdr_gdn2_chunk_fwd_noalloc(const void *q, const void *k, const void *v,
                                        const float *g, const void *b, const void *w,
                                        const float *h0, const int32_t *cu_seqlens, int32_t chunk,
                                        void *out, float *hT,
                                        const gdr_chunk_dims_t *dims, void *stream);

/*
 * gdr_gdn2_chunk_fwd_workspace_bytes - bytes of workspace gdr_gdn2_chunk_fwd's two-pass form
 * needs for these sizes, chunk and packing (packed != 0: cu_seqlens with dims->num_seqs
 * sequences). Host-only arithmetic: one slot per chunk of every sequence (packed: T / chunk +
 * num_seqs + 1), each with Hk blocks of es (3 chunk dk + 2 chunk^2) + 4 dk bytes (es = 2 for
 * bf16, 4 for fp32). Returns -1 for an unsupported dtype, chunk or dk, or negative sizes.
 */
int64_t gdr_gdn2_chunk_fwd_workspace_bytes(const gdr_chunk_dims_t *dims, int32_t chunk, int32_t packed);

/*
 * gdr_gdn2_decode_step - one GDN-2 token for N independent sequences.
 *
 *   q, k, b     [N][Hk][dk]      dtype (b: erase gate)
 *   g           [N][Hk][dk]      fp32 log decay, <= 0
 *   v, w        [N][Hv][dv]      dtype (w: write gate)
 *   state_in, state_out, out, dims, stream: as gdr_decode_step (GDR_READ_PRE, GDR_QK_L2NORM).
 *
 * Every tensor pointer 16-byte aligned. Each state element is read once and written once.
 * Errors: as gdr_decode_step.
 */
gdr_status_t gdr_gdn2_decode_step(const void *q, const void *k, const void *v,
                                  const float *g, const void *b, const void *w,
                                  const float *state_in, float *state_out, void *out,
                                  const gdr_decode_dims_t *dims, void *stream);

/* Static text for a status code. */
const char *gdr_status_string(gdr_status_t status);

/* Thread-local detail of the last non-GDR_OK status returned on this thread ("" if none). */
const char *gdr_last_error(void);

/* ABI version of this header (incremented on any incompatible change). */
int32_t gdr_abi_version(void);

/*
 * gdr_selftest_mfma - diagnostic: multiplies one 16x32 by one 32x16 matrix through the
 * library's matrix-core operand layouts and writes the 16x16 product.
 *   a   DEVICE fp32 [16][32], b DEVICE fp32 [32][16], d DEVICE fp32 [3][16][16]:
 *   d[0] through the bf16 32-deep instruction (inputs rounded to bf16),
 *   d[1] through the fp32 instruction, d[2] through the bf16 16-deep instruction on the
 *   first 16 columns of a and rows of b. Synchronous on `stream`.
 */
gdr_status_t gdr_selftest_mfma(const float *a, const float *b, float *d, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H_ */
