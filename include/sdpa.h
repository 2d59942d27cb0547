/*
 * sdpa.h - C ABI of the fused scaled dot-product attention library for
 * AMD Instinct MI355X (gfx950).  Forward and backward of multi-head
 * attention with optional additive bias, top-left causal mask, Philox
 * dropout and packed variable-length (group) mode.
 *
 * The operation (Composable Kernel, "fmha_bwd_kernel.hpp Source File",
 * the formula comment at the head of the file):
 *   S   = scale * Q K^T            S'' = S + Bias        P = softmax_row(S'')
 *   O   = (P o Z) V                LSE = row log-sum-exp of S'' (natural log)
 *   D   = rowsum(dO o O)           dV  = (P o Z)^T dO    dP = (dO V^T) o Z
 *   dS  = P o (dP - D)             dBias = dS
 *   dQ  = scale * dS K             dK  = scale * dS^T Q
 * where Z is the dropout keep mask scaled by 1/(1-p) (Z = 1 when p = 0).
 *
 * The argument list follows the problem statement of PyTorch's cuDNN
 * attention glue ("MHA.cpp", run_cudnn_SDP_fprop / run_cudnn_SDP_bprop):
 * b, h, s_q, s_kv, d_qk, d_v, scaling_factor, is_causal,
 * dropout_probability, q, k, v, optional attn_bias, softmax stats, o,
 * dropout seed and offset.  Group mode follows CK's seqstart_q / seqstart_k
 * kernel arguments (FmhaBwdDQDKDVKernel group-mode kargs).
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *     library allocates no memory and keeps no per-call state; calls are
 *     thread-safe.  Work is enqueued on `stream` (a hipStream_t; NULL = the
 *     default stream) and returns before it completes.
 *   - Errors are status codes; nothing is thrown across the ABI.  On error,
 *     sdpa_last_error_message() returns a thread-local description.
 *     Validation happens before anything is enqueued, so an error other than
 *     SDPA_ERR_HIP means no work was launched.
 *   - Any of b, h, s_q, s_kv equal to 0 is a successful no-op (PyTorch's
 *     cuDNN glue returns early on zero-element tensors).
 */
#ifndef SDPA_MI355X_H
#define SDPA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SDPA_OK = 0,
    SDPA_ERR_INVALID_ARG = 1, /* malformed arguments (null, negative, bad stride) */
    SDPA_ERR_UNSUPPORTED = 2, /* well-formed but not implemented (head dim, combination) */
    SDPA_ERR_WORKSPACE = 3,   /* workspace smaller than the size query returned */
    SDPA_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} sdpa_status_t;

/* io element type of Q, K, V, O, dO, dQ, dK, dV, bias and dBias.
 * LSE, D and all accumulation are fp32 whatever the io type (the cuDNN glue
 * fixes fp32 "intermediate" and "compute" types and fp32 stats). */
typedef enum { SDPA_F32 = 0, SDPA_F16 = 1, SDPA_BF16 = 2 } sdpa_dtype_t;

/* Element strides of a 4-D attention tensor.  The innermost dimension
 * (head dim, or s_kv for the bias) always has stride 1.
 *   batch mode : element (b, h, s, d) is at  b*batch + h*head + s*seq + d
 *   group mode : element (token t, h, d) is at  h*head + t*seq + d; `batch`
 *                is ignored (tokens of all sequences are packed). */
typedef struct {
    int64_t batch, head, seq;
} sdpa_strides_t;

typedef struct {
    uint32_t struct_size;       /* must be sizeof(sdpa_problem_t) */
    sdpa_dtype_t dtype;
    int64_t b;                  /* batch; group mode: number of sequences */
    int64_t h;                  /* query heads (key/value heads: h_kv below) */
    int64_t s_q, s_kv;          /* sequence lengths; group mode: the maxima */
    int64_t d_qk, d_v;          /* head dims of Q/K and of V/O */
    float scaling_factor;       /* multiplies Q K^T; the bias is added after it */
    int32_t is_causal;          /* top-left causal: key j visible from query i iff j <= i */
    /* 0 <= p <= 255/256, and p = 0 or p >= 1/512 (see the keep mask below:
     * outside that range the 8-bit threshold would keep everything or
     * saturate, so such p is SDPA_ERR_UNSUPPORTED). */
    float dropout_probability;
    uint64_t dropout_seed;      /* Philox key */
    uint64_t dropout_offset;    /* Philox counter word 3 (low 32 bits used) */
    /* Optional device pointer to {seed, offset} (two uint64); when non-null
     * it replaces dropout_seed / dropout_offset (CK passes either values or
     * device pointers: FmhaBwdDropoutSeedOffset). */
    const uint64_t *dropout_seed_offset_dev;
    /* Group (varlen) mode: device int32 arrays of length b+1 holding the
     * first token of each sequence (cu_seqlens; CK's seqstart_q_ptr /
     * seqstart_k_ptr).  Both null = batch mode; both non-null = group mode.
     * The host reads no element of them: s_q and s_kv must bound every
     * sequence length. */
    const int32_t *cu_seqlens_q;
    const int32_t *cu_seqlens_kv;
    /* Key/value heads (grouped-query attention); 0 means h.  Must divide h.
     * K, V, dK and dV have h_kv heads and query head i reads key/value head
     * i / (h / h_kv) (Composable Kernel's i_nhead / nhead_ratio_qk; oneDNN's
     * kv_group_size = h / h_kv).  dK and dV of a key/value head are the sums
     * over its group of query heads, accumulated in a fixed order. */
    int64_t h_kv;
    /* Mask generality (0 keeps the plain behaviour).  Key j is visible from
     * query i iff lo <= j - i - off <= hi, where
     *   off = s_kv - s_q (per sequence in group mode) with
     *         SDPA_MASK_BOTTOM_RIGHT, else 0 (top-left alignment);
     *   lo  = -window_left with SDPA_MASK_WINDOW and window_left >= 0, else
     *         unbounded;
     *   hi  = window_right with SDPA_MASK_WINDOW and window_right >= 0, else
     *         unbounded; and at most 0 when is_causal.
     * (CK builds its mask from window_size_left / window_size_right and a
     * top-left flag; oneDNN names top-left and bottom-right causal kinds.)
     * A query row with no visible key gets O = 0, LSE = -inf and no
     * gradient. */
    uint32_t mask_flags;
    int64_t window_left, window_right;
    /* ALiBi position bias (Composable Kernel's FmhaBwdAlibiKargs: one fp32
     * slope per batch entry and head, and the position encoding its backward
     * kernel builds from the mask).  Nullable device pointer; when set,
     *   s_ij += -alibi_slopes[b * alibi_batch_stride + h] * |j - i - off|
     * with off = s_kv - s_q (per sequence) for a bottom-right mask or when
     * there is no mask (is_causal = 0 and no SDPA_MASK_WINDOW), else 0.
     * alibi_batch_stride = 0 shares one slope vector [h] across the batch.
     * It takes the place of attn_bias: passing both is SDPA_ERR_UNSUPPORTED,
     * and there is no gradient for the slopes. */
    const float *alibi_slopes;
    int64_t alibi_batch_stride;
    /* Quantized K/V for the thin-query forward (the oneDNN micro SDPA host
     * driver's grouped key / value scales and zero points).  k and v hold
     * integer codes (their strides count bytes):
     *   SDPA_KV_QUANT_S8  int8 codes, one per byte;
     *   SDPA_KV_QUANT_S4  signed 4-bit codes (-8 .. 7, two's complement),
     *   SDPA_KV_QUANT_U4  unsigned 4-bit codes (0 .. 15): two per byte, code
     *                     2i of a row in the low nibble of byte i and code
     *                     2i + 1 in its high nibble (rows of d/2 bytes);
     * and
     *   K[t][c] = (code[t][c] - k_zero_points[t][c/g]) * k_scales[t][c/g]
     * (V likewise), g = kv_group_size, t a token of one (batch, K/V head).
     * Scales are fp32 and zero points int8 (nullable together: then 0), all
     * four at kv_scale_strides (elements; the group index is contiguous).
     * Supported by sdpa_fwd only, for thin-query problems (16-bit q and o,
     * s_q <= 16, d_qk = d_v = 128, no bias, ALiBi or dropout) with g in
     * {16, 32, 64, 128} for int8 and {32, 64, 128} for 4-bit codes; code
     * rows must be 16-byte aligned. */
    int32_t kv_quant;
    int32_t kv_group_size;
    const float *k_scales, *v_scales;
    const int8_t *k_zero_points, *v_zero_points;
    sdpa_strides_t kv_scale_strides;
    /* Group mode: rows of the packed q (>= cu_seqlens_q[b]; trailing rows
     * past the last sequence are allowed and left alone).  softmax_lse is
     * [h, total_q] (element (head, token) at head * total_q + token); 0
     * means total_q = cu_seqlens_q[b].  Ignored in batch mode. */
    int64_t total_q;
} sdpa_problem_t;

#define SDPA_KV_QUANT_NONE 0
#define SDPA_KV_QUANT_S8 1
#define SDPA_KV_QUANT_S4 2
#define SDPA_KV_QUANT_U4 3

#define SDPA_MASK_BOTTOM_RIGHT 1u
#define SDPA_MASK_WINDOW 2u

/* Dropout keep mask (the library's own specification; the pages give the
 * ingredients - an 8-bit threshold and a 1/(1-p) rescale in CK's
 * init_dropout, seed and offset in cuDNN's graph - but no generator):
 *   counter = (j >> 2, i >> 2, b*h_count + h, low32(offset)),
 *   key     = (low32(seed), high32(seed)),
 *   r       = Philox4x32-10(counter, key)   (Salmon et al., SC'11),
 *   byte    = (r[i & 3] >> (8 * (j & 3))) & 0xff,
 *   keep    = byte >= round(256 p);  kept values are scaled by 1/(1-p).
 * i, j are query and key positions within the sequence; in group mode b is
 * the sequence index.  The kept fraction is (256 - round(256 p)) / 256,
 * within 1/512 of 1 - p, so the expectation of a kept-and-rescaled value is
 * off by at most (1/512) / (1 - p) relative (0.17% at p = 0.1, 2% at
 * p = 0.9); the p outside [1/512, 255/256] that would round to "keep all"
 * or saturate the threshold are rejected. */

/* ------------------------------------------------------------------------ */
/* Workspace.  Bytes of device scratch the caller must pass to sdpa_fwd /    */
/* sdpa_bwd (the cuDNN glue allocates a workspace per call; the oneDNN       */
/* backward sizes its scratchpad for D).  Returns 0 when none is needed and  */
/* also 0 for a problem that fails validation.  Alignment: 256 bytes.  The   */
/* backward's workspace holds the stats described at sdpa_bwd_preprocess.    */
/* ------------------------------------------------------------------------ */
size_t sdpa_fwd_workspace_size(const sdpa_problem_t *problem);
size_t sdpa_bwd_workspace_size(const sdpa_problem_t *problem);

/* Forward (run_cudnn_SDP_fprop's contract).
 *   q [b,h,s_q,d_qk]  k [b,h,s_kv,d_qk]  v [b,h,s_kv,d_v]  o [b,h,s_q,d_v]
 *     (group mode: [T,h,d]; the strides say where each element is).
 *   attn_bias: nullable, [b,h,s_q,s_kv] with its own strides (batch mode
 *     only); added to the scaled scores before the softmax.
 *   softmax_lse: nullable fp32.  Batch mode: dense [b,h,s_q]; group mode:
 *     dense [h,total_q] (CK addresses LSE as head*T + token; total_q as in
 *     sdpa_problem_t).  Null means inference: no stats are written.
 *   dropout_keep_out: nullable debug output, dense uint8 [b,h,s_q,s_kv]
 *     (batch mode only): 1 where the element was kept.  Positions the causal
 *     mask hides are left unwritten.
 *   workspace: thin-query problems (16-bit io, s_q <= 16, no bias, p = 0;
 *     decoding, as oneDNN's thin-q configuration and its single-query
 *     batching over key/value heads) run a split-KV kernel that packs the
 *     query heads of each key/value head into one tile and splits the keys
 *     over workgroups.  Its partial results need
 *     sdpa_fwd_workspace_size(problem) bytes (16-byte aligned); with less
 *     (or null) the same kernel runs unsplit, which is correct but slower
 *     when few (batch, key/value head) pairs exist.  Other problems take no
 *     workspace.  Results do not depend on the split beyond rounding.
 * Errors: SDPA_ERR_INVALID_ARG for null tensors, bad strides, p outside
 * [0,1) or half the varlen pair; SDPA_ERR_UNSUPPORTED for head dims outside
 * the compiled set (16-bit io: (d_qk, d_v) in {(64,64), (128,128),
 * (192,128)}; fp32: d_qk, d_v <= 256, d_v % 4 == 0), for 16-bit tensors
 * whose base or batch/head/seq strides are not multiples of 16 bytes or
 * whose seq stride exceeds 16 MiB, for bias or keep output in group mode. */
sdpa_status_t sdpa_fwd(const sdpa_problem_t *problem,
                       const void *q, sdpa_strides_t q_strides,
                       const void *k, sdpa_strides_t k_strides,
                       const void *v, sdpa_strides_t v_strides,
                       const void *attn_bias, sdpa_strides_t bias_strides,
                       void *o, sdpa_strides_t o_strides,
                       float *softmax_lse,
                       uint8_t *dropout_keep_out,
                       void *workspace, size_t workspace_bytes,
                       void *stream);

/* Backward (run_cudnn_SDP_bprop's contract).  Consumes the forward's o and
 * softmax_lse (same layout as written by sdpa_fwd) and the same seed,
 * offset and probability.  Writes dq, dk, dv (shapes of q, k, v, each with
 * its own strides) and, when non-null, dbias (shape of the bias; requires
 * attn_bias).  Results are deterministic: bitwise identical from run to run.
 * workspace must hold sdpa_bwd_workspace_size(problem) bytes.
 * Errors as for sdpa_fwd, plus SDPA_ERR_WORKSPACE. */
sdpa_status_t sdpa_bwd(const sdpa_problem_t *problem,
                       const void *q, sdpa_strides_t q_strides,
                       const void *k, sdpa_strides_t k_strides,
                       const void *v, sdpa_strides_t v_strides,
                       const void *attn_bias, sdpa_strides_t bias_strides,
                       const void *o, sdpa_strides_t o_strides,
                       const void *d_o, sdpa_strides_t do_strides,
                       const float *softmax_lse,
                       void *dq, sdpa_strides_t dq_strides,
                       void *dk, sdpa_strides_t dk_strides,
                       void *dv, sdpa_strides_t dv_strides,
                       void *dbias, sdpa_strides_t dbias_strides,
                       void *workspace, size_t workspace_bytes,
                       void *stream);

/* Backward preprocess alone (CK's FmhaBwdOGradDotOKernel; oneDNN's backward
 * "preprocess" kernel): writes the backward stats, n = b*h*s_q floats each,
 *   stats[0 .. n)        D = rowsum(dO o O), fp32 accumulation
 *   stats[m .. m + n)    softmax_lse * log2(e)   (m = n rounded up to 64)
 * in the layout of softmax_lse but with group mode rows [h, b*s_q] for both.
 * `stats` needs sdpa_bwd_workspace_size(problem) bytes; sdpa_bwd does this
 * step itself into its workspace (for 16-bit io inside its dQ kernel, see
 * sdpa_bwd_dq_preprocess).  Errors as for sdpa_bwd. */
sdpa_status_t sdpa_bwd_preprocess(const sdpa_problem_t *problem,
                                  const void *o, sdpa_strides_t o_strides,
                                  const void *d_o, sdpa_strides_t do_strides,
                                  const float *softmax_lse, float *stats, void *stream);

/* The backward's two main kernels, one call each.  The dK/dV and dQ kernels
 * read only the inputs and the stats, never each other's results, so a
 * caller may run sdpa_bwd_preprocess and then these two in either order or
 * on two streams, or time them one by one.  `stats` is the preprocess
 * output above.  sdpa_bwd_dkdv writes dk, dv and (nullable) dbias;
 * sdpa_bwd_dq writes dq.  Errors as for sdpa_bwd (no workspace argument). */
sdpa_status_t sdpa_bwd_dkdv(const sdpa_problem_t *problem,
                            const void *q, sdpa_strides_t q_strides,
                            const void *k, sdpa_strides_t k_strides,
                            const void *v, sdpa_strides_t v_strides,
                            const void *attn_bias, sdpa_strides_t bias_strides,
                            const void *d_o, sdpa_strides_t do_strides,
                            const float *stats,
                            void *dk, sdpa_strides_t dk_strides,
                            void *dv, sdpa_strides_t dv_strides,
                            void *dbias, sdpa_strides_t dbias_strides,
                            void *stream);
sdpa_status_t sdpa_bwd_dq(const sdpa_problem_t *problem,
                          const void *q, sdpa_strides_t q_strides,
                          const void *k, sdpa_strides_t k_strides,
                          const void *v, sdpa_strides_t v_strides,
                          const void *attn_bias, sdpa_strides_t bias_strides,
                          const void *d_o, sdpa_strides_t do_strides,
                          const float *stats,
                          void *dq, sdpa_strides_t dq_strides,
                          void *stream);

/* dQ and the preprocess in one kernel (16-bit io only; SDPA_ERR_UNSUPPORTED
 * for fp32): each workgroup computes D = rowsum(dO o O) and LSE*log2(e) for
 * the query rows it owns, writes them to `stats` (layout as for
 * sdpa_bwd_preprocess, which it replaces) and then computes dq for those
 * rows.  sdpa_bwd runs this and then sdpa_bwd_dkdv on the stats, saving a
 * kernel and its launch gap.  D is summed in a different order from
 * sdpa_bwd_preprocess, so the two agree to fp32 rounding, not bitwise.
 * Errors as for sdpa_bwd_dq. */
sdpa_status_t sdpa_bwd_dq_preprocess(const sdpa_problem_t *problem,
                                     const void *q, sdpa_strides_t q_strides,
                                     const void *k, sdpa_strides_t k_strides,
                                     const void *v, sdpa_strides_t v_strides,
                                     const void *attn_bias, sdpa_strides_t bias_strides,
                                     const void *o, sdpa_strides_t o_strides,
                                     const void *d_o, sdpa_strides_t do_strides,
                                     const float *softmax_lse, float *stats,
                                     void *dq, sdpa_strides_t dq_strides,
                                     void *stream);

/* Backward with no workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments (minus the workspace),
 * kernels and results as sdpa_bwd: the outputs are bitwise those of sdpa_bwd
 * on the same inputs.  The backward stats (D and LSE*log2(e), the workspace
 * of sdpa_bwd) live in a device array of the library instead:
 * 2 * SDPA_NOALLOC_MAX_ROWS floats (8 MiB) on each GPU the library runs on,
 * held until the process ends.  It calls no allocating routine.
 *   - b*h*s_q must not exceed SDPA_NOALLOC_MAX_ROWS, else SDPA_ERR_WORKSPACE
 *     (group mode counts b*h*s_q with s_q the maximum length);
 *   - calls that overlap on one GPU (several streams or threads) share the
 *     array and race: the caller serialises them.  The array needs no
 *     clearing: every element a call reads was written earlier in that call.
 * Errors as for sdpa_bwd; SDPA_ERR_HIP if the array's device address cannot
 * be obtained. */
#define SDPA_NOALLOC_MAX_ROWS (1 << 20)
sdpa_status_t sdpa_bwd_noalloc(const sdpa_problem_t *problem,
                               const void *q, sdpa_strides_t q_strides,
                               const void *k, sdpa_strides_t k_strides,
                               const void *v, sdpa_strides_t v_strides,
                               const void *attn_bias, sdpa_strides_t bias_strides,
                               const void *o, sdpa_strides_t o_strides,
                               const void *d_o, sdpa_strides_t do_strides,
                               const float *softmax_lse,
                               void *dq, sdpa_strides_t dq_strides,
                               void *dk, sdpa_strides_t dk_strides,
                               void *dv, sdpa_strides_t dv_strides,
                               void *dbias, sdpa_strides_t dbias_strides,
                               void *stream);

/* Human-readable name of a status code (static storage). */
const char *sdpa_status_string(sdpa_status_t status);

/* Detail of the last error on the calling thread ("" if none). */
const char *sdpa_last_error_message(void);

/* Library version, e.g. "0.1.0". */
const char *sdpa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SDPA_MI355X_H */
