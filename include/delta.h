/*
 * delta.h -- C ABI of the MI355X (gfx950) delta-rule forward library.
 *
 * The operation is the fast-weight recurrence
 *
 *     S_t = g_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,   o_t = scale * S_t^T q_t
 *
 * with S of shape d_k x d_v, covering DeltaNet (g = 1), Gated DeltaNet (scalar g_t)
 * and DeltaProduct (n_h Householder steps per token).  Sources, by page and section:
 *   - "08 linear delta rule & DPLR" page: section 1.2 (Householder form), section 2
 *     (WY representation, UT transform, chunkwise algorithm), section 3 (Gated
 *     DeltaNet and its chunkwise form with decays).
 *   - DeltaProduct reading notes: sections 2.2, 2.6 (n_h ordered steps per token,
 *     gate applied once before them) and 4.1 (expanded-sequence layout: keys,
 *     values and betas of a token's sub-steps adjacent; one output per token after
 *     its last sub-step).
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller; the library never
 *     allocates, frees or retains them.  All tensors are contiguous, row-major.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *     default stream); no entry point synchronises the host (unless DELTA_VALIDATE=1,
 *     below).
 *   - Argument errors are detected before anything is enqueued: the call returns
 *     a negative code and writes nothing.  Launch failures return DELTA_ERR_HIP.
 *   - The library keeps no state between calls and may be called from several
 *     host threads at once.
 *   - Keys are used as given: L2 normalisation belongs to the caller.
 *   - g_log is the LOG of the gate: finite and <= 0 expected (a positive value is
 *     computed as given but the chunk form's decay ratios may overflow), or -inf for
 *     g = 0, the hard reset of the DeltaProduct notes (section 3.3), which clears the
 *     state.  On the chunkwise path each log gate is raised to at least -150 first:
 *     every decay across such a position is then exactly 0 in float32, as for g = 0.
 *   - NaN or infinite inputs are not masked: they propagate to the outputs they reach.
 *
 * Environment switches, read at every call:
 *   - DELTA_VALIDATE=1: delta_fwd, delta_fwd_intra, delta_bwd, delta_decode,
 *     delta_decode_kda and delta_fwd_kda first check beta (must be finite) and the log gates (finite or
 *     -inf) and return DELTA_ERR_BAD_VALUE, having written nothing but the start of the
 *     workspace, if one is not.  The check waits for the stream (the call is then
 *     synchronous) and must not be used while the stream is being captured into a graph.
 *   - DELTA_FAULT=launch: every entry point with work to enqueue returns DELTA_ERR_HIP
 *     in place of its first launch and enqueues nothing (for testing callers' error
 *     handling).
 */
#ifndef DELTA_H
#define DELTA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and O.  beta, g_log and the state are always float32. */
enum { DELTA_F32 = 0, DELTA_BF16 = 1 };

/* Return codes. */
enum {
  DELTA_OK = 0,
  DELTA_ERR_NULL_ARG = -1,        /* a required pointer is NULL */
  DELTA_ERR_BAD_SHAPE = -2,       /* negative size, n_h < 1, chunk not a multiple of n_h, too large */
  DELTA_ERR_UNSUPPORTED_DIM = -3, /* dk not in {16,32,64,128}, dv not a multiple of 16 in [16,256],
                                     chunk not in {16,32,48,64}, unknown dtype */
  DELTA_ERR_MISALIGNED = -4,      /* a tensor pointer is not 16-byte aligned (beta, g_log: 4-byte) */
  DELTA_ERR_WORKSPACE = -5,       /* workspace NULL or smaller than delta_fwd_workspace_bytes */
  DELTA_ERR_ALIAS = -6,           /* S_final partially overlaps S0, or an output overlaps an input */
  DELTA_ERR_HIP = -7,             /* a HIP launch or runtime call failed */
  DELTA_ERR_BAD_VALUE = -8,       /* beta not finite, or a log gate NaN or +inf; reported only when
                                     the environment sets DELTA_VALIDATE=1 (see below) */
  DELTA_ERR_NOALLOC_TOO_LARGE = -9 /* delta_fwd_noalloc: the shape needs more workspace than the
                                     library's fixed device array (DELTA_NOALLOC_MAX_BYTES) */
};

/* Problem description shared by all entry points. */
typedef struct delta_shape {
  int32_t B;      /* batch size, >= 0 (0: nothing to do) */
  int32_t L;      /* tokens per sequence (NOT expanded), >= 0 (delta_decode: must be 1);
                     L = 0 writes S_final = S0 (or zeros) and no output */
  int32_t H;      /* heads, >= 0 (0: nothing to do) */
  int32_t dk;     /* key/query head dim: 16, 32, 64 or 128 */
  int32_t dv;     /* value head dim: a multiple of 16 in [16, 256] */
  int32_t n_h;    /* Householder steps per token (DeltaProduct), >= 1; 1 = DeltaNet / GDN */
  int32_t chunk;  /* chunk length C in expanded positions: 16, 32, 48 or 64, a multiple of n_h.
                     Results do not depend on C beyond rounding. */
  int32_t dtype;  /* DELTA_F32 or DELTA_BF16 */
  float scale;    /* readout scale: o = scale * S^T q */
} delta_shape;

/*
 * Bytes of device workspace delta_fwd needs for this shape (a function of the shape only).
 * Holds, per chunk, the UT-transform matrix T (C x C in the input dtype) and the in-chunk
 * cumulative log gate; and, when the sequence is split into
 * segments (see delta_fwd_segments), each segment's summary (a slot of d_k x (d_v + d_k)
 * floats: its state run from zero in float32 and its d_k x d_k transition in the input dtype)
 * and start state (float32 d_k x d_v).
 * Returns DELTA_OK and sets *bytes, or an error code.
 */
int delta_fwd_workspace_bytes(const delta_shape* s, size_t* bytes);

/*
 * Chunkwise-parallel forward pass ("08 linear delta rule & DPLR", sections 2.2-2.3 and
 * section 3; DeltaProduct notes, section 4.1).
 *
 *   q      [B, L, H, dk]          dtype      queries, one per token
 *   k      [B, L*n_h, H, dk]      dtype      keys; the n_h sub-steps of a token are adjacent
 *   v      [B, L*n_h, H, dv]      dtype      values, same layout as k
 *   beta   [B, L*n_h, H]          float32    write strengths (any real; (0,2) allows negative
 *                                            eigenvalues)
 *   g_log  [B, L, H]              float32    log gate per token, or NULL for an ungated model;
 *                                            applied once per token, before its first sub-step
 *   S0     [B, H, dk, dv]         float32    initial state, or NULL for zeros
 *   O      [B, L, H, dv]          dtype      output (written, rounded to nearest even for bf16)
 *   S_final[B, H, dk, dv]         float32    final state, or NULL; may equal S0 exactly
 *                                            (in-place update), must not partially overlap it
 *   workspace                     device memory of at least delta_fwd_workspace_bytes bytes,
 *                                 16-byte aligned; contents on entry are ignored; may be NULL
 *                                 when that size is 0
 *
 * L*n_h need not be a multiple of the chunk: the tail chunk is padded internally with
 * zero keys, values and betas, which leave the state unchanged.
 * Tensor pointers must be 16-byte aligned, except beta and g_log (4-byte).
 */
int delta_fwd(const delta_shape* s, const void* q, const void* k, const void* v,
              const float* beta, const float* g_log, const float* S0, void* O,
              float* S_final, void* workspace, size_t workspace_bytes, void* stream);

/*
 * delta_fwd for callers that cannot allocate device memory (code under graph capture, tight
 * serving loops, harnesses that forbid allocation): the same computation, with the workspace
 * taken from a fixed device array inside the library instead of a caller buffer.  It calls no
 * allocating routine.
 *   - Arguments, results and error codes as delta_fwd (no workspace arguments); shapes whose
 *     delta_fwd_workspace_bytes exceeds DELTA_NOALLOC_MAX_BYTES return
 *     DELTA_ERR_NOALLOC_TOO_LARGE before anything is enqueued.
 *   - The array holds DELTA_NOALLOC_MAX_BYTES on every device the library is used on, from the
 *     first call there until the process ends; its device address is looked up once per device.
 *   - All calls on one device share it: calls that overlap on one device (several streams or
 *     threads) race and must be serialised by the caller.  Its contents on entry do not matter.
 */
#define DELTA_NOALLOC_MAX_BYTES (96u << 20)
int delta_fwd_noalloc(const delta_shape* s, const void* q, const void* k, const void* v,
                      const float* beta, const float* g_log, const float* S0, void* O,
                      float* S_final, void* stream);

/*
 * The two phases of delta_fwd, for callers that schedule them separately (and for per-kernel
 * timing).  delta_fwd_intra computes, per chunk, the UT-transform matrix T and the in-chunk
 * cumulative log gate into the workspace (from k, beta, g_log only);
 * delta_fwd_inter then runs the state recurrence and the outputs from q, k, v, S0 and that
 * workspace (the gated causal Q K^T of each chunk is formed on chip there).  Calling
 * delta_fwd_intra then delta_fwd_inter on one stream with the same arguments and workspace
 * computes exactly what delta_fwd computes.  Arguments as for delta_fwd.
 */
int delta_fwd_intra(const delta_shape* s, const void* k, const float* beta, const float* g_log,
                    void* workspace, size_t workspace_bytes, void* stream);
int delta_fwd_inter(const delta_shape* s, const void* q, const void* k, const void* v,
                    const float* S0, void* O, float* S_final, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * How the inter-chunk phase splits each sequence: *segments segments of *chunks_per_segment
 * chunks (the last may be shorter), a function of the shape alone.  The per-step maps of the
 * recurrence are affine in the state (DeltaProduct notes, section 3), so segments run in
 * parallel: each is summarised from a zero state, the summaries are chained into segment
 * start states, and every segment is then re-run from its start state to produce outputs.
 * With one segment the first two launches do nothing.
 */
int delta_fwd_segments(const delta_shape* s, int32_t* segments, int32_t* chunks_per_segment);

/*
 * The three launches of delta_fwd_inter, for per-kernel timing; called in this order on one
 * stream after delta_fwd_intra, with the same workspace, they compute what delta_fwd_inter
 * computes.  Arguments as for delta_fwd; each reads only the tensors it lists.
 *   delta_fwd_scan_summary  k, v, S0 (segment 0 starts from S0) -> segment summaries, and
 *                           segment 0's start state (a copy of S0)
 *   delta_fwd_scan_combine  segment summaries -> the other segments' start states (sequential,
 *                           float32)
 *   delta_fwd_scan_outputs  q, k, v and the start states (S0 itself when the sequence is not
 *                           split) -> O, S_final.  With a split this launch does not read S0,
 *                           so S_final == S0 (in place) cannot race with it.
 */
int delta_fwd_scan_summary(const delta_shape* s, const void* k, const void* v, const float* S0,
                           void* workspace, size_t workspace_bytes, void* stream);
int delta_fwd_scan_combine(const delta_shape* s, void* workspace, size_t workspace_bytes, void* stream);
int delta_fwd_scan_outputs(const delta_shape* s, const void* q, const void* k, const void* v,
                           const float* S0, void* O, float* S_final, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * Intra-chunk factors only, for inspection and testing ("08 linear delta rule & DPLR",
 * section 2.2 UT transform, section 3 gated form).  Per chunk n of each (b, h):
 *   gc[i]  = sum_{j<=i} log g at position j of the chunk (g at each token's first sub-step)
 *   T      = (I + strictLower(diag(beta) (Gamma * K K^T)))^-1 diag(beta),
 *            Gamma_ij = exp(gc_i - gc_j)
 *   W      = T (exp(gc) * K),   U = T V
 * Outputs (float32, device): T [B, H, NT, C, C], W [B, H, NT, C, dk], U [B, H, NT, C, dv],
 * gc [B, H, NT, C], with NT = ceil(L*n_h / C).  W and U may be NULL (then k/v need not be
 * read for them); T and gc are required.  Inputs as for delta_fwd.
 */
int delta_chunk_wy(const delta_shape* s, const void* k, const void* v, const float* beta,
                   const float* g_log, float* T, float* W, float* U, float* gc, void* stream);

/*
 * Recurrent decode step: one token per (b, h), updating the state in place
 * ("08 linear delta rule & DPLR", recurrent reference after section 2.3; DeltaProduct
 * notes, section 2.6 pseudocode).  s->L must be 1; s->chunk is ignored.
 *   q [B, 1, H, dk], k [B, n_h, H, dk], v [B, n_h, H, dv]   dtype
 *   beta [B, n_h, H], g_log [B, 1, H] or NULL               float32
 *   S [B, H, dk, dv] float32, read and overwritten with  g (prod_j F_j) S + ...
 *   O [B, 1, H, dv] dtype
 */
int delta_decode(const delta_shape* s, const void* q, const void* k, const void* v,
                 const float* beta, const float* g_log, float* S, void* O, void* stream);

/*
 * KDA decode step: the delta rule with a decay per key channel ("08 linear delta rule & DPLR",
 * section 1.4 table and section 5: S <- (I - beta k k^T) Diag(alpha) S + beta k v^T, the
 * diagonal applied first), one token per (b, h), the state updated in place.  As delta_decode
 * with n_h = 1 (s->n_h must be 1), the scalar gate replaced by
 *   a_log [B, 1, H, dk] float32: log alpha per key channel (row r of S decays by
 *                                exp(a_log[.., r])), finite or -inf, <= 0; not NULL.
 * Same argument checks and error codes as delta_decode; a_log must be 16-byte aligned and may
 * not overlap S or O.
 */
int delta_decode_kda(const delta_shape* s, const void* q, const void* k, const void* v,
                     const float* beta, const float* a_log, float* S, void* O, void* stream);

/*
 * KDA forward over a sequence: the delta rule with a decay per key channel ("08 linear delta rule
 * & DPLR", section 1.4 table, KDA row, and section 5:
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,   o_t = scale S_t^T q_t),
 * run token by token with the state held on chip (the recurrence, not a chunked form).
 * s->n_h must be 1; s->chunk is ignored.
 *   q, k [B, L, H, dk], v [B, L, H, dv]      dtype
 *   beta [B, L, H]                            float32
 *   a_log [B, L, H, dk]                       float32   log alpha per key channel (finite or -inf,
 *                                                       <= 0); not NULL; 16-byte aligned
 *   S0 [B, H, dk, dv] float32 or NULL (zeros); O [B, L, H, dv] dtype (written);
 *   S_final [B, H, dk, dv] float32 or NULL; may equal S0 (in place).
 * Alignment, aliasing and error codes as delta_fwd (no workspace).
 */
int delta_fwd_kda(const delta_shape* s, const void* q, const void* k, const void* v,
                  const float* beta, const float* a_log, const float* S0, void* O,
                  float* S_final, void* stream);

/*
 * Bytes of device workspace delta_fwd_kda_chunked needs for this shape (see below).  Shapes other
 * than bf16, dk = dv = 128, chunk 64, n_h = 1: DELTA_ERR_UNSUPPORTED_DIM.
 */
int delta_fwd_kda_chunked_workspace_bytes(const delta_shape* s, size_t* bytes);

/*
 * KDA forward over a sequence in chunks: the same result as delta_fwd_kda (same arguments and
 * meaning), computed chunkwise ("08 linear delta rule & DPLR", section 1.4 table, KDA row, and
 * section 5 for the recurrence; the chunk form follows from it as sections 2.2-2.3 and 3 derive
 * the scalar-gated one: inside a chunk the Gram matrix and the causal Q K^T carry the decay per
 * key channel, e^{Gc_r - Gc_j} with Gc the in-chunk cumulative log decay, and the state decays
 * row by row by e^{Gc_C}).  bf16 only, dk = dv = 128, s->chunk = 64, s->n_h = 1; other shapes
 * return DELTA_ERR_UNSUPPORTED_DIM (delta_fwd_kda takes them).  Each log decay is raised to at
 * least -150 first (a -inf reset then decays to exactly 0).  Workspace: at least
 * delta_fwd_kda_chunked_workspace_bytes bytes, 16-byte aligned, overlapping no argument; its
 * contents need no clearing.  Alignment, aliasing and error codes otherwise as delta_fwd_kda.
 */
int delta_fwd_kda_chunked(const delta_shape* s, const void* q, const void* k, const void* v, const float* beta,
                          const float* a_log, const float* S0, void* O, float* S_final, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace delta_bwd needs for this shape.  bf16 inputs with dk = dv = 128 and
 * chunk 64: per chunk T (bf16), the gate prefix and (I + A)^-1 (float32), the segment summaries
 * and start states of the two state scans, and per chunk its start state (bf16) and the
 * gradient of its end state (bf16 value and bf16 rounding residual), d_k x d_v each.  Other
 * shapes: per chunk T and Q K^T weighted by the gate ratios (C x C float32 each), the gate
 * prefix, and the start state and end-state gradient in float32.  The contents need no clearing
 * between calls.  Returns DELTA_OK and sets *bytes, or an error code.
 */
int delta_bwd_workspace_bytes(const delta_shape* s, size_t* bytes);

/*
 * Backward pass of delta_fwd: the gradients of <O, dO> + <S_final, dS_final> with respect to
 * every input.  The pages define only the forward ("08 linear delta rule & DPLR", sections
 * 2.2-2.3 and 3; DeltaProduct notes, section 4.1); these are its exact derivatives, evaluated
 * chunkwise with the forward's T, gate prefix and chunk states recomputed from the inputs.
 * For bf16 inputs with dk = dv = 128 and chunk 64 the chunk products run on the bf16 MFMA with
 * float32 accumulation (the chunk states and most intermediate tiles rounded to bf16 as
 * operands); otherwise all arithmetic is float32.
 *   q, k, v, beta, g_log, S0   as passed to delta_fwd (g_log NULL: ungated, S0 NULL: zeros)
 *   dO       [B, L, H, dv]        dtype     gradient of O
 *   dS_final [B, H, dk, dv]       float32   gradient of S_final, or NULL for zero
 *   dq       [B, L, H, dk]        float32   written
 *   dk       [B, L*n_h, H, dk]    float32   written
 *   dv       [B, L*n_h, H, dv]    float32   written
 *   dbeta    [B, L*n_h, H]        float32   written
 *   dg_log   [B, L, H]            float32   written; may be NULL (not computed); ignored when
 *                                           g_log is NULL
 *   dS0      [B, H, dk, dv]       float32   written, or NULL (not computed)
 *   workspace                     at least delta_bwd_workspace_bytes bytes, 16-byte aligned
 * Outputs may not overlap the inputs, each other or the workspace.  Alignment as for
 * delta_fwd (dbeta and dg_log: 4-byte).  Error codes as for delta_fwd.
 */
int delta_bwd(const delta_shape* s, const void* q, const void* k, const void* v, const float* beta,
              const float* g_log, const float* S0, const void* dO, const float* dS_final, float* dq,
              float* dk, float* dv, float* dbeta, float* dg_log, float* dS0, void* workspace,
              size_t workspace_bytes, void* stream);

/*
 * Layer prologue ("08 linear delta rule & DPLR" page, Gated DeltaNet layer-design figure after
 * section 3: q/k through ShortConv, SiLU and L2 norm, v through ShortConv and SiLU), applied to
 * the projections before delta_fwd.  Per channel c = head * d + i, a causal depthwise filter of
 * `width` taps (1..4; tap width-1 multiplies the current token, earlier tokens of the same
 * sequence before it, zeros before the first token), then SiLU(x) = x / (1 + exp(-x)); q and k
 * rows (one head of one token) are then divided by sqrt(sum of squares + eps).
 *   xq [B, L, H, dk], xk [B, L*n_h, H, dk], xv [B, L*n_h, H, dv]     dtype    inputs
 *   wq, wk [H*dk, width], wv [H*dv, width]                           float32  filters
 *   q, k, v                                  shapes of xq, xk, xv   dtype    outputs (written)
 * k and v are filtered along their L*n_h rows in order.  Outputs may not overlap any input or
 * each other.  16-byte aligned pointers.  s->chunk and s->scale are ignored.  Error codes as
 * delta_fwd (width outside 1..4: DELTA_ERR_UNSUPPORTED_DIM; eps < 0: DELTA_ERR_BAD_SHAPE).
 */
int delta_layer_prologue(const delta_shape* s, int32_t width, float eps, const void* xq, const void* xk,
                         const void* xv, const float* wq, const float* wk, const float* wv, void* q, void* k,
                         void* v, void* stream);

/*
 * Layer prologue for one decode token (the same steps as delta_layer_prologue), the filters'
 * recent inputs carried between calls.  s->L must be 1; s->chunk and s->scale are ignored.
 *   xq [B, 1, H, dk], xk [B, n_h, H, dk], xv [B, n_h, H, dv]   dtype    this token's projections
 *   wq, wk [H*dk, width], wv [H*dv, width]                      float32  filters
 *   conv_q [B, width-1, H, dk], conv_k [B, width-1, H, dk], conv_v [B, width-1, H, dv]
 *                                        dtype, read and updated: the width-1 most recent input
 *                                        rows of each filter, oldest first (NULL when width = 1)
 *   q [B, 1, H, dk], k [B, n_h, H, dk], v [B, n_h, H, dv]      dtype    outputs (written)
 * k and v take their n_h rows in order, each a step of the filter.  After a prefill over L
 * inputs, the state is the last width-1 input rows of xq (of xk, xv: along their L*n_h rows),
 * zeros where the sequence is shorter.  No overlap between outputs, states and inputs.
 * 16-byte aligned pointers.  Error codes as delta_layer_prologue (L != 1: DELTA_ERR_BAD_SHAPE).
 */
int delta_layer_prologue_step(const delta_shape* s, int32_t width, float eps, const void* xq,
                              const void* xk, const void* xv, const float* wq, const float* wk,
                              const float* wv, void* conv_q, void* conv_k, void* conv_v, void* q,
                              void* k, void* v, void* stream);

/*
 * Layer epilogue (same figure: Norm, then the output gate): per head of each token,
 *   y = o / sqrt(mean(o^2) + eps) * weight * SiLU(g)
 *   o, g, y [B, L, H, dv] dtype; weight [dv] float32 (shared by the heads).
 * y may be o itself (in place); no other overlap.  16-byte aligned pointers.
 */
int delta_layer_epilogue(const delta_shape* s, float eps, const void* o, const void* g, const float* weight,
                         void* y, void* stream);

/* Static description of a return code. */
const char* delta_strerror(int code);

#ifdef __cplusplus
}
#endif
#endif /* DELTA_H */
