/*
 * gdn.h -- libgdn: chunked Gated DeltaNet prefill forward for AMD Instinct MI355X (gfx950).
 *
 * The operation is the gated delta rule, the recurrence inside the model's linear-attention
 * (Gated DeltaNet) layers (System1-Omni PR #186 page, "Purpose and summary"), evaluated 64
 * tokens at a time as in the fused kernel of the "open-jev-fast" README ("Phase 3", item 1),
 * which follows the Gated DeltaNet paper it lists as reference [5]:
 *
 *     S_t = exp(g_t) * S_{t-1} * (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = S_t q_t
 *
 * over packed variable-length sequences, each with its own optional fp32 initial state (the
 * prefix-continuation form: in the "open-jev-fast" README, "Phase 2" item 2, a long prompt's
 * end state seeds every candidate that continues it; PR #186, "Review scope and map", keeps a
 * separate state per candidate).
 * There is no 1/sqrt(dk) scale on q: o_t = S_t q_t exactly.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  * Every data pointer is DEVICE memory owned by the caller.  The library never allocates,
 *    frees or synchronises, and keeps no state between calls except a per-thread copy of the
 *    last HIP error.  All work is enqueued on the caller's `stream` (NULL = the default stream).
 *  * Layouts are row-major and contiguous.  bf16 tensors are raw 16-bit bf16 values.
 *      q, k    : bf16 [T, Hk, dk]          v : bf16 [T, Hv, dv]
 *      g, beta : fp32 [T, Hv]   (g is the log-decay, one value per token per v-head, <= 0;
 *                                values below -40, a decay of e^-40 = 4e-18, act as -40)
 *      cu_seqlens : int32 [N+1], cu[0] = 0, non-decreasing, cu[N] = T
 *      h0, hT  : fp32 [N, Hv, dk, dv], key-major: element [n][h][i][j] = S[j][i] (H = S^T)
 *      o       : bf16 [T, Hv, dv]
 *    v-head h reads q/k head h / (Hv / Hk) ("open-jev-fast" README, "Phase 3" item 3: q/k at 16
 *    heads, v at 32).
 *  * Alignment: bf16 tensors (q, k, v, o, qkv, z, norm_w, y), states (h0, hT) and the workspace
 *    16 bytes; conv_w 8 bytes; g, beta and cu_seqlens 4 bytes (GDN_ERR_ALIGN otherwise).
 *  * All argument checks happen on the host BEFORE anything is enqueued.  On any error nothing
 *    is launched and the outputs are untouched.  GDN_OK means "enqueued": results are valid once
 *    the stream reaches that point.  GDN_ERR_HIP means a launch failed; gdn_last_hip_error()
 *    returns the hipError_t of the calling thread's last such failure.
 *  * The library cannot read cu_seqlens without a device sync, so it trusts that they are
 *    monotone with cu[N] = T (the Python binding checks a host copy).  With N = 1 some kernels
 *    take the bounds {0, T} from the descriptor instead of reading them, so cu_seqlens must be
 *    exactly {0, T}.  Zero-length sequences are allowed: they produce no output rows and
 *    hT[n] = h0[n] (or zeros).
 *  * hT may be exactly h0 (in-place continuation).  Any other overlap of an output with an
 *    input, or of o with hT, is GDN_ERR_ALIAS.
 *  * The workspace is caller-owned device memory of at least *_workspace_size() bytes; its
 *    contents on entry are ignored and on exit are unspecified.  Calls that share a workspace
 *    must be ordered on one stream.
 *  * The calls only launch kernels on `stream` (no allocation, no memset, no synchronisation), so
 *    a caller may capture them in a HIP graph and replay it with new contents in the same buffers.
 *    gdn_mixer_fwd_fused_norm, which launches cooperatively, is the exception.
 *  * Only dk = dv = 128 is supported (GDN_ERR_UNSUPPORTED otherwise).
 */
#ifndef LIBGDN_GDN_H
#define LIBGDN_GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef GDN_EXPORT
#define GDN_EXPORT __attribute__((visibility("default")))
#endif

#define GDN_ABI_VERSION 1

typedef enum {
  GDN_OK = 0,
  GDN_ERR_NULL = 1,        /* a required pointer is NULL                                   */
  GDN_ERR_SHAPE = 2,       /* N < 1, T < 0, Hk < 1, Hv % Hk != 0, or a size overflows       */
  GDN_ERR_UNSUPPORTED = 3, /* dk or dv other than 128, or a conv/norm setting not supported  */
  GDN_ERR_ALIGN = 4,       /* a pointer is not aligned as required                          */
  GDN_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than the required size              */
  GDN_ERR_ALIAS = 6,       /* an output overlaps an input or the workspace (hT == h0 is ok) */
  GDN_ERR_HIP = 7,         /* a HIP launch failed; see gdn_last_hip_error()                 */
  GDN_ERR_SCRATCH_LIMIT = 8 /* gdn_chunk_fwd_noalloc: the shape needs more scratch than the
                               library's static buffer (GDN_NOALLOC_SCRATCH_BYTES)            */
} gdn_status;

/* Size of the static device scratch behind gdn_chunk_fwd_noalloc (per GPU). */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* Problem description.  Sizes are host values; nothing is read from device memory. */
typedef struct {
  int64_t total_tokens;   /* T = cu_seqlens[N] (>= 0)                                     */
  int32_t num_seqs;       /* N >= 1                                                       */
  int32_t num_k_heads;    /* Hk >= 1 (q and k heads)                                      */
  int32_t num_v_heads;    /* Hv, a multiple of Hk                                         */
  int32_t head_dim_k;     /* dk, must be 128                                              */
  int32_t head_dim_v;     /* dv, must be 128                                              */
  void *workspace;        /* device, caller-owned, >= gdn_chunk_fwd_workspace_size() bytes */
  size_t workspace_bytes;
} gdn_chunk_desc;

/* ABI version of the loaded library (GDN_ABI_VERSION at build time).  The PR #186 page keeps its
 * device library behind a numbered binary interface ("Purpose and summary": version 9 there) and
 * runs a contract check of it ("Test plan and results"); a caller compares this number with the
 * header it was built against.  Never fails. */
GDN_EXPORT int gdn_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL; unknown codes get a generic
 * text).  Part of the error paths of the library interface that the PR #186 page's review covers
 * ("Review scope and map": callers, error and resource paths inspected). */
GDN_EXPORT const char *gdn_status_string(int status);

/* hipError_t of the calling thread's last GDN_ERR_HIP, 0 if none (thread-local; never fails).
 * The HIP side of the same error paths (PR #186 page, "Review scope and map"). */
GDN_EXPORT int gdn_last_hip_error(void);

/* Workspace bytes gdn_chunk_fwd needs for this shape; 0 if the description is invalid.
 * The workspace and pointer fields of *d are ignored.  One sequence (N = 1) of at least 32 chunks
 * with at most 8 v-heads needs 6 MiB more: its state pass may run split along time (below).
 * The caller owns the scratch and its lifetime, as the PR #186 page's library does ("Review
 * scope and map": workspace checked against the plan, scratch address lifetime owned by the
 * executor, dirty-workspace tests). */
GDN_EXPORT size_t gdn_chunk_fwd_workspace_size(const gdn_chunk_desc *d);

/*
 * Chunked gated-delta-rule prefill forward over a packed batch.
 *   q, k, v, g, beta, cu_seqlens : inputs as laid out above (device)
 *   h0 : initial states, or NULL for zero states (device)
 *   o  : output (device), written for every token
 *   hT : final states, or NULL to skip them (device); may equal h0
 * Works in 64-token chunks: in each chunk the prefix sums of g, the key Gram matrix and the
 * unit-lower-triangular inverse of the UT transform, then a pass over the chunks in order that
 * carries the fp32 state and emits the outputs (the step list of the "open-jev-fast" README's
 * fused kernel, "Phase 3" item 1).  A single sequence whose heads
 * would leave most of the device idle has its state pass split along time (segment end states,
 * segment transitions, a scan of the segment states, then the outputs); the results meet the same
 * tolerances, and are not bitwise those of a call on a different batch shape.
 */
GDN_EXPORT int gdn_chunk_fwd(const gdn_chunk_desc *d, const void *q, const void *k, const void *v,
                  const float *g, const float *beta, const int32_t *cu_seqlens, const float *h0,
                  void *o, float *hT, void *stream);

/*
 * gdn_chunk_fwd for callers that cannot allocate device memory: code under HIP graph capture,
 * serving loops and harnesses that forbid hipMalloc.  Arguments and results are gdn_chunk_fwd's,
 * but d->workspace and d->workspace_bytes are ignored: the records and state buffers live in the
 * library's own scratch, a static device array of GDN_NOALLOC_SCRATCH_BYTES (64 MiB) on every GPU
 * the library runs on, held until the process ends.
 *  * Limit: gdn_chunk_fwd_workspace_size(d) <= GDN_NOALLOC_SCRATCH_BYTES, else
 *    GDN_ERR_SCRATCH_LIMIT with nothing launched (at Hv = 32: T / 64 + N <= 110, e.g. one sequence
 *    of up to 7,039 tokens).  Every other check and error is gdn_chunk_fwd's.
 *  * Allocates nothing and frees nothing.  The first call on a GPU looks up that GPU's copy of the
 *    array (hipGetSymbolAddress, with the GPU made current for the lookup and the previous
 *    current device restored); make one call before capturing a graph.  A failed lookup is
 *    GDN_ERR_HIP, on that call and every later one on that GPU.
 *  * Every call on one GPU shares that GPU's array: calls that overlap in time on one GPU (on
 *    different streams, or from host threads without ordering) race and give wrong results.
 *    Calls ordered on one stream are safe.  The array keeps the last call's contents; nothing in
 *    it needs clearing, since each call writes every byte of it that the call reads.
 */
GDN_EXPORT int gdn_chunk_fwd_noalloc(const gdn_chunk_desc *d, const void *q, const void *k,
                                     const void *v, const float *g, const float *beta,
                                     const int32_t *cu_seqlens, const float *h0, void *o, float *hT,
                                     void *stream);

/*
 * gdn_chunk_fwd with the initial states drawn from a pool by index: one prefix's end state seeds
 * several candidates without being copied ("open-jev-fast" README, "Phase 2" item 2; PR #186,
 * "Review scope and map", a separate state per candidate).
 *   h0       : fp32 [num_h0, Hv, dk, dv] (device), num_h0 >= 1
 *   h0_index : int32 [N] (device).  Sequence n starts from h0[h0_index[n]]; an index outside
 *              [0, num_h0) means a zero state (the library cannot check device values, so an
 *              out-of-range index is defined rather than an error).
 * Other arguments as gdn_chunk_fwd; the workspace size is gdn_chunk_fwd_workspace_size().
 * Errors: GDN_ERR_NULL if h0 or h0_index is NULL, GDN_ERR_SHAPE if num_h0 < 1, GDN_ERR_ALIAS if
 * hT overlaps h0 at all (other sequences may still read the row), or if an output overlaps
 * h0_index; GDN_ERR_ALIGN if h0_index is not 4-byte aligned.
 */
GDN_EXPORT int gdn_chunk_fwd_indexed(const gdn_chunk_desc *d, const void *q, const void *k,
                                     const void *v, const float *g, const float *beta,
                                     const int32_t *cu_seqlens, const float *h0, int32_t num_h0,
                                     const int32_t *h0_index, void *o, float *hT, void *stream);

/*
 * The two stages of gdn_chunk_fwd, callable on their own (gdn_chunk_fwd = gdn_chunk_prep, then
 * gdn_state_pass, on one stream with one workspace).  The split generalises the two-chunk path
 * of the "open-jev-fast" README ("Phase 3", item 1), which computes what does not involve the
 * recurrent state for both chunks at once and carries only the state from one to the next.
 *
 * gdn_chunk_prep: for every (chunk, v-head) in parallel -- local cumsum of g, K K^T and Q K^T,
 *   A = beta_i e^{G_i - G_j} k_i.k_j (i > j), T = (I + A)^-1 -- writes one record per (chunk,
 *   v-head) into the workspace: T diag(beta), the masked decayed Q K^T and the decays.  Reads q,
 *   k, g, beta, cu_seqlens.
 * gdn_state_pass: for every (sequence, v-head, 16 value columns) in parallel, walks the chunks
 *   in order with the fp32 state on chip, writing o and hT.  Reads q, k, v, cu_seqlens, h0 and
 *   the workspace exactly as gdn_chunk_prep left it for the same inputs and shapes.
 * Arguments, layouts and errors are those of gdn_chunk_fwd.
 */
GDN_EXPORT int gdn_chunk_prep(const gdn_chunk_desc *d, const void *q, const void *k,
                              const float *g, const float *beta, const int32_t *cu_seqlens,
                              void *stream);
GDN_EXPORT int gdn_state_pass(const gdn_chunk_desc *d, const void *q, const void *k,
                              const void *v, const int32_t *cu_seqlens, const float *h0, void *o,
                              float *hT, void *stream);

/*
 * GDN mixer: the gated delta rule between its input prep -- a depthwise causal convolution with
 * SiLU, the split into q, k and v, and the L2 normalisation of q and k -- and its SiLU-gated
 * RMSNorm (the "open-jev-fast" README, "Phase 2" item 1, has one fused kernel for each side).
 *   qkv    : bf16 [T, 2*Hk*dk + Hv*dv], channels q | k | v, head-major inside each block
 *   conv_w : bf16 [2*Hk*dk + Hv*dv, conv_taps]; tap conv_taps-1 multiplies the current token;
 *            the window holds zeros before every sequence start (no bias)
 *   per channel: c = causal depthwise conv; a = c * sigmoid(c)
 *   per (token, k-head): q, k = a / sqrt(sum a^2 + 1e-6)
 *   o = gated delta rule(q, k, v = a, g, beta, h0) as gdn_chunk_fwd
 *   y = o / sqrt(mean_dv(o^2) + norm_eps) * norm_w * z * sigmoid(z)   per (token, v-head)
 *   z : bf16 [T, Hv, dv];  norm_w : bf16 [dv], shared by all heads;  y : bf16 [T, Hv, dv]
 * Only conv_taps = 4 is supported.
 */
typedef struct {
  gdn_chunk_desc chunk;   /* shapes and workspace (gdn_mixer_fwd_workspace_size bytes) */
  int32_t conv_taps;      /* 4                                                          */
  float norm_eps;         /* RMSNorm epsilon, e.g. 1e-6                                 */
} gdn_mixer_desc;

GDN_EXPORT size_t gdn_mixer_fwd_workspace_size(const gdn_mixer_desc *d);

GDN_EXPORT int gdn_mixer_fwd(const gdn_mixer_desc *d, const void *qkv, const void *conv_w, const float *g,
                  const float *beta, const void *z, const void *norm_w,
                  const int32_t *cu_seqlens, const float *h0, void *y, float *hT, void *stream);

/*
 * gdn_mixer_fwd with the gated RMSNorm fused into the state pass's output path instead of run as a
 * kernel of its own (the "open-jev-fast" README, "Phase 3" item 4, measured this fusion on B300 and
 * kept the separate kernel).  Each of a head's column workgroups publishes its share of every
 * row's sum of squares and, a few chunks later, writes y for its own columns, so o never goes to
 * memory.  That needs every workgroup of a head resident at once: the state pass is launched
 * cooperatively, so this entry point returns GDN_ERR_UNSUPPORTED (nothing launched) when the work
 * items do not fit on the device in one round (N * Hv * 8 above the device's concurrent
 * workgroups), when one long sequence would take the time split, or when the device has no
 * cooperative launch.  Arguments, workspace (gdn_mixer_fwd_workspace_size) and tolerances are
 * gdn_mixer_fwd's; y can differ from it in the last bf16 bit (the row's sum of squares is added in
 * another order).  Measured on MI355X at T = 936, Hk = 16, Hv = 32 (48 layers): 97 us per layer
 * against 43 us for gdn_mixer_fwd, so gdn_mixer_fwd keeps the separate norm kernel.
 */
GDN_EXPORT int gdn_mixer_fwd_fused_norm(const gdn_mixer_desc *d, const void *qkv, const void *conv_w,
                                        const float *g, const float *beta, const void *z,
                                        const void *norm_w, const int32_t *cu_seqlens,
                                        const float *h0, void *y, float *hT, void *stream);

/*
 * gdn_mixer_fwd with the gate parameters made inside the mixer's first kernel from the layer's
 * projections, in place of g and beta as inputs (the "open-jev-fast" README, "Phase 2" item 1,
 * lists "gate parameters" as the last step of its fused GDN input prep).  The pages give no
 * formula; this follows the Mamba2-style gating of the Gated DeltaNet paper that README cites
 * (Yang, Kautz & Hatamizadeh, ICLR 2025): for token t and v-head h,
 *     g[t,h]    = -exp(A_log[h]) * softplus(a[t,h] + dt_bias[h])     (log-decay, < 0)
 *     beta[t,h] = sigmoid(b[t,h])
 * computed in fp32 on the hardware exp2, log2 and reciprocal (softplus without overflow, as
 * max(x, 0) + log(1 + e^-|x|)); g then meets the floor of -40 that every log-decay meets.
 *   a, b          : bf16 [T, Hv] (2-byte aligned) -- the projections' gate rows
 *   A_log, dt_bias: fp32 [Hv] (4-byte aligned)    -- per-head parameters
 * Every other argument, the workspace (gdn_mixer_fwd_workspace_size) and the errors are
 * gdn_mixer_fwd's; a, b, A_log and dt_bias may be NULL only when T == 0.  Inputs are only read.
 */
GDN_EXPORT int gdn_mixer_fwd_gates(const gdn_mixer_desc *d, const void *qkv, const void *conv_w,
                                   const void *a, const void *b, const float *A_log,
                                   const float *dt_bias, const void *z, const void *norm_w,
                                   const int32_t *cu_seqlens, const float *h0, void *y, float *hT,
                                   void *stream);

/*
 * The mixer continuing from carried states: beside the recurrent state, each sequence carries
 * the conv input window -- the last conv_taps - 1 rows of qkv before it -- so that both can pass
 * from a prefix to the candidates that continue it (the "open-jev-fast" README, "Phase 2" item 2,
 * keeps the window and the recurrent state of a candidate's path identical to a full run).
 * C = 2*Hk*dk + Hv*dv, W = conv_taps - 1 (= 3).
 *   h0       : fp32 [num_states, Hv, dk, dv] or NULL (zero states)
 *   conv_in  : bf16 [num_states, W, C] or NULL (zeros before every sequence), oldest row first:
 *              row W-1 is the input just before the sequence's first token
 *   state_index : int32 [N] or NULL.  Sequence n continues from state and window
 *              state_index[n]; an index outside [0, num_states) means zeros.  NULL: sequence n
 *              continues from state n, and num_states must be N.
 *   hT       : fp32 [N, Hv, dk, dv] or NULL;  conv_out : bf16 [N, W, C] or NULL -- the last W
 *              rows of sequence n's input stream (its window followed by its tokens), copied
 *              bit for bit: the window the next call continues from.
 * gdn_mixer_fwd is this with conv_in, state_index and conv_out NULL.  hT == h0 and conv_out ==
 * conv_in (in-place continuation) are allowed when state_index is NULL; with an index any
 * overlap of an output with a pool is GDN_ERR_ALIAS.  conv_in and conv_out need 16-byte
 * alignment, state_index 4.  GDN_ERR_SHAPE if num_states < 1, or num_states != N without an
 * index.  Workspace: gdn_mixer_fwd_workspace_size().
 */
GDN_EXPORT int gdn_mixer_fwd_cont(const gdn_mixer_desc *d, const void *qkv, const void *conv_w,
                                  const float *g, const float *beta, const void *z,
                                  const void *norm_w, const int32_t *cu_seqlens, const float *h0,
                                  const void *conv_in, int32_t num_states,
                                  const int32_t *state_index, void *y, float *hT, void *conv_out,
                                  void *stream);

/*
 * gdn_mixer_fwd_cont with the gate parameters made in the mixer's first kernel, as in
 * gdn_mixer_fwd_gates: a continuation (the "open-jev-fast" README, "Phase 2" item 2) of a layer
 * whose input prep also makes its gates ("Phase 2" item 1).  a, b, A_log and dt_bias replace g
 * and beta with gdn_mixer_fwd_gates's layouts and checks; every other argument, the workspace and
 * the errors are gdn_mixer_fwd_cont's.
 */
GDN_EXPORT int gdn_mixer_fwd_gates_cont(const gdn_mixer_desc *d, const void *qkv, const void *conv_w,
                                        const void *a, const void *b, const float *A_log,
                                        const float *dt_bias, const void *z, const void *norm_w,
                                        const int32_t *cu_seqlens, const float *h0,
                                        const void *conv_in, int32_t num_states,
                                        const int32_t *state_index, void *y, float *hT,
                                        void *conv_out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBGDN_GDN_H */
