/*
 * gdr.h -- C ABI of the gated delta rule library for AMD MI355X (gfx950).
 *
 * The operation (GatedDeltaRule.ixx File Reference, "Detailed Description"):
 * per (sequence, value head) an fp32 state S of shape [d_k, d_v] that does not
 * grow with context; for every token t
 *     S     <- S * exp(g_t)
 *     delta <- (v_t - k_t^T S) * beta_t
 *     S     <- S + k_t (outer) delta
 *     o_t   <- q_t^T S
 * where q_t and k_t are L2-normalised and q_t is further scaled by
 * 1/sqrt(d_k), and the gates are derived inside the library from the raw
 * projections a, b and the per-head parameters A_log, dt_bias:
 *     beta_t = sigmoid(b_t),   g_t = -exp(A_log) * softplus(a_t + dt_bias).
 * The same page states the two forms this library exports -- the sequential
 * recurrence for decode and a chunked (UT-transform) form for prefill with one
 * triangular solve per chunk of 32 steps -- which agree up to float
 * reassociation, and that the layer is inference-only (no backward).
 * The Track L pull request (tessera #77, "Numerics finding") adds that the rule
 * is well conditioned only with L2-normalised keys and fp32 state; this
 * library therefore always normalises q and k and always keeps S in fp32.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers to dense, row-major, contiguous
 *   memory.  q, k, v, o, q_hat, k_hat and the states must be 16-byte aligned
 *   (they move in 16-byte vectors); a, b, g, beta, A_log, dt_bias and
 *   cu_seqlens need only the alignment of their element type.  The caller
 *   owns every buffer and the stream.
 * - Layouts (total = number of tokens in the batch):
 *     q, k          [total, H_k, d_k]   dtype
 *     v             [total, H_v, d_v]   dtype
 *     a, b          [total, H_v]        dtype
 *     A_log, dt_bias[H_v]               fp32
 *     states        [num_seqs, H_v, d_k, d_v]  fp32
 *     o             [total, H_v, d_v]   dtype
 *   Value head h reads key head h / (H_v / H_k) (H_v consecutive value heads
 *   share one key head).  Dense batches hold num_seqs sequences of seq_len
 *   tokens one after another; packed batches give cu_seqlens.
 * - Every call is asynchronous on `stream`.  The library never allocates,
 *   frees or synchronises, holds no global state, and is thread-safe.
 * - Shape, dtype, pointer and alignment checks are synchronous: on failure
 *   nothing is launched and nothing is written.  Faults inside a kernel show
 *   up at the caller's next synchronisation.  GDR_ERR_LAUNCH reports a failed
 *   kernel launch.
 * - The contents of cu_seqlens are trusted (device memory is not read on the
 *   host): cu[0] = 0, nondecreasing, cu[num_seqs] = total_tokens.
 * - Outputs are fully overwritten.  final_state may be the same buffer as
 *   initial_state (in-place decode); no other aliasing is allowed.
 */
#ifndef GDR_H
#define GDR_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDR_ABI_VERSION 13

/* Symbols of this header are the only ones the shared library exports. */
#if defined(__GNUC__) || defined(__clang__)
#define GDR_API __attribute__((visibility("default")))
#else
#define GDR_API
#endif

typedef enum gdr_status {
  GDR_OK = 0,
  GDR_ERR_NULL = 1,        /* a required pointer is NULL                         */
  GDR_ERR_SHAPE = 2,       /* inconsistent sizes (H_v % H_k, totals, negatives)  */
  GDR_ERR_UNSUPPORTED = 3, /* a valid shape this build has no kernel for         */
  GDR_ERR_ALIGN = 4,       /* a tensor pointer breaks its alignment rule         */
  GDR_ERR_WORKSPACE = 5,   /* a workspace smaller than the call needs            */
  GDR_ERR_LAUNCH = 6,      /* the HIP runtime refused a kernel launch            */
  GDR_ERR_ALIAS = 7        /* an output overlaps an input it may not alias       */
} gdr_status;

typedef enum gdr_dtype {
  GDR_F32 = 0,  /* IEEE binary32                                         */
  GDR_BF16 = 1  /* bfloat16 (8-bit exponent, 7-bit stored mantissa)       */
} gdr_dtype;

/*
 * Problem description, passed by pointer to every call (read only during the
 * call; the library keeps no reference to it).
 */
typedef struct gdr_shape {
  int32_t num_seqs;          /* N >= 0: sequences in the batch                        */
  int32_t seq_len;           /* dense batches: tokens per sequence (>= 0);            */
                             /*   ignored when cu_seqlens != NULL                     */
  int64_t total_tokens;      /* tokens in the batch; dense: num_seqs * seq_len        */
  const int32_t *cu_seqlens; /* device [num_seqs + 1] prefix sums of the lengths, or  */
                             /*   NULL for a dense batch                              */
  int32_t H_k;               /* key heads (>= 1)                                      */
  int32_t H_v;               /* value heads, a multiple of H_k                        */
  int32_t d_k;               /* key/query head size: 16, 32, 64 or 128                */
  int32_t d_v;               /* value head size: 16, 32, 64 or 128                    */
  int32_t dtype;             /* gdr_dtype of q, k, v, a, b and o                      */
  int32_t chunk;             /* chunked form: tokens per chunk, 16, 32 or 64          */
                             /*   (ignored by the recurrent form and the gates)       */
  float scale;               /* extra factor on q; <= 0 selects 1/sqrt(d_k)           */
  float l2_eps;              /* normalisation x / sqrt(sum x^2 + l2_eps), >= 0        */
} gdr_shape;

/*
 * gdr_gates -- the gates and the normalised q, k, as the component derives
 * them (GatedDeltaRule.ixx File Reference, "Detailed Description"):
 *   beta = sigmoid(b), g = -exp(A_log[h]) * softplus(a + dt_bias[h])   [total, H_v] fp32
 *   q_hat = scale * q / sqrt(|q|^2 + l2_eps),  k_hat = k / sqrt(|k|^2 + l2_eps)
 *                                                          [total, H_k, d_k] dtype
 * Any of q_hat, k_hat, g, beta may be NULL (that output is skipped); the
 * inputs an output needs must then be non-NULL.  The forward entry points do
 * not call this (they derive the same quantities inside their own kernels);
 * it is exported for callers that want the gates themselves.
 */
GDR_API gdr_status gdr_gates(const gdr_shape *shape, const void *q, const void *k, const void *a,
                     const void *b, const float *A_log, const float *dt_bias, void *q_hat,
                     void *k_hat, float *g, float *beta, hipStream_t stream);

/*
 * gdr_recurrent_fwd -- the sequential (decode) form: each token updates the
 * state once, in order (GatedDeltaRule.ixx File Reference, "Detailed
 * Description": decode runs the sequential recurrence).  Works for any
 * sequence length; a decode step is a call with seq_len = 1 and
 * final_state == initial_state.
 *   initial_state : fp32 [N, H_v, d_k, d_v], or NULL for zeros
 *   o             : dtype [total, H_v, d_v]
 *   final_state   : fp32 [N, H_v, d_k, d_v], or NULL to drop it; may equal
 *                   initial_state
 */
GDR_API gdr_status gdr_recurrent_fwd(const gdr_shape *shape, const void *q, const void *k, const void *v,
                             const void *a, const void *b, const float *A_log,
                             const float *dt_bias, const float *initial_state, void *o,
                             float *final_state, hipStream_t stream);

/*
 * gdr_chunked_fwd -- the chunked (prefill) form: the same arithmetic regrouped
 * per chunk of `chunk` tokens into dense contractions plus one forward
 * substitution of (I + A) per chunk (GatedDeltaRule.ixx File Reference,
 * "Detailed Description"; Track L pull request, L2: chunk-parallel
 * UT-transform whose only non-GEMM step is the (I + A)^-1 forward
 * substitution).  Chunks restart at every sequence start; the last chunk of a
 * sequence may be partial.  Arguments as gdr_recurrent_fwd, plus:
 *   workspace       : device memory of gdr_chunked_workspace_bytes(shape)
 *                     bytes, 256-byte aligned, zero-filled before its first
 *                     use (the library leaves it zero-filled again when a call
 *                     completes), overlapping no other argument; or NULL
 *   workspace_bytes : its size; below the reported size is GDR_ERR_WORKSPACE
 * bf16 with d_k = 128, d_v = 64 or 128 and chunk = 32 runs on the matrix
 * cores with bf16 operands and fp32 accumulation and state; every other
 * supported shape runs a vector fp32 kernel and ignores the workspace.  On
 * the matrix cores, with a workspace (gdr_chunked_workspace_bytes > 0), a
 * launch of one workgroup per compute unit splits the work: producer
 * workgroups form every chunk's triangular inverse, output mask and row
 * factors once per value head, and the chain workgroups of that value head
 * read them through the workspace (a ring of records per value head, so its
 * size does not depend on the sequence length).  When the batch's chains do
 * not all fit the GPU at once, consecutive such launches each take as many
 * sequences as fit, provided the sequences average at least 1024 tokens;
 * otherwise, without a workspace, or where a launch fails, every chain
 * workgroup forms them itself in one launch.  Both give the same results up to float
 * reassociation.  Calls that share one workspace must not overlap in time.
 * The workgroups of that launch wait on one another, so they must all run
 * together: kernels of other streams that hold compute units only delay it,
 * but if a workgroup cannot start within about a second, the waits give up,
 * the results are not valid, and the 32-bit word at byte offset 8 + 128 i
 * (i < 16) of the workspace is left nonzero for some i (every such word is
 * zero after a call that completed normally).
 */
GDR_API gdr_status gdr_chunked_fwd(const gdr_shape *shape, const void *q, const void *k, const void *v,
                           const void *a, const void *b, const float *A_log, const float *dt_bias,
                           const float *initial_state, void *o, float *final_state,
                           void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace gdr_chunked_fwd uses for `shape`: 0 when the shape has
 * no cooperative path (or is invalid), else a size that depends on num_seqs,
 * H_k, H_v and d_v but not on the sequence lengths: that of one launch of the
 * sequences that fit the device at once. */
GDR_API size_t gdr_chunked_workspace_bytes(const gdr_shape *shape);

/* Size of the scratch array gdr_chunked_fwd_noalloc uses as its workspace. */
#define GDR_NOALLOC_SCRATCH_BYTES (6u << 20)

/*
 * gdr_chunked_fwd_noalloc -- gdr_chunked_fwd for callers that cannot allocate
 * device memory: code under stream capture, tight serving loops, harnesses
 * that forbid allocation.  The call allocates and frees nothing.  Its
 * cooperative workspace is the library's own scratch array of
 * GDR_NOALLOC_SCRATCH_BYTES bytes in each GPU's memory, held until the
 * process ends.  Arguments, results and errors as gdr_chunked_fwd without the
 * workspace arguments, plus:
 *   - a shape whose cooperative workspace (gdr_chunked_workspace_bytes)
 *     exceeds GDR_NOALLOC_SCRATCH_BYTES returns GDR_ERR_WORKSPACE and runs
 *     nothing;
 *   - a shape with no cooperative path runs what gdr_chunked_fwd runs without
 *     a workspace;
 *   - the first call on a device looks up that device's copy of the array
 *     (the device must be current); failure is GDR_ERR_LAUNCH;
 *   - each call clears the array's counters and flags on `stream` before its
 *     launch (a small fill kernel, no memset);
 *   - all calls on one GPU share that GPU's array: calls that overlap in time
 *     on one GPU (other streams, other threads) race.
 */
GDR_API gdr_status gdr_chunked_fwd_noalloc(const gdr_shape *shape, const void *q, const void *k,
                                           const void *v, const void *a, const void *b,
                                           const float *A_log, const float *dt_bias,
                                           const float *initial_state, void *o,
                                           float *final_state, hipStream_t stream);

/*
 * gdr_conv_silu -- the short causal convolution and SiLU that turn the in_proj
 * output into q, k, v (flashprove issue "P1: Qwen3.8-27B port, tracking": the
 * layer runs from the in_proj outputs through a 4-tap conv1d and SiLU to the
 * q/k L2 norm, the gates and the rule; PLENA_Simulator pull request 113: the
 * short convolution has per-channel weights, an optional bias and a history
 * carried between calls).  The pages print no formula; this library reads it
 * as a depthwise convolution over the C = 2 H_k d_k + H_v d_v channels of x,
 * tap width-1 on the newest input:
 *     y[t, c] = SiLU(bias[c] + sum_j weight[c, j] * x[t - (width-1) + j, c]),
 * SiLU(u) = u * sigmoid(u), inputs before a sequence's first token taken from
 * its history conv_state_in[n, c, 0 .. width-2] (oldest first; NULL for
 * zeros).  y is split by channel into q ([0, H_k d_k)), k ([H_k d_k,
 * 2 H_k d_k)) and v (the rest), each dense in the layouts above, ready for
 * gdr_chunked_fwd / gdr_recurrent_fwd.  conv_state_out receives the last
 * width-1 inputs of every sequence (older history moving up when a sequence is
 * shorter than width-1); a decode step is a call with seq_len = 1.
 *   x              : dtype [total, C]                      (16-byte aligned)
 *   weight         : fp32  [C, width], 2 <= width <= 4      (16-byte aligned)
 *   bias           : fp32  [C], or NULL for none            (16-byte aligned)
 *   conv_state_in  : dtype [num_seqs, C, width-1], or NULL for zeros
 *   q, k           : dtype [total, H_k, d_k]                (16-byte aligned)
 *   v              : dtype [total, H_v, d_v]                (16-byte aligned)
 *   conv_state_out : dtype [num_seqs, C, width-1], or NULL to drop it; may be
 *                    conv_state_in itself (in-place decode)
 * Uses num_seqs, seq_len, total_tokens, cu_seqlens, H_k, H_v, d_k, d_v and
 * dtype of `shape` (chunk, scale and l2_eps are checked but unused).
 * GDR_ERR_UNSUPPORTED for other widths.  No output may overlap an input or
 * another output, except conv_state_out == conv_state_in.
 */
GDR_API gdr_status gdr_conv_silu(const gdr_shape *shape, int32_t width, const void *x,
                                 const float *weight, const float *bias, const void *conv_state_in,
                                 void *q, void *k, void *v, void *conv_state_out,
                                 hipStream_t stream);

/*
 * gdr_gated_rmsnorm -- the gated RMSNorm that ends the layer after the rule
 * (flashprove issue "P1: Qwen3.8-27B port, tracking": the layer's output is
 * the gated RMSNorm of o).  The pages print no formula; this library reads it
 * per (token, value head) row of o as
 *     out = o / sqrt(mean(o^2) + eps) * weight * SiLU(z)
 * with one weight vector shared by all heads.
 *   o, z, out : dtype [total, H_v, d_v]   (16-byte aligned)
 *   weight    : fp32  [d_v]
 *   eps       : >= 0 and finite, else GDR_ERR_SHAPE
 * out may be o or z itself (every element is read before it is written); no
 * other overlap with an input is allowed.  Uses total_tokens, H_v, d_v and
 * dtype of `shape` (the other fields are checked but unused).
 */
GDR_API gdr_status gdr_gated_rmsnorm(const gdr_shape *shape, const void *o, const void *z,
                                     const float *weight, float eps, void *out,
                                     hipStream_t stream);

/*
 * gdr_chunked_fwd_gated_rmsnorm -- gdr_chunked_fwd followed by
 * gdr_gated_rmsnorm of its output, the rule's output and the norm that ends
 * the layer after it (flashprove issue "P1: Qwen3.8-27B port, tracking"):
 *     out = o / sqrt(mean(o^2) + norm_eps) * norm_weight * SiLU(z)
 * per (token, value head) row, o the rule's output.  Arguments as
 * gdr_chunked_fwd with o replaced by out, plus:
 *   z           : dtype [total, H_v, d_v] (16-byte aligned); must not overlap
 *                 out
 *   norm_weight : fp32 [d_v]
 *   norm_eps    : >= 0 and finite, else GDR_ERR_SHAPE
 * The call runs gdr_chunked_fwd into out (with the given workspace, as
 * gdr_chunked_fwd uses it) and then gdr_gated_rmsnorm in place, two
 * launches on `stream`.  Error behaviour as gdr_chunked_fwd; out and
 * final_state must not overlap z or norm_weight.
 */
GDR_API gdr_status gdr_chunked_fwd_gated_rmsnorm(const gdr_shape *shape, const void *q,
                                                 const void *k, const void *v, const void *a,
                                                 const void *b, const float *A_log,
                                                 const float *dt_bias, const float *initial_state,
                                                 const void *z, const float *norm_weight,
                                                 float norm_eps, void *out, float *final_state,
                                                 void *workspace, size_t workspace_bytes,
                                                 hipStream_t stream);

/*
 * gdr_chunked_fwd_split -- the chunked form with every sequence cut into
 * segments of segment_len tokens that run in parallel: a two-level scan for
 * long sequences with few heads, where one chain of chunks per (sequence,
 * value head) would leave most of the GPU idle (Track L pull request, L2, the
 * cooperative-parallel chunk kernel it lists as not yet built).  The state
 * update is affine in the state, so over a segment S_out = M S_in + S_loc,
 * with M the segment run from S_in = I on v = 0 and S_loc the run from
 * S_in = 0.  The library computes every segment's M and S_loc with two
 * chunked launches, the entry states S_in(p+1) = M_p S_in(p) + S_loc,p in a
 * short sequential pass (fp32), and the outputs with a third chunked launch
 * from those entry states: about three times the arithmetic of
 * gdr_chunked_fwd in exchange for segments-per-sequence times the parallelism.
 * M is d_k x d_k: it comes from the same kernels run with d_k-wide values,
 * so d_v may differ from d_k when both widths have a chunked kernel.
 * Results agree with gdr_chunked_fwd up to float reassociation.
 *   segment_len : a positive multiple of chunk, else GDR_ERR_SHAPE.  Dense
 *                 batches: it must divide seq_len (GDR_ERR_SHAPE), and
 *                 segment_len == seq_len runs gdr_chunked_fwd.  Packed
 *                 batches (cu_seqlens): any lengths; a sequence of L tokens
 *                 has max(1, ceil(L / segment_len)) segments, the last one
 *                 partial, and the segment map is formed on the device from
 *                 cu_seqlens (nothing is copied to the host); a batch of at
 *                 most segment_len tokens in all runs gdr_chunked_fwd
 *   workspace   : device scratch of at least the bytes gdr_chunked_split_workspace
 *                 reports (256-byte aligned; may be NULL when that is 0); it
 *                 may overlap no other argument; contents are not kept.  It
 *                 holds total / segment_len + num_seqs segment states for a
 *                 packed batch, num_seqs * seq_len / segment_len for a dense one
 * A shape whose (d_k, d_v) or (d_k, d_k) problem has no chunked kernel
 * returns GDR_ERR_UNSUPPORTED.  Other arguments as gdr_chunked_fwd
 * (final_state may be initial_state).  Several kernels are launched; a
 * launch failure after the first leaves o and final_state unspecified.
 */
GDR_API gdr_status gdr_chunked_fwd_split(const gdr_shape *shape, int32_t segment_len,
                                         const void *q, const void *k, const void *v,
                                         const void *a, const void *b, const float *A_log,
                                         const float *dt_bias, const float *initial_state,
                                         void *o, float *final_state, void *workspace,
                                         size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace gdr_chunked_fwd_split needs for `shape` and segment_len
 * (0 when there is a single segment); the same shape errors as that call. */
GDR_API gdr_status gdr_chunked_split_workspace(const gdr_shape *shape, int32_t segment_len,
                                               size_t *bytes);

/*
 * gdr_ssd_recurrent_fwd / gdr_ssd_chunked_fwd -- the Mamba-2 SSD recurrence
 * (selective SSM) on the same two forms as the rule: a sequential scan for
 * decode and the chunked scan for prefill.  The Track L pull request ("What
 * landed", L4 and L4.1) names the op's inputs x, A, B, C and delta, an
 * optional gate and an optional initial state, and a carried state for
 * streaming decode, but prints no formula; this library takes the plain
 * reading, per (sequence, head h) with an fp32 state h_t of shape [N, P]:
 *     h_t <- exp(delta_t A_h) h_{t-1} + B_t (delta_t x_t)^T
 *     y_t <- h_t^T C_t,      then y_t <- y_t * SiLU(z_t) when z is given
 * i.e. the rule with a scalar decay and no erase term: no normalisation, no
 * 1/sqrt scale, C in the place of q, B of k, x of v, g_t = delta_t A_h and
 * beta_t = delta_t.  delta and A are used as given (delta > 0, A < 0 for a
 * decaying state: no softplus, no exp).  Heads are grouped as in the rule:
 * head h reads group h / (H / G) of B and C.
 *   shape      : H_k = G groups, H_v = H heads, d_k = N (state size),
 *                d_v = P (head size); scale and l2_eps are checked but unused
 *   x, z, y    : dtype [total, H, P]   (16-byte aligned; z may be NULL)
 *   delta      : dtype [total, H]
 *   A          : fp32  [H]
 *   B, C       : dtype [total, G, N]   (16-byte aligned)
 *   states     : fp32  [num_seqs, H, N, P]   (the page's h[P, N], stored
 *                transposed so that a state row is one N index)
 * initial_state may be NULL (zero state); final_state may be NULL (dropped)
 * or initial_state itself.  The chunked form needs chunk 16, 32 or 64 and
 * runs on the matrix cores for bf16 with N = 128, P = 64 or 128 and
 * chunk 32 (gdr_chunked_path tells which, as for the rule), else on the
 * vector ALUs in fp32 (fp32 inputs always take the vector ALUs here).  The gate is a second launch over y.
 */
GDR_API gdr_status gdr_ssd_recurrent_fwd(const gdr_shape *shape, const void *x, const void *delta,
                                         const float *A, const void *B, const void *C,
                                         const float *initial_state, const void *z, void *y,
                                         float *final_state, hipStream_t stream);
GDR_API gdr_status gdr_ssd_chunked_fwd(const gdr_shape *shape, const void *x, const void *delta,
                                       const float *A, const void *B, const void *C,
                                       const float *initial_state, const void *z, void *y,
                                       float *final_state, hipStream_t stream);

/*
 * gdr_ssd_chunked_fwd_split -- the SSD recurrence of gdr_ssd_chunked_fwd in
 * the segmented form of gdr_chunked_fwd_split (Track L pull request, L4 and
 * L4.1 for the op, L2 for the cooperative-parallel chunk kernel it lists as
 * not yet built).  The SSD update h <- exp(delta A) h + B (delta x)^T is
 * affine in the state too, so each segment's S_out = M S_in + S_loc, M the
 * segment run from the identity on x = 0 (a scaled identity here, formed by
 * the same kernels).  Arguments, layouts and errors as gdr_ssd_chunked_fwd;
 * segment_len, the workspace (gdr_ssd_chunked_split_workspace bytes) and the
 * dense / packed rules as gdr_chunked_fwd_split.  The gate z applies to the
 * outputs of the last pass.
 */
GDR_API gdr_status gdr_ssd_chunked_fwd_split(const gdr_shape *shape, int32_t segment_len,
                                             const void *x, const void *delta, const float *A,
                                             const void *B, const void *C,
                                             const float *initial_state, const void *z, void *y,
                                             float *final_state, void *workspace,
                                             size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace gdr_ssd_chunked_fwd_split needs (0 for one segment). */
GDR_API gdr_status gdr_ssd_chunked_split_workspace(const gdr_shape *shape, int32_t segment_len,
                                                   size_t *bytes);

/*
 * gdr_kda_recurrent_fwd / gdr_kda_chunked_fwd -- the rule with one decay per
 * key channel (KDA): the Mamba + KDA pull requests of the PLENA compiler and
 * simulator name a KDA recurrent-state core beside the Mamba-2 one, with an
 * fp32 state, but print no formula.  This library reads it as the rule of
 * gdr_recurrent_fwd with the scalar decay exp(g_t) replaced by a diagonal
 * one on the state's rows, and the gate of the rule applied per channel:
 *     g_t[i] = -exp(A_log[h]) * softplus(a_t[i] + dt_bias[h, i])   (i < d_k)
 *     S <- diag(exp(g_t)) S;  delta <- (v_t - k_t^T S) * beta_t;
 *     S <- S + k_t (outer) delta;  o_t <- q_t^T S
 * with q, k normalised and q scaled as in the rule, beta_t = sigmoid(b_t).
 *   a        : dtype [total, H_v, d_k]   (per-channel raw gate projections)
 *   dt_bias  : fp32  [H_v, d_k]
 * All other arguments, layouts and rules as gdr_recurrent_fwd /
 * gdr_chunked_fwd.  The chunked form takes chunk 16 or 32 (64 returns
 * GDR_ERR_UNSUPPORTED).  For bf16 with d_k = 128 and chunk 32 it runs on the
 * matrix cores, in one of two ways:
 *  - with a workspace (gdr_kda_chunked_workspace bytes, 256-byte aligned,
 *    overlapping no other argument, contents not kept): two launches, first
 *    the state-free part of every chunk of the batch in parallel (gates,
 *    cumulative decays, the channel-weighted Gram matrices, (I + A)^-1 and
 *    the decay-scaled rows, written to the workspace), then the chains of
 *    chunks, which do only the state-dependent products (any d_v);
 *  - with workspace == NULL: one launch that does both per chunk on the
 *    chain (d_v = 64 or 128).
 * Other shapes and fp32 inputs run on the vector ALUs in fp32 and ignore the
 * workspace.  workspace_bytes below the reported size returns GDR_ERR_WORKSPACE.
 */
GDR_API gdr_status gdr_kda_recurrent_fwd(const gdr_shape *shape, const void *q, const void *k,
                                         const void *v, const void *a, const void *b,
                                         const float *A_log, const float *dt_bias,
                                         const float *initial_state, void *o, float *final_state,
                                         hipStream_t stream);
GDR_API gdr_status gdr_kda_chunked_fwd(const gdr_shape *shape, const void *q, const void *k,
                                       const void *v, const void *a, const void *b,
                                       const float *A_log, const float *dt_bias,
                                       const float *initial_state, void *o, float *final_state,
                                       void *workspace, size_t workspace_bytes,
                                       hipStream_t stream);

/* Bytes of workspace gdr_kda_chunked_fwd uses for `shape` (0 when that shape
 * does not run the two-launch form): one 29,696-byte record per (chunk slot,
 * value head), floor(total_tokens / 32) + num_seqs slots.  The same shape
 * errors as gdr_kda_chunked_fwd. */
GDR_API gdr_status gdr_kda_chunked_workspace(const gdr_shape *shape, size_t *bytes);

/*
 * gdr_kda_chunked_fwd_split -- the segmented form of gdr_chunked_fwd_split
 * for the per-channel-decay variant (arguments, layouts and KDA gates as
 * gdr_kda_chunked_fwd, segments, workspace and rules as
 * gdr_chunked_fwd_split).  The state update stays affine in the state, so
 * the same decomposition S_out = M S_in + S_loc holds per segment.  chunk 16
 * or 32; the workspace size is gdr_kda_chunked_split_workspace's.  Where
 * gdr_kda_chunked_fwd takes its two-launch form (bf16, d_k = 128, chunk 32),
 * the three chunked passes share one per-chunk prep over all segments, which
 * the workspace also holds.
 */
GDR_API gdr_status gdr_kda_chunked_fwd_split(const gdr_shape *shape, int32_t segment_len,
                                             const void *q, const void *k, const void *v,
                                             const void *a, const void *b, const float *A_log,
                                             const float *dt_bias, const float *initial_state,
                                             void *o, float *final_state, void *workspace,
                                             size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace gdr_kda_chunked_fwd_split needs for `shape` and
 * segment_len (0 when there is a single segment); the same shape errors as
 * that call. */
GDR_API gdr_status gdr_kda_chunked_split_workspace(const gdr_shape *shape, int32_t segment_len,
                                                   size_t *bytes);

/* Which kernel gdr_chunked_fwd runs for `shape`: GDR_PATH_VECTOR_F32 (fp32
 * on the vector ALUs), GDR_PATH_MATRIX_BF16 (matrix cores, bf16 operands,
 * fp32 accumulation and state), GDR_PATH_MATRIX_F32 (fp32 inputs with
 * d_k = 64 or 128, d_v a multiple of 16 and chunk 32: matrix cores with
 * fp32 operands, products and state), or the negated gdr_status that
 * gdr_chunked_fwd would return for this shape (pointers are not checked). */
#define GDR_PATH_VECTOR_F32 0
#define GDR_PATH_MATRIX_BF16 1
#define GDR_PATH_MATRIX_F32 2
GDR_API int gdr_chunked_path(const gdr_shape *shape);

/* Human-readable name of a status code (static storage, never NULL). */
GDR_API const char *gdr_status_string(gdr_status status);

/* GDR_ABI_VERSION of the loaded library. */
GDR_API int gdr_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H */
