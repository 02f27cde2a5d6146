/*
 * gdn.h -- C ABI of the MI355X (gfx950) Gated DeltaNet chunked forward.
 *
 * The operation.  Per value head, with state S (d_k x d_v) and tokens t:
 *     S_t = exp(g_t) (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = S_t^T q_t.
 * It is evaluated chunk by chunk (C tokens per chunk) with the gated UT/WY
 * transform T = (I+S)^-1 and the affine inter-chunk step
 *     h' = (exp(g_last) I - k_g^T w) h + k_g^T u = A h + B
 * ("Shard the GatedDeltaNet sequence under ici_context_parallelism", PR
 * description; "GatedDeltaNet does not support ici_context_parallelism",
 * section "The recurrence is affine, so it can be parallelized"), with T
 * formed by the blockwise doubling ladder X - X S_l X ("Fuse the Gated Delta
 * Net inter-chunk scan into a Pallas TPU kernel", section "Changes").  Long
 * sequences are split into chunk-groups, each folded into one (A, B) pair,
 * composed by (A2,B2) o (A1,B1) = (A2 A1, A2 B1 + B2), prefixed exclusively
 * and replayed from the incoming state (issue page, same section; PR page,
 * code-review suggestion for the incoming-state routine).
 *
 * Conventions shared by every entry point:
 *  - All tensor arguments are DEVICE pointers owned by the caller; the
 *    library never allocates, frees or synchronises.  Work is enqueued on
 *    the caller's HIP stream (`hip_stream`, a hipStream_t; NULL = the null
 *    stream) and the call returns without waiting.
 *  - Tensors are dense, row-major, with the layouts stated per argument.
 *    Every pointer must be 16-byte aligned.
 *  - Errors are returned, never aborted on.  Arguments are checked before
 *    anything is launched; on any status other than GDN_OK returned by the
 *    argument checks no output has been touched.  GDN_ERR_HIP means a
 *    launch failed after earlier launches of the same call were queued.
 *  - Calls on different streams do not interact; two calls that share an
 *    output or workspace buffer must be ordered by the caller.
 *  - Supported sizes: d_k = d_v = 128; chunk 64 or 128 for bf16 inputs,
 *    chunk 64 for fp32 inputs; any T >= 0.  A partial last chunk (T not a
 *    multiple of chunk) is padded with identity steps (k = v = 0, g = 0,
 *    beta = 0), which leave the state and the real tokens' outputs exactly
 *    as the unpadded rule gives them; nothing past T is read or written.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDN_OK = 0,
  GDN_ERR_NULL = -1,      /* a required pointer is NULL                         */
  GDN_ERR_SHAPE = -2,     /* unsupported or inconsistent sizes                  */
  GDN_ERR_DTYPE = -3,     /* unsupported dtype code                             */
  GDN_ERR_ALIGN = -4,     /* a pointer is not 16-byte aligned                   */
  GDN_ERR_WORKSPACE = -5, /* workspace smaller than gdn_workspace_size()        */
  GDN_ERR_HIP = -6        /* a kernel launch failed                             */
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

/* Problem description.
 *   B        batch
 *   T        tokens per sequence; N = ceil(T / chunk) chunks
 *   H_qk     query/key heads; H_v value heads, H_v % H_qk == 0.  Value head
 *            h reads query/key head h / (H_v / H_qk) (contiguous groups).
 *   d_k, d_v head dims (128, 128)
 *   chunk    tokens per chunk C (64 or 128)
 *   n_groups 0 or 1: one sequential walk over all N chunks per head.
 *            > 1: split the N chunks of each head into n_groups equal
 *            chunk-groups (n_groups must divide N): fold each group into
 *            one (A, B) pair, exclusive prefix, replay every group from its
 *            incoming state.  Same result up to rounding.
 *   dtype    gdn_dtype of q, k, v
 *   o_dtype  gdn_dtype of o                                                  */
typedef struct {
  int32_t B, T, H_qk, H_v, d_k, d_v, chunk, n_groups;
  int32_t dtype, o_dtype;
} gdn_shape;

/* Human-readable name of a status code (static string).  (A library
 * convention: the pages define no error handling.) */
const char *gdn_status_str(gdn_status s);

/* Host-only check of a problem description; launches nothing.  The
 * supported sizes are those above; the head dimension 128 and chunks of 64
 * and 128 are the ones the pages' runs use ("Fuse the Gated Delta Net
 * inter-chunk scan into a Pallas TPU kernel", section "Performance" and the
 * discussion thread). */
gdn_status gdn_validate(const gdn_shape *shape);

/* Bytes of device workspace gdn_chunk_fwd / gdn_chunk_fold need for `shape`
 * (a library convention; the pages define no workspace)
 * (written to *bytes).  The workspace holds per-chunk intermediates (decay
 * cumsums, W, U, chunk-start states, corrected values per value head; K^T
 * per query/key head) and, with groups, the (A, B) pairs and incoming
 * states.  It carries nothing between calls. */
gdn_status gdn_workspace_size(const gdn_shape *shape, size_t *bytes);

/* The whole chunked forward: o and the final state h_T of the per-token rule
 * above from the initial state h0, evaluated chunk by chunk (the scan that
 * takes an initial state and returns the outputs and the final state: "Fuse
 * the Gated Delta Net inter-chunk scan into a Pallas TPU kernel", sections
 * "Changes" and "Tests"; the inter-chunk affine step: "Shard the
 * GatedDeltaNet sequence under ici_context_parallelism", PR description;
 * with n_groups > 1 the two-pass composition of "GatedDeltaNet does not
 * support ici_context_parallelism", section "The recurrence is affine, so it
 * can be parallelized").
 *   q, k  [B, T, H_qk, d_k]  dtype          v [B, T, H_v, d_v] dtype
 *   g     [B, T, H_v] fp32 per-token log decay (g <= 0 expected, not required)
 *   beta  [B, T, H_v] fp32
 *   h0    [B, H_v, d_k, d_v] fp32 initial state, NULL = zero
 *   o     [B, T, H_v, d_v] o_dtype           (written)
 *   h_T   [B, H_v, d_k, d_v] fp32 final state, NULL = not wanted (written)
 *   ws    device workspace of at least gdn_workspace_size() bytes
 * No scale is applied to q; a caller folds any scale into q. */
gdn_status gdn_chunk_fwd(const gdn_shape *shape, const void *q, const void *k, const void *v,
                         const float *g, const float *beta, const float *h0, void *o,
                         float *h_T, void *ws, size_t ws_bytes, void *hip_stream);

/* gdn_chunk_fwd that also writes the affine map of the whole sequence, in
 * the same walk (the walk carries the augmented state [A | h] from [I | h0]):
 *   A [B, H_v, d_k, d_k] fp32  = the product over the tokens (latest on the
 *        left) of exp(g_t)(I - beta_t k_t k_t^T), so that h_T = A h0 + B with
 *        B the state reached from a zero state (h_T itself when h0 = NULL).
 * The optional third output of the scan ("Fuse the Gated Delta Net
 * inter-chunk scan into a Pallas TPU kernel", discussion thread, on
 * returning A beside the outputs and the final state) with which a sequence
 * shard yields its pair for the composition of "Shard the GatedDeltaNet
 * sequence under ici_context_parallelism" (PR description) without a
 * separate pass.  shape->n_groups must be 0 or 1 (GDN_ERR_SHAPE otherwise);
 * A must not be NULL.  Other arguments, checks and results as gdn_chunk_fwd
 * (o and h_T are those of gdn_chunk_fwd, bit for bit). */
gdn_status gdn_chunk_fwd_affine(const gdn_shape *shape, const void *q, const void *k,
                                const void *v, const float *g, const float *beta,
                                const float *h0, void *o, float *h_T, float *A, void *ws,
                                size_t ws_bytes, void *hip_stream);

/* The same computation issued one stage at a time, for timing each kernel
 * (the stages are the steps of the chunked forward cited at gdn_chunk_fwd).
 * `stages` is a mask of GDN_STAGE_* bits; only the selected stages are
 * launched.  The stages communicate through `ws`, so issuing every stage in
 * increasing bit order on one stream with one workspace (one call per bit,
 * or several bits at once) equals one gdn_chunk_fwd call.  Arguments and
 * checks are those of gdn_chunk_fwd.
 *   PREP    intra-chunk transform (decay cumsum, UT inverse, W, U)
 *   FOLD    per-group affine pairs            (n_groups > 1 only)
 *   PREFIX  exclusive prefix over the groups  (n_groups > 1 only; writes h_T,
 *           the composition of every group's pair applied to h0, when WALK
 *           is not among the stages)
 *   WALK    sequential chunk walk: the whole sequence, or every group from
 *           its incoming state (n_groups > 1); writes h_T, the end state of
 *           the walk (of the last group's replay)
 *   OUT     chunk outputs o                                                  */
#define GDN_STAGE_PREP 1
#define GDN_STAGE_FOLD 2
#define GDN_STAGE_PREFIX 4
#define GDN_STAGE_WALK 8
#define GDN_STAGE_OUT 16
#define GDN_STAGE_ALL 31
gdn_status gdn_chunk_fwd_stages(const gdn_shape *shape, int32_t stages, const void *q,
                                const void *k, const void *v, const float *g, const float *beta,
                                const float *h0, void *o, float *h_T, void *ws, size_t ws_bytes,
                                void *hip_stream);

/* gdn_chunk_fwd_stages that also times each launched stage's kernel: the
 * kernel of stage bit b (GDN_STAGE_* == 1 << b, b = 0..4) records its own
 * start into ev_start[b] and its end into ev_stop[b] (hipExtLaunchKernel), so
 * hipEventElapsedTime(ev_start[b], ev_stop[b]) is the kernel's duration with
 * no event packet between kernels.  The events are hipEvent_t handles the
 * caller created (with timing) and owns; ev_start or ev_stop may be null, and
 * so may any entry (that stage is then not timed).  Other arguments, checks
 * and results as gdn_chunk_fwd_stages.  Measurement aid for benchmarks.      */
gdn_status gdn_chunk_fwd_timed(const gdn_shape *shape, int32_t stages, const void *q,
                               const void *k, const void *v, const float *g, const float *beta,
                               const float *h0, void *o, float *h_T, void *ws, size_t ws_bytes,
                               void *hip_stream, void *const *ev_start, void *const *ev_stop);

/* The chunked forward over packed variable-length sequences: the forward of
 * gdn_chunk_fwd (same pages) applied to each sequence with its own initial
 * and final state; the packing itself is this library's.  shape->B
 * sequences are concatenated along one row of shape->T tokens: sequence s
 * holds tokens [cu_seqlens[s], cu_seqlens[s+1]), each with its own initial
 * and final state and no state passing between sequences.  Each sequence is
 * cut into chunks of its own, its last one partial (padded with identity
 * steps as above).  shape->n_groups must be 0 or 1 (one walk per sequence).
 *   cu_seqlens [B + 1] int32 DEVICE array: 0 = cu[0] <= cu[1] <= ... <=
 *              cu[B] = T.  Offsets outside [0, T] are clamped; for offsets
 *              that are not such a partition the results are unspecified,
 *              but nothing outside the tensors and the workspace is touched.
 *   q, k  [1, T, H_qk, d_k]   v, o [1, T, H_v, d_v]   g, beta [1, T, H_v]
 *   h0, h_T [B, H_v, d_k, d_v] fp32 (h0 NULL = zero; h_T NULL = not wanted)
 *   ws    at least gdn_workspace_size_varlen() bytes.
 * Work is planned on the device (no host copy of cu_seqlens is needed); other
 * conventions as gdn_chunk_fwd, except the sequence count: B * H_v may reach
 * 2^26 (the padded-batch entry points keep B * H_v <= 65535). */
gdn_status gdn_workspace_size_varlen(const gdn_shape *shape, size_t *bytes);
gdn_status gdn_chunk_fwd_varlen(const gdn_shape *shape, const int32_t *cu_seqlens, const void *q,
                                const void *k, const void *v, const float *g, const float *beta,
                                const float *h0, void *o, float *h_T, void *ws, size_t ws_bytes,
                                void *hip_stream);

/* Per-group affine pairs of the chunk-group split: each group's map
 * h -> A h + Bm ("GatedDeltaNet does not support ici_context_parallelism",
 * section "The recurrence is affine, so it can be parallelized"; "Shard the
 * GatedDeltaNet sequence under ici_context_parallelism", PR description: one
 * pair per device from a scan over its chunks) (shape->n_groups >= 1
 * groups of equal length; 0 is taken as 1).  For group j of value head h:
 *   A[b,h,j] = product over the group's tokens t (latest on the left) of
 *              exp(g_t)(I - beta_t k_t k_t^T)            [d_k, d_k] fp32
 *   Bm[b,h,j] = the state the group reaches from a zero state  [d_k, d_v] fp32
 * so that the group maps an incoming state h to A h + Bm.
 *   A  [B, H_v, n_groups, d_k, d_k]     Bm [B, H_v, n_groups, d_k, d_v]
 * q is not read; o is not produced. */
gdn_status gdn_chunk_fold(const gdn_shape *shape, const void *k, const void *v, const float *g,
                          const float *beta, float *A, float *Bm, void *ws, size_t ws_bytes,
                          void *hip_stream);

/* Exclusive prefix of affine pairs applied to an initial state, per
 * (batch*head) row bh (the incoming-state routine of the code-review
 * suggestion on "Shard the GatedDeltaNet sequence under
 * ici_context_parallelism": the state entering each device and the final
 * state; composition law (A2,B2) o (A1,B1) = (A2 A1, A2 B1 + B2) of
 * "GatedDeltaNet does not support ici_context_parallelism", section "The
 * recurrence is affine, so it can be parallelized"):
 *   h_in[bh,0] = h_init[bh];  h_in[bh,j+1] = A[bh,j] h_in[bh,j] + Bm[bh,j];
 *   h_final[bh] = A[bh,n-1] h_in[bh,n-1] + Bm[bh,n-1].
 *   A [batch_heads, n, d_k, d_k] fp32, Bm [batch_heads, n, d_k, d_v] fp32,
 *   h_init [batch_heads, d_k, d_v] fp32 or NULL (= zero),
 *   h_in [batch_heads, n, d_k, d_v] fp32 or NULL, h_final [batch_heads, d_k, d_v]
 *   fp32 or NULL (at least one of them non-NULL).
 * flags bit 0 (GDN_PREFIX_SPLIT_BF16): form the products from hi/lo bf16
 * halves on the bf16 matrix cores (about 1e-5 relative) instead of fp32
 * matrix-core products.
 * With h_in given, n having a divisor s >= 3 near sqrt(n), and the blocked
 * prefix expected to be faster for this (batch_heads, n) (a cost model of
 * both forms' measured step latency and traffic: long chains over few rows),
 * the prefix is blocked (depth 2 s + n / s sequential steps instead of n, the
 * log-depth composition of the issue page, section "Status", and of the
 * associative scan over gathered pairs in the code-review suggestion on the
 * PR page, in two levels): the pairs of each block of s are composed into one
 * pair, the sequential prefix runs over the blocks' pairs, and every block is
 * replayed from its incoming state; h_in holds the intermediates.  The
 * results agree with the sequential prefix to rounding.  flags bit 1
 * (GDN_PREFIX_SEQUENTIAL) forces the one-pair-at-a-time prefix, bit 2
 * (GDN_PREFIX_BLOCKED) the blocked one wherever such an s exists (both bits:
 * GDN_ERR_SHAPE). */
#define GDN_PREFIX_SPLIT_BF16 1
#define GDN_PREFIX_SEQUENTIAL 2
#define GDN_PREFIX_BLOCKED 4
gdn_status gdn_compose_prefix(int32_t batch_heads, int32_t n, int32_t d_k, int32_t d_v,
                              const float *A, const float *Bm, const float *h_init,
                              float *h_in, float *h_final, int32_t flags, void *hip_stream);

/* The intra-chunk transform alone (decay cumsum, gated strict-lower
 * beta K K^T, UT inversion by the doubling ladder, WY formation), for every
 * chunk of every value head ("Fuse the Gated Delta Net inter-chunk scan into
 * a Pallas TPU kernel", section "Changes": the triangular inverse by the
 * blockwise doubling ladder; the pages leave w, u and S undefined, and the
 * forms below are the ones under which the affine step of the PR page equals
 * the per-token rule).  N = ceil(T / chunk); the rows of a partial
 * last chunk past T are its identity padding (G repeats the last real
 * cumsum, T has unit rows, W and U zero rows).
 *   G  [B, H_v, N, C] fp32     G[r] = sum_{s<=r} g_s within the chunk
 *   Tm [B, H_v, N, C, C] fp32  (I+S)^-1, S_ri = beta_r e^{G_r-G_i} k_r.k_i (i<r);
 *                              NULL = not wanted
 *   W  [B, H_v, N, C, d_k] fp32   W = T diag(beta e^G) K
 *   U  [B, H_v, N, C, d_v] fp32   U = T diag(beta) V
 * shape->n_groups and o_dtype are ignored. */
gdn_status gdn_chunk_transform(const gdn_shape *shape, const void *k, const void *v,
                               const float *g, const float *beta, float *G, float *Tm, float *W,
                               float *U, void *hip_stream);

/* The chunked backward's state cotangents: the scan's backward walks the
 * chunks in reverse ("Fuse the Gated Delta Net inter-chunk scan into a
 * Pallas TPU kernel", section "Changes"), the cotangent of chunk n's
 * incoming state being
 *     dh_n = exp(G_last) dh_{n+1} - W^T (K_g dh_{n+1}) + ddh_n,   dh_N = dh_T,
 * with W, K_g the forward's chunk quantities (gdn_chunk_transform) and
 * ddh_n = (diag(e^G) Q - P W)^T dO_n the part that reaches the state through
 * the chunk's own outputs (P = (Q K^T) o Gamma o [i <= r]).  These are the
 * first stage of the gradients of gdn_chunk_fwd; they depend on q, k, g,
 * beta and the cotangents only (not on v or h0).
 *   q, k   [B, T, H_qk, d_k] dtype       g, beta [B, T, H_v] fp32
 *   dO     [B, T, H_v, d_v] fp32          cotangent of o
 *   dh_T   [B, H_v, d_k, d_v] fp32        cotangent of h_T, NULL = zero
 *   dh_chunks [B, H_v, N, d_k, d_v] fp32  dh_n for every chunk n, or NULL
 *   dh0    [B, H_v, d_k, d_v] fp32        cotangent of h0 (= dh_0), or NULL
 *   (at least one of dh_chunks and dh0 non-NULL)
 *   ws     at least gdn_workspace_size_bwd() bytes.
 * shape->n_groups must be 0 or 1 and shape->o_dtype is ignored; other
 * conventions as gdn_chunk_fwd. */
gdn_status gdn_workspace_size_bwd(const gdn_shape *shape, size_t *bytes);
gdn_status gdn_chunk_bwd_state(const gdn_shape *shape, const void *q, const void *k, const float *g,
                               const float *beta, const float *dO, const float *dh_T,
                               float *dh_chunks, float *dh0, void *ws, size_t ws_bytes,
                               void *hip_stream);

/* The chunked backward's gradients: of L = sum_t <o_t, dO_t> + <h_T, dh_T>
 * with respect to q, k, v, g, beta and h0, for the forward of gdn_chunk_fwd
 * ("Fuse the Gated Delta Net inter-chunk scan into a Pallas TPU kernel",
 * section "Changes": the scan's backward walks the chunks in reverse, the
 * triangular inverse has the analytic backward dS = -(T^T dT T^T) on the
 * strict lower triangle; section "Tests": every gradient, with a non-zero
 * initial state and a final-state cotangent).  Four passes on the stream:
 * the intra-chunk transform (G, T, W, U in fp32); the forward's incoming
 * state of every chunk; the reverse walk's state cotangents (as
 * gdn_chunk_bwd_state); then, per chunk and value head, the adjoint of each
 * line of the chunk's forward in reverse order.
 *   q, k [B, T, H_qk, d_k], v [B, T, H_v, d_v] in shape->dtype; g, beta
 *   [B, T, H_v] fp32; h0 [B, H_v, d_k, d_v] fp32 or NULL (zero); dO
 *   [B, T, H_v, d_v] fp32; dh_T [B, H_v, d_k, d_v] fp32 or NULL (zero).
 *   Outputs (all fp32, caller-allocated, 16-byte aligned): dq, dk
 *   [B, T, H_qk, d_k] (the sum over the value heads that read each key head),
 *   dv [B, T, H_v, d_v], dg, dbeta [B, T, H_v], dh0 [B, H_v, d_k, d_v] or
 *   NULL.
 *   ws: gdn_workspace_size_bwd_grads(shape) bytes (about 5 d_k x d_v + 2
 *   chunk x (chunk + d_v) floats per chunk and value head, plus a fixed
 *   scratch of at most 256 slots of 5 chunk x d_v + 7 chunk^2 floats).
 * shape->n_groups must be 0 or 1 (GDN_ERR_SHAPE otherwise); o_dtype is not
 * used.  Products follow the forward's precision policy (fp32 inputs: fp32
 * matrix-core products; bf16 inputs: hi/lo split bf16 products).  T = 0:
 * dh0 = dh_T (or zero); nothing else is written.  Other errors as for
 * gdn_chunk_fwd. */
gdn_status gdn_workspace_size_bwd_grads(const gdn_shape *shape, size_t *bytes);
gdn_status gdn_chunk_bwd(const gdn_shape *shape, const void *q, const void *k, const void *v,
                         const float *g, const float *beta, const float *h0, const float *dO,
                         const float *dh_T, float *dq, float *dk, float *dv, float *dg,
                         float *dbeta, float *dh0, void *ws, size_t ws_bytes, void *hip_stream);

/* gdn_chunk_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Arguments, checks and results are those of gdn_chunk_fwd, without the
 * workspace: the library's own static device array of
 * GDN_NOALLOC_SCRATCH_BYTES bytes serves as the workspace.  Every GPU the
 * library runs on holds that array until the process ends; its address is
 * looked up on the first call on each device (the current device, which must
 * be the stream's).  Nothing is allocated, freed or cleared.
 *   Returns GDN_ERR_WORKSPACE, launching nothing, when the problem needs more
 *   workspace than the array holds (gdn_workspace_size(shape) >
 *   GDN_NOALLOC_SCRATCH_BYTES; e.g. 32 value heads x 4096 tokens at chunk 128
 *   fit).
 * All calls on one GPU share its array: two calls whose work may overlap on
 * that GPU (different streams, or a graph replayed on one stream while
 * another call runs on a second) race and give undefined results; calls
 * ordered on one stream do not interact. */
#define GDN_NOALLOC_SCRATCH_BYTES (256u << 20)
gdn_status gdn_chunk_fwd_noalloc(const gdn_shape *shape, const void *q, const void *k,
                                 const void *v, const float *g, const float *beta,
                                 const float *h0, void *o, float *h_T, void *hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* GDN_H */
