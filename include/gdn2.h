/*
 * gdn2.h -- C ABI of libgdn2.so, the MI355X (gfx950) Gated DeltaNet-2 chunkwise operator.
 *
 * The operator (iplexlaw.co.kr blog on Gated DeltaNet-2, section "Independent
 * control on two axes"; the paper abstract, OpenAlex record of arXiv:2605.22791):
 * per (batch, head) a state S of dk x dv values (key axis = rows) is carried
 * through the tokens.  For token t
 *
 *     e = b_t * k_t              erase gate on the key channels
 *     z = w_t * v_t              write gate on the value channels
 *     Sbar = diag(exp(log_alpha_t)) S        channel-wise decay on the key axis
 *     S = Sbar + k_t (z - Sbar^T e)^T        read through e, write along k
 *     o_t = S^T q_t                          the query reads the updated state
 *
 * The library evaluates this rule in the chunkwise WY form with 64-token
 * chunks (same blog, section "Token path and parallel training": cumulative
 * channel decay absorbed into asymmetric erase factors, a triangular solve and
 * dense matrix products per chunk, fp32 decay, state and solve).  The backward
 * pass is the gate-aware adjoint (gradients flow through the gated e and z).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers owned by the caller, contiguous,
 *   row-major and 16-byte aligned.  The library allocates nothing, frees
 *   nothing and keeps no global mutable state; calls on different streams may
 *   run concurrently.
 * - Token tensors are [B, T, H, D]: q, k, log_alpha, b and the key-side
 *   gradients use D = dk; v, w, o and the value-side gradients use D = dv.
 *   A gate flagged in shape->gate_scalar, and its gradient, is [B, T, H] instead.
 *   States are [B, H, dk, dv] fp32 (key channel = row).
 * - q, k, v have dtype shape->qkv_dtype (fp32 or bf16).  S0, dO, dS_final and
 *   every output are fp32.  log_alpha, b, w are fp32 values or bf16 logits as
 *   shape->gate_dtype says (see gdn2_gate_dtype).
 * - With fp32 gates, log_alpha is the natural log of the per-channel decay
 *   (alpha = exp), and b and w are gate VALUES (after any sigmoid), not clamped.
 *   Gradients are taken with respect to exactly the inputs given (values or
 *   logits).  q is not scaled.
 * - Any T >= 1 is accepted; a ragged tail chunk is padded internally with
 *   identity tokens (k = 0, log_alpha = 0) that leave the state unchanged.
 * - Supported sizes: B, H >= 1, T >= 1, chunk == 64, dk and dv in {32, 64, 128},
 *   B*T*H*max(dk,dv) < 2^31 and H*max(dk,dv) < 2^24 (64 tokens of one fp32
 *   tensor span less than 4 GiB); GDN2_ERR_UNSUPPORTED otherwise.
 * - Decay range: any log_alpha <= 0 is accepted, -inf (alpha = 0) included; the
 *   blog puts no floor under alpha.  The chunk form factors the decay between two
 *   tokens of a chunk as exp(G_i) exp(-G_j); on a chunk in which some key channel
 *   decays by more than about exp(-64) that factor would leave fp32 range, so such
 *   chunks are found on the device and their intra-chunk products are recomputed
 *   with the pairwise decay exp(G_i - G_j) itself (a second, exact pass over the
 *   flagged chunks only; results stay within the stated tolerances).  A per-token
 *   log_alpha below -30 is computed as -30: the difference, a factor below 1e-13 on
 *   what the state held, is beneath fp32 resolution.  NaN inputs propagate.
 * - Execution is asynchronous on `stream` (a hipStream_t; NULL = the default
 *   stream).  Results are valid once the stream has reached the call.
 * - Errors: arguments are checked on the host before any launch; on failure
 *   nothing is launched and nothing is written.  GDN2_ERR_HIP reports a launch
 *   failure (hipGetLastError after the launch).  No C++ exception crosses the ABI.
 */
#ifndef GDN2_H
#define GDN2_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN2_OK = 0,
    GDN2_ERR_INVALID_ARG = 1,   /* null required pointer, bad size, misaligned pointer */
    GDN2_ERR_UNSUPPORTED = 2,   /* valid request outside the supported sizes/dtypes */
    GDN2_ERR_WORKSPACE = 3,     /* workspace smaller than *_workspace_size() or NULL */
    GDN2_ERR_HIP = 4,           /* the HIP runtime reported an error at launch */
    GDN2_ERR_SCRATCH = 5        /* gdn2_chunk_fwd_noalloc: larger than its static scratch */
} gdn2_status;

typedef enum { GDN2_F32 = 0, GDN2_BF16 = 1 } gdn2_dtype;

/* How the gates log_alpha, b and w are given.
 *   GDN2_GATES_F32: fp32 values (log_alpha is the natural-log decay, b and w the gate values).
 *   GDN2_GATES_BF16_LOGITS: bf16 pre-activation logits x_a, x_b, x_w; the kernels form
 *     b = sigmoid(x_b), w = sigmoid(x_w) and log_alpha = log(sigmoid(x_a)) in fp32 (the gates
 *     are sigmoid outputs of linear projections: blog on Gated DeltaNet-2, section
 *     "Independent control on two axes"), and the gradients dlog_alpha, db, dw are taken
 *     w.r.t. the logits.  Requires qkv_dtype == GDN2_BF16.  Halves the gate bytes. */
typedef enum { GDN2_GATES_F32 = 0, GDN2_GATES_BF16_LOGITS = 1 } gdn2_gate_dtype;

/* Per-token gates (bits of gdn2_shape.gate_scalar).  A gate whose bit is set is given as
 * ONE fp32 value per (batch, token, head), a [B, T, H] tensor, that applies to every
 * channel of its axis; its gradient output is then [B, T, H] too (the sum over the
 * channels of the per-channel gradient).  This covers the special cases of the rule:
 * erase and write gate both one beta per token (KDA), also a scalar decay (Gated
 * DeltaNet) (blog on Gated DeltaNet-2, section "Independent control on two axes"), and
 * the gate ablations that use the channel mean of the erase or the write gate (same
 * blog, section "Ablations and training throughput").  The per-token tensors need only
 * 4-byte alignment.  Requires qkv_dtype == GDN2_BF16 and gate_dtype == GDN2_GATES_F32. */
typedef enum {
    GDN2_SCALAR_DECAY = 1,   /* log_alpha and dlog_alpha are [B, T, H] */
    GDN2_SCALAR_ERASE = 2,   /* b and db are [B, T, H] */
    GDN2_SCALAR_WRITE = 4    /* w and dw are [B, T, H] */
} gdn2_gate_scalar;

typedef struct {
    int B, T, H;      /* batch, tokens, heads */
    int dk, dv;       /* key and value head dimensions */
    int chunk;        /* must be 64 */
    int qkv_dtype;    /* a gdn2_dtype: dtype of q, k and v */
    int gate_dtype;   /* a gdn2_gate_dtype: how log_alpha, b and w are given */
    int gate_scalar;  /* OR of gdn2_gate_scalar bits; 0 = every gate per channel */
} gdn2_shape;

/* Bytes of device workspace gdn2_chunk_fwd needs; (size_t)-1 if the shape is invalid.
 * The forward first writes forward-only chunk records (the key-side operands of every
 * chunk, about 2.3 KB per token-head at dk = 128, and one strong-decay flag per chunk)
 * and then sweeps over them; the workspace holds those records.  With bf16 q/k/v,
 * dk in {64, 128}, dv a multiple of 64, so few heads that the sweep would keep at most
 * one CU in four busy and 64 chunks or more, the sequence is also split into segments
 * swept side by side; every segment's state map and start state (dk * (2 dv + dk) fp32
 * per batch, head and segment) follow the records. */
size_t gdn2_chunk_fwd_workspace_size(const gdn2_shape *shape);

/* Forward pass: o [B,T,H,dv] and the final state S_final [B,H,dk,dv].
 * S0 == NULL means a zero start state; S_final == NULL means it is not wanted.
 * The workspace must hold gdn2_chunk_fwd_workspace_size() bytes (GDN2_ERR_WORKSPACE if
 * not, or if NULL) and is overwritten. */
int gdn2_chunk_fwd(const gdn2_shape *shape,
                   const void *q, const void *k, const void *v,
                   const void *log_alpha, const void *b, const void *w,
                   const float *S0,
                   float *o, float *S_final,
                   void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of device workspace gdn2_chunk_bwd needs: two fp32 states per chunk per
 * (batch, head) and the per-chunk adjoint factors, i.e.
 * 2 * gdn2_chunk_states_bytes() + gdn2_chunk_factors_bytes(); (size_t)-1 if invalid.
 * On the shapes where gdn2_chunk_fwd splits the sequence into segments, the backward's
 * state sweep is split the same way, and the same per-segment maps and start states
 * (dk*(2dv+dk) fp32 per batch, head and segment) follow the factors. */
size_t gdn2_chunk_bwd_workspace_size(const gdn2_shape *shape);

/* Gate-aware backward pass of loss = sum(dO * o) + sum(dS_final * S_final):
 * writes dq, dk, dlog_alpha, db [B,T,H,dk], dv, dw [B,T,H,dv] and, unless
 * dS0 == NULL, dS0 [B,H,dk,dv].  S0 == NULL and dS_final == NULL mean zeros.
 * The forward state is recomputed from the inputs; nothing from a previous
 * gdn2_chunk_fwd call is needed.  The workspace (see above) is overwritten. */
int gdn2_chunk_bwd(const gdn2_shape *shape,
                   const void *q, const void *k, const void *v,
                   const void *log_alpha, const void *b, const void *w,
                   const float *S0,
                   const float *dO, const float *dS_final,
                   float *dq, float *dk, float *dv,
                   float *dlog_alpha, float *db, float *dw,
                   float *dS0,
                   void *workspace, size_t workspace_bytes, void *stream);

/* ---- staged form (training): each call below is one or two kernel launches ----
 *
 * gdn2_chunk_bwd == gdn2_chunk_bwd_factors + gdn2_chunk_fwd_factored (states only)
 *                   + gdn2_chunk_bwd_reverse + gdn2_chunk_bwd_grads.
 * A training step runs gdn2_chunk_bwd_factors, then gdn2_chunk_fwd_factored (o and the
 * chunk states), and after the loss gdn2_chunk_bwd_reverse and gdn2_chunk_bwd_grads,
 * all on the one factor buffer; the key-side work of every chunk is done once.
 * `states` and `dstates` are [B, H, ceil(T/64), dk, dv] fp32 device buffers of
 * gdn2_chunk_states_bytes() bytes each: states[c] is the state BEFORE chunk c
 * (tokens 64c ..), dstates[c] the loss gradient w.r.t. the state AFTER chunk c. */

/* Bytes of one chunk-state buffer; (size_t)-1 if the shape is invalid. */
size_t gdn2_chunk_states_bytes(const gdn2_shape *shape);

/* Bytes of the factor buffer of gdn2_chunk_bwd_factors: per (batch, head, chunk) the
 * adjoint factors, (dk*dk + 64*dk)*4 bytes, the chunk's key-side operands,
 * 788*dk + 49152 bytes (rounded up to 256), and a strong-decay flag (4 bytes; the flags
 * rounded up to 256); (size_t)-1 if the shape is invalid. */
size_t gdn2_chunk_factors_bytes(const gdn2_shape *shape);

/* Per-chunk adjoint factors of the reverse sweep.  Unrolling the backward of one
 * chunk of the chunkwise WY form (blog on Gated DeltaNet-2, section "Token path and
 * parallel training") gives for the gradient of the chunk's start state
 *     dS = R dS' + Q2^T dO,  R = (I - W^T Kt) diag(gamma),  Q2 = Qt - P W,  W = T Et,
 * with dS' the gradient of its end state; R and Q2 depend on q, k, log_alpha and b
 * only.  Writes R and Q2^T of every (batch, head, chunk) into `factors`
 * (gdn2_chunk_factors_bytes() bytes, device memory owned by the caller, opaque
 * layout of split-bf16 MFMA tiles), followed by the key-side operands of every chunk
 * that the token gradients need as well (the decay-absorbed key and erase-key rows,
 * T = (I + A)^-1, P, the decay scan's per-block offsets) and each chunk's strong-decay
 * flag, so that they are formed once.  Two launches: every chunk, then the exact pass over flagged chunks.
 * Read by gdn2_chunk_bwd_reverse and gdn2_chunk_bwd_grads. */
int gdn2_chunk_bwd_factors(const gdn2_shape *shape, const void *q, const void *k,
                           const void *log_alpha, const void *b, void *factors, void *stream);

/* Forward sweep from the factor buffer that gdn2_chunk_bwd_factors wrote for the same
 * shape and the same q, k, log_alpha and b (their key-side chunk operands are taken
 * from it; q, k, log_alpha and b are not read again).  Reads v, w and S0 (NULL =
 * zeros); writes o [B,T,H,dv] unless NULL, S_final unless NULL, and the chunk-start
 * states unless NULL; o and states cannot both be NULL.  Results as gdn2_chunk_fwd, plus
 * the state before every chunk.  A training step runs gdn2_chunk_bwd_factors first and uses
 * the one factor buffer for this forward, gdn2_chunk_bwd_reverse and
 * gdn2_chunk_bwd_grads.  shape->gate_dtype and gate_scalar describe w. */
int gdn2_chunk_fwd_factored(const gdn2_shape *shape, const void *factors, const void *v,
                            const void *w, const float *S0, float *o, float *S_final,
                            float *states, void *stream);

/* Reverse sweep of the backward from the factors: writes dstates (required) and
 * dS0 (optional), reading dO and dS_final (NULL = zeros). */
int gdn2_chunk_bwd_reverse(const gdn2_shape *shape, const void *factors,
                           const float *dO, const float *dS_final,
                           float *dstates, float *dS0, void *stream);

/* The training step's two sweeps from one factor buffer of gdn2_chunk_bwd_factors: the
 * forward sweep of gdn2_chunk_fwd_factored (o, S_final, the state before every chunk) and the
 * reverse sweep of gdn2_chunk_bwd_reverse (dS' of every chunk, dS0), with the same arguments,
 * layouts and results as those two calls (chunk map and its adjoint: blog on Gated DeltaNet-2,
 * section "Token path and parallel training").  The sweeps are independent; where
 * gdn2_chunk_sweeps_fused() is 1 (bf16 q/k/v, dk 64 or 128, dv a multiple of 64, and few enough
 * heads that the two sweeps' 64-column tiles together need at most one workgroup per CU) they
 * run as one launch, side by side; otherwise one after the other.  o, states and dstates are
 * required; S0, dS_final (NULL = zeros), S_final and dS0 (NULL = not wanted) are optional.
 * Errors as for those two entry points; nothing is launched if an argument check fails. */
int gdn2_chunk_sweeps(const gdn2_shape *shape, const void *factors, const void *v, const void *w,
                      const float *S0, const float *dO, const float *dS_final,
                      float *o, float *S_final, float *states, float *dstates, float *dS0, void *stream);

/* 1 if gdn2_chunk_sweeps runs its two sweeps as one launch for this shape, 0 if as two,
 * -1 if the shape is invalid. */
int gdn2_chunk_sweeps_fused(const gdn2_shape *shape);

/* Token gradients from states, dstates and the factor buffer of
 * gdn2_chunk_bwd_factors (same shape and inputs): dq, dk, dlog_alpha, db [B,T,H,dk],
 * dv, dw [B,T,H,dv].  Two launches: every chunk, then the exact pass over the chunks the
 * factor buffer flags (their gradients are written again). */
int gdn2_chunk_bwd_grads(const gdn2_shape *shape,
                         const void *q, const void *k, const void *v,
                         const void *log_alpha, const void *b, const void *w,
                         const float *dO, const float *states, const float *dstates,
                         const void *factors,
                         float *dq, float *dk, float *dv,
                         float *dlog_alpha, float *db, float *dw, void *stream);

/* ---- recurrent step (decode) ----
 *
 * One token per (batch, head), the per-token rule of the blog on Gated DeltaNet-2,
 * section "Independent control on two axes": decay, read through the erase key
 * e = b*k, write z - r along the raw key with z = w*v, then the query reads the
 * updated state.  shape->T must be 1; q, k, log_alpha, b are [B,1,H,dk], v, w and
 * o are [B,1,H,dv]; S_in and S_out are [B,H,dk,dv] fp32.  S_in == NULL means a zero
 * state.  S_out may be the same buffer as S_in (in-place update); otherwise the two
 * must not overlap.  One kernel launch, no workspace; all buffers are device memory
 * owned by the caller.  Returns GDN2_ERR_INVALID_ARG for T != 1. */
int gdn2_step(const gdn2_shape *shape, const void *q, const void *k, const void *v,
              const void *log_alpha, const void *b, const void *w,
              const float *S_in, float *S_out, float *o, void *stream);

/* ---- output epilogue ----
 *
 * The operator's output of each (batch, token, head) goes through an RMS normalisation,
 * then an output gate of its own (not the write gate), then the output projection
 * (blog on Gated DeltaNet-2, section "Token path and parallel training").  The
 * normalisation runs over the dv value channels of one row with a per-channel weight;
 * the gate is given as values (its activation belongs to its projection); the
 * projection is a plain matrix product left to the caller.  Per row o of
 * o [B,T,H,dv] (shape->B, T, H, dv are used; dk must still be valid):
 *     y = o / sqrt(mean_j o_j^2 + eps) * weight * g
 * o is fp32; g [B,T,H,dv] has dtype g_dtype (GDN2_F32 or GDN2_BF16); weight [dv] fp32,
 * NULL = ones; y has dtype y_dtype (GDN2_F32 or GDN2_BF16, round to nearest even).
 * eps must be finite and >= 0.  One kernel launch, no workspace. */
int gdn2_output_fwd(const gdn2_shape *shape, const float *o, const void *g, int g_dtype,
                    const float *weight, float eps, void *y, int y_dtype, void *stream);

/* Bytes of device workspace gdn2_output_bwd needs when dweight is wanted (a partial
 * dweight row per workgroup, at most 1024 * dv floats); (size_t)-1 if invalid. */
size_t gdn2_output_bwd_workspace_size(const gdn2_shape *shape);

/* Backward of the output epilogue for loss = sum(dy * y): writes dO = dloss/do and
 * dg [B,T,H,dv] fp32 and, unless dweight == NULL, dweight [dv] fp32 (a sum over all
 * rows, added in a fixed order: reproducible bit for bit).  dy is fp32 [B,T,H,dv].
 * dO is the upstream gradient the operator's backward takes.  The workspace is needed
 * (and overwritten) only when dweight != NULL.  One launch, two with dweight. */
int gdn2_output_bwd(const gdn2_shape *shape, const float *o, const void *g, int g_dtype,
                    const float *weight, float eps, const float *dy, float *dO, float *dg,
                    float *dweight, void *workspace, size_t workspace_bytes, void *stream);

/* ---- forward with the output epilogue fused ----
 *
 * The inference forward followed by the output epilogue (blog on Gated DeltaNet-2, section
 * "Token path and parallel training": the operator's output goes through an RMS
 * normalisation and an output gate of its own before the projection), with o never written
 * to device memory:
 *     y = o / sqrt(mean_j o_j^2 + eps) * weight * g      per (b, t, h) row of dv channels,
 * o being what gdn2_chunk_fwd computes.  Inputs and S0, S_final as gdn2_chunk_fwd; g, weight,
 * eps, y, g_dtype, y_dtype as gdn2_output_fwd (g, weight, y 16-byte aligned).
 * - Fused (gdn2_chunk_fwd_output_fused() == 1: bf16 q/k/v, dk 64 or 128, dv 64 or 128, a
 *   shape the forward does not split into segments, and every workgroup of the sweep resident
 *   at once): the launches of gdn2_chunk_fwd (chunk records, their exact pass, the sweep),
 *   with the epilogue in the sweep's output stage; the sweep is a cooperative launch when a
 *   head's value columns span several workgroups.  The runtime can refuse a cooperative launch
 *   while another process on the same GPU holds the device's cooperative-launch resources (seen
 *   once that process had made a cooperative launch of its own); the call then returns
 *   GDN2_ERR_HIP after the records launch, with y and S_final not written.  Shapes with one
 *   workgroup per head launch normally.  The workspace holds the records and flags, then the
 *   exchange area (cleared by the records launch): 64-bit words {row sum of squares of one
 *   wave's columns, chunk + 1} in a ring of two chunk slots per head, and in the last 256 bytes
 *   an int that counts exchange waits that ran out (0 in a correct run; a wait runs out only if
 *   a workgroup of the head never publishes, after about 2^16 reads).
 * - Otherwise gdn2_chunk_fwd into o in the workspace, then gdn2_output_fwd: results equal to
 *   those two calls.
 * The norm's sum over a row is added in a different order from gdn2_output_fwd's, so the two
 * paths agree to rounding, not bit for bit.  Errors as gdn2_chunk_fwd and gdn2_output_fwd. */
size_t gdn2_chunk_fwd_output_workspace_size(const gdn2_shape *shape);
int gdn2_chunk_fwd_output(const gdn2_shape *shape,
                          const void *q, const void *k, const void *v,
                          const void *log_alpha, const void *b, const void *w,
                          const float *S0, const void *g, int g_dtype, const float *weight,
                          float eps, void *y, int y_dtype, float *S_final,
                          void *workspace, size_t workspace_bytes, void *stream);
/* 1 if gdn2_chunk_fwd_output fuses the epilogue for this shape on the current device, else 0. */
int gdn2_chunk_fwd_output_fused(const gdn2_shape *shape);

/* ---- forward without allocation ----
 *
 * For callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  gdn2_chunk_fwd_noalloc computes exactly
 * what gdn2_chunk_fwd computes (same arguments minus the workspace, same kernels), with the
 * chunk records in a static device array inside the library instead of a caller-given
 * workspace; it calls no hipMalloc, hipFree or allocating routine.
 * - Limit: the array holds gdn2_chunk_fwd_noalloc_max_bytes() = 256 MiB on each GPU, from
 *   the first call on that GPU until the process ends.  The batch is processed in groups of
 *   batch elements whose records fit (gdn2_chunk_fwd_workspace_size of the group); a shape
 *   whose single batch element needs more than the array (at dk = 128 about 150 KB per head
 *   and 64 tokens, so H * T up to about 114,000) returns GDN2_ERR_SCRATCH before any launch.
 * - The array is shared by every call on a GPU and keeps the last call's contents (nothing in
 *   it needs clearing: every call writes all it reads).  Calls that overlap on one GPU, on
 *   any streams, race on it and must be serialised by the caller.
 * - The kernels run on the current device (the stream must belong to it); its copy of the
 *   array is looked up once per device, on the first call there.
 * Errors as gdn2_chunk_fwd, plus GDN2_ERR_SCRATCH; GDN2_ERR_HIP if the array's address
 * cannot be obtained. */
int gdn2_chunk_fwd_noalloc(const gdn2_shape *shape,
                           const void *q, const void *k, const void *v,
                           const void *log_alpha, const void *b, const void *w,
                           const float *S0, float *o, float *S_final, void *stream);

/* Bytes of the static scratch array of gdn2_chunk_fwd_noalloc on each GPU. */
size_t gdn2_chunk_fwd_noalloc_max_bytes(void);

/* Static, human-readable description of a gdn2_status value. */
const char *gdn2_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* GDN2_H */
