/*
 * gdpa.h - C ABI of the MI355X (gfx950) Generalized Dot-Product Attention library.
 *
 * GDPA (Kunlun paper summary, section 2.2 on low-level module optimisations,
 * GDPA bullet) recasts the personalised FFN as one fused multi-head attention
 * operator: the tokens of a sample's user history are the queries, and weights
 * derived from that sample's non-sequential context are the keys and values
 * (Telegram review of the paper, layer steps 1 and 2: K and V are made from the
 * context features, and the event sequence, turned into Q, attends to them).
 *
 * For a jagged batch, sample b owns token rows offsets[b] .. offsets[b+1]-1.
 * For every token t of sample b and head h:
 *
 *     s_j      = scale * < Q[t,h,:], K[b,j,h,:] >          j = 0 .. n_kv-1
 *     p        = phi(s)    (row softmax over j, or an elementwise map)
 *     O[t,h,:] = sum_j p_j V[b,j,h,:]
 *
 * With an elementwise phi and scale = 1 this is the per-sample two-layer FFN
 * phi(x K^T) V (SiLU gives the FFN form; ReLU, GELU and the identity are the
 * other common FFN activations).  The pages give no
 * formula for phi, the scale, masking or normalisation; the readings taken are:
 * no mask (a token sees every context row of its own sample and nothing of other
 * samples), softmax over the n_kv context rows, scale chosen by the caller
 * (1/sqrt(d) for softmax and 1 for the elementwise maps are the usual values),
 * d_v = d_qk = d, no bias.
 *
 * Conventions shared by every call:
 *   - All tensor pointers are DEVICE pointers, caller-owned; the library never
 *     allocates or frees them.  Tensors are dense row-major:
 *       Q, O, dO, dQ, residual : [T][H][d]      (token-major, heads inner)
 *       K, V, dK, dV           : [B][n_kv][H][d]
 *       lse                    : [T][H] float32 (natural log)
 *       offsets                : [B+1] int32, offsets[0] = 0, non-decreasing,
 *                                offsets[B] = T, every length <= max_seqlen.
 *     The offsets contents are the caller's contract (checking them on the
 *     device would need a synchronisation); gdpa_check_offsets() checks a host
 *     copy.  Empty samples (length 0) are allowed.
 *   - dtype GDPA_BF16: bf16 tensors, fp32 accumulation, bf16 results rounded to
 *     nearest even.  dtype GDPA_F32: fp32 tensors and fp32 arithmetic.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream) and never synchronises it.  Errors in the arguments are reported
 *     before anything is launched.  A launch failure returns GDPA_ERR_HIP and
 *     stores the hipError_t for gdpa_last_hip_error() (per thread).
 *   - No exceptions cross the ABI.  The calls are safe from several threads.
 *     Two pieces of state live for the whole process: the grouped calls create
 *     three streams and their events per device on first use (kept until the
 *     process ends, guarded by a mutex), and gdpa_bwd_noalloc keeps one scratch
 *     array per device (its address looked up once, guarded by a mutex).
 *     Nothing else is global.
 */
#ifndef GDPA_H
#define GDPA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDPA_OK = 0,
  GDPA_ERR_INVALID_ARGUMENT = 1,  /* null pointer, size out of range, non-finite scale */
  GDPA_ERR_UNSUPPORTED = 2,       /* valid but not implemented: head_dim, dtype, flags */
  GDPA_ERR_WORKSPACE_TOO_SMALL = 3,
  GDPA_ERR_HIP = 4                /* a HIP launch or runtime call failed */
} gdpa_status;

/* Score maps.  SOFTMAX: row softmax over the n_kv context rows.  Elementwise:
 * SILU s / (1 + exp(-s)); RELU max(s, 0) (derivative taken as 0 at s = 0);
 * GELU s Phi(s) with Phi the standard normal CDF (the exact erf form; the bf16
 * kernels evaluate erf with a rational approximation of absolute error
 * <= 1.5e-7); IDENTITY s (GDPA is then the bilinear map (x K^T) V). */
typedef enum {
  GDPA_PHI_SOFTMAX = 0,
  GDPA_PHI_SILU = 1,
  GDPA_PHI_RELU = 2,
  GDPA_PHI_GELU = 3,
  GDPA_PHI_IDENTITY = 4
} gdpa_phi;
typedef enum { GDPA_F32 = 0, GDPA_BF16 = 1 } gdpa_dtype;

/* gdpa_fwd: O = residual + GDPA(...) instead of O = GDPA(...). `residual` may alias `q`. */
#define GDPA_FWD_RESIDUAL 0x1u
/* gdpa_bwd: dQ += result instead of dQ = result.  With this flag `dq` may alias `d_o`. */
#define GDPA_BWD_ACCUM_DQ 0x2u
/* gdpa_bwd: dQ = dO + result, the gradient of O = Q + GDPA(Q) with respect to Q
 * (a residual layer whose queries are its input tokens).  `dq` may alias `d_o`.
 * Not combined with GDPA_BWD_ACCUM_DQ. */
#define GDPA_BWD_RESIDUAL 0x4u

typedef struct {
  int32_t batch;         /* B >= 1 */
  int32_t total_tokens;  /* T = offsets[B] >= 0 */
  int32_t max_seqlen;    /* >= every sample length (host-known bound) */
  int32_t n_kv;          /* context rows per sample, >= 1 */
  int32_t heads;         /* H >= 1 */
  int32_t head_dim;      /* d: 32, 64 or 128 */
  int32_t phi;           /* gdpa_phi */
  float scale;           /* finite; applied to the scores before phi */
  int32_t dtype;         /* gdpa_dtype of Q, K, V, O, residual, dO, dQ, dK, dV */
  uint32_t flags;        /* GDPA_FWD_RESIDUAL, GDPA_BWD_ACCUM_DQ, GDPA_BWD_RESIDUAL */
} gdpa_problem;

/* Bytes of device workspace gdpa_fwd (backward = 0) or gdpa_bwd (backward = 1)
 * needs for this problem; 0 if the problem is invalid.  The workspace is
 * scratch owned by the caller; its contents need no initialisation and are
 * undefined after the call.  Two calls in flight at once need two workspaces. */
size_t gdpa_workspace_bytes(const gdpa_problem* p, int backward);

/* Forward.  q [T,H,d], k, v [B,n,H,d] in; o [T,H,d] out (overwritten).
 * lse [T,H] float32: log-sum-exp of each score row (natural log) - written when
 * non-NULL and phi = softmax, required by gdpa_bwd for softmax; ignored for the elementwise maps.
 * residual [T,H,d]: added to O when GDPA_FWD_RESIDUAL is set (may alias q;
 * must not alias o unless it is the same buffer as q and o is not q). */
gdpa_status gdpa_fwd(const gdpa_problem* p, const int32_t* offsets, const void* q,
                     const void* k, const void* v, const void* residual, void* o, float* lse,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Backward of sum(O * dO).  In: q, k, v, d_o, and for softmax also o and lse
 * from gdpa_fwd (ignored for the elementwise maps, may be NULL).  Out: dq [T,H,d] (overwritten;
 * accumulated with GDPA_BWD_ACCUM_DQ; dO added with GDPA_BWD_RESIDUAL), dk, dv
 * [B,n,H,d] (overwritten; each is
 * the sum over the sample's own tokens, zero for an empty sample).  With an elementwise map,
 * o and lse are not read and may be NULL.  The softmax row term rowsum(dO * O) equals
 * sum_j P_j dP_j; for bf16 with head_dim 128 and n_kv <= 256 (one work-group holds a
 * sample's whole context) it is summed from P and dP inside the backward, o is not
 * read and may be NULL (lse is still required). */
gdpa_status gdpa_bwd(const gdpa_problem* p, const int32_t* offsets, const void* q, const void* k,
                     const void* v, const void* o, const float* lse, const void* d_o, void* dq,
                     void* dk, void* dv, void* workspace, size_t workspace_bytes, void* stream);

/* Residual layer block (the stacked personalised FFN: the layer's input tokens
 * are its queries and its output adds GDPA to them, Kunlun paper summary
 * section 2.2, GDPA bullet, read as a plain residual): with queries x [T,H,d],
 *     o = GDPA(x; k, v)   and   y = x + o
 * written in one pass.  gdpa_fwd with GDPA_FWD_RESIDUAL writes only y; this call
 * keeps o as well, which the softmax backward of such a layer needs for its row
 * term where it reads o (o taken back as y - x would carry y's rounding, relative
 * to |x|).  The backward is gdpa_bwd with GDPA_BWD_RESIDUAL and this o.  p->flags must be 0;
 * o and y must be distinct from each other and from x, k and v.  Otherwise as
 * gdpa_fwd (lse written for softmax when non-NULL; workspace as gdpa_fwd's). */
gdpa_status gdpa_fwd_block(const gdpa_problem* p, const int32_t* offsets, const void* x, const void* k,
                           const void* v, void* o, void* y, float* lse, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Jagged context (a variant of the same op: event-level personalisation gives
 * each event type its own number of context tokens, Kunlun paper summary,
 * section 2.3, Event-Level Personalization bullet; Telegram review, the list of
 * per-event hyper-parameters, n_tokens among them).  Sample b owns context rows kv_offsets[b] ..
 * kv_offsets[b+1]-1 of k, v [rows][H][d] (dk, dv likewise); p->n_kv is the
 * largest per-sample count (it selects the kernels and sizes the workspace,
 * gdpa_workspace_bytes as for the dense form).  Every sample must own at least
 * one and at most n_kv context rows (a softmax over no rows is undefined); like
 * `offsets`, the device array is the caller's contract and gdpa_check_kv_offsets
 * checks a host copy.  Otherwise as gdpa_fwd / gdpa_bwd; a NULL kv_offsets is
 * GDPA_ERR_INVALID_ARGUMENT. */
gdpa_status gdpa_fwd_jagged_kv(const gdpa_problem* p, const int32_t* offsets, const int32_t* kv_offsets,
                               const void* q, const void* k, const void* v, const void* residual,
                               void* o, float* lse, void* workspace, size_t workspace_bytes,
                               void* stream);
gdpa_status gdpa_bwd_jagged_kv(const gdpa_problem* p, const int32_t* offsets, const int32_t* kv_offsets,
                               const void* q, const void* k, const void* v, const void* o,
                               const float* lse, const void* d_o, void* dq, void* dk, void* dv,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Residual sums of a layer stack: out = x0 + x1 (+ x2) (+ x3) over `count` bf16
 * values (count % 8 == 0, else GDPA_ERR_UNSUPPORTED), summed in fp32 and rounded
 * once; x2 and x3 may be NULL; out may alias any input.  Used by layer drivers
 * for the residual of a self-attention layer and for gradients that reach one
 * tensor through several uses (Q = K = V = X). */
gdpa_status gdpa_add_bf16(int64_t count, void* out, const void* x0, const void* x1, const void* x2,
                          const void* x3, void* stream);

/* FFN biases (a variant of the same op: a two-layer FFN carries a bias per hidden
 * unit and per output; the pages give none, so the base calls have none):
 *
 *     O[t,h,:] = phi(scale * <Q[t,h,:], K[j,h,:]> + score_bias[j,h])_j V[.,h,:] + out_bias[b,h,:]
 *
 * score_bias is float32 [B][n_kv][H] for the dense context or [rows][H] with
 * kv_offsets (one value per context row and head, like K without d); out_bias is
 * float32 [B][H][d] (one row per sample and head).  Either may be NULL (no bias).
 * kv_offsets may be NULL (dense context).  The backward also returns
 * d_score_bias (the sum over the sample's tokens of the score gradient, layout
 * of score_bias) and d_out_bias (the sum of dO over the sample's tokens,
 * [B][H][d]), each when non-NULL; for softmax it needs the forward's lse and o
 * and the same biases.  p->flags must be 0 (GDPA_ERR_UNSUPPORTED otherwise).
 * Workspace: gdpa_biased_workspace_bytes(p, backward, out_bias != NULL).  With
 * softmax, bf16 and an output bias the backward does not read o: the softmax row
 * term sum_e (P V)[t,h,e] dO[t,h,e] taken from the bf16 O = P V + out_bias would
 * carry O's rounding, relative to |P V + out_bias|, so the backward recomputes
 * P V once (one extra forward pass) into its workspace, which then also holds
 * T*H*(2d + 4) bytes for it.  Otherwise as gdpa_fwd / gdpa_bwd. */
size_t gdpa_biased_workspace_bytes(const gdpa_problem* p, int backward, int out_bias);
gdpa_status gdpa_fwd_biased(const gdpa_problem* p, const int32_t* offsets, const int32_t* kv_offsets,
                            const void* q, const void* k, const void* v, const float* score_bias,
                            const float* out_bias, void* o, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream);
gdpa_status gdpa_bwd_biased(const gdpa_problem* p, const int32_t* offsets, const int32_t* kv_offsets,
                            const void* q, const void* k, const void* v, const float* score_bias,
                            const float* out_bias, const void* o, const float* lse, const void* d_o,
                            void* dq, void* dk, void* dv, float* d_score_bias, float* d_out_bias,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Grouped launch (event-level personalisation, Kunlun paper summary section 2.3:
 * each event type, e.g. clicks and impressions, gets its own width, head count
 * and other sizes).  One call runs several independent GDPA problems, each with
 * its own gdpa_problem (heads, head_dim, n_kv, phi, dtype, scale, flags), jagged
 * batch and tensors, as gdpa_fwd / gdpa_bwd (or the _jagged_kv forms when
 * kv_offsets is non-NULL) would for that group alone.
 *
 * `groups` is a HOST array of n >= 1 descriptors; the pointers inside are device
 * pointers with the meaning of the same-named arguments of gdpa_fwd / gdpa_bwd
 * (the forward reads offsets, kv_offsets, q, k, v, residual and writes o, lse;
 * the backward reads offsets, kv_offsets, q, k, v, o, lse, d_o and writes dq, dk,
 * dv).  No group's output may be another group's output or input (such a call
 * fails with GDPA_ERR_INVALID_ARGUMENT; only equal base pointers are detected,
 * not partial overlaps).  Workspace:
 * gdpa_grouped_workspace_bytes (the sum of the groups' own, each 256-byte
 * aligned).  All groups are checked before anything is launched; an invalid
 * group fails the call with its status and launches nothing.  The groups run
 * concurrently: the call forks from `stream` onto up to three streams that the
 * library creates on the current device (default priority; created on first
 * use, kept until the process ends) and joins back, all through stream events,
 * so it stays asynchronous on `stream` and may be captured into a HIP graph.
 * `stream` must belong to the current device. */
typedef struct {
  gdpa_problem problem;
  const int32_t* offsets;    /* [B+1] token offsets */
  const int32_t* kv_offsets; /* [B+1] context row offsets, or NULL (dense [B, n_kv, H, d]) */
  const void* q;
  const void* k;
  const void* v;
  const void* residual;      /* forward with GDPA_FWD_RESIDUAL, else NULL */
  void* o;                   /* forward output; backward input (softmax) */
  float* lse;                /* forward output; backward input (softmax) */
  const void* d_o;           /* backward */
  void* dq;
  void* dk;
  void* dv;
} gdpa_group;
size_t gdpa_grouped_workspace_bytes(int32_t n, const gdpa_group* groups, int backward);
gdpa_status gdpa_fwd_grouped(int32_t n, const gdpa_group* groups, void* workspace, size_t workspace_bytes,
                             void* stream);
gdpa_status gdpa_bwd_grouped(int32_t n, const gdpa_group* groups, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Backward without allocation, for callers that cannot allocate device memory
 * (code under HIP graph capture, serving loops and harnesses that forbid it):
 * gdpa_bwd with the workspace taken from a scratch array that the library keeps
 * on each GPU, GDPA_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, set up on the first
 * call on that GPU and held until the process ends.  Same arguments, results
 * and errors as gdpa_bwd without the workspace; a problem whose gdpa_bwd
 * workspace (gdpa_workspace_bytes(p, 1)) exceeds the scratch fails with
 * GDPA_ERR_WORKSPACE_TOO_SMALL before anything is launched (for the softmax map
 * outside the one-work-group shapes named at gdpa_bwd it holds 4 * total_tokens *
 * heads bytes of row dots, so up to about 16.7 M token-head rows; otherwise a few
 * bytes per sample).
 * `stream` must belong to the current device.  The call allocates nothing and
 * nothing in the scratch needs to start at zero.  All calls on one GPU share
 * its scratch: two calls that overlap in time on one GPU (on different streams,
 * or from different threads without ordering) race and give undefined results. */
#define GDPA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
gdpa_status gdpa_bwd_noalloc(const gdpa_problem* p, const int32_t* offsets, const void* q, const void* k,
                             const void* v, const void* o, const float* lse, const void* d_o, void* dq,
                             void* dk, void* dv, void* stream);

/* Host-side check of a HOST copy of kv_offsets ([batch + 1] int32): kv_offsets[0] = 0
 * and every sample owns 1 .. n_kv rows (n_kv >= 1, batch >= 0: an empty batch is
 * {0}); GDPA_OK or GDPA_ERR_INVALID_ARGUMENT. */
gdpa_status gdpa_check_kv_offsets(const int32_t* host_kv_offsets, int32_t batch, int32_t n_kv);

/* Weight generation (paper summary section 2.1, interaction block; Telegram
 * review, layer step 1: K and V are obtained from the context features), read
 * as one linear map per layer with an output-major weight (the usual linear-layer
 * layout):  out[B, cols] = ctx[B, ctx_dim] * w[cols, ctx_dim]^T, bf16 in and out,
 * fp32 accumulation.  With cols = n_kv*H*d the output is K or V in the
 * [B][n_kv][H][d] layout.  Requires cols % 8 == 0 and ctx_dim % 8 == 0. */
gdpa_status gdpa_weightgen_fwd(int32_t batch, int32_t ctx_dim, int64_t cols, const void* ctx,
                               const void* w, void* out, void* stream);

/* Gradient of the weight-generation map w.r.t. w:  d_w[cols, ctx_dim] = d_out^T * ctx
 * (overwritten; same layout as w), bf16 in and out, fp32 accumulation over the batch. */
gdpa_status gdpa_weightgen_bwd_w(int32_t batch, int32_t ctx_dim, int64_t cols, const void* ctx,
                                 const void* d_out, void* d_w, void* stream);

/* ---------------------------------------------------------------------------
 * Sliding-window self-attention over the same jagged batch (Kunlun paper
 * summary, section 2.2, Sliding Window Attention bullet: the sequence's
 * self-attention is restricted to local windows, O(T w) instead of O(T^2);
 * Telegram review, layer step 5, and the event-level personalisation list that
 * names w, the window size).  Q, K, V come from the sequence itself, all
 * [T][H][d]; for token i (its position inside its sample) and head h:
 *
 *     s_j      = scale * < Q[i,h,:], K[j,h,:] >   for  i - window < j <= i  (same sample)
 *     O[i,h,:] = sum_j softmax(s)_j V[j,h,:]
 *
 * The window is causal and holds the token and the window - 1 tokens before it
 * (the pages restrict attention to a token's latest interactions and give no
 * formula).  bf16 only,
 * fp32 accumulation; head_dim in {32, 64, 128}.
 * ------------------------------------------------------------------------- */
typedef struct {
  int32_t batch;         /* B >= 1 samples */
  int32_t total_tokens;  /* T = offsets[B] >= 0 */
  int32_t max_seqlen;    /* >= every sample length (informational) */
  int32_t heads;         /* H >= 1 */
  int32_t head_dim;      /* d in {32, 64, 128} */
  int32_t window;        /* w >= 1 */
  float scale;           /* finite; 1/sqrt(d) is the usual value */
  int32_t dtype;         /* GDPA_BF16 (GDPA_F32: GDPA_ERR_UNSUPPORTED) */
  uint32_t flags;        /* must be 0 */
} gdpa_swa_problem;

/* Workspace bytes for gdpa_swa_fwd (backward = 0) or gdpa_swa_bwd (backward != 0);
 * 0 for an invalid problem. */
size_t gdpa_swa_workspace_bytes(const gdpa_swa_problem* p, int backward);

/* Forward.  q, k, v [T,H,d] in; o [T,H,d] out (overwritten; must not alias an
 * input); lse [T,H] float32 (natural log) written when non-NULL, required by the
 * backward.  Errors as for gdpa_fwd. */
gdpa_status gdpa_swa_fwd(const gdpa_swa_problem* p, const int32_t* offsets, const void* q,
                         const void* k, const void* v, void* o, float* lse, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Backward of sum(O * dO): q, k, v, o, lse (from gdpa_swa_fwd) and d_o in; dq, dk,
 * dv [T,H,d] out (overwritten; distinct from the inputs and from each other). */
gdpa_status gdpa_swa_bwd(const gdpa_swa_problem* p, const int32_t* offsets, const void* q,
                         const void* k, const void* v, const void* o, const float* lse,
                         const void* d_o, void* dq, void* dk, void* dv, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Self-attention block of a Kunlun layer with its residual (Telegram review,
 * layer step 5; the projections sit outside the op): Q = K = V = x [T,H,d] and
 *     y = x + O,   O = SWA(x, x, x)
 * The forward writes O (kept for the backward's softmax row term) and y in one
 * pass; y must not alias x or o.  The backward takes the block's upstream
 * gradient d_y (it reaches x through the residual and through O) and writes
 *     d_x = d_y + dQ + dK + dV
 * without separate dQ, dK, dV tensors; d_x must not alias x, o or d_y.  Problem,
 * workspace (gdpa_swa_workspace_bytes) and errors as for gdpa_swa_fwd / _bwd. */
gdpa_status gdpa_swa_block_fwd(const gdpa_swa_problem* p, const int32_t* offsets, const void* x, void* o,
                               void* y, float* lse, void* workspace, size_t workspace_bytes, void* stream);
gdpa_status gdpa_swa_block_bwd(const gdpa_swa_problem* p, const int32_t* offsets, const void* x, const void* o,
                               const float* lse, const void* d_y, void* d_x, void* workspace,
                               size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Seed pooling attention over the same jagged batch: the attention core of
 * Pooling by Multihead Attention, whose learnable seed queries Hierarchical
 * Seed Pooling builds on to summarise long sequences (Kunlun paper summary,
 * section 2.2, HSP bullet; Telegram review, layer step 3).  m learned seeds
 * [m][H][d], shared by all samples, attend over each sample's tokens K, V
 * [T][H][d]; for sample b, seed s and head h:
 *
 *     s_j        = scale * < Seeds[s,h,:], K[j,h,:] >    j over the tokens of sample b
 *     O[b,s,h,:] = sum_j softmax(s)_j V[j,h,:]
 *
 * O is [B][m][H][d] and lse [B][m][H] float32 (natural log).  An empty sample
 * pools nothing: its O rows are 0 and its lse -inf.  The compression that HSP
 * applies to the pooled seeds (SumKronLinear) has no formula on the pages and is
 * not part of this call.  bf16 only, fp32 accumulation; head_dim in {32, 64,
 * 128}; 1 <= m <= 32.
 * ------------------------------------------------------------------------- */
typedef struct {
  int32_t batch;         /* B >= 1 samples */
  int32_t total_tokens;  /* T = offsets[B] >= 0 */
  int32_t max_seqlen;    /* >= every sample length (informational) */
  int32_t heads;         /* H >= 1 */
  int32_t head_dim;      /* d in {32, 64, 128} */
  int32_t seeds;         /* m, 1 .. 32 */
  float scale;           /* finite; 1/sqrt(d) is the usual value */
  int32_t dtype;         /* GDPA_BF16 (GDPA_F32: GDPA_ERR_UNSUPPORTED) */
  uint32_t flags;        /* 0, or GDPA_PMA_BWD_KV_SUM for gdpa_pma_bwd */
} gdpa_pma_problem;

/* gdpa_pma_bwd flag for pooling a sequence with itself (K = V = X, as HSP pools
 * the token states): k and v must be the same pointer; dk receives dK + dV in
 * one tensor and dv must be NULL (GDPA_ERR_INVALID_ARGUMENT otherwise). */
#define GDPA_PMA_BWD_KV_SUM 0x1u

/* Workspace bytes for gdpa_pma_fwd (backward = 0) or gdpa_pma_bwd (backward != 0);
 * 0 for an invalid problem.  At most about (T / 1024 + B) * H * 128 * d bytes
 * (per-chunk partial results in fp32). */
size_t gdpa_pma_workspace_bytes(const gdpa_pma_problem* p, int backward);

/* Forward.  seeds [m,H,d], k, v [T,H,d] in; o [B,m,H,d] and lse [B,m,H] out
 * (overwritten; o must not alias an input; both required).  Errors as for
 * gdpa_fwd. */
gdpa_status gdpa_pma_fwd(const gdpa_pma_problem* p, const int32_t* offsets, const void* seeds,
                         const void* k, const void* v, void* o, float* lse, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Backward of sum(O * dO): seeds, k, v, o and lse (from gdpa_pma_fwd) and d_o
 * [B,m,H,d] in; d_seeds [m,H,d] (summed over every sample), dk and dv [T,H,d]
 * out (overwritten; distinct from the inputs and from each other; with
 * GDPA_PMA_BWD_KV_SUM, dk = dK + dV and dv NULL). */
gdpa_status gdpa_pma_bwd(const gdpa_pma_problem* p, const int32_t* offsets, const void* seeds,
                         const void* k, const void* v, const void* o, const float* lse,
                         const void* d_o, void* d_seeds, void* dk, void* dv, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Host-side check of a HOST copy of offsets ([batch + 1] int32): returns GDPA_OK when
 * offsets[0] = 0, the array is non-decreasing, offsets[batch] = total_tokens and every
 * length is at most max_seqlen (batch, total_tokens, max_seqlen >= 0; an empty batch
 * is {0} with total_tokens = 0); GDPA_ERR_INVALID_ARGUMENT otherwise. */
gdpa_status gdpa_check_offsets(const int32_t* host_offsets, int32_t batch, int32_t total_tokens,
                               int32_t max_seqlen);

/* Static description of a status code. */
const char* gdpa_status_str(gdpa_status s);

/* hipError_t of the last GDPA_ERR_HIP returned on this thread (0 if none). */
int gdpa_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* GDPA_H */
