/*
 * carve.h -- C ABI of the MI355X (gfx950) CARVE key-axis gated delta rule.
 *
 * The operation (CARVE pages: liuzhao09.github.io CARVE notes, sections 2.1-2.3;
 * gist.science technical summary, section 2):  per batch b and head h, with a
 * state S in R^{Dv x Dk} (rows: value index, columns: key index),
 *
 *     a_t = exp(log_g_t) * b_t                      key-axis retention x erase, in (0,1]^Dk
 *     P_t = S_{t-1} Diag(a_t)                       decay and erase right-multiply the key axis
 *     S_t = P_t + w_t (v_t - P_t k_t) k_t^T         delta-rule write of the prediction error,
 *                                                   one scalar write strength w_t per head
 *     o_t = S_t q_t                                 readout of the updated state
 *
 * computed chunk-parallel in WY form: within a chunk of tokens one strictly
 * lower-triangular coupling matrix, shared by every value channel because all
 * gating sits on the key axis, is inverted once (section 2.3 of the notes: the
 * coupling does not depend on the value index, so a single triangular solve
 * serves all d_v columns).  Optionally the erase gate is content-aware
 * (section 2.2): for chunk c of L tokens
 *
 *     b_{c,t} = sigmoid(b_x_t + U2 (U1 m_{c-1})),   m_{c-1} = mean of chunk c-1's outputs o,
 *
 * with m_{-1} = m0 (zero when not given), a zero-initialised low-rank projection
 * U_b = U2 U1 per head.
 *
 * No query scaling and no normalisation are applied; callers L2-normalise q, k.
 *
 * Conventions shared by every entry point
 *   - Pointers marked (device) are HIP device pointers; structs are host memory.
 *   - All tensors are dense, row-major, with the shapes given below, and
 *     16-byte aligned.  "dtype" tensors are float32 or bfloat16 per shape->dtype;
 *     gates, states, workspace-independent outputs marked float are float32.
 *   - The caller owns every buffer, including the workspace, which must hold at
 *     least *_workspace_size() bytes.  The library never allocates or frees
 *     device memory; its global state is a per-device cache of the compute-unit
 *     count (the size of its persistent launches) and, for carve_fwd_noalloc
 *     only, a fixed device array with its per-device address.  Calls on
 *     different streams may run concurrently as long as they use different
 *     workspaces.
 *   - Every launch is enqueued on `stream` (a hipStream_t; NULL = default
 *     stream) and the call returns without synchronising.
 *   - Argument checks run on the host before any launch.  On a non-OK status
 *     nothing has been launched and no output was touched, except
 *     CARVE_ERR_HIP, which reports a launch error (hipGetLastError) after the
 *     launches were issued.  Device faults surface at the caller's next
 *     synchronisation.  NaN/Inf inputs propagate unchecked.
 *   - Supported: Dk, Dv in {64, 128}; any T >= 0 (a final partial chunk is
 *     handled); B, H >= 0 (an empty batch, head or token axis is a no-op that
 *     still writes S_T = S0 and m_out = m0).  Chunk length L: any L >= 1 for
 *     token-only gates (the result does not depend on L; the kernels tile
 *     tokens in blocks of 32 when L <= 32 or dtype is float32, and of 64
 *     otherwise); for the content path L must be a multiple of that tile.
 *   - Unequal widths (Dk != Dv; the pages write the state as Dv x Dk with
 *     independent widths, notes section 1) are accepted by every entry point.
 *     Except for the decode step, which takes both widths directly, such a call
 *     runs at D = max(Dk, Dv) on padded copies of its operands held in front of
 *     its workspace (for the training pairs, the padded inputs in front of the
 *     saved buffer, where the saved backward reads them).  Padded key channels
 *     carry k = q = 0 and retention 1 (log g = 0 and b = 1; A = 0 and
 *     b_x = 1e30 for gates given as pre-activations; b_x = 1e30 with zero rows of
 *     U2 on the content path), padded value rows v = dO = 0 (and zero columns of
 *     U1), so every padded term is an exact zero, and the outputs are cut back to
 *     the caller's widths.  The size functions count the copies (on the content
 *     path for any rank up to 64, with room for the records).
 *   - Numerical range: any retention a = exp(log g) * b in [0, 1] is handled
 *     (the pages put no floor on the decay, notes section 2.3, and take the
 *     erase as a factor in (0, 1], section 2.1).  The kernels carry the
 *     cumulative log-retention inside each tile of tokens: a tile whose
 *     log-retention stays above -80 in every key channel refers its operands
 *     to the tile start; a stronger tile refers them to 16-token blocks, and a
 *     block beyond -64 computes its within-block ratios as running products of
 *     the retention.  Per-token log-retention is taken in [-1e4, 0] (values above
 *     0 count as 0, a retention below e^-1e4 as e^-1e4, zero in float32).
 *   - Conditioning of the erase gradient: d/db = d/dlog a / b carries the
 *     absolute error of d/dlog a (a reverse cumulative sum over the tile)
 *     divided by b, so it is ill-conditioned where b is small; d/dlog g (which
 *     equals b * d/db) and the pre-activation gradients d/db_x = d/dlog a (1 - b)
 *     of carve_bwd_logits and carve_bwd_content are well conditioned.
 */
#ifndef CARVE_H
#define CARVE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CARVE_ABI_VERSION 3

typedef enum {
  CARVE_OK = 0,
  CARVE_ERR_INVALID_ARG = 1,   /* null required pointer, negative size, b given together with content, ... */
  CARVE_ERR_UNSUPPORTED = 2,   /* shape or option outside the supported set above                    */
  CARVE_ERR_WORKSPACE = 3,     /* workspace smaller than *_workspace_size()                          */
  CARVE_ERR_HIP = 4            /* a kernel launch failed                                             */
} carve_status;

typedef enum { CARVE_F32 = 0, CARVE_BF16 = 1 } carve_dtype;   /* dtype of q, k, v, o, dO, dq, dk, dv */

typedef struct {
  int B, H, T;     /* batch, heads, tokens                         */
  int Dk, Dv;      /* key and value widths, each 64 or 128         */
  int L;           /* chunk length                                  */
  carve_dtype dtype;
} carve_shape;

/* Content-aware erase (notes section 2.2).  Pass NULL to carve_fwd for token-only gates. */
typedef struct {
  const float* b_x;  /* (device) [B,H,T,Dk] erase pre-activation (required)                     */
  const float* U1;   /* (device) [H,R,Dv] or NULL;  U1 and U2 both NULL = no projection,        */
  const float* U2;   /* (device) [H,Dk,R] or NULL;  then b = sigmoid(b_x) exactly               */
  int R;             /* rank of the projection, 1..64 (ignored when U1 = U2 = NULL)             */
  const float* m0;   /* (device) [B,H,Dv] mean output of the chunk before this call, or NULL (= 0) */
  float* m_out;      /* (device) [B,H,Dv] mean output of this call's last chunk, or NULL         */
  /* Per-period records, P = ceil(T / L) periods of L tokens (both NULL, or both given):
   * z_rec [B,H,P,Dk] the content signal z = U2 (U1 m) each period's erase gate used, and
   * m_rec [B,H,P,Dv] the mean output m it was formed from (m0 or 0 for the first period).
   * carve_fwd writes them; carve_bwd_content reads them (the records of the forward of the
   * same inputs) instead of re-running the content-aware forward to obtain them.  Either
   * way the gradients are the same bits.  Caller-owned, 16-byte aligned. */
  float* z_rec;
  float* m_rec;
} carve_content;

/* Bytes of device workspace carve_fwd needs for this shape (0 is a valid answer). */
size_t carve_fwd_workspace_size(const carve_shape* s, const carve_content* content);

/*
 * Forward pass.
 *   q, k   (device) [B,H,T,Dk] dtype          v (device) [B,H,T,Dv] dtype
 *   log_g  (device) [B,H,T,Dk] float, <= 0    log of the key-axis retention
 *   b      (device) [B,H,T,Dk] float in (0,1] erase gate, or NULL (= 1); must be NULL with content
 *   w      (device) [B,H,T]    float          scalar write strength per head and token
 *   S0     (device) [B,H,Dv,Dk] float         initial state, or NULL (= 0)
 *   content                                    NULL (token-only gates) or content-aware erase
 *   o      (device) [B,H,T,Dv] dtype          output (written)
 *   S_T    (device) [B,H,Dv,Dk] float         final state (written), or NULL
 * With few heads and a long sequence (B*H*Dk/16 < 256 and at least 32 chunks of
 * tokens) the token-only state pass runs as segments of chunks whose affine maps
 * S_in -> S_in Pi + C are chained by a short scan (the workspace then also holds
 * their float32 maps); the result agrees with the sequential pass to rounding.
 */
carve_status carve_fwd(const carve_shape* s,
                       const void* q, const void* k, const void* v,
                       const float* log_g, const float* b, const float* w,
                       const float* S0, const carve_content* content,
                       void* o, float* S_T,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Forward for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): carve_fwd with the same
 * arguments minus the workspace, which is instead a library-owned device array of
 * CARVE_NOALLOC_SCRATCH_BYTES on each device (held until the process ends; its address
 * is looked up once per device on the first call there).  The call allocates and frees
 * nothing.  A shape whose carve_fwd_workspace_size() exceeds the array returns
 * CARVE_ERR_WORKSPACE before any launch.  Every call on one device shares that device's
 * array: calls that overlap in time on one device (different streams, or host threads
 * with unsynchronised streams) race on it and must be serialised by the caller.  No part
 * of the array needs to start at zero: every byte a call reads is written earlier in the
 * same call.
 */
#define CARVE_NOALLOC_SCRATCH_BYTES (64u << 20)
carve_status carve_fwd_noalloc(const carve_shape* s,
                               const void* q, const void* k, const void* v,
                               const float* log_g, const float* b, const float* w,
                               const float* S0, const carve_content* content,
                               void* o, float* S_T, void* stream);

/* Bytes of device workspace carve_bwd needs for this shape. */
size_t carve_bwd_workspace_size(const carve_shape* s);

/*
 * Backward pass of the token-only forward (the content-aware forward has its own
 * backward, carve_bwd_content, below): the reverse-mode derivative of the chunked
 * forward, whose fused forward/backward pair and "backward scan" over chunks the notes
 * report in section 3.1 (Table 2, forward and backward error against the reference)
 * and section 4 (summary).  The pages print no backward formula; this is the exact
 * gradient of the forward defined above, reached by a reverse state pass
 * dS_c = dS_{c+1} M_c^T + (terms of chunk c's outputs), M_c the chunk's state map, and
 * per chunk back through the output, the WY factors, the inverse of (I + A) and the
 * cumulative retention.  Recomputes the forward internally.
 *   q, k, v, log_g, b, w, S0   as for carve_fwd
 *   dO     (device) [B,H,T,Dv] dtype          gradient of the loss w.r.t. o
 *   dS_T   (device) [B,H,Dv,Dk] float         gradient w.r.t. S_T, or NULL (= 0)
 * Outputs (all written, shapes as the matching input):
 *   dq, dk (dtype) [B,H,T,Dk]; dv (dtype) [B,H,T,Dv];
 *   dlog_g (float) [B,H,T,Dk]: derivative w.r.t. log g;
 *   db     (float) [B,H,T,Dk]: derivative w.r.t. the erase probability b; must be NULL iff b is NULL;
 *   dw     (float) [B,H,T]:    derivative w.r.t. w;
 *   dS0    (float) [B,H,Dv,Dk] derivative w.r.t. S0, or NULL (not written).
 */
carve_status carve_bwd(const carve_shape* s,
                       const void* q, const void* k, const void* v,
                       const float* log_g, const float* b, const float* w,
                       const float* S0, const void* dO, const float* dS_T,
                       void* dq, void* dk, void* dv, float* dlog_g, float* db, float* dw, float* dS0,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Stage timing.  The *_ex variants behave exactly like carve_fwd / carve_bwd and
 * additionally record caller-created HIP events (hipEvent_t handles) on
 * `stream` at the stage boundaries: events[i] just before stage i is
 * launched and events[i+1] just after it, for i < n_events - 1.  Nothing is
 * synchronised; the caller reads the events afterwards (hipEventElapsedTime).
 *   carve_fwd  stages: 0 = chunk prep (token-only) or the content-aware
 *                      kernel (content path, single stage), 1 = state pass
 *                      (segmented: the affine maps, their scan and the
 *                      segments' state passes)
 *   carve_bwd  stages: 0 = chunk prep, 1 = forward state pass,
 *                      2 = reverse state pass, 3 = chunk gradients
 * With profile == NULL they are carve_fwd / carve_bwd.
 */
#define CARVE_MAX_STAGES 8
typedef struct {
  void* events[CARVE_MAX_STAGES + 1];
  int n_events;
} carve_profile;

carve_status carve_fwd_ex(const carve_shape* s,
                          const void* q, const void* k, const void* v,
                          const float* log_g, const float* b, const float* w,
                          const float* S0, const carve_content* content,
                          void* o, float* S_T,
                          void* workspace, size_t workspace_bytes, void* stream,
                          const carve_profile* profile);

carve_status carve_bwd_ex(const carve_shape* s,
                          const void* q, const void* k, const void* v,
                          const float* log_g, const float* b, const float* w,
                          const float* S0, const void* dO, const float* dS_T,
                          void* dq, void* dk, void* dv, float* dlog_g, float* db, float* dw, float* dS0,
                          void* workspace, size_t workspace_bytes, void* stream,
                          const carve_profile* profile);

/*
 * Training pair: a forward that keeps what its backward needs, and a backward
 * that uses it instead of recomputing the forward (token-only gates).
 *
 * carve_fwd_save is carve_fwd (content = NULL) that also fills `saved`
 * (device, caller-owned, at least carve_saved_size() bytes) with the chunk
 * factors and the state entering every chunk.  carve_bwd_saved takes the same
 * inputs (S0 is not needed again: it is in `saved`), dO and dS_T, the `saved`
 * buffer of a carve_fwd_save call with the same shape and inputs (the library
 * cannot check that the contents match), and a workspace of
 * carve_bwd_saved_workspace_size() bytes; outputs as carve_bwd.  Stages for the
 * profile: carve_fwd_save 0 = chunk prep, 1 = state pass; carve_bwd_saved
 * 0 = reverse state pass, 1 = chunk gradients.
 */
size_t carve_saved_size(const carve_shape* s);
size_t carve_bwd_saved_workspace_size(const carve_shape* s);

carve_status carve_fwd_save(const carve_shape* s,
                            const void* q, const void* k, const void* v,
                            const float* log_g, const float* b, const float* w,
                            const float* S0, void* o, float* S_T,
                            void* saved, size_t saved_bytes, void* stream,
                            const carve_profile* profile);

carve_status carve_bwd_saved(const carve_shape* s,
                             const void* q, const void* k, const void* v,
                             const float* log_g, const float* b, const float* w,
                             const void* dO, const float* dS_T,
                             const void* saved, size_t saved_bytes,
                             void* dq, void* dk, void* dv, float* dlog_g, float* db, float* dw, float* dS0,
                             void* workspace, size_t workspace_bytes, void* stream,
                             const carve_profile* profile);

/*
 * Gates given as pre-activations, activated inside the kernels (the fused gate of
 * the notes, section 2.3: A the log-decay amplitude, f the decay logits, tau a bias,
 * the output log g <= 0; w_hat the scalar write pre-activation).  Reading taken:
 *     log g = -A softplus(f + tau),   b = sigmoid(b_x) (b = 1 without b_x),
 *     w = sigmoid(w_hat),
 * with A (> 0 for log g <= 0) and tau per head and key channel.
 */
typedef struct {
  const float* f;      /* (device) [B,H,T,Dk] decay logits                         */
  const float* A;      /* (device) [H,Dk]     decay amplitude                      */
  const float* tau;    /* (device) [H,Dk]     decay bias                           */
  const float* b_x;    /* (device) [B,H,T,Dk] erase pre-activation, or NULL (b = 1) */
  const float* w_hat;  /* (device) [B,H,T]    write pre-activation                 */
} carve_gate_logits;

/*
 * Forward with gates given as pre-activations (token-only gates): as carve_fwd with
 * log_g, b, w replaced by `gates`; workspace of carve_fwd_workspace_size(s, NULL).
 */
carve_status carve_fwd_logits(const carve_shape* s,
                              const void* q, const void* k, const void* v,
                              const carve_gate_logits* gates, const float* S0,
                              void* o, float* S_T,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Its backward: as carve_bwd, with the gate gradients in the pre-activations'
 * space: df (float) [B,H,T,Dk]; dA, dtau (float) [H,Dk], summed over batch and
 * tokens; db_x (float) [B,H,T,Dk], required iff gates->b_x is given; dw_hat (float)
 * [B,H,T].  Workspace of carve_bwd_logits_workspace_size() bytes.
 */
size_t carve_bwd_logits_workspace_size(const carve_shape* s);
carve_status carve_bwd_logits(const carve_shape* s,
                              const void* q, const void* k, const void* v,
                              const carve_gate_logits* gates, const float* S0,
                              const void* dO, const float* dS_T,
                              void* dq, void* dk, void* dv, float* df, float* dA, float* dtau,
                              float* db_x, float* dw_hat, float* dS0,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Training pair with the gates given as pre-activations: carve_fwd_logits that also fills
 * `saved` (at least carve_saved_size() bytes, the same layout as carve_fwd_save's), and
 * a backward that uses it instead of recomputing the forward: inputs as
 * carve_bwd_logits without S0 (it is in `saved`), the `saved` buffer of a
 * carve_fwd_logits_save call with the same shape and inputs (not checked), a workspace
 * of carve_bwd_logits_saved_workspace_size() bytes; outputs as carve_bwd_logits.
 * Profile stages: carve_fwd_logits_save 0 = chunk prep, 1 = state pass;
 * carve_bwd_logits_saved 0 = reverse state pass, 1 = chunk gradients, 2 = logit epilogue.
 */
size_t carve_bwd_logits_saved_workspace_size(const carve_shape* s);
carve_status carve_fwd_logits_save(const carve_shape* s,
                                   const void* q, const void* k, const void* v,
                                   const carve_gate_logits* gates, const float* S0,
                                   void* o, float* S_T, void* saved, size_t saved_bytes,
                                   void* stream, const carve_profile* profile);
carve_status carve_bwd_logits_saved(const carve_shape* s,
                                    const void* q, const void* k, const void* v,
                                    const carve_gate_logits* gates, const void* dO, const float* dS_T,
                                    const void* saved, size_t saved_bytes,
                                    void* dq, void* dk, void* dv, float* df, float* dA, float* dtau,
                                    float* db_x, float* dw_hat, float* dS0,
                                    void* workspace, size_t workspace_bytes, void* stream,
                                    const carve_profile* profile);

/*
 * Backward through the content-aware erase (notes section 2.2): gradients of the
 * content-aware forward, including the projection and the chain through each
 * chunk's mean output into the next chunk's gate.  Recomputes the forward.
 *   q, k, v, log_g, w, S0, content   as for carve_fwd (content required; its
 *                                    m_out is ignored)
 *   dO     (device) [B,H,T,Dv] dtype   gradient w.r.t. o
 *   dS_T   (device) [B,H,Dv,Dk] float  gradient w.r.t. S_T, or NULL (= 0)
 *   dm_out (device) [B,H,Dv] float     gradient w.r.t. m_out (the last chunk's mean), or NULL (= 0)
 * Outputs:
 *   dq, dk (dtype) [B,H,T,Dk]; dv (dtype) [B,H,T,Dv]; dlog_g (float) [B,H,T,Dk];
 *   db_x   (float) [B,H,T,Dk]  derivative w.r.t. the erase pre-activation b_x;
 *   dw     (float) [B,H,T];
 *   dU1    (float) [H,R,Dv], dU2 (float) [H,Dk,R]: summed over the batch; required
 *          when the projection is given, NULL without it;
 *   dm0    (float) [B,H,Dv] derivative w.r.t. m0, or NULL (not written);
 *   dS0    (float) [B,H,Dv,Dk] derivative w.r.t. S0, or NULL (not written).
 * The chunks of L tokens are swept in reverse, one sweep step per chunk (a few
 * launches each, all heads in parallel), because chunk c-1's output gradient
 * needs chunk c's gate gradient.
 */
size_t carve_bwd_content_workspace_size(const carve_shape* s, const carve_content* content);

carve_status carve_bwd_content(const carve_shape* s,
                               const void* q, const void* k, const void* v,
                               const float* log_g, const float* w, const float* S0,
                               const carve_content* content,
                               const void* dO, const float* dS_T, const float* dm_out,
                               void* dq, void* dk, void* dv, float* dlog_g, float* db_x, float* dw,
                               float* dU1, float* dU2, float* dm0, float* dS0,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Recurrent decode: one new token per (batch, head), the O(Dv Dk) per-token form
 * of the same recurrence (comparison table of the notes, section 3), with the
 * state updated in place.  shape->T must be 1; shape->L is the content period
 * (ignored for token-only gates).
 *   q, k   (device) [B,H,Dk] dtype            v (device) [B,H,Dv] dtype
 *   log_g  (device) [B,H,Dk] float, <= 0      b (device) [B,H,Dk] float or NULL (= 1)
 *   w      (device) [B,H]    float
 *   S      (device) [B,H,Dv,Dk] float         state before the token; overwritten with the
 *                                              state after it (S_T of a carve_fwd prefill
 *                                              continues a sequence)
 *   content NULL (token-only gates) or the content-aware erase carry below
 *   o      (device) [B,H,Dv] dtype            output o = S q of the updated state (written)
 * Content-aware erase (b must be NULL): this token's gate is
 * b = sigmoid(b_x + U2 (U1 m_in)) with m_in the mean output of the previous
 * complete chunk of L tokens; `csum` holds the sum of the current chunk's outputs
 * so far and `pos` the number of them (0 <= pos < L; at pos = 0 csum is not read).
 * The call writes csum (the sum including this token, or 0 when the token
 * completes the chunk) and m_out (m_in again, or this chunk's mean when pos = L-1;
 * m_out must not alias m_in: other workgroups of the head still read m_in).  A
 * carve_fwd prefill of a whole number of chunks hands over with m_in = its m_out,
 * pos = 0.  Rows of one head are updated by different workgroups: S, o, csum and
 * m_out must not alias any input.
 */
typedef struct {
  const float* b_x;   /* (device) [B,H,Dk] erase pre-activation of this token (required)   */
  const float* U1;    /* (device) [H,R,Dv] or NULL; U1 and U2 both NULL = no projection     */
  const float* U2;    /* (device) [H,Dk,R] or NULL                                          */
  int R;              /* rank, 1..64 (ignored without projection)                            */
  const float* m_in;  /* (device) [B,H,Dv] mean output of the previous chunk, or NULL (= 0)  */
  float* m_out;       /* (device) [B,H,Dv] written (see above)                               */
  float* csum;        /* (device) [B,H,Dv] read when pos > 0, written                        */
  int pos;            /* tokens of the current chunk before this one                          */
} carve_decode_content;

carve_status carve_decode_step(const carve_shape* s,
                               const void* q, const void* k, const void* v,
                               const float* log_g, const float* b, const float* w,
                               float* S, const carve_decode_content* content,
                               void* o, void* stream);

/*
 * Measurement helper, not part of the CARVE operation: copies `bytes` from src to dst
 * (both device pointers, 16-byte aligned, non-overlapping; bytes a multiple of 16) with a
 * plain streaming kernel (each byte read once and written once by 16-byte vector accesses,
 * no reuse), asynchronously on `stream`.  Its rate is the device's achievable copy
 * bandwidth, the measured denominator set beside the published HBM peak when the kernels'
 * algorithmic bytes are put against the memory roofline.  bytes = 0 launches nothing;
 * misaligned, odd-sized or overlapping arguments return CARVE_ERR_INVALID_ARG.
 */
carve_status carve_stream_copy(void* dst, const void* src, size_t bytes, void* stream);

/* Human-readable name of a status code (static storage). */
const char* carve_status_string(carve_status st);

/* CARVE_ABI_VERSION of the built library. */
int carve_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CARVE_H */
