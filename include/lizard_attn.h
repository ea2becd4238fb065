/*
 * lizard_attn.h -- C ABI of the Lizard hybrid attention layer on MI355X (gfx950).
 *
 * The layer ("Lizard: An Efficient Linearization Framework for Large Language
 * Models", explained on gist.science; German page section 2 "Methodik",
 * "Kernkomponenten") replaces softmax attention with the sum
 *
 *     Y = Y_gate + alpha * Y_anchor                        (item 3 there)
 *
 * of a gated linear attention branch (item 1: a sigmoid gate drives a
 * data-adaptive recurrence with a constant-size state) and an anchor branch
 * (item 2: a sliding window of width w plus m learnable meta-memory tokens
 * that act as attention sinks and contribute no value).  Readings taken
 * where the pages are silent:
 *
 *   gate branch   S_t = diag(g_t) S_{t-1} + k_t v_t^T,  o_t = S_t^T q_t,
 *                 S_{-1} = 0, g_t = exp(log_g_t) per token and key dim;
 *   anchor        keys s in [max(0, t-w+1), t] plus m sink keys mu_i with
 *                 logits scale*q_t.k_s and scale*q_t.mu_i in one softmax;
 *                 sink values are zero; default scale 1/sqrt(dk);
 *   no positional encoding in either branch; alpha is a constant.
 *
 * Three entry points follow from what the pages say the layer must do:
 * replace attention in a pretrained model (a forward pass), be trained in
 * two stages (de section 2 "Trainingsprozess": a backward pass), and run
 * inference with constant memory through incremental state updates (de
 * section 2 item 1 and section 4 "Effizienz": a decode step).
 *
 * Conventions for every call
 *   - Tensor pointers are DEVICE pointers owned by the caller, 16-byte
 *     aligned, contiguous, row-major in the shapes given.  Outputs never
 *     alias inputs (decode's state and rings are the only in-out buffers).
 *     Every output element the call defines is overwritten, never
 *     accumulated.
 *   - The library allocates no device memory.  The backward pass takes a
 *     caller-owned workspace sized by lizard_attn_bwd_workspace_size().
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream) and never synchronise.  The library keeps no state between
 *     calls, so calls on different streams may run concurrently.
 *   - Argument checks run before any HIP call and return a status code
 *     synchronously; nothing is launched when a check fails.  A failed
 *     launch returns LIZARD_E_LAUNCH.  Faults inside kernels surface at the
 *     caller's next synchronisation.  Inputs with NaN or Inf, or log_g > 0,
 *     are outside the contract (results undefined, no fault).
 */
#ifndef LIZARD_ATTN_H
#define LIZARD_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LIZARD_F32 = 0,  /* float32 storage, float32 MFMA                         */
  LIZARD_BF16 = 1  /* bfloat16 storage, bf16 MFMA with float32 accumulate   */
} lizard_dtype_t;

typedef enum {
  LIZARD_OK = 0,
  LIZARD_E_NULL = -1,        /* a required pointer is NULL                   */
  LIZARD_E_SHAPE = -2,       /* a size is negative or out of its range       */
  LIZARD_E_DTYPE = -3,       /* unknown dtype                                */
  LIZARD_E_ALIGN = -4,       /* a pointer is not 16-byte aligned             */
  LIZARD_E_WORKSPACE = -5,   /* workspace missing or smaller than required  */
  LIZARD_E_UNSUPPORTED = -6, /* valid sizes the library has no kernel for   */
  LIZARD_E_LAUNCH = -7       /* the HIP launch reported an error             */
} lizard_status_t;

/* Sizes and constants shared by all calls.
 *   B, H      batch and heads (>= 0; a call with B*H == 0 or L == 0 is a no-op)
 *   L         sequence length (>= 0, any value; ignored by decode)
 *   dk, dv    head dims; the library requires dk == dv, and
 *             dk in {64, 128} for LIZARD_BF16, dk == 64 for LIZARD_F32
 *   chunk     chunk length of the chunked form; must be 64
 *   window    w, 1 <= w <= 64 (keys [t-w+1, t])
 *   n_meta    m, 0 <= m <= 16 sink keys per head
 *   alpha     weight of the anchor branch
 *   softmax_scale  logit scale; 0 means 1/sqrt(dk)
 *   dtype     element type of q, k, v, meta_k, y, y_anchor, dy, dq, dk, dv,
 *             and the decode rings.  log_g, lse, states, dlog_g and dmeta_k
 *             are always float32.                                          */
typedef struct {
  int32_t B, H, L;
  int32_t dk, dv;
  int32_t chunk;
  int32_t window;
  int32_t n_meta;
  float alpha;
  float softmax_scale;
  lizard_dtype_t dtype;
} lizard_params_t;

/* Forward pass (prefill / training), chunked log-space form.
 *   q, k        [B, H, L, dk]   dtype
 *   v           [B, H, L, dv]   dtype
 *   log_g       [B, H, L, dk]   float32, finite, <= 0 (log of the sigmoid gate)
 *   meta_k      [H, n_meta, dk] dtype (may be NULL when n_meta == 0)
 *   y           [B, H, L, dv]   dtype, out
 *   lse         [B, H, L]       float32, out, nullable: natural-log softmax
 *                               normaliser of the anchor branch (needed by
 *                               the backward pass)
 *   y_anchor    [B, H, L, dv]   dtype, out, nullable: the anchor branch alone
 *   state_out   [B, H, dk, dv]  float32, out, nullable: S_{L-1}, the state a
 *                               decode continuation starts from
 * Schedule: where too few heads are given to fill the GPU with one
 * workgroup per (head, value slice) and the sequences are long (the cases
 * in which lizard_attn_fwd_split_workspace_size(p) > 0, e.g. B*H = 32 at
 * L = 32K), the call runs lizard_attn_fwd_split's segment schedule, with a
 * workspace of that size taken from HIP's stream-ordered allocator on
 * `stream` and returned to it after the call's kernels (hipMallocAsync /
 * hipFreeAsync); its results are then lizard_attn_fwd_split's, equal to
 * the one-pass results up to float rounding.  If that allocation fails it
 * runs the one-pass schedule.  lizard_attn_fwd_logit and
 * lizard_attn_fwd_continue do the same; lizard_attn_fwd_train never
 * splits. */
lizard_status_t lizard_attn_fwd(const lizard_params_t* p,
                                const void* q, const void* k, const void* v,
                                const float* log_g, const void* meta_k,
                                void* y, float* lse, void* y_anchor, float* state_out,
                                void* stream);

/* Bytes of device workspace lizard_attn_bwd needs for these sizes (0 if the
 * sizes are invalid). */
size_t lizard_attn_bwd_workspace_size(const lizard_params_t* p);

/* Backward pass of loss = sum(dy * Y) (the layer is trained end to end; de
 * section 2 "Trainingsprozess").
 *   q, k, v, log_g, meta_k   as in lizard_attn_fwd
 *   lse         [B, H, L]       float32, from lizard_attn_fwd with the same inputs
 *   dy          [B, H, L, dv]   dtype
 *   dq, dk      [B, H, L, dk]   dtype, out
 *   dv          [B, H, L, dv]   dtype, out
 *   dlog_g      [B, H, L, dk]   float32, out (gradient w.r.t. log_g)
 *   dmeta_k     [H, n_meta, dk] float32, out (summed over the batch; may be
 *                               NULL when n_meta == 0)
 *   workspace   device buffer of at least lizard_attn_bwd_workspace_size(p)
 *               bytes, caller-owned, contents need not be initialised       */
lizard_status_t lizard_attn_bwd(const lizard_params_t* p,
                                const void* q, const void* k, const void* v,
                                const float* log_g, const void* meta_k,
                                const float* lse, const void* dy,
                                void* dq, void* dk, void* dv, float* dlog_g, float* dmeta_k,
                                void* workspace, size_t workspace_bytes,
                                void* stream);

/* One constant-memory decode step for every (b, h) at absolute position pos
 * (the same for all rows).  The incoming token is written to ring slot
 * pos mod w, the state is updated, then the window max(0, pos-w+1)..pos and
 * the sinks are read.
 *   q_t, k_t    [B, H, dk]      dtype
 *   v_t         [B, H, dv]      dtype
 *   log_g_t     [B, H, dk]      float32
 *   meta_k      [H, n_meta, dk] dtype (NULL allowed when n_meta == 0)
 *   state       [B, H, dk, dv]  float32, in-out (S_{pos-1} in, S_pos out)
 *   k_ring      [B, H, w, dk]   dtype, in-out; slot p mod w holds token p
 *   v_ring      [B, H, w, dv]   dtype, in-out
 *   y_t         [B, H, dv]      dtype, out
 * After a prefill of L0 tokens: state = state_out, and slot p mod w holds
 * k_p, v_p for p in [max(0, L0-w), L0); slots not yet written are never read. */
lizard_status_t lizard_decode_step(const lizard_params_t* p, int64_t pos,
                                   const void* q_t, const void* k_t, const void* v_t,
                                   const float* log_g_t, const void* meta_k,
                                   float* state, void* k_ring, void* v_ring,
                                   void* y_t, void* stream);

/* Forward pass of a segment that continues a sequence (chunked prefill, and
 * the prefill of a prompt appended to a conversation, for constant-memory
 * generation: de section 2 item 1, section 4 "Effizienz").  The segment's
 * L tokens sit at positions P .. P + L - 1 of a sequence whose first P
 * tokens were processed before (P is not passed: nothing depends on it
 * beyond the state and the halo).
 *   log_g, gate_logit   the gates, as in lizard_attn_fwd or
 *               lizard_attn_fwd_logit: exactly one of the two is non-NULL
 *               (both non-NULL: LIZARD_E_SHAPE)
 *   state_in    [B, H, dk, dv]  float32, nullable: S_{P-1}, the state_out of
 *               the previous segment (NULL: zero, a sequence that starts here)
 *   k_halo      [B, H, halo_len, dk] dtype: keys of positions P - halo_len ..
 *               P - 1, the window's reach into the previous segment
 *   v_halo      [B, H, halo_len, dv] dtype: their values
 *   halo_len    0 <= halo_len <= window - 1; min(window - 1, P) reproduces the
 *               single-call result (k_halo / v_halo may be NULL when 0)
 * Every other argument as lizard_attn_fwd.  y, lse, y_anchor and state_out
 * equal those rows of one lizard_attn_fwd call over all P + L tokens. */
lizard_status_t lizard_attn_fwd_continue(const lizard_params_t* p,
                                         const void* q, const void* k, const void* v,
                                         const float* log_g, const void* gate_logit,
                                         const void* meta_k, const float* state_in,
                                         const void* k_halo, const void* v_halo, int32_t halo_len,
                                         void* y, float* lse, void* y_anchor, float* state_out,
                                         void* stream);

/* lizard_attn_fwd_continue for few heads over long sequences (long-context
 * prefill, de section 4 "Ergebnisse", "Effizienz": the throughput has to
 * hold over 32K-token contexts).  One head's sequence is a chain of chunks,
 * so a one-pass forward runs only B*H*(dv/64) workgroups however long L is.
 * The recurrence of de section 2 "Kernkomponenten" item 1 is linear in the
 * state, so this call cuts each sequence into segments run side by side from
 * a zero state, then a scan chains the segments' final states and each
 * output row of a later segment gets the term its incoming state adds.
 *   workspace   device memory of workspace_bytes >=
 *               lizard_attn_fwd_split_workspace_size(p), 16-byte aligned,
 *               caller-owned; may be NULL when that size is 0 (then the call
 *               runs as one pass).  Contents on entry are ignored.
 * Every other argument, and every result, as lizard_attn_fwd_continue; the
 * results equal its results up to float rounding (the split adds a second
 * rounding of y to the element type, and terms carried over a decay below
 * 2^-128 of a later segment's incoming state are dropped, gates being at
 * most one).  Returns LIZARD_E_WORKSPACE when the workspace is missing or
 * too small. */
size_t lizard_attn_fwd_split_workspace_size(const lizard_params_t* p);
lizard_status_t lizard_attn_fwd_split(const lizard_params_t* p,
                                      const void* q, const void* k, const void* v,
                                      const float* log_g, const void* gate_logit,
                                      const void* meta_k, const float* state_in,
                                      const void* k_halo, const void* v_halo, int32_t halo_len,
                                      void* y, float* lse, void* y_anchor, float* state_out,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* ---- The split forward without allocation ------------------------------
 *
 * For callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, serving loops and harnesses that forbid
 * hipMalloc.  lizard_attn_fwd_split with its workspace taken from a fixed
 * array of LIZARD_NOALLOC_SCRATCH_BYTES inside the library (one copy per GPU,
 * held until the process ends); the call itself allocates nothing.
 *   Arguments and results are those of lizard_attn_fwd_split without
 *   workspace / workspace_bytes, bit for bit.
 *   Sizes whose workspace (lizard_attn_fwd_split_workspace_size) exceeds
 *   LIZARD_NOALLOC_SCRATCH_BYTES return LIZARD_E_WORKSPACE before anything is
 *   launched (a 32-head, 32K-token bfloat16 prefill needs about 21 MB).
 *   Every call on a GPU uses that GPU's one array: calls that may run at the
 *   same time on one GPU (different streams, or host threads) race on it and
 *   must be ordered by the caller.  The array keeps the last call's contents;
 *   no call depends on them. */
#define LIZARD_NOALLOC_SCRATCH_BYTES (64u << 20)
lizard_status_t lizard_attn_fwd_split_noalloc(const lizard_params_t* p,
                                              const void* q, const void* k, const void* v,
                                              const float* log_g, const void* gate_logit,
                                              const void* meta_k, const float* state_in,
                                              const void* k_halo, const void* v_halo, int32_t halo_len,
                                              void* y, float* lse, void* y_anchor, float* state_out,
                                              void* stream);

/* ---- Training: the forward pass keeps the states the backward needs ----
 *
 * The layer is trained end to end (de section 2 "Trainingsprozess"), so the
 * backward pass follows a forward pass over the same inputs.  The backward
 * needs the state at the start of every 64-token chunk; lizard_attn_bwd
 * recomputes them in a pass of its own, while these calls let the forward
 * pass write them as it goes and the backward read them.
 *
 * Bytes of the chunk-start states for these sizes: B*H*ceil(L/64)*dk*dv
 * elements of the element type (0 on invalid sizes). */
size_t lizard_attn_chunk_states_size(const lizard_params_t* p);

/* lizard_attn_fwd (log_g non-NULL) or lizard_attn_fwd_logit (gate_logit
 * non-NULL; both non-NULL: LIZARD_E_SHAPE), which also writes
 *   chunk_states  [B, H, ceil(L/64), dk, dv] dtype, out, 16-byte aligned:
 *                 the state S before the first token of each chunk (zero
 *                 for chunk 0), rounded to dtype
 * Every other argument and result as lizard_attn_fwd; y, lse, y_anchor and
 * state_out are bit for bit those of lizard_attn_fwd.  chunk_states NULL with
 * B*H*L > 0: LIZARD_E_NULL. */
lizard_status_t lizard_attn_fwd_train(const lizard_params_t* p,
                                      const void* q, const void* k, const void* v,
                                      const float* log_g, const void* gate_logit,
                                      const void* meta_k, void* y, float* lse,
                                      void* y_anchor, float* state_out,
                                      void* chunk_states, void* stream);

/* lizard_attn_bwd (log_g non-NULL; dgate is float* dlog_g [B, H, L, dk]) or
 * lizard_attn_bwd_logit (gate_logit non-NULL; dgate is the dtype gradient of
 * the logits), reading the chunk-start states lizard_attn_fwd_train wrote
 * for the same q, k, v, gates and sizes instead of recomputing them:
 *   chunk_states  [B, H, ceil(L/64), dk, dv] dtype, in, 16-byte aligned
 * Every other argument, the workspace (lizard_attn_bwd_workspace_size) and
 * every result as lizard_attn_bwd; the results are those of lizard_attn_bwd
 * (at float32 up to the last bits of the carried state's rounding).
 * chunk_states NULL with B*H*L > 0: LIZARD_E_NULL. */
lizard_status_t lizard_attn_bwd_train(const lizard_params_t* p,
                                      const void* q, const void* k, const void* v,
                                      const float* log_g, const void* gate_logit,
                                      const void* meta_k, const float* lse,
                                      const void* chunk_states, const void* dy,
                                      void* dq, void* dk, void* dv, void* dgate,
                                      float* dmeta_k, void* workspace,
                                      size_t workspace_bytes, void* stream);

/* Serving form of the decode step (constant-memory generation for a batch
 * of sequences, de section 2 item 1 and section 4 "Effizienz"): T >= 1 new
 * tokens per row, appended in order, each batch row at its own position.
 *   pos         [B] int64, DEVICE pointer, 8-byte aligned: absolute position
 *               of row b's first new token (its tokens take positions
 *               pos[b] .. pos[b] + T - 1).  A negative value leaves row b
 *               untouched: nothing of it is read or written, its y rows keep
 *               their contents (padding slots of a continuous batch).
 *   T           new tokens per row, 1 <= T <= 65536
 *   q, k        [B, H, T, dk]   dtype
 *   v           [B, H, T, dv]   dtype
 *   log_g       [B, H, T, dk]   float32
 *   y           [B, H, T, dv]   dtype, out
 *   meta_k, state, k_ring, v_ring   as in lizard_decode_step
 * Equal to T successive lizard_decode_step calls per row; the state is read
 * and written once per call instead of once per token.  The positions are
 * read on the device, so a caller never synchronises to pass them. */
lizard_status_t lizard_decode_tokens(const lizard_params_t* p, const int64_t* pos, int32_t T,
                                     const void* q, const void* k, const void* v,
                                     const float* log_g, const void* meta_k,
                                     float* state, void* k_ring, void* v_ring,
                                     void* y, void* stream);

/* ---- The same calls with the gate given by its logits ------------------
 *
 * The gate is a sigmoid of a learned projection of the token, Gamma =
 * sigmoid(W_gamma x) (de section 2 "Kernkomponenten" item 1; it section 2
 * "Architettura Ibrida").  These entry points take that projection's output
 * x directly and compute log_g = log(sigmoid(x)) inside the kernels (and,
 * in the backward pass, the gradient w.r.t. x = dlog_g * sigmoid(-x)), so
 * the float32 log-gate never makes a round trip through memory.
 *   gate_logit    [B, H, L, dk] dtype (decode: [B, H, dk], [B, H, T, dk]);
 *                 any finite value
 *   dgate_logit   [B, H, L, dk] dtype, out
 * Every other argument, the workspace size and the error behaviour are those
 * of the log-gate calls above; the results equal theirs for log_g =
 * log(sigmoid(gate_logit)) evaluated in float32. */
lizard_status_t lizard_attn_fwd_logit(const lizard_params_t* p,
                                      const void* q, const void* k, const void* v,
                                      const void* gate_logit, const void* meta_k,
                                      void* y, float* lse, void* y_anchor, float* state_out,
                                      void* stream);

lizard_status_t lizard_attn_bwd_logit(const lizard_params_t* p,
                                      const void* q, const void* k, const void* v,
                                      const void* gate_logit, const void* meta_k,
                                      const float* lse, const void* dy,
                                      void* dq, void* dk, void* dv, void* dgate_logit, float* dmeta_k,
                                      void* workspace, size_t workspace_bytes,
                                      void* stream);

lizard_status_t lizard_decode_step_logit(const lizard_params_t* p, int64_t pos,
                                         const void* q_t, const void* k_t, const void* v_t,
                                         const void* gate_logit_t, const void* meta_k,
                                         float* state, void* k_ring, void* v_ring,
                                         void* y_t, void* stream);

lizard_status_t lizard_decode_tokens_logit(const lizard_params_t* p, const int64_t* pos, int32_t T,
                                           const void* q, const void* k, const void* v,
                                           const void* gate_logit, const void* meta_k,
                                           float* state, void* k_ring, void* v_ring,
                                           void* y, void* stream);

/* ---- Stage-1 attention transfer --------------------------------------
 *
 * The layer is trained in two stages; the first fits it to reproduce the
 * outputs of the softmax attention it replaces, on the same q, k, v (de
 * section 2 "Trainingsprozess"; it section 2 "Fase di Addestramento").  One
 * step: lizard_softmax_attn_fwd (the teacher), lizard_attn_fwd (need lse),
 * lizard_transfer_loss (dy), lizard_attn_bwd.
 *
 * Causal softmax attention over every earlier token, the teacher:
 *   y_t = sum_{s <= t} softmax_s(scale * q_t . k_s) v_s
 *   q, k, v     [B, H, L, dk]   dtype (p->window, n_meta, alpha are ignored)
 *   y           [B, H, L, dv]   dtype, out
 *   lse         [B, H, L]       float32, out, nullable: natural-log normaliser */
lizard_status_t lizard_softmax_attn_fwd(const lizard_params_t* p,
                                        const void* q, const void* k, const void* v,
                                        void* y, float* lse, void* stream);

/* The output-matching loss mean((y - y_teacher)^2) over all B*H*L*dv
 * elements and its gradient.
 *   y, y_teacher [B, H, L, dv]  dtype
 *   dy          [B, H, L, dv]   dtype, out: 2 (y - y_teacher) / N
 *   loss_bh     [B, H]          float32, out: each head's sum of squared
 *                               errors / N, summed in a fixed order (the loss
 *                               is the sum of loss_bh; deterministic) */
lizard_status_t lizard_transfer_loss(const lizard_params_t* p,
                                     const void* y, const void* y_teacher,
                                     void* dy, float* loss_bh, void* stream);

/* Static description of a status code. */
const char* lizard_status_string(lizard_status_t s);

/* ABI version of this header: 4 (version 3 had no lizard_attn_fwd_train,
 * lizard_attn_bwd_train or lizard_attn_chunk_states_size; version 2 had no
 * lizard_attn_fwd_split;
 * version 1 had none of the *_logit, lizard_attn_fwd_continue,
 * lizard_decode_tokens, lizard_softmax_attn_fwd and lizard_transfer_loss
 * entry points). */
int lizard_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIZARD_ATTN_H */
