/*
 * rat.h -- C ABI of the RAT+ layer hot path on AMD Instinct MI355X (gfx950).
 *
 * The RAT+ layer ("RAT+: Train Dense, Infer Sparse -- Recurrence Augmented
 * Attention for Dilated Inference", arXiv 2602.18196, Abstract; "RAT+ Deep
 * Dive: A New KV Cache Compression Paradigm with Dense Pretraining and
 * Dilated Inference", zhichai.net, sections 1, 2.1 and 6) has two stages:
 *
 *   1. a gated linear recurrence over keys and values,
 *        h_t = g_t * h_{t-1} + (1 - g_t) * x_t,   g_t = sigmoid(logit_t),
 *      computed for prefill as a parallel scan (Deep Dive 2.1, 7.3), over
 *      the whole sequence or a recurrence window of L tokens;
 *   2. causal dilated softmax attention: the query at position t attends to
 *      the recurrent states at t, t-D, t-2D, ... and, optionally, to the raw
 *      keys/values of the last W tokens (RAT+ Abstract: "dilated attention
 *      (optionally with local windows)"), with a per-head (D, W) so that
 *      dense and dilated heads mix in one layer (Deep Dive 6, Head-Wise
 *      Hybrid).  Decode reads a KV cache that is D times smaller (Abstract).
 *
 * Common conventions
 *  - Every tensor pointer is a DEVICE pointer owned by the caller; the
 *    library never allocates or frees device memory and keeps no pointer
 *    after a call returns.  Host arrays (D, W) are read during the call only.
 *  - Prefill tensors are [B, T, H, d] contiguous (d fastest).  Decode query
 *    and output are [B, H, d]; decode caches are [B, H, N, d].
 *  - dtype: RAT_DTYPE_F32 (float) or RAT_DTYPE_BF16 (bfloat16, round to
 *    nearest even on output).  All arithmetic is fp32.
 *  - Supported head size d: 64 or 128.  Every pointer must be 16-byte
 *    aligned.  B*T*H*d must be below 2^31; for decode caches, B*H*d and
 *    N*d (one head's rows) must be, the whole cache need not.
 *  - Every call only enqueues work on `stream` (a hipStream_t, may be NULL
 *    for the default stream) and returns without synchronising.
 *  - All validation happens on the host before any HIP call: on an error
 *    nothing is enqueued and no output is touched.  RAT_ERR_HIP reports a
 *    failed launch (outputs undefined); rat_last_hip_error() then returns
 *    the hipError_t of the calling thread's last failure.
 *  - No call prints, aborts or throws.  Calls are re-entrant; concurrent
 *    calls must not share a workspace.
 */
#ifndef RAT_H
#define RAT_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { RAT_DTYPE_F32 = 0, RAT_DTYPE_BF16 = 1 } rat_dtype;

/* Meaning of a recurrence window L < T (Deep Dive 2.1 gives a fixed window of
 * L* = 64 tokens "looking back" from the current one; the layer is also
 * described as restarting every L* tokens).  Both readings are offered:
 *   RESTART: the state is cleared at every position t with t mod L == 0;
 *   SLIDING: h_t sums exactly the last L inputs (requires L <= 64).
 * With L >= T both modes are the full-sequence recurrence (Deep Dive 2.1). */
typedef enum { RAT_RECUR_RESTART = 0, RAT_RECUR_SLIDING = 1 } rat_recur_mode;

typedef enum {
    RAT_OK = 0,
    RAT_ERR_NULL = 1,        /* a required pointer is NULL */
    RAT_ERR_SHAPE = 2,       /* a size or per-head parameter is out of range */
    RAT_ERR_UNSUPPORTED = 3, /* valid but not implemented (d, dtype, L, sizes) */
    RAT_ERR_ALIAS = 4,       /* an output aliases an input */
    RAT_ERR_WORKSPACE = 5,   /* workspace missing, too small or misaligned */
    RAT_ERR_HIP = 6,         /* a HIP launch failed */
    RAT_ERR_ALIGN = 7        /* a tensor pointer is not 16-byte aligned */
} rat_status;

/* Bytes of device workspace rat_scan_prefill needs for these sizes (0 when
 * none).  The workspace carries the cross-workgroup carries of the parallel
 * scan; it must be 256-byte aligned and ZERO-FILLED BEFORE ITS FIRST USE,
 * after which the library keeps it consistent by itself (it is reusable by
 * later scan calls of any size up to its capacity, one stream at a time). */
size_t rat_scan_workspace_bytes(int B, int T, int H, int d, int L,
                                rat_recur_mode mode, rat_dtype dtype);

/* Stage 1 (Deep Dive 2.1): recurrent key and value states.
 *   k, v, gate_logits : [B,T,H,d] inputs; the forget gate is
 *                       g = sigmoid(gate_logits), elementwise, shared by
 *                       keys and values; logits of +-inf are allowed.
 *   k_state, v_state  : [B,T,H,d] outputs,
 *                       k_state[t] = g_t*k_state[t-1] + (1-g_t)*k[t], state
 *                       zero before t = 0 (and at RESTART boundaries).
 *   L                 : recurrence window, >= 1; L >= T means full sequence.
 *   final_state       : optional (NULL for none) fp32 [B,H,2,d] output: the
 *                       key and value states at t = T-1 before rounding to
 *                       dtype, from which rat_decode_step continues.  Not
 *                       available for SLIDING with L < T (RAT_ERR_UNSUPPORTED).
 * Errors: RAT_ERR_NULL, _SHAPE (B,T,H,d,L < 1), _UNSUPPORTED (d, dtype,
 * SLIDING with 64 < L < T, sizes), _ALIAS, _ALIGN, _WORKSPACE, _HIP. */
rat_status rat_scan_prefill(const void* k, const void* v, const void* gate_logits,
                     void* k_state, void* v_state,
                     int B, int T, int H, int d, int L, rat_recur_mode mode,
                     rat_dtype dtype, void* workspace, size_t workspace_bytes,
                     float* final_state, void* stream);

/* Bytes of device workspace rat_dilated_attn_prefill needs (0 when no head
 * has a local window, or for fp32): B*T*H*2 floats holding the partial
 * softmax state of the window pass.  16-byte aligned; no initialisation. */
size_t rat_attn_prefill_workspace_bytes(int B, int T, int H, int d, const int* D, const int* W,
                                        rat_dtype dtype);

/* Stage 2, prefill (RAT+ Abstract; Deep Dive 1 and 6): for every query
 * (b, t, h) one softmax over
 *   the recurrent states  k_state/v_state at t, t-D[h], t-2D[h], ... >= 0,
 *   then the raw tokens   k_raw/v_raw     at t, t-1, ..., t-W[h]+1 >= 0,
 * with logits scale * <q, key>; out = sum softmax * value.
 *   q, k_state, v_state, k_raw, v_raw, out : [B,T,H,d];
 *   k_raw / v_raw may be NULL iff every W[h] == 0;
 *   D, W : host int[H], D[h] >= 1, W[h] >= 0 (D[h] = 1, W[h] = 0 is dense
 *          causal attention over the states);
 *   workspace : at least rat_attn_prefill_workspace_bytes(...) bytes, may
 *          be NULL when that is 0.  Calls in flight must not share it.
 * Errors: RAT_ERR_NULL, _SHAPE, _UNSUPPORTED, _ALIAS, _ALIGN, _WORKSPACE, _HIP. */
rat_status rat_dilated_attn_prefill(const void* q, const void* k_state, const void* v_state,
                             const void* k_raw, const void* v_raw, void* out,
                             int B, int T, int H, int d, const int* D, const int* W,
                             float scale, rat_dtype dtype,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Stage 2, prefill, on the chunk grid -- the absolute reading of the
 * dilated pattern, after the RAT page ("RAT: Bridging RNN Efficiency and
 * Attention Accuracy via Chunk-based Sequence Modeling", Abstract: the
 * sequence is split into chunks and attention runs across chunks): with
 * chunks of D[h] tokens, the query at position t attends in one softmax to
 * the recurrent states that end a chunk before it (positions c*D[h] - 1 < t)
 * and to its own state at t.  A decode cache under this reading holds the
 * chunk ends plus the current state, which rat_dilated_attn_decode reads
 * as its dilated cache unchanged (ceil(T/D) entries).
 *   q, k_state, v_state, out : [B,T,H,d];
 *   D : host int[H], D[h] >= 1 (D[h] = 1 is dense causal attention);
 *       at most 8 distinct values.
 * No raw local window, no workspace.  Errors: RAT_ERR_NULL, _SHAPE,
 * _UNSUPPORTED, _ALIAS, _ALIGN, _HIP. */
rat_status rat_chunk_attn_prefill(const void* q, const void* k_state, const void* v_state, void* out,
                           int B, int T, int H, int d, const int* D, float scale, rat_dtype dtype,
                           void* stream);

/* Bytes of device workspace rat_dilated_attn_decode needs (0 when none; it
 * holds split-key partial softmax states when B*H is small). 256-byte
 * aligned; no initialisation needed. */
size_t rat_decode_workspace_bytes(int B, int H, int d, int T, const int* D, const int* W);

/* Stage 2, decode (RAT+ Abstract: the KV cache holds T/D states per head):
 * one new query per sequence at position T-1 of a T-token context.
 *   q, out   : [B,H,d];
 *   kd, vd   : [B,H,nd_cap,d] dilated cache of head h, entry i = recurrent
 *              state at position ((T-1) mod D[h]) + i*D[h], for
 *              i = 0 .. ceil(T/D[h])-1 (the last entry is the query's own
 *              state); nd_cap >= ceil(T/D[h]) for every h;
 *   kw, vw   : [B,H,w_cap,d] raw ring of the last min(W[h], T) tokens in
 *              slots 0 .. min(W[h],T)-1, in any order; may be NULL iff every
 *              W[h] == 0; w_cap >= min(W[h], T).
 * Errors: RAT_ERR_NULL, _SHAPE, _UNSUPPORTED, _ALIAS, _ALIGN, _WORKSPACE, _HIP. */
rat_status rat_dilated_attn_decode(const void* q, const void* kd, const void* vd, int nd_cap,
                            const void* kw, const void* vw, int w_cap, void* out,
                            int B, int T, int H, int d, const int* D, const int* W,
                            float scale, rat_dtype dtype,
                            void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the decode
 * attention of rat_dilated_attn_decode, same arguments and results, without
 * a workspace.  Its split-key partials live in a static scratch array of
 * rat_decode_static_scratch_bytes() bytes (1 MiB) that the library defines
 * once per GPU and holds until the process ends; the call allocates and
 * frees nothing.  Every call on one GPU shares that GPU's array, so calls
 * that overlap in time on one GPU (two streams, two threads) race: order
 * them.  Nothing in the array needs to start at zero.  The partials need
 * B*H*nsplit*(d+2)*4 bytes with B*H*nsplit below 1024, so every valid call
 * fits; a call that would not returns RAT_ERR_WORKSPACE before launching.
 * Errors: as rat_dilated_attn_decode (RAT_ERR_WORKSPACE only as above). */
size_t rat_decode_static_scratch_bytes(void);
rat_status rat_dilated_attn_decode_static(const void* q, const void* kd, const void* vd, int nd_cap,
                                          const void* kw, const void* vw, int w_cap, void* out,
                                          int B, int T, int H, int d, const int* D, const int* W,
                                          float scale, rat_dtype dtype, void* stream);

/* One step of a decode loop (the recurrence of Deep Dive 2.1 for one new
 * token, then the decode attention above): the token at position T-1 of a
 * T-token context arrives with its query q, raw key / value k_new, v_new
 * and gate logit gate_new ([B,H,d] each).
 *   state  : fp32 [B,H,2,d], in: the key and value states at T-2 (zeros
 *            for T = 1, or rat_scan_prefill's final_state), out: the states
 *            at T-1.  With L < T the state is cleared first when (T-1) mod
 *            L == 0 (RESTART); SLIDING windows have their own step,
 *            rat_decode_step_sliding.
 *   kc, vc : [B,H,n_cap,d] history of the states, kept per residue: the
 *            state of position p of head h is row
 *            (p mod D[h]) * (n_cap / D[h]) + p / D[h], so that the entries a
 *            query reads -- its own residue's -- are contiguous; this call
 *            writes the row of position T-1 and needs
 *            (T-1) / D[h] < n_cap / D[h].
 *   kw, vw : [B,H,w_cap,d] ring of raw keys / values, position p in slot
 *            p mod W[h] (w_cap >= W[h]); this call writes slot (T-1) mod W[h].
 *            May be NULL iff every W[h] == 0.
 *   out    : [B,H,d], as rat_dilated_attn_decode at context T over the
 *            residue rows and ring slots above.
 *   workspace: rat_decode_workspace_bytes(B, H, d, T, D, W) bytes.
 * Errors: RAT_ERR_NULL, _SHAPE, _UNSUPPORTED, _ALIAS, _ALIGN, _WORKSPACE, _HIP. */
rat_status rat_decode_step(const void* q, const void* k_new, const void* v_new, const void* gate_new,
                    float* state, void* kc, void* vc, int n_cap, void* kw, void* vw, int w_cap,
                    void* out, int B, int T, int H, int d, int L, const int* D, const int* W,
                    float scale, rat_dtype dtype, void* workspace, size_t workspace_bytes,
                    void* stream);

/* One step of a decode loop under a SLIDING recurrence window of L tokens
 * (Deep Dive 2.1: a fixed window that looks back L* = 64 tokens; SLIDING in
 * rat_scan_prefill), then the decode attention above.  Such a window keeps
 * no single running state: the state at position p sums exactly the gated
 * inputs of positions max(0, p-L+1) .. p, so the loop keeps those positions'
 * raw inputs and runs the recurrence from a zero state over them.
 *   q, k_new, v_new, gate_new : [B,H,d], the token at position T-1;
 *   rk, rv, rg : [B,H,L,d] ring of the raw key, value and gate logit of the
 *            last L positions, position p in slot p mod L; in: positions
 *            max(0, T-L) .. T-2 (rat_sliding_state_from_prefill after a
 *            prefill, nothing before the first token); this call writes
 *            the new token into slot (T-1) mod L;  1 <= L <= 1024;
 *   kc, vc, n_cap, kw, vw, w_cap, out, D, W, scale, workspace : as
 *            rat_decode_step (the new state goes to the history row of
 *            position T-1, the raw token to ring slot (T-1) mod W[h]).
 * Errors: RAT_ERR_NULL, _SHAPE, _UNSUPPORTED (L > 1024, d, dtype, sizes),
 * _ALIAS, _ALIGN, _WORKSPACE, _HIP. */
rat_status rat_decode_step_sliding(const void* q, const void* k_new, const void* v_new, const void* gate_new,
                                   void* rk, void* rv, void* rg, int L,
                                   void* kc, void* vc, int n_cap, void* kw, void* vw, int w_cap,
                                   void* out, int B, int T, int H, int d, const int* D, const int* W,
                                   float scale, rat_dtype dtype, void* workspace, size_t workspace_bytes,
                                   void* stream);

/* The SLIDING decode state of a finished prefill (what rat_decode_step_sliding
 * continues from): the raw key, value and gate logit of positions
 * max(0, T-L) .. T-1 of k, v, gate_logits ([B,T,H,d]) into slot p mod L of
 * rk, rv, rg ([B,H,L,d]); slots with no such position are left alone.
 * 1 <= L <= 1024.  Errors: RAT_ERR_NULL, _SHAPE, _UNSUPPORTED, _ALIAS,
 * _ALIGN, _HIP. */
rat_status rat_sliding_state_from_prefill(const void* k, const void* v, const void* gate_logits,
                                          void* rk, void* rv, void* rg, int B, int T, int H, int d, int L,
                                          rat_dtype dtype, void* stream);

/* The whole prefill of the layer in one call, handing a decode loop its
 * caches: the recurrence of rat_scan_prefill (Deep Dive 2.1), then the
 * attention of rat_dilated_attn_prefill (RAT+ Abstract; Deep Dive 1 and 6),
 * with the states written once, straight into the per-residue history that
 * rat_decode_step reads and extends (the decode cache of the RAT+ Abstract).
 *   q, k, v, gate_logits : [B,T,H,d] inputs; out : [B,T,H,d], equal to
 *            rat_dilated_attn_prefill over rat_scan_prefill's states with
 *            k_raw = k, v_raw = v;
 *   kc, vc : [B,H,n_cap,d] state history, layout as for rat_decode_step:
 *            position p of head h at row (p mod D[h]) * (n_cap / D[h]) +
 *            p / D[h]; rows of positions 0 .. T-1 are written, others left
 *            alone.  (T-1) / D[h] < n_cap / D[h] for every h; B*H*n_cap*d
 *            must be below 2^31.  A decode loop can continue at T+1 when
 *            T / D[h] < n_cap / D[h] as well;
 *   kw, vw : [B,H,w_cap,d] ring, slot p mod W[h] holding raw k, v of the
 *            last W[h] positions p < T (slots with no such position, and
 *            slots >= W[h], left alone); w_cap >= W[h]; may be NULL iff
 *            every W[h] == 0;
 *   final_state : optional fp32 [B,H,2,d], as in rat_scan_prefill (not for
 *            SLIDING with L < T);
 *   L, mode : as rat_scan_prefill;  D, W, scale : as rat_dilated_attn_prefill;
 *   scan_workspace : rat_scan_workspace_bytes(...) bytes, the same
 *            zero-filled-once buffer rules as rat_scan_prefill;
 *   attn_workspace : rat_attn_prefill_workspace_bytes(...) bytes.
 * Errors: RAT_ERR_NULL, _SHAPE, _UNSUPPORTED, _ALIAS, _ALIGN, _WORKSPACE, _HIP. */
rat_status rat_layer_prefill(const void* q, const void* k, const void* v, const void* gate_logits,
                      void* out, void* kc, void* vc, int n_cap, void* kw, void* vw, int w_cap,
                      float* final_state, int B, int T, int H, int d, int L, rat_recur_mode mode,
                      const int* D, const int* W, float scale, rat_dtype dtype,
                      void* scan_workspace, size_t scan_workspace_bytes,
                      void* attn_workspace, size_t attn_workspace_bytes, void* stream);

/* The decode caches of a finished prefill, for a decode loop to continue
 * from (the decode cache of the RAT+ Abstract, kept per residue as
 * rat_decode_step reads and extends it): copies the states rat_scan_prefill
 * wrote and the raw tokens of the last W[h] positions.
 *   k_state, v_state : [B,T,H,d] prefill states;  k, v : [B,T,H,d] raw
 *            inputs (may be NULL iff every W[h] == 0);
 *   kc, vc : [B,H,n_cap,d] history: position p of head h to row
 *            (p mod D[h]) * (n_cap / D[h]) + p / D[h] for p < T, other rows
 *            left alone; (T-1) / D[h] < n_cap / D[h];
 *   kw, vw : [B,H,w_cap,d] ring: position p of the last W[h] to slot
 *            p mod W[h], other slots left alone; w_cap >= W[h]; may be NULL
 *            iff every W[h] == 0.
 * The fp32 running state for the loop is rat_scan_prefill's final_state.
 * Errors: RAT_ERR_NULL, _SHAPE, _UNSUPPORTED, _ALIAS, _ALIGN, _HIP. */
rat_status rat_build_decode_caches(const void* k_state, const void* v_state, const void* k, const void* v,
                            void* kc, void* vc, int n_cap, void* kw, void* vw, int w_cap,
                            int B, int T, int H, int d, const int* D, const int* W, rat_dtype dtype,
                            void* stream);

/* Bytes of device workspace rat_layer_backward needs: per query row the
 * log-sum-exp, dout.out and the raw window's partial softmax sums, the fp32
 * gradients of the states, and per 16-token chunk of every channel its
 * recurrence maps and carries.  256-byte aligned; no initialisation. */
size_t rat_layer_backward_workspace_bytes(int B, int T, int H, int d);

/* Backward of the layer (the training of Deep Dive 2.2, Active Recurrence
 * Learning, differentiates the forward of rat_scan_prefill and
 * rat_dilated_attn_prefill; there the recurrence runs over the full
 * sequence): given dout = dLoss/dout, the gradients of the loss with
 * respect to q, k, v and the gate logits, by the chain rule through the
 * one-softmax attention (states at t, t-D, ... and raw tokens t .. t-W+1)
 * and then through the recurrence h_t = g_t h_{t-1} + (1 - g_t) x_t walked
 * backwards (dk and dv sum the state path and the raw-window path).
 *   q, k, v, gate_logits : [B,T,H,d] forward inputs;
 *   k_state, v_state     : [B,T,H,d] forward states (rat_scan_prefill);
 *   dout                 : [B,T,H,d] incoming gradient;  all in `dtype`.
 *                          The softmax is recomputed in fp32, and the
 *                          row term <dout_t, out_t> is formed from it, so
 *                          the forward output is not an input;
 *   dq, dk, dv, dgate    : [B,T,H,d] fp32 outputs;
 *   L, mode              : the forward's recurrence: full (L >= T),
 *                          RESTART, or a SLIDING window of L tokens (each
 *                          state its own window, the gradients summed over
 *                          the windows that hold a token);
 *   D, W, scale          : as rat_dilated_attn_prefill;
 *   workspace            : rat_layer_backward_workspace_bytes(...) bytes.
 * Errors: RAT_ERR_NULL, _SHAPE, _UNSUPPORTED, _ALIAS, _ALIGN, _WORKSPACE, _HIP. */
rat_status rat_layer_backward(const void* q, const void* k, const void* v, const void* gate_logits,
                       const void* k_state, const void* v_state, const void* dout,
                       float* dq, float* dk, float* dv, float* dgate,
                       int B, int T, int H, int d, int L, rat_recur_mode mode,
                       const int* D, const int* W, float scale, rat_dtype dtype,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Static text for a status code. */
const char* rat_status_string(rat_status status);

/* hipError_t of the calling thread's last RAT_ERR_HIP (0 if none). */
int rat_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RAT_H */
