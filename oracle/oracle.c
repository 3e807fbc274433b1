/*
 * oracle.c -- plain, slow, obviously correct CPU reference for the RAT+ layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the GPU library: it is built by the host C
 * compiler from this one file, with no HIP include path.
 *
 * Everything is computed in IEEE double precision from the caller's inputs
 * (which are bf16 or fp32 values, hence exact in double).  No blocking, no
 * reassociation beyond what the definitions below state.
 *
 * Sources (the pages):
 *   [RAT+ abstract]  "RAT+: Train Dense, Infer Sparse -- Recurrence Augmented
 *                    Attention for Dilated Inference", arXiv 2602.18196,
 *                    Abstract: dilated attention with dilation D, optional
 *                    local windows, full-sequence recurrence; attention FLOPs
 *                    and KV cache fall by a factor D.
 *   [Deep Dive]      "RAT+ Deep Dive: A New KV Cache Compression Paradigm with
 *                    Dense Pretraining and Dilated Inference" (zhichai.net):
 *                    S1 (tokens skip a fixed interval), S2.1 (forget-gate
 *                    recurrence; window L*=64 looking back 64 tokens; L=T),
 *                    S3.1 table (FLOPs T/D), S6 Head-Wise Hybrid table.
 *
 * Readings taken where the pages are silent or garbled (the recurrence
 * equation itself is missing from the Deep Dive S2.1 text):
 *   - h_t = g_t * h_{t-1} + (1 - g_t) * x_t, elementwise per channel, with
 *     g_t = sigmoid(logit_t) and 1 - g_t computed as sigmoid(-logit_t);
 *     one gate per (b, t, h, channel), shared by keys and values; h_{-1} = 0.
 *   - Window L < T, mode RESTART: the state restarts (h := 0 before the
 *     update) at every position t with t mod L == 0.
 *   - Window L < T, mode SLIDING: h_t sums exactly the last L inputs,
 *     h_t = sum_{s=max(0,t-L+1)}^{t} (prod_{r=s+1}^{t} g_r) (1-g_s) x_s.
 *   - L >= T: full-sequence recurrence in either mode.
 *   - Query t of a head with dilation D and window W attends to the
 *     recurrent states at t, t-D, t-2D, ... (>= 0) and to the raw keys and
 *     values at t, t-1, ..., t-W+1 (>= 0), all in ONE softmax with logits
 *     scale * <q_t, key>.  No de-duplication between the two lists.
 *   - Chunk grid (the absolute reading, after the RAT page: "RAT:
 *     Bridging RNN Efficiency and Attention Accuracy via Chunk-based
 *     Sequence Modeling", Abstract -- the input is split into chunks and
 *     attention runs across chunks): with chunks of D tokens, query t
 *     attends to the states that end a chunk before it, at positions
 *     p = cD - 1 < t (c >= 1), and to its own state at t; no raw window.
 *   - Decode at context length T: the single query is position T-1; its
 *     dilated cache entry i holds position ((T-1) mod D) + i*D for
 *     i = 0 .. ceil(T/D)-1, and ring slots 0 .. min(W,T)-1 are valid.
 *
 * Layouts: prefill tensors are [B,T,H,d] row-major (d fastest); decode query
 * and output [B,H,d]; decode caches [B,H,N,d].
 *
 * Error behaviour: every entry point returns 0 on success and a negative
 * number on invalid arguments (no output written then).
 */
#include <math.h>
#include <omp.h>
#include <stddef.h>
#include <stdlib.h>

#define ORACLE_MODE_RESTART 0
#define ORACLE_MODE_SLIDING 1

/* Forget gate and its complement [Deep Dive S2.1]: g = 1/(1+e^{-l}),
 * 1-g = 1/(1+e^{l}).  The complement is evaluated on its own so that it does
 * not cancel when g is close to 1; l = +inf gives (1,0), l = -inf gives (0,1). */
static void gate_pair(double logit, double* g, double* gbar)
{
    *g = 1.0 / (1.0 + exp(-logit));
    *gbar = 1.0 / (1.0 + exp(logit));
}

int oracle_gates(const double* logit, double* g, double* gbar, long n)
{
    if (!logit || !g || !gbar || n < 0) return -1;
    for (long i = 0; i < n; ++i) gate_pair(logit[i], &g[i], &gbar[i]);
    return 0;
}

static size_t idx4(int b, int t, int h, int c, int T, int H, int d)
{
    return (((size_t)b * T + t) * H + h) * (size_t)d + c;
}

/* Recurrence over keys and values [Deep Dive S2.1], one channel at a time,
 * as the plain sequential loop (full / RESTART) or the explicit windowed sum
 * (SLIDING).  k, v, logit, k_state, v_state: [B,T,H,d]. */
int oracle_scan(const double* k, const double* v, const double* logit,
                double* k_state, double* v_state,
                int B, int T, int H, int d, int L, int mode)
{
    if (!k || !v || !logit || !k_state || !v_state) return -1;
    if (B <= 0 || T <= 0 || H <= 0 || d <= 0 || L < 1) return -2;
    if (mode != ORACLE_MODE_RESTART && mode != ORACLE_MODE_SLIDING) return -3;
    const int full = (L >= T);
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int c = 0; c < d; ++c) {
                if (full || mode == ORACLE_MODE_RESTART) {
                    double hk = 0.0, hv = 0.0;
                    for (int t = 0; t < T; ++t) {
                        size_t i = idx4(b, t, h, c, T, H, d);
                        double g, gb;
                        gate_pair(logit[i], &g, &gb);
                        if (!full && t % L == 0) { hk = 0.0; hv = 0.0; }
                        hk = g * hk + gb * k[i];
                        hv = g * hv + gb * v[i];
                        k_state[i] = hk;
                        v_state[i] = hv;
                    }
                } else {
                    for (int t = 0; t < T; ++t) {
                        int lo = t - L + 1;
                        if (lo < 0) lo = 0;
                        double hk = 0.0, hv = 0.0, prod = 1.0;
                        for (int s = t; s >= lo; --s) {
                            size_t i = idx4(b, s, h, c, T, H, d);
                            double g, gb;
                            gate_pair(logit[i], &g, &gb);
                            hk += prod * gb * k[i];
                            hv += prod * gb * v[i];
                            prod *= g;
                        }
                        size_t o = idx4(b, t, h, c, T, H, d);
                        k_state[o] = hk;
                        v_state[o] = hv;
                    }
                }
            }
    return 0;
}

/* Index sets of query t [Deep Dive S1; RAT+ abstract]:
 *   dilated  S_dil(t) = { t - j*D : j >= 0, t - j*D >= 0 }   (own state first)
 *   local    S_loc(t) = { t - w   : 0 <= w < W, t - w >= 0 }
 * Writes the positions in that order; returns |S_dil| + |S_loc|.  The
 * arrays must hold t/D + 1 and min(W, t+1) entries. */
long oracle_index_sets(int t, int D, int W, int* dil, int* n_dil, int* loc, int* n_loc)
{
    if (t < 0 || D < 1 || W < 0 || !n_dil || !n_loc) return -1;
    int nd = 0, nl = 0;
    for (int s = t; s >= 0; s -= D) {
        if (dil) dil[nd] = s;
        ++nd;
    }
    for (int w = 0; w < W && t - w >= 0; ++w) {
        if (loc) loc[nl] = t - w;
        ++nl;
    }
    *n_dil = nd;
    *n_loc = nl;
    return (long)nd + nl;
}

/* One softmax over an explicit list of (key, value) rows: logits
 * z_j = scale * <q, key_j>, m = max z, w_j = exp(z_j - m),
 * out = sum_j w_j value_j / sum_j w_j (two passes).  keys/vals are arrays of
 * row pointers (each d doubles).  Returns 0, or -1 for an empty list. */
static int softmax_rows(const double* q, const double* const* keys,
                        const double* const* vals, int n, int d, double scale,
                        double* z, double* out)
{
    if (n <= 0) return -1;
    double m = -INFINITY;
    for (int j = 0; j < n; ++j) {
        double dot = 0.0;
        for (int c = 0; c < d; ++c) dot += q[c] * keys[j][c];
        z[j] = scale * dot;
        if (z[j] > m) m = z[j];
    }
    double den = 0.0;
    for (int c = 0; c < d; ++c) out[c] = 0.0;
    for (int j = 0; j < n; ++j) {
        double w = exp(z[j] - m);
        den += w;
        for (int c = 0; c < d; ++c) out[c] += w * vals[j][c];
    }
    for (int c = 0; c < d; ++c) out[c] /= den;
    return 0;
}

/* Attention for one query (b, t, h) of a prefill [Deep Dive S1, S2.1;
 * RAT+ abstract]: dilated recurrent states then raw local window, one
 * softmax.  k_raw / v_raw may be NULL when W == 0. */
static int attend_one(const double* q, const double* ks, const double* vs,
                      const double* kr, const double* vr, double* out,
                      int b, int t, int h, int T, int H, int d, int D, int W,
                      double scale, const double** kp, const double** vp,
                      double* z)
{
    int n = 0;
    for (int s = t; s >= 0; s -= D) {
        kp[n] = ks + idx4(b, s, h, 0, T, H, d);
        vp[n] = vs + idx4(b, s, h, 0, T, H, d);
        ++n;
    }
    for (int w = 0; w < W && t - w >= 0; ++w) {
        kp[n] = kr + idx4(b, t - w, h, 0, T, H, d);
        vp[n] = vr + idx4(b, t - w, h, 0, T, H, d);
        ++n;
    }
    return softmax_rows(q + idx4(b, t, h, 0, T, H, d), kp, vp, n, d, scale, z,
                        out + idx4(b, t, h, 0, T, H, d));
}

static int check_heads(int H, const int* D, const int* W, int* need_raw, int* max_keys, int T)
{
    *need_raw = 0;
    *max_keys = 0;
    for (int h = 0; h < H; ++h) {
        if (D[h] < 1 || W[h] < 0) return -1;
        if (W[h] > 0) *need_raw = 1;
        int nk = (T - 1) / D[h] + 1 + (W[h] < T ? W[h] : T);
        if (nk > *max_keys) *max_keys = nk;
    }
    return 0;
}

/* Full prefill attention, every query row.  q, k_state, v_state, k_raw,
 * v_raw, out: [B,T,H,d]; D, W: per-head int arrays of length H. */
int oracle_attn_prefill(const double* q, const double* k_state, const double* v_state,
                        const double* k_raw, const double* v_raw, double* out,
                        int B, int T, int H, int d, const int* D, const int* W,
                        double scale)
{
    if (!q || !k_state || !v_state || !out || !D || !W) return -1;
    if (B <= 0 || T <= 0 || H <= 0 || d <= 0) return -2;
    int need_raw, max_keys;
    if (check_heads(H, D, W, &need_raw, &max_keys, T)) return -3;
    if (need_raw && (!k_raw || !v_raw)) return -1;
    int bad = 0;
#pragma omp parallel
    {
        const double** kp = (const double**)malloc(sizeof(double*) * max_keys);
        const double** vp = (const double**)malloc(sizeof(double*) * max_keys);
        double* z = (double*)malloc(sizeof(double) * max_keys);
        if (!kp || !vp || !z) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for collapse(3) schedule(dynamic, 16)
            for (int b = 0; b < B; ++b)
                for (int h = 0; h < H; ++h)
                    for (int t = 0; t < T; ++t)
                        attend_one(q, k_state, v_state, k_raw, v_raw, out, b, t, h,
                                   T, H, d, D[h], W[h], scale, kp, vp, z);
        }
        free(kp);
        free(vp);
        free(z);
    }
    return bad ? -4 : 0;
}

/* Prefill attention for a list of sampled query rows only.  rows holds
 * n triples (b, t, h); out_rows is [n, d]. */
int oracle_attn_prefill_rows(const double* q, const double* k_state, const double* v_state,
                             const double* k_raw, const double* v_raw,
                             const int* rows, int n, double* out_rows,
                             int B, int T, int H, int d, const int* D, const int* W,
                             double scale)
{
    if (!q || !k_state || !v_state || !rows || !out_rows || !D || !W) return -1;
    if (B <= 0 || T <= 0 || H <= 0 || d <= 0 || n < 0) return -2;
    int need_raw, max_keys;
    if (check_heads(H, D, W, &need_raw, &max_keys, T)) return -3;
    if (need_raw && (!k_raw || !v_raw)) return -1;
    for (int i = 0; i < n; ++i) {
        int b = rows[3 * i], t = rows[3 * i + 1], h = rows[3 * i + 2];
        if (b < 0 || b >= B || t < 0 || t >= T || h < 0 || h >= H) return -2;
    }
    int bad = 0;
#pragma omp parallel
    {
        const double** kp = (const double**)malloc(sizeof(double*) * max_keys);
        const double** vp = (const double**)malloc(sizeof(double*) * max_keys);
        double* z = (double*)malloc(sizeof(double) * max_keys);
        double* tmp = (double*)malloc(sizeof(double) * (size_t)d);
        if (!kp || !vp || !z || !tmp) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int i = 0; i < n; ++i) {
                int b = rows[3 * i], t = rows[3 * i + 1], h = rows[3 * i + 2];
                int nk = 0;
                for (int s = t; s >= 0; s -= D[h]) {
                    kp[nk] = k_state + idx4(b, s, h, 0, T, H, d);
                    vp[nk] = v_state + idx4(b, s, h, 0, T, H, d);
                    ++nk;
                }
                for (int w = 0; w < W[h] && t - w >= 0; ++w) {
                    kp[nk] = k_raw + idx4(b, t - w, h, 0, T, H, d);
                    vp[nk] = v_raw + idx4(b, t - w, h, 0, T, H, d);
                    ++nk;
                }
                softmax_rows(q + idx4(b, t, h, 0, T, H, d), kp, vp, nk, d, scale, z, tmp);
                for (int c = 0; c < d; ++c) out_rows[(size_t)i * d + c] = tmp[c];
            }
        }
        free(kp);
        free(vp);
        free(z);
        free(tmp);
    }
    return bad ? -4 : 0;
}

/* Decode attention at context length T [RAT+ abstract: the KV cache holds
 * T/D states per head].  q, out: [B,H,d]; kd, vd: [B,H,nd_cap,d] whose entry
 * i is the recurrent state at position ((T-1) mod D) + i*D; kw, vw:
 * [B,H,w_cap,d] raw ring, slots 0 .. min(W,T)-1 valid, in any order. */
int oracle_attn_decode(const double* q, const double* kd, const double* vd, int nd_cap,
                       const double* kw, const double* vw, int w_cap, double* out,
                       int B, int T, int H, int d, const int* D, const int* W,
                       double scale)
{
    if (!q || !kd || !vd || !out || !D || !W) return -1;
    if (B <= 0 || T <= 0 || H <= 0 || d <= 0 || nd_cap < 0 || w_cap < 0) return -2;
    int max_keys = 0, need_ring = 0;
    for (int h = 0; h < H; ++h) {
        if (D[h] < 1 || W[h] < 0) return -3;
        int nd = (T - 1) / D[h] + 1;
        int nw = W[h] < T ? W[h] : T;
        if (nd > nd_cap || nw > w_cap) return -2;
        if (nw > 0) need_ring = 1;
        if (nd + nw > max_keys) max_keys = nd + nw;
    }
    if (need_ring && (!kw || !vw)) return -1;
    int bad = 0;
#pragma omp parallel
    {
        const double** kp = (const double**)malloc(sizeof(double*) * max_keys);
        const double** vp = (const double**)malloc(sizeof(double*) * max_keys);
        double* z = (double*)malloc(sizeof(double) * max_keys);
        if (!kp || !vp || !z) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for collapse(2) schedule(dynamic)
            for (int b = 0; b < B; ++b)
                for (int h = 0; h < H; ++h) {
                    int nd = (T - 1) / D[h] + 1;
                    int nw = W[h] < T ? W[h] : T;
                    int n = 0;
                    size_t base_d = ((size_t)b * H + h) * (size_t)nd_cap * d;
                    size_t base_w = ((size_t)b * H + h) * (size_t)w_cap * d;
                    for (int i = 0; i < nd; ++i) {
                        kp[n] = kd + base_d + (size_t)i * d;
                        vp[n] = vd + base_d + (size_t)i * d;
                        ++n;
                    }
                    for (int j = 0; j < nw; ++j) {
                        kp[n] = kw + base_w + (size_t)j * d;
                        vp[n] = vw + base_w + (size_t)j * d;
                        ++n;
                    }
                    size_t qo = ((size_t)b * H + h) * (size_t)d;
                    softmax_rows(q + qo, kp, vp, n, d, scale, z, out + qo);
                }
        }
        free(kp);
        free(vp);
        free(z);
    }
    return bad ? -4 : 0;
}

/* Chunk-grid index set of query t [RAT abstract: attention across chunks]:
 * the chunk-end positions cD - 1 < t in increasing order, then t itself.
 * Returns the count; pos may be NULL (count only). */
long oracle_chunk_index_set(int t, int D, int* pos)
{
    if (t < 0 || D < 1) return -1;
    long n = 0;
    for (int p = D - 1; p < t; p += D) {
        if (pos) pos[n] = p;
        ++n;
    }
    if (pos) pos[n] = t;
    return n + 1;
}

/* Chunk-grid prefill attention for a list of query rows (b, t, h): one
 * softmax over the chunk-end states before t and the own state at t.
 * k_state, v_state, q: [B,T,H,d]; out_rows [n, d]. */
int oracle_chunk_attn_prefill_rows(const double* q, const double* k_state, const double* v_state,
                                   const int* rows, int n, double* out_rows,
                                   int B, int T, int H, int d, const int* D, double scale)
{
    if (!q || !k_state || !v_state || !rows || !out_rows || !D) return -1;
    if (B <= 0 || T <= 0 || H <= 0 || d <= 0 || n < 0) return -2;
    int max_keys = 0;
    for (int h = 0; h < H; ++h) {
        if (D[h] < 1) return -3;
        int nk = (T - 1) / D[h] + 2;
        if (nk > max_keys) max_keys = nk;
    }
    for (int i = 0; i < n; ++i) {
        int b = rows[3 * i], t = rows[3 * i + 1], h = rows[3 * i + 2];
        if (b < 0 || b >= B || t < 0 || t >= T || h < 0 || h >= H) return -2;
    }
    int bad = 0;
#pragma omp parallel
    {
        const double** kp = (const double**)malloc(sizeof(double*) * max_keys);
        const double** vp = (const double**)malloc(sizeof(double*) * max_keys);
        double* z = (double*)malloc(sizeof(double) * max_keys);
        int* pos = (int*)malloc(sizeof(int) * max_keys);
        double* tmp = (double*)malloc(sizeof(double) * (size_t)d);
        if (!kp || !vp || !z || !pos || !tmp) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int i = 0; i < n; ++i) {
                int b = rows[3 * i], t = rows[3 * i + 1], h = rows[3 * i + 2];
                int nk = (int)oracle_chunk_index_set(t, D[h], pos);
                for (int j = 0; j < nk; ++j) {
                    kp[j] = k_state + idx4(b, pos[j], h, 0, T, H, d);
                    vp[j] = v_state + idx4(b, pos[j], h, 0, T, H, d);
                }
                softmax_rows(q + idx4(b, t, h, 0, T, H, d), kp, vp, nk, d, scale, z, tmp);
                for (int c = 0; c < d; ++c) out_rows[(size_t)i * d + c] = tmp[c];
            }
        }
        free(kp);
        free(vp);
        free(z);
        free(pos);
        free(tmp);
    }
    return bad ? -4 : 0;
}

/* Backward of the layer: the gradient of a scalar loss through the forward
 * above (recurrence of Deep Dive S2.1, then the one-softmax attention of
 * Deep Dive S1 / RAT+ abstract), by the chain rule applied to those
 * definitions.  This is what the training of Deep Dive S2.2 (Active
 * Recurrence Learning: half of a batch at D = 1, half at D = 64, recurrence
 * over the full sequence) differentiates.  Every recurrence: full (L >= T),
 * RESTART and SLIDING.
 *
 * Given dout = dLoss/dout [B,T,H,d]:
 *   attention, per query t with keys/values (kappa_j, nu_j), j over the
 *   dilated states then the raw window, z_j = scale <q_t, kappa_j>,
 *   p_j = softmax(z)_j:
 *     dp_j = <dout_t, nu_j>,  delta = sum_j p_j dp_j,
 *     ds_j = p_j (dp_j - delta),
 *     dq_t += scale sum_j ds_j kappa_j,
 *     dkappa_j += scale ds_j q_t,   dnu_j += p_j dout_t;
 *   recurrence h_t = g_t h_{t-1} + (1 - g_t) x_t (h_{t-1} := 0 at t = 0 and
 *   at RESTART positions), walked backwards with lambda_t = dLoss/dh_t:
 *     lambda_t = dh_t + g_{t+1} lambda_{t+1}  (no carry into t when t + 1
 *                is a restart position, nor past the end),
 *     dx_t += (1 - g_t) lambda_t,
 *     dlogit_t = g_t (1 - g_t) sum_{x in k, v} lambda_t (h_{t-1} - x_t)
 *   (the gate is shared by keys and values; dsigma/dl = sigma (1 - sigma)).
 *   A SLIDING window (L < T) makes each state its own window: h_t is w after
 *   the steps w <- g_u w + (1 - g_u) x_u, u = max(0, t-L+1) .. t, from w = 0,
 *   and lambda_t = dh_t carries nothing.  With Q_u = g_{u+1} ... g_t (the
 *   steps after u) and w_u the value of w before step u:
 *     dx_u += (1 - g_u) Q_u lambda_t,
 *     dlogit_u += g_u (1 - g_u) sum_{x in k, v} Q_u lambda_t (w_u - x_u).
 * Outputs dq, dk, dv, dlogit: [B,T,H,d]; dk and dv sum the state path and
 * the raw-window path.
 *
 * oracle_layer_backward_states is the same chain rule evaluated at given
 * states (ks, vs) [B,T,H,d] instead of the ones the recurrence produces from
 * (k, v, logit): the keys / values of the attention and the h_{t-1} of the
 * recurrence's gate derivative are read from them.  This is what a backward
 * that is handed the forward's saved states computes; oracle_layer_backward
 * is this function at the oracle's own fp64 states, so the two share every
 * line of arithmetic.  (A SLIDING window below T re-walks each window from
 * the raw inputs, as above, and reads no state.) */
int oracle_layer_backward_states(const double* q, const double* k, const double* v, const double* logit,
                                 const double* ks, const double* vs, const double* dout, double* dq,
                                 double* dk, double* dv, double* dlogit, int B, int T, int H, int d, int L,
                                 int mode, const int* D, const int* W, double scale)
{
    if (!q || !k || !v || !logit || !ks || !vs || !dout || !dq || !dk || !dv || !dlogit || !D || !W) return -1;
    if (B <= 0 || T <= 0 || H <= 0 || d <= 0 || L < 1) return -2;
    if (mode != ORACLE_MODE_RESTART && mode != ORACLE_MODE_SLIDING) return -3;
    const int full = (L >= T);
    const int sliding = !full && mode == ORACLE_MODE_SLIDING;
    int need_raw, max_keys;
    if (check_heads(H, D, W, &need_raw, &max_keys, T)) return -3;
    const size_t n = (size_t)B * T * H * d;
    double* dks = (double*)calloc(n, sizeof(double));  /* dLoss/d state (from attention) */
    double* dvs = (double*)calloc(n, sizeof(double));
    if (!dks || !dvs) {
        free(dks); free(dvs);
        return -4;
    }
    for (size_t i = 0; i < n; ++i) { dq[i] = 0.0; dk[i] = 0.0; dv[i] = 0.0; dlogit[i] = 0.0; }
    int bad = 0;
    /* attention: the accumulations of one (b, h) touch only that head */
#pragma omp parallel
    {
        const double** kp = (const double**)malloc(sizeof(double*) * max_keys);
        const double** vp = (const double**)malloc(sizeof(double*) * max_keys);
        double** dkp = (double**)malloc(sizeof(double*) * max_keys);
        double** dvp = (double**)malloc(sizeof(double*) * max_keys);
        double* z = (double*)malloc(sizeof(double) * max_keys);
        double* p = (double*)malloc(sizeof(double) * max_keys);
        if (!kp || !vp || !dkp || !dvp || !z || !p) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for collapse(2) schedule(dynamic)
            for (int b = 0; b < B; ++b)
                for (int h = 0; h < H; ++h)
                    for (int t = 0; t < T; ++t) {
                        int nk = 0;
                        for (int s = t; s >= 0; s -= D[h]) {
                            size_t o = idx4(b, s, h, 0, T, H, d);
                            kp[nk] = ks + o; vp[nk] = vs + o; dkp[nk] = dks + o; dvp[nk] = dvs + o;
                            ++nk;
                        }
                        for (int w = 0; w < W[h] && t - w >= 0; ++w) {
                            size_t o = idx4(b, t - w, h, 0, T, H, d);
                            kp[nk] = k + o; vp[nk] = v + o; dkp[nk] = dk + o; dvp[nk] = dv + o;
                            ++nk;
                        }
                        const double* qt = q + idx4(b, t, h, 0, T, H, d);
                        const double* go = dout + idx4(b, t, h, 0, T, H, d);
                        double* gq = dq + idx4(b, t, h, 0, T, H, d);
                        double m = -INFINITY;
                        for (int j = 0; j < nk; ++j) {
                            double dot = 0.0;
                            for (int c = 0; c < d; ++c) dot += qt[c] * kp[j][c];
                            z[j] = dot * scale;
                            if (z[j] > m) m = z[j];
                        }
                        double den = 0.0;
                        for (int j = 0; j < nk; ++j) { p[j] = exp(z[j] - m); den += p[j]; }
                        double delta = 0.0;
                        for (int j = 0; j < nk; ++j) {
                            p[j] /= den;
                            double dp = 0.0;
                            for (int c = 0; c < d; ++c) dp += go[c] * vp[j][c];
                            z[j] = dp;  /* reuse: dp_j */
                            delta += p[j] * dp;
                        }
                        for (int j = 0; j < nk; ++j) {
                            double ds = p[j] * (z[j] - delta);
                            for (int c = 0; c < d; ++c) {
                                gq[c] += scale * ds * kp[j][c];
                                dkp[j][c] += scale * ds * qt[c];
                                dvp[j][c] += p[j] * go[c];
                            }
                        }
                    }
        }
        free(kp); free(vp); free(dkp); free(dvp); free(z); free(p);
    }
    if (sliding) {
        /* each window on its own: the chain rule through its steps */
#pragma omp parallel
        {
            double* Q = (double*)malloc(sizeof(double) * L);
            if (!Q) {
#pragma omp atomic write
                bad = 1;
            } else {
#pragma omp for collapse(2) schedule(dynamic)
                for (int b = 0; b < B; ++b)
                    for (int h = 0; h < H; ++h)
                        for (int c = 0; c < d; ++c)
                            for (int t = 0; t < T; ++t) {
                                const int lo = t - L + 1 < 0 ? 0 : t - L + 1;
                                double g, gb;
                                Q[t - lo] = 1.0;
                                for (int u = t; u > lo; --u) {
                                    gate_pair(logit[idx4(b, u, h, c, T, H, d)], &g, &gb);
                                    Q[u - 1 - lo] = Q[u - lo] * g;
                                }
                                const size_t it = idx4(b, t, h, c, T, H, d);
                                const double lamk = dks[it], lamv = dvs[it];
                                double wk = 0.0, wv = 0.0;
                                for (int u = lo; u <= t; ++u) {
                                    const size_t i = idx4(b, u, h, c, T, H, d);
                                    gate_pair(logit[i], &g, &gb);
                                    const double qk = Q[u - lo] * lamk, qv = Q[u - lo] * lamv;
                                    dk[i] += gb * qk;
                                    dv[i] += gb * qv;
                                    dlogit[i] += g * gb * (qk * (wk - k[i]) + qv * (wv - v[i]));
                                    wk = g * wk + gb * k[i];
                                    wv = g * wv + gb * v[i];
                                }
                            }
            }
            free(Q);
        }
        free(dks); free(dvs);
        return bad ? -4 : 0;
    }
    /* recurrence, backwards in time, one channel at a time */
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int c = 0; c < d; ++c) {
                double lk = 0.0, lv = 0.0;  /* carry g_{t+1} lambda_{t+1} into t */
                for (int t = T - 1; t >= 0; --t) {
                    size_t i = idx4(b, t, h, c, T, H, d);
                    double g, gb;
                    gate_pair(logit[i], &g, &gb);
                    const int cut = (t == 0) || (!full && t % L == 0);  /* h_{t-1} replaced by 0 */
                    double hk_prev = cut ? 0.0 : ks[idx4(b, t - 1, h, c, T, H, d)];
                    double hv_prev = cut ? 0.0 : vs[idx4(b, t - 1, h, c, T, H, d)];
                    double lamk = dks[i] + lk, lamv = dvs[i] + lv;
                    dk[i] += gb * lamk;
                    dv[i] += gb * lamv;
                    dlogit[i] = g * gb * (lamk * (hk_prev - k[i]) + lamv * (hv_prev - v[i]));
                    lk = cut ? 0.0 : g * lamk;
                    lv = cut ? 0.0 : g * lamv;
                }
            }
    free(dks); free(dvs);
    return bad ? -4 : 0;
}

int oracle_layer_backward(const double* q, const double* k, const double* v, const double* logit,
                          const double* dout, double* dq, double* dk, double* dv, double* dlogit,
                          int B, int T, int H, int d, int L, int mode, const int* D, const int* W,
                          double scale)
{
    if (!q || !k || !v || !logit || !dout || !dq || !dk || !dv || !dlogit || !D || !W) return -1;
    if (B <= 0 || T <= 0 || H <= 0 || d <= 0 || L < 1) return -2;
    if (mode != ORACLE_MODE_RESTART && mode != ORACLE_MODE_SLIDING) return -3;
    const size_t n = (size_t)B * T * H * d;
    double* ks = (double*)malloc(sizeof(double) * n);
    double* vs = (double*)malloc(sizeof(double) * n);
    if (!ks || !vs) {
        free(ks); free(vs);
        return -4;
    }
    oracle_scan(k, v, logit, ks, vs, B, T, H, d, L, mode);
    const int rc = oracle_layer_backward_states(q, k, v, logit, ks, vs, dout, dq, dk, dv, dlogit, B, T, H, d, L,
                                                mode, D, W, scale);
    free(ks); free(vs);
    return rc;
}

/* Counting mode for the FLOP / KV-size invariants [Deep Dive S3.1 table:
 * attention FLOPs T/D]: totals over all T queries of one head. */
int oracle_count_pairs(int T, int D, int W, long long* n_dil_total, long long* n_loc_total)
{
    if (T <= 0 || D < 1 || W < 0 || !n_dil_total || !n_loc_total) return -1;
    long long a = 0, b = 0;
    for (int t = 0; t < T; ++t) {
        int nd, nl;
        oracle_index_sets(t, D, W, NULL, &nd, NULL, &nl);
        a += nd;
        b += nl;
    }
    *n_dil_total = a;
    *n_loc_total = b;
    return 0;
}

/* Threads an OpenMP region of this library runs on (for reporting timings). */
int oracle_num_threads(void)
{
    return omp_get_max_threads();
}
