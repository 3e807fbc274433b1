// Backward of the RAT+ layer: the gradient of a loss through the dilated
// (+ local window) attention and the gated recurrence, as differentiated by
// the training the "RAT+ Deep Dive" page (zhichai.net) describes in section
// 2.2 (Active Recurrence Learning: half of each batch at D = 1, half at
// D = 64, the recurrence over the full sequence).
//
// Attention, per query t with keys kappa_j and values nu_j (the states at
// t, t-D, ... then the raw tokens t, ..., t-W+1) and p = softmax(scale q.k):
//   delta_t = <dout_t, out_t>,  ds_j = p_j (<dout_t, nu_j> - delta_t),
//   dq_t = scale sum_j ds_j kappa_j,  dkappa_j += scale ds_j q_t,
//   dnu_j += p_j dout_t.
// Recurrence h_t = g_t h_{t-1} + (1 - g_t) x_t (h_{t-1} := 0 at t = 0 and at
// RESTART positions), backwards: lambda_t = dh_t + g_{t+1} lambda_{t+1}
// (cut at restarts), dx_t = (1 - g_t) lambda_t,
// dlogit_t = g_t (1 - g_t) sum_{k, v} lambda_t (h_{t-1} - x_t).
//
// delta_t equals sum_j p_j <dout_t, nu_j>, so it is formed from the fp32
// probabilities of the backward's own softmax (not from a rounded copy of
// the forward output): accumulated beside the log-sum-exp with the same
// running-max rescaling, then divided by the softmax sum.
//
// Kernels (all arithmetic fp32, gradients written in fp32):
//   bwd_q_mfma / bwd_kv_mfma  bf16, on MFMA: a residue is a dense causal
//                     problem over the states r, r + D, ..., so a workgroup
//                     takes 64 rows of one residue (queries for dq, keys for
//                     dk / dv) and walks the other side's 64-row tiles
//                     through LDS.  A raw window is the same problem over
//                     consecutive positions with a band mask: its passes
//                     leave each query's partial softmax sums, from which
//                     the dilated pass forms the one softmax's statistics,
//                     then add the window's dq and give the raw keys' dk / dv
//                     (the forward's two-pass split, backwards);
//   bwd_query_kernel  fp32: one wave per query row: log-sum-exp of its
//                     softmax and delta_t, then dq_t (two passes over its keys);
//   bwd_key_kernel    fp32: one wave per key row: the state key's gradients
//                     from the queries t = s, s + D, ... and the raw key's
//                     from t = s .. s + W - 1;
//   bwd_slide_kernel  the SLIDING window (L < T): per token and channel
//                     over the windows that hold it;
//   bwd_scan_*        the reverse recurrence in chunks of kBwdChunk tokens:
//                     per-chunk affine maps (forward state map and backward
//                     carry map), a sequential pass over the chunks of each
//                     channel, then per chunk the states recomputed in fp32
//                     from the chunk's start state and walked backwards.
#include "rat_device.h"
#include "rat_internal.h"
#include "rat_mfma.h"

namespace rat {

template <typename E> __device__ __forceinline__ float ldx(const void* p, size_t i);
template <> __device__ __forceinline__ float ldx<uint16_t>(const void* p, size_t i)
{
    return __uint_as_float((uint32_t)static_cast<const uint16_t*>(p)[i] << 16);
}
template <> __device__ __forceinline__ float ldx<float>(const void* p, size_t i) { return static_cast<const float*>(p)[i]; }

// Sums over the 64 lanes of N values at once (the shuffle chains of the N
// values interleave).
template <int N>
__device__ __forceinline__ void wave_sum_n(float (&x)[N])
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
#pragma unroll
        for (int i = 0; i < N; ++i) x[i] += __shfl_xor(x[i], o);
}

// A row of d <= 128 channels across one wave: lane holds channels 2 lane and
// 2 lane + 1 (zero past d), one 4- or 8-byte load.
template <typename E> struct Row2;
template <> struct Row2<uint16_t> {
    float a, b;
    __device__ __forceinline__ void load(const void* p, size_t row, int d, int lane)
    {
        if (2 * lane < d) {
            const uint32_t w = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p) + row + 2 * lane);
            a = bf16_lo(w);
            b = bf16_hi(w);
        } else {
            a = b = 0.f;
        }
    }
};
template <> struct Row2<float> {
    float a, b;
    __device__ __forceinline__ void load(const void* p, size_t row, int d, int lane)
    {
        if (2 * lane < d) {
            const float2 w = *reinterpret_cast<const float2*>(static_cast<const float*>(p) + row + 2 * lane);
            a = w.x;
            b = w.y;
        } else {
            a = b = 0.f;
        }
    }
};
template <typename E>
__device__ __forceinline__ float part(const Row2<E>& x, const Row2<E>& y) { return fmaf(x.a, y.a, x.b * y.b); }

constexpr int kBwdGroup = 4;  // keys (or queries) per step of a row's loop: loads issued together

// ---------------------------------------------------------------- attention
template <typename E>
__global__ __launch_bounds__(kWave) void bwd_query_kernel(BwdArgs a)
{
    constexpr int G = kBwdGroup;
    const int lane = threadIdx.x;
    const int t = blockIdx.x % a.T;
    const int bh = blockIdx.x / a.T;
    const int h = bh % a.H, b = bh / a.H;
    const int d = a.d, D = a.D[h], W = a.W[h];
    const size_t pitch = (size_t)a.H * d;
    const size_t base = ((size_t)b * a.T * a.H + h) * d;  // row 0 of (b, h)
    const size_t rt = base + (size_t)t * pitch;
    Row2<E> q, go;
    q.load(a.q, rt, d, lane);
    go.load(a.dout, rt, d, lane);
    // key j: the state at t - jD (j < nd), then the raw token at t - (j - nd)
    const int nd = t / D + 1, nk = nd + min(W, t + 1);
    auto load_key = [&](int j, Row2<E>& kk, Row2<E>& vv) {
        if (j < nd) {
            const size_t r = base + (size_t)(t - j * D) * pitch;
            kk.load(a.ks, r, d, lane);
            vv.load(a.vs, r, d, lane);
        } else if (j < nk) {
            const size_t r = base + (size_t)(t - (j - nd)) * pitch;
            kk.load(a.k, r, d, lane);
            vv.load(a.v, r, d, lane);
        } else {
            kk.a = kk.b = vv.a = vv.b = 0.f;
        }
    };
    // pass 1: log-sum-exp of the logits and delta = sum_j p_j dp_j
    float m = -INFINITY, l = 0.f, u = 0.f;  // u: sum_j e^{z_j - m} dp_j
    for (int j0 = 0; j0 < nk; j0 += G) {
        Row2<E> kk[G], vv[G];
        float x[2 * G];
#pragma unroll
        for (int i = 0; i < G; ++i) load_key(j0 + i, kk[i], vv[i]);
#pragma unroll
        for (int i = 0; i < G; ++i) {
            x[2 * i] = part(q, kk[i]);
            x[2 * i + 1] = part(go, vv[i]);
        }
        wave_sum_n(x);
#pragma unroll
        for (int i = 0; i < G; ++i) {
            if (j0 + i < nk) {
                const float z = x[2 * i] * a.scale;
                const float mn = fmaxf(m, z);
                const float r = __expf(m - mn), e = __expf(z - mn);
                l = fmaf(l, r, e);
                u = fmaf(u, r, e * x[2 * i + 1]);
                m = mn;
            }
        }
    }
    const float lse = m + __logf(l);
    const float delta = u / l;
    // pass 2: dq = scale sum_j p_j (dp_j - delta) kappa_j
    float ga = 0.f, gb = 0.f;
    for (int j0 = 0; j0 < nk; j0 += G) {
        Row2<E> kk[G], vv[G];
        float x[2 * G];
#pragma unroll
        for (int i = 0; i < G; ++i) load_key(j0 + i, kk[i], vv[i]);
#pragma unroll
        for (int i = 0; i < G; ++i) {
            x[2 * i] = part(q, kk[i]);
            x[2 * i + 1] = part(go, vv[i]);
        }
        wave_sum_n(x);
#pragma unroll
        for (int i = 0; i < G; ++i) {
            // keys past the list are zero rows: their ds multiplies a zero row
            const float p = __expf(x[2 * i] * a.scale - lse);
            const float ds = p * (x[2 * i + 1] - delta) * a.scale;
            ga = fmaf(ds, kk[i].a, ga);
            gb = fmaf(ds, kk[i].b, gb);
        }
    }
    if (2 * lane < d) *reinterpret_cast<float2*>(a.dq + rt + 2 * lane) = float2{ga, gb};
    if (lane == 0) {
        const size_t r = ((size_t)b * a.T + t) * a.H + h;
        a.lse[r] = lse;
        a.delta[r] = delta;
    }
}

template <typename E>
__global__ __launch_bounds__(kWave) void bwd_key_kernel(BwdArgs a)
{
    constexpr int G = kBwdGroup;
    const int lane = threadIdx.x;
    const int s = blockIdx.x % a.T;
    const int bh = blockIdx.x / a.T;
    const int h = bh % a.H, b = bh / a.H;
    const int d = a.d, D = a.D[h], W = a.W[h];
    const size_t pitch = (size_t)a.H * d;
    const size_t base = ((size_t)b * a.T * a.H + h) * d;
    const size_t rs = base + (size_t)s * pitch;
    // one key row against the nq queries t = s + j step that see it
    auto key_grads = [&](const void* kp, const void* vp, int nq, int step, float* dk_out, float* dv_out) {
        Row2<E> kk, vv;
        kk.load(kp, rs, d, lane);
        vv.load(vp, rs, d, lane);
        float ka = 0.f, kb = 0.f, va = 0.f, vb = 0.f;
        for (int j0 = 0; j0 < nq; j0 += G) {
            Row2<E> q[G], go[G];
            float lse[G], dl[G], x[2 * G];
#pragma unroll
            for (int i = 0; i < G; ++i) {
                if (j0 + i < nq) {
                    const int t = s + (j0 + i) * step;
                    const size_t rt = base + (size_t)t * pitch;
                    const size_t r = ((size_t)b * a.T + t) * a.H + h;
                    q[i].load(a.q, rt, d, lane);
                    go[i].load(a.dout, rt, d, lane);
                    lse[i] = a.lse[r];
                    dl[i] = a.delta[r];
                } else {
                    q[i].a = q[i].b = go[i].a = go[i].b = 0.f;
                    lse[i] = INFINITY;  // p = 0
                    dl[i] = 0.f;
                }
            }
#pragma unroll
            for (int i = 0; i < G; ++i) {
                x[2 * i] = part(q[i], kk);
                x[2 * i + 1] = part(go[i], vv);
            }
            wave_sum_n(x);
#pragma unroll
            for (int i = 0; i < G; ++i) {
                const float p = __expf(x[2 * i] * a.scale - lse[i]);
                const float ds = p * (x[2 * i + 1] - dl[i]) * a.scale;
                ka = fmaf(ds, q[i].a, ka);
                kb = fmaf(ds, q[i].b, kb);
                va = fmaf(p, go[i].a, va);
                vb = fmaf(p, go[i].b, vb);
            }
        }
        if (2 * lane < d) {
            *reinterpret_cast<float2*>(dk_out + rs + 2 * lane) = float2{ka, kb};
            *reinterpret_cast<float2*>(dv_out + rs + 2 * lane) = float2{va, vb};
        }
    };
    // the state at s: queries s, s + D, ... (< T)
    key_grads(a.ks, a.vs, (a.T - 1 - s) / D + 1, D, a.dks, a.dvs);
    // the raw token at s: queries s .. s + W - 1 (< T); none writes zeros
    key_grads(a.k, a.v, min(W, a.T - s), 1, a.dk, a.dv);
}


// ---------------------------------------------------------------- MFMA path
// Work item: (head h with W = 0, batch b, residue r, block of 64 rows of
// that residue); items of head h start at a.mitem[h].  Within a head the
// block index is outermost, in the order that puts the largest blocks first
// (dq: a block's work grows with its index; dk / dv: it shrinks).
constexpr int kBwdRows = 64;  // rows of the other side's tiles
constexpr int kBwdThreads = kBwdWaves * kWave;
constexpr int kBwdOwn = 16 * kBwdWaves;  // rows a workgroup owns (16 per wave)

struct BwdItem {
    int b, h, r, blk, M, D;
    bool valid;
};

// The dispatcher deals workgroups to the chip's 8 XCDs in turn (workgroup i
// to XCD i mod 8), and each XCD has its own L2.  Workgroup i runs item
// xcd_item(i): XCD x takes one contiguous eighth of the item list, in order,
// so the workgroups resident on an XCD share one or two heads' tiles instead
// of every head's.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_item(int wg, int n)
{
    const int per = n / kXcds, extra = n % kXcds;  // XCD x runs per + (x < extra) items
    const int x = wg % kXcds, k = wg / kXcds;
    return x * per + min(x, extra) + k;
}

template <bool LAST_FIRST>
__device__ __forceinline__ BwdItem bwd_item(const BwdArgs& a, int item)
{
    BwdItem it;
    int h = 0;
    while (h + 1 < a.H && item >= a.mitem[h + 1]) ++h;
    it.h = h;
    it.D = a.D[h];
    const int Dr = min(it.D, a.T);
    const int nb = ((a.T + it.D - 1) / it.D + kBwdOwn - 1) / kBwdOwn;  // blocks of the longest residue
    const int local = item - a.mitem[h];
    const int level = local / (a.B * Dr), rest = local % (a.B * Dr);
    it.blk = LAST_FIRST ? nb - 1 - level : level;
    it.r = rest % Dr;
    it.b = rest / Dr;
    it.M = (a.T - it.r + it.D - 1) / it.D;
    it.valid = item < a.mitem[h + 1] && it.blk * kBwdOwn < it.M;
    return it;
}

// element offset of row `row` of residue r of (b, h) in a [B][T][H][DK] tensor
template <int DK>
__device__ __forceinline__ size_t res_row(const BwdArgs& a, const BwdItem& it, int row)
{
    return (((size_t)it.b * a.T + (it.r + (size_t)row * it.D)) * a.H + it.h) * DK;
}

// 64 rows (row0 ..) of a residue into a swizzled LDS tile; rows past M are zero
template <int DK>
__device__ __forceinline__ void load_rows(lds_char* tile, const void* src, const BwdArgs& a, const BwdItem& it,
                                          int row0)
{
    constexpr int CH = Geo<DK>::CH;
    for (int idx = threadIdx.x; idx < kBwdRows * CH; idx += kBwdThreads) {
        const int row = idx / CH, c = idx % CH;
        u32x4 val = {0u, 0u, 0u, 0u};
        if (row0 + row < it.M)
            val = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(src) + res_row<DK>(a, it, row0 + row) + c * 8);
        *reinterpret_cast<u32x4*>(tile + swz<DK>(row, c)) = val;
    }
}

// The same 64 rows staged through registers, so that the next tile's loads
// are in flight while the current one is computed: load, then (after the
// barrier that frees the tile) store.
template <int DK>
struct TileRegs {
    static constexpr int N = kBwdRows * Geo<DK>::CH / kBwdThreads;  // 16-byte chunks per thread
    static_assert(N * kBwdThreads == kBwdRows * Geo<DK>::CH, "whole tile per pass");
    u32x4 v[N];
    __device__ __forceinline__ void load(const void* src, const BwdArgs& a, const BwdItem& it, int row0)
    {
        constexpr int CH = Geo<DK>::CH;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const int idx = threadIdx.x + n * kBwdThreads;
            const int row = idx / CH, c = idx % CH;
            v[n] = u32x4{0u, 0u, 0u, 0u};
            if (row0 + row < it.M)
                v[n] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(src) + res_row<DK>(a, it, row0 + row) +
                                                       c * 8);
        }
    }
    __device__ __forceinline__ void store(lds_char* tile) const
    {
        constexpr int CH = Geo<DK>::CH;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const int idx = threadIdx.x + n * kBwdThreads;
            *reinterpret_cast<u32x4*>(tile + swz<DK>(idx / CH, idx % CH)) = v[n];
        }
    }
};

// B-operand fragments of one row (lane (g, i): the row of i, dims 8g + 32ks)
template <int DK>
__device__ __forceinline__ void load_frag(bf16x8 (&f)[Geo<DK>::KS], const void* src, size_t row_el, bool valid)
{
    const int g = (threadIdx.x & (kWave - 1)) >> 4;
#pragma unroll
    for (int ks = 0; ks < Geo<DK>::KS; ++ks)
        f[ks] = valid ? *reinterpret_cast<const bf16x8*>(static_cast<const uint16_t*>(src) + row_el + 8 * g + 32 * ks)
                      : bf16x8{};
}

// A-operand offset of the transposing reads (lane (g, i): rows 4g .. 4g+3
// of a 16-row group, dims 4 (i % 4) ..; XOR in the dim block as db << 5)
template <int DK>
__device__ __forceinline__ int tr_offset()
{
    const int lane = threadIdx.x & (kWave - 1);
    const int g = lane >> 4, i = lane & 15;
    const int dim = 4 * (i & 3);
    return swz<DK>(4 * g + (i >> 2), dim >> 3) + (dim & 7) * 2;
}

// A operand (rows = dims 16 db .. of a 16-dim block, k = the 32 rows of
// half hh of a 64-row tile in the order {4g + j, 16 + 4g + j})
template <int DK>
__device__ __forceinline__ bf16x8 tr_frag(const lds_char* tile, int off, int db, int hh)
{
    const lds_char* p = tile + (off ^ (db << 5)) + hh * 32 * Geo<DK>::ROWB;
    const shortx4 x0 = lds_tr(p);
    const shortx4 x1 = lds_tr(p + 16 * Geo<DK>::ROWB);
    typedef short shortx8 __attribute__((ext_vector_type(8)));
    const shortx8 v = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// dS enters the MFMA products as a pair of bf16 values, hi = bf16(x) and
// lo = bf16(x - hi) (about 16 mantissa bits together): its terms have both
// signs and sum to zero over a query's keys, so a single bf16 rounding of
// each would dominate sums that cancel.
__device__ __forceinline__ void split_bf16(float x, bf16x8& hi, bf16x8& lo, int e)
{
    const __bf16 h = (__bf16)x;
    hi[e] = h;
    lo[e] = (__bf16)(x - (float)h);
}

// Band work item, for the raw windows: (head, batch, block of kBwdOwn
// consecutive positions), the item list covering every head; the window is
// the residue of D = 1 over the whole sequence with the raw tokens as keys.
// Items of heads without a window return, or in bwd_kv_mfma write zeros
// for their raw keys' gradients.
__device__ __forceinline__ BwdItem band_item(const BwdArgs& a, int item)
{
    BwdItem it;
    const int nb = (a.T + kBwdOwn - 1) / kBwdOwn;
    it.h = item / (a.B * nb);
    const int rest = item % (a.B * nb);
    it.b = rest / nb;
    it.blk = rest % nb;
    it.r = 0;
    it.D = 1;
    it.M = a.T;
    it.valid = it.h < a.H;
    return it;
}

// dq (and each query row's log-sum-exp and delta): wave w owns queries
// 16w .. 16w+15 of the block; lane (g, i) query i.  Scores are S^T = K Q^T
// (lane: keys 16kb + 4g + j of its query), dP^T = V dO^T, and
// dQ^T += K^T dS^T with dS^T packed to bf16 as the B operand.
// MODE 0: the dilated states of every head (a head with a window starts its
// softmax statistics from the window's partial sums); MODE 1: the raw
// window's partial sums only (max, sum of e^(z - max), sum of e^(z - max) dp
// per query, into bstat); MODE 2: the raw window's share of dq, added to
// the dilated share, with the query's final log-sum-exp and delta.
template <int DK, int MODE>
__global__ __launch_bounds__(kBwdThreads, 2) void bwd_q_mfma(BwdArgs a)
{
    typedef Geo<DK> G;
    __shared__ __attribute__((aligned(1024))) char kt[kBwdRows * G::ROWB];
    __shared__ __attribute__((aligned(1024))) char vt[kBwdRows * G::ROWB];
    const int wi = xcd_item(blockIdx.x, gridDim.x);
    const BwdItem it = MODE == 0 ? bwd_item<true>(a, wi) : band_item(a, wi);
    if (!it.valid) return;
    const int Wh = a.W[it.h];
    if (MODE != 0 && Wh == 0) return;
    const void* const ksrc = MODE == 0 ? a.ks : a.k;
    const void* const vsrc = MODE == 0 ? a.vs : a.v;
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int g = lane >> 4, i = lane & 15;
    const float c = a.scale * kLog2e;
    const int qr = it.blk * kBwdOwn + 16 * wv + i;
    const bool qvalid = qr < it.M;
    const size_t qe = qvalid ? res_row<DK>(a, it, qr) : 0;
    const size_t rrow = qvalid ? ((size_t)it.b * a.T + it.r + (size_t)qr * it.D) * a.H + it.h : 0;
    bf16x8 qf[G::KS], gf[G::KS];
    load_frag<DK>(qf, a.q, qe, qvalid);
    load_frag<DK>(gf, a.dout, qe, qvalid);
    // key tiles tlo .. thi-1: up to the block's last query, and for the
    // window from the tile holding its first query's first window key
    const int thi = (min(it.M, (it.blk + 1) * kBwdOwn) - 1) / kBwdRows + 1;
    const int tlo = MODE == 0 ? 0 : max(0, it.blk * kBwdOwn - Wh + 1) / kBwdRows;
    const int nt = thi - tlo;
    constexpr int NSWEEP = MODE == 0 ? 2 : 1;
    // key row kr is seen by the lane's query: up to it, within the window
    auto visible = [&](int kr) { return kr <= qr && (MODE == 0 || kr > qr - Wh); };
    auto scores = [&](floatx4 (&st)[4], floatx4 (&dpt)[4]) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            st[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
            dpt[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < G::KS; ++ks) {
                st[kb] = mfma16(lds_b128(kt + swz<DK>(16 * kb + i, g + 4 * ks)), qf[ks], st[kb]);
                dpt[kb] = mfma16(lds_b128(vt + swz<DK>(16 * kb + i, g + 4 * ks)), gf[ks], dpt[kb]);
            }
        }
    };
    // the key / value tiles of every sweep in turn, through registers: step
    // n of the sequence is tile tlo + n mod nt
    TileRegs<DK> rk, rv;
    rk.load(ksrc, a, it, tlo * kBwdRows);
    rv.load(vsrc, a, it, tlo * kBwdRows);
    int seq = 0;
    auto next_tile = [&]() {  // the fetched tile into LDS, the following one into registers
        __syncthreads();
        rk.store(kt);
        rv.store(vt);
        __syncthreads();
        ++seq;
        if (seq < NSWEEP * nt) {
            const int tn = tlo + seq % nt;
            rk.load(ksrc, a, it, tn * kBwdRows);
            rv.load(vsrc, a, it, tn * kBwdRows);
        }
    };
    float lse2, delta;  // log2-domain log-sum-exp and delta of the lane's query
    if (MODE != 2) {
        // sweep 1: per lane group, (max, sum of e^(z - max), sum of
        // e^(z - max) dp) over its keys, rescaled once per tile: the tile's 16
        // scores of the lane (-inf where not seen) give the new max first
        float m = -INFINITY, l = 0.f, u = 0.f;
        for (int t = tlo; t < thi; ++t) {
            next_tile();
            floatx4 st[4], dpt[4];
            scores(st, dpt);
            float tm = m;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int kr = t * kBwdRows + 16 * kb + 4 * g + j;
                    st[kb][j] = visible(kr) ? st[kb][j] * c : -INFINITY;
                    tm = fmaxf(tm, st[kb][j]);
                }
            const float ts = tm == -INFINITY ? 0.f : tm;  // no visible key yet: every term is 0
            const float sc = __builtin_amdgcn_exp2f(m - ts);
            l *= sc;
            u *= sc;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float e = __builtin_amdgcn_exp2f(st[kb][j] - ts);
                    l += e;
                    u = fmaf(e, dpt[kb][j], u);
                }
            m = tm;
        }
        // combine the four lane groups of the query
        float mall = m;
        mall = fmaxf(mall, __shfl_xor(mall, 16));
        mall = fmaxf(mall, __shfl_xor(mall, 32));
        const float w = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mall);
        float lall = l * w, uall = u * w;
        lall += __shfl_xor(lall, 16);
        lall += __shfl_xor(lall, 32);
        uall += __shfl_xor(uall, 16);
        uall += __shfl_xor(uall, 32);
        if (MODE == 1) {
            if (qvalid && g == 0) {
                a.bstat[rrow * 3 + 0] = mall;
                a.bstat[rrow * 3 + 1] = lall;
                a.bstat[rrow * 3 + 2] = uall;
            }
            return;
        }
        if (Wh > 0 && qvalid) {  // the window's keys join the same softmax
            const float mb = a.bstat[rrow * 3 + 0], lb = a.bstat[rrow * 3 + 1], ub = a.bstat[rrow * 3 + 2];
            const float mn = fmaxf(mall, mb);
            const float wa = mall == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mall - mn);
            const float wb = mb == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mb - mn);
            lall = fmaf(lall, wa, lb * wb);
            uall = fmaf(uall, wa, ub * wb);
            mall = mn;
        }
        lse2 = mall + __log2f(lall);
        delta = uall / lall;
    } else {
        lse2 = qvalid ? a.lse[rrow] * kLog2e : INFINITY;  // (a row past the sequence: p = 0)
        delta = qvalid ? a.delta[rrow] : 0.f;
    }
    // sweep 2: dQ^T
    const int toff = tr_offset<DK>();
    floatx4 dqt[G::DB];
#pragma unroll
    for (int db = 0; db < G::DB; ++db) dqt[db] = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int t = tlo; t < thi; ++t) {
        next_tile();
        floatx4 st[4], dpt[4];
        scores(st, dpt);
        bf16x8 sh[2], sl[2];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int kr = t * kBwdRows + 16 * kb + 4 * g + j;
                const float p = visible(kr) ? __builtin_amdgcn_exp2f(fmaf(st[kb][j], c, -lse2)) : 0.f;
                split_bf16(p * (dpt[kb][j] - delta) * a.scale, sh[kb >> 1], sl[kb >> 1], 4 * (kb & 1) + j);
            }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int db = 0; db < G::DB; ++db) {
                const bf16x8 kf = tr_frag<DK>(kt, toff, db, hh);
                dqt[db] = mfma16(kf, sh[hh], dqt[db]);
                dqt[db] = mfma16(kf, sl[hh], dqt[db]);
            }
    }
    if (qvalid) {
        float* const o = a.dq + qe;  // same [B][T][H][DK] position, fp32
        if (MODE == 2) {  // the dilated share is there already (MODE 0 ran first)
#pragma unroll
            for (int db = 0; db < G::DB; ++db) {
                floatx4* const p = reinterpret_cast<floatx4*>(o + 16 * db + 4 * g);
                *p = *p + dqt[db];
            }
        } else {
#pragma unroll
            for (int db = 0; db < G::DB; ++db) *reinterpret_cast<floatx4*>(o + 16 * db + 4 * g) = dqt[db];
            if (g == 0) {
                a.lse[rrow] = lse2 * 0.6931471805599453f;  // natural log
                a.delta[rrow] = delta;
            }
        }
    }
}

// dk, dv: wave w owns keys 16w .. 16w+15 of the block; lane (g, i) key i.
// Scores S = Q K^T (lane: queries 16qb + 4g + j of its key), dP = dO V^T,
// dV^T += dO^T P and dK^T += Q^T dS with P and dS packed to bf16 as B
// operands.  BAND: the raw tokens of a window against the queries up to
// W - 1 after them (heads without a window write zeros); otherwise the
// states against the queries of their residue.
template <int DK, bool BAND>
__global__ __launch_bounds__(kBwdThreads, 2) void bwd_kv_mfma(BwdArgs a)
{
    typedef Geo<DK> G;
    __shared__ __attribute__((aligned(1024))) char qt[kBwdRows * G::ROWB];
    __shared__ __attribute__((aligned(1024))) char gt[kBwdRows * G::ROWB];
    __shared__ float s_lse2[kBwdRows], s_dl[kBwdRows];
    const int wi = xcd_item(blockIdx.x, gridDim.x);
    const BwdItem it = BAND ? band_item(a, wi) : bwd_item<false>(a, wi);
    if (!it.valid) return;
    const int Wh = a.W[it.h];
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int g = lane >> 4, i = lane & 15;
    const float c = a.scale * kLog2e;
    const int kr = it.blk * kBwdOwn + 16 * wv + i;
    const bool kvalid = kr < it.M;
    const size_t ke = kvalid ? res_row<DK>(a, it, kr) : 0;
    float* const dko = BAND ? a.dk : a.dks;
    float* const dvo = BAND ? a.dv : a.dvs;
    if (BAND && Wh == 0) {  // no window: the raw keys take no gradient from attention
        if (kvalid) {
#pragma unroll
            for (int db = 0; db < G::DB; ++db) {
                *reinterpret_cast<floatx4*>(dko + ke + 16 * db + 4 * g) = floatx4{0.f, 0.f, 0.f, 0.f};
                *reinterpret_cast<floatx4*>(dvo + ke + 16 * db + 4 * g) = floatx4{0.f, 0.f, 0.f, 0.f};
            }
        }
        return;
    }
    bf16x8 kf[G::KS], vf[G::KS];
    load_frag<DK>(kf, BAND ? a.k : a.ks, ke, kvalid);
    load_frag<DK>(vf, BAND ? a.v : a.vs, ke, kvalid);
    const int toff = tr_offset<DK>();
    floatx4 dkt[G::DB], dvt[G::DB];
#pragma unroll
    for (int db = 0; db < G::DB; ++db) {
        dkt[db] = floatx4{0.f, 0.f, 0.f, 0.f};
        dvt[db] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    // query tiles from the one holding the block's first key, to the one
    // holding the last query that sees the block's last key
    const int ntile = BAND ? (min(it.M, it.blk * kBwdOwn + kBwdOwn - 1 + Wh) - 1) / kBwdRows + 1
                           : (it.M + kBwdRows - 1) / kBwdRows;
    // query row q sees the lane's key: from it on, within the window
    auto sees = [&](int q) { return q >= kr && (!BAND || q < kr + Wh); };
    // query tiles from the block's own on, staged through registers
    TileRegs<DK> rq, rg;
    float rl = INFINITY, rd = 0.f;  // the tile's (lse, delta) of row threadIdx.x (< 64)
    auto fetch = [&](int t) {
        rq.load(a.q, a, it, t * kBwdRows);
        rg.load(a.dout, a, it, t * kBwdRows);
        const int q = t * kBwdRows + threadIdx.x;
        rl = INFINITY;  // rows past the residue: p = 0
        rd = 0.f;
        if (threadIdx.x < kBwdRows && q < it.M) {
            const size_t rrow = ((size_t)it.b * a.T + it.r + (size_t)q * it.D) * a.H + it.h;
            rl = a.lse[rrow] * kLog2e;
            rd = a.delta[rrow];
        }
    };
    const int t0 = it.blk * kBwdOwn / kBwdRows;  // the tile holding the block's first key
    fetch(t0);
    for (int t = t0; t < ntile; ++t) {
        __syncthreads();
        rq.store(qt);
        rg.store(gt);
        if (threadIdx.x < kBwdRows) {
            s_lse2[threadIdx.x] = rl;
            s_dl[threadIdx.x] = rd;
        }
        __syncthreads();
        if (t + 1 < ntile) fetch(t + 1);
        bf16x8 pb[2], sh[2], sl[2];
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) {
            floatx4 sv = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < G::KS; ++ks) {
                sv = mfma16(lds_b128(qt + swz<DK>(16 * qb + i, g + 4 * ks)), kf[ks], sv);
                dp = mfma16(lds_b128(gt + swz<DK>(16 * qb + i, g + 4 * ks)), vf[ks], dp);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int ql = 16 * qb + 4 * g + j;
                const int q = t * kBwdRows + ql;
                const float p = sees(q) ? __builtin_amdgcn_exp2f(fmaf(sv[j], c, -s_lse2[ql])) : 0.f;
                pb[qb >> 1][4 * (qb & 1) + j] = (__bf16)p;
                split_bf16(p * (dp[j] - s_dl[ql]) * a.scale, sh[qb >> 1], sl[qb >> 1], 4 * (qb & 1) + j);
            }
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int db = 0; db < G::DB; ++db) {
                dvt[db] = mfma16(tr_frag<DK>(gt, toff, db, hh), pb[hh], dvt[db]);
                const bf16x8 qf = tr_frag<DK>(qt, toff, db, hh);
                dkt[db] = mfma16(qf, sh[hh], dkt[db]);
                dkt[db] = mfma16(qf, sl[hh], dkt[db]);
            }
    }
    if (kvalid) {
#pragma unroll
        for (int db = 0; db < G::DB; ++db) {
            *reinterpret_cast<floatx4*>(dko + ke + 16 * db + 4 * g) = dkt[db];
            *reinterpret_cast<floatx4*>(dvo + ke + 16 * db + 4 * g) = dvt[db];
        }
    }
}

// ---------------------------------------------------------------- recurrence
// Thread (chunk, b, channel), channel fastest.
struct ChunkPos {
    int c, b, n;
    size_t cell;  // (chunk * B + b) * N + n: index of the chunk's scalars
};
__device__ __forceinline__ bool chunk_pos(const BwdArgs& a, ChunkPos& p)
{
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t N = (size_t)a.H * a.d;
    if (idx >= (size_t)a.nchunk * a.B * N) return false;
    p.n = (int)(idx % N);
    const size_t rest = idx / N;
    p.b = (int)(rest % a.B);
    p.c = (int)(rest / a.B);
    p.cell = idx;
    return true;
}

__device__ __forceinline__ bool restart_at(const BwdArgs& a, int t) { return a.L > 0 && t % a.L == 0; }

// Per chunk: the forward map h_end = A h_before + (K, V) from a zero state,
// and the backward carry map mu_out = A mu_in + (Bk, Bv), mu being the
// gradient that flows into a token from its successor (g_{t+1} lambda_{t+1}).
// Both share A, the product of the chunk's gates with restarts zeroing it.
template <typename E>
__global__ __launch_bounds__(256) void bwd_scan_maps_kernel(BwdArgs a)
{
    ChunkPos p;
    if (!chunk_pos(a, p)) return;
    const size_t N = (size_t)a.H * a.d;
    const int t0 = p.c * kBwdChunk, n = min(kBwdChunk, a.T - t0);
    const size_t x0 = ((size_t)p.b * a.T + t0) * N + p.n;
    float A = 1.f, K = 0.f, V = 0.f;
    float Bk = 0.f, Bv = 0.f;  // carry out of the chunk's first token with a zero carry in
    // a whole chunk takes the form without the per-token bound, whose loads
    // can all be in flight at once; the last, ragged chunk the guarded form
    auto walk = [&](auto whole) {
        constexpr bool FULL = decltype(whole)::value;
#pragma unroll
        for (int i = 0; i < kBwdChunk; ++i) {
            if (FULL || i < n) {
                const size_t x = x0 + (size_t)i * N;
                float g, gb;
                forget_gate(ldx<E>(a.g, x), g, gb);
                if (restart_at(a, t0 + i)) { A = 0.f; K = 0.f; V = 0.f; }
                A *= g;
                K = fmaf(g, K, gb * ldx<E>(a.k, x));
                V = fmaf(g, V, gb * ldx<E>(a.v, x));
            }
        }
#pragma unroll
        for (int i = kBwdChunk - 1; i >= 0; --i) {
            if (FULL || i < n) {
                const size_t x = x0 + (size_t)i * N;
                float g, gb;
                forget_gate(ldx<E>(a.g, x), g, gb);
                const float lk = a.dks[x] + Bk, lv = a.dvs[x] + Bv;
                const bool cut = restart_at(a, t0 + i);
                Bk = cut ? 0.f : g * lk;
                Bv = cut ? 0.f : g * lv;
            }
        }
    };
    if (n == kBwdChunk) walk(BoolC<true>{});
    else walk(BoolC<false>{});
    float* m = a.maps + p.cell * 5;
    m[0] = A; m[1] = K; m[2] = V; m[3] = Bk; m[4] = Bv;
}

// Per (b, channel), over its chunks: the state before each chunk (forward)
// and the carry into each chunk's last token (backward).  A workgroup takes
// 16 channels x 16 runs of consecutive chunks: each thread composes the maps
// of its run, the runs' carries are chained through LDS, then each thread
// walks its run again writing the per-chunk carries.
constexpr int kCarryRuns = 16;
__global__ __launch_bounds__(256) void bwd_scan_carry_kernel(BwdArgs a)
{
    __shared__ float s_run[kCarryRuns][16][5];   // run maps (A, K, V, Bk, Bv)
    __shared__ float s_in[kCarryRuns][16][4];    // state before / carry into each run
    const size_t N = (size_t)a.H * a.d;
    const int ch = threadIdx.x % 16, run = threadIdx.x / 16;
    const size_t idx = (size_t)blockIdx.x * 16 + ch;  // (b, channel)
    const bool valid = idx < (size_t)a.B * N;
    const size_t stride = (size_t)a.B * N;  // between chunks
    const float* __restrict__ maps = a.maps;
    float* __restrict__ carry = a.carry;
    const int per = (a.nchunk + kCarryRuns - 1) / kCarryRuns;
    const int c0 = run * per, c1 = min(c0 + per, a.nchunk);
    // compose the run: forward h -> A h + (K, V) over c0 .. c1 - 1, backward
    // mu -> A mu + (Bk, Bv) over c1 - 1 .. c0 (the same A)
    float A = 1.f, K = 0.f, V = 0.f, Bk = 0.f, Bv = 0.f;
    if (valid) {
        for (int c = c0; c < c1; ++c) {
            const float* m = maps + ((size_t)c * stride + idx) * 5;
            K = fmaf(m[0], K, m[1]);
            V = fmaf(m[0], V, m[2]);
            A *= m[0];
        }
        // the carry out of chunk c0 weighs chunk c's own term by the gates
        // of the chunks before it in the run: Bk = sum_c (prod_{c0 <= c' < c} A_c') Bk_c
        float Ar = 1.f;
        for (int c = c0; c < c1; ++c) {
            const float* m = maps + ((size_t)c * stride + idx) * 5;
            Bk = fmaf(Ar, m[3], Bk);
            Bv = fmaf(Ar, m[4], Bv);
            Ar *= m[0];
        }
    }
    s_run[run][ch][0] = A;
    s_run[run][ch][1] = K;
    s_run[run][ch][2] = V;
    s_run[run][ch][3] = Bk;
    s_run[run][ch][4] = Bv;
    __syncthreads();
    if (run == 0) {  // chain the runs of this channel
        float hk = 0.f, hv = 0.f;
        for (int r = 0; r < kCarryRuns; ++r) {
            s_in[r][ch][0] = hk;
            s_in[r][ch][1] = hv;
            hk = fmaf(s_run[r][ch][0], hk, s_run[r][ch][1]);
            hv = fmaf(s_run[r][ch][0], hv, s_run[r][ch][2]);
        }
        float mk = 0.f, mv = 0.f;
        for (int r = kCarryRuns - 1; r >= 0; --r) {
            s_in[r][ch][2] = mk;
            s_in[r][ch][3] = mv;
            mk = fmaf(s_run[r][ch][0], mk, s_run[r][ch][3]);
            mv = fmaf(s_run[r][ch][0], mv, s_run[r][ch][4]);
        }
    }
    __syncthreads();
    if (!valid) return;
    float hk = s_in[run][ch][0], hv = s_in[run][ch][1];
    for (int c = c0; c < c1; ++c) {
        const size_t cell = (size_t)c * stride + idx;
        const float* m = maps + cell * 5;
        carry[cell * 4 + 0] = hk;
        carry[cell * 4 + 1] = hv;
        hk = fmaf(m[0], hk, m[1]);
        hv = fmaf(m[0], hv, m[2]);
    }
    float mk = s_in[run][ch][2], mv = s_in[run][ch][3];
    for (int c = c1 - 1; c >= c0; --c) {
        const size_t cell = (size_t)c * stride + idx;
        const float* m = maps + cell * 5;
        carry[cell * 4 + 2] = mk;
        carry[cell * 4 + 3] = mv;
        mk = fmaf(m[0], mk, m[3]);
        mv = fmaf(m[0], mv, m[4]);
    }
}

// Per chunk: the fp32 states again from the chunk's start state, then the
// chunk walked backwards.  With a raw window somewhere, dk / dv already hold
// the raw-window gradients and are added to; otherwise they are written.
template <typename E>
__global__ __launch_bounds__(256) void bwd_scan_apply_kernel(BwdArgs a)
{
    ChunkPos p;
    if (!chunk_pos(a, p)) return;
    const size_t N = (size_t)a.H * a.d;
    const int t0 = p.c * kBwdChunk, n = min(kBwdChunk, a.T - t0);
    const float* cr = a.carry + p.cell * 4;
    float hk[kBwdChunk + 1], hv[kBwdChunk + 1];  // hk[i] = state before token t0 + i
    hk[0] = cr[0];
    hv[0] = cr[1];
#pragma unroll
    for (int i = 0; i < kBwdChunk; ++i) {
        if (i < n) {
            const size_t x = ((size_t)p.b * a.T + t0 + i) * N + p.n;
            float g, gb;
            forget_gate(ldx<E>(a.g, x), g, gb);
            const bool cut = restart_at(a, t0 + i);
            hk[i + 1] = fmaf(g, cut ? 0.f : hk[i], gb * ldx<E>(a.k, x));
            hv[i + 1] = fmaf(g, cut ? 0.f : hv[i], gb * ldx<E>(a.v, x));
        } else {
            hk[i + 1] = 0.f;
            hv[i + 1] = 0.f;
        }
    }
    float mk = cr[2], mv = cr[3];
#pragma unroll
    for (int i = kBwdChunk - 1; i >= 0; --i) {
        if (i < n) {
            const int t = t0 + i;
            const size_t x = ((size_t)p.b * a.T + t) * N + p.n;
            float g, gb;
            forget_gate(ldx<E>(a.g, x), g, gb);
            const bool cut = restart_at(a, t);
            const float lk = a.dks[x] + mk, lv = a.dvs[x] + mv;
            a.dk[x] = a.raw ? fmaf(gb, lk, a.dk[x]) : gb * lk;
            a.dv[x] = a.raw ? fmaf(gb, lv, a.dv[x]) : gb * lv;
            const float pk = (cut || t == 0) ? 0.f : hk[i], pv = (cut || t == 0) ? 0.f : hv[i];
            a.dg[x] = g * gb * (lk * (pk - ldx<E>(a.k, x)) + lv * (pv - ldx<E>(a.v, x)));
            mk = cut ? 0.f : g * lk;
            mv = cut ? 0.f : g * lv;
        }
    }
}

// SLIDING window below T: each state is its own window of L tokens, so the
// state gradients lambda (from the attention) carry nothing.  Per token u
// and channel, with P(a, b) = g_a ... g_b:
//   mu = sum_{t = u .. u+L-1} lambda_t P(u+1, t),   dx_u = (1 - g_u) mu,
//   dlogit_u = g_u (1 - g_u) sum_{x in k, v} (sum_t lambda_t P(u+1, t) C_t - x_u mu),
// C_t = sum_{s = max(0, t-L+1) .. u-1} P(s+1, u-1) (1 - g_s) x_s being the
// window of t up to u - 1.  The products are exponentials of window-local
// sums of log g (no division by a gate, no overflow): one pass over s < u
// forms C for t = u, a second over t >= u drops each s as it leaves the
// window.  One thread per (b, u, channel), channel fastest.
template <typename E>
__global__ __launch_bounds__(256) void bwd_slide_kernel(BwdArgs a)
{
    const size_t N = (size_t)a.H * a.d;
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (size_t)a.B * a.T * N) return;
    const size_t n = idx % N, bt = idx / N;
    const int T = a.T, L = a.L;
    const int u = (int)(bt % T), b = (int)(bt / T);
    auto at = [&](int t) { return ((size_t)b * T + t) * N + n; };
    // log g = -softplus(-logit), held above -80 (a gate below e^-80 is 0 here)
    auto log_gate = [](float l) { return fmaxf(-(fmaxf(-l, 0.f) + log1pf(__expf(-fabsf(l)))), -80.f); };
    const int lo = max(0, u - L + 1);
    float R = 0.f, ck = 0.f, cv = 0.f;  // R: sum of log g over s+1 .. u-1
    for (int s = u - 1; s >= lo; --s) {
        const size_t i = at(s);
        const float l = ldx<E>(a.g, i);
        float g, gb;
        forget_gate(l, g, gb);
        const float e = __expf(R);
        ck = fmaf(gb * ldx<E>(a.k, i), e, ck);
        cv = fmaf(gb * ldx<E>(a.v, i), e, cv);
        R += log_gate(l);
    }
    // the next s to leave the window, and its R (sum over s+1 .. u-1)
    int sr = lo;
    float rs = lo <= u - 1 ? R - log_gate(ldx<E>(a.g, at(lo))) : 0.f;
    const int tmax = min(T - 1, u + L - 1);
    float F = 0.f, mk = 0.f, mv = 0.f, sk = 0.f, sv = 0.f;  // F: sum of log g over u+1 .. t
    for (int t = u; t <= tmax; ++t) {
        if (t > u) {
            F += log_gate(ldx<E>(a.g, at(t)));
            if (t - L >= 0) {  // s = t - L (= sr) is not in the window of t
                const size_t i = at(sr);
                float g, gb;
                forget_gate(ldx<E>(a.g, i), g, gb);
                const float e = __expf(rs);
                ck = fmaf(-gb * ldx<E>(a.k, i), e, ck);
                cv = fmaf(-gb * ldx<E>(a.v, i), e, cv);
                ++sr;
                if (sr <= u - 1) rs -= log_gate(ldx<E>(a.g, at(sr)));
            }
        }
        const size_t it = at(t);
        const float p = __expf(F);
        const float lk = a.dks[it] * p, lv = a.dvs[it] * p;
        mk += lk;
        mv += lv;
        sk = fmaf(lk, ck, sk);
        sv = fmaf(lv, cv, sv);
    }
    const size_t iu = at(u);
    float g, gb;
    forget_gate(ldx<E>(a.g, iu), g, gb);
    a.dk[iu] = a.raw ? fmaf(gb, mk, a.dk[iu]) : gb * mk;
    a.dv[iu] = a.raw ? fmaf(gb, mv, a.dv[iu]) : gb * mv;
    a.dg[iu] = g * gb * (sk - ldx<E>(a.k, iu) * mk + sv - ldx<E>(a.v, iu) * mv);
}

// The same for windows of up to kSlideMaxL tokens, from an LDS tile: a
// workgroup takes kSlideTok tokens of kSlideCh channels (one thread each)
// and first stages, for every token its windows reach, the gate, 1 - gate,
// log gate, k, v and the two state gradients.  A wave's reads then fall on
// 64 consecutive words (eight tokens of eight channels).
constexpr int kSlideTok = 32, kSlideCh = 8, kSlideMaxL = 64;
constexpr int kSlideSpan = kSlideTok + 2 * (kSlideMaxL - 1);
static_assert(kSlideTok * kSlideCh == 256, "one thread per tile element");

template <typename E>
__global__ __launch_bounds__(256) void bwd_slide_tiled_kernel(BwdArgs a, int ubase)
{
    __shared__ float s_g[kSlideSpan][kSlideCh], s_gb[kSlideSpan][kSlideCh], s_lg[kSlideSpan][kSlideCh];
    __shared__ float s_k[kSlideSpan][kSlideCh], s_v[kSlideSpan][kSlideCh];
    __shared__ float s_lk[kSlideSpan][kSlideCh], s_lv[kSlideSpan][kSlideCh];
    const size_t N = (size_t)a.H * a.d;
    const int T = a.T, L = a.L;
    const size_t n0 = (size_t)blockIdx.x * kSlideCh;
    const int u0 = ubase + blockIdx.y * kSlideTok, b = blockIdx.z;
    // tokens ts .. te: the windows of the tile's first token back, of its last forward
    const int ts = max(0, u0 - (L - 1)), te = min(T - 1, u0 + kSlideTok - 1 + (L - 1));
    const int span = te - ts + 1;
    for (int idx = threadIdx.x; idx < span * kSlideCh; idx += kSlideTok * kSlideCh) {
        const int j = idx / kSlideCh, c = idx % kSlideCh;
        float g = 0.f, gb = 0.f, lg = 0.f, k = 0.f, v = 0.f, lk = 0.f, lv = 0.f;
        if (n0 + c < N) {
            const size_t i = ((size_t)b * T + ts + j) * N + n0 + c;
            const float l = ldx<E>(a.g, i);
            forget_gate(l, g, gb);
            lg = fmaxf(-(fmaxf(-l, 0.f) + log1pf(__expf(-fabsf(l)))), -80.f);
            k = ldx<E>(a.k, i);
            v = ldx<E>(a.v, i);
            lk = a.dks[i];
            lv = a.dvs[i];
        }
        s_g[j][c] = g;
        s_gb[j][c] = gb;
        s_lg[j][c] = lg;
        s_k[j][c] = k;
        s_v[j][c] = v;
        s_lk[j][c] = lk;
        s_lv[j][c] = lv;
    }
    __syncthreads();
    const int c = threadIdx.x % kSlideCh, u = u0 + threadIdx.x / kSlideCh;
    if (u >= T || n0 + c >= N) return;
    const int lo = max(0, u - L + 1);
    // pass 1 over s = u-1 .. lo: C for t = u, with P = P(s+1, u-1) as a product
    float P = 1.f, R = 0.f, ck = 0.f, cv = 0.f;
    for (int s = u - 1; s >= lo; --s) {
        const int j = s - ts;
        ck = fmaf(s_gb[j][c] * s_k[j][c], P, ck);
        cv = fmaf(s_gb[j][c] * s_v[j][c], P, cv);
        P *= s_g[j][c];
        R += s_lg[j][c];
    }
    int sr = lo;
    float rs = lo <= u - 1 ? R - s_lg[lo - ts][c] : 0.f;
    const int tmax = min(T - 1, u + L - 1);
    float P2 = 1.f, mk = 0.f, mv = 0.f, sk = 0.f, sv = 0.f;
    for (int t = u; t <= tmax; ++t) {
        const int j = t - ts;
        if (t > u) {
            P2 *= s_g[j][c];
            if (t - L >= 0) {  // s = t - L (= sr) is not in the window of t
                const int jr = sr - ts;
                const float e = __expf(rs);
                ck = fmaf(-s_gb[jr][c] * s_k[jr][c], e, ck);
                cv = fmaf(-s_gb[jr][c] * s_v[jr][c], e, cv);
                ++sr;
                if (sr <= u - 1) rs -= s_lg[sr - ts][c];
            }
        }
        const float lk = s_lk[j][c] * P2, lv = s_lv[j][c] * P2;
        mk += lk;
        mv += lv;
        sk = fmaf(lk, ck, sk);
        sv = fmaf(lv, cv, sv);
    }
    const int ju = u - ts;
    const float g = s_g[ju][c], gb = s_gb[ju][c];
    const size_t iu = ((size_t)b * T + u) * N + n0 + c;
    a.dk[iu] = a.raw ? fmaf(gb, mk, a.dk[iu]) : gb * mk;
    a.dv[iu] = a.raw ? fmaf(gb, mv, a.dv[iu]) : gb * mv;
    a.dg[iu] = g * gb * (sk - s_k[ju][c] * mk + sv - s_v[ju][c] * mv);
}

// Windows of exactly kSlideMaxL = 64 tokens, by tiles of 64 tokens (a tile
// starts at a = 64 k) whose neighbour tiles lie inside the sequence: every
// quantity of a tile comes from the tile and its two neighbours, with no
// carry between tiles.  With lambda the state gradient and P(r, s) =
// g_r ... g_s, for a token u of the tile:
//   h_u  = H_u + P(a, u) Y_{u-63}: the window's state; H runs the tile's own
//          recurrence from zero, Y_j sums the previous tile's terms s >= j
//          carried to a - 1 (P(s+1, a-1) (1 - g_s) x_s);
//   mu_u = sum_{t = u .. u+63} lambda_t P(u+1, t) = M_u + P(u+1, a+63) F_{u+63}:
//          M the tile's own reverse sum, F the next tile's prefix sum of
//          lambda_t P(a+64, t);
//   Z_u  = the sum of lambda_t (1 - g_s) x_s P(s+1, t) over the pairs
//          s < u <= t, t - s < 64.  Going from u+1 to u, the pairs that end at
//          u join (lambda_u (h_u - (1 - g_u) x_u)) and those that start at u
//          leave ((1 - g_u) x_u (mu_u - lambda_u)), so Z_u is the tile's suffix
//          sum of lambda_v h_v - (1 - g_v) x_v mu_v on top of Z at the next
//          tile's start, sum_{s in tile} (1 - g_s) x_s P(s+1, a+63) F_{s+63}.
// Then dx_u = (1 - g_u) mu_u and dlogit_u = (1 - g_u) (Z_u - g_u x_u mu_u),
// summed over x in k, v: the gradient through every gate factor of every
// window that holds u, with no division by a gate.
// Each wave takes kSlideSub consecutive tokens of the tile, and lane 2c + x
// channel c of tensor x (k, v) of 32 channels; a wave also walks as many
// positions of the previous tile, those its tokens' windows start from
// (j = u - 63), and of the next tile, those their gradients end at
// (t = u + 63).  The waves exchange the affine maps of their positions in
// each chain through LDS, then the tile's suffix sums.
// tokens per wave of the 64-token tile kernels, and their waves per tile:
// eight waves of 8 tokens for both (same-box A/B at the 16K windowed shape:
// SLIDING, with every input loaded once up front, 382 / 370 us at sixteen /
// eight waves; RESTART 318 / 252 / 321 us at four / eight / sixteen)
constexpr int kSlideSub = 8;
constexpr int kSlideWaves = kSlideMaxL / kSlideSub;
constexpr int kRestartSub = 8;
constexpr int kRestartWaves = kSlideMaxL / kRestartSub;

template <typename E>
__global__ __launch_bounds__(kSlideWaves * kWave) void bwd_slide64_kernel(BwdArgs a)
{
    constexpr int LT = kSlideMaxL, SUB = kSlideSub;
    constexpr int NWV = kSlideWaves;
    __shared__ float s_map[NWV][7][kWave];  // per wave: H end, P own, Y sum, P prev, N sum, F sum, P next
    __shared__ float s_fin[NWV][2][kWave];  // per wave: its sum of z, its part of Z at the next tile
    const size_t N = (size_t)a.H * a.d;
    const int T = a.T;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
    const int xv = lane & 1;  // 0: k, 1: v
    // workgroup: (b, tile 1 + k, block of 32 channels), channels fastest, so
    // the tiles that re-read one tile run close together
    const unsigned ncb = (unsigned)((N + 31) / 32), ntile = (unsigned)(T / LT - 2);
    const unsigned cb = blockIdx.x % ncb, rest = blockIdx.x / ncb;
    const int a0 = (int)(1 + rest % ntile) * LT, b = (int)(rest / ntile);
    const size_t n = (size_t)cb * 32 + lane / 2;
    const bool cok = n < N;
    // a lane past the last channel reads the last channel's words and writes nothing
    const size_t base = (size_t)b * T * N + (cok ? n : N - 1);
    const void* xp = xv ? a.v : a.k;
    const float* lam = xv ? a.dvs : a.dks;
    float* dx = xv ? a.dv : a.dk;
    auto at = [&](int t) { return base + (size_t)t * N; };
    const int u0 = a0 + SUB * w;           // the wave's tokens u0 .. u0 + SUB - 1
    const int j0 = u0 - (LT - 1);          // j = u - 63; j = a0 (last wave) adds no term
    const int t0 = u0 + (LT - 1);          // t = u + 63; t = a0 + 63 (wave 0) adds no term
    // Those two positions are loaded like the others (both lie in the tile)
    // and enter as a factor 1 and a term 0, without a branch.
    const bool p_last = w == NWV - 1, n_first = w == 0;

    // 0. every input of the wave's positions, loaded once, together (one
    // memory round trip per workgroup): the own tokens' gate, x, lambda (and
    // the raw windows' dx), the previous tile's gate and x, the next tile's
    // gate and lambda
    float go[SUB], gbo[SUB], xo[SUB], lo[SUB], dxr[SUB];
    float gpv[SUB], gbp[SUB], xpv[SUB], gnx[SUB], lnx[SUB];
#pragma unroll
    for (int i = 0; i < SUB; ++i) {
        const size_t e = at(u0 + i), ep = at(j0 + i), en = at(t0 + i);
        forget_gate(ldx<E>(a.g, e), go[i], gbo[i]);
        xo[i] = ldx<E>(xp, e);
        lo[i] = lam[e];
        dxr[i] = a.raw ? dx[e] : 0.f;
        forget_gate(ldx<E>(a.g, ep), gpv[i], gbp[i]);
        xpv[i] = ldx<E>(xp, ep);
        float gb;
        forget_gate(ldx<E>(a.g, en), gnx[i], gb);
        lnx[i] = lam[en];
    }
    if (p_last) {
        gpv[SUB - 1] = 1.f;
        gbp[SUB - 1] = 0.f;
    }
    if (n_first) {
        gnx[0] = 1.f;
        lnx[0] = 0.f;
    }

    // 1. the maps of the wave's positions in each chain, from zero
    float Hl = 0.f, Po = 1.f;  // own tokens forwards: H at the end, the gate product
#pragma unroll
    for (int i = 0; i < SUB; ++i) {
        Hl = fmaf(go[i], Hl, gbo[i] * xo[i]);
        Po *= go[i];
    }
    // own tokens backwards: N_u = g_u (lambda_u + N_{u+1}) from N = 0 after the last
    float Nl = 0.f;
#pragma unroll
    for (int i = SUB - 1; i >= 0; --i) Nl = go[i] * (lo[i] + Nl);
    float Yl = 0.f, Pp = 1.f;  // previous tile backwards
#pragma unroll
    for (int i = SUB - 1; i >= 0; --i) {
        Yl = fmaf(gbp[i] * xpv[i], Pp, Yl);
        Pp *= gpv[i];
    }
    float Fl = 0.f, Pn = 1.f;  // next tile forwards
#pragma unroll
    for (int i = 0; i < SUB; ++i) {
        Pn *= gnx[i];
        Fl = fmaf(lnx[i], Pn, Fl);
    }
    s_map[w][0][lane] = Hl;
    s_map[w][1][lane] = Po;
    s_map[w][2][lane] = Yl;
    s_map[w][3][lane] = Pp;
    s_map[w][4][lane] = Nl;
    s_map[w][5][lane] = Fl;
    s_map[w][6][lane] = Pn;
    __syncthreads();
    // 2. the carries: from the waves before (H, F) and after (Y, N, products)
    float Hc = 0.f, Pa = 1.f;  // H before u0, P(a, u0 - 1)
    float Fc = 0.f, Pf = 1.f;  // F before t0, P(a + 64, t0 - 1)
    for (int v = 0; v < w; ++v) {
        Hc = fmaf(s_map[v][1][lane], Hc, s_map[v][0][lane]);
        Pa *= s_map[v][1][lane];
        Fc = fmaf(Pf, s_map[v][5][lane], Fc);
        Pf *= s_map[v][6][lane];
    }
    float Yc = 0.f, Py = 1.f;  // Y after j0 + SUB - 1, P(j0 + SUB, a - 1)
    float Nc = 0.f, Ps = 1.f;  // N after u0 + SUB - 1, P(u0 + SUB, a + 63)
    for (int v = NWV - 1; v > w; --v) {
        Yc = fmaf(Py, s_map[v][2][lane], Yc);
        Py *= s_map[v][3][lane];
        Nc = fmaf(s_map[v][1][lane], Nc, s_map[v][4][lane]);
        Ps *= s_map[v][1][lane];
    }
    // 3. forwards: H, P(a, u) and F at the wave's positions
    float HH[SUB], PP[SUB], FF[SUB];
    float Hs = Hc, Pu = Pa, Fs = Fc, Pq = Pf;
#pragma unroll
    for (int i = 0; i < SUB; ++i) {
        Hs = fmaf(go[i], Hs, gbo[i] * xo[i]);
        Pu *= go[i];
        HH[i] = Hs;
        PP[i] = Pu;
        Pq *= gnx[i];
        Fs = fmaf(lnx[i], Pq, Fs);
        FF[i] = Fs;
    }
    // 4. backwards: Y, M, mu; dx; the suffix sum of z and the part of Z at the next tile
    float W[SUB];
    float Ys = Yc, Pys = Py, Nn = Nc, SP = Ps, Sl = 0.f, Zp = 0.f;
#pragma unroll
    for (int i = SUB - 1; i >= 0; --i) {
        Ys = fmaf(gbp[i] * xpv[i], Pys, Ys);
        Pys *= gpv[i];
        const size_t e = at(u0 + i);
        const float x = xo[i], l = lo[i];
        const float h = fmaf(PP[i], Ys, HH[i]);
        const float M = l + Nn;
        Nn = go[i] * M;
        if (i < SUB - 1) SP *= go[i + 1];
        const float G = SP * FF[i];
        const float mu = M + G;
        if (cok) dx[e] = a.raw ? fmaf(gbo[i], mu, dxr[i]) : gbo[i] * mu;
        const float xm = gbo[i] * x * mu;
        Sl += fmaf(l, h, -xm);
        Zp = fmaf(gbo[i] * x, G, Zp);
        W[i] = fmaf(gbo[i], Sl, -go[i] * xm);
    }
    s_fin[w][0][lane] = Sl;
    s_fin[w][1][lane] = Zp;
    __syncthreads();
    // 5. Z = Z at the next tile + the suffix sums of the waves after + the wave's own
    float add = 0.f;
    for (int v = 0; v < NWV; ++v) add += s_fin[v][1][lane] + (v > w ? s_fin[v][0][lane] : 0.f);
#pragma unroll
    for (int i = 0; i < SUB; ++i) {
        const float part = fmaf(gbo[i], add, W[i]);
        const float other = __shfl_xor(part, 1);
        if (cok && xv == 0) a.dg[at(u0 + i)] = part + other;
    }
}

// RESTART at L = kSlideMaxL: every 64-token tile is one window, so a tile's
// gradients need nothing outside it.  Per token u of the tile (a = its
// start), with Lambda_u = lambda_u + g_{u+1} Lambda_{u+1} (Lambda past the
// tile's end 0) the gradient that reaches the state h_u:
//   dx_u = (1 - g_u) Lambda_u,   dlogit_u = g_u (1 - g_u) Lambda_u (h_{u-1} - x_u),
// summed over x in k, v, with h_{a-1} = 0.  A workgroup takes the tile for
// 32 channels: it first copies the tile's rows of every input (gate
// logits, k, v, the two state gradients, and dk / dv when the raw windows
// have written them) into LDS with 16-byte loads, so that many bytes are in
// flight per load, then each wave takes kRestartSub tokens (lane 2c + x:
// channel c, tensor k or v) and the waves exchange the maps of their tokens in the
// forward state chain and the backward gradient chain through LDS.  Rows
// past T are zero and enter as a factor 1 and a term 0.  dk, dv and dlogit
// go back through LDS and leave with 16-byte stores.
constexpr int kTileCh = 32;  // channels per workgroup of the 64-token tile kernels

// Copies rows r0 .. r0 + nrows - 1 of a [B*T][N] tensor's channel segment
// c0 .. c0 + kTileCh - 1 (EB bytes per element) into LDS, rows past T as
// zero, 16 bytes per lane.
template <int EB>
__device__ __forceinline__ void stage_rows(const void* src, char* dst, size_t rowbase, int t0, int nrows, int T,
                                           size_t N, size_t c0)
{
    constexpr int RB = kTileCh * EB, PR = RB / 16;  // bytes and 16-byte pieces per row
    for (int idx = threadIdx.x; idx < nrows * PR; idx += blockDim.x) {
        const int r = idx / PR, p = idx % PR;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (t0 + r < T && t0 + r >= 0)
            v = *reinterpret_cast<const u32x4*>(static_cast<const char*>(src) +
                                                ((rowbase + t0 + r) * N + c0) * EB + 16 * p);
        *reinterpret_cast<u32x4*>(dst + r * RB + 16 * p) = v;
    }
}

// The reverse: fp32 rows of LDS back to a [B*T][N] tensor's channel
// segment, rows at or past T skipped.
__device__ __forceinline__ void unstage_rows(const char* src, float* dst, size_t rowbase, int t0, int nrows, int T,
                                             size_t N, size_t c0)
{
    constexpr int RB = kTileCh * 4, PR = RB / 16;
    for (int idx = threadIdx.x; idx < nrows * PR; idx += blockDim.x) {
        const int r = idx / PR, p = idx % PR;
        if (t0 + r < T)
            *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(dst) + ((rowbase + t0 + r) * N + c0) * 4 + 16 * p) =
                *reinterpret_cast<const u32x4*>(src + r * RB + 16 * p);
    }
}

template <typename E>
__global__ __launch_bounds__(kRestartWaves * kWave) void bwd_restart64_kernel(BwdArgs a)
{
    constexpr int LT = kSlideMaxL, SUB = kRestartSub, EB = (int)sizeof(E);
    constexpr int RE = kTileCh * EB, RF = kTileCh * 4;  // row bytes: inputs, fp32 gradients
    __shared__ __attribute__((aligned(16))) char s_g[LT * RE], s_k[LT * RE], s_v[LT * RE];
    __shared__ __attribute__((aligned(16))) char s_lk[LT * RF], s_lv[LT * RF], s_dk[LT * RF], s_dv[LT * RF];
    constexpr int NWV = kRestartWaves;
    __shared__ float s_map[NWV][3][kWave];  // per wave: H end, gate product, N sum
    const size_t N = (size_t)a.H * a.d;
    const int T = a.T;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
    const int xv = lane & 1;  // 0: k, 1: v
    const unsigned ncb = (unsigned)(N / kTileCh), ntile = (unsigned)((T + LT - 1) / LT);
    const unsigned cb = blockIdx.x % ncb, rest = blockIdx.x / ncb;
    const int a0 = (int)(rest % ntile) * LT, b = (int)(rest / ntile);
    const size_t c0 = (size_t)cb * kTileCh, rowbase = (size_t)b * T;
    stage_rows<EB>(a.g, s_g, rowbase, a0, LT, T, N, c0);
    stage_rows<EB>(a.k, s_k, rowbase, a0, LT, T, N, c0);
    stage_rows<EB>(a.v, s_v, rowbase, a0, LT, T, N, c0);
    stage_rows<4>(a.dks, s_lk, rowbase, a0, LT, T, N, c0);
    stage_rows<4>(a.dvs, s_lv, rowbase, a0, LT, T, N, c0);
    if (a.raw) {
        stage_rows<4>(a.dk, s_dk, rowbase, a0, LT, T, N, c0);
        stage_rows<4>(a.dv, s_dv, rowbase, a0, LT, T, N, c0);
    }
    __syncthreads();
    const int c = lane / 2;
    const char* sx = xv ? s_v : s_k;
    const float* sl = reinterpret_cast<const float*>(xv ? s_lv : s_lk);
    const float* sd = reinterpret_cast<const float*>(xv ? s_dv : s_dk);
    auto in = [&](const char* t, int r) {  // element (row r, channel c) of a staged input
        return EB == 2 ? __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(t)[r * kTileCh + c] << 16)
                       : reinterpret_cast<const float*>(t)[r * kTileCh + c];
    };
    const int r0 = SUB * w;  // the wave's rows r0 .. r0 + 15 of the tile

    // 1. the wave's maps from zero: H forwards, N_u = g_u (lambda_u + N_{u+1}) backwards
    float go[SUB], gbo[SUB], xs[SUB], ls[SUB];
    float Hl = 0.f, Po = 1.f;
#pragma unroll
    for (int i = 0; i < SUB; ++i) {
        forget_gate(in(s_g, r0 + i), go[i], gbo[i]);
        const bool on = a0 + r0 + i < T;
        go[i] = on ? go[i] : 1.f;
        gbo[i] = on ? gbo[i] : 0.f;
        xs[i] = in(sx, r0 + i);
        ls[i] = sl[(r0 + i) * kTileCh + c];
        Hl = fmaf(go[i], Hl, gbo[i] * xs[i]);
        Po *= go[i];
    }
    float Nl = 0.f;
#pragma unroll
    for (int i = SUB - 1; i >= 0; --i) Nl = go[i] * (ls[i] + Nl);
    s_map[w][0][lane] = Hl;
    s_map[w][1][lane] = Po;
    s_map[w][2][lane] = Nl;
    __syncthreads();
    float Hc = 0.f, Nc = 0.f;  // the state before the wave's rows, N after them
    for (int v = 0; v < w; ++v) Hc = fmaf(s_map[v][1][lane], Hc, s_map[v][0][lane]);
    for (int v = NWV - 1; v > w; --v) Nc = fmaf(s_map[v][1][lane], Nc, s_map[v][2][lane]);
    // 2. the states before each token
    float hp[SUB];
    float Hs = Hc;
#pragma unroll
    for (int i = 0; i < SUB; ++i) {
        hp[i] = Hs;
        Hs = fmaf(go[i], Hs, gbo[i] * xs[i]);
    }
    // 3. backwards: Lambda, dx, and the gate gradient (k and v of a channel
    // summed), into LDS: dx over the staged dk / dv, dlogit over the state
    // gradient of k, which no wave reads any more
    float* sdx = reinterpret_cast<float*>(xv ? s_dv : s_dk);
    float* sdg = reinterpret_cast<float*>(s_lk);
    float Nn = Nc;
#pragma unroll
    for (int i = SUB - 1; i >= 0; --i) {
        const float Lm = ls[i] + Nn;
        Nn = go[i] * Lm;
        const float part = go[i] * gbo[i] * Lm * (hp[i] - xs[i]);
        const float other = __shfl_xor(part, 1);
        const int o = (r0 + i) * kTileCh + c;
        sdx[o] = a.raw ? fmaf(gbo[i], Lm, sd[o]) : gbo[i] * Lm;
        if (xv == 0) sdg[o] = part + other;
    }
    __syncthreads();
    unstage_rows(s_dk, a.dk, rowbase, a0, LT, T, N, c0);
    unstage_rows(s_dv, a.dv, rowbase, a0, LT, T, N, c0);
    unstage_rows(s_lk, a.dg, rowbase, a0, LT, T, N, c0);
}

// the SLIDING recurrence's backward: at L = 64 the tiles whose neighbours
// lie inside the sequence take the four-wave kernel, the first tile and the
// tail the per-token LDS kernel, which also serves every other L up to 64;
// one thread per element beyond
template <typename E>
static void launch_slide(const BwdArgs& a, unsigned elems, hipStream_t stream)
{
    const size_t N = (size_t)a.H * a.d;
    const unsigned cx = (unsigned)((N + kSlideCh - 1) / kSlideCh);
    auto tiled = [&](int u_lo, int u_hi) {  // tokens u_lo .. u_hi - 1
        if (u_hi > u_lo)
            hipLaunchKernelGGL(bwd_slide_tiled_kernel<E>, dim3(cx, (unsigned)((u_hi - u_lo + kSlideTok - 1) / kSlideTok),
                                                               (unsigned)a.B),
                               dim3(kSlideTok * kSlideCh), 0, stream, a, u_lo);
    };
    if (a.L > kSlideMaxL) {
        hipLaunchKernelGGL(bwd_slide_kernel<E>, dim3(elems), dim3(256), 0, stream, a);
        return;
    }
    const int inner = a.L == kSlideMaxL ? std::max(0, a.T / kSlideMaxL - 2) : 0;  // tiles 1 .. inner
    if (inner == 0) {
        tiled(0, a.T);
        return;
    }
    const size_t wgs = (N + 31) / 32 * (size_t)inner * a.B;
    hipLaunchKernelGGL(bwd_slide64_kernel<E>, dim3((unsigned)wgs), dim3(kSlideWaves * kWave), 0, stream, a);
    tiled(0, kSlideMaxL);
    tiled((1 + inner) * kSlideMaxL, a.T);
}

// RESTART at L = 64: one workgroup per 64-token window and 32 channels
// (H d is a multiple of 64: the boundary takes d = 64 or 128)
template <typename E>
static void launch_restart64(const BwdArgs& a, hipStream_t stream)
{
    const size_t N = (size_t)a.H * a.d;
    const size_t wgs = N / kTileCh * (size_t)((a.T + kSlideMaxL - 1) / kSlideMaxL) * a.B;
    hipLaunchKernelGGL(bwd_restart64_kernel<E>, dim3((unsigned)wgs), dim3(kRestartWaves * kWave), 0, stream, a);
}

hipError_t launch_backward(const BwdArgs& a, bool bf16, hipStream_t stream)
{
    const unsigned rows = (unsigned)((size_t)a.B * a.H * a.T);
    const size_t N = (size_t)a.H * a.d;
    const unsigned cells = (unsigned)(((size_t)a.nchunk * a.B * N + 255) / 256);
    const unsigned chans = (unsigned)(((size_t)a.B * N + 15) / 16);  // 16 channels per carry workgroup
    const unsigned elems = (unsigned)(((size_t)a.B * a.T * N + 255) / 256);  // one thread per element
    if (bf16) {
        // every head on the MFMA kernels; with a window somewhere, the band
        // passes around the dilated ones: the window's partial sums, then the
        // dilated dq with the full softmax statistics, then the window's dq;
        // the states' and the raw keys' gradients from those statistics
        const unsigned items = (unsigned)a.mitem[a.H];
        const unsigned bands = a.raw ? (unsigned)((size_t)a.H * a.B * ((a.T + kBwdOwn - 1) / kBwdOwn)) : 0u;
        const dim3 blk(kBwdThreads);
        if (a.d == 128) {
            if (bands) hipLaunchKernelGGL((bwd_q_mfma<128, 1>), dim3(bands), blk, 0, stream, a);
            if (items) hipLaunchKernelGGL((bwd_q_mfma<128, 0>), dim3(items), blk, 0, stream, a);
            if (bands) hipLaunchKernelGGL((bwd_q_mfma<128, 2>), dim3(bands), blk, 0, stream, a);
            if (items) hipLaunchKernelGGL((bwd_kv_mfma<128, false>), dim3(items), blk, 0, stream, a);
            if (bands) hipLaunchKernelGGL((bwd_kv_mfma<128, true>), dim3(bands), blk, 0, stream, a);
        } else {
            if (bands) hipLaunchKernelGGL((bwd_q_mfma<64, 1>), dim3(bands), blk, 0, stream, a);
            if (items) hipLaunchKernelGGL((bwd_q_mfma<64, 0>), dim3(items), blk, 0, stream, a);
            if (bands) hipLaunchKernelGGL((bwd_q_mfma<64, 2>), dim3(bands), blk, 0, stream, a);
            if (items) hipLaunchKernelGGL((bwd_kv_mfma<64, false>), dim3(items), blk, 0, stream, a);
            if (bands) hipLaunchKernelGGL((bwd_kv_mfma<64, true>), dim3(bands), blk, 0, stream, a);
        }
        if (a.sliding) {
            launch_slide<uint16_t>(a, elems, stream);
        } else if (a.L == kSlideMaxL) {
            launch_restart64<uint16_t>(a, stream);
        } else {
            hipLaunchKernelGGL(bwd_scan_maps_kernel<uint16_t>, dim3(cells), dim3(256), 0, stream, a);
            hipLaunchKernelGGL(bwd_scan_carry_kernel, dim3(chans), dim3(256), 0, stream, a);
            hipLaunchKernelGGL(bwd_scan_apply_kernel<uint16_t>, dim3(cells), dim3(256), 0, stream, a);
        }
    } else {
        hipLaunchKernelGGL(bwd_query_kernel<float>, dim3(rows), dim3(kWave), 0, stream, a);
        hipLaunchKernelGGL(bwd_key_kernel<float>, dim3(rows), dim3(kWave), 0, stream, a);
        if (a.sliding) {
            launch_slide<float>(a, elems, stream);
        } else if (a.L == kSlideMaxL) {
            launch_restart64<float>(a, stream);
        } else {
            hipLaunchKernelGGL(bwd_scan_maps_kernel<float>, dim3(cells), dim3(256), 0, stream, a);
            hipLaunchKernelGGL(bwd_scan_carry_kernel, dim3(chans), dim3(256), 0, stream, a);
            hipLaunchKernelGGL(bwd_scan_apply_kernel<float>, dim3(cells), dim3(256), 0, stream, a);
        }
    }
    return hipGetLastError();
}

}  // namespace rat
