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
//   bwd_query_kernel  one wave per query row: log-sum-exp of its softmax
//                     and delta_t, then dq_t (two passes over its keys);
//   bwd_key_kernel    one wave per key row: the state key's gradients from
//                     the queries t = s, s + D, ... and the raw key's from
//                     t = s .. s + W - 1;
//   bwd_q_mfma / bwd_kv_mfma  the same for bf16 heads without a raw window,
//                     on MFMA: a residue is a dense causal problem over the
//                     states r, r + D, ..., so a workgroup takes 64 rows of
//                     one residue (queries for dq, keys for dk / dv) and
//                     walks the other side's 64-row tiles through LDS;
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
    if (a.mfma && W == 0) return;  // the MFMA kernels take this head
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
    // the state at s: queries s, s + D, ... (< T); the MFMA kernels take
    // heads without a raw window
    if (!(a.mfma && W == 0)) key_grads(a.ks, a.vs, (a.T - 1 - s) / D + 1, D, a.dks, a.dvs);
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

// dq (and each query row's log-sum-exp and delta): wave w owns queries
// 16w .. 16w+15 of the block; lane (g, i) query i.  Scores are S^T = K Q^T
// (lane: keys 16kb + 4g + j of its query), dP^T = V dO^T, and
// dQ^T += K^T dS^T with dS^T packed to bf16 as the B operand.
template <int DK>
__global__ __launch_bounds__(kBwdThreads, 2) void bwd_q_mfma(BwdArgs a)
{
    typedef Geo<DK> G;
    __shared__ __attribute__((aligned(1024))) char kt[kBwdRows * G::ROWB];
    __shared__ __attribute__((aligned(1024))) char vt[kBwdRows * G::ROWB];
    const BwdItem it = bwd_item<true>(a, xcd_item(blockIdx.x, gridDim.x));
    if (!it.valid) return;
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int g = lane >> 4, i = lane & 15;
    const float c = a.scale * kLog2e;
    const int qr = it.blk * kBwdOwn + 16 * wv + i;
    const bool qvalid = qr < it.M;
    const size_t qe = qvalid ? res_row<DK>(a, it, qr) : 0;
    bf16x8 qf[G::KS], gf[G::KS];
    load_frag<DK>(qf, a.q, qe, qvalid);
    load_frag<DK>(gf, a.dout, qe, qvalid);
    // key tiles up to the block's last query
    const int ntile = (min(it.M, (it.blk + 1) * kBwdOwn) - 1) / kBwdRows + 1;
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
    // key / value tiles t = 0 .. 2 ntile - 1 (both sweeps) through registers
    TileRegs<DK> rk, rv;
    rk.load(a.ks, a, it, 0);
    rv.load(a.vs, a, it, 0);
    auto next_tile = [&](int t) {  // tile t into LDS, tile t + 1 into registers
        __syncthreads();
        rk.store(kt);
        rv.store(vt);
        __syncthreads();
        const int tn = (t + 1) % ntile;
        if (t + 1 < 2 * ntile) {
            rk.load(a.ks, a, it, tn * kBwdRows);
            rv.load(a.vs, a, it, tn * kBwdRows);
        }
    };
    // sweep 1: per lane group, (max, sum of e^(z - max), sum of e^(z - max) dp)
    // over its keys, rescaled once per tile: the tile's 16 scores of the lane
    // (-inf past the query) give the new max first
    float m = -INFINITY, l = 0.f, u = 0.f;
    for (int t = 0; t < ntile; ++t) {
        next_tile(t);
        floatx4 st[4], dpt[4];
        scores(st, dpt);
        float tm = m;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int kr = t * kBwdRows + 16 * kb + 4 * g + j;
                st[kb][j] = kr <= qr ? st[kb][j] * c : -INFINITY;
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
    const float lse2 = mall + __log2f(lall);  // log2-domain log-sum-exp
    const float delta = uall / lall;
    // sweep 2: dQ^T
    const int toff = tr_offset<DK>();
    floatx4 dqt[G::DB];
#pragma unroll
    for (int db = 0; db < G::DB; ++db) dqt[db] = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int t = 0; t < ntile; ++t) {
        next_tile(ntile + t);
        floatx4 st[4], dpt[4];
        scores(st, dpt);
        bf16x8 sh[2], sl[2];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int kr = t * kBwdRows + 16 * kb + 4 * g + j;
                const float p = kr <= qr ? __builtin_amdgcn_exp2f(fmaf(st[kb][j], c, -lse2)) : 0.f;
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
        const size_t o = qe;  // same [B][T][H][DK] position, fp32
#pragma unroll
        for (int db = 0; db < G::DB; ++db)
            *reinterpret_cast<floatx4*>(a.dq + o + 16 * db + 4 * g) = dqt[db];
        if (g == 0) {
            const size_t rrow = ((size_t)it.b * a.T + it.r + (size_t)qr * it.D) * a.H + it.h;
            a.lse[rrow] = lse2 * 0.6931471805599453f;  // natural log
            a.delta[rrow] = delta;
        }
    }
}

// dk, dv of the states: wave w owns keys 16w .. 16w+15 of the block; lane
// (g, i) key i.  Scores S = Q K^T (lane: queries 16qb + 4g + j of its key),
// dP = dO V^T, dV^T += dO^T P and dK^T += Q^T dS with P and dS packed to
// bf16 as B operands.
template <int DK>
__global__ __launch_bounds__(kBwdThreads, 2) void bwd_kv_mfma(BwdArgs a)
{
    typedef Geo<DK> G;
    __shared__ __attribute__((aligned(1024))) char qt[kBwdRows * G::ROWB];
    __shared__ __attribute__((aligned(1024))) char gt[kBwdRows * G::ROWB];
    __shared__ float s_lse2[kBwdRows], s_dl[kBwdRows];
    const BwdItem it = bwd_item<false>(a, xcd_item(blockIdx.x, gridDim.x));
    if (!it.valid) return;
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int g = lane >> 4, i = lane & 15;
    const float c = a.scale * kLog2e;
    const int kr = it.blk * kBwdOwn + 16 * wv + i;
    const bool kvalid = kr < it.M;
    const size_t ke = kvalid ? res_row<DK>(a, it, kr) : 0;
    bf16x8 kf[G::KS], vf[G::KS];
    load_frag<DK>(kf, a.ks, ke, kvalid);
    load_frag<DK>(vf, a.vs, ke, kvalid);
    const int toff = tr_offset<DK>();
    floatx4 dkt[G::DB], dvt[G::DB];
#pragma unroll
    for (int db = 0; db < G::DB; ++db) {
        dkt[db] = floatx4{0.f, 0.f, 0.f, 0.f};
        dvt[db] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    const int ntile = (it.M + kBwdRows - 1) / kBwdRows;
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
                const float p = q >= kr ? __builtin_amdgcn_exp2f(fmaf(sv[j], c, -s_lse2[ql])) : 0.f;
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
            *reinterpret_cast<floatx4*>(a.dks + ke + 16 * db + 4 * g) = dkt[db];
            *reinterpret_cast<floatx4*>(a.dvs + ke + 16 * db + 4 * g) = dvt[db];
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

hipError_t launch_backward(const BwdArgs& a, bool bf16, hipStream_t stream)
{
    const unsigned rows = (unsigned)((size_t)a.B * a.H * a.T);
    const size_t N = (size_t)a.H * a.d;
    const unsigned cells = (unsigned)(((size_t)a.nchunk * a.B * N + 255) / 256);
    const unsigned chans = (unsigned)(((size_t)a.B * N + 15) / 16);  // 16 channels per carry workgroup
    if (bf16) {
        const unsigned items = (unsigned)a.mitem[a.H];
        if (a.mfma && items > 0) {
            if (a.d == 128) hipLaunchKernelGGL(bwd_q_mfma<128>, dim3(items), dim3(kBwdThreads), 0, stream, a);
            else hipLaunchKernelGGL(bwd_q_mfma<64>, dim3(items), dim3(kBwdThreads), 0, stream, a);
        }
        // the per-row kernels: heads with a raw window (and the raw-window
        // gradients, zero for the other heads); none when no head has one
        if (a.raw) hipLaunchKernelGGL(bwd_query_kernel<uint16_t>, dim3(rows), dim3(kWave), 0, stream, a);
        if (a.mfma && items > 0) {
            if (a.d == 128) hipLaunchKernelGGL(bwd_kv_mfma<128>, dim3(items), dim3(kBwdThreads), 0, stream, a);
            else hipLaunchKernelGGL(bwd_kv_mfma<64>, dim3(items), dim3(kBwdThreads), 0, stream, a);
        }
        if (a.raw) hipLaunchKernelGGL(bwd_key_kernel<uint16_t>, dim3(rows), dim3(kWave), 0, stream, a);
        hipLaunchKernelGGL(bwd_scan_maps_kernel<uint16_t>, dim3(cells), dim3(256), 0, stream, a);
        hipLaunchKernelGGL(bwd_scan_carry_kernel, dim3(chans), dim3(256), 0, stream, a);
        hipLaunchKernelGGL(bwd_scan_apply_kernel<uint16_t>, dim3(cells), dim3(256), 0, stream, a);
    } else {
        hipLaunchKernelGGL(bwd_query_kernel<float>, dim3(rows), dim3(kWave), 0, stream, a);
        hipLaunchKernelGGL(bwd_key_kernel<float>, dim3(rows), dim3(kWave), 0, stream, a);
        hipLaunchKernelGGL(bwd_scan_maps_kernel<float>, dim3(cells), dim3(256), 0, stream, a);
        hipLaunchKernelGGL(bwd_scan_carry_kernel, dim3(chans), dim3(256), 0, stream, a);
        hipLaunchKernelGGL(bwd_scan_apply_kernel<float>, dim3(cells), dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace rat
