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
//   bwd_scan_*        the reverse recurrence in chunks of kBwdChunk tokens:
//                     per-chunk affine maps (forward state map and backward
//                     carry map), a sequential pass over the chunks of each
//                     channel, then per chunk the states recomputed in fp32
//                     from the chunk's start state and walked backwards.
#include "rat_device.h"
#include "rat_internal.h"

namespace rat {

template <typename E> __device__ __forceinline__ float ldx(const void* p, size_t i);
template <> __device__ __forceinline__ float ldx<uint16_t>(const void* p, size_t i)
{
    return __uint_as_float((uint32_t)static_cast<const uint16_t*>(p)[i] << 16);
}
template <> __device__ __forceinline__ float ldx<float>(const void* p, size_t i) { return static_cast<const float*>(p)[i]; }

__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// A row of d <= 128 channels across one wave: lane holds channels lane and
// lane + 64 (zero past d).
template <typename E>
struct Row2 {
    float a, b;
    __device__ __forceinline__ void load(const void* p, size_t row, int d, int lane)
    {
        a = lane < d ? ldx<E>(p, row + lane) : 0.f;
        b = lane + kWave < d ? ldx<E>(p, row + lane + kWave) : 0.f;
    }
    __device__ __forceinline__ float dot(const Row2& o) const { return wave_sum(a * o.a + b * o.b); }
};

// ---------------------------------------------------------------- attention
template <typename E>
__global__ __launch_bounds__(kWave) void bwd_query_kernel(BwdArgs a)
{
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
    // pass 1: log-sum-exp of the logits and delta = sum_j p_j dp_j
    float m = -INFINITY, l = 0.f, u = 0.f;  // u: sum_j e^{z_j - m} dp_j
    auto stat = [&](const void* kp, const void* vp, size_t row) {
        Row2<E> kk, vv;
        kk.load(kp, row, d, lane);
        vv.load(vp, row, d, lane);
        const float z = q.dot(kk) * a.scale;
        const float dp = go.dot(vv);
        const float mn = fmaxf(m, z);
        const float r = __expf(m - mn), e = __expf(z - mn);
        l = fmaf(l, r, e);
        u = fmaf(u, r, e * dp);
        m = mn;
    };
    for (int s = t; s >= 0; s -= D) stat(a.ks, a.vs, base + (size_t)s * pitch);
    for (int w = 0; w < W && t - w >= 0; ++w) stat(a.k, a.v, base + (size_t)(t - w) * pitch);
    const float lse = m + __logf(l);
    const float delta = u / l;
    // pass 2: dq = scale sum_j p_j (dp_j - delta) kappa_j
    float ga = 0.f, gb = 0.f;
    auto grad = [&](const void* kp, const void* vp, size_t row) {
        Row2<E> kk, vv;
        kk.load(kp, row, d, lane);
        vv.load(vp, row, d, lane);
        const float p = __expf(q.dot(kk) * a.scale - lse);
        const float ds = p * (go.dot(vv) - delta) * a.scale;
        ga = fmaf(ds, kk.a, ga);
        gb = fmaf(ds, kk.b, gb);
    };
    for (int s = t; s >= 0; s -= D) grad(a.ks, a.vs, base + (size_t)s * pitch);
    for (int w = 0; w < W && t - w >= 0; ++w) grad(a.k, a.v, base + (size_t)(t - w) * pitch);
    if (lane < d) a.dq[rt + lane] = ga;
    if (lane + kWave < d) a.dq[rt + lane + kWave] = gb;
    if (lane == 0) {
        const size_t r = ((size_t)b * a.T + t) * a.H + h;
        a.lse[r] = lse;
        a.delta[r] = delta;
    }
}

template <typename E>
__global__ __launch_bounds__(kWave) void bwd_key_kernel(BwdArgs a)
{
    const int lane = threadIdx.x;
    const int s = blockIdx.x % a.T;
    const int bh = blockIdx.x / a.T;
    const int h = bh % a.H, b = bh / a.H;
    const int d = a.d, D = a.D[h], W = a.W[h];
    const size_t pitch = (size_t)a.H * d;
    const size_t base = ((size_t)b * a.T * a.H + h) * d;
    const size_t rs = base + (size_t)s * pitch;
    // one key row against the queries that see it
    auto key_grads = [&](const void* kp, const void* vp, int t0, int t1, int step, float* dk_out, float* dv_out) {
        Row2<E> kk, vv;
        kk.load(kp, rs, d, lane);
        vv.load(vp, rs, d, lane);
        float ka = 0.f, kb = 0.f, va = 0.f, vb = 0.f;
        for (int t = t0; t <= t1; t += step) {
            const size_t rt = base + (size_t)t * pitch;
            const size_t r = ((size_t)b * a.T + t) * a.H + h;
            Row2<E> q, go;
            q.load(a.q, rt, d, lane);
            go.load(a.dout, rt, d, lane);
            const float p = __expf(q.dot(kk) * a.scale - a.lse[r]);
            const float ds = p * (go.dot(vv) - a.delta[r]) * a.scale;
            ka = fmaf(ds, q.a, ka);
            kb = fmaf(ds, q.b, kb);
            va = fmaf(p, go.a, va);
            vb = fmaf(p, go.b, vb);
        }
        if (lane < d) {
            dk_out[rs + lane] = ka;
            dv_out[rs + lane] = va;
        }
        if (lane + kWave < d) {
            dk_out[rs + lane + kWave] = kb;
            dv_out[rs + lane + kWave] = vb;
        }
    };
    // the state at s: queries s, s + D, ... (< T)
    key_grads(a.ks, a.vs, s, a.T - 1, D, a.dks, a.dvs);
    // the raw token at s: queries s .. s + W - 1 (an empty range writes zeros)
    key_grads(a.k, a.v, s, min(s + W - 1, a.T - 1), 1, a.dk, a.dv);
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
    const int t0 = p.c * kBwdChunk, t1 = min(t0 + kBwdChunk, a.T);
    float A = 1.f, K = 0.f, V = 0.f;
    for (int t = t0; t < t1; ++t) {
        const size_t i = ((size_t)p.b * a.T + t) * N + p.n;
        float g, gb;
        forget_gate(ldx<E>(a.g, i), g, gb);
        if (restart_at(a, t)) { A = 0.f; K = 0.f; V = 0.f; }
        A *= g;
        K = fmaf(g, K, gb * ldx<E>(a.k, i));
        V = fmaf(g, V, gb * ldx<E>(a.v, i));
    }
    float Bk = 0.f, Bv = 0.f;  // carry out of the chunk's first token with a zero carry in
    for (int t = t1 - 1; t >= t0; --t) {
        const size_t i = ((size_t)p.b * a.T + t) * N + p.n;
        float g, gb;
        forget_gate(ldx<E>(a.g, i), g, gb);
        const float lk = a.dks[i] + Bk, lv = a.dvs[i] + Bv;
        const bool cut = restart_at(a, t);
        Bk = cut ? 0.f : g * lk;
        Bv = cut ? 0.f : g * lv;
    }
    float* m = a.maps + p.cell * 5;
    m[0] = A; m[1] = K; m[2] = V; m[3] = Bk; m[4] = Bv;
}

// Per (b, channel), over its chunks: the state before each chunk (forward)
// and the carry into each chunk's last token (backward).
__global__ __launch_bounds__(256) void bwd_scan_carry_kernel(BwdArgs a)
{
    const size_t N = (size_t)a.H * a.d;
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (size_t)a.B * N) return;
    const size_t stride = (size_t)a.B * N;  // between chunks
    float hk = 0.f, hv = 0.f;
    for (int c = 0; c < a.nchunk; ++c) {
        const size_t cell = (size_t)c * stride + idx;
        a.carry[cell * 4 + 0] = hk;
        a.carry[cell * 4 + 1] = hv;
        const float* m = a.maps + cell * 5;
        hk = fmaf(m[0], hk, m[1]);
        hv = fmaf(m[0], hv, m[2]);
    }
    float mk = 0.f, mv = 0.f;
    for (int c = a.nchunk - 1; c >= 0; --c) {
        const size_t cell = (size_t)c * stride + idx;
        a.carry[cell * 4 + 2] = mk;
        a.carry[cell * 4 + 3] = mv;
        const float* m = a.maps + cell * 5;
        mk = fmaf(m[0], mk, m[3]);
        mv = fmaf(m[0], mv, m[4]);
    }
}

// Per chunk: the fp32 states again from the chunk's start state, then the
// chunk walked backwards.  dk / dv already hold the raw-window gradients.
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
            a.dk[x] = fmaf(gb, lk, a.dk[x]);
            a.dv[x] = fmaf(gb, lv, a.dv[x]);
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
    const unsigned chans = (unsigned)(((size_t)a.B * N + 255) / 256);
    if (bf16) {
        hipLaunchKernelGGL(bwd_query_kernel<uint16_t>, dim3(rows), dim3(kWave), 0, stream, a);
        hipLaunchKernelGGL(bwd_key_kernel<uint16_t>, dim3(rows), dim3(kWave), 0, stream, a);
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
