// Decode step of the RAT+ layer: the new query at position T-1 attends to
// the dilated KV cache -- the recurrent states of its residue,
// ((T-1) mod D) + i*D for i < ceil(T/D), a cache D times smaller than a
// dense one ("RAT+: Train Dense, Infer Sparse", arXiv 2602.18196, Abstract;
// "RAT+ Deep Dive", zhichai.net, section 3.1: KV cache and attention FLOPs
// cut by D) -- plus the raw tokens of the local window (ring of the last
// min(W, T) tokens).
//
// One query per (b, h): a matrix-vector product, HBM-bound at ~1 FLOP/byte,
// so the kernel streams key/value rows with wide coalesced loads and does
// the dot products on the VALU (no MFMA).  DK/8 lanes share one 16-byte
// slice each of a key row, so a wave reads 64/(DK/8) whole rows per load;
// every key group keeps its own online-softmax state, merged across lane
// groups and waves at the end.  Long caches with few (b, h) pairs are split
// over several workgroups whose partial states a second kernel merges.
#include <mutex>

#include "rat_device.h"
#include "rat_internal.h"
#include "rat_plan.h"

namespace rat {

template <typename E> struct Row8;
template <> struct Row8<uint16_t> {  // 8 bf16 = 16 bytes
    static __device__ __forceinline__ void load(const uint16_t* p, float (&x)[8])
    {
        const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = bf16_lo(w[j]);
            x[2 * j + 1] = bf16_hi(w[j]);
        }
    }
    static __device__ __forceinline__ void store(uint16_t* p, const float (&x)[8])
    {
        u32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = pack_bf16x2(x[2 * j], x[2 * j + 1]);
        *reinterpret_cast<u32x4*>(p) = w;
    }
};
template <> struct Row8<float> {  // 8 fp32 = 32 bytes
    static __device__ __forceinline__ void load(const float* p, float (&x)[8])
    {
        const floatx4 a = *reinterpret_cast<const floatx4*>(p);
        const floatx4 b = *reinterpret_cast<const floatx4*>(p + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[j] = a[j];
            x[4 + j] = b[j];
        }
    }
    static __device__ __forceinline__ void store(float* p, const float (&x)[8])
    {
        *reinterpret_cast<floatx4*>(p) = floatx4{x[0], x[1], x[2], x[3]};
        *reinterpret_cast<floatx4*>(p + 4) = floatx4{x[4], x[5], x[6], x[7]};
    }
};

// A row slice of 8 elements as loaded (one or two 16-byte words), unpacked
// to fp32 where it is used.  Cache rows are read once per call: the loads
// are non-temporal (streamed past the caches that later reads would use).
template <typename E> struct Raw8;
template <> struct Raw8<uint16_t> {
    u32x4 w;
    __device__ __forceinline__ void load(const uint16_t* p)
    {
        w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    }
    __device__ __forceinline__ float operator[](int j) const { return (j & 1) ? bf16_hi(w[j >> 1]) : bf16_lo(w[j >> 1]); }
};
template <> struct Raw8<float> {
    floatx4 a, b;
    __device__ __forceinline__ void load(const float* p)
    {
        a = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p));
        b = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p + 4));
    }
    __device__ __forceinline__ float operator[](int j) const { return j < 4 ? a[j] : b[j - 4]; }
};

#ifndef RAT_DEC_UNROLL
#define RAT_DEC_UNROLL 4
#endif
// keys per lane group in flight per iteration; waves per SIMD the register
// budget must allow (six: every (b, h) of the 2.6B-scale decode batch runs
// in one round of workgroups)
constexpr int kDecUnroll = RAT_DEC_UNROLL;
#ifndef RAT_DEC_OCC
#define RAT_DEC_OCC 6
#endif

template <typename E, int DK>
__global__ __launch_bounds__(kDecWaves * kWave) __attribute__((amdgpu_waves_per_eu(RAT_DEC_OCC)))
void decode_kernel(DecodeArgs a)
{
    constexpr int LPK = DK / 8;          // lanes per key row
    constexpr int KPI = kWave / LPK;     // keys per wave step
    __shared__ float s_m[kDecWaves][KPI], s_l[kDecWaves][KPI];
    __shared__ float s_acc[kDecWaves][KPI][DK];

    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int slice = lane % LPK;        // dims 8*slice .. 8*slice+7
    const int kg = lane / LPK;           // key group in the wave
    const int split = blockIdx.x % a.nsplit;
    const int bh = blockIdx.x / a.nsplit;
    const int h = bh % a.H;
    const int D = a.D[h], W = a.W[h];
    const int nd = (a.T - 1) / D + 1;
    const int nw = min(W, a.T);
    const int n = nd + nw;
    const int per_split = (n + a.nsplit - 1) / a.nsplit;
    const int k_begin = split * per_split;
    const int k_end = min(n, k_begin + per_split);
    const int per_wave = (max(k_end - k_begin, 0) + kDecWaves - 1) / kDecWaves;
    const int w_begin = k_begin + wv * per_wave;
    const int w_end = min(k_end, w_begin + per_wave);

    const size_t drow = (size_t)bh * a.nd_cap + a.dil_off[h];
    const E* kd = static_cast<const E*>(a.kd) + drow * DK + 8 * slice;
    const E* vd = static_cast<const E*>(a.vd) + drow * DK + 8 * slice;
    const E* kw = static_cast<const E*>(a.kw) + (size_t)bh * a.w_cap * DK + 8 * slice;
    const E* vw = static_cast<const E*>(a.vw) + (size_t)bh * a.w_cap * DK + 8 * slice;

    float q[8];
    Row8<E>::load(static_cast<const E*>(a.q) + (size_t)bh * DK + 8 * slice, q);
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] *= a.scale_log2;

    float m = -INFINITY, l = 0.f, acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.f;

    for (int k0 = w_begin; k0 < w_end; k0 += KPI * kDecUnroll) {
        Raw8<E> kx[kDecUnroll], vx[kDecUnroll];
        bool ok[kDecUnroll];
#pragma unroll
        for (int u = 0; u < kDecUnroll; ++u) {
            const int key = k0 + u * KPI + kg;
            ok[u] = key < w_end;
            const int kk = ok[u] ? key : w_begin;
            const E* kr = kk < nd ? kd + (size_t)kk * DK : kw + (size_t)(kk - nd) * DK;
            const E* vr = kk < nd ? vd + (size_t)kk * DK : vw + (size_t)(kk - nd) * DK;
            kx[u].load(kr);
            vx[u].load(vr);
        }
        float s[kDecUnroll];
#pragma unroll
        for (int u = 0; u < kDecUnroll; ++u) {
            float dot = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) dot = fmaf(q[j], kx[u][j], dot);
#pragma unroll
            for (int o = 1; o < LPK; o <<= 1) dot += __shfl_xor(dot, o);
            s[u] = ok[u] ? dot : -INFINITY;
        }
        float mx = s[0];
#pragma unroll
        for (int u = 1; u < kDecUnroll; ++u) mx = fmaxf(mx, s[u]);
        const float mn = fmaxf(m, mx);
        const float ms = mn == -INFINITY ? 0.f : mn;
        const float al = __builtin_amdgcn_exp2f(m - ms);
        l *= al;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] *= al;
#pragma unroll
        for (int u = 0; u < kDecUnroll; ++u) {
            const float p = __builtin_amdgcn_exp2f(s[u] - ms);
            l += p;
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] = fmaf(p, vx[u][j], acc[j]);
        }
        m = mn;
    }

    // merge key groups and waves through LDS
    if (slice == 0) {
        s_m[wv][kg] = m;
        s_l[wv][kg] = l;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) s_acc[wv][kg][8 * slice + j] = acc[j];
    __syncthreads();
    if (wv == 0 && kg == 0) {
        float M = -INFINITY;
        for (int w2 = 0; w2 < kDecWaves; ++w2)
            for (int g2 = 0; g2 < KPI; ++g2) M = fmaxf(M, s_m[w2][g2]);
        const float Ms = M == -INFINITY ? 0.f : M;
        float L = 0.f, o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int w2 = 0; w2 < kDecWaves; ++w2)
            for (int g2 = 0; g2 < KPI; ++g2) {
                const float f = __builtin_amdgcn_exp2f(s_m[w2][g2] - Ms);
                L += f * s_l[w2][g2];
#pragma unroll
                for (int j = 0; j < 8; ++j) o[j] = fmaf(f, s_acc[w2][g2][8 * slice + j], o[j]);
            }
        if (a.nsplit == 1) {
            const float inv = 1.0f / L;
#pragma unroll
            for (int j = 0; j < 8; ++j) o[j] *= inv;
            Row8<E>::store(static_cast<E*>(a.out) + (size_t)bh * DK + 8 * slice, o);
        } else {
            float* pp = a.part + ((size_t)bh * a.nsplit + split) * (DK + 2);
#pragma unroll
            for (int j = 0; j < 8; ++j) pp[8 * slice + j] = o[j];
            if (slice == 0) {
                pp[DK] = M;
                pp[DK + 1] = L;
            }
        }
    }
}

// Combines the split partials of one (b, h): lanes own 8 output dims each.
template <typename E, int DK>
__global__ __launch_bounds__(kWave) void decode_merge_kernel(DecodeArgs a)
{
    const int bh = blockIdx.x;
    const int slice = threadIdx.x;
    if (slice >= DK / 8) return;
    const float* pp = a.part + (size_t)bh * a.nsplit * (DK + 2);
    float M = -INFINITY;
    for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, pp[s * (DK + 2) + DK]);
    const float Ms = M == -INFINITY ? 0.f : M;
    float L = 0.f, o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < a.nsplit; ++s) {
        const float* p = pp + s * (DK + 2);
        const float f = __builtin_amdgcn_exp2f(p[DK] - Ms);
        L += f * p[DK + 1];
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = fmaf(f, p[8 * slice + j], o[j]);
    }
    const float inv = 1.0f / L;
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] *= inv;
    Row8<E>::store(static_cast<E*>(a.out) + (size_t)bh * DK + 8 * slice, o);
}

template <typename E, int DK>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream)
{
    const unsigned nbh = (unsigned)(a.B * a.H);
    hipLaunchKernelGGL((decode_kernel<E, DK>), dim3(nbh * a.nsplit), dim3(kDecWaves * kWave), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit == 1) return e;
    hipLaunchKernelGGL((decode_merge_kernel<E, DK>), dim3(nbh), dim3(kWave), 0, stream, a);
    return hipGetLastError();
}

// One thread per 16 bytes of a (b, h) row (CPL = 16 / sizeof(E) channels):
// h = g * h_prev + (1 - g) * x for keys and values (the recurrence of "RAT+
// Deep Dive" section 2.1, one token), kept in fp32 in `state`, stored in the
// element type into the state history and, with the raw token, into the
// window ring.
template <typename E>
__global__ __launch_bounds__(256) void decode_step_kernel(StepArgs a)
{
    typedef Row16<E> R16;
    constexpr int CPL = R16::CPL;
    const int vpr = a.d / CPL;  // 16-byte vectors per row
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)a.B * a.H * vpr) return;
    const int c = (int)(idx % vpr) * CPL;
    const size_t bh = idx / vpr;
    const int h = (int)(bh % a.H);
    const size_t e = bh * a.d + c;  // the (b, h, c) element of a [B][H][d] row
    const u32x4 rg = *reinterpret_cast<const u32x4*>(static_cast<const E*>(a.g_new) + e);
    const u32x4 rk = *reinterpret_cast<const u32x4*>(static_cast<const E*>(a.k_new) + e);
    const u32x4 rv = *reinterpret_cast<const u32x4*>(static_cast<const E*>(a.v_new) + e);
    float* st = a.state + bh * 2 * a.d + c;
    float sk[CPL], sv[CPL], hk[CPL], hv[CPL];
#pragma unroll
    for (int j = 0; j < CPL; j += 4) {
        *reinterpret_cast<float4*>(sk + j) = *reinterpret_cast<const float4*>(st + j);
        *reinterpret_cast<float4*>(sv + j) = *reinterpret_cast<const float4*>(st + a.d + j);
    }
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        float g, gb;
        forget_gate(R16::get(rg, j), g, gb);
        if (a.restart) g = 0.f;
        hk[j] = fmaf(g, sk[j], gb * R16::get(rk, j));
        hv[j] = fmaf(g, sv[j], gb * R16::get(rv, j));
    }
#pragma unroll
    for (int j = 0; j < CPL; j += 4) {
        *reinterpret_cast<float4*>(st + j) = *reinterpret_cast<const float4*>(hk + j);
        *reinterpret_cast<float4*>(st + a.d + j) = *reinterpret_cast<const float4*>(hv + j);
    }
    const size_t rc = (bh * a.n_cap + a.slot_c[h]) * a.d + c;
    *reinterpret_cast<u32x4*>(static_cast<E*>(a.kc) + rc) = R16::pack(hk);
    *reinterpret_cast<u32x4*>(static_cast<E*>(a.vc) + rc) = R16::pack(hv);
    if (a.slot_w[h] >= 0) {
        const size_t rw = (bh * a.w_cap + a.slot_w[h]) * a.d + c;
        *reinterpret_cast<u32x4*>(static_cast<E*>(a.kw) + rw) = rk;
        *reinterpret_cast<u32x4*>(static_cast<E*>(a.vw) + rw) = rv;
    }
}

// One thread per 16 bytes of a (b, h) row: the SLIDING window's state at
// the new position p is the recurrence h = g h + (1 - g) x run from a zero
// state over positions max(0, p - L + 1) .. p ("RAT+ Deep Dive" section 2.1:
// a fixed window that looks back L tokens), i.e. exactly the sum over the
// window of the gated inputs, each weighted by the gates after it.  The
// positions before p come from the ring (slot position mod L), the new
// token from its inputs, which then take its slot (it held p - L, outside
// the window).  State and raw token are stored as decode_step_kernel does.
template <typename E>
__global__ __launch_bounds__(256) void decode_step_sliding_kernel(SlideStepArgs a)
{
    typedef Row16<E> R16;
    constexpr int CPL = R16::CPL;
    const int vpr = a.d / CPL;  // 16-byte vectors per row
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)a.B * a.H * vpr) return;
    const int c = (int)(idx % vpr) * CPL;
    const size_t bh = idx / vpr;
    const int h = (int)(bh % a.H);
    const size_t e = bh * a.d + c;  // the (b, h, c) element of a [B][H][d] row
    const u32x4 ng = *reinterpret_cast<const u32x4*>(static_cast<const E*>(a.g_new) + e);
    const u32x4 nk = *reinterpret_cast<const u32x4*>(static_cast<const E*>(a.k_new) + e);
    const u32x4 nv = *reinterpret_cast<const u32x4*>(static_cast<const E*>(a.v_new) + e);
    const size_t ring = bh * a.L * a.d + c;  // slot 0 of this (b, h, c) in the recurrence ring
    float hk[CPL], hv[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) { hk[j] = 0.f; hv[j] = 0.f; }
    const int first = max(0, a.p - a.L + 1);
    int slot = first % a.L;
#pragma unroll 4
    for (int s = first; s < a.p; ++s) {
        const size_t o = ring + (size_t)slot * a.d;
        const u32x4 rgv = *reinterpret_cast<const u32x4*>(static_cast<const E*>(a.rg) + o);
        const u32x4 rkv = *reinterpret_cast<const u32x4*>(static_cast<const E*>(a.rk) + o);
        const u32x4 rvv = *reinterpret_cast<const u32x4*>(static_cast<const E*>(a.rv) + o);
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            float g, gb;
            forget_gate(R16::get(rgv, j), g, gb);
            hk[j] = fmaf(g, hk[j], gb * R16::get(rkv, j));
            hv[j] = fmaf(g, hv[j], gb * R16::get(rvv, j));
        }
        slot = slot + 1 == a.L ? 0 : slot + 1;
    }
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        float g, gb;
        forget_gate(R16::get(ng, j), g, gb);
        hk[j] = fmaf(g, hk[j], gb * R16::get(nk, j));
        hv[j] = fmaf(g, hv[j], gb * R16::get(nv, j));
    }
    const size_t on = ring + (size_t)(a.p % a.L) * a.d;
    *reinterpret_cast<u32x4*>(static_cast<E*>(a.rk) + on) = nk;
    *reinterpret_cast<u32x4*>(static_cast<E*>(a.rv) + on) = nv;
    *reinterpret_cast<u32x4*>(static_cast<E*>(a.rg) + on) = ng;
    const size_t rc = (bh * a.n_cap + a.slot_c[h]) * a.d + c;
    *reinterpret_cast<u32x4*>(static_cast<E*>(a.kc) + rc) = R16::pack(hk);
    *reinterpret_cast<u32x4*>(static_cast<E*>(a.vc) + rc) = R16::pack(hv);
    if (a.slot_w[h] >= 0) {
        const size_t rw = (bh * a.w_cap + a.slot_w[h]) * a.d + c;
        *reinterpret_cast<u32x4*>(static_cast<E*>(a.kw) + rw) = nk;
        *reinterpret_cast<u32x4*>(static_cast<E*>(a.vw) + rw) = nv;
    }
}

// The recurrence ring of a finished SLIDING prefill: one thread per 16
// bytes of a ring row; slot s of (b, h) holds the latest position p < T with
// p mod L = s (positions T - L .. T-1); slots with no such position are left
// alone.
template <typename E>
__global__ __launch_bounds__(256) void sliding_fill_kernel(SlideFillArgs a)
{
    constexpr int EPV = 16 / sizeof(E);
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    const int vpr = a.d / EPV;
    if (idx >= (size_t)a.B * a.H * a.L * vpr) return;
    const int c = (int)(idx % vpr) * EPV;
    const size_t row = idx / vpr;  // (b H + h) L + slot
    const int slot = (int)(row % a.L);
    const size_t bh = row / a.L;
    const int h = (int)(bh % a.H), b = (int)(bh / a.H);
    const int p = (a.T - 1) - ((a.T - 1 - slot) % a.L + a.L) % a.L;  // latest position of the slot
    if (p < 0) return;
    const size_t src = (((size_t)b * a.T + p) * a.H + h) * a.d + c;
    const size_t dst = row * a.d + c;
    *reinterpret_cast<u32x4*>(static_cast<E*>(a.rk) + dst) = *reinterpret_cast<const u32x4*>(static_cast<const E*>(a.k) + src);
    *reinterpret_cast<u32x4*>(static_cast<E*>(a.rv) + dst) = *reinterpret_cast<const u32x4*>(static_cast<const E*>(a.v) + src);
    *reinterpret_cast<u32x4*>(static_cast<E*>(a.rg) + dst) = *reinterpret_cast<const u32x4*>(static_cast<const E*>(a.g) + src);
}

hipError_t launch_decode_step_sliding(const SlideStepArgs& a, bool bf16, hipStream_t stream)
{
    const size_t n = (size_t)a.B * a.H * (a.d / (bf16 ? 8 : 4));
    const unsigned blocks = (unsigned)((n + 255) / 256);
    if (bf16) hipLaunchKernelGGL(decode_step_sliding_kernel<uint16_t>, dim3(blocks), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(decode_step_sliding_kernel<float>, dim3(blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_sliding_fill(const SlideFillArgs& a, bool bf16, hipStream_t stream)
{
    const size_t n = (size_t)a.B * a.H * a.L * (a.d / (bf16 ? 8 : 4));
    if (n == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((n + 255) / 256);
    if (bf16) hipLaunchKernelGGL(sliding_fill_kernel<uint16_t>, dim3(blocks), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(sliding_fill_kernel<float>, dim3(blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

// Raw ring after a prefill: slot s of head h holds the latest position
// p < T with p mod W[h] = s (so positions T - W[h] .. T-1); slots with no
// such position, and slots at or past W[h], are left alone.  One thread per
// 16 bytes of a row.
template <typename E>
__global__ __launch_bounds__(256) void ring_fill_kernel(RingFillArgs a)
{
    constexpr int EPV = 16 / sizeof(E);  // elements per 16-byte vector
    size_t src, dst;
    if (!ring_fill_at(a, (size_t)blockIdx.x * 256 + threadIdx.x, EPV, src, dst)) return;
    *reinterpret_cast<u32x4*>(static_cast<E*>(a.kw) + dst) = *reinterpret_cast<const u32x4*>(static_cast<const E*>(a.k) + src);
    *reinterpret_cast<u32x4*>(static_cast<E*>(a.vw) + dst) = *reinterpret_cast<const u32x4*>(static_cast<const E*>(a.v) + src);
}

hipError_t launch_ring_fill(const RingFillArgs& a, bool bf16, hipStream_t stream)
{
    const size_t n = (size_t)a.B * a.H * a.w_cap * (a.d / (bf16 ? 8 : 4));
    if (n == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((n + 255) / 256);
    if (bf16) hipLaunchKernelGGL(ring_fill_kernel<uint16_t>, dim3(blocks), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(ring_fill_kernel<float>, dim3(blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

// One thread per 16 bytes of a prefill row (b, p, h): the state row into
// the history, and for the last W[h] positions the raw row into the ring.
template <typename E>
__global__ __launch_bounds__(256) void cache_build_kernel(CacheArgs a)
{
    constexpr int EPV = 16 / sizeof(E);
    const int vpr = a.d / EPV;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)a.B * a.T * a.H * vpr) return;
    const int c = (int)(idx % vpr) * EPV;
    const size_t row = idx / vpr;  // (b T + p) H + h
    const int h = (int)(row % a.H);
    const size_t bp = row / a.H;
    const int p = (int)(bp % a.T), b = (int)(bp / a.T);
    const int D = a.D[h], W = a.W[h];
    const size_t src = row * a.d + c;
    const size_t bh = (size_t)b * a.H + h;
    const size_t dst = (bh * a.n_cap + (size_t)(p % D) * (a.n_cap / D) + p / D) * a.d + c;
    *reinterpret_cast<u32x4*>(static_cast<E*>(a.kc) + dst) = *reinterpret_cast<const u32x4*>(static_cast<const E*>(a.ks) + src);
    *reinterpret_cast<u32x4*>(static_cast<E*>(a.vc) + dst) = *reinterpret_cast<const u32x4*>(static_cast<const E*>(a.vs) + src);
    if (W > 0 && p >= a.T - W) {
        const size_t dw = (bh * a.w_cap + (size_t)(p % W)) * a.d + c;
        *reinterpret_cast<u32x4*>(static_cast<E*>(a.kw) + dw) = *reinterpret_cast<const u32x4*>(static_cast<const E*>(a.k) + src);
        *reinterpret_cast<u32x4*>(static_cast<E*>(a.vw) + dw) = *reinterpret_cast<const u32x4*>(static_cast<const E*>(a.v) + src);
    }
}

hipError_t launch_cache_build(const CacheArgs& a, bool bf16, hipStream_t stream)
{
    const size_t n = (size_t)a.B * a.T * a.H * (a.d / (bf16 ? 8 : 4));
    if (n == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((n + 255) / 256);
    if (bf16) hipLaunchKernelGGL(cache_build_kernel<uint16_t>, dim3(blocks), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(cache_build_kernel<float>, dim3(blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_decode_step(const StepArgs& a, bool bf16, hipStream_t stream)
{
    const size_t n = (size_t)a.B * a.H * (a.d / (bf16 ? 8 : 4));  // one thread per 16 bytes of a row
    const unsigned blocks = (unsigned)((n + 255) / 256);
    if (bf16) hipLaunchKernelGGL(decode_step_kernel<uint16_t>, dim3(blocks), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(decode_step_kernel<float>, dim3(blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

// The scratch of rat_dilated_attn_decode_static: split partials
// [B*H][nsplit][d + 2] in fp32.  Host code never uses the array's name as an
// address (on the host it is a stand-in, not device memory): kernels get
// the pointer hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

hipError_t decode_scratch(void** ptr)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* cached[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!cached[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        cached[dev] = p;
    }
    *ptr = cached[dev];
    return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, int d, bool bf16, hipStream_t stream)
{
    if (bf16) return d == 128 ? launch_decode_t<uint16_t, 128>(a, stream) : launch_decode_t<uint16_t, 64>(a, stream);
    return d == 128 ? launch_decode_t<float, 128>(a, stream) : launch_decode_t<float, 64>(a, stream);
}

}  // namespace rat
