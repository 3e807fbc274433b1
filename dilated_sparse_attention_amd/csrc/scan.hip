// Stage 1 of the RAT+ layer: the gated recurrence over keys and values,
//   h_t = g_t * h_{t-1} + (1 - g_t) * x_t,   g_t = sigmoid(logit_t),
// computed for prefill as a parallel scan ("RAT+ Deep Dive", zhichai.net,
// section 2.1 Full-Sequence Recurrence, and 7.3 "Parallel prefill
// (associative scan)").  The recurrence equation itself is missing from the
// page's text; this is the forget-gate reading of its surrounding words.
//
// Layout [B,T,H,d] puts the scan axis T slowest, so lanes map to channels
// (each lane owns two adjacent channels) and every token row is one
// coalesced 256-byte (bf16) / 512-byte (fp32) load per wave; the scan along
// T is then a per-lane sequential recurrence with no cross-lane traffic.
//
// FULL / RESTART kernel (one pass over HBM):
//   * a workgroup owns a chunk of C = 8 waves x TPL tokens of one
//     (batch, 128-channel block); each wave holds its TPL tokens in
//     registers;
//   * pass 1: each wave runs the recurrence over its tokens from a zero
//     state, keeping per token the local state H_t and the gate product
//     P_t since its first token; the last ones form the wave's affine map
//     h -> A*h + B (A = prod g, B = gated sum), per channel;
//   * waves combine their maps through LDS; the chunk's map is published
//     and the carry-in is found by a decoupled look-back over the chunks
//     before it (Merrill & Garland's single-pass scan), through 64-bit
//     words that carry (value, epoch tag) and so need no memory fence;
//   * pass 2 applies the carry c of the wave: h_t = H_t + P_t * c (one FMA
//     per element; the gates are evaluated once).
//   Chunk order comes from a ticket counter so that every chunk a
//   workgroup waits for belongs to a workgroup that is already running;
//   the same 64-bit atomic returns the call's epoch.
//   RESTART (state cleared where t mod L == 0) is the same recurrence with
//   g forced to 0 at those positions; a map with A == 0 ends the look-back.
//
// SLIDING kernel (h_t sums exactly the last L <= 64 inputs):
//   with tiles aligned to multiples of L, t = mL + j, the window of t is
//   the prefix 0..j of tile m plus the suffix j+1..L-1 of tile m-1:
//     h_t = H_t + P_t * X_{j},
//   H_t / P_t the in-tile recurrence / gate product from the tile start and
//   X_j the suffix sum of tile m-1 from j+1 (a reverse scan).  No
//   subtraction or division.  Each lane keeps its X_j in LDS.
#include "rat_device.h"
#include "rat_internal.h"

namespace rat {

constexpr int kScanThreads = kScanWaves * kWave;
constexpr int kScanCh = 2 * kWave;  // channels per workgroup
constexpr uint32_t kLookbackSpinLimit = 1u << 22;  // polls before the watchdog fires

// Two adjacent channels of one token row.
template <typename E> struct Pair2;
// Inputs are read once and outputs written once: nontemporal accesses keep
// the stream from displacing other data in the caches (measured ~5-10%
// faster on this access pattern).
typedef float floatx2 __attribute__((ext_vector_type(2)));
template <> struct Pair2<float> {
    typedef floatx2 raw;
    static __device__ __forceinline__ raw load(const float* p) { return __builtin_nontemporal_load(reinterpret_cast<const floatx2*>(p)); }
    static __device__ __forceinline__ float lo(raw r) { return r[0]; }
    static __device__ __forceinline__ float hi(raw r) { return r[1]; }
    static __device__ __forceinline__ raw zero() { return floatx2{0.f, 0.f}; }
    static __device__ __forceinline__ void store(float* p, float a, float b) { __builtin_nontemporal_store(floatx2{a, b}, reinterpret_cast<floatx2*>(p)); }
};
template <> struct Pair2<uint16_t> {
    typedef uint32_t raw;
    static __device__ __forceinline__ raw load(const uint16_t* p) { return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p)); }
    static __device__ __forceinline__ float lo(raw r) { return bf16_lo(r); }
    static __device__ __forceinline__ float hi(raw r) { return bf16_hi(r); }
    static __device__ __forceinline__ raw zero() { return 0u; }
    static __device__ __forceinline__ void store(uint16_t* p, float a, float b) { __builtin_nontemporal_store(pack_bf16x2(a, b), reinterpret_cast<uint32_t*>(p)); }
};

template <typename E, int TPL>
__global__ __launch_bounds__(kScanThreads) void scan_full_kernel(ScanFullArgs a)
{
    typedef Pair2<E> P;
    __shared__ uint32_t s_ticket, s_epoch;
    __shared__ float s_map[kScanWaves][3][kScanCh];  // per-wave (A, Bk, Bv)
    __shared__ float s_carry[2][kScanCh];            // chunk carry-in (hk, hv)

    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    if (threadIdx.x == 0) {
        const uint64_t old = __hip_atomic_fetch_add(&a.hdr->tick, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_ticket = (uint32_t)old;
        s_epoch = (uint32_t)(old >> 32);
        // every ticket of this call is now handed out: start the next epoch
        if ((uint32_t)old + 1u == (uint32_t)a.nwg)
            __hip_atomic_store(&a.hdr->tick, (uint64_t)(s_epoch + 1u) << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    const uint32_t ticket = s_ticket;
    const uint32_t tag = s_epoch + 1u;
    const int chunk = (int)(ticket / (uint32_t)a.nseq);
    const int seq = (int)(ticket % (uint32_t)a.nseq);
    const int b = seq / a.nblk;
    const int cl = lane * 2;                       // channel within the block
    const int c = (seq % a.nblk) * kScanCh + cl;   // channel within the row
    const bool cvalid = c < a.N;
    const int t0 = chunk * (kScanWaves * TPL) + w * TPL;
    const size_t base = (size_t)b * a.T * a.N + c;

    const E* kp = static_cast<const E*>(a.k) + base;
    const E* vp = static_cast<const E*>(a.v) + base;
    const E* gp = static_cast<const E*>(a.g) + base;

    // RESTART positions (t mod L == 0) of this wave's tokens, as a
    // wave-uniform bit mask
    uint32_t rmask = 0;
    if (a.L > 0) {
        for (int t = ((t0 + a.L - 1) / a.L) * a.L; t < t0 + TPL; t += a.L) rmask |= 1u << (t - t0);
    }
    rmask = __builtin_amdgcn_readfirstlane(rmask);

    typename P::raw rk[TPL], rv[TPL], rg[TPL];
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
        const int t = t0 + i;
        if (cvalid && t < a.T) {
            const size_t o = (size_t)t * a.N;
            rk[i] = P::load(kp + o);
            rv[i] = P::load(vp + o);
            rg[i] = P::load(gp + o);
        } else {
            rk[i] = P::zero();
            rv[i] = P::zero();
            rg[i] = P::zero();
        }
    }

    // pass 1: local recurrence from zero; H (k, v) and gate product per token
    float A0 = 1.f, A1 = 1.f, K0 = 0.f, K1 = 0.f, V0 = 0.f, V1 = 0.f;
    float hk[TPL][2], hv[TPL][2], pg[TPL][2];
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
        if (t0 + i < a.T) {
            float g0, gb0, g1, gb1;
            forget_gate(P::lo(rg[i]), g0, gb0);
            forget_gate(P::hi(rg[i]), g1, gb1);
            if ((rmask >> i) & 1u) { g0 = 0.f; g1 = 0.f; }
            A0 *= g0; A1 *= g1;
            K0 = fmaf(g0, K0, gb0 * P::lo(rk[i]));
            K1 = fmaf(g1, K1, gb1 * P::hi(rk[i]));
            V0 = fmaf(g0, V0, gb0 * P::lo(rv[i]));
            V1 = fmaf(g1, V1, gb1 * P::hi(rv[i]));
        }
        hk[i][0] = K0; hk[i][1] = K1;
        hv[i][0] = V0; hv[i][1] = V1;
        pg[i][0] = A0; pg[i][1] = A1;
    }
    s_map[w][0][cl] = A0; s_map[w][0][cl + 1] = A1;
    s_map[w][1][cl] = K0; s_map[w][1][cl + 1] = K1;
    s_map[w][2][cl] = V0; s_map[w][2][cl + 1] = V1;
    __syncthreads();

    if (w == 0) {
        // the chunk's map: waves in token order
        float cA[2] = {1.f, 1.f}, cK[2] = {0.f, 0.f}, cV[2] = {0.f, 0.f};
#pragma unroll
        for (int ww = 0; ww < kScanWaves; ++ww)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float wa = s_map[ww][0][cl + j];
                cK[j] = fmaf(wa, cK[j], s_map[ww][1][cl + j]);
                cV[j] = fmaf(wa, cV[j], s_map[ww][2][cl + j]);
                cA[j] *= wa;
            }
        const size_t slot = (size_t)chunk * a.nseq + seq;
        const bool has_next = chunk + 1 < a.nchunk;
        if (has_next) {
            uint64_t* ag = a.agg + slot * (3 * kScanCh);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                store_tagged(ag + cl + j, cA[j], tag);
                store_tagged(ag + kScanCh + cl + j, cK[j], tag);
                store_tagged(ag + 2 * kScanCh + cl + j, cV[j], tag);
            }
        }
        // look back for the carry-in: (rA, rK, rV) is the map of the chunks
        // strictly between the one examined and this one
        float inK[2] = {0.f, 0.f}, inV[2] = {0.f, 0.f};
        if (chunk > 0) {
            float rA[2] = {1.f, 1.f}, rK[2] = {0.f, 0.f}, rV[2] = {0.f, 0.f};
            int p = chunk - 1;
            bool done = false;
            uint32_t spins = 0;
            while (!done) {
                if (p < 0) {
                    inK[0] = rK[0]; inK[1] = rK[1]; inV[0] = rV[0]; inV[1] = rV[1];
                    done = true;
                    break;
                }
                const size_t ps = (size_t)p * a.nseq + seq;
                const uint64_t* ic = a.incl + ps * (2 * kScanCh);
                float x0, x1, y0, y1;
                bool ok = load_tagged(ic + cl, tag, x0);
                ok &= load_tagged(ic + cl + 1, tag, x1);
                ok &= load_tagged(ic + kScanCh + cl, tag, y0);
                ok &= load_tagged(ic + kScanCh + cl + 1, tag, y1);
                if (ok) {
                    inK[0] = fmaf(rA[0], x0, rK[0]); inK[1] = fmaf(rA[1], x1, rK[1]);
                    inV[0] = fmaf(rA[0], y0, rV[0]); inV[1] = fmaf(rA[1], y1, rV[1]);
                    done = true;
                    break;
                }
                const uint64_t* pg = a.agg + ps * (3 * kScanCh);
                float pa0, pa1, pk0, pk1, pv0, pv1;
                bool ok2 = load_tagged(pg + cl, tag, pa0);
                ok2 &= load_tagged(pg + cl + 1, tag, pa1);
                ok2 &= load_tagged(pg + kScanCh + cl, tag, pk0);
                ok2 &= load_tagged(pg + kScanCh + cl + 1, tag, pk1);
                ok2 &= load_tagged(pg + 2 * kScanCh + cl, tag, pv0);
                ok2 &= load_tagged(pg + 2 * kScanCh + cl + 1, tag, pv1);
                if (ok2) {
                    rK[0] = fmaf(rA[0], pk0, rK[0]); rK[1] = fmaf(rA[1], pk1, rK[1]);
                    rV[0] = fmaf(rA[0], pv0, rV[0]); rV[1] = fmaf(rA[1], pv1, rV[1]);
                    rA[0] *= pa0; rA[1] *= pa1;
                    --p;
                    if (rA[0] == 0.f && rA[1] == 0.f) p = -1;  // nothing earlier reaches us
                } else if (++spins > kLookbackSpinLimit) {
                    // watchdog: a carry that never appears poisons the output
                    // instead of hanging the device
                    inK[0] = inK[1] = inV[0] = inV[1] = __builtin_nanf("");
                    done = true;
                } else {
                    __builtin_amdgcn_s_sleep(2);
                }
            }
        }
        if (has_next) {
            uint64_t* ic = a.incl + slot * (2 * kScanCh);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                store_tagged(ic + cl + j, fmaf(cA[j], inK[j], cK[j]), tag);
                store_tagged(ic + kScanCh + cl + j, fmaf(cA[j], inV[j], cV[j]), tag);
            }
        }
        s_carry[0][cl] = inK[0]; s_carry[0][cl + 1] = inK[1];
        s_carry[1][cl] = inV[0]; s_carry[1][cl + 1] = inV[1];
    }
    __syncthreads();

    // carry into this wave: chunk carry-in, then the waves before it
    float hk0 = s_carry[0][cl], hk1 = s_carry[0][cl + 1];
    float hv0 = s_carry[1][cl], hv1 = s_carry[1][cl + 1];
    for (int ww = 0; ww < w; ++ww) {
        const float a0 = s_map[ww][0][cl], a1 = s_map[ww][0][cl + 1];
        hk0 = fmaf(a0, hk0, s_map[ww][1][cl]); hk1 = fmaf(a1, hk1, s_map[ww][1][cl + 1]);
        hv0 = fmaf(a0, hv0, s_map[ww][2][cl]); hv1 = fmaf(a1, hv1, s_map[ww][2][cl + 1]);
    }

    // pass 2: the states, h_t = H_t + P_t * carry
    E* ksp = static_cast<E*>(a.ks) + base;
    E* vsp = static_cast<E*>(a.vs) + base;
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
        const int t = t0 + i;
        if (cvalid && t < a.T) {
            const size_t o = (size_t)t * a.N;
            P::store(ksp + o, fmaf(pg[i][0], hk0, hk[i][0]), fmaf(pg[i][1], hk1, hk[i][1]));
            P::store(vsp + o, fmaf(pg[i][0], hv0, hv[i][0]), fmaf(pg[i][1], hv1, hv[i][1]));
        }
    }

}

// ---------------------------------------------------------------- SLIDING
constexpr int kSlideMaxL = 64;

template <typename E> __device__ __forceinline__ float load1(const E* p);
template <> __device__ __forceinline__ float load1<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float load1<uint16_t>(const uint16_t* p) { return __uint_as_float((uint32_t)*p << 16); }
template <typename E> __device__ __forceinline__ void store1(E* p, float x);
template <> __device__ __forceinline__ void store1<float>(float* p, float x) { *p = x; }
template <> __device__ __forceinline__ void store1<uint16_t>(uint16_t* p, float x) { *p = __builtin_bit_cast(uint16_t, (__bf16)x); }

// One wave = 64 channels (one per lane) x a span of `tiles_per_span` tiles
// of L tokens; the tile before the span is re-read to seed the suffix sums.
template <typename E>
__global__ __launch_bounds__(kWave) void scan_sliding_kernel(ScanSlideArgs a)
{
    __shared__ float s_x[2][kSlideMaxL][kWave];  // suffix sums X_j (k, v) of the previous tile
    const int lane = threadIdx.x;
    const int cgroups = (a.N + kWave - 1) / kWave;
    const int span = blockIdx.x / (a.B * cgroups);
    const int rem = blockIdx.x % (a.B * cgroups);
    const int b = rem / cgroups;
    const int c = (rem % cgroups) * kWave + lane;
    const bool cvalid = c < a.N;
    const int L = a.L;
    const int tile_first = span * a.tiles_per_span;
    const int ntiles = (a.T + L - 1) / L;
    const int tile_end = min(tile_first + a.tiles_per_span, ntiles);
    const size_t base = (size_t)b * a.T * a.N + (cvalid ? c : 0);
    const E* kp = static_cast<const E*>(a.k) + base;
    const E* vp = static_cast<const E*>(a.v) + base;
    const E* gp = static_cast<const E*>(a.g) + base;
    E* ksp = static_cast<E*>(a.ks) + base;
    E* vsp = static_cast<E*>(a.vs) + base;

    for (int j = 0; j < L; ++j) { s_x[0][j][lane] = 0.f; s_x[1][j][lane] = 0.f; }

    for (int m = (tile_first > 0 ? tile_first - 1 : 0); m < tile_end; ++m) {
        const int ts = m * L;
        const int n = min(L, a.T - ts);
        float rk[kSlideMaxL], rv[kSlideMaxL], rg[kSlideMaxL];
#pragma unroll
        for (int j = 0; j < kSlideMaxL; ++j) {
            if (j < n && cvalid) {
                const size_t o = (size_t)(ts + j) * a.N;
                rk[j] = load1<E>(kp + o);
                rv[j] = load1<E>(vp + o);
                rg[j] = load1<E>(gp + o);
            } else {
                rk[j] = 0.f; rv[j] = 0.f; rg[j] = 0.f;
            }
        }
        if (m >= tile_first) {
            // forward: in-tile recurrence plus the previous tile's suffix
            float P = 1.f, Hk = 0.f, Hv = 0.f;
#pragma unroll
            for (int j = 0; j < kSlideMaxL; ++j) {
                if (j < n) {
                    float g, gb;
                    forget_gate(rg[j], g, gb);
                    P *= g;
                    Hk = fmaf(g, Hk, gb * rk[j]);
                    Hv = fmaf(g, Hv, gb * rv[j]);
                    if (cvalid) {
                        const size_t o = (size_t)(ts + j) * a.N;
                        store1<E>(ksp + o, fmaf(P, s_x[0][j][lane], Hk));
                        store1<E>(vsp + o, fmaf(P, s_x[1][j][lane], Hv));
                    }
                }
            }
        }
        // reverse: X_j = sum_{i=j+1}^{L-1} (prod_{r=i+1}^{L-1} g_r)(1-g_i) x_i
        float Q = 1.f, Xk = 0.f, Xv = 0.f;
#pragma unroll
        for (int j = kSlideMaxL - 1; j >= 0; --j) {
            if (j < L) {
                s_x[0][j][lane] = Xk;
                s_x[1][j][lane] = Xv;
                if (j < n) {
                    float g, gb;
                    forget_gate(rg[j], g, gb);
                    Xk = fmaf(Q * gb, rk[j], Xk);
                    Xv = fmaf(Q * gb, rv[j], Xv);
                    Q *= g;
                }
            }
        }
    }
}

// ---------------------------------------------------------------- launches
hipError_t launch_scan_full(const ScanFullArgs& a, bool bf16, hipStream_t stream)
{
    if (bf16)
        hipLaunchKernelGGL((scan_full_kernel<uint16_t, kScanTplBf16>), dim3(a.nwg), dim3(kScanThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((scan_full_kernel<float, kScanTplF32>), dim3(a.nwg), dim3(kScanThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_scan_sliding(const ScanSlideArgs& a, int nblocks, bool bf16, hipStream_t stream)
{
    if (bf16)
        hipLaunchKernelGGL((scan_sliding_kernel<uint16_t>), dim3(nblocks), dim3(kWave), 0, stream, a);
    else
        hipLaunchKernelGGL((scan_sliding_kernel<float>), dim3(nblocks), dim3(kWave), 0, stream, a);
    return hipGetLastError();
}

}  // namespace rat
