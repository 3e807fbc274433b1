// Stage 1 of the RAT+ layer: the gated recurrence over keys and values,
//   h_t = g_t * h_{t-1} + (1 - g_t) * x_t,   g_t = sigmoid(logit_t),
// computed for prefill as a parallel scan ("RAT+ Deep Dive", zhichai.net,
// section 2.1 Full-Sequence Recurrence, and 7.3 "Parallel prefill
// (associative scan)").  The recurrence equation itself is missing from the
// page's text; this is the forget-gate reading of its surrounding words.
//
// Layout [B,T,H,d] puts the scan axis T slowest, so lanes map to channels
// (each lane owns two adjacent channels) and the scan along T is a per-lane
// sequential recurrence with no cross-lane traffic.
//
// FULL / RESTART kernel (one pass over HBM), eight waves per workgroup:
//   * a workgroup owns a chunk of tokens of one block of channels; lane
//     (r, c) of a wave holds 16 bytes of a token row (8 bf16 / 4 fp32
//     channels) for 4 consecutive tokens, so every access is a 16-byte load
//     or store.  Two geometries (ScanGeo): the narrow one spans a 256-byte
//     row segment (128 bf16 / 64 fp32 channels, 16 lanes) with 128-token
//     chunks; the wide one, for the bf16 full recurrence and RESTART periods
//     above 256, a 128-byte segment (64 channels, 8 lanes) with 256-token
//     chunks, half as many chunks per sequence and so half the look-back
//     chain.  The chunk stays in registers from load to store (no LDS
//     staging); 2 workgroups fit on a compute unit;
//   * pass 1: each lane runs the recurrence over its 4 tokens from a zero
//     state; the last state with the gate product forms the segment's
//     affine map h -> A*h + B per channel (the raw inputs stay in
//     registers);
//   * one or two waves turn the chunk's 32 (narrow) or 64 (wide) segment
//     maps into exclusive prefixes (and the chunk's map, which they
//     publish) while another finds the chunk's carry-in by a decoupled
//     look-back over the chunks before it (Merrill & Garland's single-pass
//     scan), through 64-bit words that carry (value, epoch tag) and so need
//     no memory fence;
//   * pass 2 runs the recurrence again from the segment's carry-in (gates
//     evaluated again) and stores the states.
//   Chunk order comes from a ticket counter so that every chunk a
//   workgroup waits for belongs to a workgroup that is already running;
//   the same 64-bit atomic returns the call's epoch.
//   The update is written h = x + g (h - x): one exp and one reciprocal
//   per element give g, and 1 - g is never formed.
//   RESTART (state cleared where t mod L == 0) is the same recurrence with
//   the state before those positions set to 0; a chunk that starts at a restart
//   needs no carry, and a map with A == 0 is published as an inclusive
//   prefix at once and ends the look-back of its successors.
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
#include "rat_plan.h"

namespace rat {

constexpr int kScanThreads = kScanWaves * kWave;
constexpr uint32_t kLookbackSpinLimit = 1u << 22;  // look-back rounds before the watchdog fires
#ifndef RAT_SCAN_LOOKBACK
#define RAT_SCAN_LOOKBACK 1
#endif
constexpr int kLookbackWindow = RAT_SCAN_LOOKBACK;  // predecessors examined per round

template <typename E, bool HIST, bool WIDE>
__global__ __launch_bounds__(kScanFullWaves * kWave, 4) void scan_full_kernel(ScanFullArgs a)
{
    typedef Row16<E> R16;
    constexpr int CPL = R16::CPL;                // channels per lane
    constexpr int LPR = ScanGeo<E, WIDE>::LPR;  // lanes per token row of the block
    constexpr int BW = LPR * CPL;           // channels per block
    constexpr int GPW = kWave / LPR;        // token segments per wave
    constexpr int NSEG = kScanFullWaves * GPW;  // segments per chunk
    constexpr int TPL = kScanTpl;           // tokens per segment
    constexpr int CT = NSEG * TPL;          // tokens per chunk
    constexpr int C0 = BW / kWave;          // channels per lane of the single-wave steps
    constexpr int PW = C0 > 1 ? 2 : 1;      // waves of the segment prefix step
    constexpr int CP = BW / (PW * kWave);   // channels per lane there
    static_assert(CT == ScanGeo<E, WIDE>::CT && BW == ScanGeo<E, WIDE>::BW, "geometry shared with the host plan");
    // segment maps (A, K, V) per channel; then their exclusive prefixes
    __shared__ float s_seg[NSEG][3][BW];
    __shared__ float s_carry[2][BW];  // chunk carry-in (hk, hv)
    __shared__ float s_tot[3][BW];    // the chunk's map
    __shared__ uint32_t s_ticket, s_epoch;

    const int lane = threadIdx.x & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
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
    // lane (r, c): channels cblk + CPL c .. +CPL, tokens t0 .. t0 + TPL - 1
    const ScanLane sl = scan_lane<CPL, LPR>(a, ticket, w, lane);
    const int chunk = sl.chunk, seq = sl.seq, b = sl.b;
    const int cblk = sl.cblk;  // first channel of the block
    const int tb = sl.tb;      // first token of the chunk
    const int c = sl.c, seg = sl.seg, ch0 = sl.ch0, t0 = sl.t0;
    const bool cvalid = sl.cvalid;
    // element offset of the lane's first token row; token t0 + i is i N further
    // (one 64-bit offset per lane, the i N terms uniform)
    const size_t obase = ((size_t)b * a.T + t0) * a.N + ch0;

    u32x4 rk[TPL], rv[TPL], rg[TPL];
    if (tb + CT <= a.T && cblk + BW <= a.N) {  // the whole chunk exists (uniform)
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            const size_t o = obase + (size_t)i * a.N;
            rk[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const E*>(a.k) + o));
            rv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const E*>(a.v) + o));
            rg[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const E*>(a.g) + o));
        }
    } else {
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            if (cvalid && t0 + i < a.T) {
                const size_t o = obase + (size_t)i * a.N;
                rk[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const E*>(a.k) + o));
                rv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const E*>(a.v) + o));
                rg[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const E*>(a.g) + o));
            } else {
                rk[i] = rv[i] = rg[i] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    }
    // RESTART positions (t mod L == 0) of this segment, as a bit mask
    uint32_t rmask = 0;
    if (a.L > 0) {
        for (int t = ((t0 + a.L - 1) / a.L) * a.L; t < t0 + TPL; t += a.L) rmask |= 1u << (t - t0);
    }

    // Both passes come in two forms.  The fast one serves a wave whose
    // segments all lie inside the sequence and hold no RESTART position
    // (every wave of a whole chunk of the full recurrence): with no per-token
    // liveness or restart test, the gates of all tokens and channels form
    // straight-line code the compiler can interleave.  The general form
    // handles the ragged end and the restarts.
    const bool fast = tb + CT <= a.T && cblk + BW <= a.N && !__any(rmask != 0u);

    // pass 1: the segment's map h -> A h + (K, V), its recurrence from a
    // zero state (the raw inputs stay in registers for pass 2)
    float A[CPL], K[CPL], V[CPL];
    auto pass1 = [&](auto fast_form) {
        constexpr bool FAST = decltype(fast_form)::value;
#pragma unroll
        for (int j = 0; j < CPL; ++j) { A[j] = 1.f; K[j] = 0.f; V[j] = 0.f; }
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            const bool live = FAST || t0 + i < a.T;
            const bool restart = !FAST && ((rmask >> i) & 1u);
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const float g = gate(R16::get(rg[i], j));
                if (restart) {  // the state before this token is cleared: the map forgets its input
                    A[j] = 0.f;
                    K[j] = 0.f;
                    V[j] = 0.f;
                }
                if (live) {
                    const float xk = R16::get(rk[i], j), xv = R16::get(rv[i], j);
                    A[j] *= g;
                    K[j] = fmaf(g, K[j] - xk, xk);
                    V[j] = fmaf(g, V[j] - xv, xv);
                }
            }
        }
    };
    if (fast) pass1(BoolC<true>{});
    else pass1(BoolC<false>{});
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        s_seg[seg][0][c * CPL + j] = A[j];
        s_seg[seg][1][c * CPL + j] = K[j];
        s_seg[seg][2][c * CPL + j] = V[j];
    }
    __syncthreads();

    const size_t slot = (size_t)chunk * a.nseq + seq;
    const bool has_next = chunk + 1 < a.nchunk;
    uint64_t* ic_out = a.incl + slot * (2 * BW);
    if (w == 0) {
        // the carry-in (decoupled look-back); no carry is needed at the first
        // chunk or when the chunk starts at a restart
        float inK[C0], inV[C0];
#pragma unroll
        for (int j = 0; j < C0; ++j) { inK[j] = 0.f; inV[j] = 0.f; }
        if (chunk > 0 && !(a.L > 0 && tb % a.L == 0)) {
            // (rA, rK, rV): map of the chunks strictly between the one
            // examined and this one
            float rA[C0], rK[C0], rV[C0];
#pragma unroll
            for (int j = 0; j < C0; ++j) { rA[j] = 1.f; rK[j] = 0.f; rV[j] = 0.f; }
            // each round loads the words of kLookbackWindow predecessors at
            // once (one memory latency), then walks them newest first
            int p = chunk - 1;
            uint32_t spins = 0;
            bool done = false;
            while (!done) {
                float x[kLookbackWindow][C0], y[kLookbackWindow][C0];
                float pa[kLookbackWindow][C0], pk[kLookbackWindow][C0], pv[kLookbackWindow][C0];
                bool ok[kLookbackWindow], ok2[kLookbackWindow];
#pragma unroll
                for (int q = 0; q < kLookbackWindow; ++q) {
                    ok[q] = ok2[q] = false;
                    if (p - q < 0) continue;
                    const size_t ps = (size_t)(p - q) * a.nseq + seq;
                    const uint64_t* ic = a.incl + ps * (2 * BW);
                    const uint64_t* ag = a.agg + ps * (3 * BW);
                    ok[q] = ok2[q] = true;
#pragma unroll
                    for (int j = 0; j < C0; ++j) {
                        ok[q] &= load_tagged(ic + lane * C0 + j, tag, x[q][j]);
                        ok[q] &= load_tagged(ic + BW + lane * C0 + j, tag, y[q][j]);
                        ok2[q] &= load_tagged(ag + lane * C0 + j, tag, pa[q][j]);
                        ok2[q] &= load_tagged(ag + BW + lane * C0 + j, tag, pk[q][j]);
                        ok2[q] &= load_tagged(ag + 2 * BW + lane * C0 + j, tag, pv[q][j]);
                    }
                }
                bool stalled = false;
#pragma unroll
                for (int q = 0; q < kLookbackWindow; ++q) {
                    if (done || stalled) continue;
                    if (p < 0) {  // before the first chunk: the carry is the map of zero
#pragma unroll
                        for (int j = 0; j < C0; ++j) { inK[j] = rK[j]; inV[j] = rV[j]; }
                        done = true;
                    } else if (ok[q]) {  // inclusive prefix of chunk p
#pragma unroll
                        for (int j = 0; j < C0; ++j) {
                            inK[j] = fmaf(rA[j], x[q][j], rK[j]);
                            inV[j] = fmaf(rA[j], y[q][j], rV[j]);
                        }
                        done = true;
                    } else if (ok2[q]) {  // aggregate of chunk p: fold it in, go on
                        bool zero = true;
#pragma unroll
                        for (int j = 0; j < C0; ++j) {
                            rK[j] = fmaf(rA[j], pk[q][j], rK[j]);
                            rV[j] = fmaf(rA[j], pv[q][j], rV[j]);
                            rA[j] *= pa[q][j];
                            zero &= rA[j] == 0.f;
                        }
                        --p;
                        if (zero) p = -1;  // nothing earlier reaches this chunk
                    } else {
                        stalled = true;  // chunk p has published nothing yet
                    }
                }
                if (!done && p < 0) {
#pragma unroll
                    for (int j = 0; j < C0; ++j) { inK[j] = rK[j]; inV[j] = rV[j]; }
                    done = true;
                }
                if (!done && stalled) {
                    if (++spins > kLookbackSpinLimit) {
                        // watchdog: a carry that never appears poisons the
                        // output instead of hanging the device
#pragma unroll
                        for (int j = 0; j < C0; ++j) inK[j] = inV[j] = __builtin_nanf("");
                        done = true;
                    } else {
                        __builtin_amdgcn_s_sleep(1);
                    }
                }
            }
        }
#pragma unroll
        for (int j = 0; j < C0; ++j) {
            s_carry[0][lane * C0 + j] = inK[j];
            s_carry[1][lane * C0 + j] = inV[j];
        }
    } else if (w <= PW) {
        // meanwhile, waves 1 .. PW (a share of the channels each): exclusive
        // prefix maps of the segments (in place), the chunk's map and its
        // publication (the aggregate, or at once the inclusive prefix when a
        // restart makes the map ignore its carry-in)
        bool closed = true;
        float cA[CP], cK[CP], cV[CP];
#pragma unroll
        for (int j = 0; j < CP; ++j) {
            const int ch = ((w - 1) * kWave + lane) * CP + j;
            float pA = 1.f, pK = 0.f, pV = 0.f;
#pragma unroll 8
            for (int s2 = 0; s2 < NSEG; ++s2) {
                const float sa = s_seg[s2][0][ch], sk = s_seg[s2][1][ch], sv = s_seg[s2][2][ch];
                s_seg[s2][0][ch] = pA;
                s_seg[s2][1][ch] = pK;
                s_seg[s2][2][ch] = pV;
                pK = fmaf(sa, pK, sk);
                pV = fmaf(sa, pV, sv);
                pA *= sa;
            }
            cA[j] = pA; cK[j] = pK; cV[j] = pV;
            s_tot[0][ch] = pA; s_tot[1][ch] = pK; s_tot[2][ch] = pV;
            closed &= pA == 0.f;
        }
        // the successors' look-back reads the words of C0 adjacent channels
        // per lane and needs them all of one kind: decide over that group
        // (adjacent lanes here when CP < C0)
        if (CP < C0) {
#pragma unroll
            for (int m = CP; m < C0; m *= 2) closed &= __shfl_xor((int)closed, m / CP) != 0;
        }
        if (has_next) {
            const int ch0p = ((w - 1) * kWave + lane) * CP;
            if (closed) {
#pragma unroll
                for (int j = 0; j < CP; ++j) {
                    store_tagged(ic_out + ch0p + j, cK[j], tag);
                    store_tagged(ic_out + BW + ch0p + j, cV[j], tag);
                }
            } else {
                uint64_t* ag = a.agg + slot * (3 * BW);
#pragma unroll
                for (int j = 0; j < CP; ++j) {
                    store_tagged(ag + ch0p + j, cA[j], tag);
                    store_tagged(ag + BW + ch0p + j, cK[j], tag);
                    store_tagged(ag + 2 * BW + ch0p + j, cV[j], tag);
                }
            }
        }
    }
    __syncthreads();
    if (w == 0 && has_next) {
        // the inclusive prefix of this chunk (already out when closed)
        bool closed = true;
#pragma unroll
        for (int j = 0; j < C0; ++j) closed &= s_tot[0][lane * C0 + j] == 0.f;
        if (!closed) {
#pragma unroll
            for (int j = 0; j < C0; ++j) {
                const int ch = lane * C0 + j;
                store_tagged(ic_out + ch, fmaf(s_tot[0][ch], s_carry[0][ch], s_tot[1][ch]), tag);
                store_tagged(ic_out + BW + ch, fmaf(s_tot[0][ch], s_carry[1][ch], s_tot[2][ch]), tag);
            }
        }
    }

    // pass 2: the recurrence again, from the segment's carry-in (gates
    // evaluated again; the empty asm hides the logits' identity from
    // common-subexpression elimination, which would keep pass 1's gates in
    // 8 more registers per token)
    HistRow hr;
    size_t hbase = 0;
    if (HIST) {  // the lane's head, its history block and the row of t0
        hr.init(t0, scan_hist_D(a, sl), a.hist.n_cap);
        hbase = scan_hist_base(a, sl);
    }
    float ck[CPL], cv[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int ch = c * CPL + j;
        const float pa = s_seg[seg][0][ch];
        ck[j] = fmaf(pa, s_carry[0][ch], s_seg[seg][1][ch]);
        cv[j] = fmaf(pa, s_carry[1][ch], s_seg[seg][2][ch]);
    }
    // the store offset, formed again from the lane index: the empty asm hides
    // that it equals the loads' offset, so no 64-bit address stays live (and
    // spills) across the passes
    int lane2 = lane;
    asm volatile("" : "+v"(lane2));
    const size_t sbase = ((size_t)b * a.T + tb + (w * GPW + lane2 / LPR) * TPL) * a.N + cblk + (lane2 % LPR) * CPL;
    // the last position's states in fp32, for a decode loop to continue from
    // (a lane's CPL channels lie in one head: d is a multiple of 64)
    float* fin = nullptr;
    if (a.fin && cvalid) fin = a.fin + scan_fin_offset(a, sl);
    auto pass2 = [&](auto fast_form) {
        constexpr bool FAST = decltype(fast_form)::value;
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            asm volatile("" : "+v"(rg[i]));
            const bool restart = !FAST && ((rmask >> i) & 1u);
            float ok[CPL], ov[CPL];
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const float g = gate(R16::get(rg[i], j));
                if (restart) {  // cleared state before this token
                    ck[j] = 0.f;
                    cv[j] = 0.f;
                }
                const float xk = R16::get(rk[i], j), xv = R16::get(rv[i], j);
                ck[j] = fmaf(g, ck[j] - xk, xk);
                cv[j] = fmaf(g, cv[j] - xv, xv);
                ok[j] = ck[j];
                ov[j] = cv[j];
            }
            // non-temporal stores: measured, they leave the attention that
            // reads the states next faster than cacheable ones do (the scan
            // itself runs as fast either way)
            if (FAST || (cvalid && t0 + i < a.T)) {
                const size_t o = HIST ? hbase + (size_t)hr.row() * a.d : sbase + (size_t)i * a.N;
                __builtin_nontemporal_store(R16::pack(ok), reinterpret_cast<u32x4*>(static_cast<E*>(a.ks) + o));
                __builtin_nontemporal_store(R16::pack(ov), reinterpret_cast<u32x4*>(static_cast<E*>(a.vs) + o));
            }
            if (HIST) hr.next();
            if (!FAST && fin && t0 + i == a.T - 1) {
#pragma unroll
                for (int j = 0; j < CPL; ++j) {
                    fin[j] = ok[j];
                    fin[a.d + j] = ov[j];
                }
            }
        }
        // fast form: every token of the segment is live, so the state after
        // the loop is that of its last token
        if (FAST && fin && t0 + TPL == a.T) {
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                fin[j] = ck[j];
                fin[a.d + j] = cv[j];
            }
        }
    };
    if (fast) pass2(BoolC<true>{});
    else pass2(BoolC<false>{});
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
template <typename E, bool HIST>
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
    int hD = 1;
    if (HIST) {  // the lane's head and its history block
        const int hh = (cvalid ? c : 0) / a.hist.d;
        hD = a.hist.D[hh];
        const size_t hb = ((size_t)b * a.hist.H + hh) * a.hist.n_cap * a.hist.d + ((cvalid ? c : 0) - hh * a.hist.d);
        ksp = static_cast<E*>(a.ks) + hb;
        vsp = static_cast<E*>(a.vs) + hb;
    }

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
            HistRow hr;
            if (HIST) hr.init(ts, hD, a.hist.n_cap);
#pragma unroll
            for (int j = 0; j < kSlideMaxL; ++j) {
                if (j < n) {
                    float g, gb;
                    forget_gate(rg[j], g, gb);
                    P *= g;
                    Hk = fmaf(g, Hk, gb * rk[j]);
                    Hv = fmaf(g, Hv, gb * rv[j]);
                    if (cvalid) {
                        const size_t o = HIST ? (size_t)hr.row() * a.hist.d : (size_t)(ts + j) * a.N;
                        store1<E>(ksp + o, fmaf(P, s_x[0][j][lane], Hk));
                        store1<E>(vsp + o, fmaf(P, s_x[1][j][lane], Hv));
                    }
                    if (HIST) hr.next();
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

// ------------------------------------------------------- SLIDING, L = 64
// bf16 fast path of the pages' window L* = 64: a workgroup takes 128 tokens
// (two 64-token tiles) of one 64-channel block plus the 64 tokens before
// them, copied into LDS 16 bytes per lane.  Wave w owns tokens 16w .. 16w+15
// of the chunk, lane = channel: a forward recurrence from zero over its
// tokens, and a reverse one over the same 16 offsets of the previous tile.
// Through LDS each wave then takes the in-tile carry from the waves before
// it and the previous tile's suffix from the waves after it, which gives
// every token its suffix
// X_j = sum_{s=j+1}^{63} (prod_{r=s+1}^{63} g_r)(1-g_s) x_s, and
// h_t = H_t + P_t * X_j with H_t, P_t the in-tile state and gate product.
// The previous tile is re-read once per chunk (1.5x input bytes); two
// workgroups fit on a compute unit.
constexpr int kSlideCT = 128, kSlideHalo = 64, kSlideBW = 64;

template <bool HIST>
__global__ __launch_bounds__(kScanThreads) void scan_slide64_kernel(ScanSlideArgs a)
{
    constexpr int ROWB = kSlideBW * 2;           // bytes of a 64-channel bf16 row
    constexpr int NROW = kSlideCT + kSlideHalo;  // rows per tensor in LDS
    constexpr int RPG = 1024 / ROWB;             // rows per 1 KiB wave copy
    constexpr int LPR = ROWB / 16;               // lanes per row in a wave copy
    constexpr int TPW = kSlideCT / kScanWaves;   // tokens per wave
    constexpr int NIN = 3 * NROW / RPG;
    constexpr int NOUT = 2 * kSlideCT / RPG;
    static_assert(NIN % kScanWaves == 0 && NOUT % kScanWaves == 0 && NROW % RPG == 0, "even copies");
    static_assert(kSlideBW == kWave, "one channel per lane");
    extern __shared__ __attribute__((aligned(1024))) char s_tile[];  // [3][NROW][ROWB]: k, v, logits
    // forward segment maps (A, K, V) and previous-tile segments (Q, Sk, Sv):
    // 12 KiB over the first k rows of the tile, written once every wave has
    // read its inputs there.  Separate arrays would take the workgroup to
    // 84 KiB, and two would no longer fit a CU's 160 KiB of LDS.
    typedef float SegMaps[3][kSlideBW];
    SegMaps* s_map = reinterpret_cast<SegMaps*>(s_tile);
    SegMaps* s_rev = reinterpret_cast<SegMaps*>(s_tile + sizeof(SegMaps) * kScanWaves);
    static_assert(2 * sizeof(SegMaps) * kScanWaves <= (size_t)NROW * ROWB, "segment maps fit the k rows");
    __shared__ int s_hrow[HIST ? kSlideCT : 1];         // history row of each token of the chunk

    const int lane = threadIdx.x & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int nblk = a.N / kSlideBW;
    const int blk = blockIdx.x % nblk;
    const int b = (blockIdx.x / nblk) % a.B;
    const int chunk = blockIdx.x / (nblk * a.B);
    const int tb = chunk * kSlideCT;             // first token of the chunk
    const int r0 = tb - kSlideHalo;              // token of LDS row 0
    const size_t rowbase = (size_t)b * a.T * a.N + (size_t)blk * kSlideBW;
    size_t hbase = 0;  // the block's channels in its head's history (one head: d is 64 or 128)
    if (HIST) {
        const int hh = blk * kSlideBW / a.hist.d;
        hbase = ((size_t)b * a.hist.H + hh) * a.hist.n_cap * a.hist.d + (blk * kSlideBW - hh * a.hist.d);
        if (threadIdx.x < kSlideCT) {
            const int D = a.hist.D[hh], t = tb + threadIdx.x;
            s_hrow[threadIdx.x] = (t % D) * (a.hist.n_cap / D) + t / D;
        }
    }

    {
        const uint16_t* src[3] = {static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v),
                                  static_cast<const uint16_t*>(a.g)};
#pragma unroll
        for (int j = 0; j < NIN / kScanWaves; ++j) {
            const int q = j * kScanWaves + w;
            const int row = q * RPG + lane / LPR;
            const int t = min(max(r0 + row % NROW, 0), a.T - 1);
            dma16(src[row / NROW] + rowbase + (size_t)t * a.N + (lane % LPR) * 8, s_tile + q * 1024);
        }
    }
    wait_vmcnt<0>();
    __syncthreads();

    auto at = [&](int tensor, int row) -> float {  // channel `lane` of an LDS row
        const uint16_t x = *reinterpret_cast<const uint16_t*>(s_tile + (tensor * NROW + row) * ROWB + lane * 2);
        return __uint_as_float((uint32_t)x << 16);
    };

    // forward: local recurrence over this wave's tokens from a zero state
    // (h = x + g (h - x))
    const int rw = kSlideHalo + w * TPW;  // LDS row of the wave's first token
    float A = 1.f, K = 0.f, V = 0.f;
    float hk[TPW], hv[TPW], pg[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const float g = gate(at(2, rw + i));
        const float xk = at(0, rw + i), xv = at(1, rw + i);
        A *= g;
        K = fmaf(g, K - xk, xk);
        V = fmaf(g, V - xv, xv);
        hk[i] = K; hv[i] = V; pg[i] = A;
    }
    // reverse over the same offsets of the previous tile (LDS rows
    // 64 tl + 16 wt ..): lk / lv[i] = the segment's suffix after offset
    // 16 wt + i, weighted to the segment's end; (Q, Sk, Sv) = the whole
    // segment's gate product and suffix
    const int tl = w / 4, wt = w % 4;
    const bool has_prev = tb + 64 * tl > 0;
    const int pr = 64 * tl + TPW * wt;
    float lk[TPW], lv[TPW];
    float Q = 1.f, Sk = 0.f, Sv = 0.f;
#pragma unroll
    for (int i = TPW - 1; i >= 0; --i) {
        lk[i] = Sk;
        lv[i] = Sv;
        float g, gb;
        forget_gate(at(2, pr + i), g, gb);
        const float qg = Q * gb;
        Sk = fmaf(qg, at(0, pr + i), Sk);
        Sv = fmaf(qg, at(1, pr + i), Sv);
        Q *= g;
    }
    __syncthreads();  // every wave is done reading the k rows the maps overwrite
    s_map[w][0][lane] = A;
    s_map[w][1][lane] = K;
    s_map[w][2][lane] = V;
    s_rev[w][0][lane] = Q;
    s_rev[w][1][lane] = Sk;
    s_rev[w][2][lane] = Sv;
    __syncthreads();

    // in-tile carry: the waves of this tile before this one
    float cA = 1.f, cK = 0.f, cV = 0.f;
    for (int ww = 4 * tl; ww < w; ++ww) {
        const float sa = s_map[ww][0][lane];
        cK = fmaf(sa, cK, s_map[ww][1][lane]);
        cV = fmaf(sa, cV, s_map[ww][2][lane]);
        cA *= sa;
    }
    // the previous tile's segments after this one: suffix Z and gate product G
    float G = 1.f, Zk = 0.f, Zv = 0.f;
    for (int ww = 4 * tl + 3; ww > w; --ww) {
        Zk = fmaf(s_rev[ww][1][lane], G, Zk);
        Zv = fmaf(s_rev[ww][2][lane], G, Zv);
        G *= s_rev[ww][0][lane];
    }
    // X_j = G * l_j + Z over the window's part in the previous tile, then
    // h = H + P (carry + A X_j)
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const float xk = has_prev ? fmaf(G, lk[i], Zk) : 0.f;
        const float xv = has_prev ? fmaf(G, lv[i], Zv) : 0.f;
        hk[i] = fmaf(pg[i], fmaf(cA, xk, cK), hk[i]);
        hv[i] = fmaf(pg[i], fmaf(cA, xv, cV), hv[i]);
    }
    __syncthreads();  // every wave is done reading the inputs

    // states over the chunk's key / value rows, then 16-byte stores
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        *reinterpret_cast<uint16_t*>(s_tile + (rw + i) * ROWB + lane * 2) = __builtin_bit_cast(uint16_t, (__bf16)hk[i]);
        *reinterpret_cast<uint16_t*>(s_tile + (NROW + rw + i) * ROWB + lane * 2) =
            __builtin_bit_cast(uint16_t, (__bf16)hv[i]);
    }
    __syncthreads();
    {
        uint16_t* dst[2] = {static_cast<uint16_t*>(a.ks), static_cast<uint16_t*>(a.vs)};
#pragma unroll
        for (int j = 0; j < NOUT / kScanWaves; ++j) {
            const int q = j * kScanWaves + w;
            const int row = q * RPG + lane / LPR;  // 0 .. 2 CT - 1
            const int tensor = row / kSlideCT, tok = row % kSlideCT;
            const u32x4 val = *reinterpret_cast<const u32x4*>(
                s_tile + (tensor * NROW + kSlideHalo + tok) * ROWB + (lane % LPR) * 16);
            if (tb + tok < a.T) {
                const size_t o = HIST ? hbase + (size_t)s_hrow[tok] * a.hist.d : rowbase + (size_t)(tb + tok) * a.N;
                *reinterpret_cast<u32x4*>(dst[tensor] + o + (lane % LPR) * 8) = val;
            }
        }
    }
}

// ---------------------------------------------------------------- launches
hipError_t launch_scan_full(const ScanFullArgs& a, bool bf16, bool hist, bool wide, hipStream_t stream)
{
    const dim3 grid(a.nwg), block(kScanFullWaves * kWave);
    if (bf16 && wide && hist) hipLaunchKernelGGL((scan_full_kernel<uint16_t, true, true>), grid, block, 0, stream, a);
    else if (bf16 && wide) hipLaunchKernelGGL((scan_full_kernel<uint16_t, false, true>), grid, block, 0, stream, a);
    else if (bf16 && hist) hipLaunchKernelGGL((scan_full_kernel<uint16_t, true, false>), grid, block, 0, stream, a);
    else if (bf16) hipLaunchKernelGGL((scan_full_kernel<uint16_t, false, false>), grid, block, 0, stream, a);
    else if (hist) hipLaunchKernelGGL((scan_full_kernel<float, true, false>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((scan_full_kernel<float, false, false>), grid, block, 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_scan_sliding(const ScanSlideArgs& a, int nblocks, bool bf16, bool hist, hipStream_t stream)
{
    const dim3 grid(nblocks), block(kWave);
    if (bf16 && hist) hipLaunchKernelGGL((scan_sliding_kernel<uint16_t, true>), grid, block, 0, stream, a);
    else if (bf16) hipLaunchKernelGGL((scan_sliding_kernel<uint16_t, false>), grid, block, 0, stream, a);
    else if (hist) hipLaunchKernelGGL((scan_sliding_kernel<float, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((scan_sliding_kernel<float, false>), grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace rat

namespace rat {
hipError_t launch_scan_slide64(const ScanSlideArgs& a, bool hist, hipStream_t stream)
{
    static bool attr[2] = {false, false};
    const size_t lds = 3 * (size_t)(kSlideCT + kSlideHalo) * kSlideBW * 2;
    const void* fn = hist ? (const void*)scan_slide64_kernel<true> : (const void*)scan_slide64_kernel<false>;
    if (!attr[hist]) {
        (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        attr[hist] = true;
    }
    const int nchunk = (a.T + kSlideCT - 1) / kSlideCT;
    const dim3 grid(nchunk * a.B * (a.N / kSlideBW)), block(kScanThreads);
    if (hist) hipLaunchKernelGGL(scan_slide64_kernel<true>, grid, block, lds, stream, a);
    else hipLaunchKernelGGL(scan_slide64_kernel<false>, grid, block, lds, stream, a);
    return hipGetLastError();
}
}  // namespace rat
