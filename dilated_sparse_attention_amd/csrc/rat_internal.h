// Internal launch interface between the C ABI (abi.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rat {

constexpr int kAttnMaxHeads = 256;

// Per-residue state history (the decode cache): the state of head h at
// position p is row (p mod D[h]) * (n_cap / D[h]) + p / D[h] of that head's
// [n_cap][d] block, heads [B][H] outermost.  The rows of one residue are
// contiguous and in position order.
struct StateHist {
    int n_cap;  // rows per head
    int d, H;
    int D[kAttnMaxHeads];
};

// ---------------------------------------------------------------- scan
// Tile of the full / RESTART scan: a workgroup of kScanFullWaves waves
// covers one block of BW channels x CT tokens; each lane holds 16 bytes of a
// row (CPL = 8 bf16 / 4 fp32 channels) for kScanTpl consecutive tokens, LPR
// lanes per token row.  Narrow: 16 lanes (256-byte row segments, four token
// segments per wave).  Wide (bf16 only): 8 lanes (128-byte segments of 64
// channels, eight token segments per wave), so a chunk holds twice the
// tokens and a sequence half the chunks: shorter look-back chains, a
// longer in-chunk segment prefix.
constexpr int kScanWaves = 8;  // the SLIDING L = 64 kernel's workgroup
#ifndef RAT_SCAN_FULL_WAVES
#define RAT_SCAN_FULL_WAVES 8
#endif
constexpr int kScanFullWaves = RAT_SCAN_FULL_WAVES;  // the full / RESTART kernel's workgroup
constexpr int kScanTpl = 4;
template <typename E, bool WIDE>
struct ScanGeo {
    static constexpr int CPL = 16 / (int)sizeof(E);
    static constexpr int LPR = (WIDE && sizeof(E) == 2) ? 8 : 16;
    static constexpr int BW = LPR * CPL;                               // channels per block
    static constexpr int CT = kScanFullWaves * (64 / LPR) * kScanTpl;  // tokens per chunk
};

struct ScanHeader {
    // low 32 bits: next chunk ticket of the running call; high 32 bits:
    // calls completed on this workspace (carry tags are epoch + 1).  One
    // atomic add hands a workgroup both; the workgroup that draws the last
    // ticket starts the next epoch with ticket 0.
    uint64_t tick;
    uint32_t pad[62];
};

struct ScanFullArgs {
    const void* k;
    const void* v;
    const void* g;
    void* ks;
    void* vs;
    int T, N;      // tokens; channels per token (H*d)
    int nblk;      // 128-channel blocks per token row
    int nseq;      // B * nblk
    int nchunk;    // chunks along T
    int L;         // RESTART period, 0 for none
    int nwg;       // nchunk * nseq
    uint64_t* agg;   // [nchunk*nseq][3][block] tagged words
    uint64_t* incl;  // [nchunk*nseq][2][block] tagged words
    ScanHeader* hdr;
    float* fin;      // optional fp32 states at t = T-1, [B][H][2][d] (NULL: none)
    int d;           // head size (for `fin`)
    StateHist hist;  // state layout of the history-writing instances
};

struct ScanSlideArgs {
    const void* k;
    const void* v;
    const void* g;
    void* ks;
    void* vs;
    int B, T, N, L, tiles_per_span;
    StateHist hist;  // state layout of the history-writing instances
};

// hist: write the states as a StateHist instead of [B][T][H][d]
hipError_t launch_scan_full(const ScanFullArgs& a, bool bf16, bool hist, bool wide, hipStream_t stream);
hipError_t launch_scan_sliding(const ScanSlideArgs& a, int nblocks, bool bf16, bool hist, hipStream_t stream);
// SLIDING with L = 64 in bf16 (N a multiple of 64)
hipError_t launch_scan_slide64(const ScanSlideArgs& a, bool hist, hipStream_t stream);

// ---------------------------------------------------------------- attention
constexpr int kAttnMaxClasses = 8;

struct AttnClass {
    int D, W;
    int nheads;      // heads in this class
    int head_off;    // first entry in AttnArgs::heads
    int levels;      // cost levels (dispatched most expensive first)
    int per_level;   // items per level
    int block_begin; // first item of the class
};

struct AttnArgs {
    const void* q;
    const void* ks;
    const void* vs;
    const void* kr;
    const void* vr;
    void* out;
    float* ml;         // [B][T][H][2] partial (m, l) of the band pass (heads with W > 0)
    int B, T, H;
    float scale_log2;  // softmax scale * log2(e)
    int chunk;         // 1: chunk grid -- keys are the chunk-end states (residue D-1), strictly before the query
    int n_cap;         // > 0: ks / vs are a StateHist with n_cap rows per head (relative dilation only)
    int nclass;
    int nblocks;
    int rows;          // query rows per item: 32 per wave of the kernel that runs the plan
    AttnClass cls[kAttnMaxClasses];
    int heads[kAttnMaxHeads];  // 32-bit: scalar loads have no 16-bit form
};

// dilated states of the plan's classes: persistent kernel, `grid`
// workgroups (nblocks = items) of a.rows / 32 waves -- eight waves on a
// deep ring, one workgroup per CU (a.rows = 256), or four waves on a
// two-slot ring, two workgroups per CU (a.rows = 128)
hipError_t launch_attn_dilated_bf16(const AttnArgs& a, int d, int grid, hipStream_t stream);
// raw-key band of heads with W > 0: the same kernel over items of a.rows
// contiguous queries (four waves, a.rows = 128)
hipError_t launch_attn_band_bf16(const AttnArgs& a, int d, int grid, hipStream_t stream);

// Simple fp32 path (one workgroup per query row; exact fp32 arithmetic).
struct AttnF32Args {
    const float* q;
    const float* ks;
    const float* vs;
    const float* kr;
    const float* vr;
    float* out;
    int B, T, H, d;
    float scale;
    int chunk;  // 1: chunk grid (chunk-end states before t, then the own state)
    int n_cap;  // > 0: ks / vs are a StateHist with n_cap rows per head
    int D[kAttnMaxHeads];
    int W[kAttnMaxHeads];
};
hipError_t launch_attn_prefill_f32(const AttnF32Args& a, hipStream_t stream);

// ---------------------------------------------------------------- decode
constexpr int kDecWaves = 4;

struct DecodeArgs {
    const void* q;
    const void* kd;
    const void* vd;
    const void* kw;
    const void* vw;
    void* out;
    float* part;     // split partials [B*H][nsplit][d + 2] (NULL when nsplit == 1)
    int B, H, T, nd_cap, w_cap;
    int nsplit;      // key-range splits per (b, h)
    float scale_log2;
    int D[kAttnMaxHeads];
    int W[kAttnMaxHeads];
    int dil_off[kAttnMaxHeads];  // first cache row of head h's dilated entries
};
hipError_t launch_decode(const DecodeArgs& a, int d, bool bf16, hipStream_t stream);

// Split partials of the decode entry point that allocates nothing: a
// file-scope device array of kDecodeScratchBytes per GPU, held until the
// process ends.  decode_scratch returns its address on the current device
// (looked up once per device, with that device current).
constexpr size_t kDecodeScratchBytes = (size_t)1 << 20;
hipError_t decode_scratch(void** ptr);

// Recurrence step of the decode loop: the new token's state from the
// running fp32 state, written to the state history and the raw ring.
struct StepArgs {
    const void* k_new;
    const void* v_new;
    const void* g_new;   // [B][H][d]
    float* state;        // [B][H][2][d] running states (k, v), in / out
    void* kc;
    void* vc;            // [B][H][n_cap][d] state history
    void* kw;
    void* vw;            // [B][H][w_cap][d] raw ring
    int B, H, d, n_cap, w_cap;
    int restart;         // 1: the new position starts a RESTART period (state cleared)
    int slot_c[kAttnMaxHeads];  // history row of the new position
    int slot_w[kAttnMaxHeads];  // ring slot of the new position, -1 without a window
};
hipError_t launch_decode_step(const StepArgs& a, bool bf16, hipStream_t stream);

// Recurrence step of the decode loop under a SLIDING window of L tokens: the
// new state is the recurrence from a zero state over the last L positions,
// whose raw key, value and gate logit a ring of L slots keeps (position p in
// slot p mod L; the new token's slot is written here).
struct SlideStepArgs {
    const void* k_new;
    const void* v_new;
    const void* g_new;   // [B][H][d]
    void* rk;
    void* rv;
    void* rg;            // [B][H][L][d] raw ring of the recurrence window
    void* kc;
    void* vc;            // [B][H][n_cap][d] state history
    void* kw;
    void* vw;            // [B][H][w_cap][d] raw ring of the attention window
    int B, H, d, n_cap, w_cap, L;
    int p;               // position of the new token (T - 1)
    int slot_c[kAttnMaxHeads];  // history row of the new position
    int slot_w[kAttnMaxHeads];  // attention-ring slot of the new position, -1 without a window
};
hipError_t launch_decode_step_sliding(const SlideStepArgs& a, bool bf16, hipStream_t stream);

// The SLIDING decode state of a prefill: raw k, v, gate logits of positions
// max(0, T - L) .. T-1 ([B][T][H][d]) into slot p mod L of rk, rv, rg
// ([B][H][L][d]).
struct SlideFillArgs {
    const void* k;
    const void* v;
    const void* g;
    void* rk;
    void* rv;
    void* rg;
    int B, T, H, d, L;
};
hipError_t launch_sliding_fill(const SlideFillArgs& a, bool bf16, hipStream_t stream);

// Raw ring of a prefill: positions max(0, T - W[h]) .. T-1 of k, v
// ([B][T][H][d]) into slots p mod W[h] of kw, vw ([B][H][w_cap][d]).
struct RingFillArgs {
    const void* k;
    const void* v;
    void* kw;
    void* vw;
    int B, T, H, d, w_cap;
    int W[kAttnMaxHeads];
};
hipError_t launch_ring_fill(const RingFillArgs& a, bool bf16, hipStream_t stream);

// Decode caches from a prefill's states: state (b, p, h) of [B][T][H][d]
// into row (p mod D[h]) (n_cap / D[h]) + p / D[h] of head (b, h)'s history
// [B][H][n_cap][d]; raw k, v of the last W[h] positions into ring slot
// p mod W[h] of [B][H][w_cap][d].
struct CacheArgs {
    const void* ks;
    const void* vs;
    const void* k;
    const void* v;
    void* kc;
    void* vc;
    void* kw;
    void* vw;
    int B, T, H, d, n_cap, w_cap;
    int D[kAttnMaxHeads];
    int W[kAttnMaxHeads];
};
hipError_t launch_cache_build(const CacheArgs& a, bool bf16, hipStream_t stream);

// ---------------------------------------------------------------- backward
constexpr int kBwdChunk = 16;  // tokens per chunk of the reverse recurrence
#ifndef RAT_BWD_WAVES
#define RAT_BWD_WAVES 4
#endif
constexpr int kBwdWaves = RAT_BWD_WAVES;  // waves of an MFMA backward workgroup (16 owned rows each)

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* g;     // gate logits
    const void* ks;
    const void* vs;    // forward states
    const void* dout;  // [B][T][H][d] in the layer's dtype
    float* dq;
    float* dk;
    float* dv;
    float* dg;         // [B][T][H][d] fp32 gradients
    float* lse;
    float* delta;      // [B][T][H] per query row
    float* dks;
    float* dvs;        // [B][T][H][d] gradients of the states
    float* maps;       // [nchunk][B][H d][5] per-chunk maps
    float* carry;      // [nchunk][B][H d][4] state before / carry into each chunk
    float* bstat;      // [B][T][H][3] per query row: (max, sum, sum p dp) over its raw window
    int B, T, H, d;
    int L;             // RESTART period, 0 for the full recurrence
    int nchunk;        // ceil(T / kBwdChunk)
    float scale;
    int mfma;          // bf16: every head runs on the MFMA kernels (fp32: the per-row kernels)
    int raw;           // dk / dv hold raw-window gradients before the recurrence adds its own:
                       // some head has a window (bf16), always (fp32)
    int sliding;       // SLIDING window L < T: each state its own window (L is then the window)
    int D[kAttnMaxHeads];
    int W[kAttnMaxHeads];
    int mitem[kAttnMaxHeads + 1];  // first MFMA work item of each head; [H] = total
};
hipError_t launch_backward(const BwdArgs& a, bool bf16, hipStream_t stream);

// Kernel-argument layouts, asserted in both the host and the device
// compilation (a struct laid out differently by the two would hand the
// kernels shifted fields), and within the 4 KiB kernel-argument segment.
static_assert(sizeof(StateHist) == 1036, "StateHist layout");
static_assert(sizeof(ScanFullArgs) == 1144 && offsetof(ScanFullArgs, fin) == 96 &&
              offsetof(ScanFullArgs, hist) == 108, "ScanFullArgs layout");
static_assert(sizeof(ScanSlideArgs) == 1096 && offsetof(ScanSlideArgs, hist) == 60, "ScanSlideArgs layout");
static_assert(sizeof(AttnArgs) == 1344 && offsetof(AttnArgs, cls) == 92 && offsetof(AttnArgs, heads) == 316,
              "AttnArgs layout");
static_assert(sizeof(RingFillArgs) == 1080 && sizeof(DecodeArgs) == 3160 && sizeof(StepArgs) == 2136 &&
              sizeof(CacheArgs) == 2136 && sizeof(BwdArgs) == 3264 && sizeof(AttnF32Args) == 2128 &&
              sizeof(SlideStepArgs) == 2160 && sizeof(SlideFillArgs) == 72, "kernel-argument sizes");
static_assert(sizeof(BwdArgs) < 4096 && sizeof(DecodeArgs) < 4096, "kernel arguments fit their segment");

}  // namespace rat
