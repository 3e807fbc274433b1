// Stage 2 of the RAT+ layer for prefill: causal dilated softmax attention
// over the recurrent states, optionally joined by a window of raw tokens,
// with a per-head (D, W) ("RAT+: Train Dense, Infer Sparse", arXiv
// 2602.18196, Abstract; "RAT+ Deep Dive", zhichai.net, section 1 (tokens
// skip a fixed interval D) and section 6 (Head-Wise Hybrid)).
//
// Query t of head h sees the states at t, t-D, t-2D, ... (>= 0) and the raw
// tokens t, t-1, ..., t-W+1 (>= 0), in one softmax.  Queries of one residue
// r = t mod D share their state keys: residue r is a dense causal problem
// of length M_r = ceil((T - r) / D) over q[r::D], states[r::D].  The raw
// window is a band over contiguous positions instead.
//
// bf16 MFMA (v_mfma_f32_16x16x32_bf16) with fp32 accumulation and an fp32
// online softmax in the log2 domain.  Per 16-query fragment a wave computes
// S^T = K Q^T (keys x queries), so each lane owns one query: the softmax
// statistics and the output O^T = V^T P^T stay per lane and P^T is the MFMA
// B operand exactly as S^T leaves the accumulator.  V^T comes from a
// row-major V tile in LDS through ds_read_b64_tr_b16.  LDS tiles are
// XOR-swizzled in 16-byte chunks so that both the K-fragment reads and the
// transposing V reads avoid bank conflicts, and are filled by direct
// global->LDS loads.
//
// Path A (every head, including dense D = 1): work items are
// (b, h, r, chunk of rows of residue r).  Persistent workgroups take items
// in rounds over the cost-sorted item list, in one of two shapes: eight
// waves over 256-row chunks on a four- or five-slot LDS ring (one workgroup
// per CU; launches with residues longer than 1024 rows), or four waves over
// 128-row chunks on a two-slot ring (two per CU).  Each wave owns two 16-row
// blocks (w and 2 NW - 1 - w, which balances the causal work) so that every
// K/V fragment read from LDS feeds two MFMA row blocks.  K/V tiles of 64
// keys stream through the ring, whose prefetch runs on into the next item,
// so every state row is read from HBM once per chunk.
//
// Local window (heads with W > 0): the raw-key band runs first, over
// contiguous queries (where the band is dense), in a kernel that leaves a
// partial softmax state per query -- normalised output in `out`, (m, l) in
// a small workspace; path A then starts each query's online softmax from
// that state and continues over the dilated states, so both branches share
// one softmax and each runs on full 16-row MFMA fragments.
#include "rat_device.h"
#include "rat_internal.h"
#include "rat_mfma.h"
#include "rat_plan.h"

namespace rat {


// max of three scores: IEEE maximum (NaN-propagating), which gfx950 issues
// as one v_maximum3_f32 with no quieting of its operands.  Written as a
// builtin rather than asm so that the compiler sees the operation and
// needs no hazard padding around it.
__device__ __forceinline__ float max3(float a, float b, float c)
{
    return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// max over the four lanes l, l^16, l^32, l^48 (the four 16-lane rows) with
// the gfx950 row-swap permutes (VALU only, no LDS traffic)
__device__ __forceinline__ float max_over_rows(float x)
{
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = max3(__uint_as_float(a[0]), __uint_as_float(a[1]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return max3(__uint_as_float(b[0]), __uint_as_float(b[1]), __uint_as_float(b[1]));
}

// Online-softmax state of one 16-query fragment (lane (g, i) owns query i;
// m is replicated over the four lane groups, l is this lane's partial sum).
template <int DK>
struct Frag {
    bf16x8 q[Geo<DK>::KS];
    floatx4 acc[Geo<DK>::DB];
    float m, l;

    __device__ __forceinline__ void reset()
    {
#pragma unroll
        for (int i = 0; i < Geo<DK>::DB; ++i) acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
        m = -INFINITY;
        l = 0.f;
    }

    // Q fragment (B operand): lane (g, i) holds q[row i][dims 8g + 32ks .. +8]
    __device__ __forceinline__ void load_q(const uint16_t* row_ptr, bool valid)
    {
        const int g = (threadIdx.x & (kWave - 1)) >> 4;
#pragma unroll
        for (int ks = 0; ks < Geo<DK>::KS; ++ks) {
            if (valid)
                q[ks] = *reinterpret_cast<const bf16x8*>(row_ptr + 8 * g + 32 * ks);
            else
                q[ks] = bf16x8{};
        }
    }

    // Start from a partial softmax state over other keys of the same
    // queries: its running max m (log2 domain), its sum l and its
    // normalised output o (acc = o * l).  `rows` is the first of the
    // block's 16 rows of o in a swizzled LDS slot, `ml` its (m, l) pairs.
    // Lane (g, i) of query i takes dims 16db + 4g .. +3; only lane group 0
    // carries l.
    __device__ __forceinline__ void init_partial_lds(const lds_char* rows, const float* ml, bool valid)
    {
        if (!valid) return;
        const int lane = threadIdx.x & (kWave - 1);
        const int g = lane >> 4, i = lane & 15;
        const float pm = ml[2 * i], pl = ml[2 * i + 1];
        m = pm;
        l = g == 0 ? pl : 0.f;
#pragma unroll
        for (int db = 0; db < Geo<DK>::DB; ++db) {
            const int dim = 16 * db + 4 * g;
            const u32x2 o = *reinterpret_cast<const u32x2*>(rows + swz<DK>(i, dim >> 3) + (dim & 7) * 2);
            acc[db] = floatx4{bf16_lo(o[0]) * pl, bf16_hi(o[0]) * pl, bf16_lo(o[1]) * pl, bf16_hi(o[1]) * pl};
        }
    }

    // Chunk grid: the softmax starts from the query's own state.  krow /
    // vrow: the block's first row in the K / V half of an own-state slot
    // (query i's own key and value at row i of the block); koff0: the
    // lane's K-fragment offset of k-step 0.  Score in the log2 domain.
    __device__ __forceinline__ void init_own_lds(const lds_char* krow, int koff0, const lds_char* vrow, float c)
    {
        const int lane = threadIdx.x & (kWave - 1);
        const int g = lane >> 4, i = lane & 15;
        float dot = 0.f;
#pragma unroll
        for (int ks = 0; ks < Geo<DK>::KS; ++ks) {
            const bf16x8 kf = *reinterpret_cast<const bf16x8*>(krow + (koff0 ^ (ks << 6)));
#pragma unroll
            for (int e = 0; e < 4; ++e)
                dot = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{q[ks][2 * e], q[ks][2 * e + 1]},
                                                      bf16x2{kf[2 * e], kf[2 * e + 1]}, dot, false);
        }
        // the four lane groups hold the dims of one query: sum them
        auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(dot), __float_as_uint(dot), false, false);
        dot = __uint_as_float(a[0]) + __uint_as_float(a[1]);
        auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(dot), __float_as_uint(dot), false, false);
        dot = __uint_as_float(b[0]) + __uint_as_float(b[1]);
        m = dot * c;
        l = g == 0 ? 1.f : 0.f;
#pragma unroll
        for (int db = 0; db < Geo<DK>::DB; ++db) {
            const int dim = 16 * db + 4 * g;
            const u32x2 o = *reinterpret_cast<const u32x2*>(vrow + swz<DK>(i, dim >> 3) + (dim & 7) * 2);
            acc[db] = floatx4{bf16_lo(o[0]), bf16_hi(o[0]), bf16_lo(o[1]), bf16_hi(o[1])};
        }
    }

    __device__ __forceinline__ float total_l() const
    {
        float t = l + __shfl_xor(l, 16);
        return t + __shfl_xor(t, 32);
    }

    // O row of query i: lane (g, i) stores dims 16db + 4g .. +3
    __device__ __forceinline__ void store(uint16_t* row_ptr, bool valid) const
    {
        const float lt = total_l();
        if (!valid) return;
        const float inv = 1.0f / lt;
        const int g = (threadIdx.x & (kWave - 1)) >> 4;
#pragma unroll
        for (int db = 0; db < Geo<DK>::DB; ++db) {
            u32x2 o;
            o[0] = pack_bf16x2(acc[db][0] * inv, acc[db][1] * inv);
            o[1] = pack_bf16x2(acc[db][2] * inv, acc[db][3] * inv);
            *reinterpret_cast<u32x2*>(row_ptr + 16 * db + 4 * g) = o;
        }
    }

    // Partial state for a later pass: normalised o in bf16 and (m, l)
    __device__ __forceinline__ void store_partial(uint16_t* o_row, float* ml, bool valid) const
    {
        const float lt = total_l();
        store(o_row, valid);
        if (valid && (threadIdx.x & (kWave - 1)) < 16) {
            ml[0] = m;
            ml[1] = lt;
        }
    }
};

// ------------------------------------------------------------------ path A
// (items, the cursor over ring steps and the copies' addresses: rat_plan.h)

// Source tensors of the ring DMA, held in scalar registers for the whole
// kernel and handed to the issue as values (a selection among kernel
// argument fields, or among fields of a struct in memory, inside the loop
// becomes a memory load of the selected field on every step).
struct DmaSrc {
    uint64_t q, out, kv;  // kv: this wave's half of a key tile (K or V rows)
};

template <int NW, bool BAND>
__device__ __forceinline__ DmaSrc dma_sources(const AttnArgs& a, int wv)
{
    uint64_t q = (uint64_t)(uintptr_t)a.q, out = (uint64_t)(uintptr_t)a.out;
    uint64_t k = (uint64_t)(uintptr_t)(BAND ? a.kr : a.ks), v = (uint64_t)(uintptr_t)(BAND ? a.vr : a.vs);
    asm volatile("" : "+s"(q), "+s"(out), "+s"(k), "+s"(v));
    uint64_t kv = wv >= NW / 2 ? v : k;
    asm volatile("" : "+s"(kv));
    return DmaSrc{q, out, kv};
}

// Per-lane constants of the ring DMA (dma_lane_a)
template <int DK>
struct DmaLane {
    uint32_t lq, col16;
    __device__ __forceinline__ void init() { dma_lane_a<DK>((int)(threadIdx.x & (kWave - 1)), lq, col16); }
};

// DMA of the cursor's ring step into slot `buf`: the wave's copies as
// step_copies_a / step_lane_offset_a form them, and for partial-output
// steps the (m, l) words into `side` on waves 0-3 (step_side_word_a).
// When the step is a whole key tile, its plan and lane offsets go to
// `run` / `run_voff` for the key tiles that follow, and it returns true.
template <int DK, int NW, bool BAND, bool CHUNK, bool HIST>
__device__ __forceinline__ bool issue_step_a(const AttnArgs& a, const CursorA<BAND, CHUNK, HIST>& c, uint64_t src_q,
                                             uint64_t src_out, uint64_t src_kv, const DmaLane<DK>& dl, uint32_t buf,
                                             uint32_t side, KeyRunA& run,
                                             uint32_t (&run_voff)[StepCopiesA<DK, NW>::PER_WAVE])
{
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x & (kWave - 1);
    StepCopiesA<DK, NW> sc;
    step_copies_a<DK, NW>(a, c, wv, buf, sc);
    // (the source as step_copies_a picks it, selected here from the cursor
    // itself so that the choice stays in scalar registers)
    const int ko = c.t - c.nq - c.no;
    const uint64_t tsrc = ko < 0 ? (c.t < c.nq ? src_q : src_out) : src_kv;
    // m0[j] = m0[0] + 1024 j: one M0, the copy's immediate offset supplies the rest
    constexpr int PW = StepCopiesA<DK, NW>::PER_WAVE;
    uint64_t base[PW];
    uint32_t voff[PW];
#pragma unroll
    for (int j = 0; j < PW; ++j) base[j] = tsrc + sc.rel[j] - 1024u * (j % 4);
    bool keys = false;
    if (sc.whole) {  // (uniform: the common case computes only its own lane offsets)
#pragma unroll
        for (int j = 0; j < PW; ++j) voff[j] = step_lane_offset_whole_a<DK, NW>(sc, wv, j, dl.lq, dl.col16);
        if (step_key_tile_a(c) >= 0) {
            run = KeyRunA{sc.rel[0], sc.dp2, sc.row0, sc.last};
#pragma unroll
            for (int j = 0; j < PW; ++j) run_voff[j] = voff[j];
            keys = true;
        }
    } else {
#pragma unroll
        for (int j = 0; j < PW; ++j) voff[j] = step_lane_offset_clamped_a<DK, NW>(sc, wv, j, dl.lq, dl.col16);
    }
    dma16_group<PW>(base, voff, sc.m0[0]);
    const int64_t side_word = step_side_word_a(a, c, wv, lane);
    if (side_word >= 0) {
        const float* p = a.ml + side_word;
        asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(p), "{m0}"(side + wv * 256) : "memory");
    }
    return keys;
}

// DMA of the next key tile of a run (key_run_next_a has moved `run` to it):
// the copy bases one add apart, the lane offsets those of the run's first tile.
template <int DK, int NW>
__device__ __forceinline__ void issue_key_run_a(const KeyRunA& run, const uint32_t (&voff)[StepCopiesA<DK, NW>::PER_WAVE],
                                                uint64_t src_kv, uint32_t buf)
{
    constexpr int PW = StepCopiesA<DK, NW>::PER_WAVE;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    // copy j at src + key_run_rel_a(run, j), lowered by 1024 (j mod 4) for
    // its immediate offset
    const uint64_t step = (uint64_t)Geo<DK>::RPI * run.dp2;
    uint64_t base[PW];
    base[0] = src_kv + run.rel0;
#pragma unroll
    for (int j = 1; j < PW; ++j) base[j] = base[j - 1] + step + (j % 4 ? (uint64_t)0 - 1024u : (uint64_t)3072);
    dma16_group<PW>(base, voff, buf + wv * PW * 1024);
}

// Per-lane byte offsets inside a swizzled tile: K fragment of k-step ks for
// key block 0 (key block kb adds kb * 16 rows), and the first transposing V
// read of 16-dim block db for key half 0 (half hh adds 32 rows, the second
// read 16 rows).  Only the offsets of ks = 0 and db = 0 are kept: the
// fragment index enters the swizzled chunk as a plain XOR (chunk g + 4 ks
// = g | 4 ks, and chunk 2 db + c = 2 db | c, while the XOR key of the row
// touches neither bit range), which also leaves the row and in-chunk bits
// of the offset alone.  Two registers instead of KS + DB.
template <int DK>
struct LaneOffsets {
    int k0, v0;

    __device__ __forceinline__ void init()
    {
        const int lane = threadIdx.x & (kWave - 1);
        const int g = lane >> 4, i = lane & 15, s = lane & 15;
        k0 = swz<DK>(i, g);
        const int r0 = 4 * g + (s >> 2);
        const int dim = 4 * (s & 3);
        v0 = swz<DK>(r0, dim >> 3) + (dim & 7) * 2;
    }
    // The per-fragment offsets are recomputed at every use (one XOR each):
    // an empty asm hides the base so that the compiler neither hoists the
    // KS + DB values out of the tile loop nor spills them there.
    __device__ __forceinline__ int kbase() const
    {
        int x = k0;
        asm volatile("" : "+v"(x));
        return x;
    }
    __device__ __forceinline__ int vbase() const
    {
        int x = v0;
        asm volatile("" : "+v"(x));
        return x;
    }
};


// Online softmax over one 64-key tile for one 16-row block.  Scores s[kb]
// hold keys 16kb + 4g + j of the lane's query (raw q.k).  The running max
// m (log2 domain) is only raised -- with the rescale of acc and l -- when
// some query's tile max exceeds it by more than kLazyRescale; otherwise the
// stale max stays the exponent reference (weights up to 2^kLazyRescale, the
// result is the same softmax).  Returns P^T operands for the two key halves.
constexpr float kLazyRescale = 8.0f;

// MASK: only keys in [lo, row] are visible to the lane's query.
template <int DK, bool MASK>
__device__ __forceinline__ void softmax64(Frag<DK>& f, floatx4 (&s)[4], int row, int lo, int k0, float c,
                                          bf16x8 (&pb)[2])
{
    const int g = (threadIdx.x & (kWave - 1)) >> 4;
    if (MASK) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int key = k0 + 16 * kb + 4 * g + j;
                if (key > row || key < lo) s[kb][j] = -INFINITY;
            }
    }
    float mx = max3(s[0][0], s[0][1], s[0][2]);
    mx = max3(mx, s[0][3], s[1][0]);
    mx = max3(mx, s[1][1], s[1][2]);
    mx = max3(mx, s[1][3], s[2][0]);
    mx = max3(mx, s[2][1], s[2][2]);
    mx = max3(mx, s[2][3], s[3][0]);
    mx = max3(mx, s[3][1], s[3][2]);
    mx = max3(mx, s[3][3], s[3][3]);
    mx = max_over_rows(mx) * c;
    if (__builtin_amdgcn_ballot_w64(mx > f.m + kLazyRescale)) {
        const float mn = fmaxf(f.m, mx);
        const float alpha = __builtin_amdgcn_exp2f(f.m - (mn == -INFINITY ? 0.f : mn));
        f.l *= alpha;
#pragma unroll
        for (int db = 0; db < Geo<DK>::DB; ++db) f.acc[db] *= alpha;
        f.m = mn;
    }
    const float nm = f.m == -INFINITY ? 0.f : -f.m;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            pb[hh][j] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[2 * hh][j], c, nm));
            pb[hh][4 + j] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[2 * hh + 1][j], c, nm));
        }
    }
    // the denominator sums the same bf16-rounded weights that multiply V
    // (one v_dot2 with (1, 1) per weight pair, exact products, fp32 sums)
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        s0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[0][2 * q], pb[0][2 * q + 1]}, one, s0, false);
        s1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[1][2 * q], pb[1][2 * q + 1]}, one, s1, false);
    }
    f.l += s0 + s1;
}

template <int BITS>
struct Mask {
    static constexpr int value = BITS;
};

// NW waves per workgroup, two row blocks of 16 queries per wave: block w
// and its mirror 2 NW - 1 - w, so that every wave has the same causal work.
// Every K / V fragment read from LDS feeds both blocks' MFMAs.
template <int NW>
__device__ __forceinline__ int row_block(int wv, int j)
{
    return j == 0 ? wv : 2 * NW - 1 - wv;
}

// CHUNK: the chunk grid (keys of residue D - 1 strictly before the query,
// the softmax started from the query's own state).  HIST: the states are a
// per-residue history ([B][H][n_cap][d], a residue's rows contiguous).
// Items of 32 NW query rows.  Eight waves run one workgroup per CU on a
// deep ring; four waves on a two-slot ring run two workgroups per CU.
template <int DK, int NW, int RING, bool BAND, bool CHUNK, bool HIST>
__global__ __launch_bounds__(NW * kWave, NW == 4 ? 2 : 1) void attn_dilated_kernel(AttnArgs a)
{
    typedef Geo<DK> G;
    constexpr int NB = 2;  // row blocks per wave
    static_assert(NW == 4 || NW == 8, "four or eight waves");
    constexpr int TILE_BYTES = kSlotRows * G::ROWB;
    constexpr int PER_WAVE = (kSlotRows / G::RPI) / NW;
    static_assert((kSlotRows / G::RPI) % NW == 0, "slot loads split evenly over waves");
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    // (m, l) words of partial-output slots, 1 KiB each; a ring of more than
    // four slots is only used without windowed classes and has no side buffers
    lds_char* side = smem + (RING > 4 ? 0 : RING * TILE_BYTES);

    const int lane = threadIdx.x & (kWave - 1);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int i = lane & 15;
    // keys strictly before the query (chunk grid) or up to it
    constexpr int sh = CHUNK ? 1 : 0;

    LaneOffsets<DK> off;
    off.init();
    DmaLane<DK> dl;
    dl.init();
    const DmaSrc dsrc = dma_sources<NW, BAND>(a, wv);
    CursorA<BAND, CHUNK, HIST> issue, comp;
    issue.seek(a, 0, gridDim.x, blockIdx.x);
    comp = issue;
    // ring steps issued and consumed; step n lives in slot n mod RING (a
    // wrapping slot counter instead raises the register use of the band
    // kernel past the point where it spills)
    int issued = 0, consumed = 0;
    const uint32_t smem_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)smem);
    const uint32_t side_lds = smem_lds + (uint32_t)(side - smem);
    // the key tile last issued, when it was whole (key_run_next_a)
    KeyRunA run{};
    bool run_ok = false;
    uint32_t run_voff[PER_WAVE];
    auto issue_next = [&]() {
        const int sl = issued % RING;
        if (run_ok && key_run_next_a<DK, NW>(issue, run))
            issue_key_run_a<DK, NW>(run, run_voff, dsrc.kv, smem_lds + sl * TILE_BYTES);
        else
            run_ok = issue_step_a<DK, NW, BAND, CHUNK, HIST>(a, issue, dsrc.q, dsrc.out, dsrc.kv, dl,
                                                             smem_lds + sl * TILE_BYTES, side_lds + sl * 1024, run,
                                                             run_voff);
        ++issued;
        issue.advance(a, gridDim.x, blockIdx.x);
    };
    auto consume = [&]() { ++consumed; };
#pragma unroll
    for (int j = 0; j < RING - 1; ++j)
        if (issue.it.valid) issue_next();
    // Wait until ring step `consumed + d` has landed, then barrier; refill
    // the ring when a slot is free (the oldest step still read after this
    // barrier is `consumed`).
    auto wait_tile = [&](int d) {
        const int ahead = issued - consumed - d - 1;  // ring steps issued after the awaited one
        if (RING > 4 && ahead >= 3) wait_vmcnt<3 * PER_WAVE>();
        else if (ahead >= 2) wait_vmcnt<2 * PER_WAVE>();
        else if (ahead == 1) wait_vmcnt<PER_WAVE>();
        else wait_vmcnt<0>();
        __syncthreads();
        if (issue.it.valid && issued < consumed + RING) issue_next();
    };

    Frag<DK> f[NB];
    while (comp.it.valid) {
        const ItemA it = comp.it;
        int rs[NB];    // first row of each block
        bool has[NB];  // block holds rows of the item
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            rs[j] = it.R0 + 16 * row_block<NW>(wv, j);
            has[j] = rs[j] < it.R1;
            f[j].reset();
#pragma unroll
            for (int ks = 0; ks < G::KS; ++ks) f[j].q[ks] = bf16x8{};
        }
        // query rows from the ring (lane (g, i): row i, dims 8g + 32ks .. +8)
        for (int s = 0; s < comp.nq; ++s) {
            wait_tile(0);
            const lds_char* qt = smem + (consumed % RING) * TILE_BYTES;
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int r = 16 * row_block<NW>(wv, j);
                if (r / kSlotRows == s) {
#pragma unroll
                    for (int ks = 0; ks < G::KS; ++ks) f[j].q[ks] = lds_b128(qt + (r % kSlotRows) * G::ROWB + (off.k0 ^ (ks << 6)));
                }
            }
            consume();
        }
        // windowed classes: continue from the band pass's partial state
        for (int s = 0; s < comp.no; ++s) {
            wait_tile(0);
            const lds_char* ot = smem + (consumed % RING) * TILE_BYTES;
            const float* ml = reinterpret_cast<const float*>(side + (consumed % RING) * 1024);
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int r = 16 * row_block<NW>(wv, j);
                if (r / kSlotRows == s)
                    f[j].init_partial_lds(ot + (r % kSlotRows) * G::ROWB, ml + (r % kSlotRows) * 2, rs[j] + i < it.R1);
            }
            consume();
        }
        // chunk grid: each query's softmax starts from its own state (64
        // query rows per ring step)
        for (int u = 0; CHUNK && u < comp.nown; ++u) {
            wait_tile(0);
            const lds_char* sl = smem + (consumed % RING) * TILE_BYTES;
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int r = 16 * row_block<NW>(wv, j);
                if (r / kTileA == u)
                    f[j].init_own_lds(sl + (r % kTileA) * G::ROWB, off.k0, sl + (kTileA + r % kTileA) * G::ROWB,
                                      a.scale_log2);
            }
            consume();
        }

        // k-steps outermost: 4 x NB independent accumulation chains sit
        // between two MFMAs of the same chain, so no MFMA waits for the
        // result of the one before it
        // `act` (a Mask<bits>): the row blocks whose MFMAs run
        auto qk = [&](auto act, int sl, floatx4 (&sc)[NB][4]) {
            constexpr int ACT = decltype(act)::value;
            const lds_char* kt = smem + sl * TILE_BYTES;
            const int kb0 = off.kbase();
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    if ((ACT >> j) & 1) sc[j][kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < G::KS; ++ks) {
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    const bf16x8 kf = lds_b128(kt + (kb0 ^ (ks << 6)) + kb * 16 * G::ROWB);
#pragma unroll
                    for (int j = 0; j < NB; ++j)
                        if ((ACT >> j) & 1) sc[j][kb] = mfma16(kf, f[j].q[ks], sc[j][kb]);
                }
            }
        };
        auto pv = [&](auto act, int sl, const bf16x8 (&pb)[NB][2]) {
            constexpr int ACT = decltype(act)::value;
            const lds_char* vt = smem + sl * TILE_BYTES + kTileA * G::ROWB;
            const int vb0 = off.vbase();
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
                for (int db = 0; db < G::DB; ++db) {
                    const lds_char* vp = vt + (vb0 ^ (db << 5)) + hh * 32 * G::ROWB;
                    const shortx4 x0 = lds_tr(vp);
                    const shortx4 x1 = lds_tr(vp + 16 * G::ROWB);
                    typedef short shortx8 __attribute__((ext_vector_type(8)));
                    const shortx8 v8 = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
                    const bf16x8 vf = __builtin_bit_cast(bf16x8, v8);
#pragma unroll
                    for (int j = 0; j < NB; ++j)
                        if ((ACT >> j) & 1) f[j].acc[db] = mfma16(vf, pb[j][hh], f[j].acc[db]);
                }
            }
        };
        constexpr Mask<(1 << NB) - 1> all;

        floatx4 sc[NB][4];
        int tt = 0;
        // Tiles wholly below the chunk's first row are visible to every row
        // of the chunk and need no mask.  With two blocks per wave they run
        // software-pipelined (the QK^T MFMAs of tile t+1 are issued before
        // the softmax of tile t); four blocks have no registers for a
        // second set of scores and rely on the MFMAs of one block running
        // while the softmax of another is computed.
        const int nfull = BAND ? 0 : min(it.R0 / kTileA, comp.ntile - 1);
        bool have_scores = false;
        if constexpr (!BAND && RING >= 3) {  // (the pipelined tiles keep two slots busy)
            if (nfull > 0) {
                wait_tile(0);
                qk(all, consumed % RING, sc);
                for (; tt < nfull; ++tt) {
                    wait_tile(1);  // the current tile still feeds P V
                    floatx4 nx[NB][4];
                    qk(all, (consumed + 1) % RING, nx);
                    bf16x8 pb[NB][2];
#pragma unroll
                    for (int j = 0; j < NB; ++j) softmax64<DK, false>(f[j], sc[j], 0, 0, 0, a.scale_log2, pb[j]);
                    pv(all, consumed % RING, pb);
                    consume();
#pragma unroll
                    for (int j = 0; j < NB; ++j)
#pragma unroll
                        for (int kb = 0; kb < 4; ++kb) sc[j][kb] = nx[j][kb];
                }
                have_scores = true;  // tile nfull's scores are in sc
            }
        }
        for (; tt < comp.ntile; ++tt) {
            const int k0 = it.kbeg + tt * kTileA;
            // a wave whose blocks see no key of the tile skips it: causal
            // rows rs .. rs+15 see keys up to rs+15, a band item's rows only
            // from rs-W+1
            bool skip = true;
#pragma unroll
            for (int j = 0; j < NB; ++j)
                skip &= !(has[j] && k0 <= rs[j] + 15 - sh && (!BAND || k0 + kTileA - 1 >= rs[j] - it.W + 1));
            if (!have_scores) {
                wait_tile(0);
                if (!skip) qk(all, consumed % RING, sc);
            }
            have_scores = false;
            if (skip) {  // (the wave still keeps the ring in step)
                consume();
                continue;
            }
            bf16x8 pb[NB][2];
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                pb[j][0] = bf16x8{};
                pb[j][1] = bf16x8{};
                if (BAND) {
                    if (has[j] && k0 <= rs[j] + 15 && k0 + kTileA - 1 >= rs[j] - it.W + 1) {
                        // a tile inside every row's band needs no mask
                        if (k0 >= rs[j] + 16 - it.W && k0 + kTileA - 1 <= rs[j])
                            softmax64<DK, false>(f[j], sc[j], 0, 0, 0, a.scale_log2, pb[j]);
                        else
                            softmax64<DK, true>(f[j], sc[j], rs[j] + i, rs[j] + i - it.W + 1, k0, a.scale_log2, pb[j]);
                    }
                } else if (has[j] && k0 <= rs[j] + 15 - sh) {
                    // key row j is visible to query row i when j <= i - sh
                    if (k0 + kTileA - 1 <= rs[j] - sh) softmax64<DK, false>(f[j], sc[j], 0, 0, 0, a.scale_log2, pb[j]);
                    else softmax64<DK, true>(f[j], sc[j], rs[j] + i - sh, 0, k0, a.scale_log2, pb[j]);
                }
            }
            pv(all, consumed % RING, pb);
            consume();
        }
        uint16_t* const out16 = static_cast<uint16_t*>(a.out);
        const size_t orow0 = item_out_row0(a, it);
        if (BAND) {  // partial state for the dilated pass: o in `out`, (m, l) in the workspace
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const size_t orow = item_out_row(a, it, orow0, rs[j] + i);
                f[j].store_partial(out16 + orow * DK, a.ml + orow * 2, rs[j] + i < it.R1);
            }
        } else {
#pragma unroll
            for (int j = 0; j < NB; ++j) f[j].store(out16 + item_out_row(a, it, orow0, rs[j] + i) * DK, rs[j] + i < it.R1);
        }
        comp.seek(a, comp.round + 1, gridDim.x, blockIdx.x);
    }
}

// ------------------------------------------------------------------ band pass
// Local window of raw keys for heads with W > 0 runs through the same
// persistent kernel with BAND = true: an item is 256 contiguous queries of
// one (b, h) and the key tiles cover [t0-W+1, t0+255]; waves skip the tiles
// that neither of their blocks sees, and the item ends with a partial
// softmax state per query -- the normalised output in `out` and (m, l) in
// the workspace -- from which the dilated pass continues.

// ring slots plus the (m, l) side buffers of path A
size_t attn_lds_bytes_a(int d, int ring) { return (size_t)ring * (2 * kTileA * d * 2 + 1024); }
// five slots, no side buffers (no windowed classes): 160 KiB at d = 128
size_t attn_lds_bytes_a5(int d) { return (size_t)5 * 2 * kTileA * d * 2; }

template <typename K>
static void set_lds(K kernel, size_t lds, bool& done)
{
    if (!done) {
        (void)hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        done = true;
    }
}

template <int DK, int NW, int RING, bool BAND, bool CHUNK, bool HIST>
static hipError_t launch_a(const AttnArgs& a, int grid, size_t lds, hipStream_t stream)
{
    static bool done = false;
    set_lds(attn_dilated_kernel<DK, NW, RING, BAND, CHUNK, HIST>, lds, done);
    hipLaunchKernelGGL((attn_dilated_kernel<DK, NW, RING, BAND, CHUNK, HIST>), dim3(grid), dim3(NW * kWave), lds,
                       stream, a);
    return hipGetLastError();
}

// The kernel shape follows the plan's rows per item: 256 -> eight waves,
// five slots (four and the (m, l) buffers when a class is windowed); 128 ->
// four waves, two slots with the buffers.
template <bool BAND, bool CHUNK, bool HIST>
static hipError_t launch_path_a(const AttnArgs& a, int d, int grid, bool windowed, hipStream_t stream)
{
    if (a.rows == kAttnRowsShort) {
        const size_t lds = attn_lds_bytes_a(d, 2);
        return d == 128 ? launch_a<128, 4, 2, BAND, CHUNK, HIST>(a, grid, lds, stream)
                        : launch_a<64, 4, 2, BAND, CHUNK, HIST>(a, grid, lds, stream);
    }
    if (a.rows != kAttnRowsLong) return hipErrorInvalidValue;
    if (!windowed) {
        const size_t lds = attn_lds_bytes_a5(d);
        return d == 128 ? launch_a<128, 8, 5, BAND, CHUNK, HIST>(a, grid, lds, stream)
                        : launch_a<64, 8, 5, BAND, CHUNK, HIST>(a, grid, lds, stream);
    }
    if constexpr (CHUNK || BAND) {
        return hipErrorInvalidValue;  // the chunk grid has no windowed classes; the band runs on four waves
    } else {
        const size_t lds = attn_lds_bytes_a(d, kRingA);
        return d == 128 ? launch_a<128, 8, kRingA, false, false, HIST>(a, grid, lds, stream)
                        : launch_a<64, 8, kRingA, false, false, HIST>(a, grid, lds, stream);
    }
}

hipError_t launch_attn_dilated_bf16(const AttnArgs& a, int d, int grid, hipStream_t stream)
{
    bool windowed = false;
    for (int c = 0; c < a.nclass; ++c) windowed |= a.cls[c].W > 0;
    if (a.chunk) return launch_path_a<false, true, false>(a, d, grid, false, stream);  // no windowed classes
    if (a.n_cap > 0) return launch_path_a<false, false, true>(a, d, grid, windowed, stream);
    return launch_path_a<false, false, false>(a, d, grid, windowed, stream);
}

hipError_t launch_attn_band_bf16(const AttnArgs& a, int d, int grid, hipStream_t stream)
{
    return launch_path_a<true, false, false>(a, d, grid, false, stream);
}

// ------------------------------------------------------------------ fp32
// One workgroup (one wave) per query row; lanes split the head dimension.
// Exact fp32 FMA dot products and expf; meant for small fp32 problems.
__global__ __launch_bounds__(kWave) void attn_prefill_f32_kernel(AttnF32Args a)
{
    const int lane = threadIdx.x;
    const int t = blockIdx.x % a.T;
    const int bh = blockIdx.x / a.T;
    const int h = bh % a.H, b = bh / a.H;
    const int d = a.d, D = a.D[h], W = a.W[h];
    const size_t pitch = (size_t)a.H * d;
    const size_t base = ((size_t)b * a.T * a.H + h) * d;
    const float q0 = lane < d ? a.q[base + t * pitch + lane] : 0.f;
    const float q1 = lane + kWave < d ? a.q[base + t * pitch + lane + kWave] : 0.f;
    float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
    // row s of a state tensor: [B][T][H][d], or a per-residue history
    const size_t hbase = (size_t)bh * a.n_cap * d;
    const int mcap = a.n_cap > 0 ? a.n_cap / D : 0;
    auto srow = [&](int s) -> size_t { return a.n_cap > 0 ? hbase + (size_t)((s % D) * mcap + s / D) * d : base + s * pitch; };
    auto visit = [&](const float* kbase, const float* vbase, size_t row) {
        const float* kr = kbase + row;
        float dot = (lane < d ? q0 * kr[lane] : 0.f) + (lane + kWave < d ? q1 * kr[lane + kWave] : 0.f);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) dot += __shfl_xor(dot, o);
        const float z = dot * a.scale;
        const float mn = fmaxf(m, z);
        const float al = expf(m - mn), p = expf(z - mn);
        const float* vr = vbase + row;
        o0 = o0 * al + p * (lane < d ? vr[lane] : 0.f);
        o1 = o1 * al + p * (lane + kWave < d ? vr[lane + kWave] : 0.f);
        l = l * al + p;
        m = mn;
    };
    if (a.chunk) {  // chunk-end states before t, then the own state
        for (int s = D - 1; s < t; s += D) visit(a.ks, a.vs, srow(s));
        visit(a.ks, a.vs, srow(t));
    } else {
        for (int s = t; s >= 0; s -= D) visit(a.ks, a.vs, srow(s));
        for (int w = 0; w < W && t - w >= 0; ++w) visit(a.kr, a.vr, base + (size_t)(t - w) * pitch);
    }
    if (lane < d) a.out[base + t * pitch + lane] = o0 / l;
    if (lane + kWave < d) a.out[base + t * pitch + lane + kWave] = o1 / l;
}

hipError_t launch_attn_prefill_f32(const AttnF32Args& a, hipStream_t stream)
{
    hipLaunchKernelGGL(attn_prefill_f32_kernel, dim3((unsigned)(a.B * a.H * a.T)), dim3(kWave), 0, stream, a);
    return hipGetLastError();
}

}  // namespace rat
