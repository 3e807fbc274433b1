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
// Path A (heads with W = 0, including dense D = 1): work items are
// (b, h, r, 256-row chunk).  Persistent workgroups of 8 waves take items in
// a snake order over the cost-sorted item list; each wave owns two 16-row
// blocks (w and 15-w, which balances the causal work) so that every K/V
// fragment read from LDS feeds two MFMA row blocks.  K/V tiles of 64 keys
// stream through a 4-deep LDS ring whose prefetch runs on into the next
// item, so every state row is read from HBM once per chunk.
//
// Path B (heads with W > 0): one workgroup per 2-D block of up to 16
// residues x 16 rows.  Local phase: wave p takes 16 CONTIGUOUS queries
// (for D >= 16: residues r0..r0+15 at one row) against their band of
// W + 15 raw keys; the partial softmax state (m, l, acc) goes to LDS.
// Dilated phase: wave g takes residue r0 + g (16 rows), starts its online
// softmax from the local partials of those queries and runs over the
// residue's states.  The hand-over through LDS is what lets both branches
// use full 16-row MFMA fragments.
#include "rat_device.h"
#include "rat_internal.h"

namespace rat {

typedef __attribute__((address_space(3))) shortx4 lds_s4;

__device__ __forceinline__ floatx4 mfma16(bf16x8 a, bf16x8 b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}


template <int DK>
struct Geo {
    static constexpr int CH = DK / 8;           // 16-byte chunks per row
    static constexpr int ROWB = DK * 2;         // bytes per bf16 row
    static constexpr int KS = DK / 32;          // 32-dim k-steps of QK^T
    static constexpr int DB = DK / 16;          // 16-dim blocks of the output
    static constexpr int RPI = 1024 / ROWB;     // rows per 1 KiB wave load
};

// XOR key of row r: the low bits of r rotated left by one.  Over any CH
// consecutive rows it is a permutation (conflict-free K-fragment reads of
// one logical chunk), and over CH/2 consecutive rows it maps the chunk pair
// (2j, 2j+1) onto CH distinct chunks (conflict-free transposing V reads).
template <int DK>
__device__ __forceinline__ int swz_key(int r)
{
    constexpr int HALF = Geo<DK>::CH / 2;
    return ((r & (HALF - 1)) << 1) | ((r / HALF) & 1);
}

// byte offset of chunk c of row r in a swizzled tile
template <int DK>
__device__ __forceinline__ int swz(int r, int c)
{
    return r * Geo<DK>::ROWB + ((c ^ swz_key<DK>(r)) << 4);
}

// One wave copies RPI rows (1 KiB) global -> LDS: lane l fills row l / (CH)
// of the group, physical chunk l % CH, with the global chunk that the
// swizzle puts there.  `row_ptr` is the global address of the lane's row.
template <int DK>
__device__ __forceinline__ void copy_rows_lds(const uint16_t* row_ptr, int tile_row, lds_char* dst)
{
    constexpr int CH = Geo<DK>::CH;
    const int lane = threadIdx.x & (kWave - 1);
    const int p = lane % CH;
    const int c = p ^ swz_key<DK>(tile_row);
    dma16(row_ptr + c * 8, dst);
}

// K fragment (MFMA A operand of S^T = K Q^T) for keys 16*kb .. 16*kb+15 of
// a tile, k-step ks: lane (g, i) holds K[key 16kb+i][dims 8g+32ks .. +8].
template <int DK>
__device__ __forceinline__ bf16x8 k_frag_lds(const lds_char* tile, int kb, int ks)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int r = kb * 16 + (lane & 15);
    const int c = (lane >> 4) + 4 * ks;
    return *reinterpret_cast<const bf16x8*>(tile + swz<DK>(r, c));
}

// V^T fragment (MFMA A operand of O^T += V^T P^T) for 16-dim block db over
// the 32 keys 32*hh .. 32*hh+31 of a tile.  K-slot order of lane group g:
// slots 0-3 = keys 4g..4g+3, slots 4-7 = keys 16+4g..16+4g+3 (the order in
// which S^T leaves them).  Lane (g, i) receives V[key][dim 16db + i].
template <int DK>
__device__ __forceinline__ bf16x8 v_frag_lds(const lds_char* tile, int hh, int db)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int g = lane >> 4, s = lane & 15;
    const int dim = 16 * db + 4 * (s & 3);
    const int c = dim >> 3, off = (dim & 7) * 2;
    const int r0 = 32 * hh + 4 * g + (s >> 2);
    const int r1 = r0 + 16;
    shortx4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(tile + swz<DK>(r0, c) + off));
    shortx4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(tile + swz<DK>(r1, c) + off));
    typedef short shortx8 __attribute__((ext_vector_type(8)));
    shortx8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// max over the four lanes l, l^16, l^32, l^48 (the four 16-lane rows) with
// the gfx950 row-swap permutes (VALU only, no LDS traffic)
__device__ __forceinline__ float max_over_rows(float x)
{
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
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

    // Scores of 32 keys (two S^T blocks) -> masked, scaled (log2 domain) ->
    // softmax update -> P^T fragment.  `valid[kb][j]` says whether key
    // 16kb + 4g + j is visible to this lane's query.
    __device__ __forceinline__ bf16x8 softmax_step(floatx4 s0, floatx4 s1, const bool (&valid)[2][4], float scale_log2)
    {
        float x[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[j] = valid[0][j] ? s0[j] * scale_log2 : -INFINITY;
            x[4 + j] = valid[1][j] ? s1[j] * scale_log2 : -INFINITY;
        }
        float mx = x[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) mx = fmaxf(mx, x[j]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(m, mx);
        const float msafe = mnew == -INFINITY ? 0.f : mnew;
        const float alpha = __builtin_amdgcn_exp2f(m - msafe);
        m = mnew;
        float p[8], sum = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            p[j] = __builtin_amdgcn_exp2f(x[j] - msafe);
            sum += p[j];
        }
        l = l * alpha + sum;
#pragma unroll
        for (int i = 0; i < Geo<DK>::DB; ++i) acc[i] *= alpha;
        bf16x8 pb;
#pragma unroll
        for (int j = 0; j < 8; ++j) pb[j] = (__bf16)p[j];
        return pb;
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
};

// ------------------------------------------------------------------ path A
constexpr int kWavesA = 8;
constexpr int kTileA = 64;   // keys per K/V tile
constexpr int kRingA = 4;    // LDS ring depth

struct ItemA {
    int b, h, D, r, R0, R1;
    bool valid;
};

// Item `item` of the cost-sorted list: class by block range, levels (the
// 256-row chunk index) most expensive first, then head fastest, residue,
// batch -- consecutive items read the same positions of different heads,
// i.e. whole contiguous token rows.
__device__ __forceinline__ ItemA decode_item_a(const AttnArgs& a, int item)
{
    ItemA it;
    it.valid = false;
    if (item < 0 || item >= a.nblocks) return it;
    int c = 0;
    while (c + 1 < a.nclass && item >= a.cls[c + 1].block_begin) ++c;
    const AttnClass& k = a.cls[c];
    const int local = item - k.block_begin;
    const int level = k.levels - 1 - local / k.per_level;
    int idx = local % k.per_level;
    it.h = a.heads[k.head_off + idx % k.nheads];
    idx /= k.nheads;
    it.r = idx % k.D;
    it.b = idx / k.D;
    it.D = k.D;
    const int M = it.r < a.T ? (a.T - it.r + k.D - 1) / k.D : 0;
    it.R0 = level * kAttnRowsA;
    it.R1 = min(it.R0 + kAttnRowsA, M);
    it.valid = it.R0 < M;
    return it;
}

// Walks this workgroup's items (snake order over rounds of gridDim.x) and
// their tiles; the DMA issue cursor and the compute cursor are two copies.
struct CursorA {
    int round, t, ntile;
    ItemA it;

    __device__ __forceinline__ int item_of(int rnd) const
    {
        const int G = gridDim.x;
        return rnd * G + ((rnd & 1) ? G - 1 - (int)blockIdx.x : (int)blockIdx.x);
    }
    // first valid item at or after round `rnd`; it.valid false when none
    __device__ __forceinline__ void seek(const AttnArgs& a, int rnd)
    {
        for (round = rnd; round * (int)gridDim.x < a.nblocks; ++round) {
            it = decode_item_a(a, item_of(round));
            if (it.valid) {
                t = 0;
                ntile = (it.R1 + kTileA - 1) / kTileA;
                return;
            }
        }
        it.valid = false;
    }
    __device__ __forceinline__ void advance(const AttnArgs& a)
    {
        if (++t == ntile) seek(a, round + 1);
    }
};

template <int DK>
__device__ __forceinline__ void issue_tile_a(const AttnArgs& a, const CursorA& c, lds_char* buf)
{
    typedef Geo<DK> G;
    constexpr int INSTR = 2 * kTileA / G::RPI;
    constexpr int PER_WAVE = INSTR / kWavesA;
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int pitch = a.H * DK;
    const size_t base = ((size_t)c.it.b * a.T * a.H + c.it.h) * DK;
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
        const int instr = wv * PER_WAVE + j;
        const int trow = instr * G::RPI + lane / G::CH;  // K rows then V rows
        const bool isv = trow >= kTileA;
        const int kr = isv ? trow - kTileA : trow;
        const int key = min(c.t * kTileA + kr, c.it.R1 - 1);
        const uint16_t* src = static_cast<const uint16_t*>(isv ? a.vs : a.ks) + base +
                              (size_t)(c.it.r + key * c.it.D) * pitch;
        copy_rows_lds<DK>(src, kr, buf + instr * 1024);
    }
}

// Per-lane byte offsets inside a swizzled tile, hoisted out of the tile
// loop: K fragment of k-step ks for key block 0 (key block kb adds
// kb * 16 rows), and the first transposing V read of 16-dim block db for
// key half 0 (half hh adds 32 rows, the second read 16 rows).
template <int DK>
struct LaneOffsets {
    int k[Geo<DK>::KS];
    int v[Geo<DK>::DB];

    __device__ __forceinline__ void init()
    {
        const int lane = threadIdx.x & (kWave - 1);
        const int g = lane >> 4, i = lane & 15, s = lane & 15;
#pragma unroll
        for (int ks = 0; ks < Geo<DK>::KS; ++ks) k[ks] = swz<DK>(i, g + 4 * ks);
        const int r0 = 4 * g + (s >> 2);
#pragma unroll
        for (int db = 0; db < Geo<DK>::DB; ++db) {
            const int dim = 16 * db + 4 * (s & 3);
            v[db] = swz<DK>(r0, dim >> 3) + (dim & 7) * 2;
        }
    }
};

__device__ __forceinline__ bf16x8 lds_b128(const lds_char* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ __forceinline__ shortx4 lds_tr(const lds_char* p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)p);
}

// Online softmax over one 64-key tile for one 16-row block.  Scores s[kb]
// hold keys 16kb + 4g + j of the lane's query (raw q.k).  The running max
// m (log2 domain) is only raised -- with the rescale of acc and l -- when
// some query's tile max exceeds it by more than kLazyRescale; otherwise the
// stale max stays the exponent reference (weights up to 2^kLazyRescale, the
// result is the same softmax).  Returns P^T operands for the two key halves.
constexpr float kLazyRescale = 8.0f;

template <int DK, bool MASK>
__device__ __forceinline__ void softmax64(Frag<DK>& f, floatx4 (&s)[4], int row, int k0, float c, bf16x8 (&pb)[2])
{
    const int g = (threadIdx.x & (kWave - 1)) >> 4;
    if (MASK) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (k0 + 16 * kb + 4 * g + j > row) s[kb][j] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3]));
#pragma unroll
    for (int kb = 1; kb < 4; ++kb) mx = fmaxf(mx, fmaxf(fmaxf(s[kb][0], s[kb][1]), fmaxf(s[kb][2], s[kb][3])));
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
    float sum = 0.f;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(s[2 * hh][j], c, nm));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(s[2 * hh + 1][j], c, nm));
            sum += p0 + p1;
            pb[hh][j] = (__bf16)p0;
            pb[hh][4 + j] = (__bf16)p1;
        }
    }
    f.l += sum;
}

template <int DK>
__global__ __launch_bounds__(kWavesA * kWave) void attn_dilated_kernel(AttnArgs a)
{
    typedef Geo<DK> G;
    constexpr int TILE_BYTES = 2 * kTileA * G::ROWB;
    constexpr int PER_WAVE = (2 * kTileA / G::RPI) / kWavesA;
    static_assert((2 * kTileA / G::RPI) % kWavesA == 0, "tile loads split evenly over waves");
    extern __shared__ __attribute__((aligned(1024))) char smem[];

    const int lane = threadIdx.x & (kWave - 1);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int i = lane & 15;
    const int pitch = a.H * DK;

    LaneOffsets<DK> off;
    off.init();
    CursorA issue, comp;
    issue.seek(a, 0);
    comp = issue;
    int issued = 0, consumed = 0;
#pragma unroll
    for (int j = 0; j < kRingA - 1; ++j) {
        if (issue.it.valid) {
            issue_tile_a<DK>(a, issue, smem + (issued % kRingA) * TILE_BYTES);
            ++issued;
            issue.advance(a);
        }
    }

    while (comp.it.valid) {
        const ItemA it = comp.it;
        const size_t base = ((size_t)it.b * a.T * a.H + it.h) * DK;
        const uint16_t* qp = static_cast<const uint16_t*>(a.q) + base;
        uint16_t* op = static_cast<uint16_t*>(a.out) + base;
        const int rsA = it.R0 + 16 * wv, rsB = it.R0 + 16 * (15 - wv);
        const bool hasA = rsA < it.R1, hasB = rsB < it.R1;
        Frag<DK> fA, fB;
        fA.reset();
        fB.reset();
        fA.load_q(qp + (size_t)(it.r + (rsA + i) * it.D) * pitch, rsA + i < it.R1);
        fB.load_q(qp + (size_t)(it.r + (rsB + i) * it.D) * pitch, rsB + i < it.R1);

        // Tiles wholly below the chunk's first row are visible to every row
        // of the chunk: they run software-pipelined (the QK^T MFMAs of tile
        // t+1 are issued before the softmax of tile t, so MFMA and VALU work
        // overlap within a wave) with no masks; the diagonal tiles follow on
        // the general path.
        const int nfull = min(it.R0 / kTileA, comp.ntile - 1);
        // Wait until ring tile `seq` has landed, then barrier; refill the
        // ring when the slot after tile `oldest` (the oldest tile still read
        // after this barrier) is free.
        auto wait_tile = [&](int seq, int oldest) {
            const int ahead = issued - seq - 1;
            if (ahead >= 2) wait_vmcnt<2 * PER_WAVE>();
            else if (ahead == 1) wait_vmcnt<PER_WAVE>();
            else wait_vmcnt<0>();
            __syncthreads();
            if (issue.it.valid && issued < oldest + kRingA) {
                issue_tile_a<DK>(a, issue, smem + (issued % kRingA) * TILE_BYTES);
                ++issued;
                issue.advance(a);
            }
        };
        auto qk = [&](int seq, floatx4 (&sa)[4], floatx4 (&sb)[4]) {
            const lds_char* kt = smem + (seq % kRingA) * TILE_BYTES;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                sa[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
                sb[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < G::KS; ++ks) {
                    const bf16x8 kf = lds_b128(kt + off.k[ks] + kb * 16 * G::ROWB);
                    sa[kb] = mfma16(kf, fA.q[ks], sa[kb]);
                    sb[kb] = mfma16(kf, fB.q[ks], sb[kb]);
                }
            }
        };
        auto pv = [&](int seq, const bf16x8 (&pa)[2], const bf16x8 (&pbb)[2]) {
            const lds_char* vt = smem + (seq % kRingA) * TILE_BYTES + kTileA * G::ROWB;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
                for (int db = 0; db < G::DB; ++db) {
                    const lds_char* vp = vt + off.v[db] + hh * 32 * G::ROWB;
                    const shortx4 x0 = lds_tr(vp);
                    const shortx4 x1 = lds_tr(vp + 16 * G::ROWB);
                    typedef short shortx8 __attribute__((ext_vector_type(8)));
                    const shortx8 v8 = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
                    const bf16x8 vf = __builtin_bit_cast(bf16x8, v8);
                    fA.acc[db] = mfma16(vf, pa[hh], fA.acc[db]);
                    fB.acc[db] = mfma16(vf, pbb[hh], fB.acc[db]);
                }
            }
        };

        floatx4 sA[4], sB[4];
        bool have_scores = false;
        if (nfull > 0) {
            wait_tile(consumed, consumed);
            qk(consumed, sA, sB);
            for (int tt = 0; tt < nfull; ++tt) {
                wait_tile(consumed + 1, consumed);  // tile `consumed` still feeds P V
                floatx4 nA[4], nB[4];
                qk(consumed + 1, nA, nB);
                bf16x8 pA[2], pB[2];
                softmax64<DK, false>(fA, sA, 0, 0, a.scale_log2, pA);
                softmax64<DK, false>(fB, sB, 0, 0, a.scale_log2, pB);
                pv(consumed, pA, pB);
                ++consumed;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    sA[kb] = nA[kb];
                    sB[kb] = nB[kb];
                }
            }
            have_scores = true;  // tile nfull's scores are in sA / sB
        }
        for (int tt = nfull; tt < comp.ntile; ++tt) {
            if (!have_scores) {
                wait_tile(consumed, consumed);
                qk(consumed, sA, sB);
            }
            have_scores = false;
            const int k0 = tt * kTileA;
            const bool needA = hasA && k0 <= rsA + 15;
            const bool needB = hasB && k0 <= rsB + 15;
            bf16x8 pA[2] = {}, pB[2] = {};
            if (needA) {
                if (k0 + kTileA - 1 <= rsA) softmax64<DK, false>(fA, sA, rsA + i, k0, a.scale_log2, pA);
                else softmax64<DK, true>(fA, sA, rsA + i, k0, a.scale_log2, pA);
            }
            if (needB) {
                if (k0 + kTileA - 1 <= rsB) softmax64<DK, false>(fB, sB, rsB + i, k0, a.scale_log2, pB);
                else softmax64<DK, true>(fB, sB, rsB + i, k0, a.scale_log2, pB);
            }
            pv(consumed, pA, pB);
            ++consumed;
        }
        fA.store(op + (size_t)(it.r + (rsA + i) * it.D) * pitch, rsA + i < it.R1);
        fB.store(op + (size_t)(it.r + (rsB + i) * it.D) * pitch, rsB + i < it.R1);
        comp.seek(a, comp.round + 1);
    }
}

// ------------------------------------------------------------------ path B
// Each wave streams its own 32-key tiles: K fragments straight from HBM into
// registers, V rows into the wave's private swizzled LDS tile.
template <int DK>
struct WaveStream {
    typedef Geo<DK> G;
    static constexpr int TILE = 32;

    // key rows: position of key j of the tile is pos0 + j * step (clamped to last)
    __device__ __forceinline__ static void load_v(const uint16_t* vbase, size_t pitch, int pos0, int step, int nkeys,
                                                  lds_char* vt)
    {
        const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
        for (int j = 0; j < TILE / G::RPI; ++j) {
            const int tr = j * G::RPI + lane / G::CH;
            const int key = min(tr, nkeys - 1);
            copy_rows_lds<DK>(vbase + (size_t)(pos0 + key * step) * pitch, tr, vt + j * 1024);
        }
    }

    __device__ __forceinline__ static void load_k(const uint16_t* kbase, size_t pitch, int pos0, int step, int nkeys,
                                                  bf16x8 (&kf)[2][G::KS])
    {
        const int lane = threadIdx.x & (kWave - 1);
        const int g = lane >> 4, i = lane & 15;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int key = min(16 * kb + i, nkeys - 1);
            const uint16_t* p = kbase + (size_t)(pos0 + key * step) * pitch + 8 * g;
#pragma unroll
            for (int ks = 0; ks < G::KS; ++ks) kf[kb][ks] = *reinterpret_cast<const bf16x8*>(p + 32 * ks);
        }
    }
};

// Streams keys at positions pos0 + j*step, j in [0, nkeys), through fragment
// f; `vis(j)` tells whether key j is visible to this lane's query.
template <int DK, typename Vis>
__device__ __forceinline__ void stream_keys(Frag<DK>& f, const uint16_t* kbase, const uint16_t* vbase, size_t pitch,
                                            int pos0, int step, int nkeys, lds_char* vt, float scale_log2, Vis vis)
{
    typedef Geo<DK> G;
    const int g = (threadIdx.x & (kWave - 1)) >> 4;
    for (int k0 = 0; k0 < nkeys; k0 += 32) {
        const int n = min(32, nkeys - k0);
        bf16x8 kf[2][G::KS];
        WaveStream<DK>::load_v(vbase, pitch, pos0 + k0 * step, step, n, vt);
        WaveStream<DK>::load_k(kbase, pitch, pos0 + k0 * step, step, n, kf);
        wait_vmcnt<0>();
        __builtin_amdgcn_wave_barrier();
        floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < G::KS; ++ks) {
            s0 = mfma16(kf[0][ks], f.q[ks], s0);
            s1 = mfma16(kf[1][ks], f.q[ks], s1);
        }
        bool valid[2][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int ka = k0 + 4 * g + j, kb = k0 + 16 + 4 * g + j;
            valid[0][j] = ka < nkeys && vis(ka);
            valid[1][j] = kb < nkeys && vis(kb);
        }
        const bf16x8 pb = f.softmax_step(s0, s1, valid, scale_log2);
#pragma unroll
        for (int db = 0; db < G::DB; ++db) f.acc[db] = mfma16(v_frag_lds<DK>(vt, 0, db), pb, f.acc[db]);
        __builtin_amdgcn_wave_barrier();  // tr reads done before the tile is refilled
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): LDS reads retired
    }
}

template <int DK>
__device__ void path_b(const AttnArgs& a, int b, int h, int D, int W, int rgroup, int iblock, lds_char* smem)
{
    typedef Geo<DK> G;
    const int T = a.T, pitch = a.H * DK;
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int i = lane & 15, g = lane >> 4;
    const size_t base = ((size_t)b * T * a.H + h) * DK;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + base;
    const uint16_t* ksp = static_cast<const uint16_t*>(a.ks) + base;
    const uint16_t* vsp = static_cast<const uint16_t*>(a.vs) + base;
    const uint16_t* krp = static_cast<const uint16_t*>(a.kr) + base;
    const uint16_t* vrp = static_cast<const uint16_t*>(a.vr) + base;
    uint16_t* op = static_cast<uint16_t*>(a.out) + base;

    const int r0 = D >= 16 ? 16 * rgroup : 0;
    const int R = D >= 16 ? min(16, D - r0) : D;      // residues in the block
    const int i0 = kAttnRowsB * iblock;               // first row
    const int npieces = D >= 16 ? 16 : D;

    // exchange area: slot = (residue - r0) * 16 + (row - i0)
    float* xacc = reinterpret_cast<float*>(smem);
    float* xm = xacc + 256 * DK;
    float* xl = xm + 256;
    lds_char* vt = smem + wv * (32 * G::ROWB);         // this wave's V tile

    // ---- local phase: piece wv = contiguous positions [P, P + n)
    Frag<DK> f;
    f.reset();
    int P = 0, n = 0;
    if (wv < npieces) {
        P = D >= 16 ? r0 + (i0 + wv) * D : i0 * D + 16 * wv;
        const int len = D >= 16 ? R : 16;
        n = P < T ? min(len, T - P) : 0;
    }
    const int tq = P + i;                               // this lane's query
    const bool lvalid = i < n;
    if (n > 0) {
        f.load_q(qp + (size_t)tq * pitch, lvalid);
        const int u0 = max(0, P - W + 1);
        const int nk = P + n - u0;
        stream_keys<DK>(f, krp, vrp, (size_t)pitch, u0, 1, nk, vt, a.scale_log2,
                        [&](int j) { const int u = u0 + j; return lvalid && u <= tq && tq - u < W; });
    }
    const float lt = f.total_l();
    __syncthreads();  // V tiles retired; the area becomes the exchange buffer
    if (n > 0 && lvalid) {
        const int slot = ((tq % D) - r0) * 16 + (tq / D - i0);
#pragma unroll
        for (int db = 0; db < G::DB; ++db)
            *reinterpret_cast<floatx4*>(xacc + slot * DK + 16 * db + 4 * g) = f.acc[db];
        if (g == 0) {
            xm[slot] = f.m;
            xl[slot] = lt;
        }
    }
    __syncthreads();

    // ---- dilated phase: residue r0 + wv, rows i0 .. i0+15, seeded by the local partials
    const int r = r0 + wv;
    const int M = r < D && r < T ? (T - r + D - 1) / D : 0;
    const int row = i0 + i;
    const bool dvalid = wv < R && row < M;
    Frag<DK> fd;
    fd.reset();
    if (dvalid) {
        const int slot = wv * 16 + i;
#pragma unroll
        for (int db = 0; db < G::DB; ++db)
            fd.acc[db] = *reinterpret_cast<const floatx4*>(xacc + slot * DK + 16 * db + 4 * g);
        fd.m = xm[slot];
        fd.l = g == 0 ? xl[slot] : 0.f;
    }
    __syncthreads();  // exchange read; the area returns to V tiles
    if (wv < R && i0 < M) {
        fd.load_q(qp + (size_t)(r + row * D) * pitch, dvalid);
        const int nk = min(i0 + 16, M);
        stream_keys<DK>(fd, ksp, vsp, (size_t)pitch, r, D, nk, vt, a.scale_log2,
                        [&](int j) { return dvalid && j <= row; });
        fd.store(op + (size_t)(r + row * D) * pitch, dvalid);
    }
}

// ------------------------------------------------------------------ kernels
template <int DK>
__global__ __launch_bounds__(kAttnWaves * kWave) void attn_window_kernel(AttnArgs a)
{
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const int blk = blockIdx.x;
    int c = 0;
    while (c + 1 < a.nclass && blk >= a.cls[c + 1].block_begin) ++c;
    const AttnClass& k = a.cls[c];
    const int local = blk - k.block_begin;
    const int level = k.levels - 1 - local / k.per_level;  // most expensive first
    int idx = local % k.per_level;
    const int ngroups = k.D >= 16 ? (k.D + 15) / 16 : 1;
    const int rg = idx % ngroups;
    idx /= ngroups;
    const int h = a.heads[k.head_off + idx % k.nheads];
    const int b = idx / k.nheads;
    path_b<DK>(a, b, h, k.D, k.W, rg, level, smem);
}

size_t attn_lds_bytes_a(int d) { return (size_t)kRingA * 2 * kTileA * d * 2; }

size_t attn_lds_bytes_b(int d)
{
    const size_t vt = kAttnWaves * 32 * (size_t)d * 2;     // V tiles
    const size_t xch = 256 * (size_t)d * 4 + 2 * 256 * 4;  // exchange
    return vt > xch ? vt : xch;
}

template <typename K>
static void set_lds(K kernel, size_t lds, bool& done)
{
    if (!done) {
        (void)hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        done = true;
    }
}

hipError_t launch_attn_dilated_bf16(const AttnArgs& a, int d, int grid, hipStream_t stream)
{
    const size_t lds = attn_lds_bytes_a(d);
    static bool s128 = false, s64 = false;
    if (d == 128) {
        set_lds(attn_dilated_kernel<128>, lds, s128);
        hipLaunchKernelGGL(attn_dilated_kernel<128>, dim3(grid), dim3(kWavesA * kWave), lds, stream, a);
    } else {
        set_lds(attn_dilated_kernel<64>, lds, s64);
        hipLaunchKernelGGL(attn_dilated_kernel<64>, dim3(grid), dim3(kWavesA * kWave), lds, stream, a);
    }
    return hipGetLastError();
}

hipError_t launch_attn_window_bf16(const AttnArgs& a, int d, hipStream_t stream)
{
    const size_t lds = attn_lds_bytes_b(d);
    static bool s128 = false, s64 = false;
    if (d == 128) {
        set_lds(attn_window_kernel<128>, lds, s128);
        hipLaunchKernelGGL(attn_window_kernel<128>, dim3(a.nblocks), dim3(kAttnWaves * kWave), lds, stream, a);
    } else {
        set_lds(attn_window_kernel<64>, lds, s64);
        hipLaunchKernelGGL(attn_window_kernel<64>, dim3(a.nblocks), dim3(kAttnWaves * kWave), lds, stream, a);
    }
    return hipGetLastError();
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
    auto visit = [&](const float* kbase, const float* vbase, int s) {
        const float* kr = kbase + base + s * pitch;
        float dot = (lane < d ? q0 * kr[lane] : 0.f) + (lane + kWave < d ? q1 * kr[lane + kWave] : 0.f);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) dot += __shfl_xor(dot, o);
        const float z = dot * a.scale;
        const float mn = fmaxf(m, z);
        const float al = expf(m - mn), p = expf(z - mn);
        const float* vr = vbase + base + s * pitch;
        o0 = o0 * al + p * (lane < d ? vr[lane] : 0.f);
        o1 = o1 * al + p * (lane + kWave < d ? vr[lane + kWave] : 0.f);
        l = l * al + p;
        m = mn;
    };
    for (int s = t; s >= 0; s -= D) visit(a.ks, a.vs, s);
    for (int w = 0; w < W && t - w >= 0; ++w) visit(a.kr, a.vr, t - w);
    if (lane < d) a.out[base + t * pitch + lane] = o0 / l;
    if (lane + kWave < d) a.out[base + t * pitch + lane + kWave] = o1 / l;
}

hipError_t launch_attn_prefill_f32(const AttnF32Args& a, hipStream_t stream)
{
    hipLaunchKernelGGL(attn_prefill_f32_kernel, dim3((unsigned)(a.B * a.H * a.T)), dim3(kWave), 0, stream, a);
    return hipGetLastError();
}

}  // namespace rat
