// Work plans and address formation of the RAT+ kernels, shared by the
// kernels, the C ABI's launch planning and a host-side address check.
//
// Everything here is plain integer arithmetic: the __host__ __device__
// functions are the ones the kernels call to form every global address of
// the state-history (decode cache) paths and of the attention's ring
// copies, so that the same code can be walked on the host over a whole
// launch grid and each address compared with its buffer's extent.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "rat_internal.h"
#include "rat_mfma.h"

namespace rat {

__host__ __device__ __forceinline__ int imin(int a, int b) { return a < b ? a : b; }
__host__ __device__ __forceinline__ int imax(int a, int b) { return a > b ? a : b; }

// ---------------------------------------------------------------- scan
// Workspace plan of the full / RESTART scan: chunks of CT tokens of one
// BW-channel block (ScanGeo), a 256-byte header, then per chunk the tagged
// aggregate words [3][block] and inclusive words [2][block].  `wide`: the
// wide bf16 geometry, taken unless the recurrence restarts every 256 tokens
// or sooner (then every chunk starts at, or right after, a restart and
// needs no long look-back, and the narrow chunk's shorter prefix wins).
struct ScanPlan {
    int chunk, nblk, nseq, nchunk, nwg;
    bool wide;
    size_t agg_off, incl_off, bytes;
};

inline bool scan_wide(int T, int L, bool bf16) { return bf16 && !(L < T && L <= 256); }

inline ScanPlan scan_plan(int B, int T, int H, int d, int L, bool bf16)
{
    ScanPlan p;
    p.wide = scan_wide(T, L, bf16);
    p.chunk = !bf16 ? ScanGeo<float, false>::CT : p.wide ? ScanGeo<uint16_t, true>::CT : ScanGeo<uint16_t, false>::CT;
    const int bw = !bf16 ? ScanGeo<float, false>::BW : p.wide ? ScanGeo<uint16_t, true>::BW : ScanGeo<uint16_t, false>::BW;
    const int N = H * d;
    p.nblk = (N + bw - 1) / bw;
    p.nseq = B * p.nblk;
    p.nchunk = (T + p.chunk - 1) / p.chunk;
    p.nwg = p.nchunk * p.nseq;
    const size_t slots = (size_t)p.nwg;
    p.agg_off = sizeof(ScanHeader);
    p.incl_off = p.agg_off + slots * 3 * bw * sizeof(uint64_t);
    p.bytes = p.incl_off + slots * 2 * bw * sizeof(uint64_t);
    return p;
}

// Where lane `lane` of wave `w` works in the chunk of ticket `ticket`:
// channels ch0 .. ch0 + CPL - 1 (CPL = 16 / element size) of tokens t0 ..
// t0 + kScanTpl - 1 (LPR lanes per row segment, 64 / LPR segments per wave).
struct ScanLane {
    int chunk, seq, b, cblk, tb, c, seg, ch0, t0;
    bool cvalid;
};

template <int CPL, int LPR>
__host__ __device__ __forceinline__ ScanLane scan_lane(const ScanFullArgs& a, uint32_t ticket, int w, int lane)
{
    constexpr int BW = LPR * CPL, GPW = 64 / LPR, CT = kScanFullWaves * GPW * kScanTpl;
    ScanLane s;
    s.chunk = (int)(ticket / (uint32_t)a.nseq);
    s.seq = (int)(ticket % (uint32_t)a.nseq);
    s.b = s.seq / a.nblk;
    s.cblk = (s.seq % a.nblk) * BW;
    s.tb = s.chunk * CT;
    s.c = lane % LPR;
    s.seg = w * GPW + lane / LPR;
    s.ch0 = s.cblk + s.c * CPL;
    s.cvalid = s.ch0 < a.N;
    s.t0 = s.tb + s.seg * kScanTpl;
    return s;
}

// Row of position t in a StateHist head with dilation D and mcap = n_cap / D
// rows per residue, walked token by token without a division.
struct HistRow {
    int res, q, D, mcap;
    __host__ __device__ __forceinline__ void init(int t, int D_, int n_cap)
    {
        D = D_;
        mcap = n_cap / D_;
        q = t / D_;
        res = t - q * D_;
    }
    __host__ __device__ __forceinline__ int row() const { return res * mcap + q; }
    __host__ __device__ __forceinline__ void next()
    {
        if (++res == D) {
            res = 0;
            ++q;
        }
    }
};

// History-writing scan: the lane's head (its CPL channels lie in one head,
// d being a multiple of 64), that head's dilation, and the element offset
// of the lane's first channel in row 0 of its history block.
__host__ __device__ __forceinline__ int scan_hist_head(const ScanFullArgs& a, int ch0) { return ch0 / a.d; }
__host__ __device__ __forceinline__ int scan_hist_D(const ScanFullArgs& a, const ScanLane& s)
{
    return a.hist.D[s.cvalid ? scan_hist_head(a, s.ch0) : 0];
}
__host__ __device__ __forceinline__ size_t scan_hist_base(const ScanFullArgs& a, const ScanLane& s)
{
    const int hh = scan_hist_head(a, s.ch0);
    return ((size_t)s.b * a.hist.H + hh) * a.hist.n_cap * a.d + (s.ch0 - hh * a.d);
}
// element offset of the lane's channels in the fp32 final state [B][H][2][d]
// (the key states; the value states are d further)
__host__ __device__ __forceinline__ size_t scan_fin_offset(const ScanFullArgs& a, const ScanLane& s)
{
    const int hh = s.ch0 / a.d;
    return ((size_t)(s.b * (a.N / a.d) + hh) * 2) * a.d + (s.ch0 - hh * a.d);
}

// ---------------------------------------------------------------- ring fill
// Thread `idx` (one per `epv` elements of a ring row) of the raw-ring fill:
// false when it copies nothing, else the element offsets of its source in
// [B][T][H][d] and its destination in [B][H][w_cap][d].
__host__ __device__ __forceinline__ bool ring_fill_at(const RingFillArgs& a, size_t idx, int epv, size_t& src,
                                                      size_t& dst)
{
    const int vpr = a.d / epv;  // vectors per row
    if (idx >= (size_t)a.B * a.H * a.w_cap * vpr) return false;
    const int c = (int)(idx % vpr) * epv;
    const size_t row = idx / vpr;  // (b H + h) w_cap + slot
    const int slot = (int)(row % a.w_cap);
    const size_t bh = row / a.w_cap;
    const int h = (int)(bh % a.H), b = (int)(bh / a.H);
    const int W = a.W[h];
    if (slot >= W) return false;
    const int p = (a.T - 1) - ((a.T - 1 - slot) % W + W) % W;  // latest position of the slot
    if (p < 0) return false;
    src = (((size_t)b * a.T + p) * a.H + h) * a.d + c;
    dst = row * a.d + c;
    return true;
}

// ---------------------------------------------------------------- attention
constexpr int kTileA = 64;   // keys per K/V tile
constexpr int kRingA = 4;    // LDS ring depth
constexpr int kSlotRows = 2 * kTileA;  // rows of one ring slot

struct ItemA {
    int b, h, D, W, r, R0, R1;
    int kbeg;  // first key (0, or the start of a band item's key range)
    int kres;  // residue of the key rows: r, or D - 1 on the chunk grid (0 for a band item)
    int nkey;  // key rows the item's queries can see: R1, or R1 - 1 on the chunk grid
    bool valid;
};

// Item `item` of the cost-sorted list: class by block range, levels (the
// 256-row chunk index) most expensive first, then head fastest, residue,
// batch -- consecutive items read the same positions of different heads,
// i.e. whole contiguous token rows.
template <bool BAND, bool CHUNK>
__host__ __device__ __forceinline__ ItemA decode_item_a(const AttnArgs& a, int item)
{
    ItemA it;
    it.valid = false;
    if (item < 0 || item >= a.nblocks) return it;
    int c = 0;
    while (c + 1 < a.nclass && item >= a.cls[c + 1].block_begin) ++c;
    const AttnClass& k = a.cls[c];
    const int local = item - k.block_begin;
    it.W = k.W;
    if (BAND) {
        // band item: 256 contiguous queries of (b, h), keys t0-W+1 .. t0+255
        const int idx = local % k.per_level;
        it.h = a.heads[k.head_off + idx % k.nheads];
        it.b = idx / k.nheads;
        it.r = 0;
        it.D = 1;
        it.R0 = (local / k.per_level) * a.rows;
        it.R1 = imin(it.R0 + a.rows, a.T);
        it.kbeg = imax(0, it.R0 - k.W + 1) & ~(kTileA - 1);
        it.kres = 0;
        it.nkey = it.R1;
        it.valid = it.R0 < a.T;
        return it;
    }
    // Levels most expensive first.  With a few levels (short residues, the
    // four-wave kernel), the items of eight residues alternate by level in
    // groups of eight: a residue's items lie eight apart, so workgroups on
    // one XCD (workgroup i runs on XCD i mod 8) take them in the same round
    // and its L2 serves the key tiles they share.  Residues past the last
    // whole group of eight keep the level-major order.
    int level, idx;
    const int p8 = (k.per_level / 8) * 8;
    if (k.levels > 1 && k.levels <= 4 && local < p8 * k.levels) {
        const int w = local % (8 * k.levels);
        level = k.levels - 1 - w / 8;
        idx = (local / (8 * k.levels)) * 8 + w % 8;
    } else if (k.levels > 1 && k.levels <= 4) {
        const int rest = k.per_level - p8, r = local - p8 * k.levels;
        level = k.levels - 1 - r / rest;
        idx = p8 + r % rest;
    } else {
        level = k.levels - 1 - local / k.per_level;
        idx = local % k.per_level;
    }
    it.h = a.heads[k.head_off + idx % k.nheads];
    idx /= k.nheads;
    it.r = idx % k.D;
    it.b = idx / k.D;
    it.D = k.D;
    const int M = it.r < a.T ? (a.T - it.r + k.D - 1) / k.D : 0;
    it.R0 = level * a.rows;
    it.R1 = imin(it.R0 + a.rows, M);
    it.kbeg = 0;
    // chunk grid: query row i (position r + iD) sees the chunk ends
    // jD + D - 1 with j < i, all of which exist
    it.kres = CHUNK ? k.D - 1 : it.r;
    it.nkey = CHUNK ? it.R1 - 1 : it.R1;
    it.valid = it.R0 < M;
    return it;
}

// Walks a workgroup's items (snake order over rounds of G workgroups) and
// the ring steps of each: nq slots of query rows (128 rows each), for
// windowed classes as many slots of partial outputs, on the chunk grid the
// own-state steps, then the key tiles.
template <bool BAND, bool CHUNK, bool HIST>
struct CursorA {
    int round, t, nq, no, nown, ntile;
    int rowidx;   // (b T + r) H + h: first row of the item in units of head rows
    int krowidx;  // the same for its key rows (residue kres); with HIST the first
                  // history row of the residue, (b H + h) n_cap + r n_cap / D
    int dstride;  // min(D, T) H: head rows between consecutive rows of the item
    ItemA it;

    // G: workgroups of the launch; blk: this workgroup
    __host__ __device__ __forceinline__ static int item_of(int rnd, int G, int blk)
    {
        return rnd * G + ((rnd & 1) ? G - 1 - blk : blk);
    }
    // first valid item at or after round `rnd`; it.valid false when none
    __host__ __device__ __forceinline__ void seek(const AttnArgs& a, int rnd, int G, int blk)
    {
        for (round = rnd; round * G < a.nblocks; ++round) {
            it = decode_item_a<BAND, CHUNK>(a, item_of(round, G, blk));
            if (it.valid) {
                t = 0;
                nq = (it.R1 - it.R0 + kSlotRows - 1) / kSlotRows;
                no = (!BAND && it.W > 0) ? nq : 0;
                // chunk grid: the item's own states, 64 query rows per step
                nown = CHUNK ? (it.R1 - it.R0 + kTileA - 1) / kTileA : 0;
                ntile = imax(0, (CHUNK ? it.nkey : it.R1) - it.kbeg + kTileA - 1) / kTileA;
                rowidx = (it.b * a.T + it.r) * a.H + it.h;
                krowidx = HIST    ? (it.b * a.H + it.h) * a.n_cap + it.r * (a.n_cap / it.D)
                          : CHUNK ? (it.b * a.T + it.kres) * a.H + it.h
                                  : rowidx;
                // a residue of D >= T holds one row: min(D, T) keeps byte
                // strides below 2^32 without changing any address
                dstride = imin(it.D, a.T) * a.H;
                return;
            }
        }
        it.valid = false;
    }
    __host__ __device__ __forceinline__ void advance(const AttnArgs& a, int G, int blk)
    {
        if (++t == nq + no + (CHUNK ? nown : 0) + ntile) seek(a, round + 1, G, blk);
    }
};

// Per-lane constants of the ring copies: row lq = lane / CH of each
// RPI-row copy, and the swizzled 16-byte chunk the lane fetches for a copy
// whose first slot row is a multiple of RPI (the XOR key is linear in the
// row bits, so copy j only XORs in the key of row RPI j, a uniform value).
template <int DK>
__host__ __device__ __forceinline__ void dma_lane_a(int lane, uint32_t& lq, uint32_t& col16)
{
    lq = (uint32_t)(lane / Geo<DK>::CH);
    col16 = (uint32_t)(((lane % Geo<DK>::CH) ^ swz_key<DK>((int)lq)) << 4);
}

// The copies of one wave for the cursor's ring step into the slot at LDS
// byte address `buf`: PER_WAVE copies of RPI rows, copy j from tensor `src`
// (0: q, 1: out -- partial outputs --, 2: the wave's K or V rows) at byte
// offset rel[j] + lane offset from the tensor's start, landing at LDS
// m0[j] + 16 lane.  Rows past the item's last row R1 - 1 are clamped to it.
// The wave-uniform part (source, rel, m0, the clamp limits) is formed
// apart from the lanes' offsets so that it stays in scalar registers.
template <int DK, int NW>
struct StepCopiesA {
    static constexpr int INSTR = kSlotRows / Geo<DK>::RPI;
    static constexpr int PER_WAVE = INSTR / NW;
    int src;
    bool whole;               // every row of the wave's share exists (no clamp)
    uint32_t dp2;             // bytes between consecutive rows of the item
    int row0, last;           // the wave's first row of the step; the item's last row
    uint64_t rel[PER_WAVE];
    uint32_t lim[PER_WAVE];   // clamped copies: the lane row offset is at most lim
    uint32_t m0[PER_WAVE];
};

template <int DK, int NW, bool BAND, bool CHUNK, bool HIST>
__host__ __device__ __forceinline__ void step_copies_a(const AttnArgs& a, const CursorA<BAND, CHUNK, HIST>& c, int wv,
                                                       uint32_t buf, StepCopiesA<DK, NW>& s)
{
    typedef Geo<DK> G;
    constexpr int PER_WAVE = StepCopiesA<DK, NW>::PER_WAVE;
    static_assert(PER_WAVE * G::RPI <= kTileA && kTileA % (PER_WAVE * G::RPI) == 0, "a wave copies K or V rows only");
    (void)a;
    const int ko = c.t - c.nq - c.no;  // own-state step, then key tile; < 0 for query / partial steps
    const bool own = CHUNK && ko >= 0 && ko < c.nown;
    const int kt = CHUNK && ko >= 0 ? ko - c.nown : ko;  // key tile index (< 0 also for own-state steps)
    // first row of the wave's share of the slot, and the tensor it comes from
    int row0;
    if (ko < 0) {  // query rows, or partial outputs, R0 + 128 s + 16 PER_WAVE wv ...
        const int st = c.t < c.nq ? c.t : c.t - c.nq;
        row0 = c.it.R0 + st * kSlotRows + wv * PER_WAVE * G::RPI;
        s.src = c.t < c.nq ? 0 : 1;
    } else if (own) {  // K rows (waves 0 .. NW/2-1) or V rows of the own states, R0 + 64 ko ...
        row0 = c.it.R0 + ko * kTileA + (wv * PER_WAVE * G::RPI) % kTileA;
        s.src = 2;
    } else {       // K rows (waves 0 .. NW/2-1) or V rows of key tile kt
        row0 = c.it.kbeg + kt * kTileA + (wv * PER_WAVE * G::RPI) % kTileA;
        s.src = 2;
    }
    // a key tile read elsewhere than the query rows: the chunk ends
    // (residue kres), or the residue's contiguous rows of a state history
    const bool keys = (CHUNK || HIST) && ko >= 0 && !own;
    const uint32_t item_el = (uint32_t)(keys ? c.krowidx : c.rowidx) * DK;
    s.dp2 = (HIST && keys ? 1u : (uint32_t)c.dstride) * (2 * DK);
    const int last = (CHUNK && ko >= 0 && !own ? c.it.nkey : c.it.R1) - 1;
    const uint32_t slot = buf + wv * PER_WAVE * 1024;  // LDS byte address of the wave's first copy
    s.row0 = row0;
    s.last = last;
    s.whole = row0 + PER_WAVE * G::RPI - 1 <= last;
    if (s.whole) {
        // every row of the wave's share exists: copy j starts RPI rows after
        // copy j - 1 (one 64-bit add each), lane offsets need no clamp
        const uint64_t step = (uint64_t)G::RPI * s.dp2;
        uint64_t rel = 2ull * item_el + (uint64_t)(uint32_t)row0 * s.dp2;
#pragma unroll
        for (int j = 0; j < PER_WAVE; ++j) {
            s.m0[j] = slot + j * 1024;
            s.rel[j] = rel;
            s.lim[j] = 0xffffffffu;
            rel += step;
        }
    } else {
        // the item ends inside the wave's share: rows past R1 - 1 read row R1 - 1
#pragma unroll
        for (int j = 0; j < PER_WAVE; ++j) {
            const int first = imin(row0 + j * G::RPI, last);
            s.m0[j] = slot + j * 1024;
            s.rel[j] = 2ull * (item_el + (uint32_t)first * (s.dp2 >> 1));
            s.lim[j] = (uint32_t)(last - first) * s.dp2;
        }
    }
}

// A key-tile step of the cursor: a step past the item's query, partial and
// own-state steps.
template <bool BAND, bool CHUNK, bool HIST>
__host__ __device__ __forceinline__ int step_key_tile_a(const CursorA<BAND, CHUNK, HIST>& c)
{
    return c.t - c.nq - c.no - (CHUNK ? c.nown : 0);  // key tile index, < 0 for other steps
}

// Runs of key tiles.  Key tile kt + 1 of an item is key tile kt moved by
// kTileA rows: the same tensor, row stride and last row, so while the
// wave's share of the tile stays whole its copy j starts at
// rel0 + j RPI dp2, rel0 one add further than the tile before.  KeyRunA
// holds a wave's plan of the key tile last issued (taken from a whole
// step_copies_a); key_run_next_a moves it to the cursor's step when that
// step is the next key tile of the same item and still whole, and returns
// false otherwise (the step then takes the full plan).
struct KeyRunA {
    uint64_t rel0;  // byte offset of copy 0 from the key tensor's start
    uint32_t dp2;   // bytes between consecutive rows
    int row0, last;
};

template <int DK, int NW, bool BAND, bool CHUNK, bool HIST>
__host__ __device__ __forceinline__ bool key_run_next_a(const CursorA<BAND, CHUNK, HIST>& c, KeyRunA& k)
{
    constexpr int SPAN = StepCopiesA<DK, NW>::PER_WAVE * Geo<DK>::RPI;  // rows of the wave's share
    if (step_key_tile_a(c) < 1) return false;  // the step before was no key tile of this item
    const int row0 = k.row0 + kTileA;
    if (row0 + SPAN - 1 > k.last) return false;
    k.row0 = row0;
    k.rel0 += (uint64_t)kTileA * k.dp2;
    return true;
}

// Byte offset of copy j of a key run's tile (what step_copies_a's rel[j] is)
template <int DK>
__host__ __device__ __forceinline__ uint64_t key_run_rel_a(const KeyRunA& k, int j)
{
    return k.rel0 + (uint64_t)j * Geo<DK>::RPI * k.dp2;
}

// The lane's byte offset within copy j: its row lq of the copy (clamped to
// the copy's limit unless the wave's share is whole) and its swizzled
// 16-byte chunk.  The whole and the clamped forms are apart so that the
// issue of a whole share runs only the first.
template <int DK, int NW>
__host__ __device__ __forceinline__ uint32_t step_chunk_a(int wv, int j, uint32_t col16)
{
    const int instr = wv * StepCopiesA<DK, NW>::PER_WAVE + j;
    return col16 ^ (uint32_t)(swz_key<DK>(instr * Geo<DK>::RPI) << 4);
}

template <int DK, int NW>
__host__ __device__ __forceinline__ uint32_t step_lane_offset_whole_a(const StepCopiesA<DK, NW>& s, int wv, int j,
                                                                      uint32_t lq, uint32_t col16)
{
    return lq * s.dp2 + step_chunk_a<DK, NW>(wv, j, col16);  // < 2^32: the row exists
}

template <int DK, int NW>
__host__ __device__ __forceinline__ uint32_t step_lane_offset_clamped_a(const StepCopiesA<DK, NW>& s, int wv, int j,
                                                                        uint32_t lq, uint32_t col16)
{
    const uint64_t lrow64 = (uint64_t)lq * s.dp2;  // saturated: only its min with the limit is used
    const uint32_t lrow = lrow64 > 0xffffffffull ? 0xffffffffu : (uint32_t)lrow64;
    return (lrow < s.lim[j] ? lrow : s.lim[j]) + step_chunk_a<DK, NW>(wv, j, col16);
}

template <int DK, int NW>
__host__ __device__ __forceinline__ uint32_t step_lane_offset_a(const StepCopiesA<DK, NW>& s, int wv, int j,
                                                                uint32_t lq, uint32_t col16)
{
    return s.whole ? step_lane_offset_whole_a<DK, NW>(s, wv, j, lq, col16)
                   : step_lane_offset_clamped_a<DK, NW>(s, wv, j, lq, col16);
}

// A partial-output step's (m, l) words on waves 0-3: lane l of wave wv
// reads float word side_word of the workspace (-1: none this step).
template <bool BAND, bool CHUNK, bool HIST>
__host__ __device__ __forceinline__ int64_t step_side_word_a(const AttnArgs& a, const CursorA<BAND, CHUNK, HIST>& c,
                                                              int wv, int lane)
{
    const int ko = c.t - c.nq - c.no;
    if (!(ko < 0 && c.t >= c.nq && wv < 4)) return -1;
    // (m, l) of the slot's 128 rows: 64 words per wave on waves 0-3, lane l -> word l
    const int w = wv * 64 + lane;
    const int row = imin(c.it.R0 + (c.t - c.nq) * kSlotRows + (w >> 1), c.it.R1 - 1);
    const size_t t = (size_t)c.it.b * a.T + c.it.r + (size_t)row * c.it.D;
    return (int64_t)((t * a.H + c.it.h) * 2 + (w & 1));
}

// Row (position) of query row `row` of an item in [B][T][H][d] terms: the
// output row of a dilated item, the query row itself of a band item.  The
// item's first row and the row step are apart so that a loop over the
// item's rows forms the first once.
__host__ __device__ __forceinline__ size_t item_out_row0(const AttnArgs& a, const ItemA& it)
{
    return ((size_t)it.b * a.T + it.r) * a.H + it.h;
}

__host__ __device__ __forceinline__ size_t item_out_row(const AttnArgs& a, const ItemA& it, size_t row0, int row)
{
    return row0 + (size_t)(row * it.D) * a.H;
}

// ---------------------------------------------------------------- host plan
// Prefill attention plan: heads grouped into (D, W) classes, the classes
// with the longest single items first, each class's levels most expensive
// first; `dil` holds every head's dilated items, `band` the raw-window band
// items of the classes with W > 0.  Returns false when there are more than
// kAttnMaxClasses classes or more than 2^31 items.
inline bool attn_plan(int B, int T, int H, const int* D, const int* W, float scale, int chunk, int n_cap,
                      int rows, AttnArgs& dil, AttnArgs& band)
{
    struct Cls { int D, W; std::vector<int> heads; double item_cost; };
    std::vector<Cls> cls;
    for (int h = 0; h < H; ++h) {
        auto it = std::find_if(cls.begin(), cls.end(), [&](const Cls& c) { return c.D == D[h] && c.W == W[h]; });
        if (it == cls.end()) {
            cls.push_back(Cls{D[h], W[h], {}, 0.0});
            it = cls.end() - 1;
        }
        it->heads.push_back(h);
    }
    if ((int)cls.size() > kAttnMaxClasses) return false;
    for (auto& c : cls) {
        const int Mmax = (T + c.D - 1) / c.D;
        c.item_cost = (double)std::min(Mmax, rows) * Mmax;
    }
    std::stable_sort(cls.begin(), cls.end(), [](const Cls& x, const Cls& y) { return x.item_cost > y.item_cost; });
    dil.B = B; dil.T = T; dil.H = H;
    dil.scale_log2 = scale * 1.4426950408889634f;
    dil.nclass = 0;
    dil.rows = rows;
    band = dil;
    dil.chunk = chunk;
    dil.n_cap = n_cap;  // states as a per-residue history (0: [B][T][H][d])
    int64_t items = 0, blocks = 0;
    int hoff = 0;
    for (const Cls& c : cls) {
        AttnClass& k = dil.cls[dil.nclass++];
        k.D = c.D; k.W = c.W;
        k.nheads = (int)c.heads.size(); k.head_off = hoff;
        for (int hh : c.heads) { dil.heads[hoff] = hh; band.heads[hoff] = hh; ++hoff; }
        const int Mmax = (T + c.D - 1) / c.D;
        k.levels = (Mmax + rows - 1) / rows;
        k.per_level = B * k.nheads * c.D;
        k.block_begin = (int)items;
        items += (int64_t)k.levels * k.per_level;
        if (c.W > 0) {
            AttnClass& kb = band.cls[band.nclass++];
            kb = k;
            kb.levels = (T + rows - 1) / rows;
            kb.per_level = B * k.nheads;
            kb.block_begin = (int)blocks;
            blocks += (int64_t)kb.levels * kb.per_level;
        }
        if (items >= ((int64_t)1 << 31) || blocks >= ((int64_t)1 << 31)) return false;
    }
    dil.nblocks = (int)items;
    band.nblocks = (int)blocks;
    return true;
}

// Rows per item of the two kernel shapes, and the residue length from which
// a plan runs on the long-item shape.  Eight waves on a five-slot ring (one
// workgroup per CU) software-pipeline the unmasked key tiles, which pays
// once residues are long; four waves on a two-slot ring run two workgroups
// per CU whose phases overlap, which pays on short residues and the band.
constexpr int kAttnRowsLong = 256;
constexpr int kAttnRowsShort = 128;
constexpr int kAttnLongResidue = 1024;

// The launches of a prefill attention: the raw-window band of every
// windowed class on the four-wave kernel, then every class in one launch,
// on the eight-wave kernel (`lng`) when some class has residues longer
// than kAttnLongResidue rows, else on the four-wave kernel (`sht`); the
// other of the two has no items.  (One launch keeps the short classes
// filling the long classes' tail.)  Returns false when attn_plan refuses
// the heads.
inline bool attn_launch_plans(int B, int T, int H, const int* D, const int* W, float scale, int chunk, int n_cap,
                              AttnArgs& lng, AttnArgs& sht, AttnArgs& band)
{
    AttnArgs unused;
    if (!attn_plan(B, T, H, D, W, scale, chunk, n_cap, kAttnRowsLong, lng, unused)) return false;
    if (!attn_plan(B, T, H, D, W, scale, chunk, n_cap, kAttnRowsShort, sht, band)) return false;
    bool any_long = false;
    for (int c = 0; c < lng.nclass; ++c) any_long |= (T + lng.cls[c].D - 1) / lng.cls[c].D > kAttnLongResidue;
    AttnArgs& idle = any_long ? sht : lng;
    idle.nclass = 0;
    idle.nblocks = 0;
    return true;
}

}  // namespace rat
