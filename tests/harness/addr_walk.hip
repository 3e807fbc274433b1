// Host-side walk of the global addresses the RAT+ kernels form, over whole
// launch grids.  TEST INFRASTRUCTURE: compiled for the host only; it calls
// the same address functions (rat_plan.h) the kernels call and checks every
// access against the extent of the buffer it falls in.  It launches
// nothing and needs no GPU.
//
//   addr_walk B T H d L mode dtype n_cap w_cap fin D0,D1,.. W0,W1,..
//     mode: 0 RESTART, 1 SLIDING; dtype: 0 fp32, 1 bf16; n_cap 0: the
//     plain [B,T,H,d] state layout (no history); fin: 1 if the fp32 final
//     state is written.
// Prints one line per check and "OK" or the first failures; exit status 1
// on any out-of-range access.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <set>
#include <string>
#include <vector>

#include "rat_plan.h"

using namespace rat;

static long g_fail = 0;
static long g_checked = 0;

static void check(bool ok, const char* what, long long a, long long b, long long c)
{
    ++g_checked;
    if (!ok) {
        if (g_fail < 20) fprintf(stderr, "OUT OF RANGE: %s (%lld, %lld, %lld)\n", what, a, b, c);
        ++g_fail;
    }
}

static std::vector<int> parse_list(const char* s)
{
    std::vector<int> v;
    for (const char* p = s; *p;) {
        v.push_back(atoi(p));
        const char* q = strchr(p, ',');
        if (!q) break;
        p = q + 1;
    }
    return v;
}

// ---------------------------------------------------------------- scan
template <typename E, bool HIST, bool WIDE>
static void walk_scan(int B, int T, int H, int d, int L, int n_cap, bool fin, const std::vector<int>& D)
{
    constexpr int CPL = 16 / (int)sizeof(E);
    const ScanPlan p = scan_plan(B, T, H, d, L, sizeof(E) == 2);
    check(p.wide == WIDE, "scan geometry as the launcher picks it", T, L, p.wide);
    ScanFullArgs a;
    memset(&a, 0, sizeof(a));
    a.T = T; a.N = H * d; a.nblk = p.nblk; a.nseq = p.nseq; a.nchunk = p.nchunk;
    a.L = L >= T ? 0 : L; a.nwg = p.nwg; a.d = d;
    if (HIST) {
        a.hist.n_cap = n_cap; a.hist.d = d; a.hist.H = H;
        for (int h = 0; h < H; ++h) a.hist.D[h] = D[h];
    }
    const long long in_el = (long long)B * T * H * d;
    const long long hist_el = (long long)B * H * n_cap * d;
    const long long fin_el = (long long)B * H * 2 * d;
    std::vector<unsigned char> written(HIST ? (size_t)hist_el / CPL : 0, 0);
    for (uint32_t ticket = 0; ticket < (uint32_t)p.nwg; ++ticket) {
        for (int w = 0; w < kScanFullWaves; ++w) {
            for (int lane = 0; lane < 64; ++lane) {
                const ScanLane sl = scan_lane<CPL, ScanGeo<E, WIDE>::LPR>(a, ticket, w, lane);
                check((size_t)sl.chunk * a.nseq + sl.seq < (size_t)p.nwg, "scan workspace slot", ticket, w, lane);
                const size_t obase = ((size_t)sl.b * a.T + sl.t0) * a.N + sl.ch0;
                HistRow hr;
                size_t hbase = 0;
                if (HIST) {
                    hr.init(sl.t0, scan_hist_D(a, sl), a.hist.n_cap);
                    hbase = scan_hist_base(a, sl);
                }
                for (int i = 0; i < kScanTpl; ++i) {
                    const bool live = sl.cvalid && sl.t0 + i < T;
                    if (live) {
                        const long long o = (long long)(obase + (size_t)i * a.N);
                        check(o >= 0 && o + CPL <= in_el, "scan input row", ticket, lane, i);
                        if (HIST) {
                            const long long ho = (long long)(hbase + (size_t)hr.row() * a.d);
                            check(ho >= 0 && ho + CPL <= hist_el, "scan history store", ticket, lane, ho);
                            if (ho >= 0 && ho + CPL <= hist_el) {
                                check(written[ho / CPL] == 0, "history element written twice", ticket, lane, ho);
                                written[ho / CPL] = 1;
                            }
                        }
                        if (fin && sl.t0 + i == T - 1) {
                            const long long fo = (long long)scan_fin_offset(a, sl);
                            check(fo >= 0 && fo + a.d + CPL <= fin_el, "scan final state", ticket, lane, fo);
                        }
                    }
                    if (HIST) hr.next();
                }
            }
        }
    }
    if (HIST) {  // every position of every head written exactly once, where the decode step reads it
        long long n = 0;
        for (unsigned char x : written) n += x;
        check(n == in_el / CPL, "history elements written", n, in_el / CPL, 0);
        for (int b = 0; b < B; ++b)
            for (int h = 0; h < H; ++h)
                for (int t = 0; t < T; ++t) {
                    const long long row = (long long)(t % D[h]) * (n_cap / D[h]) + t / D[h];
                    const long long el = ((long long)(b * H + h) * n_cap + row) * d;
                    check(written[el / CPL] == 1, "history row of a position", b, h, t);
                }
    }
    printf("scan%s %s: %d chunks x 512 lanes\n", HIST ? " (history)" : "", sizeof(E) == 2 ? "bf16" : "fp32", p.nwg);
}

// ---------------------------------------------------------------- ring fill
static void walk_ring(int B, int T, int H, int d, int w_cap, const std::vector<int>& W, bool bf16)
{
    RingFillArgs r;
    memset(&r, 0, sizeof(r));
    r.B = B; r.T = T; r.H = H; r.d = d; r.w_cap = w_cap;
    for (int h = 0; h < H; ++h) r.W[h] = W[h];
    const int epv = bf16 ? 8 : 4;
    const size_t n = (size_t)B * H * w_cap * (d / epv);
    const size_t grid = (n + 255) / 256 * 256;  // the launch's threads
    long copies = 0;
    for (size_t idx = 0; idx < grid; ++idx) {
        size_t src, dst;
        if (!ring_fill_at(r, idx, epv, src, dst)) continue;
        ++copies;
        check(src + epv <= (size_t)B * T * H * d, "ring source", (long long)idx, (long long)src, 0);
        check(dst + epv <= (size_t)B * H * w_cap * d, "ring slot", (long long)idx, (long long)dst, 0);
    }
    printf("ring fill: %zu threads, %ld copies\n", grid, copies);
}

// ---------------------------------------------------------------- attention
template <int DK, int NW, int RING, bool BAND, bool CHUNK, bool HIST>
static void walk_attn(const AttnArgs& a, int grid, long long kv_bytes, const char* what)
{
    const long long row_bytes = (long long)a.B * a.T * a.H * DK * 2;  // q and out
    const long long tile = (long long)kSlotRows * DK * 2;
    const long long lds = RING > 4 ? RING * tile : RING * (tile + 1024);
    long steps = 0, items = 0, run_steps = 0;
    for (int blk = 0; blk < grid; ++blk) {
        CursorA<BAND, CHUNK, HIST> c;
        c.seek(a, 0, grid, blk);
        int issued = 0;
        int last_round = -1;
        // each wave's key run, kept as the kernel keeps it
        KeyRunA run[NW];
        bool run_ok[NW] = {};
        while (c.it.valid) {
            if (c.round != last_round) {
                ++items;
                last_round = c.round;
                for (int row = c.it.R0; row < c.it.R1; ++row) {
                    const long long orow = (long long)item_out_row(a, c.it, item_out_row0(a, c.it), row);
                    check(orow >= 0 && orow < (long long)a.B * a.T * a.H, "output row", blk, c.round, row);
                }
            }
            const uint32_t buf = (uint32_t)((issued % RING) * tile);
            for (int wv = 0; wv < NW; ++wv) {
                // the kernel's choice: the next tile of a key run, or the full plan
                StepCopiesA<DK, NW> full;
                step_copies_a<DK, NW>(a, c, wv, buf, full);
                if (run_ok[wv] && key_run_next_a<DK, NW>(c, run[wv])) {
                    ++run_steps;
                    check(full.whole && full.src == 2, "key run on a step that is no whole key tile", blk, c.t, wv);
                    for (int j = 0; j < StepCopiesA<DK, NW>::PER_WAVE; ++j)
                        check(key_run_rel_a<DK>(run[wv], j) == full.rel[j] && full.dp2 == run[wv].dp2,
                              "key run copy offset differs from the full plan", blk, c.t, j);
                } else {
                    run_ok[wv] = full.whole && step_key_tile_a(c) >= 0;
                    if (run_ok[wv]) run[wv] = KeyRunA{full.rel[0], full.dp2, full.row0, full.last};
                }
                for (int lane = 0; lane < 64; ++lane) {
                    uint32_t lq, col16;
                    dma_lane_a<DK>(lane, lq, col16);
                    StepCopiesA<DK, NW> s;
                    step_copies_a<DK, NW>(a, c, wv, buf, s);
                    const long long lim = s.src == 2 ? kv_bytes : row_bytes;
                    for (int j = 0; j < StepCopiesA<DK, NW>::PER_WAVE; ++j) {
                        const long long addr =
                            (long long)s.rel[j] + step_lane_offset_a<DK, NW>(s, wv, j, lq, col16);
                        check(addr >= 0 && addr + 16 <= lim, what, blk, c.t, addr);
                        check((long long)s.m0[j] + 16 * lane + 16 <= lds, "ring slot in LDS", blk, c.t, s.m0[j]);
                    }
                    const int64_t side_word = step_side_word_a(a, c, wv, lane);
                    if (side_word >= 0)
                        check(side_word < (long long)a.B * a.T * a.H * 2, "partial (m, l) word", blk, c.t,
                              side_word);
                }
            }
            ++issued;
            ++steps;
            c.advance(a, grid, blk);
        }
    }
    printf("%s: %d workgroups, %ld items, %ld ring steps (%ld wave steps as key runs)\n", what, grid, items, steps,
           run_steps);
}

// The kernel's ring schedule at step granularity: per item the waits
// (wait_tile(d): step consumed + d must have landed) and consumes the kernel
// makes, with one free slot refilled after each wait's barrier.  Checks that
// each awaited step has been issued by then, and that every issued step is
// consumed.
template <int NW, int RING, bool BAND, bool CHUNK, bool HIST>
static void walk_ring_schedule(const AttnArgs& a, int grid, const char* what)
{
    long waits = 0;
    for (int blk = 0; blk < grid; ++blk) {
        CursorA<BAND, CHUNK, HIST> issue, comp;
        issue.seek(a, 0, grid, blk);
        comp = issue;
        long issued = 0, consumed = 0;
        for (int j = 0; j < RING - 1 && issue.it.valid; ++j) {
            ++issued;
            issue.advance(a, grid, blk);
        }
        auto wait = [&](int d) {
            ++waits;
            check(issued > consumed + d, what, blk, consumed, d);
            if (issue.it.valid && issued < consumed + RING) {
                ++issued;
                issue.advance(a, grid, blk);
            }
        };
        while (comp.it.valid) {
            for (int s = 0; s < comp.nq + comp.no + (CHUNK ? comp.nown : 0); ++s) { wait(0); ++consumed; }
            int tt = 0;
            bool have = false;
            const int nfull = BAND ? 0 : std::min(comp.it.R0 / kTileA, comp.ntile - 1);
            if (!BAND && RING >= 3 && nfull > 0) {
                wait(0);
                for (; tt < nfull; ++tt) { wait(1); ++consumed; }
                have = true;
            }
            for (; tt < comp.ntile; ++tt) {
                if (!have) wait(0);
                have = false;
                ++consumed;
            }
            comp.seek(a, comp.round + 1, grid, blk);
        }
        check(consumed == issued, "every issued step consumed", blk, consumed, issued);
    }
    printf("%s: %ld waits, every awaited step issued in time\n", what, waits);
}

// Every (class, level, residue) of a plan is exactly one item: the item
// order is a permutation of the plan's work.
template <bool BAND, bool CHUNK>
static void check_items(const AttnArgs& a, const char* what)
{
    std::vector<char> seen;
    long long valid = 0;
    for (int c = 0; c < a.nclass; ++c) {
        const AttnClass& k = a.cls[c];
        seen.assign((size_t)k.levels * k.per_level, 0);
        for (int local = 0; local < k.levels * k.per_level; ++local) {
            const ItemA it = decode_item_a<BAND, CHUNK>(a, k.block_begin + local);
            // recover (level, idx) from the item: level from R0, idx from (b, head, residue)
            const int level = it.R0 / a.rows;
            int hslot = -1;
            for (int hh = 0; hh < k.nheads; ++hh)
                if (a.heads[k.head_off + hh] == it.h) hslot = hh;
            const long long idx = BAND ? (long long)it.b * k.nheads + hslot
                                       : ((long long)it.b * k.D + it.r) * k.nheads + hslot;
            const bool in = hslot >= 0 && level >= 0 && level < k.levels && idx >= 0 && idx < k.per_level;
            check(in, what, c, local, idx);
            if (!in) continue;
            char& s = seen[(size_t)level * k.per_level + idx];
            check(s == 0, "item decoded twice", c, local, idx);
            s = 1;
            valid += it.valid;
        }
        for (size_t q = 0; q < seen.size(); ++q) check(seen[q] == 1, "item never decoded", c, (long long)q, 0);
    }
    printf("%s: every item once (%lld with rows)\n", what, valid);
}

template <int DK>
static void walk_prefill_attn(int B, int T, int H, const std::vector<int>& D, const std::vector<int>& W, int n_cap)
{
    // the launches as the library makes them: the band pass on four-wave
    // workgroups (two per CU, two ring slots), the classes on eight-wave
    // workgroups (five slots, four with windows) when a residue is long,
    // else on four-wave ones
    AttnArgs lng, sht, band;
    memset(&lng, 0, sizeof(lng));
    sht = lng;
    if (!attn_launch_plans(B, T, H, D.data(), W.data(), 0.1f, 0, n_cap, lng, sht, band)) {
        printf("attention plan refused\n");
        ++g_fail;
        return;
    }
    AttnArgs all, unused;
    memset(&all, 0, sizeof(all));
    attn_plan(B, T, H, D.data(), W.data(), 0.1f, 0, n_cap, kAttnRowsShort, all, unused);
    long long short_rows = 0, all_rows = 0;  // query rows the short plan covers, against the whole plan's
    for (int c = 0; c < sht.nclass; ++c) short_rows += (long long)sht.cls[c].nheads * B * T;
    for (int c = 0; c < all.nclass; ++c) all_rows += (long long)all.cls[c].nheads * B * T;
    long long long_rows = 0;
    for (int c = 0; c < lng.nclass; ++c) long_rows += (long long)lng.cls[c].nheads * B * T;
    check(short_rows + long_rows == all_rows && (sht.nblocks == 0 || lng.nblocks == 0),
          "one of the two plans covers every head once", short_rows, long_rows, all_rows);
    bool windowed = false;
    for (int i = 0; i < lng.nclass; ++i) windowed |= lng.cls[i].W > 0;
    const long long raw_bytes = (long long)B * T * H * DK * 2;
    const long long kv_bytes = n_cap > 0 ? (long long)B * H * n_cap * DK * 2 : raw_bytes;
    const int cu = 256;
    check_items<true, false>(band, "band items");
    check_items<false, false>(lng, "eight-wave items");
    check_items<false, false>(sht, "four-wave items");
    if (band.nblocks > 0) {
        const int grid = std::min(band.nblocks, 2 * cu);
        walk_attn<DK, 4, 2, true, false, false>(band, grid, raw_bytes, "band pass copies");
        walk_ring_schedule<4, 2, true, false, false>(band, grid, "band pass ring");
    }
    if (lng.nblocks > 0) {
        const int grid = std::min(lng.nblocks, cu);
        if (n_cap > 0 && windowed) {
            walk_attn<DK, 8, 4, false, false, true>(lng, grid, kv_bytes, "eight waves (history, 4 slots)");
            walk_ring_schedule<8, 4, false, false, true>(lng, grid, "eight-wave ring (history, 4 slots)");
        } else if (n_cap > 0) {
            walk_attn<DK, 8, 5, false, false, true>(lng, grid, kv_bytes, "eight waves (history, 5 slots)");
            walk_ring_schedule<8, 5, false, false, true>(lng, grid, "eight-wave ring (history, 5 slots)");
        } else if (windowed) {
            walk_attn<DK, 8, 4, false, false, false>(lng, grid, kv_bytes, "eight waves (4 slots)");
            walk_ring_schedule<8, 4, false, false, false>(lng, grid, "eight-wave ring (4 slots)");
        } else {
            walk_attn<DK, 8, 5, false, false, false>(lng, grid, kv_bytes, "eight waves (5 slots)");
            walk_ring_schedule<8, 5, false, false, false>(lng, grid, "eight-wave ring (5 slots)");
        }
    }
    if (sht.nblocks > 0) {
        const int grid = std::min(sht.nblocks, 2 * cu);
        if (n_cap > 0) {
            walk_attn<DK, 4, 2, false, false, true>(sht, grid, kv_bytes, "four waves (history, 2 slots)");
            walk_ring_schedule<4, 2, false, false, true>(sht, grid, "four-wave ring (history)");
        } else {
            walk_attn<DK, 4, 2, false, false, false>(sht, grid, kv_bytes, "four waves (2 slots)");
            walk_ring_schedule<4, 2, false, false, false>(sht, grid, "four-wave ring");
        }
    }
    // the chunk grid (own-state steps, no windows) on the same shapes
    AttnArgs clng, csht, cband;
    memset(&clng, 0, sizeof(clng));
    csht = clng;
    std::vector<int> W0(H, 0);
    if (n_cap == 0 && attn_launch_plans(B, T, H, D.data(), W0.data(), 0.1f, 1, 0, clng, csht, cband)) {
        if (clng.nblocks > 0) {
            const int grid = std::min(clng.nblocks, cu);
            walk_attn<DK, 8, 5, false, true, false>(clng, grid, raw_bytes, "chunk grid, eight waves");
            walk_ring_schedule<8, 5, false, true, false>(clng, grid, "chunk grid ring, eight waves");
        }
        if (csht.nblocks > 0) {
            const int grid = std::min(csht.nblocks, 2 * cu);
            walk_attn<DK, 4, 2, false, true, false>(csht, grid, raw_bytes, "chunk grid, four waves");
            walk_ring_schedule<4, 2, false, true, false>(csht, grid, "chunk grid ring, four waves");
        }
    }
}

int main(int argc, char** argv)
{
    if (argc != 13) {
        fprintf(stderr, "usage: addr_walk B T H d L mode dtype n_cap w_cap fin D0,.. W0,..\n");
        return 2;
    }
    const int B = atoi(argv[1]), T = atoi(argv[2]), H = atoi(argv[3]), d = atoi(argv[4]), L = atoi(argv[5]);
    const int mode = atoi(argv[6]), dtype = atoi(argv[7]), n_cap = atoi(argv[8]), w_cap = atoi(argv[9]);
    const bool fin = atoi(argv[10]) != 0;
    const std::vector<int> D = parse_list(argv[11]), W = parse_list(argv[12]);
    if ((int)D.size() != H || (int)W.size() != H) {
        fprintf(stderr, "need H values of D and W\n");
        return 2;
    }
    const bool bf16 = dtype == 1;
    const bool full_or_restart = L >= T || mode == 0;
    if (full_or_restart) {
        const bool wide = scan_wide(T, L, bf16);
        if (n_cap > 0) {
            if (bf16 && wide) walk_scan<uint16_t, true, true>(B, T, H, d, L, n_cap, fin, D);
            else if (bf16) walk_scan<uint16_t, true, false>(B, T, H, d, L, n_cap, fin, D);
            else walk_scan<float, true, false>(B, T, H, d, L, n_cap, fin, D);
        } else {
            if (bf16 && wide) walk_scan<uint16_t, false, true>(B, T, H, d, L, 1, fin, D);
            else if (bf16) walk_scan<uint16_t, false, false>(B, T, H, d, L, 1, fin, D);
            else walk_scan<float, false, false>(B, T, H, d, L, 1, fin, D);
        }
    }
    bool any_w = false;
    for (int x : W) any_w |= x > 0;
    if (any_w && w_cap > 0) walk_ring(B, T, H, d, w_cap, W, bf16);
    if (bf16) {
        if (d == 128) walk_prefill_attn<128>(B, T, H, D, W, n_cap);
        else walk_prefill_attn<64>(B, T, H, D, W, n_cap);
    }
    printf("%ld accesses checked, %ld out of range\n", g_checked, g_fail);
    if (g_fail == 0) printf("OK\n");
    return g_fail ? 1 : 0;
}
