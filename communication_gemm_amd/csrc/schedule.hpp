// schedule.hpp -- the one schedule that drives both the chunk producer and
// the persistent consumer GEMM (PTO-ISA AllGather+GEMM README, optimisation
// notes: the communication side sends chunks in the order the compute side
// consumes them; the local row-group is computed first with no wait).
//
// Everything here is plain integer arithmetic usable on the host (planning,
// tests) and on the device (kernels map their position to work with it).
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define AGG_HD __host__ __device__ inline
#else
#define AGG_HD inline
#endif

namespace agg {

constexpr int kMaxShards = 64;

// Workspace header: one 32-bit summary counter per source shard, each on
// its own 128-byte line, then the error word, the pacing origin, the start
// word (the epoch of the last call whose consumer has started), the
// chunk flag matrix (one 32-bit word per source and chunk: the epoch of the
// call that released it), the piece counters (one 32-bit running total per
// source and chunk, to which every call adds exactly kPieceTotal in
// weighted piece counts; the region keeps 64-bit slots) and, for a
// bounded workspace, the stage counters (one
// 64-bit word per source and ring stage: the call's epoch above the number
// of tiles finished on that stage), then the split-K tickets.  The PTO-ISA
// README keeps the first
// two structures: per-chunk flags and a per-source summary counter.
constexpr int kCounterStride = 128;                       // bytes
constexpr int kErrorOffset = kMaxShards * kCounterStride; // uint32
constexpr int kClockOffset = kErrorOffset + kCounterStride; // uint64
constexpr int kStartOffset = kClockOffset + kCounterStride; // uint32
// The start word is kept in kStartCopies copies kStartStride bytes apart:
// consumer workgroup b writes copy b % copies and producer workgroup b
// polls copy b % copies, so the producer's first polls do not all queue
// on one memory channel.
constexpr int kStartCopies = 8;
constexpr int kStartStride = 896;
constexpr int kFlagOffset = 16384;
constexpr int kFlagCap = 1024;       // chunks per source the flag matrix holds
constexpr int kPieceOffset = kFlagOffset + kMaxShards * kFlagCap * 4;
constexpr int kMaxStages = 8;        // ring stages per source, at most
constexpr int kStageOffset = kPieceOffset + kMaxShards * kFlagCap * 8;
// Split-K tickets: one 32-bit running total per output tile, to which each
// K part adds its weight (piece_weight over ks parts); the part whose add
// completes the total sums the parts.
constexpr int kTicketOffset = kStageOffset + kMaxShards * kMaxStages * 8;
constexpr int kMaxSplitTiles = 4096;
// Piece flags: one 32-bit word per source, chunk and piece (at most
// kPieceFlags pieces a chunk), the epoch of the call whose piece's stores
// were performed.  Calls with three or more remote sources whose chunks
// have at most kPieceFlags pieces store them (not with one serial paced
// link), and a consumer may take a chunk whose piece flags are all set as
// released -- in a paced call once the chunk's paced time has passed --
// without waiting for the chunk flag that the last piece's running-total
// add leads to.
constexpr int kPieceFlags = 4;
constexpr int kPieceFlagOffset = kTicketOffset + kMaxSplitTiles * 4;
constexpr int kHeaderBytes = kPieceFlagOffset + kMaxShards * kFlagCap * kPieceFlags * 4;
static_assert(kStartOffset + kStartCopies * kStartStride <= kFlagOffset,
              "start word copies overlap the flag matrix");

// The producer copies a chunk in pieces, dealt to its waves in send order,
// so that a chunk is shared by many waves and all of them work on the
// earliest chunks first.  A wave moves 8 KiB per sweep (64 lanes x 8
// vectors of 16 bytes).  The planner's automatic piece is between one
// sweep and kPieceMax: in pipelined calls about kPiecesPerChunk pieces a
// chunk (chunks then land close to their send order, and one chunk's
// pieces do not all contend for its running total), in copy-only and
// sequential calls the copy's bytes over the producer's waves.
constexpr int kWaveSweepBytes = 8192;
constexpr int kPieceMax = 8 * kWaveSweepBytes;
constexpr int kPiecesPerChunk = 4;

// Completion of a chunk without a per-call reset: the pieces of a chunk add
// weights that sum to kPieceTotal, every weight at least 1, to the chunk's
// running total.  A call starts from a multiple of kPieceTotal (the header
// is zeroed when made and after a failed call), so exactly one add, the
// last, brings the total back to a multiple of it, whatever the order of
// the adds; modulo 2^32, which kPieceTotal divides, this still holds.
constexpr uint32_t kPieceTotal = 1u << 20;
constexpr int kMaxPiecesPerChunk = 1 << 18;   // weights stay >= 4

AGG_HD uint32_t piece_weight(int q, int ppc)
{
    const uint32_t w = kPieceTotal / (uint32_t)ppc;
    return q == ppc - 1 ? kPieceTotal - (uint32_t)(ppc - 1) * w : w;
}

struct Schedule {
    int n_shards;
    int local;             // shard read in place
    int link_model;        // 0 = parallel links, 1 = one serial link
    int cr;                // rows per chunk
    int cps;               // chunks per source: rcs row chunks x nkb K-blocks
    int rcs;               // row chunks per source, ceil(S / cr)
    int nkb;               // K-blocks per row chunk (1: a chunk spans all of K)
    int64_t kbk;           // elements of K per K-block (the last one also takes
                           // the remainder of K); K when nkb == 1
    int tm, tn;            // output tile
    int mt;                // m-tiles per shard
    int nt;                // n-tiles
    int64_t S, K, N;
    int order[kMaxShards]; // order[0] = local, order[1..n-1] = send order
    int slot[kMaxShards];  // workspace slot of each shard (-1: local)
    int xf;                // XCD blocking: n-tile groups per round (0 = none)
    int gm;                // grouped placement (when xf is 0): row panels per
                           // group, tiles column by column inside a group;
                           // 0 = list order
    int ring;              // workspace stages per remote source (0 = a full
                           // slot of S rows); stage g holds the row panel
                           // (m-tile) m with m % ring == g
    int pv;                // 0: per-source counters, local shard first.
                           // >= 1: the barrier scheme, iterations of pv
                           // m-tiles over every shard, each tile waiting
                           // for the whole iteration of every source
    int ks;                // K parts per output tile (split-K; 1 = none)
    int64_t kc;            // elements of K per part (a multiple of 256)
};

constexpr int kXcds = 8;   // XCDs; workgroup b of a grid runs on XCD b % 8

AGG_HD int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Row chunks of a source that m-tile `m` needs: the one holding the
// tile's last row, and all before it.
AGG_HD int need_chunks(const Schedule& s, int m)
{
    int64_t last = (int64_t)(m + 1) * s.tm;
    if (last > s.S) last = s.S;
    return (int)cdiv(last, s.cr);
}

// Chunks are K-block major inside a source: chunk j = kb * rcs + row chunk
// (a chunk of rows x all of K when nkb == 1).  Counter value that m-tile m
// needs before it reads K-block kb: every chunk of the K-blocks before kb,
// and the tile's row chunks of kb -- a prefix of the source's chunk order,
// so one monotonic counter per source still says it.
AGG_HD int need_at(const Schedule& s, int m, int kb)
{
    return kb * s.rcs + need_chunks(s, m);
}

// K-block of element k (the last K-block takes the remainder of K).
AGG_HD int kblock_of(const Schedule& s, int64_t k)
{
    const int64_t b = k / s.kbk;
    return b < s.nkb ? (int)b : s.nkb - 1;
}

// First element of K-block kb, and the first element after it.
AGG_HD int64_t kblock_begin(const Schedule& s, int kb) { return (int64_t)kb * s.kbk; }
AGG_HD int64_t kblock_end(const Schedule& s, int kb)
{
    return kb + 1 >= s.nkb ? s.K : (int64_t)(kb + 1) * s.kbk;
}

AGG_HD int64_t total_tiles(const Schedule& s)
{
    return (int64_t)s.n_shards * s.mt * s.ks * s.nt;
}

AGG_HD int64_t total_chunks(const Schedule& s)
{
    return (int64_t)(s.n_shards - 1) * s.cps;
}

// Index r of a run of `panels` row panels of nt tiles each -> (panel, n).
// List order is panel by panel; the grouped placement takes gm panels at a
// time and walks them column by column (n-tile after n-tile, the group's
// panels inside each), so that a stretch of consecutive positions covers a
// block of a few panels x a few n-tiles rather than one long panel.  Both
// are bijections of [0, panels * nt).
AGG_HD void group_decode(const Schedule& s, int64_t r, int64_t panels, int64_t* panel,
                         int64_t* n)
{
    if (s.gm <= 0) {
        *panel = r / s.nt;
        *n = r % s.nt;
        return;
    }
    const int64_t per_group = (int64_t)s.gm * s.nt;
    const int64_t g = r / per_group, w = r % per_group;
    const int64_t left = panels - g * s.gm;
    const int64_t gsz = left < s.gm ? left : s.gm;   // the last group may be short
    *panel = g * s.gm + w % gsz;
    *n = w / gsz;
}

struct TileRef {
    int shard;   // source shard of the A rows
    int m;       // m-tile within the shard
    int n;       // n-tile
    int need;    // counter value to wait for (0 = local, no wait)
    int kp;      // part of K (split-K; 0 otherwise)
};

// Consumer position p -> tile.  Local tiles first; then remote tiles in
// arrival order: with parallel links every source delivers its rows at the
// same time, so tiles go m-tile by m-tile across sources; with one serial
// link sources arrive one after the other.
//
// The barrier scheme (the Triton-distributed tutorial's comparison point:
// each iteration gathers pvalue row blocks of every rank, then a
// barrier_all, then every core computes the gathered block): iteration i
// holds m-tiles [i pv, (i + 1) pv) of every shard, in shard order, and each
// of its tiles, the local shard's included, waits until every remote source
// has delivered the iteration's last row.
AGG_HD TileRef tile_at(const Schedule& s, int64_t p)
{
    TileRef t;
    if (s.pv > 0) {
        const int64_t full = (int64_t)s.n_shards * s.pv * s.nt;   // tiles per iteration
        const int64_t i = p / full;
        const int64_t q = p - i * full;
        const int64_t m0 = i * s.pv;
        const int64_t cm = (s.mt - m0) < s.pv ? (s.mt - m0) : s.pv;   // m-tiles in it
        const int64_t per_shard = cm * s.nt;
        t.shard = (int)(q / per_shard);
        const int64_t r = q % per_shard;
        t.m = (int)(m0 + r / s.nt);
        t.n = (int)(r % s.nt);
        t.need = s.n_shards > 1 ? need_chunks(s, (int)(m0 + cm - 1)) : 0;
        t.kp = 0;   // the barrier scheme runs without split-K
        return t;
    }
    // Split-K: part after part, each part's tiles in the order below, so
    // that the row panels of one part (which read the same B rows) are
    // neighbours and share an XCD's L2.
    t.kp = 0;
    if (s.ks > 1) {
        const int64_t base = (int64_t)s.n_shards * s.mt * s.nt;
        t.kp = (int)(p / base);
        p -= (int64_t)t.kp * base;
    }
    int64_t local_tiles = (int64_t)s.mt * s.nt;
    int64_t panel, n;
    if (p < local_tiles) {
        group_decode(s, p, s.mt, &panel, &n);
        t.shard = s.local;
        t.m = (int)panel;
        t.n = (int)n;
        t.need = 0;
        return t;
    }
    int64_t q = p - local_tiles;
    int remotes = s.n_shards - 1;
    int src;
    if (s.link_model == 0) {
        // panels (m, source) in m-major order
        group_decode(s, q, (int64_t)s.mt * remotes, &panel, &n);
        t.m = (int)(panel / remotes);
        src = (int)(panel % remotes);
        t.n = (int)n;
    } else {
        int64_t per_src = (int64_t)s.mt * s.nt;
        src = (int)(q / per_src);
        group_decode(s, q % per_src, s.mt, &panel, &n);
        t.m = (int)panel;
        t.n = (int)n;
    }
    t.shard = s.order[1 + src];
    t.need = need_chunks(s, t.m);
    return t;
}

struct ChunkRef {
    int shard;   // source shard
    int src;     // its position in the send order (0-based over remotes)
    int j;       // chunk index within the shard: kb * rcs + jr
    int jr;      // row chunk: rows [jr * cr, min((jr + 1) * cr, S))
    int kb;      // K-block
};

// Producer position c -> chunk, in the order the consumer needs them.
// Parallel links: K-block after K-block (one K-block when chunks span all
// of K); inside a K-block, group g holds the row chunks first needed by
// m-tile g (row chunk j belongs to group j * cr / tm), every source in send
// order, row chunks ascending inside a source.  Group g starts at row chunk
// f = ceil(g tm / cr); as f * remotes <= c exactly when f <= c / remotes,
// the group of position c is the group of row chunk c / remotes.
// One serial link: source after source, each source's chunks in its own
// (K-block major) order.
// 32-bit arithmetic: positions stay below kMaxShards * kFlagCap, and
// j * cr below S (at most 2^30).
AGG_HD ChunkRef chunk_at(const Schedule& s, int64_t c64)
{
    ChunkRef r;
    const uint32_t remotes = (uint32_t)(s.n_shards - 1);
    const uint32_t cps = (uint32_t)s.cps, rcs = (uint32_t)s.rcs;
    const uint32_t cr = (uint32_t)s.cr, tm = (uint32_t)s.tm;
    if (c64 < 0 || remotes == 0 || c64 >= (int64_t)remotes * cps) {
        r.src = -1; r.j = -1; r.shard = -1; r.jr = -1; r.kb = -1;   // out of range
        return r;
    }
    const uint32_t c = (uint32_t)c64;
    if (s.link_model == 0) {
        const uint32_t per_kb = remotes * rcs;
        const uint32_t kb = c / per_kb;
        const uint32_t q = c - kb * per_kb;
        const uint32_t g = (q / remotes) * cr / tm;
        const uint32_t f = (g * tm + cr - 1) / cr;           // first row chunk of group g
        uint32_t e = ((g + 1) * tm + cr - 1) / cr;           // first row chunk after it
        if (e > rcs) e = rcs;
        const uint32_t gs = e - f;                           // row chunks per source in g
        const uint32_t rel = q - f * remotes;
        r.src = (int)(rel / gs);
        r.jr = (int)(f + rel % gs);
        r.kb = (int)kb;
    } else {
        r.src = (int)(c / cps);
        const uint32_t j = c % cps;
        r.kb = (int)(j / rcs);
        r.jr = (int)(j % rcs);
    }
    r.j = r.kb * s.rcs + r.jr;
    r.shard = s.order[1 + r.src];
    return r;
}

// ---- XCD-aware placement of consumer positions --------------------------
//
// The consumer runs in rounds: round r covers positions [rG, rG + G) of the
// tile list, one per workgroup (G = grid size).  A round is a set of row
// panels (one shard's m-tile, all nt n-tiles) taken in list order.  Each of
// the 8 XCDs has its own L2, and the workgroups of one XCD are b = x,
// x + 8, ...; so that they share A and B there, XCD x takes one block of
// the round: P/gp panels x nt/f n-tiles, with gp * f = 8.  Workgroups on
// one XCD move through K together, so a panel's slice is fetched into that
// L2 once for all of them.  Per round, A panels are then fetched f times
// and B panels gp times (instead of up to 8 times each).

// The n-tile split f for a grid of G workgroups (0 = keep list order):
// minimises f * P * tm + (8 / f) * nt * tn, the A and B rows fetched.
AGG_HD int pick_xcd_split(const Schedule& s, int64_t G)
{
    if (G < kXcds || G % kXcds != 0 || s.nt <= 0 || G % s.nt != 0) return 0;
    const int64_t P = G / s.nt;   // panels per round
    int best = 0;
    int64_t best_cost = 0;
    for (int f = 1; f <= kXcds; f *= 2) {
        const int gp = kXcds / f;
        if (s.nt % f != 0 || P % gp != 0) continue;
        const int64_t cost = (int64_t)f * P * s.tm + (int64_t)gp * s.nt * s.tn;
        if (best == 0 || cost < best_cost) {
            best = f;
            best_cost = cost;
        }
    }
    return best;
}

// Grouped placement, for the grids pick_xcd_split declines (rounds that do
// not hold whole panels, such as 107 n-tiles on 256 workgroups): XCD x
// takes the x-th stretch of G/8 consecutive positions of every round, and
// the tile list is walked in groups of gm panels, column by column
// (group_decode), so that stretch is a block of about gm panels x
// G/(8 gm) n-tiles.  gm minimises the A and B rows one stretch fetches,
// gm tm + (G / (8 gm)) tn, over the divisors of G/8 up to 16.  Not with a
// workspace ring (a group could need more panels than the ring holds), the
// barrier scheme or split-K, which keep list order.
AGG_HD int pick_group(const Schedule& s, int64_t G)
{
    if (s.xf > 0 || G < kXcds || G % kXcds != 0 || s.ring > 0 || s.pv > 0 || s.ks > 1 ||
        s.nt <= 0)
        return 0;
    const int64_t per = G / kXcds;
    int best = 0;
    int64_t best_cost = 0;
    for (int g = 1; g <= 16 && g <= per; ++g) {
        if (per % g != 0) continue;
        const int64_t cost = (int64_t)g * s.tm + (per / g) * s.tn;
        if (best == 0 || cost < best_cost) {
            best = g;
            best_cost = cost;
        }
    }
    return best;
}

// First position (within round 0) of workgroup b; it then takes that
// position plus multiples of G.  A permutation of [0, G) for every grid
// pick_xcd_split or pick_group accepted, the identity otherwise.
AGG_HD int64_t wg_position(const Schedule& s, int64_t b, int64_t G)
{
    if (s.gm > 0) return (b % kXcds) * (G / kXcds) + b / kXcds;
    const int f = s.xf;
    if (f <= 0) return b;
    const int64_t P = G / s.nt;
    const int gp = kXcds / f;
    const int64_t bp = P / gp;          // panels per XCD block
    const int64_t bn = s.nt / f;        // n-tiles per XCD block
    const int64_t x = b % kXcds, slot = b / kXcds;
    const int64_t g = x / f, h = x % f;
    const int64_t panel = g * bp + slot / bn;
    const int64_t n = h * bn + slot % bn;
    return panel * s.nt + n;
}

// Workspace row of source row `row` in its shard's slot.  A full slot
// keeps the shard's layout; a ring of `ring` panels of tm rows puts panel
// m in stage m % ring (chunks never straddle panels in that case).
AGG_HD int64_t slot_row(const Schedule& s, int64_t row)
{
    if (s.ring <= 0) return row;
    return ((row / s.tm) % s.ring) * s.tm + row % s.tm;
}

// Tiles finished on a ring stage that the producer must see before it
// writes panel m there: every tile of the panels that used the stage
// before (m - ring, m - 2 ring, ...).  0 for the first `ring` panels.
AGG_HD int64_t stage_tiles_before(const Schedule& s, int m)
{
    if (s.ring <= 0 || m < s.ring) return 0;
    return (int64_t)(m / s.ring) * s.nt;
}

// Rows of chunk j: [j*cr, min((j+1)*cr, S)).
AGG_HD int64_t chunk_row_end(const Schedule& s, int j)
{
    int64_t e = (int64_t)(j + 1) * s.cr;
    return e < s.S ? e : s.S;
}

// Bytes that must have crossed the emulated link before chunk r may be
// released: its own source's bytes up to the chunk's end in the source's
// order -- every row of the K-blocks before it, then its K-block's rows up
// to the chunk's last (parallel links) -- or everything sent before it on
// the one link too (serial).
AGG_HD int64_t paced_bytes(const Schedule& s, const ChunkRef& r, int elt)
{
    int64_t b = kblock_begin(s, r.kb) * s.S +
                chunk_row_end(s, r.jr) * (kblock_end(s, r.kb) - kblock_begin(s, r.kb));
    if (s.link_model != 0) b += (int64_t)r.src * s.S * s.K;
    return b * elt;
}

}  // namespace agg
