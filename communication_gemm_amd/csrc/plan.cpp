// plan.cpp -- argument checks, chunk size choice and the shared schedule.
// Host code only; no HIP calls, so it is testable without a GPU.
#include "plan.hpp"

#include <math.h>
#include <string.h>

namespace agg {

namespace {

// K-blocks of the automatic 2-D chunks: four, or eight for pipelined calls
// with three or more remote sources (make_plan).
constexpr int kAutoKBlocks = 4;
constexpr int kAutoKBlocksFine = 8;

// Output tiles the consumer kernels are instantiated for, largest first.
// Ids 1, 6, 7, 8 and 9 are the same 256 x 256 tile with different K
// pipelines and wave grids (see the Cfg table of the consumer); 8 (eight
// waves, two per SIMD, 128-byte slices) measured fastest on both paths,
// so it is the one picked automatically.  Ids 3, 12 and 13 are the 64 x 64
// tile; 13 (four 256-byte slices in the ring) keeps the most of a small
// tile's K in flight and measured fastest whenever a 64 x 64 tile is the
// choice, down to one tile per CU (small M).
// Apart from 8, 9, 10 and 11 all use 4 waves of 64 lanes.  The big tiles keep the MFMA pipes fed at
// large shapes; the smaller ones give enough tiles to fill 256 CUs and to
// follow the chunks as they arrive at smaller shapes.  Every one of these
// kernels, at its full occupancy, leaves registers, LDS and wave slots for
// producer waves on each CU (checked against the compiler's resource
// report by the test suite), so the producer always finds room beside a
// consumer grid that fills the chip.
// fp16 and bf16: the eight-wave half tiles come before the four-wave ones
// of the same size (at 2 x 1024 rows, K = N = 4096, id 11 ran 75 us
// compute-only against 96 us for id 4).
const TileShape kF16Shapes[] = {
    // 256 x 256 on 16 x 16 MFMA blocks: the same tile as id 8 at a higher
    // clock under the board's power limit (8 x 1024 rows, K = N = 4096,
    // compute-only: 226 against 240 us, fp16 and bf16 alike)
    {15, 256, 256, 512, true},
    {8, 256, 256, 512, false},
    {11, 128, 256, 512, true},
    {10, 256, 128, 512, true},
    {2, 128, 128, 256, true},
    {13, 64, 64, 256, true},
    {1, 256, 256, 256, false},
    {3, 64, 64, 256, false},
    {4, 256, 128, 256, false},
    {5, 128, 256, 256, false},
    {6, 256, 256, 256, false},
    {7, 256, 256, 256, false},
    {9, 256, 256, 512, false},
    {12, 64, 64, 256, false},
    {14, 32, 256, 256, false},
};
const TileShape kI8Shapes[] = {
    {8, 256, 256, 512, true},
    {4, 256, 128, 256, true},
    {5, 128, 256, 256, true},
    {2, 128, 128, 256, true},
    {13, 64, 64, 256, true},
    {1, 256, 256, 256, false},
    {3, 64, 64, 256, false},
    {6, 256, 256, 256, false},
    {7, 256, 256, 256, false},
    {9, 256, 256, 512, false},
    {10, 256, 128, 512, false},
    {11, 128, 256, 512, false},
    {12, 64, 64, 256, false},
    {14, 32, 256, 256, false},
    // id 8 on 16 x 16 blocks: it holds a higher clock but moves the same
    // operands, and the int8 slices are bound by that (2 x 8192 rows, K
    // 27392: 1566 against 1569 us); id 8 stays first
    {15, 256, 256, 512, false},
};
// fp8: the configurations whose slices hold whole 64-byte MFMA steps in
// pairs (128- or 256-byte slices).  Id 8 is left out: with 32-byte
// operands per lane, two steps' fragments and the 128 accumulators of a
// 128 x 64 wave block do not fit beside a producer wave; id 15 is that
// tile with one rolling operand set, and it is the automatic choice: on
// 8 x 1024 rows, K = N = 4096 it ran 118.6 / 127.9 us compute-only /
// pipelined against 124.4 / 134.4 for the four-wave id 6.
const TileShape kFP8Shapes[] = {
    {15, 256, 256, 512, true},
    {6, 256, 256, 256, false},
    {10, 256, 128, 512, true},
    {11, 128, 256, 512, true},
    {2, 128, 128, 256, true},
    {13, 64, 64, 256, true},
    {3, 64, 64, 256, false},
    {12, 64, 64, 256, false},
    {14, 32, 256, 256, false},
};

}  // namespace

const TileShape* tile_shapes(Kind kind, int* count)
{
    if (kind == kF16 || kind == kBF16) {   // bf16 runs the fp16 engine
        *count = (int)(sizeof(kF16Shapes) / sizeof(kF16Shapes[0]));
        return kF16Shapes;
    }
    if (kind == kFP8) {
        *count = (int)(sizeof(kFP8Shapes) / sizeof(kFP8Shapes[0]));
        return kFP8Shapes;
    }
    *count = (int)(sizeof(kI8Shapes) / sizeof(kI8Shapes[0]));
    return kI8Shapes;
}

void producer_cu_mask(int cus, uint32_t words[8])
{
    for (int i = 0; i < 8; ++i) words[i] = 0;
    for (int bit = 0; bit < cus && bit < 256; ++bit) words[bit / 32] |= 1u << (bit % 32);
}

int pick_chunk_rows(int64_t S)
{
    if (S < 1) return 0;
    int64_t cr = S / 64;          // ceil(S / cr) then lies in [64, 127]
    if (cr < 1) cr = 1;
    if (cr > (int64_t)0x7fffffff) cr = 0x7fffffff;
    return (int)cr;
}

static size_t slot_bytes(int64_t S, int64_t K, int elt)
{
    size_t b = (size_t)S * (size_t)K * (size_t)elt;
    return (b + 255) & ~(size_t)255;
}

size_t workspace_bytes(int n_shards, int64_t M, int64_t K, int elt)
{
    if (n_shards < 1 || n_shards > kMaxShards || M < 0 || K < 0 || elt < 1 ||
        M % n_shards)
        return 0;
    int64_t S = M / n_shards;
    return (size_t)kHeaderBytes + (size_t)(n_shards - 1) * slot_bytes(S, K, elt);
}

int make_plan(Kind kind, int n_shards, int64_t M, int64_t K, int64_t N,
              int chunk_rows, const agg_options* opt, int num_cus, Plan* out)
{
    agg_options def;
    ag_gemm_options_init(&def);
    if (!opt) opt = &def;
    if (opt->struct_size < sizeof(agg_options)) return AGG_E_INVALID;
    if (n_shards < 1) return AGG_E_INVALID;
    if (n_shards > kMaxShards) return AGG_E_UNSUPPORTED;
    if (M < 0 || K < 0 || N < 0) return AGG_E_INVALID;
    if (M % n_shards) return AGG_E_INVALID;
    const int64_t S = M / n_shards;
    if (chunk_rows < 0 || (S > 0 && chunk_rows > S)) return AGG_E_INVALID;
    const int kvec = 16 / elt_bytes(kind);      // elements per 16-byte load
    if (K % kvec || N % 8) return AGG_E_UNSUPPORTED;
    if (opt->local_shard < 0 || opt->local_shard >= n_shards) return AGG_E_INVALID;
    if (opt->mode < AGG_MODE_PIPELINED || opt->mode > AGG_MODE_COPY_ONLY)
        return AGG_E_INVALID;
    if (!(opt->link_gbps >= 0.0) || isinf(opt->link_gbps)) return AGG_E_INVALID;
    if (opt->link_model != AGG_LINKS_PARALLEL && opt->link_model != AGG_LINKS_SERIAL)
        return AGG_E_INVALID;
    if (opt->producer_wgs < 0 || opt->consumer_wgs < 0) return AGG_E_INVALID;
    if (opt->producer_piece_bytes < 0 || opt->producer_piece_bytes % kWaveSweepBytes)
        return AGG_E_INVALID;
    if (opt->k_splits < 0) return AGG_E_INVALID;
    if (!(opt->timeout_ms >= 0.0)) return AGG_E_INVALID;
    if (!(opt->debug_delay_us >= 0.0) || isinf(opt->debug_delay_us)) return AGG_E_INVALID;
    if (opt->producer < AGG_PRODUCER_KERNEL || opt->producer > AGG_PRODUCER_FUSED)
        return AGG_E_INVALID;
    if (opt->producer_cus < 0) return AGG_E_INVALID;
    const bool sdma = opt->producer == AGG_PRODUCER_SDMA;
    if (opt->producer_cus && ((opt->producer_cus != 32 && opt->producer_cus != 64) || sdma))
        return AGG_E_UNSUPPORTED;
    // the DMA engines copy whole ranges and cannot be paced or delayed
    if (sdma && (opt->link_gbps > 0.0 || opt->workspace_stages > 0 ||
                 opt->debug_drop_chunk >= 0 || opt->debug_delay_us > 0.0 ||
                 (opt->k_block > 0 && opt->k_block < K)))
        return AGG_E_UNSUPPORTED;
    if (num_cus <= 0) num_cus = 256;
    if (opt->producer_cus >= num_cus) return AGG_E_UNSUPPORTED;
    // Row and element offsets are formed in 64-bit; per-tile loop counters
    // in 32-bit.
    // The consumer addresses a tile's A rows, a slice's B rows and a
    // tile's output rows with 32-bit buffer offsets: 256 rows of K, 128
    // rows of N and 256 rows of N fp32 values must stay below 2^31 bytes.
    if (S > (1LL << 30) || K > (1LL << 21) || N > (1LL << 20))
        return AGG_E_UNSUPPORTED;

    Plan p;
    memset(&p, 0, sizeof p);
    Schedule& s = p.sched;
    s.n_shards = n_shards;
    s.local = opt->local_shard;
    s.link_model = opt->link_model;
    s.S = S;
    s.K = K;
    s.N = N;
    if (opt->workspace_stages < 0 || opt->workspace_stages > kMaxStages) return AGG_E_INVALID;
    if (opt->scheme != AGG_SCHEME_COUNTERS && opt->scheme != AGG_SCHEME_BARRIER)
        return AGG_E_INVALID;
    if (opt->pvalue < 0) return AGG_E_INVALID;
    // a ring needs the consumer running beside the producer to free its
    // stages (copy-only calls skip that wait, since nothing reads the rows)
    if (opt->workspace_stages > 0 && opt->mode == AGG_MODE_SEQUENTIAL)
        return AGG_E_UNSUPPORTED;

    // send order: a permutation of the remote shards
    for (int i = 0; i < kMaxShards; ++i) { s.order[i] = -1; s.slot[i] = -1; }
    s.order[0] = s.local;
    bool seen[kMaxShards] = {false};
    seen[s.local] = true;
    for (int q = 1; q < n_shards; ++q) {
        int id = opt->send_order ? opt->send_order[q - 1]
                                 : (s.local + q) % n_shards;
        if (id < 0 || id >= n_shards || seen[id]) return AGG_E_INVALID;
        seen[id] = true;
        s.order[q] = id;
        s.slot[id] = q - 1;
    }

    // output tile
    int count = 0;
    const TileShape* shapes = tile_shapes(kind, &count);
    const TileShape* pick = nullptr;
    if (opt->tile) {
        for (int i = 0; i < count; ++i)
            if (shapes[i].id == opt->tile) pick = &shapes[i];
        if (!pick) return AGG_E_INVALID;
    } else {
        // the largest tile that still gives every CU a tile (a full first
        // round), else the smallest: a bigger tile wins on MFMA efficiency
        // by more than a second round would gain in overlap
        const TileShape* smallest = nullptr;
        for (int i = 0; i < count && !pick; ++i) {
            if (!shapes[i].auto_pick) continue;
            int64_t tiles = (int64_t)n_shards * cdiv(S, shapes[i].tm) *
                            cdiv(N, shapes[i].tn);
            if (tiles >= num_cus) pick = &shapes[i];
            smallest = &shapes[i];
        }
        if (!pick) pick = smallest;
    }
    // Split-K, on request only.  On the decode-like int8 shape (2 x 32 rows,
    // K 16384, N 7168) it lost to the unsplit 64 x 64 tile (59-64 against
    // 50-55 us compute-only with 4 parts on the 32 x 256 tile), so the
    // automatic choice does not split.
    const bool can_split = opt->scheme == AGG_SCHEME_COUNTERS && opt->workspace_stages == 0 &&
                           S > 0 && K > 0 && N > 0;
    const int ks_req = opt->k_splits;
    s.ks = 1;
    s.kc = K;
    if (ks_req > 1) {
        // at most 64 parts: a tile's parts then span at most 2 MiB (32-bit
        // offsets in the kernel)
        if (ks_req > 64) return AGG_E_UNSUPPORTED;
        const int id = pick->id;
        if (!can_split || (id != 3 && id != 12 && id != 13 && id != kSplitTile))
            return AGG_E_UNSUPPORTED;
        if ((int64_t)n_shards * cdiv(S, pick->tm) * cdiv(N, pick->tn) > kMaxSplitTiles)
            return AGG_E_UNSUPPORTED;
        s.kc = cdiv(cdiv(K, ks_req), 256) * 256;
        s.ks = (int)cdiv(K, s.kc);
    }
    p.shape = *pick;
    s.tm = pick->tm;
    s.tn = pick->tn;
    s.mt = (int)cdiv(S, s.tm);
    s.nt = (int)cdiv(N, s.tn);

    // chunks, and the workspace ring
    s.cr = chunk_rows ? chunk_rows : pick_chunk_rows(S);
    if (s.cr < 1) s.cr = 1;
    s.ring = 0;
    if (opt->workspace_stages > 0 && (int64_t)opt->workspace_stages * s.tm < S) {
        // a chunk must lie inside one row panel of the ring
        if (chunk_rows == 0) {
            int d = s.cr < s.tm ? s.cr : s.tm;
            while (s.tm % d) --d;
            s.cr = d;
        } else if (s.tm % s.cr) {
            return AGG_E_UNSUPPORTED;
        }
        s.ring = opt->workspace_stages;
    }
    // K-blocks (2-D chunks): whole KiB of every row segment, so that the
    // producer's 1 KiB vectors never straddle two rows
    if (opt->k_block < 0) return AGG_E_INVALID;
    s.nkb = 1;
    s.kbk = K;
    const int64_t kib = 1024 / elt_bytes(kind);
    const bool two_d_ok = s.ring == 0 && opt->scheme == AGG_SCHEME_COUNTERS && s.ks == 1 &&
                          !sdma;
    if (opt->k_block > 0 && opt->k_block < K) {
        if (opt->k_block % kib || K % kib) return AGG_E_UNSUPPORTED;
        if (!two_d_ok) return AGG_E_UNSUPPORTED;
        s.kbk = opt->k_block;
        s.nkb = (int)(K / s.kbk);           // the last K-block takes the rest
    } else if (opt->k_block == 0 && chunk_rows == 0 && two_d_ok && K % (kAutoKBlocks * kib) == 0 &&
               n_shards > 1 && S > 0) {
        // Pipelined calls with three or more remote sources: eight K-blocks
        // where K allows.  A remote tile's first K-block of its rows is then
        // half the bytes, and a chunk of it (S/16 rows) half the sweeps of
        // a producer wave, so it lands sooner, paced or not: 8 x 1024 rows
        // at K = N = 4096 ran 239.7 against 243.0 us and 235.8 against
        // 238.0 (two boxes; 8 KiB or 16 KiB pieces alike, 128-row chunks
        // 240.8), and paced at 153 GB/s per link the 4 x 1024 rows below.
        // (With one remote source, 2 x 1024 rows at K = N = 4096 paced at
        // 153 GB/s, four K-blocks on every CU stayed ahead: 89.3-89.9
        // against 91.7 us.)
        const bool eight = opt->mode == AGG_MODE_PIPELINED && n_shards >= 4 &&
                           K % (kAutoKBlocksFine * kib) == 0;
        const int nkb = eight ? kAutoKBlocksFine : kAutoKBlocks;
        // Automatic chunks where K-blocks are allowed: S/16 rows x a quarter
        // of K, still 64 chunks per source (the PTO-ISA README's 64-128;
        // 128 with eight K-blocks).
        // Measured against whole-K chunks of S/64 rows (interleaved, one
        // box): 147 against 176 us on 4 x 1024 rows at K = N = 4096 paced at
        // 153 GB/s per link, level (277 / 279 us, 40 / 39 us) on 8 x 1024
        // rows at K = N = 4096 and on 2 x 1024 rows at K = 2048, N = 1024.
        s.kbk = K / nkb;
        s.nkb = nkb;
        s.cr = (int)(S / 16 > 0 ? S / 16 : 1);
    }
    s.rcs = S > 0 ? (int)cdiv(S, s.cr) : 0;
    if ((int64_t)s.rcs * s.nkb > kFlagCap && n_shards > 1) return AGG_E_UNSUPPORTED;
    s.cps = s.rcs * s.nkb;
    s.pv = opt->scheme == AGG_SCHEME_BARRIER ? (opt->pvalue > 0 ? opt->pvalue : 1) : 0;
    if (s.pv > s.mt) s.pv = s.mt > 0 ? s.mt : 1;
    // a tile of iteration i waits for every panel of the iteration, so a
    // ring must hold at least one iteration per source, or the producer
    // would wait for tiles that wait for it
    if (s.pv > 0 && s.ring > 0 && s.ring < s.pv) return AGG_E_UNSUPPORTED;
    // nor with one serial link: sources arrive one after the other, so the
    // producer would wait on a stage of the first source for tiles that
    // wait for the next source's rows
    if (s.pv > 0 && s.ring > 0 && s.link_model == AGG_LINKS_SERIAL) return AGG_E_UNSUPPORTED;
    // the producer moves a chunk with 32-bit buffer offsets
    if ((int64_t)s.cr * K * elt_bytes(kind) >= (1LL << 31)) return AGG_E_UNSUPPORTED;

    int64_t tiles = total_tiles(s);
    int64_t chunks = total_chunks(s);
    // with CUs reserved for the producer, the consumer grid covers the rest
    const int consumer_cus = opt->mode == AGG_MODE_PIPELINED ? num_cus - opt->producer_cus : num_cus;
    int cw = opt->consumer_wgs ? opt->consumer_wgs : consumer_cus;
    if (cw > tiles) cw = (int)(tiles > 0 ? tiles : 1);
    if (cw < 1) cw = 1;
    // pieces per chunk (the largest chunk: the last K-block's)
    const int64_t chunk_bytes =
        (int64_t)s.cr * (kblock_end(s, s.nkb - 1) - kblock_begin(s, s.nkb - 1)) * elt_bytes(kind);
    // Automatic piece, in whole sweeps, between one sweep and kPieceMax.
    // Pipelined: about kPiecesPerChunk pieces a chunk, so that chunks land
    // close to their send order (the consumer takes them as they land)
    // while one chunk's pieces do not all contend for its running total.
    // Copy-only and sequential calls, where nothing waits for the order:
    // the copy's bytes over the producer's waves, the best throughput.
    int64_t piece = opt->producer_piece_bytes;
    if (!piece) {
        const int64_t waves = 4 * (int64_t)(opt->producer_wgs ? opt->producer_wgs : num_cus);
        const bool pipelined = opt->mode == AGG_MODE_PIPELINED;
        const int64_t want = pipelined ? cdiv(chunk_bytes, kPiecesPerChunk)
                                       : cdiv(chunks * chunk_bytes, waves);
        piece = cdiv(want, kWaveSweepBytes) * kWaveSweepBytes;
        // copy-only and sequential: a power-of-two number of sweeps, which
        // divides the chunks that are powers of two (no short tail piece)
        if (!pipelined) {
            int64_t p2 = kWaveSweepBytes;
            while (p2 < piece) p2 *= 2;
            piece = p2;
        }
        if (piece > kPieceMax) piece = kPieceMax;
        if (piece < kWaveSweepBytes) piece = kWaveSweepBytes;
    }
    const int64_t ppc64 = chunk_bytes > 0 ? cdiv(chunk_bytes, piece) : 1;
    if (ppc64 > kMaxPiecesPerChunk) return AGG_E_UNSUPPORTED;
    const int ppc = (int)ppc64;
    const int64_t items = chunks * ppc;
    const int producer_cus =
        opt->mode == AGG_MODE_PIPELINED && opt->producer_cus ? opt->producer_cus : num_cus;
    // Automatic producer grid: every CU, except in an unpaced pipelined
    // call on all CUs, where half of them.  There the copy is far shorter
    // than the GEMM and fewer producer waves take fewer issue slots and
    // memory requests from the consumer beside them: 8 x 1024 rows, K = N =
    // 4096 ran 249 us pipelined with 128 producer workgroups against 258
    // with 256, the int8 2 x 8192 x 27392 x 4096 call 1580 against 1603 us;
    // the first chunk lands no later (about 12 us after the consumer starts
    // either way) and the small shapes did not change.  A paced producer
    // keeps every CU: a wave waiting for its chunk's paced time holds back
    // its next pieces, and fewer waves fell behind the pace -- except with
    // the automatic paced chunks of eight K-blocks, where a quarter of the
    // CUs still keep up with the pace (the last chunk of 4 x 1024 rows at
    // K = N = 4096, 153 GB/s per link, lands at 61 us against 55 by the
    // pace) and take less from the consumer: 124.1-126.9 us pipelined
    // against 128.5-134.4 with four K-blocks on every CU (three boxes);
    // eight K-blocks on every CU took 136.1-138.1 us, and on 8 x 1024 rows
    // the quarter grid changed nothing (239-240 us, mesh or ring).
    int pw = opt->producer_wgs ? opt->producer_wgs : producer_cus;
    if (!opt->producer_wgs && opt->mode == AGG_MODE_PIPELINED && !opt->producer_cus &&
        opt->producer != AGG_PRODUCER_SDMA && num_cus >= 4) {
        if (!(opt->link_gbps > 0.0))
            pw = num_cus / 2;
        else if (s.nkb == kAutoKBlocksFine && opt->k_block == 0 && chunk_rows == 0)
            pw = num_cus / 4;
    }
    if (pw > items) pw = (int)(items > 0 ? items : 1);
    if (pw < 1) pw = 1;
    // One launch for both (pipelined): by default when the consumer's tile
    // has a fused build and the two grids fit on the CUs together, each
    // workgroup on a CU of its own -- the calls that leave most of the
    // device idle, whose time is the launches'.  An automatic producer
    // grid is then rounded up to whole multiples of 8 workgroups, so the
    // consumer's workgroups, which follow them in the grid, keep their
    // XCDs (workgroup b runs on XCD b mod 8).
    bool fused = false;
    if (opt->mode == AGG_MODE_PIPELINED &&
        (opt->producer == AGG_PRODUCER_KERNEL || opt->producer == AGG_PRODUCER_FUSED)) {
        const bool can = fusable_tile(p.shape) && s.ring == 0 && !opt->producer_cus;
        if (opt->producer == AGG_PRODUCER_FUSED && !can) return AGG_E_UNSUPPORTED;
        const int pw_fused = opt->producer_wgs ? pw : (pw + 7) / 8 * 8;
        fused = can && (opt->producer == AGG_PRODUCER_FUSED || cw + pw_fused <= num_cus);
        if (fused) pw = pw_fused;
        // The separate producer kernel on every CU waits for the consumer's
        // start word, and a consumer workgroup needs all but one producer
        // wave's registers of each SIMD: more producer workgroups than CUs
        // could take every CU's room before any consumer workgroup starts
        // (the producers would then wait out their start bound), or leave
        // producer workgroups, and the chunks they copy, queued behind a
        // consumer grid that waits for those chunks.  One producer
        // workgroup per CU at most: workgroups are dealt to the XCDs in
        // turn, so no XCD gets more of them than it has CUs, and each
        // XCD keeps room for consumer workgroups to start.
        if (!fused && !opt->producer_cus && pw > num_cus) return AGG_E_UNSUPPORTED;
    }
    p.consumer_wgs = cw;
    p.producer_wgs = pw;
    p.ppc = ppc;
    p.piece = piece;
    p.mode = opt->mode;
    p.link_gbps = opt->link_gbps;
    p.elt = elt_bytes(kind);
    p.M = M;
    p.slot_bytes = slot_bytes(s.ring > 0 ? (int64_t)s.ring * s.tm : S, K, p.elt);
    p.ws_bytes = (size_t)kHeaderBytes + (size_t)(n_shards - 1) * p.slot_bytes;
    p.part_off = p.ws_bytes;
    if (s.ks > 1) {
        // partial sums: every part of every tile, tm x tn values of 4 bytes
        p.ws_bytes += (size_t)((int64_t)n_shards * s.mt * s.nt * s.ks * s.tm * s.tn * 4);
    }
    p.drop_chunk = opt->debug_drop_chunk;
    p.producer = opt->producer;
    p.fused = fused;
    p.producer_cus = opt->mode == AGG_MODE_PIPELINED ? opt->producer_cus : 0;
    *out = p;
    return AGG_OK;
}

}  // namespace agg

extern "C" {

void ag_gemm_options_init(agg_options* opt)
{
    if (!opt) return;
    memset(opt, 0, sizeof *opt);
    opt->struct_size = sizeof(agg_options);
    opt->local_shard = 0;
    opt->send_order = nullptr;
    opt->mode = AGG_MODE_PIPELINED;
    opt->link_gbps = 0.0;
    opt->link_model = AGG_LINKS_PARALLEL;
    opt->debug_drop_chunk = -1;
}

int ag_gemm_pick_chunk_rows(int64_t shard_rows)
{
    return agg::pick_chunk_rows(shard_rows);
}

size_t ag_gemm_workspace_bytes(int n_shards, int64_t M, int64_t K, int elt_bytes)
{
    return agg::workspace_bytes(n_shards, M, K, elt_bytes);
}

const char* ag_gemm_status_string(int status)
{
    switch (status) {
    case AGG_OK: return "ok";
    case AGG_E_INVALID: return "invalid argument";
    case AGG_E_UNSUPPORTED: return "unsupported shape or alignment";
    case AGG_E_NOMEM: return "out of device memory";
    case AGG_E_HIP: return "HIP runtime error";
    case AGG_E_TIMEOUT: return "counter wait timed out";
    case AGG_E_TOO_LARGE: return "workspace needed exceeds the allocation-free entry point's scratch";
    default: return "unknown status";
    }
}

int ag_gemm_plan(int kind, int n_shards, int64_t M, int64_t K, int64_t N,
                 int chunk_rows, const agg_options* opt, int num_cus,
                 agg_plan_info* info, int32_t* tile_order, int32_t* chunk_order)
{
    if (kind < 0 || kind > 3) return AGG_E_INVALID;
    agg::Plan p;
    int rc = agg::make_plan(static_cast<agg::Kind>(kind), n_shards, M, K,
                            N, chunk_rows, opt, num_cus, &p);
    if (rc) return rc;
    // the placement the launch picks for a grid of consumer_wgs workgroups
    agg::Schedule s = p.sched;
    s.xf = agg::pick_xcd_split(s, p.consumer_wgs);
    s.gm = agg::pick_group(s, p.consumer_wgs);
    if (info) {
        info->shard_rows = s.S;
        info->chunk_rows = s.cr;
        info->chunks_per_source = s.cps;
        info->tile_m = s.tm;
        info->tile_n = s.tn;
        info->m_tiles_per_shard = s.mt;
        info->n_tiles = s.nt;
        info->total_tiles = agg::total_tiles(s);
        info->total_chunks = agg::total_chunks(s);
        info->consumer_wgs = p.consumer_wgs;
        info->producer_wgs = p.producer_wgs;
        info->tile_id = p.shape.id;
        info->trace_words = 1 + agg::total_chunks(s) + 3 * agg::total_tiles(s);
        info->workspace_stages = s.ring;
        info->workspace_bytes = (int64_t)p.ws_bytes;
        info->k_splits = s.ks;
        info->k_blocks = s.nkb;
        info->k_block = s.kbk;
        info->producer_fused = p.fused ? 1 : 0;
    }
    if (tile_order) {
        int64_t T = agg::total_tiles(s);
        for (int64_t i = 0; i < T; ++i) {
            agg::TileRef t = agg::tile_at(s, i);
            tile_order[4 * i + 0] = t.shard;
            tile_order[4 * i + 1] = t.m;
            tile_order[4 * i + 2] = t.n;
            tile_order[4 * i + 3] = t.need;
        }
    }
    if (chunk_order) {
        int64_t C = agg::total_chunks(s);
        for (int64_t i = 0; i < C; ++i) {
            agg::ChunkRef c = agg::chunk_at(s, i);
            chunk_order[2 * i + 0] = c.shard;
            chunk_order[2 * i + 1] = c.j;
        }
    }
    return AGG_OK;
}

}  // extern "C"
