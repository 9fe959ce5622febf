// plan.hpp -- host-side argument checks and planning (no HIP calls).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "aggemm.h"
#include "schedule.hpp"

namespace agg {

enum Kind { kF16 = 0, kI8 = 1, kBF16 = 2, kFP8 = 3 };

// Bytes per element of A and B.
inline int elt_bytes(Kind k) { return (k == kI8 || k == kFP8) ? 1 : 2; }

struct TileShape {
    int id;         // 1-based id accepted by agg_options.tile
    int tm, tn;     // output tile
    int threads;    // workgroup size
    // Considered by the automatic choice (the others are alternative
    // pipelines of the same tile, selected by id only).
    bool auto_pick;
};

// A tile for split-K: 32 rows x 256 columns, so B is read in 256-element
// row segments.
constexpr int kSplitTile = 14;

// Output tiles the consumer kernels are built for, per path.
const TileShape* tile_shapes(Kind kind, int* count);

// Whether the fused kernel (producer and consumer in one launch) is built
// for a tile: four waves, like a producer workgroup, and at most 128 x 128
// outputs (the small calls whose time is launch cost).
inline bool fusable_tile(const TileShape& t) { return t.threads == 256 && t.tm * t.tn <= 128 * 128; }

struct Plan {
    Schedule sched;
    TileShape shape;
    int mode;
    double link_gbps;
    int consumer_wgs;
    int producer_wgs;
    int ppc;            // producer pieces per chunk
    int64_t piece;      // bytes per producer piece
    int elt;            // bytes per A element
    int64_t M;
    size_t slot_bytes;  // workspace bytes per remote shard (full slot or ring)
    size_t ws_bytes;    // workspace bytes this call needs
    size_t part_off;    // split-K partial sums: offset in the workspace
    int drop_chunk;
    int producer;       // enum agg_producer, as asked
    bool fused;         // pipelined: producer and consumer in one launch
    int producer_cus;   // CUs the pipelined producer is masked to (0: all)
};

// CU mask bits of a `cus`-CU producer set (32 or 64): bits 0 .. cus - 1.
// The driver deals a queue's mask bits round-robin over the XCDs (bit b on
// XCD b % 8, measured), so that is cus / 8 CUs on every XCD.  Smaller sets
// are not offered: with 8 to 24 CUs reserved, 5 to 19 of the remaining CUs
// could not take a 128 KiB-LDS workgroup at once on the masked queue
// (measured), which a workspace ring, whose producer waits for consumer
// tiles, cannot tolerate; with 32 or 64 all of them could.  words: 8 x 32
// bits.
void producer_cu_mask(int cus, uint32_t words[8]);

// Validate arguments and build the plan.  num_cus: CUs of the target device.
int make_plan(Kind kind, int n_shards, int64_t M, int64_t K, int64_t N,
              int chunk_rows, const agg_options* opt, int num_cus, Plan* out);

int pick_chunk_rows(int64_t shard_rows);
size_t workspace_bytes(int n_shards, int64_t M, int64_t K, int elt);

}  // namespace agg
