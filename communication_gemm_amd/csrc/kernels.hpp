// kernels.hpp -- arguments and launchers of the device kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "schedule.hpp"

namespace agg {

// Chunk producer: copies every remote shard's chunks into its workspace
// slot, then releases them one by one on the shard's counter.
struct ProducerArgs {
    Schedule s;
    const char* src[kMaxShards];   // shard base pointers
    char* dst[kMaxShards];         // workspace slot of each remote shard
    uint32_t* counters;            // header base; counter of shard i at i * 32
    uint32_t* flags;               // chunk flag matrix: [shard][kFlagCap]
    uint32_t* pieces;              // piece running totals: [shard][kFlagCap]
    uint32_t* piece_flags;         // [shard][kFlagCap][kPieceFlags], or nullptr: none
    int ppc;                       // pieces per chunk (the last chunk's may be empty)
    int64_t piece;                 // bytes per piece, a multiple of kWaveSweepBytes
    uint32_t* err;
    uint64_t* clock;               // pacing origin slot
    uint32_t base[kMaxShards];     // counter values at the start of the call
    uint32_t epoch;
    int elt;                       // bytes per element
    int64_t drop;                  // producer position whose release is withheld
    uint32_t delay_seed;           // test hook: each piece starts after a pseudo-random
    uint32_t delay_max;            // delay in [0, delay_max] ticks (0: none)
    double ticks_per_byte;         // pacing; 0 = unpaced
    uint64_t limit;                // wait limit in clock ticks
    uint64_t* trace;               // optional timestamps (see agg_options.trace)
    const uint32_t* start;         // pipelined mode: wait until it holds the epoch
                                   // (copy blockIdx % start_copies of it)
    int start_copies;
                                   // before reading a shard (nullptr: no wait)
    uint64_t start_limit;          // bound of that wait in clock ticks: the work
                                   // queued ahead of the call on the caller's
                                   // stream may take far longer than a chunk
    const uint64_t* stages;        // workspace ring: tiles finished per source and
                                   // stage, [shard][kMaxStages] (nullptr: no wait)
};

// Persistent consumer GEMM.
struct ConsumerArgs {
    Schedule s;
    const char* a[kMaxShards];     // rows of each shard: local in place, remote in the workspace
    const char* B;
    void* C;
    uint32_t* counters;
    const uint32_t* flags;         // chunk flag matrix
    const uint32_t* piece_flags;   // [shard][kFlagCap][kPieceFlags], or nullptr: none
    int ppc;                       // pieces per chunk, with piece_flags
    // paced calls with piece flags: a piece-flagged chunk counts only once
    // its paced time (clock ticks per 1024 elements, 16 fraction bits,
    // rounded up) has passed since the pacing origin in *clock; 0: unpaced
    uint32_t ticks_per_kib_q16;
    const uint64_t* clock;
    uint32_t* err;
    uint32_t base[kMaxShards];
    uint32_t epoch;
    int no_wait;                   // compute-only mode: take every chunk as ready
    uint64_t limit;
    // int8 path
    const int32_t* bias;
    const float* scale;
    int32_t* acc_out;
    uint64_t* trace;               // optional timestamps, consumer part
    uint64_t* trace_start;         // word 0 of the timestamps (call start)
    uint32_t* start;               // pipelined mode: set to the epoch on entry
                                   // (copy blockIdx % start_copies of it)
    int start_copies;
    uint64_t* stages;              // workspace ring: count each finished remote
                                   // tile on its stage (nullptr: no count)
    // split-K (s.ks > 1): partial sums, [tile][part][register][thread] of 4
    // bytes, and one ticket (running total of part weights) per tile
    char* partials;
    uint32_t* tickets;
};

hipError_t launch_producer(const ProducerArgs& a, int wgs, hipStream_t st);
hipError_t launch_consumer_f16(const ConsumerArgs& a, int tile_id, int wgs,
                               hipStream_t st);
hipError_t launch_consumer_i8(const ConsumerArgs& a, int tile_id, int wgs,
                              hipStream_t st);
hipError_t launch_consumer_bf16(const ConsumerArgs& a, int tile_id, int wgs,
                                hipStream_t st);
hipError_t launch_consumer_fp8(const ConsumerArgs& a, int tile_id, int wgs,
                               hipStream_t st);
hipError_t launch_header_reset(uint32_t* header, size_t bytes, hipStream_t st);
// Producer and consumer in one launch on `st`: `producers` producer
// workgroups, then `wgs` consumer workgroups (kind: 0 fp16, 1 int8, 2 bf16,
// 3 fp8).  Built for the tiles fused_built() names.
hipError_t launch_fused(int kind, const ConsumerArgs& c, const ProducerArgs& p, int tile_id,
                        int wgs, int producers, hipStream_t st);
bool fused_built(int kind, int tile_id);

// The allocation-free entry point's workspace: a file-scope device array of
// kScratchBytes per GPU.  scratch_address() gives its address on the
// current device (256-byte aligned).
constexpr size_t kScratchBytes = (size_t)64 << 20;
hipError_t scratch_address(void** out);

// Workgroups of a consumer tile shape that fit on one CU at once (kind:
// 0 fp16, 1 int8, 2 bf16, 3 fp8).
int consumer_occupancy(int kind, int tile_id);

}  // namespace agg
