// producer_body.hpp -- the chunk producer's device code: plays the links of
// an AllGather on one GPU.  For every remote shard it moves chunk after chunk (chunk_rows
// rows x all of K) from the shard into the shard's workspace slot and
// publishes it (PTO-ISA AllGather+GEMM README: the communication kernel
// transfers a chunk, then notifies with an atomic add on the per-source
// summary counter; several communication blocks per destination; chunks
// sent in the order they are consumed).
//
// Each chunk is cut into pieces (8-32 KiB, planned); piece q of producer
// position c is item c * P + q, and wave w of the producer grid copies items
// w, w + W, w + 2W, ..., so every wave works on the earliest chunks first
// and chunks complete in about the order they are sent.  Waves run on
// their own, with no workgroup barrier after the start.  A finished chunk
// is published in three steps, none of which waits for another wave:
//   * each piece's wave waits until its device-scope (write-through) stores
//     are performed in memory, then adds the piece's weight to the chunk's
//     running total; the add that completes the chunk's total is the last;
//   * that wave stores the call's epoch in the chunk's flag (the chunk flag
//     matrix);
//   * the wave then advances the source's summary counter over every
//     flagged chunk contiguous with it (64 flags per read, one lane each),
//     in one compare-and-swap.
// So a counter value c means "chunks 0..c-1 are flagged", and the counter
// moves as soon as the lowest missing chunk lands, whoever copied it.  The
// consumer waits on the counter, then reads the flags of the chunks it
// needs and acquires (invalidating what its caches may hold of the
// workspace): a flag it sees was stored after the chunk's data reached
// memory.  Counter and flags are updated with relaxed device-scope
// atomics only, and the producer does no cache maintenance at all.
//
// A wave's memory operations are waited for at one point per sweep, where
// its loads must land before they are stored: the stores of the previous
// piece are complete there too, so the piece's add is issued then, and its
// result is looked at the next such point.  Copy, count and release of
// consecutive pieces thus overlap instead of queueing.
//
// Pacing: with ticks_per_byte > 0 a chunk is not flagged before the
// emulated link could have carried it (parallel links: its own source's
// bytes up to and including the chunk; serial link: everything sent before
// it too), measured from the moment the first producer workgroup started.
//
// The code is shared by the producer kernel (its own grid, on a stream of
// its own) and by the fused kernel of the consumer (the first workgroups of
// the consumer's grid, in one launch); `block` and `blocks` are the
// workgroup's index among the producer workgroups and their number.
#pragma once

#include "kernels.hpp"
#include "sync.hpp"

namespace agg {
namespace {
namespace prod {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(4 * sizeof(unsigned int)))) unsigned int v4u32;

constexpr int kProducerThreads = 256;
constexpr int kProducerWaves = kProducerThreads / 64;
constexpr int kRsrcWord3 = 0x00020000;   // untyped 32-bit buffer accesses
// Cache policy of the copy's loads and stores: device scope.  The loads
// read what is coherent at that scope (no stale cached line of a shard);
// the stores are written through, so that their completion alone
// publishes them.
constexpr int kDevice = 16;
constexpr int kUnroll = 8;               // 16-byte vectors in flight per lane
constexpr int kLaneStep = 64 * 16;       // bytes per vector across a wave
static_assert(kUnroll * kLaneStep == kWaveSweepBytes, "sweep size");

// Advance the summary counter of one source over the flagged chunks that
// follow it, a wave at a time: lane i reads the flag i places past the
// counter, and the run of set flags from lane 0 on is how far the counter
// can move (one memory round trip per 64 flags, where a single lane walking
// them paid one per flag).  Runs after the wave's own flag store has been
// performed at device scope.  Two waves racing: the compare-and-swap lets
// one win and the other re-read; a flag stored before a wave reads the
// counter is seen either by that wave or by the wave that moved the counter
// past the chunk before it.
__device__ void advance(uint32_t* ctr, const uint32_t* flags, uint32_t base, int cps,
                        uint32_t epoch, int lane)
{
    for (;;) {
        const uint32_t cur = __builtin_amdgcn_readfirstlane(load_agent(ctr));
        const int i = (int)(cur - base) + lane;
        const bool set = i < cps && load_agent(flags + i) == epoch;
        const uint64_t run = __builtin_amdgcn_ballot_w64(set);
        const int k = run == ~0ull ? 64 : __builtin_ctzll(~run);
        if (k == 0) return;
        uint32_t won = 0;
        if (lane == 0) {
            uint32_t want = cur;
            won = __hip_atomic_compare_exchange_strong(ctr, &want, cur + (uint32_t)k,
                                                       __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
        }
        // Done once the counter moved over a run that ended at an unset
        // flag: whoever sets it advances past it (by the argument above).
        // Otherwise (a lost swap, or all 64 flags set) look again.
        if (__builtin_amdgcn_readfirstlane(won) && k < 64) return;
    }
}

// Test hook: a pseudo-random delay for item `item` (a hash of the seed
// and the item: 32-bit multiply-xorshift mixing), so that pieces, and with
// them chunks, complete in an order unrelated to the send order.
__device__ __forceinline__ uint32_t item_delay(uint32_t seed, uint32_t item, uint32_t max)
{
    uint32_t h = seed * 0x9E3779B9u ^ item;
    h ^= h >> 16;
    h *= 0x7FEB352Du;
    h ^= h >> 15;
    h *= 0x846CA68Bu;
    h ^= h >> 16;
    return h % (max + 1u);
}

__device__ __forceinline__ int32_t uniform(int32_t x)
{
    return __builtin_amdgcn_readfirstlane(x);
}

__device__ __forceinline__ void* uniform_ptr(const void* p)
{
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Release chunk c (the wave whose add completed it): wait for the emulated
// link if paced, stamp, flag (lane 0), advance the summary counter (the
// whole wave).
__device__ void release_chunk(const ProducerArgs& a, int64_t c, uint64_t origin, int lane)
{
    const ChunkRef r = chunk_at(a.s, c);
    if (a.ticks_per_byte > 0.0) {
        const double b = (double)paced_bytes(a.s, r, a.elt);
        const double delta = b * a.ticks_per_byte;
        // a pace slower than the wait limit is a failed call, not a hang
        if (delta > (double)a.limit) {
            if (lane == 0) raise_error(a.err, a.epoch);
            return;
        }
        wait_until(origin, (uint64_t)delta);
    }
    uint32_t* flags = a.flags + r.shard * kFlagCap;
    if (lane == 0) {
        // stamped before the flag, so a consumer that saw the flag started
        // after this time
        if (a.trace) a.trace[1 + c] = ticks();
        __hip_atomic_store(flags + r.j, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // the flag store is performed before the counter is read
    __builtin_amdgcn_s_waitcnt(0);
    advance(a.counters + r.shard * (kCounterStride / 4), flags, a.base[r.shard], a.s.cps,
            a.epoch, lane);
}

// Workgroup-shared state of a producer workgroup.  Declared by each kernel
// that runs the producer and handed in, so that every LDS variable belongs
// to one kernel.
struct ProducerShared {
    uint64_t origin;
    int stop;
};

// The producer: workgroup `block` of `blocks`, four waves each.
__device__ __forceinline__ void produce(const ProducerArgs& a, uint32_t block, uint32_t blocks,
                                        ProducerShared& sh)
{
    const Schedule& s = a.s;
    const int64_t chunks = total_chunks(s);
    const int64_t row_bytes = s.K * a.elt;
    uint64_t& origin_sh = sh.origin;
    int& stop_sh = sh.stop;

    // Producer waves share their SIMDs with consumer waves; they issue few
    // instructions, each of which the consumer is waiting on, so they go
    // first when both are ready.
    __builtin_amdgcn_s_setprio(3);
    // Pipelined mode: this kernel runs on a stream of its own with no
    // dependency on the caller's stream, so it must not read a shard
    // before the work queued ahead of the call has finished.  The consumer
    // runs on the caller's stream, so its start proves that; each of its
    // workgroups writes the call's epoch to the start word on entry.
    // The shards were written before the consumer started, but this kernel
    // may have been resident since before that, and the caches of its CU
    // and XCD may hold lines of an earlier call's shards: the copy's loads
    // are device-scope loads, which are coherent at that scope and take no
    // such line (so no cache invalidation, which cost the consumer its
    // cached panels, is needed here).
    // The bound of this wait is its own, far above a chunk's: it covers
    // whatever the caller queued ahead of the call.  In the consumer's
    // grid (one launch on the caller's stream) there is no start word:
    // stream order alone puts the work ahead of the call before it.
    // "Reached" (at least the epoch, modulo 2^32), not "equal": a workgroup
    // with no item of its own may still be here when the next call's
    // consumer has written a later epoch, and it must then pass.  Stale
    // contents of a fresh or reused workspace cannot be read here: the
    // reset that zeroes the header is ordered before this stream's next
    // work (ag_gemm_workspace_reset and the internal allocation both do
    // that).
    if (a.start) {
        if (threadIdx.x == 0)
            stop_sh = !reached(poll_until(a.start + (block % a.start_copies) *
                                                        (kStartStride / 4),
                                          a.epoch, a.err, a.epoch, a.start_limit),
                               a.epoch);
        __syncthreads();
        if (stop_sh) return;
    }
    if (threadIdx.x == 0) {
        origin_sh = a.ticks_per_byte > 0.0 ? pacing_origin(a.clock, a.epoch) : 0;
        stop_sh = 0;
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int64_t waves = (int64_t)blocks * kProducerWaves;
    const int32_t lane_off = lane * 16;

    // Piece bookkeeping of this wave (uniform across its lanes): `pend`,
    // the chunk of the piece whose stores were issued last and are not
    // counted yet (-1: none), with its running total and weight; `cnt`,
    // the chunk of the piece whose add is in flight (-1: none), with its
    // weight.  `old` is the running total the add returned (lane 0).
    // (Positions and total indices fit 32 bits: at most kMaxShards x
    // kFlagCap chunks.)
    int32_t pend = -1, cnt = -1;
    uint32_t pend_total = 0, pend_w = 0, pend_q = 0, cnt_w = 0, old = 0;

    // The piece being copied: item chunk * ppc + q (producer position
    // `chunk`, piece q of it), stepped by `waves` items without dividing;
    // its running total and weight, its bytes and descriptors, and the
    // next sweep's offset.
    const int64_t first = (int64_t)block * kProducerWaves +
                          __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t ppc = (uint32_t)a.ppc;
    const int32_t nchunks = (int32_t)chunks;
    // steps past the last chunk are clamped: the wave is done then anyway
    const int64_t sc = waves / ppc;
    const int32_t step_c = sc < nchunks ? (int32_t)sc : nchunks;
    const uint32_t step_q = (uint32_t)(waves % ppc);
    const int64_t c0 = first / ppc;
    int32_t chunk = c0 < nchunks ? (int32_t)c0 : nchunks;
    uint32_t q = (uint32_t)(first % ppc);
    uint32_t total = 0, weight = 0;
    int32_t n = 0, off = 0;
    const char* src = nullptr;
    char* dst = nullptr;
    // A chunk of one K-block (2-D chunks) is `rows` row segments of `seg`
    // bytes, row_bytes apart in the shard and in the slot alike; a piece is
    // bytes [begin, begin + n) of the chunk taken segment after segment.
    // seg == 0: the chunk spans all of K, so it is contiguous and src/dst
    // point at the piece itself.  Otherwise src/dst point at the chunk's
    // first element, the descriptors span the chunk (`ext` bytes), and
    // (pr, pc) is the row and byte within its segment of the piece's next
    // 1 KiB vector.  Segments are whole KiB, so a vector never straddles
    // two rows and every offset is uniform across the wave.
    int32_t seg = 0, ext = 0, pr = 0, pc = 0;
    const int32_t rb32 = (int32_t)row_bytes;   // a row is below 2^31 bytes
    bool timed_out = false;   // a stage wait timed out (reported at the end)
    // Workspace ring: the current item may be copied once the stage counter
    // `wait_word` reaches `wait_for` (null: no wait); polls so far, and the
    // time of the first.
    const uint64_t* wait_word = nullptr;
    uint32_t wait_for = 0, wait_spins = 0;
    uint32_t wait_t0 = 0;   // low half of the clock: waits stay below 2^32 ticks
    const uint32_t wait_limit = a.limit < 0xffffffffull ? (uint32_t)a.limit : 0xffffffffu;
    // Set up the current item; false when there is none.
    auto setup = [&]() -> bool {
        if (chunk >= nchunks) return false;
        const ChunkRef r = chunk_at(s, chunk);
        const int64_t row0 = (int64_t)r.jr * s.cr;
        // Workspace ring: the chunk's panel goes over the panel that used
        // the stage before; wait until the consumer has finished every
        // tile of that one (its reads of the stage are complete then).
        // The wait itself happens in the copy loop, once this wave has
        // counted every piece it copied (the consumer may need them to
        // finish those tiles).
        if (a.stages) {
            const int m = (int)(row0 / s.tm);
            const int64_t before = stage_tiles_before(s, m);
            if (before > 0) {
                wait_word = a.stages + r.shard * kMaxStages + m % s.ring;
                wait_for = (uint32_t)before;
                wait_spins = 0;
            }
        }
        total = (uint32_t)(r.shard * kFlagCap + r.j);
        weight = piece_weight((int)q, a.ppc);
        if (a.delay_max) {
            const uint32_t d = __builtin_amdgcn_readfirstlane(
                item_delay(a.delay_seed, (uint32_t)uniform(chunk) * ppc + (uint32_t)uniform((int32_t)q),
                           a.delay_max));
            const uint64_t t = ticks();
            while (ticks() - t < d) __builtin_amdgcn_s_sleep(1);
        }
        const int64_t rows = chunk_row_end(s, r.jr) - row0;
        const int64_t k0 = kblock_begin(s, r.kb);
        const int64_t sb = (kblock_end(s, r.kb) - k0) * a.elt;   // bytes per row segment
        const int64_t bytes = rows * sb;
        const int64_t begin = q * a.piece;
        const int64_t end = begin + a.piece < bytes ? begin + a.piece : bytes;
        // an empty piece of a short last chunk copies nothing but counts
        n = end > begin ? (int32_t)(end - begin) : 0;  // a chunk is below 2 GiB
        off = 0;
        if (sb == row_bytes) {
            seg = 0;
            src = a.src[r.shard] + row0 * row_bytes + begin;
            dst = a.dst[r.shard] + slot_row(s, row0) * row_bytes + begin;
        } else {
            seg = (int32_t)sb;
            ext = (int32_t)((rows - 1) * row_bytes + sb);
            src = a.src[r.shard] + row0 * row_bytes + k0 * a.elt;
            dst = a.dst[r.shard] + slot_row(s, row0) * row_bytes + k0 * a.elt;
            pr = (int32_t)(begin / sb);
            pc = (int32_t)(begin - (int64_t)pr * sb);
        }
        return true;
    };

    bool have = setup();
    for (;;) {
        u32x4 v[kUnroll];
        const bool copy = have && !wait_word && off < n;
        // Buffer accesses: lane offsets stay fixed, the sweep's step goes
        // into the scalar offset; the descriptors end where the piece ends
        // (a multiple of 16 bytes), so lanes past it load zeros and store
        // nothing.  Built from first-lane copies, which are uniform to the
        // compiler (loop-carried, it would take them as per-lane values).
        const int32_t sg = uniform(seg);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            uniform_ptr(src), 0, sg ? uniform(ext) : uniform(n), kRsrcWord3);
        const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
            uniform_ptr(dst), 0, sg ? uniform(ext) : uniform(n), kRsrcWord3);
        // Scalar offset of vector u of the sweep.  2-D chunk: the vector
        // lies in row segment r at byte c, and (r, c) steps on by one
        // vector.  A vector past the piece's end (pieces are whole KiB, so
        // it is whole too) copies vector 0 of the sweep again: the same
        // bytes to the same place, with no branch.  The offsets are made
        // again for the stores rather than kept across the wait.
        const int32_t r0 = uniform(pr), c0 = uniform(pc);
        auto vec_off = [&](int u, int32_t& r, int32_t& c) -> int32_t {
            const int32_t o = uniform(off) + u * kLaneStep;
            if (!sg) return o;
            const int32_t at = o < uniform(n) ? r * rb32 + c : r0 * rb32 + c0;
            c += kLaneStep;
            if (c >= sg) {
                c -= sg;
                ++r;
            }
            return at;
        };
        if (copy) {
            int32_t r = r0, c = c0;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int32_t so = vec_off(u, r, c);
                v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                     rs, lane_off, so, kDevice));
            }
        }
        // The one wait point of a sweep: this wave's loads have landed, and
        // its earlier stores and add are performed.  Store the sweep (its
        // registers are free once the stores are issued), look at the add
        // that was in flight, then count the piece whose stores were last.
        __builtin_amdgcn_s_waitcnt(0);
        if (copy) {
            int32_t r = r0, c = c0;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int32_t so = vec_off(u, r, c);
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32, v[u]), rd,
                                                       lane_off, so, kDevice);
            }
            off += kWaveSweepBytes;
            pr = r;
            pc = c;
        }
        if (cnt >= 0) {
            // lane 0's add returned the running total before it
            const uint32_t total = __builtin_amdgcn_readfirstlane(old + cnt_w);
            if ((total & (kPieceTotal - 1)) == 0 && cnt != a.drop)
                release_chunk(a, cnt, origin_sh, lane);
            cnt = -1;
        }
        if (pend >= 0) {
            // the piece's stores are performed (the wait above): count it,
            // and flag it where piece flags are kept
            if (lane == 0) {
                old = __hip_atomic_fetch_add(a.pieces + pend_total, pend_w, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
                // (paced calls: the consumer takes a piece-flagged chunk
                // only once the chunk's paced time has passed)
                if (a.piece_flags && pend != a.drop)
                    __hip_atomic_store(a.piece_flags + pend_total * kPieceFlags + pend_q, a.epoch,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            cnt = pend;
            cnt_w = pend_w;
            pend = -1;
        }
        if (have && wait_word) {
            // Poll the stage once this wave holds no uncounted piece.  The
            // wait is bounded: it fails after the call's limit, or when
            // another workgroup of the call has failed; the wave then
            // stops copying.
            if (pend < 0 && cnt < 0) {
                const uint64_t w =
                    __hip_atomic_load(wait_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)w);
                const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(w >> 32));
                if (tagged_count(((uint64_t)hi << 32) | lo, a.epoch) >= wait_for) {
                    wait_word = nullptr;
                } else {
                    if (wait_spins == 0) wait_t0 = (uint32_t)ticks();
                    __builtin_amdgcn_s_sleep(2);
                    if ((++wait_spins & 31u) == 0) {
                        if (reached(__builtin_amdgcn_readfirstlane(load_agent(a.err)), a.epoch)) {
                            have = false;
                        } else if ((uint32_t)ticks() - wait_t0 > wait_limit) {
                            timed_out = true;
                            have = false;
                        }
                    }
                }
            }
        } else if (have && off >= n) {        // the piece's stores are all issued
            pend = chunk;
            pend_total = total;
            pend_w = weight;
            pend_q = q;
            chunk += step_c;
            q += step_q;
            if (q >= ppc) {
                q -= ppc;
                ++chunk;
            }
            have = setup();
        } else if (!have && cnt < 0) {
            break;                     // drained: nothing stored or added is left
        }
    }
    if (timed_out && lane == 0) raise_error(a.err, a.epoch);
}

}  // namespace prod
}  // namespace
}  // namespace agg
