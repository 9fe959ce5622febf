// producer.hip -- the chunk producer: plays the links of an AllGather on
// one GPU.  For every remote shard it moves chunk after chunk (chunk_rows
// rows x all of K) from the shard into the shard's workspace slot and
// publishes it (PTO-ISA AllGather+GEMM README: the communication kernel
// transfers a chunk, then notifies with an atomic add on the per-source
// summary counter; several communication blocks per destination; chunks
// sent in the order they are consumed).
//
// Each chunk is cut into 512 KiB pieces; piece q of producer position c is
// item c * P + q, and workgroup w copies items w, w + G, w + 2G, ..., so
// all workgroups work on the earliest chunks first and chunks complete in
// about the order they are sent.  A finished chunk is published in three
// steps, none of which waits for another workgroup:
//   * each piece's copier waits until its device-scope (write-through)
//     stores are performed in memory, then counts the piece in the chunk's
//     piece counter;
//   * the copier of the chunk's last piece stores the call's epoch in the
//     chunk's flag (the chunk flag matrix);
//   * it then advances the source's summary counter over every flagged
//     chunk contiguous with it, in one compare-and-swap.
// So a counter value c means "chunks 0..c-1 are flagged", and the counter
// moves as soon as the lowest missing chunk lands, whoever copied it.  The
// consumer waits on the counter, then reads the flags of the chunks it
// needs and acquires (invalidating what its caches may hold of the
// workspace): a flag it sees was stored after the chunk's data reached
// memory.  Counter and flags are updated with relaxed device-scope
// atomics only, and the producer does no cache maintenance at all.
//
// Pacing: with ticks_per_byte > 0 a chunk is not flagged before the
// emulated link could have carried it (parallel links: its own source's
// bytes up to and including the chunk; serial link: everything sent before
// it too), measured from the moment the first producer workgroup started.
#include "kernels.hpp"
#include "sync.hpp"

namespace agg {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(4 * sizeof(unsigned int)))) unsigned int v4u32;

constexpr int kProducerThreads = 256;
constexpr int kRsrcWord3 = 0x00020000;   // untyped 32-bit buffer accesses
// Cache policy of the copy's stores: device scope (written through to
// memory), so that their completion alone publishes them.
constexpr int kStoreDevice = 16;
constexpr int kUnroll = 8;   // 16-byte vectors in flight per lane

// Copy `bytes` (a multiple of 16, both ends 16-byte aligned) with buffer
// accesses: lane offsets stay fixed, the step goes into the scalar offset,
// so eight 16-byte loads per lane are in flight on a handful of registers.
__device__ __forceinline__ void copy_bytes(char* __restrict__ dst,
                                           const char* __restrict__ src,
                                           int64_t bytes)
{
    const int32_t n = (int32_t)bytes;   // a chunk is far below 2 GiB
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, n, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(dst, 0, n, kRsrcWord3);
    const int32_t lane_off = threadIdx.x * 16;
    constexpr int32_t kStep = kProducerThreads * 16;          // bytes per sweep
    int32_t base = 0;
    for (; base + kUnroll * kStep <= n; base += kUnroll * kStep) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 rs, lane_off, base + u * kStep, 0));
        // every load is issued before the first store: the compiler would
        // otherwise pair each load with its store and keep one in flight
        asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]),
                          "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]));
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32, v[u]), rd,
                                                   lane_off, base + u * kStep, kStoreDevice);
    }
    // the tail: lanes past the end are out of range and do nothing.  The
    // whole offset goes into the lane offset, which the range check covers
    for (; base < n; base += kStep) {
        const int32_t off = base + lane_off;
        v4u32 t = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(t, rd, off, 0, kStoreDevice);
    }
}

// Advance the summary counter of one source over the flagged chunks that
// follow it.  Runs on one lane after that lane's own flag store has been
// performed at device scope.  Two lanes racing: the compare-and-swap lets
// one win and the other re-read; a flag stored before a lane reads the
// counter is seen either by that lane or by the lane that moved the
// counter past the chunk before it.
__device__ void advance(uint32_t* ctr, const uint32_t* flags, uint32_t base, int cps,
                        uint32_t epoch)
{
    for (;;) {
        uint32_t cur = load_agent(ctr);
        int rel = (int)(cur - base);
        int k = 0;
        while (rel + k < cps && load_agent(flags + rel + k) == epoch) ++k;
        if (k == 0) return;
        uint32_t want = cur;
        __hip_atomic_compare_exchange_strong(ctr, &want, cur + (uint32_t)k,
                                             __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        // success or not, look again: more chunks may have landed
    }
}

// Count one copied piece of a chunk; true for the piece that completes it.
// The word holds the call's epoch above the count, so it needs no reset: a
// word left by an earlier call restarts at one.
__device__ bool count_piece(uint64_t* word, uint32_t epoch, int ppc)
{
    uint64_t cur = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (;;) {
        const uint64_t next = (uint32_t)(cur >> 32) == epoch
                                  ? cur + 1
                                  : ((uint64_t)epoch << 32) | 1u;
        if (__hip_atomic_compare_exchange_strong(word, &cur, next, __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
            return (uint32_t)next == (uint32_t)ppc;
    }
}

}  // namespace

__global__ __launch_bounds__(kProducerThreads) void producer_kernel(ProducerArgs a)
{
    const Schedule& s = a.s;
    const int64_t items = total_chunks(s) * a.ppc;
    const int64_t row_bytes = s.K * a.elt;
    __shared__ uint64_t origin_sh;
    __shared__ int stop_sh;

    // Producer waves share their SIMDs with consumer waves; they issue few
    // instructions, each of which the consumer is waiting on, so they go
    // first when both are ready.
    __builtin_amdgcn_s_setprio(3);
    // Pipelined mode: this kernel runs on a stream of its own with no
    // dependency on the caller's stream, so it must not read a shard
    // before the work queued ahead of the call has finished.  The consumer
    // runs on the caller's stream, so its start proves that; each of its
    // workgroups writes the call's epoch to the start word on entry.
    if (a.start) {
        if (threadIdx.x == 0)
            stop_sh = !reached(poll_until(a.start, a.epoch, a.err, a.epoch, a.limit), a.epoch);
        __syncthreads();
        if (stop_sh) return;
        // the shards were written before the consumer started; drop any
        // stale copies of them from this CU's caches
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    if (threadIdx.x == 0) {
        origin_sh = a.ticks_per_byte > 0.0 ? pacing_origin(a.clock, a.epoch) : 0;
        stop_sh = 0;
    }
    __syncthreads();

    for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
        const int64_t c = it / a.ppc;                  // producer position
        const int64_t q = it % a.ppc;                  // piece of its chunk
        const ChunkRef r = chunk_at(s, c);
        const int64_t row0 = (int64_t)r.j * s.cr;
        // Workspace ring: the chunk's panel goes over the panel that used
        // the stage before; wait until the consumer has finished every
        // tile of that one (its reads of the stage are complete then).
        if (a.stages) {
            const int m = (int)(row0 / s.tm);
            const int64_t before = stage_tiles_before(s, m);
            if (before > 0) {
                if (threadIdx.x == 0)
                    stop_sh = !poll_count(a.stages + r.shard * kMaxStages + m % s.ring, a.epoch,
                                          (uint32_t)before, a.err, a.limit);
                __syncthreads();
                if (stop_sh) break;
            }
        }
        const int64_t bytes = (chunk_row_end(s, r.j) - row0) * row_bytes;
        const int64_t begin = q * kPieceBytes;
        const int64_t end = begin + kPieceBytes < bytes ? begin + kPieceBytes : bytes;
        if (begin < end)
            copy_bytes(a.dst[r.shard] + slot_row(s, row0) * row_bytes + begin,
                       a.src[r.shard] + row0 * row_bytes + begin, end - begin);
        // The copy's stores are device-scope stores, written through to
        // memory; a store is counted done only once it is performed there.
        // Waiting for them is what makes the piece visible to every CU, so
        // no cache write-back (what a release fence would add, for the
        // whole L2) is needed before the piece is counted.
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x == 0 &&
            count_piece(a.pieces + r.shard * kFlagCap + r.j, a.epoch, a.ppc) && c != a.drop) {
            // every piece of the chunk is in memory: release it
            bool ok = true;
            if (a.ticks_per_byte > 0.0) {
                const double b = (double)paced_bytes(s, r, a.elt);
                const double delta = b * a.ticks_per_byte;
                // a pace slower than the wait limit is a failed call, not a hang
                if (delta > (double)a.limit) {
                    raise_error(a.err, a.epoch);
                    ok = false;
                } else {
                    wait_until(origin_sh, (uint64_t)delta);
                }
            }
            if (ok) {
                uint32_t* flags = a.flags + r.shard * kFlagCap;
                // stamped before the flag, so a consumer that saw the flag
                // started after this time
                if (a.trace) a.trace[1 + c] = ticks();
                __hip_atomic_store(flags + r.j, a.epoch, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                // the flag store is performed before the counter is read
                __builtin_amdgcn_s_waitcnt(0);
                advance(a.counters + r.shard * (kCounterStride / 4), flags,
                        a.base[r.shard], s.cps, a.epoch);
            }
        }
        // stop early once a workgroup of this call has failed; one lane
        // decides for the whole workgroup, so every wave leaves together
        if (threadIdx.x == 0) stop_sh = reached(load_agent(a.err), a.epoch);
        __syncthreads();
        if (stop_sh) break;
    }
}

// Zero `bytes` bytes of a workspace header (counters, error word, pacing
// slot, chunk flags).
__global__ void header_reset_kernel(uint32_t* header, size_t words)
{
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < words;
         i += (size_t)gridDim.x * blockDim.x)
        header[i] = 0;
}

hipError_t launch_producer(const ProducerArgs& a, int wgs, hipStream_t st)
{
    hipLaunchKernelGGL(producer_kernel, dim3(wgs), dim3(kProducerThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_header_reset(uint32_t* header, size_t bytes, hipStream_t st)
{
    hipLaunchKernelGGL(header_reset_kernel, dim3(64), dim3(256), 0, st, header, bytes / 4);
    return hipGetLastError();
}

}  // namespace agg
