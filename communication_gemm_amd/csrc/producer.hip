// producer.hip -- the chunk producer: plays the links of an AllGather on
// one GPU.  For every remote shard it moves chunk after chunk (chunk_rows
// rows x all of K) from the shard into the shard's workspace slot and
// releases each chunk on the shard's counter (PTO-ISA AllGather+GEMM
// README: the communication kernel transfers a chunk, then notifies with an
// atomic add on the per-source counter; several communication blocks per
// destination; chunks sent in the order they are consumed).
//
// Workgroups take producer positions from a ticket counter, in order.
// Copies proceed in parallel; releases of one source happen in chunk order
// (a workgroup waits for the source's counter to reach its chunk index
// before adding one), so a counter value c always means "chunks 0..c-1 are
// in place".  A workgroup only ever waits for a chunk whose ticket was taken
// before its own, by a workgroup that is already running, so the producer
// makes progress however few of its workgroups fit on the GPU at once.
//
#include "kernels.hpp"
#include "sync.hpp"

namespace agg {

namespace {

constexpr int kProducerThreads = 256;
constexpr int kUnroll = 8;   // 16-byte vectors in flight per lane

__device__ __forceinline__ void copy_bytes(char* __restrict__ dst,
                                           const char* __restrict__ src,
                                           int64_t bytes)
{
    // bytes is a multiple of 16 and both pointers are 16-byte aligned
    const int64_t nvec = bytes >> 4;
    const uint4* s = reinterpret_cast<const uint4*>(src);
    uint4* d = reinterpret_cast<uint4*>(dst);
    const int tid = threadIdx.x;
    const int64_t step = (int64_t)kProducerThreads * kUnroll;
    int64_t i = tid;
    for (; i + (kUnroll - 1) * kProducerThreads < nvec; i += step) {
        uint4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = s[i + u * kProducerThreads];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) d[i + u * kProducerThreads] = v[u];
    }
    for (; i < nvec; i += kProducerThreads) d[i] = s[i];
}

}  // namespace

__global__ __launch_bounds__(kProducerThreads) void producer_kernel(ProducerArgs a)
{
    const Schedule& s = a.s;
    const int64_t total = total_chunks(s);
    const int64_t row_bytes = s.K * a.elt;
    __shared__ uint64_t origin_sh;
    __shared__ int failed_sh;

    if (threadIdx.x == 0) {
        origin_sh = a.ticks_per_byte > 0.0 ? pacing_origin(a.clock, a.epoch) : 0;
        failed_sh = 0;
    }
    __syncthreads();

    __shared__ int64_t pos_sh;
    for (;;) {
        if (threadIdx.x == 0) {
            uint32_t t = __hip_atomic_fetch_add(a.ticket, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
            pos_sh = failed_sh ? total : (int64_t)(uint32_t)(t - a.ticket_base);
        }
        __syncthreads();
        const int64_t c = pos_sh;
        if (c >= total) break;
        const ChunkRef r = chunk_at(s, c);
        const int64_t row0 = (int64_t)r.j * s.cr;
        const int64_t rows = chunk_row_end(s, r.j) - row0;
        copy_bytes(a.dst[r.shard] + row0 * row_bytes,
                   a.src[r.shard] + row0 * row_bytes, rows * row_bytes);
        // each lane makes its own stores visible at device scope before
        // the single release below
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __syncthreads();
        if (threadIdx.x == 0) {
            uint32_t* ctr = a.counters + r.shard * (kCounterStride / 4);
            const uint32_t mine = a.base[r.shard] + (uint32_t)r.j;
            uint32_t seen = acquire_wait(ctr, mine, a.err, a.epoch, a.limit);
            if (!reached(seen, mine)) {
                failed_sh = 1;
            } else {
                if (a.ticks_per_byte > 0.0) {
                    double b = (double)paced_bytes(s, r, a.elt);
                    wait_until(origin_sh, (uint64_t)(b * a.ticks_per_byte));
                }
                if (c != a.drop) release_add(ctr);
            }
        }
        __syncthreads();
    }
}

// Counters, error word and pacing slot to zero; run once per workspace.
__global__ void header_reset_kernel(uint32_t* header)
{
    for (int i = threadIdx.x; i < kHeaderBytes / 4; i += blockDim.x) header[i] = 0;
}

hipError_t launch_producer(const ProducerArgs& a, int wgs, hipStream_t st)
{
    hipLaunchKernelGGL(producer_kernel, dim3(wgs), dim3(kProducerThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_header_reset(uint32_t* header, hipStream_t st)
{
    hipLaunchKernelGGL(header_reset_kernel, dim3(1), dim3(256), 0, st, header);
    return hipGetLastError();
}

}  // namespace agg
