// producer.hip -- the producer kernel (the chunk producer's own grid, on a
// stream of its own or in the caller's stream order) and the workspace
// header reset.  The producer's device code is in producer_body.hpp.
#include "producer_body.hpp"

namespace agg {

__global__ __launch_bounds__(prod::kProducerThreads) void producer_kernel(ProducerArgs a)
{
    __shared__ prod::ProducerShared sh;
    prod::produce(a, blockIdx.x, gridDim.x, sh);
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
    hipLaunchKernelGGL(producer_kernel, dim3(wgs), dim3(prod::kProducerThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_header_reset(uint32_t* header, size_t bytes, hipStream_t st)
{
    hipLaunchKernelGGL(header_reset_kernel, dim3(64), dim3(256), 0, st, header, bytes / 4);
    return hipGetLastError();
}

}  // namespace agg
