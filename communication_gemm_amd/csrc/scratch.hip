// scratch.hip -- the fixed workspace of the allocation-free entry point
// (ag_gemm_f16_noalloc): one file-scope device array per GPU, held from the
// moment the library's code is loaded on that GPU until the process ends.
//
// In host code the array's name only stands for the symbol: its device
// address differs from GPU to GPU and is taken here, once per device, with
// that device current.  Every other use (kernel arguments, the header
// reset) goes through that address.
#include "kernels.hpp"

namespace agg {

static __device__ __align__(256) char scratch[kScratchBytes];

hipError_t scratch_address(void** out)
{
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255u)) return hipErrorInvalidSymbol;
    *out = p;
    return hipSuccess;
}

}  // namespace agg
