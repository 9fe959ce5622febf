// probe.hip -- a measurement helper, not part of the library's interface:
// matrix instructions on operands held in registers, with no memory traffic
// inside the loop.  It gives the rate the matrix cores sustain on this board
// when nothing else limits them, with operands that toggle many bits
// (random values) or few (one constant), since the board's power limit
// sets the clock under load.  Built into its own small library; only the
// benchmark script loads it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int intx8 __attribute__((ext_vector_type(8)));

constexpr int kChains = 8;   // independent accumulators per wave

__device__ uint32_t mix(uint32_t x)
{
    // xorshift-multiply integer hash
    x ^= x >> 16;
    x *= 0x7FEB352Du;
    x ^= x >> 15;
    x *= 0x846CA68Bu;
    x ^= x >> 16;
    return x;
}

// One operand register word: random values of magnitude [1, 2) and either
// sign, or the constant 1.0 in every element.
__device__ uint32_t word_f16(uint32_t h, bool random)
{
    if (!random) return 0x3C003C00u;
    return (h & 0x83FF83FFu) | 0x3C003C00u;
}

__device__ uint32_t word_fp8(uint32_t h, bool random)
{
    // E4M3: exponent field 7 is 2^0
    if (!random) return 0x38383838u;
    return (h & 0x87878787u) | 0x38383838u;
}

template <int KIND>
__global__ __launch_bounds__(512, 1) void mfma_probe(int64_t iters, uint32_t seed, int random,
                                                     float* out)
{
    const uint32_t tid = blockIdx.x * blockDim.x + threadIdx.x;
    floatx16 acc[kChains];
    for (int c = 0; c < kChains; ++c)
        for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
    if constexpr (KIND == 0) {
        half8 a[2], b[2];
        for (int v = 0; v < 2; ++v) {
            uint32_t wa[4], wb[4];
            for (int w = 0; w < 4; ++w) {
                wa[w] = word_f16(mix(seed ^ (tid * 16 + v * 8 + w)), random != 0);
                wb[w] = word_f16(mix(~seed ^ (tid * 16 + v * 8 + w + 4)), random != 0);
            }
            a[v] = __builtin_bit_cast(half8, *reinterpret_cast<uint4*>(wa));
            b[v] = __builtin_bit_cast(half8, *reinterpret_cast<uint4*>(wb));
        }
        for (int64_t i = 0; i < iters; ++i)
#pragma unroll
            for (int c = 0; c < kChains; ++c)
                acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[c & 1], b[(c >> 1) & 1],
                                                                 acc[c], 0, 0, 0);
    } else {
        intx8 a[2], b[2];
        for (int v = 0; v < 2; ++v)
            for (int w = 0; w < 8; ++w) {
                a[v][w] = (int)word_fp8(mix(seed ^ (tid * 32 + v * 16 + w)), random != 0);
                b[v][w] = (int)word_fp8(mix(~seed ^ (tid * 32 + v * 16 + w + 8)), random != 0);
            }
        for (int64_t i = 0; i < iters; ++i)
#pragma unroll
            for (int c = 0; c < kChains; ++c)
                acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    a[c & 1], b[(c >> 1) & 1], acc[c], 0, 0, 0, 0, 0, 0);
    }
    float s = 0.f;
    for (int c = 0; c < kChains; ++c)
        for (int e = 0; e < 16; ++e) s += acc[c][e];
    out[tid] = s;
}

}  // namespace

extern "C" {

// Launches the probe: `wgs` workgroups of 8 waves (two per SIMD, one
// workgroup per CU), each wave issuing iters x 8 matrix instructions
// (kind 0: fp16 32x32x16, 32768 flops each; kind 1: fp8 E4M3 32x32x64,
// 131072 flops each).  out: wgs * 512 floats of device memory.  stream:
// a hipStream_t (nullptr = the null stream).  Returns a hipError_t.
int agg_probe_mfma(int kind, int random, int64_t iters, int wgs, uint32_t seed, float* out,
                   void* stream)
{
    if (kind < 0 || kind > 1 || iters < 0 || wgs < 1 || !out) return (int)hipErrorInvalidValue;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (kind == 0)
        hipLaunchKernelGGL(mfma_probe<0>, dim3(wgs), dim3(512), 0, st, iters, seed, random, out);
    else
        hipLaunchKernelGGL(mfma_probe<1>, dim3(wgs), dim3(512), 0, st, iters, seed, random, out);
    return (int)hipGetLastError();
}

}  // extern "C"
