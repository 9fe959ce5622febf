// probe.hip -- measurement helpers, not part of the library's interface.
// mfma_probe: matrix instructions on operands held in registers, with no
// memory traffic inside the loop.  It gives the rate the matrix cores
// sustain on this board when nothing else limits them, with operands that
// toggle many bits (random values) or few (one constant), since the board's
// power limit sets the clock under load.  load_probe and stream_probe: the
// operand movement of the consumer's K slices (direct loads into LDS, LDS
// reads) and the rate at which a whole matrix streams into LDS in a given
// access pattern, with no arithmetic.  Built into its own small library;
// only the benchmark script loads it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef int intx16 __attribute__((ext_vector_type(16)));

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
    if constexpr (KIND == 0 || KIND == 2) {
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
        if constexpr (KIND == 0) {
            for (int64_t i = 0; i < iters; ++i)
#pragma unroll
                for (int c = 0; c < kChains; ++c)
                    acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[c & 1], b[(c >> 1) & 1],
                                                                     acc[c], 0, 0, 0);
        } else {
            // two 16x16x32 instructions per chain and iteration: the same
            // flops as one 32x32x16, on four-register accumulators
            floatx4 acc4[2 * kChains];
            for (int c = 0; c < 2 * kChains; ++c)
                for (int e = 0; e < 4; ++e) acc4[c][e] = 0.f;
            for (int64_t i = 0; i < iters; ++i)
#pragma unroll
                for (int c = 0; c < 2 * kChains; ++c)
                    acc4[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[c & 1], b[(c >> 1) & 1],
                                                                      acc4[c], 0, 0, 0);
            for (int c = 0; c < kChains; ++c)
                for (int e = 0; e < 4; ++e) {
                    acc[c][e] = acc4[2 * c][e];
                    acc[c][4 + e] = acc4[2 * c + 1][e];
                }
        }
    } else if constexpr (KIND == 3 || KIND == 4) {
        // int8: random bytes, or 1 in every byte
        intx4 a[2], b[2];
        for (int v = 0; v < 2; ++v)
            for (int w = 0; w < 4; ++w) {
                a[v][w] = random ? (int)mix(seed ^ (tid * 16 + v * 8 + w)) : 0x01010101;
                b[v][w] = random ? (int)mix(~seed ^ (tid * 16 + v * 8 + w + 4)) : 0x01010101;
            }
        if constexpr (KIND == 3) {
            intx16 acc_i[kChains];
            for (int c = 0; c < kChains; ++c)
                for (int e = 0; e < 16; ++e) acc_i[c][e] = 0;
            for (int64_t i = 0; i < iters; ++i)
#pragma unroll
                for (int c = 0; c < kChains; ++c)
                    acc_i[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[c & 1], b[(c >> 1) & 1],
                                                                      acc_i[c], 0, 0, 0);
            for (int c = 0; c < kChains; ++c)
                for (int e = 0; e < 16; ++e) acc[c][e] = (float)acc_i[c][e];
        } else {
            intx4 acc_i[2 * kChains];
            for (int c = 0; c < 2 * kChains; ++c)
                for (int e = 0; e < 4; ++e) acc_i[c][e] = 0;
            for (int64_t i = 0; i < iters; ++i)
#pragma unroll
                for (int c = 0; c < 2 * kChains; ++c)
                    acc_i[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[c & 1], b[(c >> 1) & 1],
                                                                      acc_i[c], 0, 0, 0);
            for (int c = 0; c < kChains; ++c)
                for (int e = 0; e < 4; ++e) {
                    acc[c][e] = (float)acc_i[2 * c][e];
                    acc[c][4 + e] = (float)acc_i[2 * c + 1][e];
                }
        }
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

#define LDS_PTR __attribute__((address_space(3)))
constexpr int kRsrcWord3 = 0x00020000;   // untyped 32-bit buffer accesses

// Operand-movement probe: per iteration every workgroup (eight waves, one
// per CU) moves one 64 KiB slice into LDS with the direct global-to-LDS load
// and/or reads 192 KiB out of LDS with ds_read_b128, then waits for all of
// it and meets at a barrier -- the traffic of one K slice of the 256 x 256
// fp16 consumer tile.  pattern 0: the slice is 64 KiB contiguous;
// pattern 1: the tile's shape, A 256 rows x 128 B and B 64 rows x 512 B at
// a row pitch of `pitch` bytes, the workgroups of one XCD on a block of
// 4 row panels x 8 n-tiles (as the consumer places them), the slice index
// stepping through `nslices` slices of K.  what: 1 loads, 2 LDS reads,
// 3 both.  A holds at least 4096 rows and B 64 nslices rows of `pitch`
// bytes; both descriptors are bounded by a_bytes and b_bytes, so nothing
// outside the buffers is touched.
__global__ __launch_bounds__(512, 1) void load_probe(const char* A, const char* B,
                                                    uint32_t a_bytes, uint32_t b_bytes,
                                                    int pattern, int what, int iters,
                                                    uint32_t pitch, uint32_t nslices, float* out)
{
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const __amdgpu_buffer_rsrc_t ra =
        __builtin_amdgcn_make_buffer_rsrc((void*)A, 0, (int)a_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rb =
        __builtin_amdgcn_make_buffer_rsrc((void*)B, 0, (int)b_bytes, kRsrcWord3);
    const int x = blockIdx.x % 8, slot = blockIdx.x / 8 % 32;
    const uint32_t mt = (uint32_t)((x / 2) * 4 + slot / 8);   // row panel 0..15
    const uint32_t nt = (uint32_t)((x % 2) * 8 + slot % 8);   // n-tile 0..15
    uint32_t acc = 0;
    for (int it = 0; it < iters; ++it) {
        char* ld = lds + ((it + 1) & 1) * 65536;
        const char* rd = lds + (it & 1) * 65536;
        if (what & 1) {
            const uint32_t ks = (uint32_t)it % nslices;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int q = wave * 4 + u;                    // 32 A instructions
                const uint32_t off = pattern == 0
                    ? (uint32_t)(((mt * 16 + nt) * 65536u + (uint32_t)q * 1024u + lane * 16u) % a_bytes)
                    : (mt * 256u + (uint32_t)(q * 8 + lane / 8)) * pitch + ks * 128u + (lane % 8) * 16u;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (LDS_PTR void*)(ld + q * 1024), 16, off,
                                                         0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int q = wave * 4 + u;                    // 32 B instructions
                const uint32_t off = pattern == 0
                    ? (uint32_t)(((mt * 16 + nt) * 65536u + 32768u + (uint32_t)q * 1024u + lane * 16u) % b_bytes)
                    : (ks * 64u + (uint32_t)(q * 2 + lane / 32)) * pitch + nt * 512u + (lane % 32) * 16u;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (LDS_PTR void*)(ld + 32768 + q * 1024),
                                                         16, off, 0, 0, 0);
            }
        }
        if (what & 2) {
#pragma unroll
            for (int r = 0; r < 24; ++r) {                     // 24 KiB per wave
                const uint4 v = *reinterpret_cast<const uint4*>(rd + ((wave * 24 + r) % 64) * 1024 +
                                                                lane * 16);
                acc ^= v.x + v.y + v.z + v.w;
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    out[blockIdx.x * blockDim.x + threadIdx.x] = (float)(acc & 1u);
}

// Streaming probe: one launch loads the whole of a rows x row_bytes matrix
// into LDS once, 64 KiB per workgroup per step (eight 1 KiB direct loads per
// wave, then a wait and a barrier).  pattern 0: column strips 64 bytes wide,
// workgroup w on strip w / parts and on part w % parts of the rows (16 rows
// per wave and load: the way a narrow-tile consumer walks its B columns);
// pattern 1: each workgroup on one contiguous range of total / grid bytes.
// The host checks that rows / parts is a multiple of 1024 (pattern 0) and
// that the ranges are whole 64 KiB steps (pattern 1), and the descriptor is
// bounded by the matrix, so every access stays inside it.
__global__ __launch_bounds__(512, 1) void stream_probe(const char* B, uint32_t rows,
                                                      uint32_t row_bytes, int pattern,
                                                      uint32_t parts, float* out)
{
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const uint32_t total = rows * row_bytes;
    const __amdgpu_buffer_rsrc_t rb =
        __builtin_amdgcn_make_buffer_rsrc((void*)B, 0, (int)total, kRsrcWord3);
    if (pattern == 0) {
        const uint32_t strip = blockIdx.x / parts, part = blockIdx.x % parts;
        const uint32_t per = rows / parts, row0 = part * per;
        for (uint32_t r = 0; r < per; r += 1024) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint32_t row = row0 + r + (uint32_t)(u * 128 + wave * 16 + lane / 4);
                const uint32_t off = row * row_bytes + strip * 64u + (uint32_t)(lane % 4) * 16u;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rb, (LDS_PTR void*)(lds + u * 8192 + wave * 1024), 16, off, 0, 0, 0);
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
    } else {
        const uint32_t len = total / gridDim.x, base = blockIdx.x * len;
        for (uint32_t o = 0; o < len; o += 65536) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint32_t off = base + o + (uint32_t)(u * 8192 + wave * 1024 + lane * 16);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rb, (LDS_PTR void*)(lds + u * 8192 + wave * 1024), 16, off, 0, 0, 0);
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
    }
    if (threadIdx.x == 0) out[blockIdx.x] = (float)lds[lane];
}

}  // namespace

extern "C" {

// Launches the probe: `wgs` workgroups of 8 waves (two per SIMD, one
// workgroup per CU), each wave issuing iters x 8 matrix instructions
// (kind 0: fp16 32x32x16, 32768 flops each; kind 1: fp8 E4M3 32x32x64,
// 131072 flops each) or iters x 16 (kind 2: fp16 16x16x32, 16384 flops
// each; kind 3: int8 32x32x32, 65536 operations each; kind 4: int8
// 16x16x64, two per chain and iteration, 32768 each).  out: wgs * 512
// floats of device memory.  stream: a hipStream_t (nullptr = the null
// stream).  Returns a hipError_t.
int agg_probe_mfma(int kind, int random, int64_t iters, int wgs, uint32_t seed, float* out,
                   void* stream)
{
    if (kind < 0 || kind > 4 || iters < 0 || wgs < 1 || !out) return (int)hipErrorInvalidValue;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (kind == 0)
        hipLaunchKernelGGL(mfma_probe<0>, dim3(wgs), dim3(512), 0, st, iters, seed, random, out);
    else if (kind == 2)
        hipLaunchKernelGGL(mfma_probe<2>, dim3(wgs), dim3(512), 0, st, iters, seed, random, out);
    else if (kind == 3)
        hipLaunchKernelGGL(mfma_probe<3>, dim3(wgs), dim3(512), 0, st, iters, seed, random, out);
    else if (kind == 4)
        hipLaunchKernelGGL(mfma_probe<4>, dim3(wgs), dim3(512), 0, st, iters, seed, random, out);
    else
        hipLaunchKernelGGL(mfma_probe<1>, dim3(wgs), dim3(512), 0, st, iters, seed, random, out);
    return (int)hipGetLastError();
}

// Launches the operand-movement probe (load_probe above) on `wgs`
// workgroups of 512 threads with 128 KiB of LDS.  A: a_bytes (at least
// 4096 * pitch for pattern 1), B: b_bytes (at least 64 * nslices * pitch);
// both below 2^31.  out: wgs * 512 floats.  Returns a hipError_t.
int agg_probe_loads(int pattern, int what, int iters, int wgs, const void* A, uint32_t a_bytes,
                    const void* B, uint32_t b_bytes, uint32_t pitch, uint32_t nslices,
                    float* out, void* stream)
{
    if (pattern < 0 || pattern > 1 || what < 1 || what > 3 || iters < 0 || wgs < 1 || !A ||
        !B || !out || nslices < 1 || nslices > 64 || a_bytes < 65536 || b_bytes < 65536 ||
        a_bytes > 0x7fffffffu || b_bytes > 0x7fffffffu)
        return (int)hipErrorInvalidValue;
    if (pattern == 1 && ((uint64_t)4096 * pitch > a_bytes || (uint64_t)64 * nslices * pitch > b_bytes ||
                         pitch < 8192 || nslices * 128u > pitch))
        return (int)hipErrorInvalidValue;
    static bool attr = false;
    if (!attr) {
        const hipError_t e = hipFuncSetAttribute((const void*)load_probe,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, 131072);
        if (e != hipSuccess) return (int)e;
        attr = true;
    }
    hipLaunchKernelGGL(load_probe, dim3(wgs), dim3(512), 131072, static_cast<hipStream_t>(stream),
                       static_cast<const char*>(A), static_cast<const char*>(B), a_bytes, b_bytes,
                       pattern, what, iters, pitch, nslices, out);
    return (int)hipGetLastError();
}

// Launches the streaming probe (stream_probe above) on a rows x row_bytes
// matrix B of device memory (at most 2^31 - 1 bytes), with 64 KiB of LDS per
// workgroup.  pattern 0: `n` parts per 64-byte column strip, so the grid is
// row_bytes / 64 x n workgroups; rows / n must be a multiple of 1024.
// pattern 1: `n` workgroups on contiguous ranges; the matrix must hold a
// multiple of n x 64 KiB.  out: one float per workgroup.  Returns a
// hipError_t.
int agg_probe_stream(int pattern, int n, const void* B, uint32_t rows, uint32_t row_bytes,
                     float* out, void* stream)
{
    if (pattern < 0 || pattern > 1 || n < 1 || !B || !out || rows == 0 || row_bytes == 0 ||
        (uint64_t)rows * row_bytes > 0x7fffffffu)
        return (int)hipErrorInvalidValue;
    const uint32_t total = rows * row_bytes;
    int wgs = n;
    if (pattern == 0) {
        if (row_bytes % 64 || rows % (uint32_t)n || (rows / (uint32_t)n) % 1024)
            return (int)hipErrorInvalidValue;
        wgs = (int)(row_bytes / 64) * n;
    } else if (total % 65536 || (total / 65536) % (uint32_t)n) {
        return (int)hipErrorInvalidValue;
    }
    static bool attr = false;
    if (!attr) {
        const hipError_t e = hipFuncSetAttribute((const void*)stream_probe,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, 65536);
        if (e != hipSuccess) return (int)e;
        attr = true;
    }
    hipLaunchKernelGGL(stream_probe, dim3(wgs), dim3(512), 65536, static_cast<hipStream_t>(stream),
                       static_cast<const char*>(B), rows, row_bytes, pattern, (uint32_t)n, out);
    return (int)hipGetLastError();
}

}  // extern "C"
