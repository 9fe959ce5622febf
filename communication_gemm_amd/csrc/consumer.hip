// consumer.hip -- the persistent MFMA consumer GEMM (fp16 -> fp32 and
// int8 -> int32 + bias -> per-channel dequant -> fp16).
//
// One workgroup per CU walks the tile list of the shared schedule: first
// the local shard's tiles (no wait), then the remote tiles in the order
// their rows arrive (PTO-ISA AllGather+GEMM README: phase 1 computes the
// local row-group with no wait, phase 2 waits on each remote source's
// summary counter and computes as soon as the rows are there).  Before a
// remote tile, one lane waits until the source's counter covers the tile's
// last row; what a workgroup has already seen of a counter is remembered,
// so most tiles pass without touching it.
//
// Tile main loop (PTO-ISA README: continuous K accumulation, two-level
// double buffering): 4 waves, each owning a (BM/2) x (BN/2) block of
// 32x32 MFMA accumulators kept in registers for the whole K loop; A and B
// k-slices are staged in LDS, double buffered, the next slice's HBM loads
// (16 bytes per lane) in flight while the current one is multiplied.
//
// LDS layout: every operand row holds one k-slice of 128 bytes as eight
// 16-byte pieces; piece p of row r is stored at position p ^ swz(r), which
// keeps both the row-wise 16-byte stores and the column-wise MFMA operand
// reads free of bank conflicts.  A is stored as it lies in memory (row =
// output row, k along the row); B is stored transposed (row = output
// column, k along the row), because an MFMA operand lane holds consecutive
// k of one column.  The transpose happens in registers on the way in.
#include "kernels.hpp"
#include "sync.hpp"

namespace agg {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef int intx16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;   // 4 waves
constexpr int kRowBytes = 128;  // one k-slice of one operand row in LDS

__device__ __forceinline__ int swz(int r) { return (r + (r >> 3)) & 7; }

__device__ __forceinline__ int lds_off(int row, int piece)
{
    return row * kRowBytes + ((piece ^ swz(row)) << 4);
}

// ---- element traits ---------------------------------------------------

struct F16 {
    static constexpr int kElt = 2;        // bytes per element
    static constexpr int kBK = 64;        // k per slice (128 bytes)
    static constexpr int kBRows = 8;      // B rows (k) per transposed block
    typedef floatx16 Acc;

    __device__ static Acc zero() { Acc z; for (int i = 0; i < 16; ++i) z[i] = 0.f; return z; }

    __device__ static Acc mma(const uint4& a, const uint4& b, const Acc& c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(
            __builtin_bit_cast(half8, a), __builtin_bit_cast(half8, b), c, 0, 0, 0);
    }

    // One B block: k rows [k, k+8) x columns [n, n+8) -> eight 16-byte
    // column pieces (8 k values of one column each).
    __device__ static void load_b(const char* __restrict__ B, int64_t N, int64_t K,
                                  int64_t k, int64_t n, uint4 (&raw)[8])
    {
        const bool ncol = n < N;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            if (ncol && k + r < K)
                raw[r] = *reinterpret_cast<const uint4*>(B + ((k + r) * N + n) * 2);
            else
                raw[r] = make_uint4(0, 0, 0, 0);
        }
    }

    __device__ static void transpose_b(const uint4 (&raw)[8], uint4 (&col)[8])
    {
        // raw[r] holds columns 0..7 of row r as 4 words of 2 halves;
        // col[c] must hold rows 0..7 of column c.
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            uint32_t w[4];
#pragma unroll
            for (int rp = 0; rp < 4; ++rp) {
                const uint4& x4 = raw[2 * rp];
                const uint4& y4 = raw[2 * rp + 1];
                uint32_t x = (c >> 1) == 0 ? x4.x : (c >> 1) == 1 ? x4.y : (c >> 1) == 2 ? x4.z : x4.w;
                uint32_t y = (c >> 1) == 0 ? y4.x : (c >> 1) == 1 ? y4.y : (c >> 1) == 2 ? y4.z : y4.w;
                w[rp] = (c & 1) ? ((x >> 16) | (y & 0xffff0000u))
                                : ((x & 0xffffu) | (y << 16));
            }
            col[c] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
};

struct I8 {
    static constexpr int kElt = 1;
    static constexpr int kBK = 128;
    static constexpr int kBRows = 16;
    typedef intx16 Acc;

    __device__ static Acc zero() { Acc z; for (int i = 0; i < 16; ++i) z[i] = 0; return z; }

    __device__ static Acc mma(const uint4& a, const uint4& b, const Acc& c)
    {
        return __builtin_amdgcn_mfma_i32_32x32x32_i8(
            __builtin_bit_cast(intx4, a), __builtin_bit_cast(intx4, b), c, 0, 0, 0);
    }

    // One B block: k rows [k, k+16) x columns [n, n+8), as 16 pieces of 8
    // bytes, kept two rows per uint4 (raw[q] = rows 2q, 2q+1).
    __device__ static void load_b(const char* __restrict__ B, int64_t N, int64_t K,
                                  int64_t k, int64_t n, uint4 (&raw)[8])
    {
        const bool ncol = n < N;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            uint2 lo = make_uint2(0, 0), hi = make_uint2(0, 0);
            if (ncol && k + 2 * q < K)
                lo = *reinterpret_cast<const uint2*>(B + (k + 2 * q) * N + n);
            if (ncol && k + 2 * q + 1 < K)
                hi = *reinterpret_cast<const uint2*>(B + (k + 2 * q + 1) * N + n);
            raw[q] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
    }

    __device__ static uint32_t byte_of(const uint4 (&raw)[8], int r, int c)
    {
        // byte c (0..7) of row r (0..15)
        const uint4& v = raw[r >> 1];
        uint32_t w;
        const int wi = ((r & 1) << 1) | (c >> 2);
        w = wi == 0 ? v.x : wi == 1 ? v.y : wi == 2 ? v.z : v.w;
        return (w >> ((c & 3) * 8)) & 0xffu;
    }

    __device__ static void transpose_b(const uint4 (&raw)[8], uint4 (&col)[8])
    {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            uint32_t w[4];
#pragma unroll
            for (int d = 0; d < 4; ++d)
                w[d] = byte_of(raw, 4 * d, c) | (byte_of(raw, 4 * d + 1, c) << 8) |
                       (byte_of(raw, 4 * d + 2, c) << 16) | (byte_of(raw, 4 * d + 3, c) << 24);
            col[c] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
};

// ---- the tile engine --------------------------------------------------

template <class T, int BM, int BN>
struct Engine {
    static constexpr int kTM = BM / 64;             // 32x32 blocks per wave along M
    static constexpr int kTN = BN / 64;             // ... along N
    static constexpr int kAVec = BM * 8 / kThreads; // A pieces per lane per slice
    static constexpr int kBBlk = (BN + kThreads - 1) / kThreads; // B blocks per lane
    static constexpr int kStage = (BM + BN) * kRowBytes;         // one LDS buffer
    static_assert(kAVec >= 1, "tile too small");

    uint4 a_reg[kAVec];
    uint4 b_reg[kBBlk][8];

    __device__ void gload(const char* __restrict__ arows, int64_t rows_valid,
                          const char* __restrict__ B, int64_t K, int64_t N,
                          int64_t n0, int64_t k0)
    {
        const int tid = threadIdx.x;
#pragma unroll
        for (int u = 0; u < kAVec; ++u) {
            const int q = tid + u * kThreads;
            const int row = q >> 3, piece = q & 7;
            const int64_t k = k0 + (int64_t)piece * (16 / T::kElt);
            if (row < rows_valid && k < K)
                a_reg[u] = *reinterpret_cast<const uint4*>(arows + (row * K + k) * T::kElt);
            else
                a_reg[u] = make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kBBlk; ++u) {
            const int b = tid + u * kThreads;
            if (b < BN) {
                const int nb = b % (BN / 8), kb = b / (BN / 8);
                T::load_b(B, N, K, k0 + (int64_t)kb * T::kBRows, n0 + nb * 8, b_reg[u]);
            }
        }
    }

    __device__ void sstore(char* lds)
    {
        const int tid = threadIdx.x;
        char* As = lds;
        char* Bs = lds + BM * kRowBytes;
#pragma unroll
        for (int u = 0; u < kAVec; ++u) {
            const int q = tid + u * kThreads;
            *reinterpret_cast<uint4*>(As + lds_off(q >> 3, q & 7)) = a_reg[u];
        }
#pragma unroll
        for (int u = 0; u < kBBlk; ++u) {
            const int b = tid + u * kThreads;
            if (b < BN) {
                const int nb = b % (BN / 8), kb = b / (BN / 8);
                uint4 col[8];
                T::transpose_b(b_reg[u], col);
#pragma unroll
                for (int c = 0; c < 8; ++c)
                    *reinterpret_cast<uint4*>(Bs + lds_off(nb * 8 + c, kb)) = col[c];
            }
        }
    }

    __device__ void compute(const char* lds, typename T::Acc (&acc)[kTM][kTN])
    {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int wm = (wave >> 1) * (BM / 2), wn = (wave & 1) * (BN / 2);
        const char* As = lds;
        const char* Bs = lds + BM * kRowBytes;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int piece = 2 * kk + (lane >> 5);
            uint4 af[kTM], bf[kTN];
#pragma unroll
            for (int i = 0; i < kTM; ++i)
                af[i] = *reinterpret_cast<const uint4*>(As + lds_off(wm + i * 32 + (lane & 31), piece));
#pragma unroll
            for (int j = 0; j < kTN; ++j)
                bf[j] = *reinterpret_cast<const uint4*>(Bs + lds_off(wn + j * 32 + (lane & 31), piece));
#pragma unroll
            for (int i = 0; i < kTM; ++i)
#pragma unroll
                for (int j = 0; j < kTN; ++j)
                    acc[i][j] = T::mma(af[i], bf[j], acc[i][j]);
        }
    }
};

// Output row of accumulator element r of lane `lane` in a 32x32 block.
__device__ __forceinline__ int acc_row(int lane, int r)
{
    return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

template <class T, int BM, int BN>
__device__ __forceinline__ void store_tile(const ConsumerArgs& a, int shard, int m,
                                           int n, typename T::Acc (&acc)[BM / 64][BN / 64])
{
    const Schedule& s = a.s;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = (wave >> 1) * (BM / 2), wn = (wave & 1) * (BN / 2);
    const int64_t row0 = (int64_t)m * BM;          // within the shard
    const int64_t col0 = (int64_t)n * BN;
    const int64_t out_row0 = (int64_t)shard * s.S; // shard's first row of C
#pragma unroll
    for (int i = 0; i < BM / 64; ++i) {
#pragma unroll
        for (int j = 0; j < BN / 64; ++j) {
            const int64_t col = col0 + wn + j * 32 + (lane & 31);
            if (col >= s.N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = row0 + wm + i * 32 + acc_row(lane, r);
                if (row >= s.S) continue;
                const int64_t idx = (out_row0 + row) * s.N + col;
                if constexpr (T::kElt == 2) {
                    static_cast<float*>(a.C)[idx] = acc[i][j][r];
                } else {
                    const int32_t v = (int32_t)((uint32_t)acc[i][j][r] + (uint32_t)a.bias[col]);
                    if (a.acc_out) a.acc_out[idx] = v;
                    const float f = (float)v * a.scale[col];
                    static_cast<_Float16*>(a.C)[idx] = (_Float16)f;
                }
            }
        }
    }
}

template <class T, int BM, int BN>
__global__ __launch_bounds__(kThreads, 1) void consumer_kernel(ConsumerArgs a)
{
    typedef Engine<T, BM, BN> E;
    extern __shared__ __attribute__((aligned(16))) char lds[];
    __shared__ uint32_t seen_sh[kMaxShards];
    __shared__ int ok_sh;

    const Schedule& s = a.s;
    const int tid = threadIdx.x;
    for (int i = tid; i < kMaxShards; i += kThreads) seen_sh[i] = 0;
    __syncthreads();

    const int64_t tiles = total_tiles(s);
    const int nk = (int)cdiv(s.K, T::kBK);
    E eng;

    for (int64_t p = blockIdx.x; p < tiles; p += gridDim.x) {
        const TileRef t = tile_at(s, p);
        if (t.need > 0 && !a.no_wait) {
            if (tid == 0) {
                int ok = 1;
                if (seen_sh[t.shard] < (uint32_t)t.need) {
                    const uint32_t target = a.base[t.shard] + (uint32_t)t.need;
                    const uint32_t v = acquire_wait(a.counters + t.shard * (kCounterStride / 4),
                                                    target, a.err, a.epoch, a.limit);
                    if (reached(v, target)) seen_sh[t.shard] = v - a.base[t.shard];
                    else ok = 0;
                }
                ok_sh = ok;
            }
            __syncthreads();
            if (!ok_sh) break;   // the call has failed; every lane leaves
        }

        const int64_t row0 = (int64_t)t.m * BM;
        const int64_t rows_valid = s.S - row0;
        const char* arows = a.a[t.shard] + row0 * s.K * T::kElt;
        const int64_t n0 = (int64_t)t.n * BN;

        typename T::Acc acc[BM / 64][BN / 64];
#pragma unroll
        for (int i = 0; i < BM / 64; ++i)
#pragma unroll
            for (int j = 0; j < BN / 64; ++j) acc[i][j] = T::zero();

        if (nk > 0) {
            eng.gload(arows, rows_valid, a.B, s.K, s.N, n0, 0);
            eng.sstore(lds);
            __syncthreads();
            for (int kt = 0; kt < nk; ++kt) {
                const int cur = kt & 1;
                if (kt + 1 < nk)
                    eng.gload(arows, rows_valid, a.B, s.K, s.N, n0,
                              (int64_t)(kt + 1) * T::kBK);
                eng.compute(lds + cur * E::kStage, acc);
                if (kt + 1 < nk) eng.sstore(lds + (cur ^ 1) * E::kStage);
                __syncthreads();
            }
        }
        store_tile<T, BM, BN>(a, t.shard, t.m, t.n, acc);
    }
}

template <class T, int BM, int BN>
hipError_t launch_one(const ConsumerArgs& a, int wgs, hipStream_t st)
{
    const size_t lds = 2 * (size_t)Engine<T, BM, BN>::kStage;
    auto kern = consumer_kernel<T, BM, BN>;
    static bool attr_set = false;   // one-time opt-in to > 64 KiB of LDS
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3(wgs), dim3(kThreads), lds, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_consumer_f16(const ConsumerArgs& a, int tile_id, int wgs, hipStream_t st)
{
    switch (tile_id) {
    case 1: return launch_one<F16, 256, 256>(a, wgs, st);
    case 2: return launch_one<F16, 128, 128>(a, wgs, st);
    case 3: return launch_one<F16, 64, 64>(a, wgs, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_consumer_i8(const ConsumerArgs& a, int tile_id, int wgs, hipStream_t st)
{
    switch (tile_id) {
    case 1: return launch_one<I8, 256, 256>(a, wgs, st);
    case 2: return launch_one<I8, 128, 128>(a, wgs, st);
    case 3: return launch_one<I8, 64, 64>(a, wgs, st);
    default: return hipErrorInvalidValue;
    }
}

int consumer_occupancy(int kind, int tile_id)
{
    int n = 0;
    size_t lds = 0;
    const void* f = nullptr;
    if (kind == 0) {
        switch (tile_id) {
        case 1: f = (const void*)consumer_kernel<F16, 256, 256>; lds = 2 * Engine<F16, 256, 256>::kStage; break;
        case 2: f = (const void*)consumer_kernel<F16, 128, 128>; lds = 2 * Engine<F16, 128, 128>::kStage; break;
        case 3: f = (const void*)consumer_kernel<F16, 64, 64>; lds = 2 * Engine<F16, 64, 64>::kStage; break;
        }
    } else {
        switch (tile_id) {
        case 1: f = (const void*)consumer_kernel<I8, 256, 256>; lds = 2 * Engine<I8, 256, 256>::kStage; break;
        case 2: f = (const void*)consumer_kernel<I8, 128, 128>; lds = 2 * Engine<I8, 128, 128>::kStage; break;
        case 3: f = (const void*)consumer_kernel<I8, 64, 64>; lds = 2 * Engine<I8, 64, 64>::kStage; break;
        }
    }
    if (!f) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, kThreads, lds) != hipSuccess)
        return 0;
    return n;
}

}  // namespace agg
