// consumer.hip -- the persistent MFMA consumer GEMM (fp16 -> fp32, its
// bf16 -> fp32 and fp8 (E4M3) -> fp32 variants, and int8 -> int32 + bias
// -> per-channel dequant -> fp16).
//
// One workgroup per CU walks the tile list of the shared schedule: first
// the local shard's tiles (no wait), then the remote tiles in the order
// their rows arrive (PTO-ISA AllGather+GEMM README: phase 1 computes the
// local row-group with no wait, phase 2 waits on each remote source's
// summary counter and computes as soon as the rows are there).  Before a
// remote tile, wave 0 waits until the chunks of the tile's rows in its
// first K-block are released (the source's counter, or the chunk flags);
// inside the K loop it waits again only where a slice enters a K-block not
// yet known to be in.  What a workgroup has already seen of a source is
// remembered, so most waits pass without touching memory.
//
// Tile main loop (PTO-ISA README: continuous K accumulation, multi-level
// buffering): WM x WN waves (four, or eight with two per SIMD), each owning
// a (BM/WM) x (BN/WN) block of 32x32 MFMA accumulators kept in registers
// for the whole K loop.  K is walked in slices of SB bytes per row; NS
// slices live in an LDS ring, NS-1 of them in flight from HBM while the
// oldest is multiplied.  Inside a slice the operand reads of MFMA step s+1
// are issued between the MFMAs of step s, and the last step's MFMAs run
// across the barrier that publishes the next slice.
//
// HBM -> LDS moves use the gfx950 direct global-to-LDS load (16 bytes per
// lane, written lane by lane at the instruction's LDS base), so no
// registers stage the tiles.  Each slice's loads go through buffer
// descriptors that end where the matrix does, and a lane whose piece lies
// beyond K or N gets an out-of-range offset: such loads return zeros.  A is stored as it lies in memory
// (row = output row, k along the row); B is stored row-major too (row = k)
// and read with the LDS transpose loads, which hand each lane consecutive k
// of one column.  16-byte pieces are XOR-swizzled per row, the swizzle
// applied by choosing which global piece each lane fetches.
#include <type_traits>

#include "kernels.hpp"
#include "producer_body.hpp"
#include "sync.hpp"

namespace agg {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef int intx16 __attribute__((ext_vector_type(16)));
typedef int intx2 __attribute__((ext_vector_type(2)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef short short4_ __attribute__((ext_vector_type(4)));
#define LDS_PTR __attribute__((address_space(3)))
#define GLB_PTR __attribute__((address_space(1)))

constexpr int kLdsBytes = 163840;
// Buffer descriptor word 3 for untyped 32-bit accesses, and an offset no
// buffer of this code reaches (range checks return zero for it).
constexpr int kRsrcWord3 = 0x00020000;
constexpr uint32_t kOutOfRange = 0x80000000u;

// ---- element traits ---------------------------------------------------
//
// Every path moves 16-byte pieces: 8 fp16 or 16 int8 / fp8 values along K.
// An MFMA operand is kPair pieces per lane: lanes 0-31 and 32-63 take
// pieces 2q and 2q + 1 of each 32-byte group q of K, for q = 0..kPair-1, in
// A (row of the lane) and in B (column of the lane) alike, so the k that
// one instruction sums over are the same in both operands.  Inside every
// 16-lane group, lane i of a b16 transpose load receives element i % 4 of
// the 8 bytes loaded by lane 4e + i/4 (e = 0..3), and of a b8 transpose
// load byte i % 8 of lane 2e + i/8 (e = 0..7).

struct F16 {
    static constexpr int kElt = 2;        // bytes per element
    static constexpr int kPair = 1;       // 16-byte pieces per MFMA operand
    static constexpr int kBlk = 32;       // MFMA block: kBlk x kBlk outputs
    static constexpr int kAccN = 16;      // accumulators per lane and block
    static constexpr bool kRoll = false;  // one rolling operand set (see Engine)
    static constexpr bool kDequant = false;
    typedef floatx16 Acc;
    typedef float Out;                    // element of C

    __device__ static Acc zero() { Acc z; for (int i = 0; i < 16; ++i) z[i] = 0.f; return z; }

    __device__ static Acc mma(const uint4 (&a)[1], const uint4 (&b)[1], const Acc& c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(
            __builtin_bit_cast(half8, a[0]), __builtin_bit_cast(half8, b[0]), c, 0, 0, 0);
    }

    // B piece swizzle, LB bytes per B row in LDS.  The LDS has 64 banks of
    // 4 bytes, and a b64 read is served 32 lanes (256 bytes) at a time: two
    // 16-lane groups that read 4 rows x 32 bytes each, 16 pieces in all.
    // Rows of 256 bytes or more all start at bank 0, so rows k % 4 = 0..3
    // take pieces 4(k % 4) + 0..3; rows of 128 bytes alternate halves of
    // the banks, so rows k and k + 2 are set apart instead.  It depends only
    // on k % 4 (and k / 2 % 2), which the slice's other reads, 4 and 16 rows
    // on, leave unchanged.
    template <int LB>
    __device__ static int swz_b(int k)
    {
        return LB >= 256 ? 4 * (k & 3) : 4 * ((k >> 1) & 1);
    }

    // B operand of 32 columns, MFMA step kk of the slice: 8 values
    // k = 16kk + 8(lane/32) + 0..7 from two b16 transpose loads.  b_offset
    // gives the lane's address of the first load (step 0, half 0) within a
    // stage's B part; the other loads of the slice are 4 and 16 rows on,
    // which the swizzle leaves unchanged (it only looks at k % 4 and
    // k / 8 % 2 of rows 0..15 of a group).
    template <int LB>
    __device__ static int b_offset(int lane, int n_base)
    {
        const int g = lane >> 4, jj = lane & 15;
        const int n = n_base + 16 * (g & 1) + 4 * (jj & 3);      // first of 4 halves
        const int k = 8 * (g >> 1) + (jj >> 2);
        const int phys = (n >> 3) ^ (swz_b<LB>(k) & (LB / 16 - 1));
        return k * LB + phys * 16 + (n & 7) * 2;
    }

    template <int LB>
    __device__ static uint4 read_b(const char* p, int kk)
    {
        short4_ v[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
            v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (LDS_PTR short4_*)(p + (16 * kk + 4 * h) * LB));
        uint2 lo = __builtin_bit_cast(uint2, v[0]), hi = __builtin_bit_cast(uint2, v[1]);
        return make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
};

// bfloat16: the fp16 engine (same 16-bit layout, swizzles and transpose
// reads) with the bf16 MFMA.
struct BF16 : F16 {
    __device__ static Acc mma(const uint4 (&a)[1], const uint4 (&b)[1], const Acc& c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, a[0]), __builtin_bit_cast(bf16x8, b[0]), c, 0, 0, 0);
    }
};

struct I8 {
    static constexpr int kElt = 1;
    static constexpr int kPair = 1;
    static constexpr int kBlk = 32;
    static constexpr int kAccN = 16;
    static constexpr bool kRoll = false;
    static constexpr bool kDequant = true;   // + bias, x scale, -> fp16
    typedef intx16 Acc;
    typedef _Float16 Out;

    __device__ static Acc zero() { Acc z; for (int i = 0; i < 16; ++i) z[i] = 0; return z; }

    __device__ static Acc mma(const uint4 (&a)[1], const uint4 (&b)[1], const Acc& c)
    {
        return __builtin_amdgcn_mfma_i32_32x32x32_i8(
            __builtin_bit_cast(intx4, a[0]), __builtin_bit_cast(intx4, b[0]), c, 0, 0, 0);
    }

    // B piece swizzle: a b64 read's 32 lanes read 8 rows x 32 bytes, 16
    // pieces in all.  Rows of 256 bytes or more start at bank 0 and take
    // pieces 2(k % 8) + 0..1; rows of 128 bytes alternate halves of the
    // banks, so the even rows (and the odd ones) are spread by k / 2 % 4.
    // Reads 8 and 32 rows on keep the same swizzle.
    template <int LB>
    __device__ static int swz_b(int k)
    {
        return LB >= 256 ? 2 * (k & 7) : 2 * ((k >> 1) & 3);
    }

    // B operand: 16 values k = 32kk + 16(lane/32) + 0..15 from two b8
    // transpose loads, 8 and 32 rows apart (the swizzle only looks at
    // k % 8).
    template <int LB>
    __device__ static int b_offset(int lane, int n_base)
    {
        const int g = lane >> 4, jj = lane & 15;
        const int n = n_base + 16 * (g & 1) + 8 * (jj & 1);      // first of 8 bytes
        const int k = 16 * (g >> 1) + (jj >> 1);
        const int phys = (n >> 4) ^ (swz_b<LB>(k) & (LB / 16 - 1));
        return k * LB + phys * 16 + (n & 15);
    }

    template <int LB>
    __device__ static uint4 read_b(const char* p, int kk)
    {
        intx2 v[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
            v[h] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (LDS_PTR intx2*)(p + (32 * kk + 8 * h) * LB));
        return make_uint4(v[0][0], v[0][1], v[1][0], v[1][1]);
    }
};

// OCP FP8 E4M3: the int8 byte layout (swizzles, transpose reads), fp32
// accumulators, and the gfx950 fp8 MFMA that sums 64 k per instruction,
// 32 bytes per lane: two 16-byte pieces.  Format code 0 in both operands
// selects E4M3; zero scale operands select the unscaled instruction.
struct FP8 : I8 {
    static constexpr int kPair = 2;
    static constexpr bool kDequant = false;
    typedef floatx16 Acc;
    typedef float Out;

    __device__ static Acc zero() { Acc z; for (int i = 0; i < 16; ++i) z[i] = 0.f; return z; }

    __device__ static Acc mma(const uint4 (&a)[2], const uint4 (&b)[2], const Acc& c)
    {
        const intx8 av = {(int)a[0].x, (int)a[0].y, (int)a[0].z, (int)a[0].w,
                          (int)a[1].x, (int)a[1].y, (int)a[1].z, (int)a[1].w};
        const intx8 bv = {(int)b[0].x, (int)b[0].y, (int)b[0].z, (int)b[0].w,
                          (int)b[1].x, (int)b[1].y, (int)b[1].z, (int)b[1].w};
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 0, 0, 0, 0, 0, 0);
    }
};

// fp8 on the eight-wave 256 x 256 tile: the same 32 x 32 blocks, with one
// rolling operand set (two sets of 32-byte operands would not fit beside
// the 128 accumulators of a 128 x 64 wave block and a producer wave).
struct FP8x : FP8 {
    static constexpr bool kRoll = true;
};

// 16 x 16 blocks (v_mfma_*_16x16x32 for 16-bit inputs, 16x16x64 for int8):
// the same products in instructions that draw less power per flop than the
// 32 x 32 ones -- with operands that toggle many bits the board's power
// limit holds them at a higher clock (2.13 against 1.79 GHz in the
// register-only probe, 19% more flops per second).  Lane l holds row
// (column) l % 16 of a block and k = 8(l / 16) + 0..7 of a 32-element
// group of K (16-bit; int8: 16(l / 16) + 0..15 of 64), so an operand is
// still one 16-byte piece, and a step covers 64 bytes of K: lane group
// l / 16 takes piece 4q + l / 16 of group q.  Accumulator r (0..3) of lane
// l is row 4(l / 16) + r, column l % 16.  B is read with the same
// transpose loads, lane group g taking rows 8g.. (16-bit; int8: 16g..) of
// all 16 columns; the swizzle spreads the 16 pieces a half-wave reads (rows
// k and k + 8 of it, int8: k and k + 16) over distinct banks, for rows of
// 256 bytes or more.
struct F16x {
    static constexpr int kElt = 2;
    static constexpr int kPair = 1;
    static constexpr int kBlk = 16;
    static constexpr int kAccN = 4;
    static constexpr bool kRoll = true;
    static constexpr bool kDequant = false;
    typedef floatx4 Acc;
    typedef float Out;

    __device__ static Acc zero() { Acc z; for (int i = 0; i < 4; ++i) z[i] = 0.f; return z; }

    __device__ static Acc mma(const uint4 (&a)[1], const uint4 (&b)[1], const Acc& c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(
            __builtin_bit_cast(half8, a[0]), __builtin_bit_cast(half8, b[0]), c, 0, 0, 0);
    }

    template <int LB>
    __device__ static int swz_b(int k)
    {
        static_assert(LB >= 256, "16-column blocks read rows of 256 bytes or more");
        return 2 * (k & 3) + 8 * ((k >> 3) & 1);
    }

    // lane group g = lane / 16 reads rows 8g + (lane % 16) / 4 (and 4 on),
    // 4 columns each, so that lane i of the group receives column i
    template <int LB>
    __device__ static int b_offset(int lane, int n_base)
    {
        const int g = lane >> 4, jj = lane & 15;
        const int n = n_base + 4 * (jj & 3);
        const int k = 8 * g + (jj >> 2);
        const int phys = (n >> 3) ^ (swz_b<LB>(k) & (LB / 16 - 1));
        return k * LB + phys * 16 + (n & 7) * 2;
    }

    template <int LB>
    __device__ static uint4 read_b(const char* p, int kk)
    {
        short4_ v[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
            v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (LDS_PTR short4_*)(p + (32 * kk + 4 * h) * LB));
        uint2 lo = __builtin_bit_cast(uint2, v[0]), hi = __builtin_bit_cast(uint2, v[1]);
        return make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
};

struct BF16x : F16x {
    __device__ static Acc mma(const uint4 (&a)[1], const uint4 (&b)[1], const Acc& c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, a[0]), __builtin_bit_cast(bf16x8, b[0]), c, 0, 0, 0);
    }
};

struct I8x {
    static constexpr int kElt = 1;
    static constexpr int kPair = 1;
    static constexpr int kBlk = 16;
    static constexpr int kAccN = 4;
    static constexpr bool kRoll = true;
    static constexpr bool kDequant = true;
    typedef intx4 Acc;
    typedef _Float16 Out;

    __device__ static Acc zero() { Acc z; for (int i = 0; i < 4; ++i) z[i] = 0; return z; }

    __device__ static Acc mma(const uint4 (&a)[1], const uint4 (&b)[1], const Acc& c)
    {
        return __builtin_amdgcn_mfma_i32_16x16x64_i8(
            __builtin_bit_cast(intx4, a[0]), __builtin_bit_cast(intx4, b[0]), c, 0, 0, 0);
    }

    template <int LB>
    __device__ static int swz_b(int k)
    {
        static_assert(LB >= 256, "16-column blocks read rows of 256 bytes or more");
        return (k & 7) + 8 * ((k >> 4) & 1);
    }

    // lane group g reads rows 16g + (lane % 16) / 2 (and 8 on), 8 columns
    // each, so that lane i of the group receives column i
    template <int LB>
    __device__ static int b_offset(int lane, int n_base)
    {
        const int g = lane >> 4, jj = lane & 15;
        const int n = n_base + 8 * (jj & 1);
        const int k = 16 * g + (jj >> 1);
        const int phys = (n >> 4) ^ (swz_b<LB>(k) & (LB / 16 - 1));
        return k * LB + phys * 16 + (n & 15);
    }

    template <int LB>
    __device__ static uint4 read_b(const char* p, int kk)
    {
        intx2 v[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
            v[h] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (LDS_PTR intx2*)(p + (64 * kk + 8 * h) * LB));
        return make_uint4(v[0][0], v[0][1], v[1][0], v[1][1]);
    }
};

// The lane index, hidden from the optimiser: addresses derived from it are
// recomputed where they are used (a few VALU ops beside the MFMAs) instead
// of being hoisted out of the K loop, where they would pin dozens of
// registers.
__device__ __forceinline__ int opaque_lane()
{
    int l = threadIdx.x & 63;
    asm volatile("" : "+v"(l));
    return l;
}

// s_waitcnt with vmcnt(n), lgkmcnt(0), expcnt untouched (gfx9 encoding).
template <int n>
__device__ __forceinline__ void wait_vm_lgkm0()
{
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4));
}

// A value every lane of the workgroup holds alike (read back from LDS after
// a barrier), marked as such: the compiler cannot tell that an LDS read is
// uniform, and a branch or address that depends on one would otherwise be
// taken as divergent -- every buffer descriptor derived from it would sit in
// vector registers and each load would be wrapped in a loop over its
// distinct values.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint32_t uniform(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

// A buffer descriptor over `bytes` bytes from p (at most 2^31 - 1), built
// from scalar registers.  Its fields are the same in every lane, but they
// are often computed with vector instructions (64-bit products and
// divisions have no scalar form), and a descriptor left in vector
// registers makes the compiler wrap every load and store through it in a
// loop over the lanes' distinct values.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t scalar_rsrc(const void* p, int64_t bytes)
{
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint64_t base = (uint64_t)uniform((uint32_t)a) | ((uint64_t)uniform((uint32_t)(a >> 32)) << 32);
    const int n = uniform((int)(bytes < 0x7fffffff ? bytes : 0x7fffffff));
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(base), 0, n, kRsrcWord3);
}

// Workgroup barrier without the release/acquire fences of __syncthreads:
// those would wait for every load still in flight, including the slices
// being prefetched.  Callers wait for exactly what the barrier publishes
// (their own finished loads and LDS reads) before it.  The empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void bare_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ---- the tile engine --------------------------------------------------

template <class T, int BM, int BN, int SB, int NS, int WM, int WN>
struct Engine {
    static constexpr int kWaves = WM * WN;          // WM x WN grid of waves
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kBE = T::kBlk;             // MFMA block edge (32 or 16)
    static constexpr int kTM = BM / (kBE * WM);     // blocks per wave along M
    static constexpr int kTN = BN / (kBE * WN);     // ... along N
    static constexpr int kPieces = SB / 16;         // 16-byte pieces per A row
    static constexpr int kP = T::kPair;             // pieces per MFMA operand
    static constexpr int kLG = 64 / kBE;            // lane groups: pieces per K group
    static constexpr int kHalfSteps = SB / (16 * kLG);  // K groups per slice
    static constexpr int kSteps = kHalfSteps / kP;  // MFMA steps per slice
    // The eight-wave 256 x 256 tile on 16 x 16 blocks (and fp8's 32-byte
    // operands on 32 x 32 blocks) keeps one operand set, each block re-read
    // for the next step as soon as its last MFMA of this one is issued (two
    // sets would not fit beside the accumulators); the other configurations
    // alternate two sets
    static constexpr bool kRoll = T::kRoll;
    static constexpr int kBK = SB / T::kElt;        // k per slice
    static constexpr int kLB = BN * T::kElt;        // bytes per B row in LDS
    static constexpr int kABytes = BM * SB;         // A part of a stage
    static constexpr int kBBytes = kBK * kLB;       // B part of a stage
    static constexpr int kStage = kABytes + kBBytes;
    static constexpr int kLds = NS * kStage;
    static constexpr int kAInstr = kABytes / 1024;  // 1 KiB per load instruction
    static constexpr int kBInstr = kBBytes / 1024;
    static constexpr int kGroup = (kAInstr + kBInstr) / kWaves;   // loads per wave per slice
    static_assert(kAInstr % kWaves == 0 && kBInstr % kWaves == 0, "loads split over the waves");
    static_assert(kTM >= 1 && kTN >= 1 && kWaves % 4 == 0, "wave grid");
    static_assert(kSteps % 2 == 0 && NS >= 2 && NS <= 8, "pipeline shape");
    static_assert(kLds + 1024 <= kLdsBytes, "LDS ring too large");
    static_assert(kGroup * (NS - 2) < 64, "vmcnt range");

    static constexpr int kAPer = kAInstr / kWaves;  // A loads per wave per slice
    static constexpr int kBPer = kBInstr / kWaves;  // B loads per wave per slice

    // A piece swizzle: the 16 rows of a quarter-wave reading one piece land
    // on 16 distinct 16-byte bank groups.  Rows 32 apart share it.
    __device__ static int swz_a(int r) { return (r / (256 / SB)) % kPieces; }

    struct Src {
        const char* arows;   // first A row of the tile
        int64_t rows_valid;  // A rows that exist
        const char* B;
        int64_t K, N, n0;
        int64_t kb;          // first k of the tile's K range (split-K part)
    };

    // Per-lane byte offsets, computed once per kernel: where this lane's
    // pieces come from (relative to a slice's A and B origins) and where its
    // MFMA operands sit in a stage.  All loads and LDS reads of the K loop
    // are these plus uniform or immediate offsets.
    struct Lane {
        uint32_t a_ld[kAPer];   // A piece of load u: row * K + k, in bytes
        uint32_t b_ld[kBPer];   // B piece of load u: row * N + n, in bytes
        uint32_t a_rd[kHalfSteps];  // A piece of K group g, block 0
        uint32_t b_rd[kTN];     // first transpose load of block j (step 0, half 0)
    };

    __device__ static void lane_offsets(Lane& L, int64_t K, int64_t N)
    {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int wm = (wave / WN) * (BM / WM), wn = (wave % WN) * (BN / WN);
#pragma unroll
        for (int u = 0; u < kAPer; ++u) {
            const int q = wave * kAPer + u;
            const int r = q * (1024 / SB) + lane / kPieces;
            const int p = (lane % kPieces) ^ swz_a(r);
            L.a_ld[u] = (uint32_t)(r * K * T::kElt + p * 16);
        }
#pragma unroll
        for (int u = 0; u < kBPer; ++u) {
            const int q = wave * kBPer + u;
            const int pos = q * 1024 + lane * 16;
            const int r = pos / kLB;
            const int p = ((pos % kLB) >> 4) ^ (T::template swz_b<kLB>(r) & (kLB / 16 - 1));
            L.b_ld[u] = (uint32_t)(r * N * T::kElt + p * 16);
        }
#pragma unroll
        for (int g = 0; g < kHalfSteps; ++g) {
            const int r = wm + (lane % kBE);
            const int piece = kLG * g + lane / kBE;
            L.a_rd[g] = (uint32_t)(r * SB + ((piece ^ swz_a(r)) << 4));
        }
#pragma unroll
        for (int j = 0; j < kTN; ++j)
            L.b_rd[j] = (uint32_t)(kABytes + T::template b_offset<kLB>(lane, wn + j * kBE));
    }

    // Loads of one slice into `stage`.  Rows of A past the tile and rows of
    // B past K fall outside the buffer ranges and read as zero; on an edge
    // slice (K not reached by a whole slice, or the tile past N) the lanes
    // whose piece lies beyond K or N are pushed out of range too.
    __device__ static void load_slice(char* stage, const Src& src, const Lane& L, int64_t k0)
    {
        const int64_t elt = T::kElt;
        const int64_t a_left = (src.rows_valid * src.K - k0) * elt;
        const int64_t b_left = ((src.K - k0) * src.N - src.n0) * elt;
        const __amdgpu_buffer_rsrc_t ra = scalar_rsrc(src.arows + k0 * elt, a_left);
        const __amdgpu_buffer_rsrc_t rb = scalar_rsrc(src.B + (k0 * src.N + src.n0) * elt, b_left);
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const bool edge = k0 + kBK > src.K || src.n0 + BN > src.N;
        if (!edge) {
#pragma unroll
            for (int u = 0; u < kAPer; ++u)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    ra, (LDS_PTR void*)(stage + (wave * kAPer + u) * 1024), 16, L.a_ld[u], 0,
                    0, 0);
#pragma unroll
            for (int u = 0; u < kBPer; ++u)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rb, (LDS_PTR void*)(stage + kABytes + (wave * kBPer + u) * 1024), 16,
                    L.b_ld[u], 0, 0, 0);
            return;
        }
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int u = 0; u < kAPer; ++u) {
            const int q = wave * kAPer + u;
            const int r = q * (1024 / SB) + lane / kPieces;
            const int p = (lane % kPieces) ^ swz_a(r);
            const bool in = k0 + p * (16 / T::kElt) < src.K;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ra, (LDS_PTR void*)(stage + q * 1024), 16, in ? L.a_ld[u] : kOutOfRange, 0, 0,
                0);
        }
#pragma unroll
        for (int u = 0; u < kBPer; ++u) {
            const int q = wave * kBPer + u;
            const int pos = q * 1024 + lane * 16;
            const int r = pos / kLB;
            const int p = ((pos % kLB) >> 4) ^ (T::template swz_b<kLB>(r) & (kLB / 16 - 1));
            const bool in = src.n0 + p * (16 / T::kElt) < src.N;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rb, (LDS_PTR void*)(stage + kABytes + q * 1024), 16,
                in ? L.b_ld[u] : kOutOfRange, 0, 0, 0);
        }
    }

    // Operand fragments of one MFMA step (32 kP bytes of K): kP pieces per
    // lane for each of the kTM A blocks and kTN B blocks.
    struct Step {
        uint4 a[kTM][kP];
        uint4 b[kTN][kP];
    };

    __device__ __forceinline__ static void read_step(const char* st, const Lane& L, int kk,
                                                     Step& f)
    {
#pragma unroll
        for (int q = 0; q < kP; ++q) {
            // in the order the step's first MFMAs use them: A block 0,
            // every B block, then the other A blocks
            f.a[0][q] = *reinterpret_cast<const uint4*>(st + L.a_rd[kP * kk + q]);
#pragma unroll
            for (int j = 0; j < kTN; ++j)
                f.b[j][q] = T::template read_b<kLB>(st + L.b_rd[j], kP * kk + q);
#pragma unroll
            for (int i = 1; i < kTM; ++i)
                f.a[i][q] = *reinterpret_cast<const uint4*>(st + L.a_rd[kP * kk + q] +
                                                            i * kBE * SB);
        }
    }

    __device__ __forceinline__ static void mma_step(const Step& f,
                                                    typename T::Acc (&acc)[kTM][kTN])
    {
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
            for (int j = 0; j < kTN; ++j)
                acc[i][j] = T::mma(f.a[i], f.b[j], acc[i][j]);
    }

    // Issue order inside one MFMA step: the LDS reads of the next step
    // two after each of the first MFMAs, so the reads overlap the matrix
    // pipe instead of queueing in front of it (one wave per SIMD cannot
    // hide a stall otherwise), and the last of them still has half a step
    // to land.  (One read after each MFMA measured 1.1-1.4% slower on the
    // 8 x 1024-row fp16 shape, compute-only; four after each of the first
    // two, the same as two.)
    __device__ __forceinline__ static void interleave_reads()
    {
        constexpr int kR = kP * (kTM + 2 * kTN);   // LDS reads per step
        constexpr int kM = kTM * kTN;       // MFMAs per step
#pragma unroll
        for (int i = 0; i < kM; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
            if (2 * i + 1 < kR) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // two LDS reads
            else if (2 * i < kR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
    }

    // One operand set: the MFMAs of one step on the operands in f, column
    // block by column block, each operand block of f re-read from step kk
    // of `st` once its last MFMA here is issued: B block j after the column's
    // kTM MFMAs (kTN (kTM - 1) + 1 MFMAs ahead of its next use), A block i
    // after its MFMA in the last column (kTM - 1 MFMAs ahead).  A fence after
    // each MFMA and its reads keeps that order.
    __device__ __forceinline__ static void step_roll(Step& f, const char* st, const Lane& L,
                                                     int kk, typename T::Acc (&acc)[kTM][kTN])
    {
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
#pragma unroll
            for (int i = 0; i < kTM; ++i) {
                acc[i][j] = T::mma(f.a[i], f.b[j], acc[i][j]);
#pragma unroll
                for (int q = 0; q < kP; ++q) {
                    if (j == kTN - 1)
                        f.a[i][q] = *reinterpret_cast<const uint4*>(
                            st + L.a_rd[kP * kk + q] + i * kBE * SB);
                    if (i == kTM - 1)
                        f.b[j][q] = T::template read_b<kLB>(st + L.b_rd[j], kP * kk + q);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

    // Wait until at most `behind` slices of this wave's loads are still in
    // flight (and every LDS read has returned).
    // `behind` is at most NS - 2.
    template <int kB = NS - 2>
    __device__ __forceinline__ static void wait_slices(int behind)
    {
        if constexpr (kB > 0) {
            if (behind >= kB) { wait_vm_lgkm0<kB * kGroup>(); return; }
            wait_slices<kB - 1>(behind);
        } else {
            wait_vm_lgkm0<0>();
        }
    }

    // One k-slice.  On entry f0 holds step 0 of `cur`; on exit it holds
    // step 0 of `nxt` (when there is a next slice).  `ld` is the stage that
    // receives slice kt + NS - 1.  The three stages are distinct
    // (restrict), so the compiler does not make the reads wait for the
    // loads; the explicit waits below do the ordering that matters.
    __device__ __attribute__((always_inline)) static void slice(
        const char* __restrict__ cur, const char* __restrict__ nxt, char* __restrict__ ld,
        bool load, int64_t k_load, int behind, bool more, const Src& src, const Lane& L,
        Step& f0, Step& f1, typename T::Acc (&acc)[kTM][kTN])
    {
        if (load) load_slice(ld, src, L, k_load);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kRoll) {
            // f0 is the one operand set: step st - 1's MFMAs, step st's reads
#pragma unroll
            for (int st = 1; st < kSteps; ++st) step_roll(f0, cur, L, st, acc);
            wait_slices(behind);
            bare_barrier();
            step_roll(f0, nxt, L, 0, acc);
            return;
        }
#pragma unroll
        for (int st = 1; st < kSteps; ++st) {
            read_step(cur, L, st, (st & 1) ? f1 : f0);
            mma_step((st & 1) ? f0 : f1, acc);
            interleave_reads();
            __builtin_amdgcn_sched_barrier(0);
        }
        // the next slice has landed for this wave; every wave is done with
        // reading `cur`, which a later slice's loads will overwrite
        wait_slices(behind);
        bare_barrier();
        // after the last slice this reads a stage nobody uses again (still
        // inside the ring); reading unconditionally keeps the reads and the
        // MFMAs in one scheduling region
        read_step(nxt, L, 0, f0);
        mma_step(f1, acc);
        interleave_reads();
        __builtin_amdgcn_sched_barrier(0);
    }

    // The whole K loop of one tile over the NS stages starting at `ring`.
    // The previous tile left no load in flight (its last slice waited for
    // all of them) and no LDS read pending (its last barrier came after
    // them), so the ring can be refilled at once.  gate(k) is called, by
    // every wave alike, before the loads of each slice after the first
    // NS - 1 (k: the slice's first element).  (The loop has no early exit:
    // one would make the register allocator give up the accumulators'
    // registers; a gate that fails lets the tile run on, and the caller
    // drops it.)
    template <class Gate>
    __device__ __attribute__((always_inline)) static void run(
        char* ring, int nk, const Src& src, const Lane& L, typename T::Acc (&acc)[kTM][kTN],
        Gate& gate)
    {
#pragma unroll
        for (int s = 0; s < NS - 1; ++s)
            if (s < nk) load_slice(ring + s * kStage, src, L, src.kb + (int64_t)s * kBK);
        // slice 0 has landed; the rest of the prologue may still be loading
        wait_slices((nk < NS - 1 ? nk : NS - 1) - 1);
        bare_barrier();
        Step f0, f1;
        read_step(ring, L, 0, f0);
        for (int kt = 0; kt < nk; ++kt) {
            const int l = kt + NS - 1;            // slice to load now
            // slices still loading once slice kt + 1 has landed
            const int last = l < nk ? l : nk - 1;
            const int behind = last - (kt + 1) > 0 ? last - (kt + 1) : 0;
            if (l < nk) gate(src.kb + (int64_t)l * kBK);
            slice(ring + (kt % NS) * kStage, ring + ((kt + 1) % NS) * kStage,
                  ring + (l % NS) * kStage, l < nk, src.kb + (int64_t)l * kBK, behind, kt + 1 < nk,
                  src, L, f0, f1, acc);
        }
    }
};

// Epilogue.  Accumulator element r of lane l in a 32x32 block belongs to
// row 8(r/4) + 4(l/32) + r%4 and column l%32, so each store instruction
// writes two 32-column row segments; in a 16x16 block to row 4(l/16) + r
// and column l%16 (pairs of blocks are regrouped to the same two-segment
// stores, below).  The stores go through a buffer
// descriptor that starts at the tile's first output row and ends after its
// last valid row: rows past the shard fall out of range and are dropped,
// columns past N get an out-of-range lane offset, so no store needs a
// branch or a 64-bit address.  Offsets stay below 2^31 because a tile
// spans at most 256 rows of at most 2^20 columns of 4 bytes.
//
// fp16 path: the fp32 accumulators are the result (written non-temporal:
// C is not read again here).  int8 path: the int32 accumulator plus the
// column's bias (modulo 2^32), optionally kept in acc_out, then scaled in
// fp32 and rounded to fp16.
constexpr int kStoreStream = 2;   // non-temporal

// One int32 accumulator, copied out of its AGPR where it is used.  Read
// through plain code, the accumulators of the whole tile would be given
// VGPRs where the K loop ends and copied there at once.
__device__ __forceinline__ uint32_t acc_read(int32_t x)
{
    uint32_t v;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(x));
    return v;
}

template <class T, int BM, int BN, int WM, int WN, bool kKeepAcc>
__device__ __forceinline__ void store_tile_as(
    const ConsumerArgs& a, int shard, int m, int n,
    typename T::Acc (&acc)[BM / (T::kBlk * WM)][BN / (T::kBlk * WN)])
{
    constexpr int kE = T::kBlk;             // block edge
    typedef typename T::Out Out;
    const Schedule& s = a.s;
    const int lane = opaque_lane(), wave = threadIdx.x >> 6;
    const int wm = (wave / WN) * (BM / WM), wn = (wave % WN) * (BN / WN);
    const int64_t row0 = (int64_t)m * BM;
    const int64_t left = s.S - row0;
    const uint32_t rows = (uint32_t)(left < BM ? left : BM);
    const int64_t origin = ((int64_t)shard * s.S + row0) * s.N + (int64_t)n * BN;
    const uint32_t row_out = (uint32_t)s.N * (uint32_t)sizeof(Out);
    const __amdgpu_buffer_rsrc_t rc =
        scalar_rsrc(static_cast<Out*>(a.C) + origin, (int64_t)rows * row_out);
    __amdgpu_buffer_rsrc_t racc = rc;
    const uint32_t row_acc = (uint32_t)s.N * 4u;
    if constexpr (kKeepAcc)
        racc = scalar_rsrc(a.acc_out + origin, (int64_t)rows * row_acc);
    if constexpr (kE == 16) {
        // 16 x 16 blocks, column blocks in pairs (2jp, 2jp + 1): one
        // v_permlane16_swap per accumulator pair trades the pair's odd
        // 16-lane rows for the other's even ones, after which lanes 0-31 of
        // each result hold 32 consecutive columns of one output row (rows
        // r and 8 + r of the block in the first result, 4 + r and 12 + r in
        // the second), so every store writes two whole 128-byte row
        // segments, as in the 32 x 32 blocks' epilogue.
        constexpr int kTN = BN / (kE * WN);
        static_assert(kTN % 2 == 0, "column blocks in pairs");
        const uint32_t lrow = (uint32_t)(wm + 8 * (lane >> 5));
        const int64_t col_lane = (int64_t)n * BN + wn + (lane & 31);
#pragma unroll
        for (int jp = 0; jp < kTN / 2; ++jp) {
            const bool in = col_lane + 32 * jp < s.N;
            const uint32_t c = (uint32_t)(wn + (lane & 31) + 32 * jp);
            const uint32_t vo = in ? lrow * row_out + c * (uint32_t)sizeof(Out) : kOutOfRange;
            const uint32_t vacc = in ? lrow * row_acc + c * 4u : kOutOfRange;
            int32_t bias = 0;
            float scale = 0.f;
            if constexpr (T::kDequant) {
                if (in) {
                    bias = a.bias[col_lane + 32 * jp];
                    scale = a.scale[col_lane + 32 * jp];
                }
            }
#pragma unroll
            for (int i = 0; i < BM / (kE * WM); ++i) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const auto x0 = acc[i][2 * jp][r], x1 = acc[i][2 * jp + 1][r];
                    const auto sw = __builtin_amdgcn_permlane16_swap(
                        __builtin_bit_cast(uint32_t, x0), __builtin_bit_cast(uint32_t, x1),
                        false, false);
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const uint32_t roff = (uint32_t)(i * 16 + 4 * h + r);
                        const uint32_t bits = sw[h];
                        if constexpr (!T::kDequant) {
                            __builtin_amdgcn_raw_buffer_store_b32(bits, rc, vo + roff * row_out,
                                                                  0, kStoreStream);
                        } else {
                            const uint32_t v = bits + (uint32_t)bias;
                            if constexpr (kKeepAcc)
                                __builtin_amdgcn_raw_buffer_store_b32(
                                    v, racc, vacc + roff * row_acc, 0, kStoreStream);
                            const _Float16 hv = (_Float16)((float)(int32_t)v * scale);
                            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, hv),
                                                                  rc, vo + roff * row_out, 0,
                                                                  kStoreStream);
                        }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        return;
    }
    const uint32_t lrow = (uint32_t)(wm + 4 * (lane / kE));
    const int64_t col_lane = (int64_t)n * BN + wn + (lane % kE);
#pragma unroll
    for (int j = 0; j < BN / (kE * WN); ++j) {
        const bool in = col_lane + kE * j < s.N;
        const uint32_t c = (uint32_t)(wn + (lane % kE) + kE * j);
        const uint32_t vo = in ? lrow * row_out + c * (uint32_t)sizeof(Out) : kOutOfRange;
        const uint32_t vacc = in ? lrow * row_acc + c * 4u : kOutOfRange;
        int32_t bias = 0;
        float scale = 0.f;
        if constexpr (T::kDequant) {
            if (in) {
                bias = a.bias[col_lane + kE * j];
                scale = a.scale[col_lane + kE * j];
            }
        }
#pragma unroll
        for (int i = 0; i < BM / (kE * WM); ++i) {
#pragma unroll
            for (int r = 0; r < T::kAccN; ++r) {
                const uint32_t roff =
                    (uint32_t)(i * kE + (kE == 32 ? 8 * (r >> 2) + (r & 3) : r));
                if constexpr (!T::kDequant) {
                    // the element is copied out first: a bit cast applied
                    // to a vector element directly reads element 0
                    const float x = acc[i][j][r];
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), rc,
                                                          vo + roff * row_out, 0, kStoreStream);
                } else {
                    const uint32_t v = acc_read(acc[i][j][r]) + (uint32_t)bias;
                    if constexpr (kKeepAcc)
                        __builtin_amdgcn_raw_buffer_store_b32(v, racc, vacc + roff * row_acc,
                                                              0, kStoreStream);
                    const _Float16 h = (_Float16)((float)(int32_t)v * scale);
                    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, h), rc,
                                                          vo + roff * row_out, 0, kStoreStream);
                }
            }
            // one block at a time: the scheduler would otherwise copy many
            // blocks' accumulators into VGPRs ahead of their stores
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

template <class T, int BM, int BN, int WM, int WN>
__device__ __forceinline__ void store_tile(
    const ConsumerArgs& a, int shard, int m, int n,
    typename T::Acc (&acc)[BM / (T::kBlk * WM)][BN / (T::kBlk * WN)])
{
    if constexpr (T::kDequant) {
        if (a.acc_out) {
            store_tile_as<T, BM, BN, WM, WN, true>(a, shard, m, n, acc);
            return;
        }
    }
    store_tile_as<T, BM, BN, WM, WN, false>(a, shard, m, n, acc);
}

// Paced calls: whether chunk j of a source (K-block j / rcs, row group
// j % rcs) is past its paced time, the time the emulated link could have
// carried the source's bytes up to and including it (parallel links),
// measured from this call's pacing origin; false while the producer has
// not set the origin yet.  The bytes are counted in whole KiB of elements,
// rounded up, as the ticks per KiB are: never earlier than the chunk flag's
// own paced time.
__device__ __forceinline__ bool paced_time_passed(const ConsumerArgs& a, uint32_t j)
{
    const uint64_t slot = __hip_atomic_load(a.clock, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t mask = (1ull << 40) - 1;
    if ((slot >> 40) != (uint64_t)(a.epoch & 0xffffffu)) return false;
    const Schedule& s = a.s;
    const int kb = (int)(j / (uint32_t)s.rcs), jr = (int)(j % (uint32_t)s.rcs);
    const int64_t k0 = kblock_begin(s, kb);
    const int64_t elts = k0 * s.S + chunk_row_end(s, jr) * (kblock_end(s, kb) - k0);
    const uint64_t due = ((uint64_t)((elts + 1023) >> 10) * a.ticks_per_kib_q16 >> 16) + 1;
    return ((ticks() - (slot & mask)) & mask) >= due;
}

// Wave 0 of a workgroup: wait until chunks [0, need) of source `shard` are
// known released, `have` of them known already.  Either of the PTO-ISA
// README's two structures says so: the source's summary counter covering
// `need`, or the chunk flags of [have, need) all holding the call's epoch.
// The counter moves only once the chunk before the first unflagged one is
// flagged (and then in a compare-and-swap after a flag walk), so it lags the
// flags; the flags alone cost one wave-wide load per 64 chunks.  Where the
// call keeps piece flags, a chunk whose pieces are all flagged counts as
// released too (for the first 16 chunks of a poll: four lanes a chunk);
// they come about two round trips before the chunk flag, which waits for
// the last piece's running-total add to return.  Each poll issues the
// counter load and the flag loads together: one memory round trip.  A
// piece flag is stored only after its piece's data was performed in
// memory, a chunk flag only after every piece of the chunk was, and the
// counter passes a chunk only after some wave saw its flag, so each
// vouches for the data.  Returns the chunks now known released (>= need),
// or 0 after a time-out or a failure elsewhere in the call.  kPieces: look
// at the piece flags too (the wait before a tile; inside the K loop the
// registers the extra lanes' work takes are not there to spare, and the
// chunk flags are in by then as a rule).
template <bool kPieces>
__device__ __forceinline__ uint32_t poll_ready(const ConsumerArgs& a, int shard, uint32_t have,
                                               uint32_t need, int tid)
{
    const uint32_t base = a.base[shard];
    const uint32_t* ctr = a.counters + shard * (kCounterStride / 4);
    const uint32_t* fl = a.flags + shard * kFlagCap;
    const uint32_t* pf =
        kPieces && a.piece_flags ? a.piece_flags + shard * kFlagCap * kPieceFlags : nullptr;
    uint64_t t0 = 0;
    uint32_t spins = 0;
    for (;;) {
        const uint32_t c = load_agent(ctr);          // one request for the wave
        const uint32_t j = have + (uint32_t)tid;
        bool set = j >= need || load_agent(fl + j) == a.epoch;
        if (kPieces && pf) {
            // lane 4i + q: piece q of chunk have + i
            const uint32_t jp = have + (uint32_t)tid / kPieceFlags;
            const uint32_t q = (uint32_t)tid % kPieceFlags;
            bool pset = jp >= need || q >= (uint32_t)a.ppc ||
                        load_agent(pf + jp * kPieceFlags + q) == a.epoch;
            if (a.ticks_per_kib_q16 && jp < need)
                pset = pset && paced_time_passed(a, jp);
            uint64_t m = __builtin_amdgcn_ballot_w64(pset);
            m &= m >> 1;
            m &= m >> 2;                              // bit 4i: all of chunk have + i
            set = set || (tid < 64 / kPieceFlags && ((m >> (kPieceFlags * tid)) & 1));
        }
        const uint32_t cur = __builtin_amdgcn_readfirstlane(c) - base;
        if (cur >= need && cur <= (uint32_t)kFlagCap) return cur;
        const uint64_t unset = __builtin_amdgcn_ballot_w64(!set);
        if (!unset) {
            if (have + 64 >= need) return need;
            have += 64;                              // the next 64 at once
            continue;
        }
        have += (uint32_t)__builtin_ctzll(unset);    // the flagged run so far
        if (spins == 0) t0 = ticks();
        __builtin_amdgcn_s_sleep(2);
        if ((++spins & 31u) == 0) {
            if (reached(__builtin_amdgcn_readfirstlane(load_agent(a.err)), a.epoch)) return 0;
            if (ticks() - t0 > a.limit) {
                if (tid == 0) raise_error(a.err, a.epoch);
                return 0;
            }
        }
    }
}

// Wave 0 of a workgroup, before a tile: wait until chunks [0, need) of
// source `shard` are released (poll_ready), then, with `acquire`, an
// agent-scope fence, which invalidates this CU's L1 and this XCD's L2 and
// so drops any line an earlier call left at these workspace addresses.
// What the workgroup has already seen of the source is kept in
// seen[shard], so a satisfied wait touches no memory.  Returns 0 after a
// time-out or a failure elsewhere in the call.
//
// Without a workspace ring a workgroup needs one such fence per call, and
// the consumer takes it on entry, before any load (the caller passes
// acquire = false); with a ring of stages reused within the call, every
// wait fences.  Every workspace address is written once per call, every
// load of one is issued after its chunk's release was seen, and each
// workgroup fences before its first such load; so after that fence its
// CU's L1 and its XCD's L2 can take a line at a workspace address only
// from a load that follows the line's release, which reads the released
// data.  A stale line could only be an earlier call's, and the earlier
// call's consumer ended before this one started.  (The fence costs some
// microseconds, and it empties the L2 of the panels every other workgroup
// of the XCD is sharing: on entry there are none yet.)
template <bool kPieces>
__device__ __forceinline__ int wait_source(const ConsumerArgs& a, int shard, int need,
                                           uint32_t* seen, int tid, bool acquire)
{
    const uint32_t have = seen[shard];
    uint32_t got = have;
    if (have < (uint32_t)need) {
        got = poll_ready<kPieces>(a, shard, have, (uint32_t)need, tid);
        if (!got) return 0;
    }
    if (acquire) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (tid == 0) seen[shard] = got;
    return 1;
}

// Wave 0 inside a tile's K loop: the same wait, with no acquire fence,
// which on gfx950 invalidates the CU's L1 and the whole L2 of the XCD (the
// panels every other workgroup there is sharing).  None is needed here:
//   * a load of a chunk is issued only after its release was seen, and the
//     release comes after the chunk's data stores (write-through) were
//     performed in memory;
//   * so a load can only be served stale data by a cache line that held
//     the address before the data was written.  In this call nobody reads
//     a chunk before its release (every read is gated) and chunk edges are
//     cache-line edges (rows and K-blocks are whole KiB), so such a line
//     can only be left over from an earlier call -- and the workgroup's
//     first acquire of the call (at this tile's first wait or an earlier
//     tile's; at this tile's with a ring of stages), after which this wave
//     issues every load of the tile, dropped every such line from this CU's
//     L1 and this XCD's L2.
__device__ __forceinline__ int wait_counter(const ConsumerArgs& a, int shard, int need,
                                            uint32_t* seen, int tid)
{
    const uint32_t have = seen[shard];
    if (have >= (uint32_t)need) return 1;
    const uint32_t got = poll_ready<false>(a, shard, have, (uint32_t)need, tid);
    if (!got) return 0;
    if (tid == 0) seen[shard] = got;
    return 1;
}

// With `have` chunks of a source known released, the K-blocks whose chunks
// of m-tile m's rows (`rows` row chunks) -- and everything before them in
// the source's order -- are all in: [0, covered).  32-bit: at most 1024
// chunks per source.
__device__ __forceinline__ int covered_kblocks(const Schedule& s, uint32_t rows, uint32_t have)
{
    if (have < rows) return 0;
    const uint32_t c = (have - rows) / (uint32_t)s.rcs + 1;
    return c < (uint32_t)s.nkb ? (int)c : s.nkb;
}

// Split-K: one part of a tile's K range is done.  Its accumulators go to
// the tile's partial sums (register-major: each store of a wave writes 256
// contiguous bytes), written through at device scope; once they are
// performed, thread 0 adds the part's weight to the tile's ticket.  The
// part whose add completes the ticket's total (the last to finish) reads
// every part back in part order, with device-scope loads that take no
// stale cached line, and adds them: the sum order is fixed, whichever part
// finishes last.  Returns true in the workgroup that then runs the tile's
// epilogue.
template <class T, class E>
__device__ bool split_reduce(const ConsumerArgs& a, const TileRef& t, int tid, int* last,
                             typename T::Acc (&acc)[E::kTM][E::kTN])
{
    static_assert(T::kBlk == 32, "split-K parts are built on 32 x 32 blocks");
    constexpr int R = E::kTM * E::kTN * 16;   // accumulators per thread
    constexpr int TH = E::kThreads;
    constexpr int kDevice = 16;               // device-scope cache policy
    constexpr bool kInt = T::kDequant;        // int32 accumulators
    const Schedule& s = a.s;
    const int64_t tb = ((int64_t)t.shard * s.mt + t.m) * s.nt + t.n;
    // the tile's parts: ks x R x TH words, far below 2^31 bytes
    const __amdgpu_buffer_rsrc_t rp =
        scalar_rsrc(a.partials + tb * s.ks * R * TH * 4, (int64_t)s.ks * R * TH * 4);
    const int own = t.kp * R * TH * 4 + tid * 4;
#pragma unroll
    for (int i = 0; i < E::kTM; ++i)
#pragma unroll
        for (int j = 0; j < E::kTN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                // the element is copied out first, as in the epilogue: a bit
                // cast applied to a vector element directly reads element 0
                uint32_t bits;
                if constexpr (kInt) {
                    bits = acc_read(acc[i][j][e]);
                } else {
                    const float x = acc[i][j][e];
                    bits = __builtin_bit_cast(uint32_t, x);
                }
                __builtin_amdgcn_raw_buffer_store_b32(
                    bits, rp, own + ((i * E::kTN + j) * 16 + e) * TH * 4, 0, kDevice);
            }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const uint32_t w = piece_weight(t.kp, s.ks);
        const uint32_t old = __hip_atomic_fetch_add(a.tickets + tb, w, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        *last = ((old + w) & (kPieceTotal - 1)) == 0;
    }
    __syncthreads();
    if (!uniform(*last)) return false;
    // pairs with the other parts' performed stores, seen through the ticket
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
#pragma unroll
    for (int i = 0; i < E::kTM; ++i)
#pragma unroll
        for (int j = 0; j < E::kTN; ++j) acc[i][j] = T::zero();
    for (int kp = 0; kp < s.ks; ++kp) {
        const int at = kp * R * TH * 4 + tid * 4;
#pragma unroll
        for (int i = 0; i < E::kTM; ++i)
#pragma unroll
            for (int j = 0; j < E::kTN; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(
                        rp, at + ((i * E::kTN + j) * 16 + e) * TH * 4, 0, kDevice);
                    if constexpr (kInt)
                        acc[i][j][e] = (int)((uint32_t)acc[i][j][e] + v);
                    else
                        acc[i][j][e] += __builtin_bit_cast(float, v);
                }
    }
    return true;
}

// Workgroup-shared state of a consumer workgroup: what it has seen of each
// source, and two flags wave 0 hands the other waves.  Declared by each
// kernel that runs the consumer (with the dynamic LDS of the tile ring) and
// handed in, so that every LDS variable belongs to one kernel.
struct ConsumerShared {
    uint32_t seen[kMaxShards];
    int ok;
    int last;
};

// The consumer: workgroup `block` of `blocks` (blockIdx.x and gridDim.x in
// the consumer kernel; past the producer workgroups in the fused one).
template <class T, int BM, int BN, int SB, int NS, int WM, int WN>
__device__ __forceinline__ void consume(const ConsumerArgs& a, uint32_t block, uint32_t blocks,
                                        ConsumerShared& sh, char* lds)
{
    typedef Engine<T, BM, BN, SB, NS, WM, WN> E;
    // the wait before a tile looks at piece flags on the large eight-wave
    // tiles, whose round-0 waits the first chunks' release sets; the small
    // tiles keep the plain wait (the extra loads cost them more than they
    // gain), and so do the four-wave 256 x 256 ones and the int8 ones, whose
    // accumulators (in AGPRs for int8) leave no registers for it
    constexpr bool kPieceWait = BM * BN >= 256 * 128 && E::kWaves == 8 && !T::kDequant;
    uint32_t* seen_sh = sh.seen;
    int& ok_sh = sh.ok;
    int& last_sh = sh.last;

    const Schedule& s = a.s;
    const int tid = threadIdx.x;
    for (int i = tid; i < kMaxShards; i += E::kThreads) seen_sh[i] = 0;
    // tell the producer that the work ahead of the call on this stream is
    // done (any workgroup may be the first to run)
    if (a.start && tid == 0)
        __hip_atomic_store(a.start + (block % a.start_copies) * (kStartStride / 4), a.epoch,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (a.trace_start && block == 0 && tid == 0) a.trace_start[0] = ticks();
    // the call's one acquire fence without a workspace ring (see below);
    // the barrier holds the other waves until it is done
    if (!a.no_wait && s.ring == 0 && tid < 64) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    __syncthreads();

    const int64_t tiles = total_tiles(s);
    typename E::Lane L;
    E::lane_offsets(L, s.K, s.N);
    // Whether this workgroup has fenced in this call (wait_source).  Without
    // a workspace ring one fence per call suffices, and it is taken here,
    // before any load: it drops the lines an earlier call left at workspace
    // addresses from this CU's L1 and this XCD's L2, and every later load
    // of a workspace line follows that line's release.  Taken at the first
    // remote tile instead, it came mid-call for the workgroups whose first
    // tile is local, and each such fence emptied the L2 of the panels the
    // XCD's other workgroups were sharing.
    bool acquired = !a.no_wait && s.ring == 0;   // (fenced in the prologue)

    for (int64_t p = wg_position(s, block, blocks); p < tiles; p += blocks) {
        const TileRef t = tile_at(s, p);
        // K range: all of K, or part kp of a split-K tile (parts hold a
        // multiple of 256 k, a whole number of slices)
        const int64_t kb = (int64_t)t.kp * s.kc;
        const int64_t ke = kb + s.kc < s.K ? kb + s.kc : s.K;
        const int nk = ke > kb ? (int)cdiv(ke - kb, E::kBK) : 0;
        // Loads of K below `open_k` need no wait: all of K for a local tile,
        // in a mode without waits, or once every K-block is in; `open_kb` is
        // the first K-block not known to be in.  (32-bit: K <= 2^21.)
        int32_t open_k = INT32_MAX, open_kb = s.nkb;
        const uint32_t rows_need = (uint32_t)t.need;   // the tile's row chunks
        const bool gated = t.need > 0 && !a.no_wait;
        if (a.trace && tid == 0) a.trace[3 * p] = ticks();
        if (gated) {
            // Before the first slices (the NS - 1 loaded before the loop),
            // wave 0 waits for the K-blocks they read -- with chunks of all
            // of K, for the tile's rows; the other waves hold at the barrier.
            if (tid < 64) {
                int ok = 1;
                if (s.pv > 0) {
                    // barrier scheme: the iteration's rows of every source
                    for (int q = 1; q < s.n_shards && ok; ++q)
                        ok = wait_source<kPieceWait>(a, s.order[q], t.need, seen_sh, tid,
                                         q == s.n_shards - 1 && (!acquired || s.ring > 0));
                } else {
                    const int64_t pro = kb + (int64_t)(NS - 1) * E::kBK;
                    const int kb0 = kblock_of(s, (pro < ke ? pro : ke) - 1);
                    ok = wait_source<kPieceWait>(a, t.shard, need_at(s, t.m, kb0), seen_sh, tid,
                                     !acquired || s.ring > 0);
                }
                if (tid == 0) ok_sh = ok;
            }
            __syncthreads();
            if (!uniform(ok_sh)) break;   // the call has failed; every lane leaves
            acquired = true;
            if (s.pv == 0) {
                open_kb = covered_kblocks(s, rows_need, uniform(seen_sh[t.shard]));
                open_k = open_kb >= s.nkb ? INT32_MAX : (int32_t)(open_kb * s.kbk);
            }
        }
        if (a.trace && tid == 0) a.trace[3 * p + 1] = ticks();

        // Before a slice's loads: when the slice reaches past open_k, wave 0
        // waits for its K-block and every wave learns the new open_k.  The
        // test is uniform (open_k is the same in every wave), so the extra
        // barrier is taken by all waves or by none.  The barrier is a bare
        // one: slices already loading stay in flight.
        // A slice is at most one K-block long (K-blocks are whole KiB of
        // elements, slices at most 256 bytes), so the block it enters past
        // open_k is open_kb itself.
        // A failed wait opens all of K (no further waits) and marks the
        // tile, which the workgroup then drops.
        bool failed = false;
        auto gate = [&](int64_t k) {
            const int32_t end = (int32_t)(k + E::kBK < s.K ? k + E::kBK : s.K);
            if (end <= open_k) return;
            if (tid < 64) {
                const int ok = wait_counter(a, t.shard, open_kb * s.rcs + (int)rows_need,
                                            seen_sh, tid);
                if (tid == 0) ok_sh = ok;
                wait_vm_lgkm0<63>();   // the LDS stores are done (loads may fly)
            }
            bare_barrier();
            if (!uniform(ok_sh)) {
                failed = true;
                open_k = INT32_MAX;
                return;
            }
            open_kb = covered_kblocks(s, rows_need, uniform(seen_sh[t.shard]));
            open_k = open_kb >= s.nkb ? INT32_MAX : (int32_t)(open_kb * s.kbk);
        };

        const int64_t row0 = (int64_t)t.m * BM;
        const int64_t rows = s.S - row0;
        // remote rows sit in the workspace (a full slot or a ring stage)
        const int64_t arow = t.shard == s.local ? row0 : slot_row(s, row0);
        const typename E::Src src{a.a[t.shard] + arow * s.K * T::kElt,
                                  rows < BM ? rows : BM, a.B, s.K, s.N, (int64_t)t.n * BN, kb};

        typename T::Acc acc[E::kTM][E::kTN];
#pragma unroll
        for (int i = 0; i < E::kTM; ++i)
#pragma unroll
            for (int j = 0; j < E::kTN; ++j) acc[i][j] = T::zero();

        if (nk > 0) E::run(lds, nk, src, L, acc, gate);
        if (failed) break;   // the call has failed; every lane leaves
        // every wave's loads of the tile have completed (the last slice
        // waited for them before its barrier): the stage may be reused
        if (a.stages && t.shard != s.local && tid == 0)
            count_one(a.stages + t.shard * kMaxStages + t.m % s.ring, a.epoch);
        // split-K is planned only on tiles of one or two 32 x 32 blocks
        // per wave (ids 3, 12, 13, 14); the others are built without it,
        // which keeps their registers as they were
        if constexpr (E::kTM * E::kTN <= 2) {
            if (s.ks > 1 && !split_reduce<T, E>(a, t, tid, &last_sh, acc)) {
                if (a.trace && tid == 0) a.trace[3 * p + 2] = ticks();
                continue;   // another part of the tile adds the parts
            }
        }
        store_tile<T, BM, BN, WM, WN>(a, t.shard, t.m, t.n, acc);
        if (a.trace && tid == 0) a.trace[3 * p + 2] = ticks();
    }
}

template <class T, int BM, int BN, int SB, int NS, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN, 1) void consumer_kernel(ConsumerArgs a)
{
    extern __shared__ __attribute__((aligned(16))) char lds[];
    __shared__ ConsumerShared sh;
    consume<T, BM, BN, SB, NS, WM, WN>(a, blockIdx.x, gridDim.x, sh, lds);
}

// Producer and consumer in one launch on the caller's stream: workgroups
// 0 .. producers - 1 run the producer, the others the consumer.  The
// producer workgroups come first, so they are dispatched before any
// consumer workgroup that could wait for them, and they wait for nothing
// themselves (stream order replaces the start word): the launch cannot
// starve even when its workgroups do not all fit on the device at once.
// Built for the four-wave tiles of up to 128 x 128, whose workgroups have
// the producer's four waves.
template <class T, int BM, int BN, int SB, int NS, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN, 1) void fused_kernel(ConsumerArgs a, ProducerArgs p,
                                                                 int producers)
{
    static_assert(WM * WN == prod::kProducerWaves, "producer workgroups of four waves");
    extern __shared__ __attribute__((aligned(16))) char lds[];
    __shared__ ConsumerShared sh;
    __shared__ prod::ProducerShared psh;
    if ((int)blockIdx.x < producers) {
        prod::produce(p, blockIdx.x, (uint32_t)producers, psh);
        return;
    }
    consume<T, BM, BN, SB, NS, WM, WN>(a, blockIdx.x - (uint32_t)producers,
                                        gridDim.x - (uint32_t)producers, sh, lds);
}

// Tile configurations: output tile, slice width (bytes of K per row), LDS
// ring depth and wave grid, by the id the host plans with.  The big tiles
// walk K in 64-byte slices with four stages (three in flight) or in
// 128-byte slices with two; the small ones use two 128-byte stages so that
// several workgroups share a CU.  The 8-wave configurations put two waves
// on each SIMD (each owning a 128 x 64 block), so that one wave's waits
// overlap the other's MFMAs.
template <int ID> struct Cfg;
template <> struct Cfg<1> { static constexpr int BM = 256, BN = 256, SB = 64, NS = 4, WM = 2, WN = 2; };
template <> struct Cfg<2> { static constexpr int BM = 128, BN = 128, SB = 128, NS = 2, WM = 2, WN = 2; };
template <> struct Cfg<3> { static constexpr int BM = 64, BN = 64, SB = 128, NS = 2, WM = 2, WN = 2; };
template <> struct Cfg<4> { static constexpr int BM = 256, BN = 128, SB = 64, NS = 4, WM = 2, WN = 2; };
template <> struct Cfg<5> { static constexpr int BM = 128, BN = 256, SB = 64, NS = 4, WM = 2, WN = 2; };
template <> struct Cfg<6> { static constexpr int BM = 256, BN = 256, SB = 128, NS = 2, WM = 2, WN = 2; };
template <> struct Cfg<7> { static constexpr int BM = 256, BN = 256, SB = 64, NS = 3, WM = 2, WN = 2; };
template <> struct Cfg<8> { static constexpr int BM = 256, BN = 256, SB = 128, NS = 2, WM = 2, WN = 4; };
template <> struct Cfg<9> { static constexpr int BM = 256, BN = 256, SB = 64, NS = 4, WM = 2, WN = 4; };
template <> struct Cfg<10> { static constexpr int BM = 256, BN = 128, SB = 128, NS = 2, WM = 4, WN = 2; };
template <> struct Cfg<11> { static constexpr int BM = 128, BN = 256, SB = 128, NS = 2, WM = 2, WN = 4; };
template <> struct Cfg<12> { static constexpr int BM = 64, BN = 64, SB = 128, NS = 8, WM = 2, WN = 2; };
template <> struct Cfg<13> { static constexpr int BM = 64, BN = 64, SB = 256, NS = 4, WM = 2, WN = 2; };
// 32 rows x 256 columns for decode-like shapes (split-K): B is read in rows
// of 256 elements, one 32 x 64 block per wave, three slices in flight.
template <> struct Cfg<14> { static constexpr int BM = 32, BN = 256, SB = 128, NS = 4, WM = 1, WN = 4; };
// id 8's tile, pipeline and wave grid on 16 x 16 MFMA blocks (fp16, bf16,
// int8): each wave owns 8 x 4 blocks of 16 x 16.
template <> struct Cfg<15> { static constexpr int BM = 256, BN = 256, SB = 128, NS = 2, WM = 2, WN = 4; };

// The element traits a configuration is built with: the path's own (two
// operand sets), or for id 15 its one-set form -- on 16 x 16 blocks for
// fp16, bf16 and int8, on 32 x 32 blocks for fp8.
template <class T, int ID> struct TraitsFor { typedef T type; };
template <> struct TraitsFor<F16, 15> { typedef F16x type; };
template <> struct TraitsFor<BF16, 15> { typedef BF16x type; };
template <> struct TraitsFor<I8, 15> { typedef I8x type; };
template <> struct TraitsFor<FP8, 15> { typedef FP8x type; };

template <class T0, int ID>
struct Kern {
    typedef typename TraitsFor<T0, ID>::type T;
    typedef Cfg<ID> C;
    typedef Engine<T, C::BM, C::BN, C::SB, C::NS, C::WM, C::WN> E;
    static const void* fn()
    {
        return reinterpret_cast<const void*>(
            consumer_kernel<T, C::BM, C::BN, C::SB, C::NS, C::WM, C::WN>);
    }
    static hipError_t launch(const ConsumerArgs& a, int wgs, hipStream_t st)
    {
        static bool attr_set = false;   // one-time opt-in to > 64 KiB of LDS
        if (!attr_set) {
            hipError_t e = hipFuncSetAttribute(fn(), hipFuncAttributeMaxDynamicSharedMemorySize,
                                               E::kLds);
            if (e != hipSuccess) return e;
            attr_set = true;
        }
        hipLaunchKernelGGL((consumer_kernel<T, C::BM, C::BN, C::SB, C::NS, C::WM, C::WN>),
                           dim3(wgs), dim3(E::kThreads), (size_t)E::kLds, st, a);
        return hipGetLastError();
    }
    static const void* fused_fn()
    {
        return reinterpret_cast<const void*>(
            fused_kernel<T, C::BM, C::BN, C::SB, C::NS, C::WM, C::WN>);
    }
    static hipError_t launch_fused(const ConsumerArgs& a, const ProducerArgs& p, int wgs,
                                   int producers, hipStream_t st)
    {
        static bool attr_set = false;
        if (!attr_set) {
            hipError_t e = hipFuncSetAttribute(
                fused_fn(), hipFuncAttributeMaxDynamicSharedMemorySize, E::kLds);
            if (e != hipSuccess) return e;
            attr_set = true;
        }
        hipLaunchKernelGGL((fused_kernel<T, C::BM, C::BN, C::SB, C::NS, C::WM, C::WN>),
                           dim3(producers + wgs), dim3(E::kThreads), (size_t)E::kLds, st, a, p,
                           producers);
        return hipGetLastError();
    }
    static int occupancy()
    {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn(), E::kThreads, E::kLds) !=
            hipSuccess)
            return 0;
        return n;
    }
};

// Whether configuration ID is built for traits T.  A slice must hold an
// even number of MFMA steps (the fp8 MFMA takes 64 bytes of K, so its
// slices are 128 or 256 bytes), and the registers one wave needs -- its
// accumulators, two steps' operand fragments and about 40 for addresses
// and loop state -- times the waves per SIMD must leave 48 of the 512 for
// a producer wave.  (The compiler's own count is checked by the tests;
// this only keeps configurations that cannot fit from being built.)
template <class T0, int ID>
constexpr bool supported()
{
    typedef typename TraitsFor<T0, ID>::type T;
    if constexpr (std::is_void_v<T>) {
        return false;
    } else {
        typedef Cfg<ID> C;
        constexpr int tm = C::BM / (T::kBlk * C::WM), tn = C::BN / (T::kBlk * C::WN);
        // operand fragments: two sets, or one rolling set
        constexpr int sets = T::kRoll ? 1 : 2;
        constexpr int regs = tm * tn * T::kAccN + sets * T::kPair * 4 * (tm + tn) + 40;
        constexpr int per_simd = C::WM * C::WN / 4;
        return C::SB % (64 * T::kPair) == 0 && per_simd * regs <= 512 - 48;
    }
}

template <class T, int ID>
hipError_t launch_id(const ConsumerArgs& a, int wgs, hipStream_t st)
{
    if constexpr (supported<T, ID>())
        return Kern<T, ID>::launch(a, wgs, st);
    else
        return hipErrorInvalidValue;
}

// Whether the fused kernel is built for configuration ID and traits T: the
// four-wave tiles of up to 128 x 128 (the small calls it is for).
template <class T, int ID>
constexpr bool fusable()
{
    typedef Cfg<ID> C;
    return supported<T, ID>() && C::WM * C::WN == 4 && C::BM * C::BN <= 128 * 128;
}

template <class T, int ID>
hipError_t launch_fused_id(const ConsumerArgs& a, const ProducerArgs& p, int wgs, int producers,
                           hipStream_t st)
{
    if constexpr (fusable<T, ID>())
        return Kern<T, ID>::launch_fused(a, p, wgs, producers, st);
    else
        return hipErrorInvalidValue;
}

template <class T, int ID>
int occupancy_id()
{
    if constexpr (supported<T, ID>())
        return Kern<T, ID>::occupancy();
    else
        return 0;
}

template <class T>
hipError_t launch_kind(const ConsumerArgs& a, int tile_id, int wgs, hipStream_t st)
{
    switch (tile_id) {
    case 1: return launch_id<T, 1>(a, wgs, st);
    case 2: return launch_id<T, 2>(a, wgs, st);
    case 3: return launch_id<T, 3>(a, wgs, st);
    case 4: return launch_id<T, 4>(a, wgs, st);
    case 5: return launch_id<T, 5>(a, wgs, st);
    case 6: return launch_id<T, 6>(a, wgs, st);
    case 7: return launch_id<T, 7>(a, wgs, st);
    case 8: return launch_id<T, 8>(a, wgs, st);
    case 9: return launch_id<T, 9>(a, wgs, st);
    case 10: return launch_id<T, 10>(a, wgs, st);
    case 11: return launch_id<T, 11>(a, wgs, st);
    case 12: return launch_id<T, 12>(a, wgs, st);
    case 13: return launch_id<T, 13>(a, wgs, st);
    case 14: return launch_id<T, 14>(a, wgs, st);
    case 15: return launch_id<T, 15>(a, wgs, st);
    default: return hipErrorInvalidValue;
    }
}

template <class T>
hipError_t launch_fused_kind(const ConsumerArgs& a, const ProducerArgs& p, int tile_id, int wgs,
                             int producers, hipStream_t st)
{
    switch (tile_id) {
    case 2: return launch_fused_id<T, 2>(a, p, wgs, producers, st);
    case 3: return launch_fused_id<T, 3>(a, p, wgs, producers, st);
    case 12: return launch_fused_id<T, 12>(a, p, wgs, producers, st);
    case 13: return launch_fused_id<T, 13>(a, p, wgs, producers, st);
    case 14: return launch_fused_id<T, 14>(a, p, wgs, producers, st);
    default: return hipErrorInvalidValue;
    }
}

template <class T>
bool fused_kind(int tile_id)
{
    switch (tile_id) {
    case 2: return fusable<T, 2>();
    case 3: return fusable<T, 3>();
    case 12: return fusable<T, 12>();
    case 13: return fusable<T, 13>();
    case 14: return fusable<T, 14>();
    default: return false;
    }
}

template <class T>
int occupancy_kind(int tile_id)
{
    switch (tile_id) {
    case 1: return occupancy_id<T, 1>();
    case 2: return occupancy_id<T, 2>();
    case 3: return occupancy_id<T, 3>();
    case 4: return occupancy_id<T, 4>();
    case 5: return occupancy_id<T, 5>();
    case 6: return occupancy_id<T, 6>();
    case 7: return occupancy_id<T, 7>();
    case 8: return occupancy_id<T, 8>();
    case 9: return occupancy_id<T, 9>();
    case 10: return occupancy_id<T, 10>();
    case 11: return occupancy_id<T, 11>();
    case 12: return occupancy_id<T, 12>();
    case 13: return occupancy_id<T, 13>();
    case 14: return occupancy_id<T, 14>();
    case 15: return occupancy_id<T, 15>();
    default: return 0;
    }
}

}  // namespace

hipError_t launch_consumer_f16(const ConsumerArgs& a, int tile_id, int wgs, hipStream_t st)
{
    return launch_kind<F16>(a, tile_id, wgs, st);
}

hipError_t launch_consumer_bf16(const ConsumerArgs& a, int tile_id, int wgs, hipStream_t st)
{
    return launch_kind<BF16>(a, tile_id, wgs, st);
}

hipError_t launch_consumer_i8(const ConsumerArgs& a, int tile_id, int wgs, hipStream_t st)
{
    return launch_kind<I8>(a, tile_id, wgs, st);
}

hipError_t launch_consumer_fp8(const ConsumerArgs& a, int tile_id, int wgs, hipStream_t st)
{
    return launch_kind<FP8>(a, tile_id, wgs, st);
}

hipError_t launch_fused(int kind, const ConsumerArgs& a, const ProducerArgs& p, int tile_id,
                        int wgs, int producers, hipStream_t st)
{
    return kind == 0 ? launch_fused_kind<F16>(a, p, tile_id, wgs, producers, st)
         : kind == 2 ? launch_fused_kind<BF16>(a, p, tile_id, wgs, producers, st)
         : kind == 3 ? launch_fused_kind<FP8>(a, p, tile_id, wgs, producers, st)
                     : launch_fused_kind<I8>(a, p, tile_id, wgs, producers, st);
}

bool fused_built(int kind, int tile_id)
{
    return kind == 0 ? fused_kind<F16>(tile_id)
         : kind == 2 ? fused_kind<BF16>(tile_id)
         : kind == 3 ? fused_kind<FP8>(tile_id)
                     : fused_kind<I8>(tile_id);
}

int consumer_occupancy(int kind, int tile_id)
{
    return kind == 0 ? occupancy_kind<F16>(tile_id)
         : kind == 2 ? occupancy_kind<BF16>(tile_id)
         : kind == 3 ? occupancy_kind<FP8>(tile_id)
                     : occupancy_kind<I8>(tile_id);
}

}  // namespace agg
