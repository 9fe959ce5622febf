/*
 * aggemm.h -- streamed AllGather + GEMM on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libaggemm.so.  No C++ or torch types cross this boundary: data
 * arguments are plain device pointers, sizes are int64_t, a stream is a
 * hipStream_t passed as void* (NULL = the default stream).
 *
 * The operation (PTO-ISA AllGather+GEMM README, "compute function"; the
 * Triton-distributed AllGather GEMM tutorial's reference function):
 *
 *   A = [A_0; A_1; ...; A_{n-1}]       row blocks stacked in shard order,
 *                                       shard s = rows [s*S, (s+1)*S), S = M/n
 *   C = A x B                           B: K x N, replicated
 *
 * computed as a stream: the shards other than the local one reach a
 * workspace chunk by chunk (a chunk = chunk_rows consecutive rows of one
 * shard, all of K), each chunk released by a monotonic per-source counter;
 * the GEMM starts on the local shard, which needs no wait, and consumes the
 * remote chunks in the order they are sent (PTO-ISA README, "streaming
 * pipeline" and "optimisation notes").  On one GPU every shard is a local
 * allocation; a producer kernel on a side stream plays the links.
 *
 * Result: C rows [s*S, (s+1)*S) = A_s x B for every shard s, whatever the
 * local shard, the send order, the chunk size, the mode or the pacing.
 *
 * Return values: AGG_OK (0) or a positive agg_status.  Argument errors are
 * reported synchronously and nothing is enqueued.  Kernel time-outs (a
 * counter that never reaches its value) are reported by ag_gemm_check().
 * Faults of asynchronous work surface at stream synchronisation, as in HIP.
 *
 * Threading: calls that use the library's internal workspace on one device
 * must be issued from one host thread at a time and are ordered on their
 * streams; two calls in flight on different streams of one device would
 * share the workspace and race.
 *
 * Streams (pipelined mode): the consumer GEMM runs on `stream`; the producer
 * runs on a stream of the library's own, with no event between the two
 * (unless both run in one launch on `stream`: AGG_PRODUCER_FUSED).
 * The producer reads no shard before the consumer has started (the
 * consumer's start, in `stream` order, proves that the work queued ahead of
 * the call is done; the producer waits for it on the device, for at most
 * 120 s or the call's time limit if that is longer, so work queued ahead
 * of a call does not count against the chunk waits' limit).  `stream` does
 * not wait for the producer: the consumer ends only after every chunk is
 * released, which comes after all of the producer's reads of the shards
 * and writes of the workspace.  After a failed call the producer may still
 * be running when `stream` passes the call; ag_gemm_check() waits for it.
 */
#ifndef AGGEMM_H
#define AGGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum agg_status {
    AGG_OK = 0,
    AGG_E_INVALID = 1,      /* null pointer, bad size, bad permutation ...   */
    AGG_E_UNSUPPORTED = 2,  /* K or N not a multiple of the vector width,
                               misaligned pointer, too many shards, or a
                               size past the limits below                   */
    AGG_E_NOMEM = 3,        /* workspace allocation failed                   */
    AGG_E_HIP = 4,          /* a HIP call failed while enqueueing            */
    AGG_E_TIMEOUT = 5,      /* a counter wait exceeded its limit (reported
                               by ag_gemm_check)                             */
    AGG_E_TOO_LARGE = 6     /* ag_gemm_f16_noalloc: the call needs more
                               workspace than its fixed scratch holds
                               (AGG_NOALLOC_MAX_BYTES)                       */
};

/* What one call runs (PTO-ISA README, "benchmark and output"). */
enum agg_mode {
    AGG_MODE_PIPELINED = 0,    /* producer and consumer run concurrently     */
    AGG_MODE_COMPUTE_ONLY = 1, /* consumer only; every chunk taken as ready,
                                  remote rows read from the workspace as the
                                  previous call on it left them              */
    AGG_MODE_SEQUENTIAL = 2,   /* producer finishes, then the consumer runs  */
    AGG_MODE_COPY_ONLY = 3     /* producer only; C is not written            */
};

/* How the consumer learns that rows are there. */
enum agg_scheme {
    AGG_SCHEME_COUNTERS = 0, /* per-source summary counters; the local shard
                                first, then remote tiles as their rows
                                arrive (PTO-ISA README)                   */
    AGG_SCHEME_BARRIER = 1   /* comparison scheme after the Triton-distributed
                                AllGather GEMM tutorial: iterations of
                                `pvalue` row panels of every shard; each
                                tile of an iteration, the local shard's
                                included, waits until every source has
                                delivered the iteration (a barrier in place
                                of per-source counters)                  */
};

/* What moves the remote chunks (PTO-ISA README, "AI Core resources": the
 * communication runs on engines of its own beside the compute). */
enum agg_producer {
    AGG_PRODUCER_KERNEL = 0, /* the producer kernel: compute-unit loads and
                                stores, per-piece release (default).  In a
                                pipelined call whose consumer tile has four
                                waves and at most 128 x 128 outputs, and
                                whose producer and consumer grids fit on
                                the device's CUs together, both run in one
                                launch (as AGG_PRODUCER_FUSED); otherwise as
                                AGG_PRODUCER_SEPARATE                      */
    AGG_PRODUCER_SDMA = 1,   /* the DMA engines: one copy per row group of
                                one m-tile and source, in send order, on the
                                library's stream, each followed by a stream
                                write of the source's counter (the release,
                                ordered after the copy by the stream).  No
                                compute unit moves data.  Chunks span all of
                                K; no pacing, workspace ring, trace of
                                releases or test hooks (AGG_E_UNSUPPORTED)  */
    AGG_PRODUCER_SEPARATE = 2, /* the producer kernel as a launch of its own:
                                on the library's stream in pipelined calls
                                (see "Streams" above)                      */
    AGG_PRODUCER_FUSED = 3   /* pipelined calls: producer and consumer in one
                                launch on `stream`, the producer's
                                workgroups first in the grid (one host
                                launch instead of two; the small calls are
                                bound by launch cost).  Stream order puts
                                the work ahead of the call before it, so
                                there is no start word.  Consumer tiles with
                                four waves and at most 128 x 128 outputs
                                only; no workspace ring or producer_cus
                                (AGG_E_UNSUPPORTED).  Outside the pipelined
                                mode, as AGG_PRODUCER_KERNEL              */
};

/* How the emulated links are paced when link_gbps > 0. */
enum agg_link_model {
    AGG_LINKS_PARALLEL = 0,  /* one link per source, all in parallel (full
                                mesh): chunk j of every source is released
                                no earlier than t0 + bytes(chunks 0..j)/rate */
    AGG_LINKS_SERIAL = 1     /* one link shared by all sources in send order */
};

#define AGG_MAX_SHARDS 64

typedef struct agg_options {
    uint32_t struct_size;   /* sizeof(agg_options); set by ag_gemm_options_init */
    int local_shard;        /* shard read in place, never waited on (default 0) */
    const int *send_order;  /* HOST array of the n-1 remote shard ids in send
                               order, or NULL for local+1, local+2, ... mod n */
    int mode;               /* enum agg_mode (default PIPELINED)              */
    double link_gbps;       /* per-link pacing in GB/s (1e9 B/s); 0 = none    */
    int link_model;         /* enum agg_link_model (default PARALLEL)         */
    int producer_wgs;       /* producer workgroups; 0 = automatic; a
                               pipelined call with the producer kernel on
                               every CU (no producer_cus, not fused) takes at
                               most one per CU (AGG_E_UNSUPPORTED above)      */
    int consumer_wgs;       /* consumer workgroups; 0 = automatic; at most
                               as many as can be resident at once are used */
    int tile;               /* consumer tile shape id; 0 = automatic          */
    int32_t *acc_out;       /* int8 path only: optional DEVICE int32 [M, N]
                               receiving A x B + bias before the dequant     */
    void *workspace;        /* optional caller-owned DEVICE workspace, made
                               ready once by ag_gemm_workspace_reset()       */
    size_t workspace_bytes; /* its size (>= ag_gemm_workspace_bytes(...))    */
    double timeout_ms;      /* bound on every counter wait; 0 = 2000 ms      */
    int debug_drop_chunk;   /* test hook: index (in send order) of a chunk
                               whose release is withheld; -1 = off           */
    void *consumer_events[2]; /* optional hipEvent_t pair recorded right
                                 before and after the consumer kernel, on
                                 the stream it runs on                       */
    int workspace_stages;   /* 0 (default): the workspace holds every remote
                               shard whole (S rows each).  1..8: a ring of
                               that many row panels (one consumer tile high)
                               per remote shard; the producer writes panel m
                               over panel m - stages only after the consumer
                               has finished every tile of that panel
                               (catccos page: a double-buffered workspace with
                               per-slot flags; Triton-distributed tutorial:
                               WORKSPACE_STAGES).  Needs chunks inside one
                               panel: an explicit chunk_rows must divide the
                               tile height (AGG_E_UNSUPPORTED otherwise); the
                               automatic one is cut to a divisor of it.  Not
                               with AGG_MODE_SEQUENTIAL (AGG_E_UNSUPPORTED);
                               a copy-only call does not wait for stages.
                               agg_plan_info.workspace_bytes gives the size. */
    int scheme;             /* enum agg_scheme (default COUNTERS)             */
    int pvalue;             /* barrier scheme: row panels (consumer tiles
                               high) per iteration; 0 = 1.  With a workspace
                               ring, workspace_stages must be at least this
                               (AGG_E_UNSUPPORTED otherwise): a stage is
                               reused only after the tiles of its panel,
                               which wait for their whole iteration; and a
                               ring is refused with AGG_LINKS_SERIAL, whose
                               source-by-source order would have the
                               producer wait on tiles that wait for it.     */
    uint64_t *trace;        /* optional DEVICE buffer of at least
                               agg_plan_info.trace_words uint64, 8-byte
                               aligned, receiving 100 MHz device timestamps:
                                 [0]            consumer start (its first
                                                workgroup; the consumer is
                                                launched before the producer)
                                 [1 + c]        release of producer position c
                                 [1 + C + 3p + 0..2]  consumer position p:
                                                wait start, compute start, end
                               (C = total_chunks).  Entries a call does not
                               reach keep their contents; the caller clears
                               the buffer.  A chunk's release is stamped
                               before its flag is published.                 */
    int64_t producer_piece_bytes; /* bytes a producer wave copies before it
                               counts them towards their chunk: a multiple
                               of 8192; 0 = automatic, 8192 to 65536:
                               pipelined calls about 4 pieces a chunk,
                               copy-only and sequential calls the copy's
                               bytes over the producer's waves.  Smaller pieces
                               spread a chunk over more waves, so chunks
                               land closer to their send order.  Invalid
                               (AGG_E_INVALID) if negative or not a
                               multiple of 8192; a chunk may be cut into at
                               most 2^18 pieces (AGG_E_UNSUPPORTED).        */
    int k_splits;           /* parts K is cut into per output tile (split-K):
                               each part's workgroup writes its partial sums
                               to the workspace and the last to finish adds
                               the parts in part order, then runs the
                               epilogue.  0 or 1 = no split (the automatic
                               choice; on the decode-like shapes measured
                               the unsplit small tile was faster).  > 1
                               needs the counters scheme, no workspace
                               ring, tile 3, 12, 13 or 14 (14: 32 x 256),
                               at most 64 parts and 4096 output tiles
                               (AGG_E_UNSUPPORTED otherwise).  Parts hold a
                               multiple of 256 of K, so the count used may
                               be lower (agg_plan_info.k_splits), and the
                               workspace grows by the partial sums
                               (agg_plan_info.workspace_bytes).  The sum
                               order is fixed, so results do not depend on
                               which part finishes last.                   */
    double debug_delay_us;  /* test hook: each producer piece starts after a
                               pseudo-random delay in [0, debug_delay_us]
                               (a hash of debug_delay_seed and the piece),
                               so pieces and chunks complete in an order
                               unrelated to the send order; 0 = off; must be
                               below the time limit (AGG_E_INVALID if
                               negative or not finite)                     */
    uint32_t debug_delay_seed;
    int producer;           /* enum agg_producer (default KERNEL)            */
    int producer_cus;       /* 0 (default): producer and consumer share every
                               CU.  32 or 64: in pipelined calls the
                               producer kernel runs on a stream masked to
                               that many CUs (the same number on each of
                               the 8 XCDs) and the consumer on a stream
                               masked to the others, with a grid sized to
                               them; the two are forked from and joined to
                               `stream` by events.  Other values, or with
                               SDMA: AGG_E_UNSUPPORTED (smaller masks leave
                               the remaining CUs unable to hold a full
                               consumer grid at once).  Ignored outside the
                               pipelined mode.                             */
    int64_t k_block;        /* elements of K per chunk; 0 (default): the
                               automatic choice that goes with chunk_rows 0
                               (see ag_gemm_f16), or all of K for an
                               explicit chunk_rows; >= K: a chunk spans all
                               of K.  Otherwise a chunk is
                               chunk_rows rows x one K-block of this many
                               elements (the last K-block also takes the
                               remainder of K): the chunk flag matrix of the
                               PTO-ISA README read as row groups x K-blocks.
                               A source's chunks are sent and counted
                               K-block after K-block, and a tile waits at
                               each K-block it enters, not for all of its
                               rows x K at once.  The same results, bit for
                               bit.  Needs k_block and K to be whole KiB of
                               elements (multiples of 512 for fp16/bf16, of
                               1024 for int8/fp8), at most 1024 chunks per
                               source (rows chunks x K-blocks), and the
                               counters scheme without a workspace ring or
                               split-K (AGG_E_UNSUPPORTED otherwise);
                               negative: AGG_E_INVALID.                    */
} agg_options;

/* Fill *opt with the defaults above. */
void ag_gemm_options_init(agg_options *opt);

/*
 * fp16 x fp16 -> fp32 streamed AllGather + GEMM.
 *   shards     HOST array of n_shards DEVICE pointers, each an fp16 [S, K]
 *              row-major block (S = M / n_shards), 16-byte aligned.
 *   B          DEVICE fp16 [K, N] row-major, 16-byte aligned.
 *   C          DEVICE fp32 [M, N] row-major, fully overwritten; must not
 *              alias any input.
 *   chunk_rows rows per chunk; 0 = automatic: with agg_options.k_block
 *              also 0 and K-blocks allowed (K a multiple of 4 KiB of
 *              elements, the counters scheme, no workspace ring or
 *              split-K), S/16 rows x one quarter of K (64 chunks per
 *              source), or x one eighth of K (128 chunks per source) in a
 *              pipelined call with three or more remote shards where K is
 *              a multiple of 8 KiB of elements; otherwise
 *              ag_gemm_pick_chunk_rows(S) rows x all of K.  agg_plan_info
 *              reports the choice.
 * Requires K % 8 == 0 and N % 8 == 0 (AGG_E_UNSUPPORTED otherwise).
 * Size limits (both paths, AGG_E_UNSUPPORTED past them): n_shards <= 64,
 * S <= 2^30, K <= 2^21, N <= 2^20, at most 1024 chunks per shard, and one
 * chunk (chunk_rows x K elements) below 2 GiB.
 * Inputs are read only; the caller owns every buffer.
 * PTO-ISA AllGather+GEMM README, "spec" table: A M x K fp16 (split on M
 * across ranks), B K x N fp16 (replicated), C M x N fp32.
 */
int ag_gemm_f16(const void *const *shards, int n_shards, const void *B,
                float *C, int64_t M, int64_t K, int64_t N, int chunk_rows,
                void *stream);
int ag_gemm_f16_ex(const void *const *shards, int n_shards, const void *B,
                   float *C, int64_t M, int64_t K, int64_t N, int chunk_rows,
                   void *stream, const agg_options *opt);

/*
 * ag_gemm_f16_ex for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same operation, arguments, kernels and results (bit for bit), but
 * the workspace is a fixed device array of AGG_NOALLOC_MAX_BYTES that the
 * library holds on every GPU it runs on, from the first use of its code on
 * that GPU until the process ends.  The call makes no hipMalloc or hipFree
 * and calls no allocating routine.
 *   opt         as for ag_gemm_f16_ex (may be NULL); opt->workspace must be
 *               NULL (AGG_E_INVALID otherwise).
 *   Size limit  the workspace the call needs (a counter header plus the
 *               remote shards' slots, agg_plan_info.workspace_bytes) must
 *               fit in AGG_NOALLOC_MAX_BYTES, else AGG_E_TOO_LARGE and
 *               nothing is enqueued.  With full slots that is
 *               (n_shards - 1) * S * K * 2 bytes plus about 0.8 MiB (8
 *               shards of 1024 x 4096 fit); a workspace ring
 *               (opt->workspace_stages) brings larger shapes under it.
 *   Set-up      the library's per-device set-up (run by the first call of
 *               any entry point on a device, with that device current)
 *               takes the array's address there, which loads the code that
 *               holds it, and zeroes its counter header on that call's
 *               stream (a kernel, no memset); allocation-free calls then go
 *               straight to the kernels.
 *   Sharing     every call on one GPU uses the same array, which keeps what
 *               the last call left in it: calls that overlap in time on one
 *               GPU (two streams, two host threads) race and give wrong
 *               results.  Serialise them, as for the internal workspace.
 *   Errors      as ag_gemm_f16_ex; a time-out is reported by
 *               ag_gemm_check(), which also re-arms the array's header.
 */
#define AGG_NOALLOC_MAX_BYTES ((size_t)64 << 20)
int ag_gemm_f16_noalloc(const void *const *shards, int n_shards, const void *B,
                        float *C, int64_t M, int64_t K, int64_t N,
                        int chunk_rows, void *stream, const agg_options *opt);

/*
 * bf16 x bf16 -> fp32 streamed AllGather + GEMM: the fp16 operation above
 * with bfloat16 shards and B (same layouts, alignment, size limits and
 * errors; C fp32).  A variant of the PTO-ISA README's fp16 path in the
 * other 16-bit input format.
 */
int ag_gemm_bf16(const void *const *shards, int n_shards, const void *B,
                 float *C, int64_t M, int64_t K, int64_t N, int chunk_rows,
                 void *stream);
int ag_gemm_bf16_ex(const void *const *shards, int n_shards, const void *B,
                    float *C, int64_t M, int64_t K, int64_t N, int chunk_rows,
                    void *stream, const agg_options *opt);

/*
 * fp8 x fp8 -> fp32 streamed AllGather + GEMM: the fp16 operation above
 * with OCP FP8 E4M3 shards and B (1 byte per element, the float8_e4m3fn
 * format of the FP8 grouped-GEMM variant on the Ascend SHMEM blog page).
 * Same layouts, alignment, size limits and errors as ag_gemm_f16, except
 * that K must be a multiple of 16 (one 16-byte load holds 16 elements; N
 * stays a multiple of 8); C fp32.  NaN inputs propagate as the matrix
 * cores make them.
 */
int ag_gemm_fp8(const void *const *shards, int n_shards, const void *B,
                float *C, int64_t M, int64_t K, int64_t N, int chunk_rows,
                void *stream);
int ag_gemm_fp8_ex(const void *const *shards, int n_shards, const void *B,
                   float *C, int64_t M, int64_t K, int64_t N, int chunk_rows,
                   void *stream, const agg_options *opt);

/*
 * int8 x int8 -> int32, + bias, x per-channel scale -> fp16
 * (catccos AllGatherMatmulDequant design doc, sections 1.2 and 2.2):
 *   v = A x B + bias[n]        exact int32
 *   C = fp16_rne(fp32_rne(v) * scale[n])
 *   shards  HOST array of n_shards DEVICE int8 [S, K] row-major blocks.
 *   B       DEVICE int8 [K, N] row-major.
 *   bias    DEVICE int32 [N];  scale DEVICE fp32 [N] (per output channel).
 *   C       DEVICE fp16 [M, N] row-major, fully overwritten.
 * Requires K % 16 == 0 and N % 8 == 0.  The caller guarantees that every
 * |v| < 2^31 (int32 accumulation does not saturate).
 */
int ag_gemm_i8_dequant(const int8_t *const *shards, int n_shards,
                       const int8_t *B, const int32_t *bias,
                       const float *scale, void *C, int64_t M, int64_t K,
                       int64_t N, int chunk_rows, void *stream);
int ag_gemm_i8_dequant_ex(const int8_t *const *shards, int n_shards,
                          const int8_t *B, const int32_t *bias,
                          const float *scale, void *C, int64_t M, int64_t K,
                          int64_t N, int chunk_rows, void *stream,
                          const agg_options *opt);

/*
 * Rows per chunk so that each source has 64 to 127 chunks of all of K:
 * max(1, S / 64) (PTO-ISA README, "dynamic chunk size": 64-128 chunks per
 * source).  The automatic choice for whole-K chunks; where K-blocks are
 * allowed the automatic chunks are S/16 rows x K/4 (see ag_gemm_f16).
 * Returns 0 for S < 1.
 */
int ag_gemm_pick_chunk_rows(int64_t shard_rows);

/* Bytes of workspace one call needs with full slots (workspace_stages 0):
 * a counter header plus one slot of S x K elements for every remote shard.
 * 0 on invalid sizes.  A call with a workspace ring needs less, as
 * ag_gemm_plan reports in agg_plan_info.workspace_bytes. */
size_t ag_gemm_workspace_bytes(int n_shards, int64_t M, int64_t K,
                               int elt_bytes);

/* Make a caller-owned workspace ready (zeroes its counter header on
 * `stream`); needed once after allocating it, and again before a memory
 * area that held another workspace (or anything else) is used as one.
 * The library's side stream is ordered after the reset (one event), so no
 * producer of a later call reads the header before it is zeroed.  Call
 * ag_gemm_check() after the last call that used it before freeing it.
 * A library convention (query the size, prepare, then execute), not an
 * operation of the pages. */
int ag_gemm_workspace_reset(void *workspace, size_t bytes, void *stream);

/*
 * Synchronise `stream` and the library's side stream and report whether
 * the calls issued since the last check on this device timed out
 * (AGG_E_TIMEOUT) or failed in HIP (AGG_E_HIP).  Looks only at workspaces
 * used since the last check; clears the recorded error and re-arms the
 * counters of a workspace whose call failed.
 */
int ag_gemm_check(void *stream);

/* Human-readable text for an agg_status value. */
const char *ag_gemm_status_string(int status);

/* Free the internal workspaces and side streams of every device. */
void ag_gemm_release(void);

/* ---- planning queries (host only, no GPU needed) ----------------------- */

typedef struct agg_plan_info {
    int64_t shard_rows;     /* S */
    int chunk_rows;         /* rows per chunk */
    int chunks_per_source;  /* ceil(S / chunk_rows) x k_blocks */
    int tile_m, tile_n;     /* consumer output tile */
    int m_tiles_per_shard;  /* ceil(S / tile_m) */
    int n_tiles;            /* ceil(N / tile_n) */
    int64_t total_tiles;    /* n_shards * m_tiles_per_shard * n_tiles
                               (times k_splits with split-K)             */
    int64_t total_chunks;   /* (n_shards - 1) * chunks_per_source */
    int consumer_wgs;       /* persistent consumer grid */
    int producer_wgs;       /* producer grid */
    int tile_id;            /* consumer tile configuration (agg_options.tile) */
    int64_t trace_words;    /* 1 + total_chunks + 3 * total_tiles          */
    int workspace_stages;   /* ring stages per remote shard (0: full slots) */
    int64_t workspace_bytes; /* workspace this call needs (a caller-owned
                                workspace must be at least this large)     */
    int k_splits;           /* parts of K per output tile (1: no split-K)   */
    int k_blocks;           /* K-blocks per row chunk (1: chunks span K)    */
    int64_t k_block;        /* elements of K per K-block (K when 1 block)   */
    int producer_fused;     /* 1: producer and consumer in one launch        */
} agg_plan_info;

/*
 * The schedule one call would run, for inspection and tests.
 *   kind: 0 = fp16 path, 1 = int8 path, 2 = bf16 path, 3 = fp8 path; num_cus: CUs of
 *   the device to plan for (0 = 256).  tile_order (nullable, capacity total_tiles * 4 int32):
 *   per consumer position: shard, m-tile, n-tile, counter value waited for
 *   before the tile's first K-block (0 for the local shard), for a grid of
 *   consumer_wgs workgroups (when its rounds do not hold whole row panels,
 *   positions walk groups of a few panels column by column, so that each
 *   XCD's stretch of a round is a compact block); with split-K the positions run part after
 *   part, each part's positions in the same order, so each (shard, m-tile,
 *   n-tile) appears once per part.  chunk_order (nullable, capacity
 *   total_chunks * 2 int32): per producer position: shard, chunk index
 *   (K-block * ceil(S / chunk_rows) + row chunk).
 */
int ag_gemm_plan(int kind, int n_shards, int64_t M, int64_t K, int64_t N,
                 int chunk_rows, const agg_options *opt, int num_cus,
                 agg_plan_info *info, int32_t *tile_order,
                 int32_t *chunk_order);

#ifdef __cplusplus
}
#endif
#endif /* AGGEMM_H */
