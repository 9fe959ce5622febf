// api.cpp -- the C ABI: argument checks, per-device state (side stream,
// events, workspace, counter bookkeeping) and the launch sequence of one
// call (PTO-ISA AllGather+GEMM README: the host enqueues the communication
// kernel and the compute kernel on two streams, then waits for both).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <map>
#include <mutex>

#include "aggemm.h"
#include "kernels.hpp"
#include "plan.hpp"

namespace agg {
namespace {

// Counter bookkeeping of one workspace: the value every counter holds once
// all calls issued on it have finished, the last call's epoch and the last
// epoch whose outcome ag_gemm_check() has reported.
struct Track {
    uint32_t base[kMaxShards];
    uint32_t epoch;
    uint32_t checked;
    int device;
    bool used;                 // a call ran on it since the last check
    // A stream other than the caller's on which a producer of this
    // workspace was queued last (the library's side stream or a CU-masked
    // one), or null.  Such a producer can still be finishing its last
    // counter update when the call's consumer has ended; a producer queued
    // elsewhere must not start before that, or the two would work on the
    // same counters out of order.
    hipStream_t pending;
};

struct Device {
    bool ready = false;        // side stream and events made
    int id = 0;
    int num_cus = 0;           // 0 until the attributes were read
    double clock_hz = 0;       // rate of the device's constant clock
    hipStream_t side = nullptr;
    hipEvent_t fork = nullptr;  // orders a ring-mode producer after the consumer
    hipEvent_t join = nullptr;  // joins a CU-masked consumer back to the caller
    hipEvent_t drain = nullptr; // orders a producer after one on another stream
    hipStream_t pmask[3] = {};  // CU-masked producer / consumer streams, by
    hipStream_t cmask[3] = {};  //   producer CUs / 32 (made on first use)
    char* scratch = nullptr;   // the allocation-free entry point's array here
    char* ws = nullptr;        // internal workspace
    size_t ws_bytes = 0;
    Track track{};
    int occ[4][32] = {{0}};   // by kind and tile id
};

std::mutex g_mu;
std::map<int, Device> g_dev;
std::map<void*, Track> g_user_ws;   // caller-owned workspaces, by address

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Bound of a pipelined producer's wait for its consumer to start: the work
// queued ahead of a call on the caller's stream may take long, and a call
// must not fail for it (the chunk waits keep the call's own limit).
constexpr double kStartWaitSeconds = 120.0;

// The device's entry with its CU count and clock rate (attribute queries
// only: nothing is created or enqueued, so argument errors can still be
// reported before any side effect).
int device_entry(Device** out)
{
    int id = 0;
    if (hipGetDevice(&id) != hipSuccess) return AGG_E_HIP;
    Device& d = g_dev[id];
    if (!d.num_cus) {
        int cus = 0, khz = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, id) != hipSuccess)
            return AGG_E_HIP;
        if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, id) != hipSuccess)
            return AGG_E_HIP;
        d.num_cus = cus > 0 ? cus : 256;
        d.clock_hz = (khz > 0 ? khz : 100000) * 1000.0;
        d.id = id;
    }
    *out = &d;
    return AGG_OK;
}

// The side stream must not run a producer before a header reset queued on
// `st` has run: the producer polls words of the header (start word, error
// word, counters) that hold stale values until then.  One event, once per
// reset (a one-time preparation, so its cross-stream cost does not recur).
int order_side_after(Device& d, hipStream_t st)
{
    if (hipEventRecord(d.fork, st) != hipSuccess) return AGG_E_HIP;
    if (hipStreamWaitEvent(d.side, d.fork, 0) != hipSuccess) return AGG_E_HIP;
    return AGG_OK;
}

// Per-device set-up, at the first call of any entry point on the device
// (with it current): the side stream and event, and the allocation-free
// entry point's fixed array -- its address here (taking it loads the code
// that holds the array, which the runtime places on the device then, not
// inside a later allocation-free call) and its counter header zeroed on
// `st`, registered like a caller-owned workspace so that ag_gemm_check()
// looks at it and re-arms it after a failure.
int device_ready(Device& d, hipStream_t st)
{
    if (d.ready) return AGG_OK;
    if (!d.side && hipStreamCreateWithFlags(&d.side, hipStreamNonBlocking) != hipSuccess)
        return AGG_E_HIP;
    if (!d.fork && hipEventCreateWithFlags(&d.fork, hipEventDisableTiming) != hipSuccess)
        return AGG_E_HIP;
    if (!d.join && hipEventCreateWithFlags(&d.join, hipEventDisableTiming) != hipSuccess)
        return AGG_E_HIP;
    if (!d.drain && hipEventCreateWithFlags(&d.drain, hipEventDisableTiming) != hipSuccess)
        return AGG_E_HIP;
    void* p = nullptr;
    if (scratch_address(&p) != hipSuccess) {
        (void)hipGetLastError();
        return AGG_E_HIP;
    }
    if (launch_header_reset(static_cast<uint32_t*>(p), kHeaderBytes, st) != hipSuccess)
        return AGG_E_HIP;
    int rc = order_side_after(d, st);
    if (rc) return rc;
    Track t;
    memset(&t, 0, sizeof t);
    t.device = d.id;
    g_user_ws[p] = t;
    d.scratch = static_cast<char*>(p);
    memset(&d.track, 0, sizeof d.track);
    d.track.device = d.id;
    d.ready = true;
    return AGG_OK;
}

int device_state(Device** out, hipStream_t st)
{
    int rc = device_entry(out);
    if (rc) return rc;
    return device_ready(**out, st);
}

// ---- plan cache --------------------------------------------------------
//
// A call's plan depends only on its sizes, the options that shape the
// schedule and the device's CU count; calls in a loop repeat the same
// ones, so the last few plans are kept (looked up under the library lock).
struct PlanKey {
    int kind, n, chunk_rows, num_cus;
    int64_t M, K, N;
    uint32_t struct_size;
    int local_shard, mode, link_model, producer_wgs, consumer_wgs, tile;
    int workspace_stages, scheme, pvalue, k_splits, debug_drop_chunk, producer, producer_cus;
    double link_gbps, timeout_ms, delay_us;
    int64_t piece, k_block;
    int has_order;
    int order[kMaxShards];
};

struct PlanSlot {
    bool used;
    PlanKey key;
    int rc;
    Plan plan;
};

constexpr int kPlanSlots = 8;
PlanSlot g_plans[kPlanSlots];
int g_plan_next = 0;

void plan_key(PlanKey* k, Kind kind, int n, int64_t M, int64_t K, int64_t N, int chunk_rows,
              const agg_options* o, int num_cus)
{
    memset(k, 0, sizeof *k);   // padding bytes take part in the comparison
    k->kind = (int)kind;
    k->n = n;
    k->chunk_rows = chunk_rows;
    k->num_cus = num_cus;
    k->M = M;
    k->K = K;
    k->N = N;
    k->struct_size = o->struct_size;
    k->local_shard = o->local_shard;
    k->mode = o->mode;
    k->link_model = o->link_model;
    k->producer_wgs = o->producer_wgs;
    k->consumer_wgs = o->consumer_wgs;
    k->tile = o->tile;
    k->workspace_stages = o->workspace_stages;
    k->scheme = o->scheme;
    k->pvalue = o->pvalue;
    k->k_splits = o->k_splits;
    k->debug_drop_chunk = o->debug_drop_chunk;
    k->producer = o->producer;
    k->producer_cus = o->producer_cus;
    k->link_gbps = o->link_gbps;
    k->timeout_ms = o->timeout_ms;
    k->delay_us = o->debug_delay_us;
    k->piece = o->producer_piece_bytes;
    k->k_block = o->k_block;
    k->has_order = o->send_order != nullptr;
    if (o->send_order && n > 1 && n <= kMaxShards)
        for (int i = 0; i + 1 < n; ++i) k->order[i] = o->send_order[i];
}

// The plan of a call (made, or found among the last few); a positive
// status for invalid arguments.
int cached_plan(Kind kind, int n, int64_t M, int64_t K, int64_t N, int chunk_rows,
                const agg_options* o, int num_cus, const Plan** out)
{
    PlanKey k;
    plan_key(&k, kind, n, M, K, N, chunk_rows, o, num_cus);
    for (int i = 0; i < kPlanSlots; ++i) {
        PlanSlot& sl = g_plans[i];
        if (sl.used && memcmp(&sl.key, &k, sizeof k) == 0) {
            *out = &sl.plan;
            return sl.rc;
        }
    }
    PlanSlot& sl = g_plans[g_plan_next];
    g_plan_next = (g_plan_next + 1) % kPlanSlots;
    sl.used = true;
    sl.key = k;
    sl.rc = make_plan(kind, n, M, K, N, chunk_rows, o, num_cus, &sl.plan);
    *out = &sl.plan;
    return sl.rc;
}

int occupancy(Device& d, int kind, int tile)
{
    int& o = d.occ[kind][tile & 31];
    if (!o) o = consumer_occupancy(kind, tile);
    return o;
}

// The internal workspace, grown on demand.  Growing frees the old one,
// which waits for work still using it.
int internal_workspace(Device& d, size_t need, hipStream_t st, char** ws, Track** tr)
{
    if (d.ws_bytes < need) {
        if (d.ws) {
            if (hipDeviceSynchronize() != hipSuccess) return AGG_E_HIP;
            (void)hipFree(d.ws);
            d.ws = nullptr;
            d.ws_bytes = 0;
        }
        size_t bytes = need + (need >> 3);   // some headroom against regrowth
        if (hipMalloc(&d.ws, bytes) != hipSuccess) {
            d.ws = nullptr;
            (void)hipGetLastError();
            return AGG_E_NOMEM;
        }
        d.ws_bytes = bytes;
        if (launch_header_reset(reinterpret_cast<uint32_t*>(d.ws), kHeaderBytes, st) != hipSuccess)
            return AGG_E_HIP;
        // fresh memory holds anything: no producer may look at the header
        // before the reset has run
        int rc = order_side_after(d, st);
        if (rc) return rc;
        uint32_t keep = d.track.epoch;
        memset(&d.track, 0, sizeof d.track);
        d.track.epoch = keep;
        d.track.checked = keep;
    }
    *ws = d.ws;
    *tr = &d.track;
    return AGG_OK;
}

// The CU-masked stream pair for a producer of `cus` CUs (32 or 64): the
// producer's CUs spread evenly over the XCDs, the consumer's the rest.
int masked_streams(Device& d, int cus, hipStream_t* prod, hipStream_t* cons)
{
    const int i = cus / 32;
    if (!d.pmask[i]) {
        uint32_t m[8];
        producer_cu_mask(cus, m);
        uint32_t c[8];
        for (int w = 0; w < 8; ++w) c[w] = ~m[w];
        hipStream_t ps = nullptr, cs = nullptr;
        if (hipExtStreamCreateWithCUMask(&ps, 8, m) != hipSuccess) return AGG_E_HIP;
        if (hipExtStreamCreateWithCUMask(&cs, 8, c) != hipSuccess) {
            (void)hipStreamDestroy(ps);
            return AGG_E_HIP;
        }
        d.pmask[i] = ps;
        d.cmask[i] = cs;
    }
    *prod = d.pmask[i];
    *cons = d.cmask[i];
    return AGG_OK;
}

// The DMA producer (AGG_PRODUCER_SDMA): row group after row group in send
// order (group g: the row chunks m-tile g needs first), one copy per remote
// source on the DMA engines, then a stream write of the source's counter
// past the group's chunks -- the release, which the stream performs only
// after the copy has completed.  Chunks span all of K here.
hipError_t enqueue_sdma(const Schedule& s, const ProducerArgs& pa, int elt, hipStream_t st)
{
    const size_t row_bytes = (size_t)s.K * (size_t)elt;
    const int remotes = s.n_shards - 1;
    auto group = [&](int src, int g) -> hipError_t {
        const int shard = s.order[1 + src];
        const int f = g == 0 ? 0 : need_chunks(s, g - 1);
        const int e = need_chunks(s, g);
        if (e <= f) return hipSuccess;   // chunks taller than a tile: empty group
        const int64_t r0 = (int64_t)f * s.cr, r1 = chunk_row_end(s, e - 1);
        hipError_t err = hipMemcpyAsync(pa.dst[shard] + r0 * row_bytes, pa.src[shard] + r0 * row_bytes,
                                        (size_t)(r1 - r0) * row_bytes,
                                        hipMemcpyDeviceToDeviceNoCU, st);
        if (err != hipSuccess) return err;
        return hipStreamWriteValue32(st, pa.counters + shard * (kCounterStride / 4),
                                     pa.base[shard] + (uint32_t)e, 0);
    };
    hipError_t err = hipSuccess;
    if (s.link_model == 0) {
        for (int g = 0; g < s.mt && err == hipSuccess; ++g)
            for (int src = 0; src < remotes && err == hipSuccess; ++src) err = group(src, g);
    } else {
        for (int src = 0; src < remotes && err == hipSuccess; ++src)
            for (int g = 0; g < s.mt && err == hipSuccess; ++g) err = group(src, g);
    }
    return err;
}

struct Call {
    Kind kind;
    const void* const* shards;
    int n;
    const void* B;
    const int32_t* bias;
    const float* scale;
    void* C;
    int64_t M, K, N;
    int chunk_rows;
    hipStream_t st;
    const agg_options* opt;
    bool scratch;   // the allocation-free entry point: the fixed array as workspace
};

int run(const Call& c)
{
    agg_options def;
    ag_gemm_options_init(&def);
    const agg_options* opt = c.opt ? c.opt : &def;

    // pointer checks first: they need no device
    if (!c.shards || c.n < 1) return AGG_E_INVALID;
    if (c.n > kMaxShards) return AGG_E_UNSUPPORTED;
    if (c.M < 0 || c.K < 0 || c.N < 0) return AGG_E_INVALID;
    const bool empty = c.M == 0 || c.N == 0;
    if (!empty) {
        if (c.K > 0) {
            for (int i = 0; i < c.n; ++i) {
                if (!c.shards[i]) return AGG_E_INVALID;
                if (!aligned(c.shards[i], 16)) return AGG_E_UNSUPPORTED;
            }
            if (!c.B) return AGG_E_INVALID;
            if (!aligned(c.B, 16)) return AGG_E_UNSUPPORTED;
        }
        if (!c.C) return AGG_E_INVALID;
        if (!aligned(c.C, 16)) return AGG_E_UNSUPPORTED;
        if (c.kind == kI8) {
            if (!c.bias || !c.scale) return AGG_E_INVALID;
            if (!aligned(c.bias, 4) || !aligned(c.scale, 4)) return AGG_E_UNSUPPORTED;
            if (opt->acc_out && !aligned(opt->acc_out, 16)) return AGG_E_UNSUPPORTED;
        }
    }
    if (opt->trace && !aligned(opt->trace, 8)) return AGG_E_UNSUPPORTED;
    // DMA copies leave no release stamps
    if (opt->trace && opt->producer == AGG_PRODUCER_SDMA) return AGG_E_UNSUPPORTED;
    if (c.scratch && opt->workspace) return AGG_E_INVALID;

    // Every argument check runs before anything is created or enqueued:
    // the plan needs only the device's attributes (and argument errors are
    // reported even where no device can be queried: the plan then assumes
    // 256 CUs).
    std::lock_guard<std::mutex> lock(g_mu);
    Device* d = nullptr;
    const int drc = device_entry(&d);
    const Plan* pp = nullptr;
    int rc = cached_plan(c.kind, c.n, c.M, c.K, c.N, c.chunk_rows, opt,
                         drc == AGG_OK ? d->num_cus : 0, &pp);
    if (rc) return rc;
    const Plan& p = *pp;
    if (c.scratch && p.ws_bytes > kScratchBytes) return AGG_E_TOO_LARGE;
    if (empty) return AGG_OK;   // nothing to compute or move
    if (drc) return drc;
    rc = device_ready(*d, c.st);
    if (rc) return rc;

    const int kind = static_cast<int>(c.kind);
    const bool run_producer = p.mode != AGG_MODE_COMPUTE_ONLY && c.n > 1 && c.K > 0;
    const bool run_consumer = p.mode != AGG_MODE_COPY_ONLY;

    // workspace
    char* ws = nullptr;
    Track* tr = nullptr;
    if (opt->workspace) {
        auto it = g_user_ws.find(opt->workspace);
        if (it == g_user_ws.end() || opt->workspace_bytes < p.ws_bytes) return AGG_E_INVALID;
        ws = static_cast<char*>(opt->workspace);
        tr = &it->second;
    } else if (c.scratch) {
        // set up with the device (device_ready): no allocation, no reset here
        ws = d->scratch;
        tr = &g_user_ws[d->scratch];
    } else {
        rc = internal_workspace(*d, p.ws_bytes, c.st, &ws, &tr);
        if (rc) return rc;
    }
    const uint32_t epoch = ++tr->epoch;
    tr->used = true;
    const double timeout_ms = opt->timeout_ms > 0 ? opt->timeout_ms : 2000.0;
    const uint64_t limit = (uint64_t)(timeout_ms * 1e-3 * d->clock_hz);
    uint32_t* header = reinterpret_cast<uint32_t*>(ws);

    const Schedule& s = p.sched;
    const size_t slot = p.slot_bytes;
    ConsumerArgs ca;
    memset(&ca, 0, sizeof ca);
    ProducerArgs pa;
    memset(&pa, 0, sizeof pa);
    ca.s = s;
    pa.s = s;
    for (int i = 0; i < c.n; ++i) {
        const char* src = static_cast<const char*>(c.shards[i]);
        char* dst = s.slot[i] >= 0 ? ws + kHeaderBytes + slot * (size_t)s.slot[i] : nullptr;
        ca.a[i] = (i == s.local) ? src : dst;
        pa.src[i] = src;
        pa.dst[i] = dst;
        ca.base[i] = tr->base[i];
        pa.base[i] = tr->base[i];
    }
    ca.B = static_cast<const char*>(c.B);
    ca.C = c.C;
    ca.counters = header;
    ca.flags = header + kFlagOffset / 4;
    ca.err = header + kErrorOffset / 4;
    ca.epoch = epoch;
    // the consumer waits on counters only while a producer runs beside it
    ca.no_wait = !(p.mode == AGG_MODE_PIPELINED && run_producer);
    ca.limit = limit;
    ca.bias = c.bias;
    ca.scale = c.scale;
    ca.acc_out = opt->acc_out;
    ca.trace = opt->trace ? opt->trace + 1 + total_chunks(s) : nullptr;
    ca.partials = s.ks > 1 ? ws + p.part_off : nullptr;
    ca.tickets = header + kTicketOffset / 4;
    ca.trace_start = opt->trace;
    pa.trace = opt->trace;
    pa.counters = header;
    pa.flags = header + kFlagOffset / 4;
    pa.pieces = reinterpret_cast<uint32_t*>(ws + kPieceOffset);
    pa.piece = p.piece;
    pa.ppc = p.ppc;
    // Piece flags (a chunk counts as released once each of its pieces is
    // flagged, before the last piece's running-total add returns): for the
    // producer kernel with at most kPieceFlags pieces a chunk and three or
    // more remote sources, whose round-0 tiles wait for the first chunks (on
    // 2 x 1024 rows, K 2048, N 1024 they cost 1 us a call).  Paced, the
    // consumer takes a piece-flagged chunk only once the chunk's paced time
    // has passed (parallel links: a source's own bytes set it).
    const bool piece_flags = p.producer != AGG_PRODUCER_SDMA && p.ppc <= kPieceFlags &&
                             c.n >= 4 && !(p.link_gbps > 0 && s.link_model != 0);
    pa.piece_flags = piece_flags ? header + kPieceFlagOffset / 4 : nullptr;
    ca.piece_flags = pa.piece_flags;
    ca.ppc = p.ppc;
    pa.err = header + kErrorOffset / 4;
    pa.clock = reinterpret_cast<uint64_t*>(ws + kClockOffset);
    pa.epoch = epoch;
    pa.elt = p.elt;
    pa.drop = p.drop_chunk;
    pa.delay_seed = opt->debug_delay_seed;
    pa.delay_max = (uint32_t)(opt->debug_delay_us * 1e-6 * d->clock_hz);
    pa.ticks_per_byte = p.link_gbps > 0 ? d->clock_hz / (p.link_gbps * 1e9) : 0.0;
    {
        // the paced time a consumer gives a piece-flagged chunk is never
        // earlier than the chunk flag's: whole KiB and ticks per KiB both
        // rounded up, one tick added
        const double q = std::ceil(pa.ticks_per_byte * p.elt * 1024.0 * 65536.0);
        ca.ticks_per_kib_q16 =
            p.link_gbps > 0 ? (q < 4294967295.0 && q >= 1.0 ? (uint32_t)q : 0xffffffffu) : 0;
        ca.clock = pa.clock;
    }
    pa.limit = limit;
    // the producer's wait for the consumer's start covers the work queued
    // ahead of the call on the caller's stream, not a chunk: its own bound
    pa.start_limit = limit > (uint64_t)(kStartWaitSeconds * d->clock_hz)
                         ? limit : (uint64_t)(kStartWaitSeconds * d->clock_hz);

    int occ = occupancy(*d, kind, p.shape.id);
    if (occ < 1) return AGG_E_HIP;
    // the plan's rule for a fused launch and the kernels built agree
    if (p.fused && !fused_built(kind, p.shape.id)) return AGG_E_UNSUPPORTED;
    int cwgs = p.consumer_wgs;
    // a persistent grid larger than what can be resident at once gains
    // nothing, and its waiting workgroups would sit in front of the producer
    const int ccus = d->num_cus - p.producer_cus;
    if (cwgs > ccus * occ) cwgs = ccus * occ;
    // No slots are held back for the producer: every consumer kernel leaves
    // room for producer waves on each CU even at full occupancy.
    // Workgroups of one XCD take neighbouring tiles (the grid is now final).
    ca.s.xf = pick_xcd_split(ca.s, cwgs);
    ca.s.gm = pick_group(ca.s, cwgs);

    hipEvent_t* cev = reinterpret_cast<hipEvent_t*>(const_cast<void**>(opt->consumer_events));
    auto consumer = [&](hipStream_t st) -> hipError_t {
        hipError_t e = hipSuccess;
        if (cev[0]) e = hipEventRecord(cev[0], st);
        if (e == hipSuccess)
            e = c.kind == kF16    ? launch_consumer_f16(ca, p.shape.id, cwgs, st)
                : c.kind == kBF16 ? launch_consumer_bf16(ca, p.shape.id, cwgs, st)
                : c.kind == kFP8  ? launch_consumer_fp8(ca, p.shape.id, cwgs, st)
                                  : launch_consumer_i8(ca, p.shape.id, cwgs, st);
        if (e == hipSuccess && cev[1]) e = hipEventRecord(cev[1], st);
        return e;
    };

    const bool sdma = p.producer == AGG_PRODUCER_SDMA;
    // the producer of this call goes on stream x: after this workspace's
    // last producer if that one was queued on another stream (a one-time
    // cross-stream wait when calls change how they run)
    auto producer_on = [&](hipStream_t x) -> hipError_t {
        hipError_t r = hipSuccess;
        if (tr->pending && tr->pending != x) {
            r = hipEventRecord(d->drain, tr->pending);
            if (r == hipSuccess) r = hipStreamWaitEvent(x, d->drain, 0);
        }
        tr->pending = x == c.st ? nullptr : x;
        return r;
    };
    hipError_t e = hipSuccess;
    if (p.mode == AGG_MODE_PIPELINED && run_producer && run_consumer && p.fused) {
        // One launch on the caller's stream, the producer's workgroups
        // first; stream order replaces the start word.
        e = producer_on(c.st);
        if (e == hipSuccess && cev[0]) e = hipEventRecord(cev[0], c.st);
        if (e == hipSuccess)
            e = launch_fused(kind, ca, pa, p.shape.id, cwgs, p.producer_wgs, c.st);
        if (e == hipSuccess && cev[1]) e = hipEventRecord(cev[1], c.st);
    } else if (p.mode == AGG_MODE_PIPELINED && run_producer && run_consumer) {
        // In the default form the producer is queued first, so that its
        // workgroups are dispatched while the consumer's start; each
        // kernel fits beside the other on a CU, so neither order keeps a
        // consumer workgroup off the chip.  No event joins the two streams
        // (a cross-stream dependency costs about 13 us on this stack, each
        // way):
        // - the producer waits on the device for the consumer's start word
        //   instead of an event on the caller's stream;
        // - the caller's stream does not wait for the producer: the
        //   consumer waits for every chunk's release, and the producer
        //   releases a chunk only after all of its reads of the shards and
        //   all of its writes of the chunk, so once the consumer is done
        //   the producer neither reads the caller's buffers nor writes
        //   anything the caller or the next call can see.  Calls that
        //   share a workspace stay ordered: the next producer is queued
        //   behind this one on the side stream and waits for the next
        //   consumer's start.
        ca.start = header + kStartOffset / 4;
        pa.start = header + kStartOffset / 4;
        // every copy is written by some consumer workgroup
        ca.start_copies = cwgs < kStartCopies ? cwgs : kStartCopies;
        pa.start_copies = ca.start_copies;
        if (s.ring > 0) {
            ca.stages = reinterpret_cast<uint64_t*>(ws + kStageOffset);
            pa.stages = ca.stages;
        }
        if (sdma) {
            // DMA copies cannot wait on a word: an event on the caller's
            // stream, recorded before the consumer, holds them back until
            // the work ahead of the call is done.  The join is as above:
            // the counter writes follow the copies on the library's stream.
            e = producer_on(d->side);
            if (e == hipSuccess) e = hipEventRecord(d->fork, c.st);
            if (e == hipSuccess) e = consumer(c.st);
            if (e == hipSuccess) e = hipStreamWaitEvent(d->side, d->fork, 0);
            if (e == hipSuccess) e = enqueue_sdma(s, pa, p.elt, d->side);
        } else if (p.producer_cus) {
            // Disjoint CU sets: the consumer on the complement-masked
            // stream, forked from and joined to `stream` by events (the
            // start word still gates the producer).  With disjoint CUs the
            // producer cannot keep a consumer workgroup off its CU, so a
            // workspace ring needs no further ordering.
            hipStream_t ps = nullptr, cs = nullptr;
            rc = masked_streams(*d, p.producer_cus, &ps, &cs);
            if (rc) return rc;
            e = producer_on(ps);
            if (e == hipSuccess) e = hipEventRecord(d->fork, c.st);
            if (e == hipSuccess) e = hipStreamWaitEvent(cs, d->fork, 0);
            if (e == hipSuccess) e = consumer(cs);
            if (e == hipSuccess) e = launch_producer(pa, p.producer_wgs, ps);
            if (e == hipSuccess) e = hipEventRecord(d->join, cs);
            if (e == hipSuccess) e = hipStreamWaitEvent(c.st, d->join, 0);
        } else if (s.ring > 0) {
            // With a workspace ring the producer also waits for consumer
            // tiles, so consumer workgroups must not be kept off the CUs by
            // producer workgroups dispatched ahead of them.  An event on
            // the caller's stream, recorded before the consumer, holds the
            // producer back until the work ahead of the call is done, by
            // which time the consumer's grid has been dispatched.  (Should
            // a wait still starve, it ends at the time limit as an error.)
            e = producer_on(d->side);
            if (e == hipSuccess) e = hipEventRecord(d->fork, c.st);
            if (e == hipSuccess) e = consumer(c.st);
            if (e == hipSuccess) e = hipStreamWaitEvent(d->side, d->fork, 0);
            if (e == hipSuccess) e = launch_producer(pa, p.producer_wgs, d->side);
        } else {
            e = producer_on(d->side);
            if (e == hipSuccess) e = launch_producer(pa, p.producer_wgs, d->side);
            if (e == hipSuccess) e = consumer(c.st);
        }
    } else {
        if (run_producer) {
            e = producer_on(c.st);
            if (e == hipSuccess)
                e = sdma ? enqueue_sdma(s, pa, p.elt, c.st)
                         : launch_producer(pa, p.producer_wgs, c.st);
        }
        if (e == hipSuccess && run_consumer) e = consumer(c.st);
    }
    if (e != hipSuccess) return AGG_E_HIP;
    if (run_producer) {
        for (int i = 0; i < c.n; ++i)
            if (i != s.local) tr->base[i] += (uint32_t)s.cps;
    }
    return AGG_OK;
}

int check_track(Track& t, uint32_t* header, hipStream_t st)
{
    uint32_t err = 0;
    if (hipMemcpy(&err, header + kErrorOffset / 4, sizeof err, hipMemcpyDeviceToHost) != hipSuccess)
        return AGG_E_HIP;
    int rc = AGG_OK;
    if (err && (int32_t)(err - t.checked) > 0) {
        rc = AGG_E_TIMEOUT;
        // a failed call leaves counters short: start over from zero
        if (launch_header_reset(header, kHeaderBytes, st) != hipSuccess) return AGG_E_HIP;
        if (hipStreamSynchronize(st) != hipSuccess) return AGG_E_HIP;
        memset(t.base, 0, sizeof t.base);
    }
    t.checked = t.epoch;
    t.used = false;
    return rc;
}

}  // namespace
}  // namespace agg

using namespace agg;

extern "C" {

int ag_gemm_f16(const void* const* shards, int n_shards, const void* B, float* C,
                int64_t M, int64_t K, int64_t N, int chunk_rows, void* stream)
{
    return ag_gemm_f16_ex(shards, n_shards, B, C, M, K, N, chunk_rows, stream, nullptr);
}

int ag_gemm_f16_ex(const void* const* shards, int n_shards, const void* B, float* C,
                   int64_t M, int64_t K, int64_t N, int chunk_rows, void* stream,
                   const agg_options* opt)
{
    Call c{kF16, shards, n_shards, B, nullptr, nullptr, C, M, K, N, chunk_rows,
           static_cast<hipStream_t>(stream), opt, false};
    return run(c);
}

int ag_gemm_f16_noalloc(const void* const* shards, int n_shards, const void* B, float* C,
                        int64_t M, int64_t K, int64_t N, int chunk_rows, void* stream,
                        const agg_options* opt)
{
    Call c{kF16, shards, n_shards, B, nullptr, nullptr, C, M, K, N, chunk_rows,
           static_cast<hipStream_t>(stream), opt, true};
    return run(c);
}

int ag_gemm_bf16(const void* const* shards, int n_shards, const void* B, float* C,
                 int64_t M, int64_t K, int64_t N, int chunk_rows, void* stream)
{
    return ag_gemm_bf16_ex(shards, n_shards, B, C, M, K, N, chunk_rows, stream, nullptr);
}

int ag_gemm_bf16_ex(const void* const* shards, int n_shards, const void* B, float* C,
                    int64_t M, int64_t K, int64_t N, int chunk_rows, void* stream,
                    const agg_options* opt)
{
    Call c{kBF16, shards, n_shards, B, nullptr, nullptr, C, M, K, N, chunk_rows,
           static_cast<hipStream_t>(stream), opt, false};
    return run(c);
}

int ag_gemm_fp8(const void* const* shards, int n_shards, const void* B, float* C,
                int64_t M, int64_t K, int64_t N, int chunk_rows, void* stream)
{
    return ag_gemm_fp8_ex(shards, n_shards, B, C, M, K, N, chunk_rows, stream, nullptr);
}

int ag_gemm_fp8_ex(const void* const* shards, int n_shards, const void* B, float* C,
                   int64_t M, int64_t K, int64_t N, int chunk_rows, void* stream,
                   const agg_options* opt)
{
    Call c{kFP8, shards, n_shards, B, nullptr, nullptr, C, M, K, N, chunk_rows,
           static_cast<hipStream_t>(stream), opt, false};
    return run(c);
}

int ag_gemm_i8_dequant(const int8_t* const* shards, int n_shards, const int8_t* B,
                       const int32_t* bias, const float* scale, void* C, int64_t M,
                       int64_t K, int64_t N, int chunk_rows, void* stream)
{
    return ag_gemm_i8_dequant_ex(shards, n_shards, B, bias, scale, C, M, K, N,
                                 chunk_rows, stream, nullptr);
}

int ag_gemm_i8_dequant_ex(const int8_t* const* shards, int n_shards, const int8_t* B,
                          const int32_t* bias, const float* scale, void* C, int64_t M,
                          int64_t K, int64_t N, int chunk_rows, void* stream,
                          const agg_options* opt)
{
    Call c{kI8, reinterpret_cast<const void* const*>(shards), n_shards, B, bias, scale,
           C, M, K, N, chunk_rows, static_cast<hipStream_t>(stream), opt, false};
    return run(c);
}

int ag_gemm_workspace_reset(void* workspace, size_t bytes, void* stream)
{
    if (!workspace || bytes < (size_t)kHeaderBytes) return AGG_E_INVALID;
    if (!aligned(workspace, 256)) return AGG_E_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_mu);
    Device* d = nullptr;
    hipStream_t st = static_cast<hipStream_t>(stream);
    int rc = device_state(&d, st);
    if (rc) return rc;
    if (launch_header_reset(static_cast<uint32_t*>(workspace), kHeaderBytes, st) != hipSuccess)
        return AGG_E_HIP;
    // The memory may hold anything (a workspace's earlier life, a caller's
    // fill): a pipelined producer, which starts on the side stream without
    // waiting for `stream`, must not read the header before the reset.
    rc = order_side_after(*d, st);
    if (rc) return rc;
    Track t;
    memset(&t, 0, sizeof t);
    t.device = d->id;
    g_user_ws[workspace] = t;
    return AGG_OK;
}

int ag_gemm_check(void* stream)
{
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (hipStreamSynchronize(st) != hipSuccess) return AGG_E_HIP;
    std::lock_guard<std::mutex> lock(g_mu);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return AGG_E_HIP;
    // a pipelined call's producer runs on the side stream, which the
    // caller's stream does not wait for: finish it too before reading the
    // error word (or resetting the header after a failure)
    auto it = g_dev.find(dev);
    int rc = AGG_OK;
    if (it != g_dev.end() && it->second.ready) {
        Device& d = it->second;
        if (hipStreamSynchronize(d.side) != hipSuccess) return AGG_E_HIP;
        for (int i = 0; i < 3; ++i)
            if (d.pmask[i] && hipStreamSynchronize(d.pmask[i]) != hipSuccess) return AGG_E_HIP;
        if (d.ws && d.track.used) {
            int r = check_track(d.track, reinterpret_cast<uint32_t*>(d.ws), st);
            if (r) rc = r;
        }
    }
    // only workspaces that calls used since the last check: one the caller
    // has freed since then is never touched again
    for (auto& kv : g_user_ws) {
        if (kv.second.device != dev || !kv.second.used) continue;
        int r = check_track(kv.second, static_cast<uint32_t*>(kv.first), st);
        if (r && !rc) rc = r;
    }
    return rc;
}

void ag_gemm_release(void)
{
    std::lock_guard<std::mutex> lock(g_mu);
    int cur = 0;
    (void)hipGetDevice(&cur);
    for (auto& kv : g_dev) {
        Device& d = kv.second;
        if (!d.ready) continue;
        (void)hipSetDevice(kv.first);
        (void)hipDeviceSynchronize();
        if (d.ws) (void)hipFree(d.ws);
        if (d.fork) (void)hipEventDestroy(d.fork);
        if (d.join) (void)hipEventDestroy(d.join);
        for (int i = 0; i < 3; ++i) {
            if (d.pmask[i]) (void)hipStreamDestroy(d.pmask[i]);
            if (d.cmask[i]) (void)hipStreamDestroy(d.cmask[i]);
        }
        if (d.side) (void)hipStreamDestroy(d.side);
    }
    g_dev.clear();
    g_user_ws.clear();
    (void)hipSetDevice(cur);
}

}  // extern "C"
