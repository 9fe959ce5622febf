// sync.hpp -- device-side counter primitives for chunk readiness.
//
// A source's summary counter only grows: it counts the chunks of the
// source that are in place, in chunk order (PTO-ISA AllGather+GEMM README:
// the communication side atomically increments a per-source summary
// counter after each chunk; the compute side blocks until the counter
// reaches the value it expects).  Counters are never reset between calls: each call
// waits for base + n, the base carried over from the calls before it, and
// values are compared modulo 2^32 (the Pallas collective matmul page waits
// on a semaphore whose expected value grows with the step for the same
// reason).
//
// gfx950 has no compare-and-block on memory inside a kernel, so the waiting
// side polls with one lane, sleeps between polls and gives up after a time
// limit, leaving an error mark instead of hanging.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace agg {

__device__ inline uint64_t ticks()
{
    return __builtin_amdgcn_s_memrealtime();   // constant-rate clock
}

__device__ inline uint32_t load_agent(const uint32_t* p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline bool reached(uint32_t value, uint32_t target)
{
    return (int32_t)(value - target) >= 0;
}

// Mark the call `epoch` as failed (the error word keeps the largest
// failing epoch).
__device__ inline void raise_error(uint32_t* err, uint32_t epoch)
{
    __hip_atomic_fetch_max(err, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Poll *ctr until it reaches `target` (mod 2^32).  Relaxed: the caller
// acquires through the chunk flags afterwards.  Returns the value seen, or
// target - 1 after a time-out or after another workgroup of the same call
// failed.
__device__ inline uint32_t poll_until(const uint32_t* ctr, uint32_t target, uint32_t* err,
                                      uint32_t epoch, uint64_t limit)
{
    uint32_t v = load_agent(ctr);
    if (!reached(v, target)) {
        const uint64_t t0 = ticks();
        uint32_t spins = 0;
        do {
            __builtin_amdgcn_s_sleep(2);
            if ((++spins & 31u) == 0) {
                if (reached(load_agent(err), epoch)) return target - 1;
                if (ticks() - t0 > limit) {
                    raise_error(err, epoch);
                    return target - 1;
                }
            }
            v = load_agent(ctr);
        } while (!reached(v, target));
    }
    return v;
}

// Wait (relaxed) until *flag holds `epoch`; false after a time-out or a
// failure elsewhere in the call.
__device__ inline bool poll_flag(const uint32_t* flag, uint32_t epoch, uint32_t* err,
                                 uint64_t limit)
{
    if (load_agent(flag) == epoch) return true;
    const uint64_t t0 = ticks();
    uint32_t spins = 0;
    while (load_agent(flag) != epoch) {
        __builtin_amdgcn_s_sleep(2);
        if ((++spins & 31u) == 0) {
            if (reached(load_agent(err), epoch)) return false;
            if (ticks() - t0 > limit) {
                raise_error(err, epoch);
                return false;
            }
        }
    }
    return true;
}

// An epoch-tagged count: the call's epoch in the upper half, the count in
// the lower; a word left by an earlier call counts as zero, so it needs no
// reset between calls.
__device__ inline uint32_t tagged_count(uint64_t w, uint32_t epoch)
{
    return (uint32_t)(w >> 32) == epoch ? (uint32_t)w : 0u;
}

// Add one to an epoch-tagged count (relaxed, device scope).
__device__ inline void count_one(uint64_t* word, uint32_t epoch)
{
    uint64_t cur = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (;;) {
        const uint64_t next = ((uint64_t)epoch << 32) | (tagged_count(cur, epoch) + 1u);
        if (__hip_atomic_compare_exchange_strong(word, &cur, next, __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
            return;
    }
}

// Wait (relaxed) until an epoch-tagged count reaches `target`; false after
// a time-out or a failure elsewhere in the call.
__device__ inline bool poll_count(const uint64_t* word, uint32_t epoch, uint32_t target,
                                  uint32_t* err, uint64_t limit)
{
    auto seen = [&]() {
        return tagged_count(__hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                            epoch);
    };
    if (seen() >= target) return true;
    const uint64_t t0 = ticks();
    uint32_t spins = 0;
    while (seen() < target) {
        __builtin_amdgcn_s_sleep(2);
        if ((++spins & 31u) == 0) {
            if (reached(load_agent(err), epoch)) return false;
            if (ticks() - t0 > limit) {
                raise_error(err, epoch);
                return false;
            }
        }
    }
    return true;
}

// Pacing origin shared by all producer workgroups of one call: the first
// one to arrive stamps the clock, tagged with the call's epoch.
__device__ inline uint64_t pacing_origin(uint64_t* slot, uint32_t epoch)
{
    const uint64_t mask = (1ull << 40) - 1;
    const uint64_t tag = (uint64_t)(epoch & 0xffffffu);
    uint64_t now = ticks() & mask;
    uint64_t mine = (tag << 40) | now;
    uint64_t cur = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (;;) {
        if ((cur >> 40) == tag) return cur & mask;
        if (__hip_atomic_compare_exchange_strong(slot, &cur, mine, __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT))
            return now;
    }
}

// Sleep until the 40-bit clock has advanced `delta` past `origin`.
__device__ inline void wait_until(uint64_t origin, uint64_t delta)
{
    const uint64_t mask = (1ull << 40) - 1;
    while (((ticks() - origin) & mask) < delta)
        __builtin_amdgcn_s_sleep(1);
}

}  // namespace agg
