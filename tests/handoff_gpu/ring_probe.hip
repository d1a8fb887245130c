// ring_probe.hip -- test infrastructure, not part of libkda: the record handoff
// a fused prefill would need, run on the GPU.  Producer workgroups stream
// records into a ring of slots; every record is read by R consumer workgroups
// (one per value tile in a fused chain).  The protocol is the one modelled with
// host threads in tests/handoff_model/ring_model.cpp:
//
//   producer of chunk c:  wait until done[slot] >= R * (c / S)  (slot = c % S),
//                         write the record, then store ready[slot] = c + 1
//                         with release semantics at agent (device) scope;
//   consumer of chunk c:  wait until ready[slot] >= c + 1 with acquire loads at
//                         agent scope, read and check the record, then add 1 to
//                         done[slot] with a release at agent scope.
//
// Agent scope makes the flags and the records coherent across the XCDs'
// separate L2s (a release writes the producer's dirty L2 lines back, an
// acquire invalidates the consumer's stale ones), so no role needs to share an
// XCD with another.  Every wait is bounded and also polls one abort word: the
// first wait that runs out of polls stores its code there, and every other
// wait then returns at once, so the kernel always ends within about one bound.
// The host reads the abort word, the count of bad words and each workgroup's
// progress.
//
// Mode 2 keeps every stream inside one XCD instead and hands records over
// through that XCD's L2 alone, with no cache write-back or invalidation:
// workgroups are dispatched to the XCDs round-robin by id, so stream p's
// producer and consumers all get ids congruent to p mod 8.  The producer waits
// until its record stores are acknowledged (vector L1 writes through to L2)
// and then stores the flag; consumers poll the flag and read the record with
// loads that miss the vector L1 and are served by L2.  That is the ordering
// the memory model uses between the CUs of one XCD; it is not a scope the
// language offers, so each workgroup also reports the XCD it ran on and the
// test checks the placement and every word.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint32_t load_acquire(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_relaxed(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// How a wait observes the flag it polls, and what it does once the flag is
// seen: acquire loads on every poll (agent scope), relaxed agent-scope polls
// and one acquire fence after the poll that succeeds, or, within one XCD,
// relaxed polls alone (they miss the vector L1 and read L2).
enum class Poll { Acquire = 0, OneFence = 1, OneL2 = 2 };

// Polls *p until it reaches `want`.  All lanes read the same words, so the
// loop is uniform across the wave.  Returns false if the abort word is set, or
// if `spin_limit` polls pass or the wall clock passes `deadline` (then this
// wait's code goes into the abort word unless another code is already there).
// The deadline bounds the whole kernel, however the waits add up.
__device__ bool wait_at_least(const uint32_t *p, uint32_t want, uint32_t *abort_word, uint32_t code,
                              uint32_t spin_limit, uint64_t deadline, Poll mode) {
    for (uint32_t it = 0;; ++it) {
        if (mode == Poll::Acquire) {
            if (load_acquire(p) >= want) return true;
        } else if (load_relaxed(p) >= want) {
            if (mode == Poll::OneFence) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            // no later memory access of this wave moves above the poll that succeeded
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            return true;
        }
        if (load_relaxed(abort_word) != 0u) return false;
        if (it >= spin_limit || (uint64_t)wall_clock64() > deadline) {
            atomicCAS(abort_word, 0u, code);
            return false;
        }
        __builtin_amdgcn_s_sleep(2);
    }
}

// Publishes ready = c + 1 after this wave's record stores.  Agent scope: a
// release store.  One XCD: wait until every store of the wave is acknowledged
// (they have reached L2, where the consumers' polls and loads are served),
// then a relaxed store of the flag.
__device__ __forceinline__ void publish(uint32_t *flag, uint32_t v, Poll mode) {
    if (mode == Poll::OneL2) {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0); expcnt, lgkmcnt left at their maxima
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __hip_atomic_store(flag, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        __hip_atomic_store(flag, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
}

__device__ __forceinline__ uint32_t pattern(uint32_t p, uint32_t c, uint32_t i) {
    uint32_t x = p * 0x9E3779B1u ^ (c + 1u) * 0x85EBCA77u ^ i * 0xC2B2AE3Du;
    x ^= x >> 15;
    x *= 0x2C1B3C6Du;
    return x ^ (x >> 12);
}

// One wave per workgroup.  Roles: producer of stream p (role index p) or
// consumer r of stream p (role index P + p R + r).  Modes 0 and 1 give block b
// role b.  Mode 2 (P a multiple of 8) gives the blocks of XCD x = b mod 8, in
// the order k = b / 8, first the producers of streams x, x + 8, ..., then their
// consumers, so every stream's roles sit on one XCD.  Only the first
// n_active_producers streams produce; the others' consumers wait for records
// that never come (a host-forced timeout, for testing the abort path).
__global__ __launch_bounds__(64) void ring_probe_kernel(uint4 *__restrict__ ring, uint32_t *ready,
                                                        uint32_t *done, uint32_t *abort_word,
                                                        uint32_t *bad_words, uint32_t *progress,
                                                        uint32_t *xcc, int P, int R, int S,
                                                        int n_chunks, int rec_vec,
                                                        int n_active_producers, uint32_t spin_limit,
                                                        uint64_t max_ticks, int poll_mode) {
    const int b = blockIdx.x, lane = threadIdx.x;
    const Poll mode = static_cast<Poll>(poll_mode);
    const uint64_t deadline = (uint64_t)wall_clock64() + max_ticks;
    int role = b;
    if (mode == Poll::OneL2) {
        const int x = b & 7, k = b >> 3, per = P >> 3;
        role = k < per ? x + 8 * k : P + (x + 8 * ((k - per) / R)) * R + (k - per) % R;
    }
    if (xcc && lane == 0) xcc[role] = __builtin_amdgcn_s_getreg((3 << 11) | 20) & 15u;   // XCC_ID
    if (role < P) {
        const int p = role;
        int c = 0;
        if (p < n_active_producers) {
            for (; c < n_chunks; ++c) {
                const int slot = c % S;
                if (c >= S &&
                    !wait_at_least(done + p * S + slot, (uint32_t)(R * (c / S)), abort_word,
                                   1u + (uint32_t)role, spin_limit, deadline, mode))
                    break;
                uint4 *rec = ring + ((size_t)p * S + slot) * rec_vec;
                for (int v = lane; v < rec_vec; v += 64) {
                    const uint32_t i = 4u * (uint32_t)v;
                    rec[v] = make_uint4(pattern(p, c, i), pattern(p, c, i + 1), pattern(p, c, i + 2),
                                        pattern(p, c, i + 3));
                }
                // Every lane publishes its own stores (same word, same value).
                publish(ready + p * S + slot, (uint32_t)(c + 1), mode);
            }
        }
        if (lane == 0) progress[role] = (uint32_t)c;
        return;
    }
    const int q = role - P, p = q / R;
    uint32_t bad = 0;
    int c = 0;
    for (; c < n_chunks; ++c) {
        const int slot = c % S;
        if (!wait_at_least(ready + p * S + slot, (uint32_t)(c + 1), abort_word, 1u + (uint32_t)role,
                           spin_limit, deadline, mode))
            break;
        const uint4 *rec = ring + ((size_t)p * S + slot) * rec_vec;
        // One XCD: the record's lines may still sit in this CU's vector L1
        // from the slot's previous use, so read them with loads that miss it
        // (device scope, sc1), through a buffer resource sized to the record.
        __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint4 *>(rec), 0, rec_vec * 16, 0x00020000);
        for (int v = lane; v < rec_vec; v += 64) {
            uint4 x;
            if (mode == Poll::OneL2) {
                const auto y = __builtin_amdgcn_raw_buffer_load_b128(rs, v * 16, 0, 16);
                x = make_uint4(y[0], y[1], y[2], y[3]);
            } else {
                x = rec[v];
            }
            const uint32_t i = 4u * (uint32_t)v;
            bad += (x.x != pattern(p, c, i)) + (x.y != pattern(p, c, i + 1)) +
                   (x.z != pattern(p, c, i + 2)) + (x.w != pattern(p, c, i + 3));
        }
        // All lanes' reads come before the count the producer waits for: the
        // barrier orders them within the workgroup (each read's value has been
        // compared, so it has returned), lane 0's store of the count beyond it.
        __syncthreads();
        if (lane == 0) {
            if (mode == Poll::OneL2)
                __hip_atomic_fetch_add(done + p * S + slot, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else
                __hip_atomic_fetch_add(done + p * S + slot, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (bad) atomicAdd(bad_words, bad);
    if (lane == 0) progress[role] = (uint32_t)c;
}

}  // namespace

// Launches the probe on `stream`.  Device buffers (all caller-owned):
//   ring        P * S * rec_bytes bytes (rec_bytes a multiple of 16)
//   ready, done P * S words each, zeroed by the caller
//   abort_word  1 word, zeroed; afterwards 0, or 1 + the role index of the
//               first wait that ran out of polls
//   bad_words   1 word, zeroed; afterwards the number of record words that
//               did not match
//   progress    P * (1 + R) words: the chunks each role completed (producer of
//               stream p at p, consumer r of stream p at P + p R + r)
//   xcc         P * (1 + R) words, or null: the XCD each role ran on
// Every wait gives up after `spin_limit` polls, and every workgroup after
// `max_seconds` (0 < max_seconds <= 10) of wall-clock time from its start.
// poll_mode 0: every poll is an acquire load; 1: relaxed polls and one acquire
// fence after the poll that succeeds; 2: each stream on one XCD, handed over
// through its L2 (P a multiple of 8).
// Returns 0, or -1 for arguments outside these bounds, or a HIP error code.
extern "C" int ring_probe_launch(void *ring, uint32_t *ready, uint32_t *done, uint32_t *abort_word,
                                 uint32_t *bad_words, uint32_t *progress, uint32_t *xcc, int P, int R,
                                 int S, int n_chunks, int rec_bytes, int n_active_producers,
                                 uint32_t spin_limit, double max_seconds, int poll_mode,
                                 hipStream_t stream) {
    if (!ring || !ready || !done || !abort_word || !bad_words || !progress) return -1;
    if (P < 1 || P > 256 || R < 1 || R > 16 || S < 1 || S > 64 || n_chunks < 0 ||
        n_chunks > (1 << 20) || rec_bytes < 16 || rec_bytes % 16 || rec_bytes > (1 << 20) ||
        n_active_producers < 0 || n_active_producers > P || !(max_seconds > 0.0) ||
        max_seconds > 10.0 || poll_mode < 0 || poll_mode > 2 || (poll_mode == 2 && P % 8 != 0))
        return -1;
    int dev = 0, khz = 0;
    hipError_t e;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return (int)e;
    if ((e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev)) != hipSuccess)
        return (int)e;
    if (khz <= 0) return -1;
    const uint64_t max_ticks = (uint64_t)(max_seconds * 1000.0 * (double)khz);
    hipLaunchKernelGGL(ring_probe_kernel, dim3(P * (1 + R)), dim3(64), 0, stream,
                       static_cast<uint4 *>(ring), ready, done, abort_word, bad_words, progress, xcc, P,
                       R, S, n_chunks, rec_bytes / 16, n_active_producers, spin_limit, max_ticks,
                       poll_mode);
    return (int)hipGetLastError();
}
