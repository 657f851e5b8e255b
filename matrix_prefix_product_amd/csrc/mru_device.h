// Device-side helpers shared by the MRU scan kernels (gfx950, wave64).
//
// Multi-chunk scans run in one launch.  A sequence of T tokens is cut into
// chunks of K tokens, and consecutive chunks are grouped into "supers" of Z
// chunks.  Each chunk is owned by one chain (a group of lanes, or a whole wave
// for the matrix-core kernels), which
//   1. computes its chunk aggregate (the product of its matrices, or the affine
//      map of the backward recurrence) and publishes it with flag AGG;
//   2. composes the aggregates of the earlier chunks of its super, in a fixed
//      left-to-right order, waiting for their AGG flags;
//   3. if the super is not its sequence's first, waits for the PREFIX flag of
//      the previous super's last chunk and applies that prefix; the super's
//      last chunk then publishes its own inclusive prefix with flag PREFIX;
//   4. re-runs its chunk from the resulting carry and writes the outputs.
// Every product is taken in an order fixed by (K, Z) alone, so results are
// bitwise reproducible run to run; a chunk waits on at most Z-1 aggregates
// and the serial part is one hop per super.  Chains take their chunk from a
// ticket counter (not blockIdx), so a chain only waits on chunks whose owners
// are already running, and every wait ends.  Associativity of the matrix
// product is what makes the regrouping legal ("MRU Update: ...", section
// "What MRU Actually Does").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mru {

constexpr int kNoExp = INT32_MIN;  // max_exp of an all-zero set

constexpr uint32_t kFlagEmpty = 0;
constexpr uint32_t kFlagAgg = 1;
constexpr uint32_t kFlagPrefix = 2;

// Status bits left in the workspace header by a kernel.
constexpr uint32_t kStatusSpinTimeout = 1;

// Upper bound on polls of one flag.  With ticket ordering every poll loop ends;
// the bound only turns a logic error into a recorded status instead of a hang.
constexpr uint32_t kSpinLimit = 1u << 21;

// Workspace layout (all offsets 256-byte aligned):
//   [0, 256)          header: ticket counter, status word
//   flags             uint32[nchunks]
//   slot 0 .. slot k  nchunks * n * n elements of the chain's accumulator type
//   exponents         int32[nslots][nchunks]: power-of-two exponents of the
//                     slots' matrices (used by the scaled forward scan only)
struct WsHeader {
    uint32_t ticket;
    uint32_t status;
    uint32_t pad[62];
};

__host__ __device__ constexpr size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct WsLayout {
    size_t flags_off;
    size_t slot_off[3];
    size_t exp_off;
    size_t total;
};

__host__ __device__ inline WsLayout ws_layout(int64_t nchunks, int n, int elem_bytes, int nslots) {
    WsLayout L{};
    size_t off = align256(sizeof(WsHeader));
    L.flags_off = off;
    off = align256(off + size_t(nchunks) * sizeof(uint32_t));
    for (int i = 0; i < 3; ++i) {
        L.slot_off[i] = off;
        if (i < nslots) off = align256(off + size_t(nchunks) * size_t(n) * n * elem_bytes);
    }
    L.exp_off = off;
    off = align256(off + size_t(nchunks) * size_t(nslots) * sizeof(int32_t));
    L.total = off;
    return L;
}

__device__ inline uint32_t load_flag(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline void store_flag(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Publishing protocol of the look-back workspace: every published matrix entry
// and every flag is written and read with agent-scope atomic accesses, which
// the compiler makes coherent across all XCDs of the device (they bypass the
// per-XCD L2 for this data).  A writer waits for its data stores to complete
// (vmcnt 0) before it stores the flag; a reader only issues its data loads
// after it has seen the flag.  No cache-wide write-back or invalidate is
// needed, so other waves' streaming traffic through L2 is not disturbed.
template <class T>
__device__ inline void ws_store(T* p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <class T>
__device__ inline T ws_load(const T* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Between a writer's data stores and its flag store.
__device__ inline void fence_release() { __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Between a reader's flag loads and its data loads (the data loads are issued
// only after the flag value is known; this keeps the compiler from hoisting them).
__device__ inline void fence_acquire() { __asm__ volatile("" ::: "memory"); }

// Ticket order of a multi-chunk scan: ticket t takes chunk group t / S of
// sequence t % S, i.e. sequences are interleaved.  Chunks that run at the same
// time then come from many sequences, and every chunk's predecessors were handed
// out at least S tickets earlier, which keeps the carry chains short.  A chunk
// only ever waits on earlier chunks of its own sequence, which have smaller
// tickets.  Returns the first chunk index of the group (groups of G chunks);
// t must be below S * groups_per_seq (larger tickets map back into range).
__device__ inline int64_t ticket_to_chunk(int64_t t, int64_t S, int64_t groups_per_seq, int G) {
    const int64_t s = t % S;
    return (s * groups_per_seq + t / S) * G;
}

// One ticket per wave, taken by lane 0 and broadcast.
__device__ inline uint32_t wave_ticket(uint32_t* counter) {
    uint32_t t = 0;
    if ((threadIdx.x & 63) == 0) t = atomicAdd(counter, 1u);
    return __builtin_amdgcn_readfirstlane(t);
}

// Wave-uniform wait until *flag == want.  Must be reached by the whole wave.
// Records a timeout in the header instead of hanging.
__device__ inline void wait_flag_eq(const uint32_t* flag, uint32_t want, WsHeader* hdr) {
    uint32_t polls = 0;
    for (;;) {
        const uint32_t f = __builtin_amdgcn_readfirstlane(load_flag(flag));
        if (f == want) return;
        if (++polls >= kSpinLimit) {
            if ((threadIdx.x & 63) == 0) atomicOr(&hdr->status, kStatusSpinTimeout);
            return;
        }
        __builtin_amdgcn_s_sleep(2);
    }
}

// Wave-cooperative wait until every flag in [lo, hi) is non-empty; lane i polls
// flags lo+i, lo+i+64, ...  Must be reached by the whole wave.
__device__ inline void wait_range_nonempty(const uint32_t* flags, int64_t lo, int64_t hi,
                                           WsHeader* hdr) {
    const int lane = threadIdx.x & 63;
    for (int64_t base = lo; base < hi; base += 64) {
        const int64_t j = base + lane;
        uint32_t polls = 0;
        for (;;) {
            const bool ok = j >= hi || load_flag(&flags[j]) != kFlagEmpty;
            if (__all(ok)) break;
            if (++polls >= kSpinLimit) {
                if (lane == 0) atomicOr(&hdr->status, kStatusSpinTimeout);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
}

// Orders a one-wave workgroup's LDS staging: the scan kernels run one wave per
// workgroup, so no workgroup barrier is needed, but the wave waits until its
// own LDS operations have completed (s_waitcnt lgkmcnt(0)) before the accesses
// that follow.  Without that wait (the fence alone, relying on a wave's LDS
// instructions taking effect in issue order) the n = 16 layer backward to dx
// read stale staged data at every other token in some builds of identical
// machine code placed differently in the library, while the wait makes every
// build correct.  The wavefront-scope fence keeps the compiler from moving LDS
// accesses across it.
__device__ inline void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
}

// frexp exponent: a finite nonzero v with exponent e has 2^(e-1) <= |v| < 2^e.
// max_exp folds the exponent of a nonzero v into a running maximum that starts
// at kNoExp (so an all-zero set keeps kNoExp).
__device__ inline int frexp_exp(float v) { return __builtin_amdgcn_frexp_expf(v); }
__device__ inline int frexp_exp(double v) { return __builtin_amdgcn_frexp_exp(v); }

template <class T>
__device__ inline int max_exp(int e, T v) {
    return v != T(0) ? max(e, frexp_exp(v)) : e;
}

// Maximum of e over groups of W consecutive lanes (W a power of two <= 64).
template <int W>
__device__ inline int group_max(int e) {
#pragma unroll
    for (int m = 1; m < W; m <<= 1) e = max(e, __shfl_xor(e, m, 64));
    return e;
}

// Kernel that clears the workspace header and flags before a multi-chunk scan.
__global__ void ws_reset_kernel(uint32_t* words, int64_t nwords);

}  // namespace mru
