// Self-validating slots: how workgroups of one kernel hand results to later
// workgroups of the same kernel on gfx950 without release fences.
//
// A slot holds a value stored bit-inverted, so an all-zero slot means "not
// written yet" (the inverted bits of any non-NaN float or double are never
// all zero).  Producers write a slot once with a relaxed agent-scope atomic
// store; consumers poll it with relaxed agent-scope atomic loads until it is
// non-zero.  Each datum validates itself, so no ordering between different
// slots is needed: an agent-scope release (an L2 writeback on this
// multi-XCD part) per workgroup would cost far more than the work.
//
// Waiting is safe because a consumer only waits for workgroups with a lower
// index in the same grid: those were dispatched before it, never wait for it,
// and therefore finish.  A poll gives up after kSpinLimit rounds (far beyond
// any legitimate wait), raises an error bit in the workspace header and
// continues with a harmless value, so every wave always exits.
//
// The last consumer of a slot writes zero back, so the workspace is all zero
// again when the kernel ends and ready for the next call.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace specdec {

constexpr int kSpinLimit = 1 << 20;

__device__ __forceinline__ uint32_t enc_f32(float f) { return ~__float_as_uint(f); }
__device__ __forceinline__ float dec_f32(uint32_t u) { return __uint_as_float(~u); }
__device__ __forceinline__ uint64_t enc_f64(double d) { return ~(uint64_t)__double_as_longlong(d); }
__device__ __forceinline__ double dec_f64(uint64_t u) { return __longlong_as_double((long long)~u); }

__device__ __forceinline__ void slot_put(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void slot_put(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t slot_peek(const uint32_t* p) {
    return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t slot_peek(const uint64_t* p) {
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void count_up(uint32_t* p) {
    __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Sleep between polls: about 1000 cycles, so that waiting workgroups put
// almost no load on the memory system while others stream.
__device__ __forceinline__ void poll_pause() { __builtin_amdgcn_s_sleep(16); }

// Poll a counter until it reaches `target` (relaxed loads; one lane).
// Returns false on time-out (after flagging the error).
__device__ __forceinline__ bool wait_count(const uint32_t* p, uint32_t target, uint32_t* err) {
    int n = 0;
    while (slot_peek(p) < target) {
        if (++n > kSpinLimit) {
            atomicOr(err, 2u);
            return false;
        }
        poll_pause();
    }
    return true;
}

// Poll until the slot is written; on time-out flag the error and return
// `fallback`.
template <typename T>
__device__ __forceinline__ T slot_wait(const T* p, uint32_t* err, T fallback) {
    T v = slot_peek(p);
    int n = 0;
    while (v == 0) {
        if (++n > kSpinLimit) {
            atomicOr(err, 1u);
            return fallback;
        }
        __builtin_amdgcn_s_sleep(2);
        v = slot_peek(p);
    }
    return v;
}

}  // namespace specdec
