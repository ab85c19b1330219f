// Self-validating slots: how workgroups of one kernel hand results to other
// workgroups on gfx950 without release fences.
//
// A slot holds a value stored bit-inverted, so an all-zero slot means "not
// written yet".  NaNs are stored as the canonical quiet NaN, so the inverted
// bits of a stored float or double are never all zero.  Producers write a
// slot once with a relaxed agent-scope atomic store; consumers poll it with
// relaxed agent-scope atomic loads until it is non-zero.  Each datum
// validates itself, so no ordering between different slots is needed: an
// agent-scope release (an L2 writeback on this multi-XCD part) per workgroup
// would cost far more than the work.
//
// Waiting is safe because a consumer only waits for workgroups with a lower
// index in the same grid: the hardware dispatches those no later than the
// consumer, and they never wait themselves, so they finish.  A poll gives up
// only after kWaitTicks (far beyond any legitimate wait) have passed AND one
// more read still finds the slot empty; it then raises an error bit in the
// workspace header, tells its caller (which marks the affected outputs
// invalid) and continues with a harmless value, so every wave always exits.
//
// A slot must read zero before its producer runs: an earlier kernel of the
// same call empties it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace specdec {

// A wait gives up after 50 ms of wall-clock time (100 MHz counter), far
// beyond any legitimate wait (the library's default; tests of the error
// path set a shorter limit through specdec_debug_bounded_wait).
constexpr uint64_t kWaitTicks = 5000000;

__device__ __forceinline__ uint32_t enc_f32(float f) {
    return ~(f != f ? 0x7FC00000u : __float_as_uint(f));
}
__device__ __forceinline__ float dec_f32(uint32_t u) { return __uint_as_float(~u); }
__device__ __forceinline__ uint64_t enc_f64(double d) {
    return ~(d != d ? 0x7FF8000000000000ull : (uint64_t)__double_as_longlong(d));
}
__device__ __forceinline__ double dec_f64(uint64_t u) { return __longlong_as_double((long long)~u); }

// Two floats in one self-validating 64-bit slot: each half is enc_f32 of its
// value, so the word is never zero once written.
__device__ __forceinline__ uint64_t enc_f32x2(float hi, float lo) {
    return ((uint64_t)enc_f32(hi) << 32) | (uint64_t)enc_f32(lo);
}
__device__ __forceinline__ float dec_hi(uint64_t u) { return dec_f32((uint32_t)(u >> 32)); }
__device__ __forceinline__ float dec_lo(uint64_t u) { return dec_f32((uint32_t)u); }

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

// Finish a poll that began with a value v already loaded from p: poll until
// the slot is written.  The deadline is checked only after a read that still
// found the slot empty, so a wave that was descheduled past the deadline
// reads once more before it gives up.  On giving up: flag the error word, set
// `lost` and return `fallback`.
template <typename T>
__device__ __forceinline__ T settle(const T* p, T v, uint32_t* err, T fallback, bool& lost,
                                   uint64_t ticks = kWaitTicks) {
    if (v != 0) return v;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    for (;;) {
        __builtin_amdgcn_s_sleep(2);
        v = slot_peek(p);
        if (v != 0) return v;
        if (__builtin_amdgcn_s_memrealtime() - t0 > ticks) {
            atomicOr(err, 1u);
            lost = true;
            return fallback;
        }
    }
}

template <typename T>
__device__ __forceinline__ T slot_wait(const T* p, uint32_t* err, T fallback, bool& lost,
                                      uint64_t ticks = kWaitTicks) {
    return settle(p, slot_peek(p), err, fallback, lost, ticks);
}

}  // namespace specdec
