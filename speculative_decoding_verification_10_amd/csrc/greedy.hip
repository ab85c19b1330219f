// Greedy verify step on gfx950 ("3.5 Speculative Decoding", section "Proof
// that the output distribution is exactly p", greedy remark, and "Worked
// example"; "Speculative Decoding from First Principles", "Draft, verify,
// keep what matches"): keep a draft iff it equals the target argmax, emit the
// target argmax at the first mismatch, or the argmax after the last draft
// when every draft matches.  No exponentials: one pass over the target rows.
//
// One kernel, one workgroup per (target row i <= k_b, tile): the tile's
// (max, lowest index of the max) goes to a self-validating slot.  The first
// wave of the request's last workgroup -- last tile of row k_b, the highest
// index of the request's workgroups -- waits for the other slots of its
// request (lower indices, dispatched no later, and they never wait), merges
// each row's tiles, compares the argmaxes with the drafts with a ballot,
// writes the outputs and zeroes the slots for the next call.
#include <hip/hip_ext.h>

#include "internal.h"
#include "slots.h"

namespace specdec {
namespace {

__device__ __forceinline__ int greedy_k(const GreedyParams& a, int b) {
    return a.kpr ? min(max(a.kpr[b], 0), a.K) : a.K;
}

// (value, index) order: larger value first, lower index on equal values.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
    return (v > bv) || (v == bv && i < bi);
}

// A (value, index) pair as one self-validating word: never all ones, since
// NaN values are stored canonically and indices are below 2^31.
__device__ __forceinline__ uint64_t enc_pair(float v, int i) {
    const uint32_t vb = (v != v) ? 0x7FC00000u : __float_as_uint(v);
    return ~(((uint64_t)vb << 32) | (uint32_t)i);
}
__device__ __forceinline__ void dec_pair(uint64_t s, float& v, int& i) {
    const uint64_t w = ~s;
    v = __uint_as_float((uint32_t)(w >> 32));
    i = (int)(uint32_t)w;
}

// One DPP step of a (value, index) reduction: the pair a DPP move brings in
// replaces this lane's if it is better (lanes the move skips see the
// identity (-inf, INT_MAX)).
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ void best_step(float& v, int& i) {
    const float ov = dpp<CTRL, ROWS>(v, -INFINITY);
    const int oi = dpp<CTRL, ROWS>(i, 0x7FFFFFFF);
    if (better(ov, oi, v, i)) {
        v = ov;
        i = oi;
    }
}

// Best pair over each row of 16 lanes, in every lane of the row.
__device__ __forceinline__ void row16_best(float& v, int& i) {
    best_step<kDppQuad1032>(v, i);
    best_step<kDppQuad2301>(v, i);
    best_step<kDppRowHalfMirror>(v, i);
    best_step<kDppRowMirror>(v, i);
}

// Best pair over the wave, in lane 63.
__device__ __forceinline__ void wave_best(float& v, int& i) {
    row16_best(v, i);
    best_step<kDppRowBcast15, 0xA>(v, i);
    best_step<kDppRowBcast31, 0xC>(v, i);
}

struct GreedyShared {
    float lv[kWaves];
    int li[kWaves];
    int am[kMaxK + 1];
};

// The request's decision, by one wave of its last workgroup (the other waves
// have left, so a waiting decider holds one wave slot, not four).
__device__ void greedy_decide(const GreedyParams& a, int b, int kb, GreedyShared& sh) {
    const int K = a.K, C = a.C;
    const int lane = threadIdx.x & 63, sub = lane & 15;
    uint64_t* slots = a.slot + (size_t)b * (K + 1) * C;
    // Rows 16 lanes at a time, four rows per pass.
    for (int base = 0; base <= kb; base += 4) {
        const int r = base + (lane >> 4);
        float bv = -INFINITY;
        int bi = 0x7FFFFFFF;
        if (r <= kb) {
            for (int c = sub; c < C; c += 16) {
                const uint64_t* p = slots + (size_t)r * C + c;
                float v;
                int i;
                dec_pair(slot_wait(p, a.err, enc_pair(-INFINITY, 0)), v, i);
                if (better(v, i, bv, bi)) { bv = v; bi = i; }
            }
        }
        row16_best(bv, bi);
        if (sub == 0 && r <= kb) sh.am[r] = min(max(bi, 0), a.V - 1);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // First mismatch, 64 positions at a time.
    int j = kb;
    for (int t0 = 0; t0 < kb; t0 += 64) {
        const int t = t0 + lane;
        const unsigned long long m = __ballot(t < kb && a.tokens[(size_t)b * K + t] != sh.am[t]);
        if (m) {
            j = t0 + __ffsll((long long)m) - 1;
            break;
        }
    }
    for (int i = lane; i <= K; i += 64) {
        int32_t v = -1;
        if (i < j) v = a.tokens[(size_t)b * K + i];
        else if (i == j) v = sh.am[j];
        a.out[(size_t)b * (K + 1) + i] = v;
        if (a.amax) a.amax[(size_t)b * (K + 1) + i] = (i <= kb) ? sh.am[i] : -1;
    }
    if (lane == 0) a.nacc[b] = j;
    // Every slot of the request was awaited above, by this wave.
    for (int s = lane; s < (kb + 1) * C; s += 64) slot_put(slots + s, (uint64_t)0);
}

// Workgroup (x, y, z): tile x of target row y of request z.
template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void greedy_rows(GreedyParams a) {
    constexpr int E = Elem<DT>::E;
    constexpr int S = Elem<DT>::S;
    __shared__ GreedyShared sh;
    const int tile = blockIdx.x;
    const int i = blockIdx.y;
    const int b = blockIdx.z;
    const int kb = greedy_k(a, b);
    if (i > kb) return;
    const size_t rid = (size_t)b * (a.K + 1) + i;
    const void* row = static_cast<const char*>(a.target) + rid * a.V * S;
    const int v0 = tile * kTileVec + threadIdx.x;
    u32x4 raw[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) raw[u] = load_raw<DT, VEC, true>(row, a.V, a.NV, v0 + u * kThreads);
    // The thread's elements in ascending id; strict ">" keeps the first max.
    float bv;
    int bi;
    {
        float x[E];
        decode<DT>(raw[0], x);
        bv = x[0];
        bi = v0 * E;
#pragma unroll
        for (int e = 1; e < E; ++e)
            if (x[e] > bv) { bv = x[e]; bi = v0 * E + e; }
    }
#pragma unroll
    for (int u = 1; u < kUnroll; ++u) {
        float x[E];
        decode<DT>(raw[u], x);
        const int t0 = (v0 + u * kThreads) * E;
#pragma unroll
        for (int e = 0; e < E; ++e)
            if (x[e] > bv) { bv = x[e]; bi = t0 + e; }
    }
    wave_best(bv, bi);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 63) { sh.lv[w] = bv; sh.li[w] = bi; }
    __syncthreads();
    if (threadIdx.x == 0) {
        float rv = sh.lv[0];
        int ri = sh.li[0];
        for (int k = 1; k < kWaves; ++k)
            if (better(sh.lv[k], sh.li[k], rv, ri)) { rv = sh.lv[k]; ri = sh.li[k]; }
        slot_put(a.slot + rid * a.C + tile, enc_pair(rv, ri));
    }
    if (i == kb && tile == a.C - 1 && threadIdx.x < 64) greedy_decide(a, b, kb, sh);
}

template <int DT, bool VEC>
hipError_t launch(const GreedyParams& p, hipStream_t s, hipEvent_t const* events) {
    if (p.B == 0) return hipSuccess;
    hipExtLaunchKernelGGL((greedy_rows<DT, VEC>), dim3(p.C, p.K + 1, p.B), dim3(kThreads), 0, s,
                          events ? events[0] : nullptr, events ? events[1] : nullptr, 0, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_greedy(const GreedyParams& p, int dtype, bool vec, hipStream_t s,
                         hipEvent_t const* events) {
    if (dtype == kBF16) return vec ? launch<kBF16, true>(p, s, events) : launch<kBF16, false>(p, s, events);
    return vec ? launch<kFP32, true>(p, s, events) : launch<kFP32, false>(p, s, events);
}

}  // namespace specdec
