// Greedy verify step on gfx950 ("3.5 Speculative Decoding", section "Proof
// that the output distribution is exactly p", greedy remark, and "Worked
// example"; "Speculative Decoding from First Principles", "Draft, verify,
// keep what matches"): keep a draft iff it equals the target argmax, emit the
// target argmax at the first mismatch, or the argmax after the last draft
// when every draft matches.  No exponentials: one pass over the target rows.
//
// Two stream-ordered kernels, no waits inside either:
//  greedy_rows       one workgroup per (target row i <= k_b, tile): the
//                    tile's (max, lowest index of the max), one word per tile;
//  greedy_decisions  one wave per request: merges each row's tiles, compares
//                    the argmaxes with the drafts by ballot, writes the
//                    outputs.
#include <hip/hip_ext.h>

#include "internal.h"

namespace specdec {
namespace {

__device__ __forceinline__ int greedy_k(const GreedyParams& a, int b) {
    return a.kpr ? min(max(a.kpr[b], 0), a.K) : a.K;
}

// (value, index) order: larger value first, lower index on equal values.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
    return (v > bv) || (v == bv && i < bi);
}

// A (value, index) pair as one 8-byte word.
__device__ __forceinline__ uint64_t enc_pair(float v, int i) {
    return ((uint64_t)__float_as_uint(v) << 32) | (uint32_t)i;
}
__device__ __forceinline__ void dec_pair(uint64_t w, float& v, int& i) {
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

// The decision of request b, by one wave (its own workgroup): the row
// maxima come from the tile slots the previous kernel wrote.
__device__ void greedy_decide(const GreedyParams& a, int b, int* am) {
    const int K = a.K, C = a.C;
    const int kb = greedy_k(a, b);
    const int lane = threadIdx.x & 63, sub = lane & 15;
    const uint64_t* slots = a.slot + (size_t)b * (K + 1) * C;
    // Rows 16 lanes at a time, four rows per pass; every load of a pass is
    // issued before any is used.
    for (int base = 0; base <= kb; base += 4) {
        const int r = base + (lane >> 4);
        float bv = -INFINITY;
        int bi = 0x7FFFFFFF;
        if (r <= kb) {
            for (int c0 = sub; c0 < C; c0 += 64) {
                uint64_t got[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c = c0 + 16 * q;
                    got[q] = (c < C) ? slots[(size_t)r * C + c] : 0;
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (c0 + 16 * q >= C) break;
                    float v;
                    int i;
                    dec_pair(got[q], v, i);
                    if (better(v, i, bv, bi)) { bv = v; bi = i; }
                }
            }
        }
        row16_best(bv, bi);
        if (sub == 0 && r <= kb) am[r] = min(max(bi, 0), a.V - 1);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // First mismatch, 64 positions at a time.
    int j = kb;
    for (int t0 = 0; t0 < kb; t0 += 64) {
        const int t = t0 + lane;
        const unsigned long long m = __ballot(t < kb && a.tokens[(size_t)b * K + t] != am[t]);
        if (m) {
            j = t0 + __ffsll((long long)m) - 1;
            break;
        }
    }
    for (int i = lane; i <= K; i += 64) {
        int32_t v = -1;
        if (i < j) v = a.tokens[(size_t)b * K + i];
        else if (i == j) v = am[j];
        a.out[(size_t)b * (K + 1) + i] = v;
        if (a.amax) a.amax[(size_t)b * (K + 1) + i] = (i <= kb) ? am[i] : -1;
    }
    if (lane == 0) a.nacc[b] = j;
}

// Workgroup (x, y, z): tile x of target row y of request z.
template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void greedy_rows(GreedyParams a) {
    constexpr int E = Elem<DT>::E;
    constexpr int S = Elem<DT>::S;
    __shared__ float lv[kWaves];
    __shared__ int li[kWaves];
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
    if ((threadIdx.x & 63) == 63) { lv[w] = bv; li[w] = bi; }
    __syncthreads();
    if (threadIdx.x == 0) {
        float rv = lv[0];
        int ri = li[0];
        for (int k = 1; k < kWaves; ++k)
            if (better(lv[k], li[k], rv, ri)) { rv = lv[k]; ri = li[k]; }
        a.slot[rid * a.C + tile] = enc_pair(rv, ri);
    }
}

// Decisions: workgroup x (one wave) takes request x.
__global__ __launch_bounds__(64) void greedy_decisions(GreedyParams a) {
    __shared__ int am[kMaxK + 1];
    greedy_decide(a, blockIdx.x, am);
}

template <int DT, bool VEC>
hipError_t launch(const GreedyParams& p, hipStream_t s, hipEvent_t const* events) {
    if (p.B == 0) return hipSuccess;
    hipExtLaunchKernelGGL((greedy_rows<DT, VEC>), dim3(p.C, p.K + 1, p.B), dim3(kThreads), 0, s,
                          events ? events[0] : nullptr, events ? events[1] : nullptr, 0, p);
    hipExtLaunchKernelGGL(greedy_decisions, dim3(p.B), dim3(64), 0, s, nullptr,
                          events ? events[2] : nullptr, 0, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_greedy(const GreedyParams& p, int dtype, bool vec, hipStream_t s,
                         hipEvent_t const* events) {
    if (dtype == kBF16) return vec ? launch<kBF16, true>(p, s, events) : launch<kBF16, false>(p, s, events);
    return vec ? launch<kFP32, true>(p, s, events) : launch<kFP32, false>(p, s, events);
}

}  // namespace specdec
