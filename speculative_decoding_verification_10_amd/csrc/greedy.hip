// Greedy verify step on gfx950 ("3.5 Speculative Decoding", section "Proof
// that the output distribution is exactly p", greedy remark, and "Worked
// example"; "Speculative Decoding from First Principles", "Draft, verify,
// keep what matches"): keep a draft iff it equals the target argmax, emit the
// target argmax at the first mismatch, or the argmax after the last draft
// when every draft matches.  No exponentials: one pass over the target rows.
//
//  1. greedy_partial  one workgroup per (target row i <= k_b, tile): the
//                     tile's (max, lowest index of the max).
//  2. greedy_decide   one wave per request: merges the tiles of each row in
//                     ascending order (the first tile holding the max wins,
//                     so ties resolve to the lowest id), compares with the
//                     drafts with a ballot and writes the outputs.
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

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void greedy_partial(GreedyParams a) {
    constexpr int E = Elem<DT>::E;
    constexpr int S = Elem<DT>::S;
    __shared__ float lv[kWaves];
    __shared__ int li[kWaves];
    const int tile = blockIdx.x;
    const int i = blockIdx.y;
    const int b = blockIdx.z;
    const size_t rid = (size_t)b * (a.K + 1) + i;
    const size_t item = rid * a.C + tile;
    if (i > greedy_k(a, b)) return;
    const void* row = static_cast<const char*>(a.target) + (size_t)rid * a.V * S;
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
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) { lv[w] = bv; li[w] = bi; }
    __syncthreads();
    if (threadIdx.x == 0) {
        float rv = lv[0];
        int ri = li[0];
        for (int k = 1; k < kWaves; ++k)
            if (better(lv[k], li[k], rv, ri)) { rv = lv[k]; ri = li[k]; }
        a.part_v[item] = rv;
        a.part_i[item] = ri;
    }
}

__global__ __launch_bounds__(64) void greedy_decide(GreedyParams a) {
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const int K = a.K;
    const int kb = greedy_k(a, b);
    int j = kb;
    int aj = 0;
    for (int base = 0; base <= kb; base += 64) {
        const int i = base + lane;
        int am = -1;
        bool miss = false;
        if (i <= kb) {
            const size_t rid = (size_t)b * (K + 1) + i;
            float bv = a.part_v[rid * a.C];
            int bi = a.part_i[rid * a.C];
            for (int t = 1; t < a.C; ++t) {
                const float v = a.part_v[rid * a.C + t];
                if (v > bv) { bv = v; bi = a.part_i[rid * a.C + t]; }
            }
            am = min(bi, a.V - 1);
            if (a.amax) a.amax[rid] = am;
            if (i < kb) miss = (a.tokens[(size_t)b * K + i] != am);
        }
        const unsigned long long mask = __ballot(miss);
        if (j == kb) {
            if (mask) j = base + __ffsll((long long)mask) - 1;
            if (j - base >= 0 && j - base < 64) aj = __shfl(am, j - base, 64);
        }
    }
    for (int i = lane; i <= K; i += 64) {
        int32_t v = -1;
        if (i < j) v = a.tokens[(size_t)b * K + i];
        else if (i == j) v = aj;
        a.out[(size_t)b * (K + 1) + i] = v;
        if (a.amax && i > kb) a.amax[(size_t)b * (K + 1) + i] = -1;
    }
    if (lane == 0) a.nacc[b] = j;
}

template <int DT, bool VEC>
hipError_t launch(const GreedyParams& p, hipStream_t s) {
    if (p.B == 0) return hipSuccess;
    // Workgroup (x, y, z): tile x of row y of request z.
    hipLaunchKernelGGL((greedy_partial<DT, VEC>), dim3(p.C, p.K + 1, p.B), dim3(kThreads), 0, s, p);
    hipLaunchKernelGGL(greedy_decide, dim3((unsigned)p.B), dim3(64), 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_greedy(const GreedyParams& p, int dtype, bool vec, hipStream_t s) {
    if (dtype == kBF16) return vec ? launch<kBF16, true>(p, s) : launch<kBF16, false>(p, s);
    return vec ? launch<kFP32, true>(p, s) : launch<kFP32, false>(p, s);
}

}  // namespace specdec
