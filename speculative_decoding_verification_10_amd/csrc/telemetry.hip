// Acceptance telemetry on gfx950: per drafted position i, over the requests
// of one verify step, the number that drafted i (i < k_b), tested it (i < k_b
// and every earlier draft accepted, i <= n_b) and accepted it (i < n_b) --
// the serving engine's drafted / accepted counters, per position
// ("Speculative Decoding from First Principles", "What the numbers say"),
// and the tests performed ("246 Speculative Decoding", 3.4).
//
// Each count is a suffix sum of a histogram: drafted_i = #{k_b > i},
// tested_i = #{min(k_b, n_b + 1) > i}, accepted_i = #{n_b > i}.  A
// workgroup takes 256 requests, builds the three histograms over 0..K in
// LDS, turns them into per-position counts and adds those to the caller's
// 64-bit counters with atomic adds (one per position and counter).
#include "internal.h"

namespace specdec {
namespace {

__global__ __launch_bounds__(kThreads) void acceptance_counts(TelemetryParams a) {
    __shared__ uint32_t hist[3][kMaxK + 2];
    const int K = a.K;
    for (int v = threadIdx.x; v < 3 * (kMaxK + 2); v += kThreads) (&hist[0][0])[v] = 0;
    __syncthreads();
    const int b = blockIdx.x * kThreads + threadIdx.x;
    if (b < a.B) {
        // Values outside [0, K] (a broken precondition) are clamped, never
        // used to address memory.
        const int k = a.kpr ? min(max(a.kpr[b], 0), K) : K;
        const int n = min(max(a.nacc[b], 0), k);
        atomicAdd(&hist[0][k], 1u);
        atomicAdd(&hist[1][min(k, n + 1)], 1u);
        atomicAdd(&hist[2][n], 1u);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < K; i += kThreads) {
        uint32_t c[3] = {0, 0, 0};
        for (int v = i + 1; v <= K; ++v)
#pragma unroll
            for (int r = 0; r < 3; ++r) c[r] += hist[r][v];
#pragma unroll
        for (int r = 0; r < 3; ++r)
            if (c[r]) atomicAdd(reinterpret_cast<unsigned long long*>(a.counters + (size_t)r * K + i),
                                (unsigned long long)c[r]);
    }
}

}  // namespace

hipError_t launch_acceptance_counts(const TelemetryParams& p, hipStream_t s) {
    if (p.B == 0 || p.K == 0) return hipSuccess;
    hipLaunchKernelGGL(acceptance_counts, dim3((p.B + kThreads - 1) / kThreads), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace specdec
