// n-gram (prompt-lookup) drafter on gfx950: find the last few tokens earlier
// in the context and propose what followed them there ("3.5 Speculative
// Decoding", "Choosing a draft", n-gram / prompt lookup; "Speculative
// Decoding: Mathematical Foundations ...", "Non-Parametric Drafters"; "Speculative
// Decoding from First Principles", "Four kinds of drafter").  The proposals
// feed the greedy verify step (one-hot drafts).
//
// One workgroup per request.  The last n_max tokens (the suffix, newest
// first) go to LDS; every thread takes end positions e = L-2-t, L-2-t-256,
// ... and measures how many tokens ending at e match the suffix, capped at
// n_max.  The occurrence kept is the largest (matched length, e): the longest
// suffix that occurs earlier, and its latest occurrence.  The proposal is the
// up to K tokens after e, cut at the end of the context.
#include "internal.h"

namespace specdec {
namespace {

__device__ __forceinline__ unsigned long long max_u64(unsigned long long a, unsigned long long b) {
    return a > b ? a : b;
}

__global__ __launch_bounds__(kThreads) void ngram_propose(NgramParams a) {
    __shared__ int32_t suf[kMaxNgram];
    __shared__ unsigned long long red[kWaves];
    const int b = blockIdx.x;
    const int L = min(max(a.len[b], 0), a.Ls);
    const int32_t* c = a.ctx + (size_t)b * a.Ls;
    const int ns = min(a.n_max, L);
    for (int i = threadIdx.x; i < ns; i += kThreads) suf[i] = c[L - 1 - i];
    __syncthreads();
    // Key (matched length << 32 | e + 1); 0 = no occurrence of >= n_min tokens.
    // Each pass loads the last token of kBatch end positions per thread at
    // once; only positions whose last token matches read further back.
    constexpr int kBatch = 8;
    unsigned long long best = 0;
    const int32_t s0 = (ns > 0) ? suf[0] : 0;
    for (int base = L - 2 - (int)threadIdx.x; base >= a.n_min - 1; base -= kBatch * kThreads) {
        int32_t tok[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int e = base - j * kThreads;
            tok[j] = (e >= a.n_min - 1) ? c[e] : ~s0;
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            if (tok[j] != s0) continue;
            const int e = base - j * kThreads;
            int m = 1;
            while (m < ns && m <= e && c[e - m] == suf[m]) ++m;
            if (m >= a.n_min) best = max_u64(best, ((unsigned long long)m << 32) | (unsigned)(e + 1));
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) best = max_u64(best, __shfl_xor(best, o, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = best;
    __syncthreads();
    best = red[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) best = max_u64(best, red[w]);
    const int e = (int)(unsigned)(best & 0xFFFFFFFFu) - 1;
    const int kb = best ? min(a.K, L - 1 - e) : 0;
    for (int i = threadIdx.x; i < a.K; i += kThreads) a.drafts[(size_t)b * a.K + i] = (i < kb) ? c[e + 1 + i] : -1;
    if (threadIdx.x == 0) a.kpr[b] = kb;
}

}  // namespace

hipError_t launch_ngram(const NgramParams& p, hipStream_t s) {
    if (p.B == 0) return hipSuccess;
    hipLaunchKernelGGL(ngram_propose, dim3(p.B), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace specdec
