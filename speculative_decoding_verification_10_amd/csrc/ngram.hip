// n-gram (prompt-lookup) drafter on gfx950: find the last few tokens earlier
// in the context and propose what followed them there ("3.5 Speculative
// Decoding", "Choosing a draft", n-gram / prompt lookup; "Speculative
// Decoding: Mathematical Foundations ...", "Non-Parametric Drafters"; "Speculative
// Decoding from First Principles", "Four kinds of drafter").  The proposals
// feed the greedy verify step (one-hot drafts).
//
// One workgroup per request.  The last n_max tokens (the suffix, newest
// first) go to LDS.  The end positions e = L-2, L-3, ... are taken in
// chunks of 8,192, newest first: each chunk's tokens (with the 63 before
// it, which a match may extend into) are staged in LDS with coalesced
// loads, every thread takes end positions e, e-256, ... and measures how
// many tokens ending at e match the suffix, capped at n_max.  The kept
// occurrence is the largest (matched length, e): the longest suffix that
// occurs earlier, at its latest occurrence.  Once a chunk holds a match of
// the full suffix length, older chunks cannot do better and are skipped.
// When the whole row (context stride Ls) fits the buffer, it is staged at
// once, before the length is known, so the suffix, the matches and the
// proposal all come from LDS after a single round trip to memory.  The
// proposal is the up to K tokens after e, cut at the end of the context.
#include "internal.h"

namespace specdec {
namespace {

constexpr int kChunk = 8192;                 // end positions per chunk
constexpr int kHalo = kMaxNgram - 1;         // tokens before a chunk a match can reach
constexpr int kLoadBatch = 8;                // staging loads in flight per thread

__device__ __forceinline__ unsigned long long max_u64(unsigned long long a, unsigned long long b) {
    return a > b ? a : b;
}

__global__ __launch_bounds__(kThreads) void ngram_propose(NgramParams a) {
    __shared__ int32_t suf[kMaxNgram];
    __shared__ int32_t buf[kHalo + kChunk];
    __shared__ unsigned long long red[kWaves];
    const int b = blockIdx.x;
    const int t = threadIdx.x;
    const int32_t* c = a.ctx + (size_t)b * a.Ls;
    // Stage tokens [base, base + n) of the row into buf.
    auto stage = [&](int base, int n) {
        for (int i0 = t; i0 < n; i0 += kLoadBatch * kThreads) {
            int32_t v[kLoadBatch];
#pragma unroll
            for (int q = 0; q < kLoadBatch; ++q) {
                const int i = i0 + q * kThreads;
                v[q] = (i < n) ? c[base + i] : 0;
            }
#pragma unroll
            for (int q = 0; q < kLoadBatch; ++q) {
                const int i = i0 + q * kThreads;
                if (i < n) buf[i] = v[q];
            }
        }
    };
    const bool whole = a.Ls <= kHalo + kChunk;          // the row fits: stage it all now
    if (whole) stage(0, a.Ls);
    const int L = min(max(a.len[b], 0), a.Ls);
    const int ns = min(a.n_max, L);
    if (whole) {
        __syncthreads();
        for (int i = t; i < ns; i += kThreads) suf[i] = buf[L - 1 - i];
    } else {
        for (int i = t; i < ns; i += kThreads) suf[i] = c[L - 1 - i];
    }
    // Key (matched length << 32 | e + 1); 0 = no occurrence of >= n_min tokens.
    unsigned long long best = 0;
    for (int hi = L - 1; hi > a.n_min - 1;) {           // end positions [lo, hi)
        const int lo = max(hi - kChunk, a.n_min - 1);
        const int base = whole ? 0 : max(lo - kHalo, 0);
        __syncthreads();                                // the previous chunk is done
        if (!whole) stage(base, hi - base);
        __syncthreads();
        const int32_t s0 = (ns > 0) ? suf[0] : 0;
        for (int e = hi - 1 - t; e >= lo; e -= kThreads) {
            if (buf[e - base] != s0) continue;
            int m = 1;
            while (m < ns && m <= e && buf[e - m - base] == suf[m]) ++m;
            if (m >= a.n_min) best = max_u64(best, ((unsigned long long)m << 32) | (unsigned)(e + 1));
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) best = max_u64(best, __shfl_xor(best, o, 64));
        if ((t & 63) == 0) red[t >> 6] = best;
        __syncthreads();
        best = red[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) best = max_u64(best, red[w]);
        if ((int)(best >> 32) >= ns) break;             // a full-length match: older ones lose
        hi = lo;
    }
    const int e = (int)(unsigned)(best & 0xFFFFFFFFu) - 1;
    const int kb = best ? min(a.K, L - 1 - e) : 0;
    for (int i = t; i < a.K; i += kThreads)
        a.drafts[(size_t)b * a.K + i] = (i < kb) ? (whole ? buf[e + 1 + i] : c[e + 1 + i]) : -1;
    if (t == 0) a.kpr[b] = kb;
}

}  // namespace

hipError_t launch_ngram(const NgramParams& p, hipStream_t s) {
    if (p.B == 0) return hipSuccess;
    hipLaunchKernelGGL(ngram_propose, dim3(p.B), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace specdec
