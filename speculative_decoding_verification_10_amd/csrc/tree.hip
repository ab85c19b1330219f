// Tree attention metadata on gfx950 ("3.5 Speculative Decoding", "Tree
// verification": every flattened draft node attends to the context, its
// ancestors and itself, and nodes at the same depth share a position index;
// "Speculative Decoding: Mathematical Foundations ...", "Tree-Based
// Verification and Custom Attention Masks": the mask opens exactly the
// ancestor links).
//
// One workgroup per request, one thread per node (N <= 255).  Each node's
// attended set is a 256-bit row in LDS, built by pointer jumping: the row
// covers the nodes from i up to (not including) its current jump target,
// and each round ORs in the jump target's row and doubles the jump, so log2
// of the depth rounds finish every row.  The rows are then written out as
// bytes, consecutive threads on consecutive bytes.
#include "internal.h"

namespace specdec {
namespace {

constexpr int kRowWords = (kMaxK + 31) / 32;       // a bit per node

__global__ __launch_bounds__(kThreads) void tree_mask_kernel(TreeMaskParams a) {
    __shared__ uint32_t bits[kMaxK][kRowWords];
    __shared__ int32_t dep[kMaxK];
    __shared__ int32_t jmp[kMaxK];
    const int b = blockIdx.x;
    const int N = a.N;
    const int n = a.nn ? min(max(a.nn[b], 0), N) : N;
    const int i = threadIdx.x;
    if (i < n) {
        const int p = a.parents[(size_t)b * N + i];
        // A link that breaks -1 <= parent[i] < i is treated as the root's.
        jmp[i] = (p >= -1 && p < i) ? p : -1;
        dep[i] = 1;
#pragma unroll
        for (int w = 0; w < kRowWords; ++w) bits[i][w] = (w == (i >> 5)) ? (1u << (i & 31)) : 0u;
    }
    __syncthreads();
    for (int r = 0; r < 8; ++r) {
        const int j = (i < n) ? jmp[i] : -1;
        if (__syncthreads_or(j >= 0) == 0) break;
        uint32_t row[kRowWords];
        int nd = 0, nj = j;
        if (j >= 0) {
#pragma unroll
            for (int w = 0; w < kRowWords; ++w) row[w] = bits[i][w] | bits[j][w];
            nd = dep[i] + dep[j];
            nj = jmp[j];
        }
        __syncthreads();
        if (j >= 0) {
#pragma unroll
            for (int w = 0; w < kRowWords; ++w) bits[i][w] = row[w];
            dep[i] = nd;
            jmp[i] = nj;
        }
        __syncthreads();
    }
    if (i < N) a.depth[(size_t)b * N + i] = (i < n) ? dep[i] : -1;
    uint8_t* m = a.mask + (size_t)b * N * N;
    const int total = N * N;
    for (int e = threadIdx.x; e < total; e += kThreads) {
        const int r = e / N, c = e - r * N;
        m[e] = (r < n && c < n) ? (uint8_t)((bits[r][c >> 5] >> (c & 31)) & 1u) : (uint8_t)0;
    }
}

}  // namespace

hipError_t launch_tree_mask(const TreeMaskParams& p, hipStream_t s) {
    if (p.B == 0 || p.N == 0) return hipSuccess;
    hipLaunchKernelGGL(tree_mask_kernel, dim3(p.B), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace specdec
