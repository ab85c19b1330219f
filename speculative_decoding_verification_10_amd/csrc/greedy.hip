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
// The tree variant runs the same row kernel over the N + 1 rows of a
// flattened draft tree, then tree_decisions (one wave per request) instead
// of greedy_decisions.
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

// Wave-level memory ordering of LDS between the lanes of one wave.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// A tile word as a key whose unsigned order is the (value, index) order:
// larger value first, lower index on equal values (-0 and +0 are equal).
__device__ __forceinline__ uint64_t order_key(uint64_t w) {
    float v;
    int i;
    dec_pair(w, v, i);
    if (v == 0.0f) v = 0.0f;
    uint32_t u = __float_as_uint(v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint32_t)~(uint32_t)i;
}

constexpr int kWordBatch = 8;   // tile words per lane in flight

// am[r] = argmax of target row r of request b, r = 0 .. kb, by one wave,
// from the tile words the row kernel wrote; visible to the whole wave on
// return.  The rows' words are contiguous: lane l takes words l, l + 64,
// ..., kWordBatch loads in flight at a time, and folds each into its row's
// key with an LDS atomic max.
__device__ void row_argmaxes(const GreedyParams& a, int b, int kb, int* am) {
    __shared__ uint64_t key[kMaxK + 1];
    const int K = a.K, C = a.C;
    const int lane = threadIdx.x & 63;
    const uint64_t* words = a.slot + (size_t)b * (K + 1) * C;
    const int W = (kb + 1) * C;
    for (int r = lane; r <= kb; r += 64) key[r] = 0;
    wave_sync();
    for (int base = 0; base < W; base += 64 * kWordBatch) {
        uint64_t got[kWordBatch];
#pragma unroll
        for (int q = 0; q < kWordBatch; ++q) {
            const int w = base + 64 * q + lane;
            got[q] = (w < W) ? words[w] : 0;
        }
#pragma unroll
        for (int q = 0; q < kWordBatch; ++q) {
            const int w = base + 64 * q + lane;
            if (w < W) atomicMax(reinterpret_cast<unsigned long long*>(&key[w / C]),
                                 (unsigned long long)order_key(got[q]));
        }
    }
    wave_sync();
    for (int r = lane; r <= kb; r += 64) am[r] = min(max((int)~(uint32_t)key[r], 0), a.V - 1);
    wave_sync();
}

// The decision of request b, by one wave (its own workgroup).
__device__ void greedy_decide(const GreedyParams& a, int b, int* am) {
    const int K = a.K;
    const int kb = greedy_k(a, b);
    const int lane = threadIdx.x & 63;
    row_argmaxes(a, b, kb, am);
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

// Greedy tree verification ("3.5 Speculative Decoding", "Tree
// verification"; "Speculative Decoding: Mathematical Foundations ...",
// "Tree-Based Verification and Custom Attention Masks"), by one wave for
// request b with n = kb nodes in flattened order (parent[i] < i, -1 = the
// root).  Node i passes its own test when its token is the argmax of its
// parent's row (row 0 for the root, row p + 1 after node p); it is accepted
// when it and every ancestor pass.  The kept path ends at the deepest
// accepted node (lowest index on ties) and is followed by the argmax of the
// row after it.
//
// Acceptance and depth by pointer jumping over the parent links
// (log2 n synchronous rounds over LDS; every lane holds up to 4 nodes), the
// 2^r-th ancestor of every node kept per round, so that each path slot finds
// its node by binary lifting from the path's end.  A node whose parent link
// breaks the precondition (-1 <= parent[i] < i) is never accepted.
constexpr int kTreeLift = 8;                       // 2^8 > kMaxK ancestors
constexpr int kTreePerLane = (kMaxK + 64) / 64;    // nodes per lane
constexpr int kTreeKeyBits = 9;                    // node index field of a path key

__device__ void tree_decide(const GreedyParams& a, int b, int* am) {
    __shared__ int32_t tok[kMaxK];
    __shared__ int32_t ok[kMaxK];
    __shared__ int32_t dep[kMaxK];
    __shared__ int16_t up[kTreeLift][kMaxK];
    const int N = a.K;
    const int n = greedy_k(a, b);
    const int lane = threadIdx.x & 63;
    const int32_t* ptok = a.tokens + (size_t)b * N;
    const int32_t* ppar = a.parents + (size_t)b * N;
    int par[kTreePerLane];
#pragma unroll
    for (int q = 0; q < kTreePerLane; ++q) {
        const int i = lane + 64 * q;
        par[q] = -1;
        if (i < n) {
            const int p = ppar[i];
            par[q] = (p >= -1 && p < i) ? p : -2;      // -2: a broken link
            tok[i] = ptok[i];
        }
    }
    row_argmaxes(a, b, n, am);
    // Own test, then the links (a broken link becomes "no parent, rejected").
    int jmp[kTreePerLane];
#pragma unroll
    for (int q = 0; q < kTreePerLane; ++q) {
        const int i = lane + 64 * q;
        jmp[q] = -1;
        if (i < n) {
            const int p = par[q];
            ok[i] = (p >= -1) && tok[i] == am[p + 1];
            dep[i] = 1;
            jmp[q] = max(p, -1);
            up[0][i] = (int16_t)jmp[q];
        }
    }
    wave_sync();
    // Round r: ok / dep cover the 2^r nodes from i up (fewer near the root),
    // jmp is the 2^r-th ancestor; afterwards the 2^(r+1)-th.
    for (int r = 0; r < kTreeLift; ++r) {
        bool linked = false;
#pragma unroll
        for (int q = 0; q < kTreePerLane; ++q) linked |= jmp[q] >= 0;
        if (__ballot(linked) == 0) break;
        int nok[kTreePerLane], ndep[kTreePerLane], njmp[kTreePerLane];
#pragma unroll
        for (int q = 0; q < kTreePerLane; ++q) {
            const int i = lane + 64 * q;
            const int j = jmp[q];
            nok[q] = 0;
            ndep[q] = 0;
            njmp[q] = j;
            if (i < n) {
                nok[q] = ok[i];
                ndep[q] = dep[i];
                if (j >= 0) {
                    nok[q] &= ok[j];
                    ndep[q] += dep[j];
                    njmp[q] = up[r][j];
                }
            }
        }
        wave_sync();
#pragma unroll
        for (int q = 0; q < kTreePerLane; ++q) {
            const int i = lane + 64 * q;
            jmp[q] = njmp[q];
            if (i < n) {
                ok[i] = nok[q];
                dep[i] = ndep[q];
                if (r + 1 < kTreeLift) up[r + 1][i] = (int16_t)njmp[q];
            }
        }
        wave_sync();
    }
    // Deepest accepted node, lowest index on ties: the largest key.
    uint32_t key = 0;
#pragma unroll
    for (int q = 0; q < kTreePerLane; ++q) {
        const int i = lane + 64 * q;
        if (i < n && ok[i])
            key = max(key, ((uint32_t)dep[i] << kTreeKeyBits) | (uint32_t)((1 << kTreeKeyBits) - 1 - i));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) key = max(key, (uint32_t)__shfl_xor((int)key, off));
    const int D = (int)(key >> kTreeKeyBits);
    const int end = key ? (1 << kTreeKeyBits) - 1 - (int)(key & ((1u << kTreeKeyBits) - 1)) : -1;
    // Slot d < D holds the ancestor of `end` at distance D - 1 - d.
    for (int d = lane; d <= N; d += 64) {
        int32_t v = -1, node = -1;
        if (d < D) {
            node = end;
            const int dist = D - 1 - d;
            for (int r = 0; r < kTreeLift; ++r)
                if ((dist >> r) & 1) node = up[r][node];
            v = tok[node];
        } else if (d == D) {
            v = am[end + 1];
        }
        a.out[(size_t)b * (N + 1) + d] = v;
        if (a.path && d < N) a.path[(size_t)b * N + d] = node;
    }
    if (lane == 0) a.nacc[b] = D;
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

// Tree decisions: workgroup x (one wave) takes request x.
__global__ __launch_bounds__(64) void tree_decisions(GreedyParams a) {
    __shared__ int am[kMaxK + 1];
    tree_decide(a, blockIdx.x, am);
}

template <int DT, bool VEC>
hipError_t launch(const GreedyParams& p, hipStream_t s, hipEvent_t const* events, bool tree) {
    if (p.B == 0) return hipSuccess;
    hipExtLaunchKernelGGL((greedy_rows<DT, VEC>), dim3(p.C, p.K + 1, p.B), dim3(kThreads), 0, s,
                          events ? events[0] : nullptr, events ? events[1] : nullptr, 0, p);
    if (tree)
        hipExtLaunchKernelGGL(tree_decisions, dim3(p.B), dim3(64), 0, s, nullptr,
                              events ? events[2] : nullptr, 0, p);
    else
        hipExtLaunchKernelGGL(greedy_decisions, dim3(p.B), dim3(64), 0, s, nullptr,
                              events ? events[2] : nullptr, 0, p);
    return hipGetLastError();
}

hipError_t dispatch(const GreedyParams& p, int dtype, bool vec, hipStream_t s,
                    hipEvent_t const* events, bool tree) {
    if (dtype == kBF16)
        return vec ? launch<kBF16, true>(p, s, events, tree) : launch<kBF16, false>(p, s, events, tree);
    return vec ? launch<kFP32, true>(p, s, events, tree) : launch<kFP32, false>(p, s, events, tree);
}

}  // namespace

hipError_t launch_greedy(const GreedyParams& p, int dtype, bool vec, hipStream_t s,
                         hipEvent_t const* events) {
    return dispatch(p, dtype, vec, s, events, false);
}

hipError_t launch_tree_greedy(const GreedyParams& p, int dtype, bool vec, hipStream_t s,
                              hipEvent_t const* events) {
    return dispatch(p, dtype, vec, s, events, true);
}

}  // namespace specdec
