// Row statistics of the temperature softmax on gfx950: row max and
// sum_t exp((l_t - max) / T) ("3.5 Speculative Decoding", section "Notation":
// p is the next-token distribution after temperature).
//
//  1. stats_partial  one workgroup per (row, tile): tile max and sum.
//  2. stats_merge    one thread per row: merges the tiles in fp64.
//
// Also the read-stream measurement helper (read_stream): the row pass's load
// pattern alone, the ceiling the row pass is measured against.
#include <hip/hip_ext.h>

#include "internal.h"

namespace specdec {
namespace {

constexpr int64_t kRowsPerZ = 32768;   // rows per grid z-slice (grid y and z stay below 2^16)

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void stats_partial(StatsParams a) {
    __shared__ float lds_f[kWaves];
    __shared__ double lds_d[kWaves];
    constexpr int S = Elem<DT>::S;
    // Workgroup (x, y, z): tile x of row z * kRowsPerZ + y.
    const int tile = blockIdx.x;
    const size_t row = (size_t)blockIdx.z * kRowsPerZ + blockIdx.y;
    if (row >= (size_t)a.rows) return;
    const size_t item = row * a.C + tile;
    const void* p = static_cast<const char*>(a.logits) + row * (size_t)a.V * S;
    float m;
    double z;
    tile_stats<DT, VEC>(p, a.V, a.NV, tile, a.sc, m, z, lds_f, lds_d);
    if (threadIdx.x == 0) {
        a.part_m[item] = m;
        a.part_s[item] = z;
    }
}

__global__ __launch_bounds__(kThreads) void stats_merge(StatsParams a) {
    const size_t row = (size_t)blockIdx.x * kThreads + threadIdx.x;
    if (row >= (size_t)a.rows) return;
    float m;
    double z;
    merge_partials(a.part_m + row * a.C, a.part_s + row * a.C, a.C, a.sc, &m, &z);
    a.row_max[row] = m;
    // z is relative to the offset fp32(m * c); the output is relative to m * c.
    a.row_sumexp[row] = (float)(z * exp2((double)offset_of(m, a.sc) - (double)m * a.sc.c));
}

template <int DT, bool VEC>
hipError_t launch(const StatsParams& p, hipStream_t s) {
    if (p.rows == 0) return hipSuccess;
    const int64_t ny = p.rows < kRowsPerZ ? p.rows : kRowsPerZ;
    const int64_t nz = (p.rows + kRowsPerZ - 1) / kRowsPerZ;
    hipLaunchKernelGGL((stats_partial<DT, VEC>), dim3(p.C, (unsigned)ny, (unsigned)nz), dim3(kThreads), 0, s, p);
    const unsigned g2 = (unsigned)((p.rows + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(stats_merge, dim3(g2), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

// The read pattern of the row pass with no other work: workgroup x reads
// the 16 KB tile x of `data` (nv 16-byte vectors), four branch-free
// nontemporal loads per thread issued before any use, and stores a word
// only when the tile's bits fold to a value no data is expected to give,
// so that the loads cannot be dropped while almost nothing is written.
__global__ __launch_bounds__(kThreads) void read_stream(const u32x4* data, int64_t nv, uint32_t* sink) {
    const int64_t v0 = (int64_t)blockIdx.x * kTileVec + threadIdx.x;
    u32x4 r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) r[u] = __builtin_nontemporal_load(data + min(v0 + u * kThreads, nv - 1));
    uint32_t x = 0;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) x ^= r[u][0] ^ r[u][1] ^ r[u][2] ^ r[u][3];
    if (x == 0x9E3779B9u) sink[blockIdx.x] = x;
}

}  // namespace

hipError_t launch_read_stream(const void* data, size_t bytes, uint32_t* sink, hipStream_t s,
                              hipEvent_t start, hipEvent_t stop) {
    const int64_t nv = (int64_t)(bytes / 16);
    if (nv == 0) return hipSuccess;
    const int64_t tiles = (nv + kTileVec - 1) / kTileVec;
    hipExtLaunchKernelGGL(read_stream, dim3((unsigned)tiles), dim3(kThreads), 0, s, start, stop, 0,
                          static_cast<const u32x4*>(data), nv, sink);
    return hipGetLastError();
}

hipError_t launch_stats(const StatsParams& p, int dtype, bool vec, hipStream_t s) {
    if (dtype == kBF16) return vec ? launch<kBF16, true>(p, s) : launch<kBF16, false>(p, s);
    return vec ? launch<kFP32, true>(p, s) : launch<kFP32, false>(p, s);
}

}  // namespace specdec
