// Row statistics of the temperature softmax on gfx950: row max and
// sum_t exp((l_t - max) / T) ("3.5 Speculative Decoding", section "Notation":
// p is the next-token distribution after temperature).
//
//  1. stats_partial  one workgroup per (row, tile): tile max and sum.
//  2. stats_merge    one thread per row: merges the tiles in fp64.
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

}  // namespace

hipError_t launch_stats(const StatsParams& p, int dtype, bool vec, hipStream_t s) {
    if (dtype == kBF16) return vec ? launch<kBF16, true>(p, s) : launch<kBF16, false>(p, s);
    return vec ? launch<kFP32, true>(p, s) : launch<kFP32, false>(p, s);
}

}  // namespace specdec
