// Device-side building blocks shared by the verify, greedy and row-statistics
// kernels for gfx950 (wave64, 256-thread workgroups).
//
// Streaming model: a row of V logits is read as 16-byte vectors (8 bf16 or 4
// fp32 values).  A workgroup reads a "tile" of 4 x 256 vectors (16 KB): each
// thread issues 4 independent 16-byte nontemporal loads before it decodes
// any of them.  Consecutive threads read consecutive vectors, so each load
// instruction of a wave covers 1 KB of contiguous memory.  A "slab" is one
// load instruction of the workgroup: 256 consecutive vectors.
//
// Softmax arithmetic: p_t = exp((l_t - m) / T) / Z is evaluated as
// exp2(l_t * c - M) with c = log2(e) / T split into two floats hi + lo
// (hi < c strictly, so lo > 0 and a -inf logit gives -inf, never NaN) and
// M = fp32(m * c), the reference offset of a thread, tile or row.  The
// exponent is fma(x, lo, fma(x, hi, -M)): two operations, c carried to about
// 48 bits, and the only rounding that varies from element to element is that
// of the final float.  The rounding of M itself is the same for every
// element that shares the reference, and every rescale between references
// (thread -> tile -> row) uses the same M values, so it cancels in p.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace specdec {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 4;                       // vectors per thread per tile
constexpr int kTileVec = kThreads * kUnroll;     // vectors per tile (16 KB)
constexpr int kSlab = 64;                        // vectors per slab: one wave's vectors of one unroll step
constexpr int kSlabsPerTile = kTileVec / kSlab;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum : int { kFP32 = 0, kBF16 = 1 };

template <int DT> struct Elem;
template <> struct Elem<kFP32> { static constexpr int E = 4; static constexpr int S = 4; };
template <> struct Elem<kBF16> { static constexpr int E = 8; static constexpr int S = 2; };

struct Scale {
    float hi;       // largest float strictly below log2(e)/T
    float lo;       // log2(e)/T - hi, rounded to float (> 0)
    double c;       // log2(e)/T in double
    double inv_t;   // 1/T in double
};

// The reference offset of a max m: M = fp32(m * c).
__host__ __device__ __forceinline__ float offset_of(float m, const Scale& s) {
    return (float)((double)m * s.c);
}

// Base-2 exponent of exp(x / T) relative to the offset M: x * c - M.
__device__ __forceinline__ float exponent2(float x, float M, const Scale& s) {
    return __fmaf_rn(x, s.lo, __fmaf_rn(x, s.hi, -M));
}

__device__ __forceinline__ float fast_exp2(float a) { return __builtin_amdgcn_exp2f(a); }

// ---------------------------------------------------------------------------
// Loads
// ---------------------------------------------------------------------------

template <int DT> __device__ __forceinline__ u32x4 neg_inf_raw() {
    if (DT == kBF16) return u32x4{0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u};
    return u32x4{0xFF800000u, 0xFF800000u, 0xFF800000u, 0xFF800000u};
}

// Vector v of a row, as raw bits.  VEC: the row start is 16-byte aligned and
// V * sizeof(elem) is a multiple of 16, so every vector is one 16-byte load.
// Otherwise elements are loaded one by one and those at index >= V (and the
// whole vector when v >= NV) read as -inf.  NT selects nontemporal loads.
template <int DT, bool VEC, bool NT>
__device__ __forceinline__ u32x4 load_raw(const void* row, int V, int NV, int v) {
    if (VEC && NT) {
        // Streaming passes, branch-free: a vector past the end re-reads the
        // last one and is then replaced, so a tile's loads issue back to
        // back.  (The re-read passes keep the branch: fewer registers.)
        const u32x4* p = reinterpret_cast<const u32x4*>(row) + min(v, NV - 1);
        u32x4 r = __builtin_nontemporal_load(p);
        const u32x4 ninf = neg_inf_raw<DT>();
        const bool past = v >= NV;
#pragma unroll
        for (int k = 0; k < 4; ++k) r[k] = past ? ninf[k] : r[k];
        return r;
    }
    if (v >= NV) return neg_inf_raw<DT>();
    if (VEC) {
        const u32x4* p = reinterpret_cast<const u32x4*>(row) + v;
        if (NT) return __builtin_nontemporal_load(p);
        return *p;
    }
    u32x4 r = neg_inf_raw<DT>();
    if (DT == kFP32) {
        const uint32_t* p = reinterpret_cast<const uint32_t*>(row);
        const int t0 = v * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (t0 + e < V) r[e] = p[t0 + e];
    } else {
        const uint16_t* p = reinterpret_cast<const uint16_t*>(row);
        const int t0 = v * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (t0 + e < V) {
                const uint32_t h = p[t0 + e];
                if (e & 1) r[e >> 1] = (r[e >> 1] & 0x0000FFFFu) | (h << 16);
                else r[e >> 1] = (r[e >> 1] & 0xFFFF0000u) | h;
            }
        }
    }
    return r;
}

// Decode raw bits into E floats in ascending token order (exact for bf16:
// a bf16 value is the top half of the float with the same value).
template <int DT>
__device__ __forceinline__ void decode(const u32x4& r, float (&x)[Elem<DT>::E]) {
    if constexpr (DT == kFP32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = __uint_as_float(r[e]);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = __uint_as_float(r[e] << 16);
            x[2 * e + 1] = __uint_as_float(r[e] & 0xFFFF0000u);
        }
    }
}

// One logit, widened to float (used for gathers at draft tokens).
template <int DT>
__device__ __forceinline__ float load_one(const void* row, int t) {
    if (DT == kFP32) return reinterpret_cast<const float*>(row)[t];
    return __uint_as_float(static_cast<uint32_t>(reinterpret_cast<const uint16_t*>(row)[t]) << 16);
}

template <int E>
__device__ __forceinline__ float pairwise_sum(const float (&v)[E]) {
    static_assert(E == 2 || E == 4 || E == 8, "pairwise_sum: 2, 4 or 8 terms");
    if constexpr (E == 2) {
        return __fadd_rn(v[0], v[1]);
    } else if constexpr (E == 4) {
        return __fadd_rn(__fadd_rn(v[0], v[1]), __fadd_rn(v[2], v[3]));
    } else {
        return __fadd_rn(__fadd_rn(__fadd_rn(v[0], v[1]), __fadd_rn(v[2], v[3])),
                         __fadd_rn(__fadd_rn(v[4], v[5]), __fadd_rn(v[6], v[7])));
    }
}

// ---------------------------------------------------------------------------
// Wave / workgroup reductions (wave64)
//
// Built on DPP moves (a few cycles each) rather than LDS-crossbar shuffles:
// quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror and row_mirror combine
// lanes within each row of 16; row_bcast:15 (into rows 1 and 3) and
// row_bcast:31 (into rows 2 and 3) carry row results up the wave, so lane 63
// ends with the whole-wave result.  Lanes a DPP move does not write keep the
// identity passed as `old`.
// ---------------------------------------------------------------------------
enum : int {
    kDppQuad1032 = 0xB1,
    kDppQuad2301 = 0x4E,
    kDppRowShr1 = 0x111,
    kDppRowShr2 = 0x112,
    kDppRowShr4 = 0x114,
    kDppRowShr8 = 0x118,
    kDppRowMirror = 0x140,
    kDppRowHalfMirror = 0x141,
    kDppRowBcast15 = 0x142,
    kDppRowBcast31 = 0x143,
};

template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dpp(float v, float old) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, ROWS, 0xF, false));
}
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ double dpp(double v, double old) {
    const int lo = __builtin_amdgcn_update_dpp(__double2loint(old), __double2loint(v), CTRL, ROWS, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(__double2hiint(old), __double2hiint(v), CTRL, ROWS, 0xF, false);
    return __hiloint2double(hi, lo);
}

template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ int dpp(int v, int old) {
    return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWS, 0xF, false);
}

__device__ __forceinline__ float lane63(float v) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ double lane63(double v) {
    return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), 63),
                            __builtin_amdgcn_readlane(__double2loint(v), 63));
}

// Max / sum over each row of 16 lanes, in every lane of the row.
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp<kDppQuad1032>(v, -INFINITY));
    v = fmaxf(v, dpp<kDppQuad2301>(v, -INFINITY));
    v = fmaxf(v, dpp<kDppRowHalfMirror>(v, -INFINITY));
    return fmaxf(v, dpp<kDppRowMirror>(v, -INFINITY));
}
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp<kDppQuad1032>(v, 0.0f);
    v += dpp<kDppQuad2301>(v, 0.0f);
    v += dpp<kDppRowHalfMirror>(v, 0.0f);
    return v + dpp<kDppRowMirror>(v, 0.0f);
}
__device__ __forceinline__ double row16_sum(double v) {
    v += dpp<kDppQuad1032>(v, 0.0);
    v += dpp<kDppQuad2301>(v, 0.0);
    v += dpp<kDppRowHalfMirror>(v, 0.0);
    return v + dpp<kDppRowMirror>(v, 0.0);
}

// Max / sum over the wave, in every lane.
__device__ __forceinline__ float wave_max(float v) {
    v = row16_max(v);
    v = fmaxf(v, dpp<kDppRowBcast15, 0xA>(v, -INFINITY));
    v = fmaxf(v, dpp<kDppRowBcast31, 0xC>(v, -INFINITY));
    return lane63(v);
}
__device__ __forceinline__ float wave_sum(float v) {
    v = row16_sum(v);
    v += dpp<kDppRowBcast15, 0xA>(v, 0.0f);
    v += dpp<kDppRowBcast31, 0xC>(v, 0.0f);
    return lane63(v);
}
__device__ __forceinline__ double wave_sum(double v) {
    v = row16_sum(v);
    v += dpp<kDppRowBcast15, 0xA>(v, 0.0);
    v += dpp<kDppRowBcast31, 0xC>(v, 0.0);
    return lane63(v);
}

// Sums over the wave of four values per lane, returned to every lane.  Two
// half-wave swaps leave values 0 and 2 summed over lane pairs (l, l + 32) in
// lanes 0-31 and values 1 and 3 in lanes 32-63; one row swap then leaves
// value 0, 2, 1, 3 in rows 0, 1, 2, 3, each summed over four lanes; the rows
// of 16 lanes are reduced with DPP.  (Against four separate wave sums: one
// reduction's instructions for four.)
__device__ __forceinline__ float swap_add32(float a, float b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap_add16(float a, float b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ double swap_add32(double a, double b) {
    const auto lo = __builtin_amdgcn_permlane32_swap((unsigned)__double2loint(a), (unsigned)__double2loint(b), false,
                                                     false);
    const auto hi = __builtin_amdgcn_permlane32_swap((unsigned)__double2hiint(a), (unsigned)__double2hiint(b), false,
                                                     false);
    return __hiloint2double((int)hi[0], (int)lo[0]) + __hiloint2double((int)hi[1], (int)lo[1]);
}
__device__ __forceinline__ double swap_add16(double a, double b) {
    const auto lo = __builtin_amdgcn_permlane16_swap((unsigned)__double2loint(a), (unsigned)__double2loint(b), false,
                                                     false);
    const auto hi = __builtin_amdgcn_permlane16_swap((unsigned)__double2hiint(a), (unsigned)__double2hiint(b), false,
                                                     false);
    return __hiloint2double((int)hi[0], (int)lo[0]) + __hiloint2double((int)hi[1], (int)lo[1]);
}
__device__ __forceinline__ float lane_at(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ double lane_at(double v, int l) {
    return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), l),
                            __builtin_amdgcn_readlane(__double2loint(v), l));
}
// Two values: after the half-wave swap, lanes 0-31 hold a and lanes 32-63 b;
// a row swap of that with itself leaves a in rows 0-1 and b in rows 2-3.
__device__ __forceinline__ void wave_sum2(float& a, float& b) {
    const float w = swap_add32(a, b);
    const float x = row16_sum(swap_add16(w, w));
    a = lane_at(x, 0);
    b = lane_at(x, 32);
}
template <typename T>
__device__ __forceinline__ void wave_sum4(const T (&v)[4], T (&out)[4]) {
    const T x = row16_sum(swap_add16(swap_add32(v[0], v[1]), swap_add32(v[2], v[3])));
    out[0] = lane_at(x, 0);
    out[2] = lane_at(x, 16);
    out[1] = lane_at(x, 32);
    out[3] = lane_at(x, 48);
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ double wave_inclusive_scan(double v) {
    v += dpp<kDppRowShr1>(v, 0.0);
    v += dpp<kDppRowShr2>(v, 0.0);
    v += dpp<kDppRowShr4>(v, 0.0);
    v += dpp<kDppRowShr8>(v, 0.0);
    v += dpp<kDppRowBcast15, 0xA>(v, 0.0);
    return v + dpp<kDppRowBcast31, 0xC>(v, 0.0);
}

// Max / sum over the workgroup, in every thread.  Each call needs an LDS
// array of its own that nothing else writes afterwards (one barrier, no
// second one to guard the array's reuse).
__device__ __forceinline__ float block_max(float v, float* lds /* [kWaves] */) {
    v = wave_max(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) lds[w] = v;
    __syncthreads();
    float r = lds[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) r = fmaxf(r, lds[i]);
    return r;
}

__device__ __forceinline__ double block_sum(double v, double* lds /* [kWaves] */) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) lds[w] = v;
    __syncthreads();
    double r = lds[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) r += lds[i];
    return r;
}

// ---------------------------------------------------------------------------
// Row statistics of one tile: (max m, sum of exp2(x * c - fp32(m * c))) over
// the tile's vectors [tile * kTileVec, (tile + 1) * kTileVec) of one row.
// Per thread: max over its vectors, then exponentials relative to that
// thread's offset, summed in fp32 per vector (pairwise) and in fp64 across
// vectors; the thread sums are rescaled to the workgroup offset and added in
// fp64.  The result is valid in thread 0 only.
// ---------------------------------------------------------------------------
template <int DT, bool VEC, bool NT = true>
__device__ __forceinline__ void tile_load(const void* row, int V, int NV, int tile,
                                          u32x4 (&raw)[kUnroll]) {
    const int v0 = tile * kTileVec + threadIdx.x;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) raw[u] = load_raw<DT, VEC, NT>(row, V, NV, v0 + u * kThreads);
}

template <int DT>
__device__ __forceinline__ void tile_reduce(const u32x4 (&raw)[kUnroll], const Scale& sc,
                                            float& m_out, double& s_out, float* lds_f,
                                            double* lds_d) {
    constexpr int E = Elem<DT>::E;
    float mt = -INFINITY;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        float x[E];
        decode<DT>(raw[u], x);
#pragma unroll
        for (int e = 0; e < E; ++e) mt = fmaxf(mt, x[e]);
    }
    const bool empty = (mt == -INFINITY);
    const float Mt = offset_of(empty ? 0.0f : mt, sc);
    double s = 0.0;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        float x[E], ev[E];
        decode<DT>(raw[u], x);
#pragma unroll
        for (int e = 0; e < E; ++e) ev[e] = fast_exp2(exponent2(x[e], Mt, sc));
        s += (double)pairwise_sum<E>(ev);
    }
    const float mb = block_max(mt, lds_f);
    const float Mb = offset_of(mb, sc);
    const double scaled = empty ? 0.0 : s * (double)fast_exp2((float)((double)Mt - (double)Mb));
    const double sb = block_sum(scaled, lds_d);
    m_out = mb;
    s_out = sb;
}

template <int DT, bool VEC, bool NT = true>
__device__ __forceinline__ void tile_stats(const void* row, int V, int NV, int tile, const Scale& sc,
                                           float& m_out, double& s_out, float* lds_f,
                                           double* lds_d) {
    u32x4 raw[kUnroll];
    tile_load<DT, VEC, NT>(row, V, NV, tile, raw);
    tile_reduce<DT>(raw, sc, m_out, s_out, lds_f, lds_d);
}

// Merge per-tile partials (m_c, s_c) of one row into (max, sum relative to
// the row offset fp32(max * c)), rescaling in fp64.  Loads go out 16 tiles
// at a time.
__device__ __forceinline__ void merge_partials(const float* pm, const double* ps, int C,
                                               const Scale& sc, float* m_out, double* z_out) {
    constexpr int G = 16;
    float m = -INFINITY;
    double z = 0.0;
    for (int g0 = 0; g0 < C; g0 += G) {
        float lm[G];
        double ls[G];
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const bool ok = g0 + i < C;
            lm[i] = ok ? pm[g0 + i] : -INFINITY;
            ls[i] = ok ? ps[g0 + i] : 0.0;
        }
        float gm = m;
#pragma unroll
        for (int i = 0; i < G; ++i) gm = fmaxf(gm, lm[i]);
        if (gm != -INFINITY) {
            const double Mg = (double)offset_of(gm, sc);
            if (m != -INFINITY && gm > m) z *= exp2((double)offset_of(m, sc) - Mg);
#pragma unroll
            for (int i = 0; i < G; ++i)
                if (lm[i] != -INFINITY) z += ls[i] * exp2((double)offset_of(lm[i], sc) - Mg);
            m = gm;
        }
    }
    *m_out = m;
    *z_out = z;
}

}  // namespace specdec
