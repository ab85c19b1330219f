// Top-k / top-p processed distributions on gfx950 ("3.5 Speculative
// Decoding", "Notation": p and q are the distributions after temperature,
// top-p and the like; "Common pitfalls" and "246 Speculative Decoding", Key
// takeaways: the target and the draft go through the same temperature /
// top-k / top-p processing).
//
// Both filters keep an upper set of logit values, so each row's processing is
// one floor: the kept tokens are those with logit >= floor.
//   top-k: the floor is the top_k-th largest logit (ties at it are kept);
//   top-p: on the top-k survivors, the largest logit v whose upper set
//          {l >= v} holds at least top_p of the survivors' mass.
//
// A small top-k (at most kCandPerTile) in the processed verify step takes
// its cuts from tile candidates (floor_cands, floor_merge, described where
// they are defined); floor_rows then takes only the rows those leave, each
// of its workgroups every kRowsGrid-th row slot.
//
// floor_rows: one workgroup of 1,024 threads per row.  The row is read from
// HBM once; the later passes over it mostly hit the L2 / Infinity Cache.  Rows of
// whole 16-byte vectors take window paths (bins over 16-bit keys for bf16,
// over the mass exponent for fp32; each is described where it is defined).
// Other rows (misaligned or of a ragged length) take the general selection:
//   1. the row max m and the offset M = fp32(m * c) of the verify step;
//   2. coarse levels of d = M - x * c (the base-2 exponent deficit of the
//      mass exp2(x * c - M)): level 0 holds d < 1, level j d < 2^j, level 8
//      the rest; counts and masses per level give the smallest level sure
//      to contain the top-k cut (exact counts) or the top-p cut (masses with
//      a safety margin).  {d < 2^j} is an upper set of logits, because d is
//      monotone in x;
//   3. the elements of that upper set become candidates in LDS (key and
//      mass); masses are summed in 2^-35 fixed point, so sums are exact and
//      free of order;
//   4. radix select over the candidates' order-preserving 32-bit keys
//      (11-bit digits in LDS histograms): the top_k-th largest key, then the
//      key at which the mass from the top reaches top_p of the survivors.
//      Candidates that overflow LDS, or a coarse estimate that missed, fall
//      back to the same selection over the whole row;
//   5. the floor, and for the verify step the row statistics of the kept
//      tokens (max, fp64 sum of exp2(x * c - M)), the logit at the draft
//      token (-inf when cut), written in the verify step's slot layout.
#include <hip/hip_ext.h>

#include "internal.h"
#include "slots.h"

namespace specdec {
namespace {

constexpr int kFT = 1024;                  // threads per row
constexpr int kFW = kFT / 64;              // waves per row
constexpr int kBins = 2048;                // radix bins (11-bit digits)
constexpr int kCand = 4096;                // LDS candidates
constexpr int kLevels = 9;                 // coarse levels: d < 2^j (j = 0..7), then the rest
constexpr double kFix = 34359738368.0;     // 2^35: fixed-point scale of a mass <= 1

// Order-preserving key of a logit (-0 and +0 share a key).
__device__ __forceinline__ uint32_t key_of(float x) {
    if (x == 0.0f) x = 0.0f;
    const uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float value_of(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ uint64_t fix_of(float e) { return __double2ull_rn((double)e * kFix); }

// Coarse level of an element from its exponent deficit d.
__device__ __forceinline__ int level_of(float d) {
    if (!(d >= 1.0f)) return 0;                       // d < 1 (and the max itself)
    const int ex = (int)((__float_as_uint(d) >> 23) & 0xFF) - 127;   // floor(log2 d), d >= 1
    return min(ex + 1, kLevels - 1);
}

struct FloorShared {
    uint64_t mass[kBins];               // radix histogram (weights)
    uint32_t ckey[kCand];               // candidates: key
    float cexp[kCand];                  //             mass exp2(x * c - M)
    float red_f[kFW];
    double red_d[kFW];
    uint64_t red_u[kFW];
    uint32_t red_c[kLevels][kFW];
    double red_m[kLevels][kFW];
    uint32_t ncand;
    int guard;
    uint32_t guard_count;
    uint32_t pick_bin;
    uint64_t pick_above;
};

// The row being processed and its offset.
struct RowRef {
    const void* row;
    int V, NV;
    float M;
    Scale sc;
};

// Workgroup reductions over 1,024 threads (fixed order: deterministic).
template <typename T, typename Op>
__device__ __forceinline__ T wg_reduce(T v, T* lds, Op op) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = op(v, __shfl_xor(v, o, 64));
    if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = v;
    __syncthreads();
    T r = lds[0];
#pragma unroll
    for (int i = 1; i < kFW; ++i) r = op(r, lds[i]);
    __syncthreads();
    return r;
}

// The same for an fp64 sum and an fp32 max, the wave step done by DPP moves
// instead of lane shuffles (no LDS round trips).
__device__ __forceinline__ double wg_sum(double v, double* lds) {
    v = wave_sum(v);
    if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = v;
    __syncthreads();
    double r = lds[0];
#pragma unroll
    for (int i = 1; i < kFW; ++i) r += lds[i];
    __syncthreads();
    return r;
}
__device__ __forceinline__ float wg_max(float v, float* lds) {
    v = wave_max(v);
    if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = lds[0];
#pragma unroll
    for (int i = 1; i < kFW; ++i) r = fmaxf(r, lds[i]);
    __syncthreads();
    return r;
}

// f(x) for every element of the row this thread visits (vectors t, t + 1024,
// ...; elements past V skipped).  The first pass over a row reads HBM; the
// later ones mostly hit the L2 / Infinity Cache.
// Four vectors per thread are loaded before any is used, so each thread
// keeps four 16-byte loads in flight.
constexpr int kRowBatch = 4;

template <int DT, bool VEC, typename F>
__device__ __forceinline__ void for_row(const RowRef& r, F&& f) {
    constexpr int E = Elem<DT>::E;
    for (int v0 = threadIdx.x; v0 < r.NV; v0 += kRowBatch * kFT) {
        u32x4 raw[kRowBatch];
#pragma unroll
        for (int u = 0; u < kRowBatch; ++u) raw[u] = load_raw<DT, VEC, false>(r.row, r.V, r.NV, v0 + u * kFT);
#pragma unroll
        for (int u = 0; u < kRowBatch; ++u) {
            const int v = v0 + u * kFT;
            float x[E];
            decode<DT>(raw[u], x);
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (v * E + e < r.V) f(x[e]);
        }
    }
}

// Sum of the fixed-point masses of the keys >= kmin: over the candidates
// (from_cand) or over the row.
template <int DT, bool VEC>
__device__ __noinline__ uint64_t mass_at_least(const RowRef& r, bool from_cand, uint32_t nc, uint32_t kmin,
                                               FloorShared& sh) {
    uint64_t s = 0;
    if (from_cand) {
        for (uint32_t c = threadIdx.x; c < nc; c += kFT)
            if (sh.ckey[c] >= kmin) s += fix_of(sh.cexp[c]);
    } else {
        for_row<DT, VEC>(r, [&](float x) {
            if (key_of(x) >= kmin) s += fix_of(fast_exp2(exponent2(x, r.M, r.sc)));
        });
    }
    return wg_reduce(s, sh.red_u, [](uint64_t p, uint64_t q) { return p + q; });
}

// Radix select over 32-bit keys, largest first, among the elements with key
// >= kmin (from the candidates or the row), each weighted by 1 (count) or by
// its fixed-point mass.  Returns the key at which the weight from the top
// first reaches `target`: the largest key K with W(keys >= K) >= target.
// 11-bit digits from the top: bf16 keys have 16 significant bits (two
// digits), fp32 keys 32 (three).
template <int DT, bool VEC>
__device__ __noinline__ uint32_t radix_select(const RowRef& r, bool from_cand, uint32_t nc, bool masses,
                                              uint32_t kmin, double target, FloorShared& sh) {
    constexpr int kDigits = (DT == kBF16) ? 2 : 3;
    uint32_t prefix = 0;
    uint64_t above = 0;                 // weight strictly above the current prefix
    for (int dg = 0; dg < kDigits; ++dg) {
        const int sh_ = dg == 0 ? 21 : dg == 1 ? (DT == kBF16 ? 16 : 10) : 0;
        const int wd = dg == 0 ? 11 : dg == 1 ? (DT == kBF16 ? 5 : 11) : 10;
        const int hi = sh_ + wd;        // key bits at and above hi are fixed
        for (int i = threadIdx.x; i < kBins; i += kFT) sh.mass[i] = 0;
        __syncthreads();
        auto add = [&](uint32_t key, uint64_t wgt) {
            if (key < kmin || (hi < 32 && (key >> hi) != prefix)) return;
            atomicAdd(reinterpret_cast<unsigned long long*>(&sh.mass[(key >> sh_) & ((1u << wd) - 1)]),
                      (unsigned long long)wgt);
        };
        if (from_cand) {
            for (uint32_t c = threadIdx.x; c < nc; c += kFT)
                add(sh.ckey[c], masses ? fix_of(sh.cexp[c]) : (uint64_t)1);
        } else {
            for_row<DT, VEC>(r, [&](float x) {
                add(key_of(x), masses ? fix_of(fast_exp2(exponent2(x, r.M, r.sc))) : (uint64_t)1);
            });
        }
        __syncthreads();
        // Thread t owns bins 2t and 2t+1; suffix sums from the top bin.
        const int t = threadIdx.x, lane = t & 63, w = t >> 6;
        const uint64_t h0 = sh.mass[2 * t], h1 = sh.mass[2 * t + 1];
        uint64_t s = h0 + h1;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint64_t n = __shfl_down(s, o, 64);
            if (lane + o < 64) s += n;
        }
        if (lane == 0) sh.red_u[w] = s;
        __syncthreads();
        for (int i = w + 1; i < kFW; ++i) s += sh.red_u[i];
        // s = weight of the bins >= 2t within the prefix.
        const uint64_t incl1 = s - h0, excl1 = incl1 - h1;
        const uint64_t incl0 = s, excl0 = s - h0;
        if ((double)(above + excl1) < target && target <= (double)(above + incl1)) {
            sh.pick_bin = 2 * t + 1;
            sh.pick_above = above + excl1;
        } else if ((double)(above + excl0) < target && target <= (double)(above + incl0)) {
            sh.pick_bin = 2 * t;
            sh.pick_above = above + excl0;
        }
        __syncthreads();
        prefix = (prefix << wd) | sh.pick_bin;
        above = sh.pick_above;
        __syncthreads();
    }
    // bf16 keys: the low 16 bits follow from the sign of the value.
    if (DT == kBF16) prefix = (prefix << 16) | ((prefix & 0x8000u) ? 0u : 0xFFFFu);
    return prefix;
}

// The floor of one row by coarse levels, LDS candidates and radix select
// (every dtype).  Returns the row max, the floor and the kept mass.
template <int DT, bool VEC>
__device__ __noinline__ void floor_by_select(const FloorParams& a, RowRef& r, FloorShared& sh, float& m_out, float& fl_out,
                                double& z_out) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const bool use_k = a.top_k > 0 && a.top_k < a.V;
    const bool use_p = a.top_p < 1.0;

    // 1. Row max and offset.
    float m = -INFINITY;
    for_row<DT, VEC>(r, [&](float x) { m = fmaxf(m, x); });
    m = wg_reduce(m, sh.red_f, [](float p, float q) { return fmaxf(p, q); });
    r.M = offset_of(m, a.sc);

    float fl = -INFINITY;
    double z = 0.0;                     // sum of the kept masses exp2(x * c - M)
    if (!use_k && !use_p) {
        for_row<DT, VEC>(r, [&](float x) { z += (double)fast_exp2(exponent2(x, r.M, r.sc)); });
        z = wg_reduce(z, sh.red_d, [](double p, double q) { return p + q; });
    } else {
        // 2. Coarse levels: per-level counts and masses, and the row's mass
        // in fixed point.
        uint32_t lc[kLevels];
        float lm[kLevels];
        uint64_t zfix = 0;
#pragma unroll
        for (int j = 0; j < kLevels; ++j) { lc[j] = 0; lm[j] = 0.0f; }
        for_row<DT, VEC>(r, [&](float x) {
            const float d = -exponent2(x, r.M, r.sc);
            const float e = fast_exp2(-d);
            const int lv = level_of(d);
            zfix += fix_of(e);
#pragma unroll
            for (int j = 0; j < kLevels; ++j) {
                lc[j] += (lv == j);
                lm[j] += (lv == j) ? e : 0.0f;
            }
        });
#pragma unroll
        for (int j = 0; j < kLevels; ++j) {
            uint32_t c = lc[j];
            double ms = (double)lm[j];
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                c += __shfl_xor(c, o, 64);
                ms += __shfl_xor(ms, o, 64);
            }
            if (lane == 0) { sh.red_c[j][w] = c; sh.red_m[j][w] = ms; }
        }
        // (This reduction's barriers also publish red_c / red_m.)
        const uint64_t zall = wg_reduce(zfix, sh.red_u, [](uint64_t p, uint64_t q) { return p + q; });
        // The guard level: the smallest level sure to hold the cut(s).  The
        // top-k cut bounds the top-p cut from below, so top-k decides when
        // both are on.  The masses carry a 0.1% margin; an exact check on
        // the candidates follows.
        if (t == 0) {
            uint32_t cc[kLevels];
            double cm[kLevels];
            uint32_t c_ = 0;
            double m_ = 0.0;
            for (int j = 0; j < kLevels; ++j) {
                for (int q = 0; q < kFW; ++q) { c_ += sh.red_c[j][q]; m_ += sh.red_m[j][q]; }
                cc[j] = c_;
                cm[j] = m_;
            }
            int g = kLevels - 1;
            const double want = a.top_p * cm[kLevels - 1] * 1.001;
            for (int j = kLevels - 1; j >= 0; --j)
                if (use_k ? cc[j] >= (uint32_t)a.top_k : cm[j] >= want) g = j;
            sh.guard = g;
            sh.guard_count = cc[g];
        }
        __syncthreads();
        const int g = sh.guard;
        bool cand = g < kLevels - 1 && sh.guard_count <= (uint32_t)kCand;
        // 3. Candidates: the upper set of the levels <= g.  Each thread
        // knows how many of its elements lie there; an exclusive scan of
        // those counts gives it a run of LDS slots, filled in element order
        // (so the candidates' order is fixed).
        uint32_t mine = 0;
#pragma unroll
        for (int j = 0; j < kLevels; ++j) mine += (j <= g) ? lc[j] : 0u;
        uint32_t base = mine;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t n = __shfl_up(base, o, 64);
            if (lane >= o) base += n;
        }
        if (lane == 63) sh.red_c[0][w] = base;          // wave totals
        __syncthreads();
        base -= mine;
        for (int q = 0; q < w; ++q) base += sh.red_c[0][q];
        if (t == kFT - 1) sh.ncand = base + mine;
        if (cand) {
            uint32_t n = base;
            for_row<DT, VEC>(r, [&](float x) {
                const float d = -exponent2(x, r.M, r.sc);
                if (level_of(d) <= g) {
                    sh.ckey[n] = key_of(x);
                    sh.cexp[n] = fast_exp2(-d);
                    ++n;
                }
            });
        }
        __syncthreads();
        const uint32_t nc = sh.ncand;
        // 4a. top-k: the top_k-th largest key.
        uint32_t fkey = 0, kkey = 0;
        if (use_k) {
            kkey = radix_select<DT, VEC>(r, cand, nc, false, 0u, (double)a.top_k, sh);
            fkey = kkey;
        }
        // 4b. top-p over the survivors (keys >= kkey): the key at which the
        // mass from the top reaches top_p of theirs.  Without top-k the
        // candidates must hold that much mass, else the row is used.
        if (use_p) {
            const uint64_t zk = use_k ? mass_at_least<DT, VEC>(r, cand, nc, kkey, sh) : zall;
            const double target = a.top_p * (double)zk;
            if (cand && !use_k && (double)mass_at_least<DT, VEC>(r, true, nc, 0u, sh) < target) cand = false;
            fkey = radix_select<DT, VEC>(r, cand, nc, true, kkey, target, sh);
        }
        fl = value_of(fkey);
        // 5. The kept mass: every kept element is a candidate when the
        // candidates were used (fixed point, exact), else a pass over the row.
        if (cand) {
            z = (double)mass_at_least<DT, VEC>(r, true, nc, fkey, sh) / kFix;
        } else {
            for_row<DT, VEC>(r, [&](float x) {
                if (x >= fl) z += (double)fast_exp2(exponent2(x, r.M, r.sc));
            });
            z = wg_reduce(z, sh.red_d, [](double p, double q) { return p + q; });
        }
    }

    m_out = m;
    fl_out = fl;
    z_out = z;
}

// ---------------------------------------------------------------------------
// bf16 rows.  Every bf16 value has a 16-bit order-preserving key; a bin per
// key holds its value's count, and a bin's mass is its count times the mass
// of its one value, so cuts found over bins are exact.
// ---------------------------------------------------------------------------
// Order-preserving 16-bit key of a bf16 value (bits h): a negative value's
// key is its inverted bits plus one, so -0 (0x8000) gets +0's key 0x8000 and
// the other keys stay distinct; keys 1..0x7F are the negative NaNs.
__device__ __forceinline__ uint32_t key16_of(uint32_t h) {
    return (h & 0x8000u) ? ((~h + 1u) & 0xFFFFu) : (h | 0x8000u);
}
__device__ __forceinline__ float value16_of(uint32_t k) {
    const uint32_t h = (k & 0x8000u) ? (k & 0x7FFFu) : (~(k - 1u) & 0xFFFFu);
    return __uint_as_float(h << 16);
}

// Sum over the threads above t (t' > t), for every t: within the wave the
// wave total less a DPP inclusive prefix sum, then the waves above.
__device__ __forceinline__ double sum_above(double v, double* lds) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const double incl = wave_inclusive_scan(v);
    const double tot = lane63(incl);
    if (lane == 0) lds[w] = tot;
    __syncthreads();
    double above = tot - incl;
    for (int q = w + 1; q < kFW; ++q) above += lds[q];
    __syncthreads();
    return above;
}

// bf16 rows (16-byte aligned, whole vectors): the thread's first 12 vectors
// stay in registers, the rest (of a 128K-logit row, about a quarter) is
// re-read by each pass from the L2 / Infinity Cache.  The row max comes first; then windows of
// 4,096 consecutive keys, from the max's key down, get one LDS bin per key
// (4 per thread).  The first window also sums the mass of everything below
// it (per thread, fp32), which gives the row's total without bins.  The
// top-k cut is the bin where the count from the top reaches top_k; the
// top-p cut is the bin where the survivors' mass from the top reaches
// top_p of theirs.  A cut below a window moves the search to the next one
// down.  The first window also stops at the keys whose mass is 2^-24 of the
// max's: the logits under it are only summed, not binned, which spares the
// LDS atomics of most of a typical row (its bulk lies far below the max).
// Their mass together is at most V * 2^-24 of the max's (< 1% for V < 2^17),
// so top-p cuts up to 0.99 and small top-k cuts almost always lie in it.
// No counter can overflow (32-bit counts).
// g(vector) for the vectors v0, v0 + 1,024, ... of a row of whole 16-byte
// vectors, re-read kTail at a time: the loads of a batch issue back to back
// (an index past the end re-reads the last vector, which is then skipped),
// so a pass costs one cache round trip per batch, not per vector.
constexpr int kTail = 4;
template <typename G>
__device__ __forceinline__ void tail_batches(const RowRef& r, int v0, G&& g) {
    const u32x4* base = reinterpret_cast<const u32x4*>(r.row);
    for (; v0 < r.NV; v0 += kTail * kFT) {
        u32x4 rv[kTail];
#pragma unroll
        for (int u = 0; u < kTail; ++u) rv[u] = base[min(v0 + u * kFT, r.NV - 1)];
#pragma unroll
        for (int u = 0; u < kTail; ++u)
            if (v0 + u * kFT < r.NV) g(rv[u]);
    }
}

constexpr int kWin = 4096;
constexpr float kFirstDeficit = 24.0f;
constexpr int kWinPerThread = kWin / kFT;              // 4

struct WinShared {
    uint32_t win[kWin];
    double red_d[kFW];
    uint32_t red_c[kFW];
    float red_f[kFW];
    uint32_t pick;
};

// Workgroup-uniform values kept in scalar registers.
__device__ __forceinline__ double uniform(double v) {
    return __hiloint2double(__builtin_amdgcn_readfirstlane(__double2hiint(v)),
                            __builtin_amdgcn_readfirstlane(__double2loint(v)));
}
__device__ __forceinline__ float uniform(float v) {
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

template <bool VEC>
__device__ __forceinline__ void floor_by_window(const FloorParams& a, const RowRef& r0, WinShared& ws, float& m_out,
                                                float& fl_out, double& z_out) {
    const int t = threadIdx.x;
    const bool use_k = a.top_k > 0 && a.top_k < a.V;
    const bool use_p = a.top_p < 1.0;
    constexpr int kHold = 12;   // vectors per thread held in registers (more spill)
    u32x4 raw[kHold];
#pragma unroll
    for (int u = 0; u < kHold; ++u) raw[u] = load_raw<kBF16, VEC, true>(r0.row, r0.V, r0.NV, t + u * kFT);
    // Every 32-bit word of this thread's vectors (two bf16 logits; rows on
    // this path have whole vectors): registers, then the rest re-read.
    auto each_word = [&](auto&& f) {
#pragma unroll
        for (int u = 0; u < kHold; ++u) asm volatile("" : "+v"(raw[u]));
#pragma unroll
        for (int u = 0; u < kHold; ++u) {
            if (t + u * kFT >= r0.NV) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) f(raw[u][q]);
        }
        tail_batches(r0, t + kHold * kFT, [&](const u32x4& rv) {
#pragma unroll
            for (int q = 0; q < 4; ++q) f(rv[q]);
        });
    };
    float m = -INFINITY;
    each_word([&](uint32_t w) { m = fmaxf(m, fmaxf(__uint_as_float(w << 16), __uint_as_float(w & 0xFFFF0000u))); });
    m = uniform(wg_max(m, ws.red_f));
    const float M = offset_of(m, r0.sc);
    const uint32_t kmax = key16_of(__float_as_uint(m) >> 16);
    auto sum_d = [&](double v) {
        return uniform(wg_sum(v, ws.red_d));
    };

    // Window [k0, khi): this thread's 4 bins (keys k0 + 4 t + j) as counts
    // and masses; with `below`, also the mass of the keys under k0.
    uint32_t c[kWinPerThread];
    double mb[kWinPerThread];
    // klow: the lowest key whose mass exceeds 2^-kFirstDeficit of the max's
    // (the exponent is monotone in the key; the keys under -inf's are NaNs
    // and fail the test).
    uint32_t klow = 1;
    for (uint32_t hi_k = kmax; klow < hi_k;) {
        const uint32_t mid = (klow + hi_k) >> 1;
        if (exponent2(value16_of(mid), M, r0.sc) > -kFirstDeficit)
            hi_k = mid;
        else
            klow = mid + 1;
    }
    uint32_t k0 = 0, khi = kmax + 1;
    auto count_window = [&](bool below) -> double {
        k0 = khi > (uint32_t)kWin ? khi - kWin : 0u;
        if (khi == kmax + 1) k0 = max(k0, klow);                 // the top window
        __syncthreads();
        for (int q = t; q < kWin; q += kFT) ws.win[q] = 0;
        __syncthreads();
        float bm = 0.0f;
        const uint32_t span = khi - k0;
        each_word([&](uint32_t w) {
            // Both keys of the word at once: a negative half is inverted and
            // incremented (no carry leaves it), the other gets its top bit set.
            const uint32_t sgn = (w >> 15) & 0x00010001u;
            const uint32_t keys = (w ^ (sgn * 0x7FFFu | 0x80008000u)) + sgn;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const uint32_t k = half ? (keys >> 16) : (keys & 0xFFFFu);
                if (k - k0 < span) atomicAdd(&ws.win[k - k0], 1u);
            }
        });
        // The mass under the window, when asked for, in a pass of its own:
        // a count-only pass then carries no exponential.  The keys under k0
        // are the values under k0's value (a NaN for k0 < 0x80: none), and
        // one FMA gives the exponent: each of these masses is below 2^-24
        // of the max's, so its few-ulp error is far below the row total's.
        if (below) {
            const float xk0 = value16_of(k0), c1 = (float)r0.sc.c;
            each_word([&](uint32_t w) {
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const float x = __uint_as_float(half ? (w & 0xFFFF0000u) : (w << 16));
                    bm += x < xk0 ? fast_exp2(__fmaf_rn(x, c1, -M)) : 0.0f;
                }
            });
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kWinPerThread; ++j) {
            c[j] = ws.win[kWinPerThread * t + j];
            const uint32_t key = k0 + kWinPerThread * t + j;
            mb[j] = c[j] ? (double)c[j] * (double)fast_exp2(exponent2(value16_of(key), M, r0.sc)) : 0.0;
        }
        return below ? sum_d((double)bm) : 0.0;
    };
    // The crossing of a window: the bin where the weight from the top (with
    // `above` from higher windows) first reaches `target`.
    auto crossing = [&](auto&& wt, double above, double target) -> uint32_t {
        if (t == 0) ws.pick = k0;        // no thread matches only if rounding left
                                         // the target past the window's weight
        double mine = 0.0;
#pragma unroll
        for (int j = 0; j < kWinPerThread; ++j) mine += wt(j);
        const double up = above + sum_above(mine, ws.red_d);
        if (up < target && target <= up + mine) {
            double cum = up;
            for (int j = kWinPerThread - 1; j >= 0; --j) {
                cum += wt(j);
                if (cum >= target) { ws.pick = k0 + kWinPerThread * t + j; break; }
            }
        }
        __syncthreads();
        const uint32_t key = __builtin_amdgcn_readfirstlane(ws.pick);
        __syncthreads();
        return key;
    };
    const uint32_t lo_off = kWinPerThread * t;
    // One loop, one window count per turn: first the top-k search (counts),
    // then the top-p search (survivors' masses), each moving down a window
    // while its cut lies lower.
    int phase = use_k ? 0 : 1;
    bool first = true;
    uint32_t k0_top = 0, kkey = 0, fkey = 0;
    double below0 = 0.0, above_c = 0.0, above_m = 0.0, zsur = 0.0, target = 0.0, above = 0.0, kept = 0.0;
    for (;;) {
        const double b = count_window(first && !use_k);
        if (first) {
            below0 = b;
            k0_top = k0;
            first = false;
        }
        double ct = 0.0, mt = 0.0, ms = 0.0;
#pragma unroll
        for (int j = 0; j < kWinPerThread; ++j) {
            ct += (double)c[j];
            mt += mb[j];
        }
        if (phase == 0) {
            const double cw = sum_d(ct), mw = sum_d(mt);
            if (above_c + cw < (double)a.top_k) {             // the cut lies lower
                above_c += cw;
                above_m += mw;
                khi = k0;
                continue;
            }
            kkey = crossing([&](int j) { return (double)c[j]; }, above_c, (double)a.top_k);
#pragma unroll
            for (int j = 0; j < kWinPerThread; ++j)
                if (k0 + lo_off + j >= kkey) ms += mb[j];
            zsur = above_m + sum_d(ms);
            fkey = kkey;
            kept = zsur;
            if (!use_p) break;
            phase = 1;
            target = a.top_p * zsur;
            if (k0 != k0_top) {                                 // search top-p from the top again
                khi = kmax + 1;
                continue;
            }
        } else if (!use_k && k0 == k0_top && above == 0.0 && zsur == 0.0) {
            // No top-k: the survivors are the whole row.
            zsur = sum_d(mt) + below0;
            fkey = 0;
            kept = zsur;
            if (!use_p) break;
            target = a.top_p * zsur;
        }
        // phase 1: the survivors' mass in this window.
        double mine = 0.0;
#pragma unroll
        for (int j = 0; j < kWinPerThread; ++j)
            if (k0 + lo_off + j >= kkey) mine += mb[j];
        const double mw = sum_d(mine);
        if (above + mw < target && k0 > kkey && k0 > 0) {
            above += mw;
            khi = k0;
            continue;
        }
        fkey = crossing([&](int j) { return (k0 + lo_off + j >= kkey) ? mb[j] : 0.0; }, above, target);
        double kp = 0.0;
#pragma unroll
        for (int j = 0; j < kWinPerThread; ++j)
            if (k0 + lo_off + j >= fkey) kp += mb[j];
        kept = above + sum_d(kp);
        break;
    }
    const bool cut = use_k || use_p;
    fl_out = cut ? value16_of(fkey) : -INFINITY;
    m_out = m;
    z_out = kept;
}

// fp32 rows (16-byte aligned): windows of 4,096 bins over the mass
// exponent.  The deficit D(x) = M - x * c is monotone in x, so bins of
// equal width in D (64 per binade of mass, a window spanning 64 binades
// below its top value) split the row into ranges of the value order, with
// equal logits always in one bin.  Each bin holds its count and the exact
// fixed-point sum of its elements' masses, so every weight below is an
// exact multiple of 2^-35 and the crossings are exact.  The first window
// starts at the row max; a window count also finds the largest logit below
// it, where the next window starts, so empty value ranges cost nothing.
// The first window's count also keeps in LDS the logits of its top 16
// binades (when they fit), which usually hold both cuts.
// A cut found in a bin is resolved to the exact key over the logits of the
// bin (or, when all top-k survivors fit, over all of them) in a selection
// set in LDS: taken from the kept logits, else gathered by one more pass
// over the row.  Up to 256 are ranked directly (every element counts the
// weight above it); more go through 8-bit digit selection from the first
// digit in which their keys differ.  A bin too large for the set is
// resolved by four digit passes over the row.  Histogram updates of a wave
// whose matching lanes share a digit are combined into one atomic pair.
// The thread's first vector stays in registers (more spill).
constexpr int kBinsPerBinade = 64;
constexpr int kKeepFrom = kWin - 16 * kBinsPerBinade;   // first bin of the kept top 16 binades
constexpr int kSet = 2048;                         // selection set capacity
constexpr int kRank = 256;                         // largest set ranked directly

struct Win32Shared {
    uint32_t cnt[kWin];
    uint64_t msum[kWin];
    uint32_t ckey[kCand];               // kept logits of the first window: key,
    uint64_t cmass[kCand];              //   fixed-point mass,
    uint16_t cpos[kCand];               //   bin
    uint32_t skey[kSet];                // selection set: key,
    uint64_t smass[kSet];               //   fixed-point mass
    uint32_t hc[256];
    uint64_t hm[256];
    double red_d[kFW];
    uint32_t red_c[kFW];
    float red_f[kFW];
    uint32_t nkeep;
    uint32_t nset;
    uint32_t pick;
    double pick_above;
    double pick_mass_above;
};

// Number of lanes below this one whose bit is set in mask.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

template <bool VEC>
__device__ __forceinline__ void floor_by_window32(const FloorParams& a, const RowRef& r0, Win32Shared& ws,
                                                  float& m_out, float& fl_out, double& z_out) {
    const int t = threadIdx.x;
    const int lane = t & 63;
    const bool use_k = a.top_k > 0 && a.top_k < a.V;
    const bool use_p = a.top_p < 1.0;
    constexpr int kHold = 1;
    u32x4 raw[kHold];
#pragma unroll
    for (int u = 0; u < kHold; ++u) raw[u] = load_raw<kFP32, VEC, true>(r0.row, r0.V, r0.NV, t + u * kFT);
    // Every logit of this thread's vectors (whole vectors on this path):
    // registers, then the rest re-read.
    auto each = [&](auto&& f) {
#pragma unroll
        for (int u = 0; u < kHold; ++u) asm volatile("" : "+v"(raw[u]));
#pragma unroll
        for (int u = 0; u < kHold; ++u) {
            if (t + u * kFT >= r0.NV) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) f(__uint_as_float(raw[u][q]));
        }
        tail_batches(r0, t + kHold * kFT, [&](const u32x4& rv) {
#pragma unroll
            for (int q = 0; q < 4; ++q) f(__uint_as_float(rv[q]));
        });
    };
    float m = -INFINITY;
    each([&](float x) { m = fmaxf(m, x); });
    m = uniform(wg_max(m, ws.red_f));
    const float M = offset_of(m, r0.sc);
    auto sum_d = [&](double v) {
        return uniform(wg_sum(v, ws.red_d));
    };
    auto deficit = [&](float x) { return -exponent2(x, M, r0.sc); };
    auto mass = [&](float x) { return fix_of(fast_exp2(exponent2(x, M, r0.sc))); };

    // The window: top value hi (its deficit Dh).  pos(x): x's bin 0..4095
    // (higher = larger logits), -1 above the window (or NaN), -2 below.
    float hi = m, Dh = deficit(m);
    bool top_window = true;
    auto pos = [&](float x) -> int {
        if (!(x <= hi)) return -1;
        const float q = (deficit(x) - Dh) * (float)kBinsPerBinade;
        return q < (float)kWin ? kWin - 1 - (int)q : -2;
    };
    // Append the logits with g set (one atomic per wave places a wave's
    // matches) to LDS arrays with counter n; f(i, x) stores entry i < cap.
    auto append = [&](bool g, uint32_t& n, uint32_t cap, auto&& f) {
        const uint64_t mask = __ballot(g);
        if (mask) {
            const int leader = __ffsll((unsigned long long)mask) - 1;
            uint32_t base = 0;
            if (lane == leader) base = atomicAdd(&n, (uint32_t)__popcll(mask));
            base = __shfl(base, leader, 64);
            const uint32_t i = base + lanes_below(mask);
            if (g && i < cap) f(i);
        }
    };

    // This thread's 4 bins (4 t + j) as counts and masses; `next` = 1 + the
    // key of the largest logit below the window (0: none); with `below`,
    // the returned value is the fp32 mass below the window; with `keep`,
    // the logits of bins >= kKeepFrom go to the kept arrays.
    uint32_t c[kWinPerThread];
    double mb[kWinPerThread];
    uint32_t next = 0;
    auto count_window = [&](bool below, bool keep) -> double {
        __syncthreads();
        for (int q = t; q < kWin; q += kFT) {
            ws.cnt[q] = 0;
            ws.msum[q] = 0;
        }
        if (t == 0 && keep) ws.nkeep = 0;
        __syncthreads();
        float bm = 0.0f;
        uint32_t nb = 0;
        each([&](float x) {
            const int p = pos(x);
            uint64_t fm = 0;
            if (p >= 0) {
                fm = mass(x);
                atomicAdd(&ws.cnt[p], 1u);
                atomicAdd(reinterpret_cast<unsigned long long*>(&ws.msum[p]), (unsigned long long)fm);
            } else if (p == -2) {
                nb = max(nb, key_of(x) + 1u);
                if (below) bm += fast_exp2(exponent2(x, M, r0.sc));
            }
            if (keep)
                append(p >= kKeepFrom, ws.nkeep, kCand, [&](uint32_t i) {
                    ws.ckey[i] = key_of(x);
                    ws.cmass[i] = fm;
                    ws.cpos[i] = (uint16_t)p;
                });
        });
        next = __builtin_amdgcn_readfirstlane(wg_reduce(nb, ws.red_c, [](uint32_t p, uint32_t q) { return max(p, q); }));
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kWinPerThread; ++j) {
            c[j] = ws.cnt[kWinPerThread * t + j];
            mb[j] = (double)ws.msum[kWinPerThread * t + j] / kFix;
        }
        return below ? sum_d((double)bm) : 0.0;
    };
    // A finite window below this one?  Then move to it.
    auto lower = [&]() -> bool {
        if (next == 0 || value_of(next - 1u) == -INFINITY) return false;
        hi = value_of(next - 1u);
        Dh = deficit(hi);
        top_window = false;
        return true;
    };
    // The bin where the weight from the top (with `above` from higher
    // windows) first reaches `target`; `up` gets the weight above that bin.
    auto crossing = [&](auto&& wt, double above, double target, double& up) -> int {
        if (t == 0) {
            ws.pick = 0;
            ws.pick_above = 0.0;
        }
        double mine = 0.0;
#pragma unroll
        for (int j = 0; j < kWinPerThread; ++j) mine += wt(j);
        const double u = above + sum_above(mine, ws.red_d);
        if (u < target && target <= u + mine) {
            double cum = u;
            for (int j = kWinPerThread - 1; j >= 0; --j) {
                const double w = wt(j);
                if (cum + w >= target) {
                    ws.pick = kWinPerThread * t + j;
                    ws.pick_above = cum;
                    break;
                }
                cum += w;
            }
        }
        __syncthreads();
        const int p = (int)__builtin_amdgcn_readfirstlane(ws.pick);
        up = uniform(ws.pick_above);
        __syncthreads();
        return p;
    };

    // The selection set: from the kept logits whose bin passes sel(p), or
    // from the row's logits with in(x).  shift0 / prefix: the first 8-bit
    // digit in which the set's keys differ and the bits above it.
    int shift0 = 24;
    uint32_t prefix = 0;
    auto set_done = [&](uint32_t kmn, uint32_t kmx) {
        kmn = __builtin_amdgcn_readfirstlane(wg_reduce(kmn, ws.red_c, [](uint32_t p, uint32_t q) { return min(p, q); }));
        kmx = __builtin_amdgcn_readfirstlane(wg_reduce(kmx, ws.red_c, [](uint32_t p, uint32_t q) { return max(p, q); }));
        const uint32_t diff = kmn ^ kmx;
        shift0 = diff ? (31 - __builtin_clz(diff)) / 8 * 8 : 0;
        prefix = shift0 >= 24 ? 0u : kmx >> (shift0 + 8);
    };
    auto set_from_kept = [&](auto&& sel) {
        __syncthreads();
        if (t == 0) ws.nset = 0;
        __syncthreads();
        uint32_t kmn = 0xFFFFFFFFu, kmx = 0;
        const uint32_t nk = min(__builtin_amdgcn_readfirstlane(ws.nkeep), (uint32_t)kCand);
        for (uint32_t i0 = 0; i0 < nk; i0 += kFT) {                 // every lane runs every turn
            const uint32_t i = i0 + t;
            const bool g = i < nk && sel((int)ws.cpos[i]);
            const uint32_t k = g ? ws.ckey[i] : 0u;
            if (g) {
                kmn = min(kmn, k);
                kmx = max(kmx, k);
            }
            append(g, ws.nset, kSet, [&](uint32_t o) {
                ws.skey[o] = k;
                ws.smass[o] = ws.cmass[i];
            });
        }
        set_done(kmn, kmx);
    };
    auto set_from_row = [&](auto&& in) {
        __syncthreads();
        if (t == 0) ws.nset = 0;
        __syncthreads();
        uint32_t kmn = 0xFFFFFFFFu, kmx = 0;
        each([&](float x) {
            const bool g = in(x);
            const uint32_t k = key_of(x);
            if (g) {
                kmn = min(kmn, k);
                kmx = max(kmx, k);
            }
            append(g, ws.nset, kSet, [&](uint32_t o) {
                ws.skey[o] = k;
                ws.smass[o] = mass(x);
            });
        });
        set_done(kmn, kmx);
    };
    // Digit histograms (counts, masses) of the keys >= kmin whose bits above
    // the digit at `shift` are `hb` (all keys at shift 24): over the set, or
    // over the row's logits with in(x).
    auto hist_clear = [&]() {
        __syncthreads();
        if (t < 256) {
            ws.hc[t] = 0;
            ws.hm[t] = 0;
        }
        if (t == 0) {
            ws.pick = 0;
            ws.pick_above = 0.0;
            ws.pick_mass_above = 0.0;
        }
        __syncthreads();
    };
    auto hist_set = [&](int shift, uint32_t hb, uint32_t kmin) {
        hist_clear();
        const uint32_t n = min(__builtin_amdgcn_readfirstlane(ws.nset), (uint32_t)kSet);
        for (uint32_t i0 = 0; i0 < n; i0 += kFT) {                   // every lane runs every turn
            const uint32_t i = i0 + t;
            const uint32_t k = i < n ? ws.skey[i] : 0u;
            const bool g = i < n && (shift == 24 || (k >> (shift + 8)) == hb) && k >= kmin;
            const uint32_t d = (k >> shift) & 255u;
            const uint64_t q = g ? ws.smass[i] : 0ull;
            const uint64_t mask = __ballot(g);
            if (!mask) continue;
            const int leader = __ffsll((unsigned long long)mask) - 1;
            const uint32_t dl = __shfl(d, leader, 64);
            if (__all(!g || d == dl)) {
                uint64_t sq = q;
#pragma unroll
                for (int o = 32; o > 0; o >>= 1) sq += __shfl_xor(sq, o, 64);
                if (lane == leader) {
                    atomicAdd(&ws.hc[dl], (uint32_t)__popcll(mask));
                    atomicAdd(reinterpret_cast<unsigned long long*>(&ws.hm[dl]), (unsigned long long)sq);
                }
            } else if (g) {
                atomicAdd(&ws.hc[d], 1u);
                atomicAdd(reinterpret_cast<unsigned long long*>(&ws.hm[d]), (unsigned long long)q);
            }
        }
        __syncthreads();
    };
    auto hist_row = [&](auto&& in, int shift, uint32_t hb, uint32_t kmin) {
        hist_clear();
        each([&](float x) {
            const uint32_t k = key_of(x);
            if (in(x) && (shift == 24 || (k >> (shift + 8)) == hb) && k >= kmin) {
                const uint32_t d = (k >> shift) & 255u;
                atomicAdd(&ws.hc[d], 1u);
                atomicAdd(reinterpret_cast<unsigned long long*>(&ws.hm[d]), (unsigned long long)mass(x));
            }
        });
        __syncthreads();
    };
    // The digit where the weight (masses, else counts) from the top reaches
    // `target`; `up` gets the weight above it and `mup` the mass above it.
    auto digit_pick = [&](bool masses, double target, double& up, double& mup) -> uint32_t {
        const double hm = (t < 256) ? (double)ws.hm[t] / kFix : 0.0;
        const double w = (t < 256) ? (masses ? hm : (double)ws.hc[t]) : 0.0;
        const double u = sum_above(w, ws.red_d);
        const double mu = sum_above(hm, ws.red_d);
        if (t < 256 && u < target && target <= u + w) {
            ws.pick = t;
            ws.pick_above = u;
            ws.pick_mass_above = mu;
        }
        __syncthreads();
        const uint32_t d = __builtin_amdgcn_readfirstlane(ws.pick);
        up = uniform(ws.pick_above);
        mup = uniform(ws.pick_mass_above);
        __syncthreads();
        return d;
    };
    // The exact key (bits above shift + 8 equal to hb) where the weight of
    // the keys >= kmin from the top reaches `target`; `mass_ge` gets the mass
    // of those keys at or above it.  fill(shift, hb, kmin) builds a level.
    auto radix = [&](auto&& fill, int top_shift, uint32_t hb, uint32_t kmin, bool masses, double target,
                     double& mass_ge) -> uint32_t {
        uint32_t key = hb;
        double mu_sum = 0.0;
        for (int sh = top_shift; sh >= 0; sh -= 8) {
            fill(sh, key, kmin);
            double up, mup;
            const uint32_t d = digit_pick(masses, target, up, mup);
            key = (key << 8) | d;
            target -= up;
            mu_sum += mup;
        }
        mass_ge = mu_sum + uniform((double)ws.hm[key & 255u] / kFix);
        return key;
    };
    // The same over the selection set: a small set by ranking (each
    // element sums the weight of the keys above it and equal to it), a
    // larger one by digits.
    auto select = [&](uint32_t kmin, bool masses, double target, double& mass_ge) -> uint32_t {
        const uint32_t n = min(__builtin_amdgcn_readfirstlane(ws.nset), (uint32_t)kSet);
        if (n > (uint32_t)kRank)
            return radix([&](int sh, uint32_t hb, uint32_t km) { hist_set(sh, hb, km); }, shift0, prefix, kmin,
                         masses, target, mass_ge);
        __syncthreads();
        if (t == 0) {
            ws.pick = 0;
            ws.pick_mass_above = 0.0;
        }
        __syncthreads();
        if ((uint32_t)t < n) {
            const uint32_t key = ws.skey[t];
            if (key >= kmin) {
                uint32_t gc = 0, ec = 0;
                uint64_t gm = 0, em = 0;
                for (uint32_t j = 0; j < n; ++j) {
                    const uint32_t kj = ws.skey[j];
                    const uint64_t mj = ws.smass[j];
                    if (kj > key) {
                        ++gc;
                        gm += mj;
                    } else if (kj == key) {
                        ++ec;
                        em += mj;
                    }
                }
                const double wg = masses ? (double)gm / kFix : (double)gc;
                const double we = masses ? (double)(gm + em) / kFix : (double)(gc + ec);
                if (wg < target && target <= we) {                    // equal keys write equal values
                    ws.pick = key;
                    ws.pick_mass_above = (double)(gm + em) / kFix;
                }
            }
        }
        __syncthreads();
        const uint32_t key = __builtin_amdgcn_readfirstlane(ws.pick);
        mass_ge = uniform(ws.pick_mass_above);
        __syncthreads();
        return key;
    };
    // kept: the kept arrays are this (top) window's logits of bins >=
    // kKeepFrom, all of them.
    bool kept_ok = false;
    // The cut inside bin p (n logits) of the current window.
    auto resolve = [&](int p, uint32_t n, uint32_t kmin, bool masses, double target, double& mass_ge) -> uint32_t {
        auto in_bin = [&](float x) { return pos(x) == p; };
        if (n <= (uint32_t)kSet) {
            if (kept_ok && top_window && p >= kKeepFrom)
                set_from_kept([&](int q) { return q == p; });
            else
                set_from_row(in_bin);
            return select(kmin, masses, target, mass_ge);
        }
        return radix([&](int sh, uint32_t hb, uint32_t km) { hist_row(in_bin, sh, hb, km); }, 24, 0u, kmin,
                     masses, target, mass_ge);
    };

    // As for bf16: first the top-k search (counts), then the top-p search
    // (survivors' masses), each moving down a window while its cut lies
    // lower.  The top-k cut kkey lies in bin pk of the window with top bk_hi;
    // of that bin only the keys >= kkey survive (mass part_bk).
    const int lo_off = kWinPerThread * t;
    int phase = use_k ? 0 : 1;
    bool first = true;
    int pk = 0;
    float bk_hi = INFINITY;
    uint32_t kkey = 0, fkey = 0;
    double below0 = 0.0, above_c = 0.0, above_m = 0.0, zsur = 0.0, target = 0.0, above = 0.0, kept = 0.0;
    double part_bk = 0.0;
    for (;;) {
        const double b = count_window(first && !use_k, first);
        if (first) {
            below0 = b;
            first = false;
            kept_ok = __builtin_amdgcn_readfirstlane(ws.nkeep) <= (uint32_t)kCand;
        }
        double ct = 0.0, mt = 0.0;
#pragma unroll
        for (int j = 0; j < kWinPerThread; ++j) {
            ct += (double)c[j];
            mt += mb[j];
        }
        if (phase == 0) {
            const double cw = sum_d(ct), mw = sum_d(mt);
            if (above_c + cw < (double)a.top_k) {                     // the cut lies lower
                above_c += cw;
                above_m += mw;
                if (lower()) continue;
                // Only -inf logits (or none) remain: the cut keeps them all.
                kkey = key_of(-INFINITY);
                bk_hi = -INFINITY;
                zsur = above_m;
                fkey = kkey;
                kept = zsur;
                if (!use_p) break;
                phase = 1;
                target = a.top_p * zsur;
                hi = m;
                Dh = deficit(m);
                top_window = true;
                continue;
            }
            double upc;
            pk = crossing([&](int j) { return (double)c[j]; }, above_c, (double)a.top_k, upc);
            const uint32_t nbk = __builtin_amdgcn_readfirstlane(ws.cnt[pk]);
            if (use_p && upc + nbk <= (double)kSet) {
                // Every survivor lies above the window or in its bins >= pk.
                if (kept_ok && top_window && pk >= kKeepFrom)
                    set_from_kept([&](int q) { return q >= pk; });
                else
                    set_from_row([&](float x) { return x > hi || pos(x) >= pk; });
                kkey = select(0u, false, (double)a.top_k, zsur);
                fkey = select(kkey, true, a.top_p * zsur, kept);
                break;
            }
            kkey = resolve(pk, nbk, 0u, false, (double)a.top_k - upc, part_bk);
            double hi_mass = 0.0;
#pragma unroll
            for (int j = 0; j < kWinPerThread; ++j)
                if (lo_off + j > pk) hi_mass += mb[j];
            zsur = above_m + sum_d(hi_mass) + part_bk;
            fkey = kkey;
            kept = zsur;
            bk_hi = hi;
            if (!use_p) break;
            phase = 1;
            target = a.top_p * zsur;
            if (!top_window) {                                        // search top-p from the top again
                hi = m;
                Dh = deficit(m);
                top_window = true;
                continue;
            }
        } else if (!use_k && top_window && above == 0.0 && zsur == 0.0) {
            // No top-k: the survivors are the whole row.
            zsur = sum_d(mt) + below0;
            kept = zsur;
            if (!use_p) break;
            target = a.top_p * zsur;
        }
        // phase 1: the survivors' masses (windows above bk_hi whole; in
        // that window, bins above pk whole and pk in part).
        const bool whole = !use_k || hi > bk_hi;
        auto sur = [&](int j) -> double {
            if (whole) return mb[j];
            const int p = lo_off + j;
            return p > pk ? mb[j] : (p == pk ? part_bk : 0.0);
        };
        double mine = 0.0;
#pragma unroll
        for (int j = 0; j < kWinPerThread; ++j) mine += sur(j);
        const double mw = sum_d(mine);
        if (above + mw < target && whole) {
            if (lower()) {
                above += mw;
                continue;
            }
            // The row's last window and still short of the target (masses
            // below the fixed-point step round to zero): keep every survivor.
            fkey = use_k ? kkey : key_of(-INFINITY);
            kept = above + mw;
            break;
        }
        double upm, mass_ge;
        const int pp = crossing(sur, above, target, upm);
        fkey = resolve(pp, __builtin_amdgcn_readfirstlane(ws.cnt[pp]), (!whole && pp == pk) ? kkey : 0u, true,
                       target - upm, mass_ge);
        kept = upm + mass_ge;
        break;
    }
    const bool cut = use_k || use_p;
    fl_out = cut ? value_of(fkey) : -INFINITY;
    m_out = m;
    z_out = kept;
}

// ---------------------------------------------------------------------------
// A small top-k (1 <= top_k <= kCandPerTile) on rows of whole 16-byte
// vectors: the cuts from tile candidates, so that no row is read more than
// once.
//
// floor_cands, one workgroup of 256 threads per 16 KB tile (grid: tile, row
// slot, request, as the verify row pass), leaves the tile's largest logits:
//   bf16: one bin per key for the 256 keys from the tile's largest down, so
//         a bin is one value; the entries are (key, count) of the nonzero
//         bins from the top down to the bin where the count reaches top_k;
//   fp32: 256 bins over the mass exponent below the tile's largest logit, 8
//         per binade (monotone in the logit: equal logits share a bin); the
//         entries are the logits of the bins down to the one where the count
//         reaches top_k.
// The entries stop one bin early where kCandPerTile would overflow.  The
// head holds the tile's largest key; L, the smallest key such that every
// logit of the tile with key >= L is an entry; the number of entries; and G,
// a key at or below the tile's own top_k-th largest (0 when the window holds
// fewer than top_k logits).
//
// The merge (merge_row, in floor_merge or floor_finish) takes each row's
// entries.  The row's top_k-th largest K* is at least every tile's own, so
// at least G of every tile: entries below the largest G are dropped.  The
// top_k-th largest of the rest is the row's when it is >= L of every tile
// (each tile then holds all its logits >= it, so every count from the top
// down to it is the row's), and then every top-k survivor is an entry, so
// the top-p cut over the survivors comes from the entries too.  Otherwise
// (the cut lies below some tile's entries, or a bin's entries overflow the
// LDS list) the row is left to the full-row path.  The row max is the
// largest head key.
// ---------------------------------------------------------------------------
constexpr int kCandBins = kThreads;             // one bin per thread of floor_cands
constexpr float kCandBinsPerBinade = 8.0f;      // fp32: bins over the mass exponent

// Inclusive prefix sum, min and max of a u32 over the wave (DPP: rows of
// 16 lanes, then the row broadcasts; min and max in every lane).
__device__ __forceinline__ uint32_t wave_incl_u32(uint32_t v) {
    int x = (int)v;
    x += dpp<kDppRowShr1>(x, 0);
    x += dpp<kDppRowShr2>(x, 0);
    x += dpp<kDppRowShr4>(x, 0);
    x += dpp<kDppRowShr8>(x, 0);
    x += dpp<kDppRowBcast15, 0xA>(x, 0);
    x += dpp<kDppRowBcast31, 0xC>(x, 0);
    return (uint32_t)x;
}
template <bool MAX>
__device__ __forceinline__ uint32_t wave_ext_u32(uint32_t v) {
    constexpr int id = MAX ? 0 : -1;
    auto f = [](uint32_t p, int q) { return MAX ? max(p, (uint32_t)q) : min(p, (uint32_t)q); };
    v = f(v, dpp<kDppQuad1032>((int)v, id));
    v = f(v, dpp<kDppQuad2301>((int)v, id));
    v = f(v, dpp<kDppRowHalfMirror>((int)v, id));
    v = f(v, dpp<kDppRowMirror>((int)v, id));
    v = f(v, dpp<kDppRowBcast15, 0xA>((int)v, id));
    v = f(v, dpp<kDppRowBcast31, 0xC>((int)v, id));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
// Exact sum of a u64 over the wave, in every lane: the same DPP steps on
// both halves, the 64-bit add carrying between them (the lanes a row mask
// leaves out add 0).
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, ROWS, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, ROWS, 0xF, false);
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_total_u64(uint64_t v) {
    v += dpp_u64<kDppQuad1032>(v);
    v += dpp_u64<kDppQuad2301>(v);
    v += dpp_u64<kDppRowHalfMirror>(v);
    v += dpp_u64<kDppRowMirror>(v);
    v += dpp_u64<kDppRowBcast15, 0xA>(v);
    v += dpp_u64<kDppRowBcast31, 0xC>(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) { return wave_ext_u32<false>(v); }
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) { return wave_ext_u32<true>(v); }

template <int DT>
__global__ __launch_bounds__(kThreads) void floor_cands(FloorParams a) {
    constexpr int E = Elem<DT>::E;
    static_assert(kCandBins == kThreads && kWaves == 4, "one bin per thread");
    __shared__ uint32_t hist[kCandBins];
    __shared__ float red_f[kWaves];
    __shared__ uint32_t sel[4];                           // b_emit, b*, then fp32: L, G
    __shared__ uint32_t nout;
    const int tile = blockIdx.x, rr = blockIdx.y, b = blockIdx.z;
    const int K = a.K;
    const int kb = a.kpr ? min(max(a.kpr[b], 0), K) : K;
    const bool draft = rr > K;
    const int i = draft ? rr - K - 1 : rr;
    if (draft ? i >= kb : i > kb) return;                // row past k_b
    const size_t ri = draft ? (size_t)b * K + i : (size_t)b * (K + 1) + i;
    const void* row = static_cast<const char*>(draft ? a.draft : a.target) + ri * (size_t)a.V * Elem<DT>::S;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    u32x4 raw[kUnroll];
    tile_load<DT, true, true>(row, a.V, a.NV, tile, raw);
    hist[t] = 0u;
    if (t == 0) {
        nout = 0u;
        sel[2] = 0xFFFFFFFFu;
        sel[3] = 0xFFFFFFFFu;
    }
    // Vectors past the row end were read as -inf: they add nothing to the
    // max and lie below every window.
    float xm = -INFINITY;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        float x[E];
        decode<DT>(raw[u], x);
#pragma unroll
        for (int e = 0; e < E; ++e) xm = fmaxf(xm, x[e]);
    }
    xm = block_max(xm, red_f);
    uint32_t km;
    float M = 0.0f, Dh = 0.0f, xlo = -INFINITY;
    if constexpr (DT == kBF16) {
        km = key16_of(__float_as_uint(xm) >> 16);
        // The window's smallest value (keys below 0x80 are NaNs: none).
        if (km >= 0x0080u + (uint32_t)(kCandBins - 1)) xlo = value16_of(km - (uint32_t)(kCandBins - 1));
    } else {
        km = key_of(xm);
        M = offset_of(xm, a.sc);
        Dh = -exponent2(xm, M, a.sc);
    }
    // fp32: bin of a logit, 0 (the largest) to 255, -1 outside the window
    // (-inf gives +inf, or NaN when the largest is -inf: outside).  bf16
    // bins are km - key, inside the window x >= xlo.
    auto bin_of = [&](float x) -> int {
        const float q = (-exponent2(x, M, a.sc) - Dh) * kCandBinsPerBinade;
        return q < (float)kCandBins ? (int)q : -1;
    };
    if (DT == kBF16 && xlo > 0.0f) {
        // A window of positive values: the bin of the 16-bit pattern h is
        // hm - h, and every pattern outside the window (smaller, negative,
        // -inf past the row end, or NaN) gives a difference above 255 as an
        // unsigned number.
        const uint32_t hm = km & 0x7FFFu;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t d0 = hm - (raw[u][q] & 0xFFFFu);
                const uint32_t d1 = hm - (raw[u][q] >> 16);
                if (d0 < (uint32_t)kCandBins) atomicAdd(&hist[d0], 1u);
                if (d1 < (uint32_t)kCandBins) atomicAdd(&hist[d1], 1u);
            }
    } else {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            float x[E];
            decode<DT>(raw[u], x);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                if constexpr (DT == kBF16) {
                    // The key of every logit (branch-free), the atomic under
                    // the window test alone.
                    const uint32_t d = km - key16_of(__float_as_uint(x[e]) >> 16);
                    if (x[e] >= xlo) atomicAdd(&hist[d], 1u);
                } else {
                    const int bn = bin_of(x[e]);
                    if (bn >= 0) atomicAdd(&hist[bn], 1u);
                }
            }
        }
    }
    __syncthreads();

    const size_t at = ((size_t)b * a.R + rr) * a.C + tile;
    uint32_t* head = a.cand_head + at * 4;
    uint32_t* ent = a.cand_ent + at * kCandPerTile;
    // Wave 0 alone selects: lane l holds the bins 4l .. 4l + 3.
    if (w == 0) {
        uint32_t c[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) c[q] = hist[4 * lane + q];
        // The counts and the nonzero bins from the top, inclusive, in one
        // 32-bit scan (a tile holds at most 8,192 logits).
        uint32_t pk[4];
        pk[0] = (c[0] << 16) | (c[0] ? 1u : 0u);
#pragma unroll
        for (int q = 1; q < 4; ++q) pk[q] = pk[q - 1] + ((c[q] << 16) | (c[q] ? 1u : 0u));
        const uint32_t before = wave_incl_u32(pk[3]) - pk[3];
        uint32_t cnt_incl[4], nz_incl[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            cnt_incl[q] = (before + pk[q]) >> 16;
            nz_incl[q] = (before + pk[q]) & 0xFFFFu;
        }
        // b*: the first bin where the count from the top reaches top_k.
        int first = -1;
#pragma unroll
        for (int q = 3; q >= 0; --q)
            if (cnt_incl[q] >= (uint32_t)a.top_k) first = 4 * lane + q;
        const uint64_t mr = __ballot(first >= 0);
        const uint32_t bstar =
            mr ? (uint32_t)__builtin_amdgcn_readlane(first, __ffsll((unsigned long long)mr) - 1) : 0xFFFFFFFFu;
        const uint32_t blast = bstar == 0xFFFFFFFFu ? (uint32_t)(kCandBins - 1) : bstar;
        // The emitted bins: a prefix (at most kCandPerTile entries); b_emit is its last.
        int last = -1;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t used = (DT == kBF16) ? nz_incl[q] : cnt_incl[q];
            if ((uint32_t)(4 * lane + q) <= blast && used <= (uint32_t)kCandPerTile) last = 4 * lane + q;
        }
        const uint64_t ml = __ballot(last >= 0);
        const int b_emit = ml ? __builtin_amdgcn_readlane(last, 63 - __clzll((long long)ml)) : -1;
        if constexpr (DT == kBF16) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int bn = 4 * lane + q;
                if (bn <= b_emit && c[q] != 0u) ent[nz_incl[q] - 1] = ((km - (uint32_t)bn) << 16) | c[q];
                if (bn == b_emit) {                       // bin 0 (the largest) always fits
                    head[0] = km;
                    head[1] = km - (uint32_t)bn;
                    head[2] = nz_incl[q];
                    head[3] = bstar == 0xFFFFFFFFu ? 0u : km - bstar;
                }
            }
        } else if (lane == 0) {
            sel[0] = (uint32_t)b_emit;
            sel[1] = bstar;
        }
    }
    if constexpr (DT == kFP32) {
        __syncthreads();
        // The logits of bins <= b_emit (a few: appended one by one), the
        // smallest of them (L), and the smallest logit of bin b* (G).
        const int b_emit = (int)sel[0];
        const uint32_t bstar = sel[1];
        uint32_t lmin = 0xFFFFFFFFu, gmin = 0xFFFFFFFFu;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float x = __uint_as_float(raw[u][e]);
                const int bn = bin_of(x);
                if (bn >= 0 && bn <= b_emit) {
                    const uint32_t key = key_of(x);
                    lmin = min(lmin, key);
                    ent[atomicAdd(&nout, 1u)] = key;
                }
                if (bn >= 0 && (uint32_t)bn == bstar) gmin = min(gmin, key_of(x));
            }
        lmin = wave_min_u32(lmin);
        gmin = wave_min_u32(gmin);
        if (lane == 0) {
            atomicMin(&sel[2], lmin);
            atomicMin(&sel[3], gmin);
        }
        __syncthreads();
        if (t == 0) {
            head[0] = km;
            // A tile of -inf only: nothing at or above key(-inf) + 1.
            head[1] = (xm == -INFINITY) ? km + 1u : sel[2];
            head[2] = nout;
            head[3] = sel[3] == 0xFFFFFFFFu ? 0u : sel[3];
        }
    }
}

// Row slot of this workgroup, and the outputs.
struct RowSlot {
    int b, rr, i, kb;
    bool skip;
    const void* row;
};

template <int DT>
__device__ __forceinline__ RowSlot row_slot_of(const FloorParams& a, int rs) {
    constexpr int S = Elem<DT>::S;
    RowSlot s;
    const int R = a.R, K = a.K;
    s.b = rs / R;
    s.rr = rs - s.b * R;
    s.kb = a.kpr ? min(max(a.kpr[s.b], 0), K) : K;
    const bool draft = s.rr > K;
    s.i = draft ? s.rr - K - 1 : s.rr;
    s.skip = draft ? s.i >= s.kb : s.i > s.kb;
    const size_t row_index = draft ? (size_t)s.b * K + s.i : (size_t)s.b * (K + 1) + s.i;
    s.row = static_cast<const char*>(draft ? a.draft : a.target) + row_index * (size_t)a.V * S;
    return s;
}
template <int DT>
__device__ __forceinline__ RowSlot row_slot(const FloorParams& a) {
    return row_slot_of<DT>(a, blockIdx.x);
}

__host__ __device__ __forceinline__ bool cands_usable(const FloorParams& a) {
    return a.cand_head != nullptr && a.top_k >= 1 && a.top_k <= kCandPerTile && a.top_k < a.V;
}

// The floor; for the verify step the processed row's slots: tile 0 holds
// the row max and the kept mass, the other tiles are empty; the logit at
// the draft token (-inf when cut); row 0 empties the request's slab and
// final-tile slots.
template <int DT>
__device__ __forceinline__ void write_outputs(const FloorParams& a, const RowSlot& s, float m, float fl, double z,
                                              int t = threadIdx.x, int stride = kFT, bool have_l = false,
                                              float l_in = 0.0f) {
    const size_t rs = (size_t)s.b * a.R + s.rr;
    if (t == 0) a.floors[rs] = fl;
    if (!a.slot_m) return;
    const int C = a.C;
    for (int c = t; c < C; c += stride) {
        slot_put(a.slot_m + rs * C + c, enc_f32(c == 0 ? m : -INFINITY));
        slot_put(a.slot_s + rs * C + c, enc_f64(c == 0 ? z : 0.0));
    }
    if (t == 0 && s.i < s.kb && a.tokens) {
        float l = l_in;
        if (!have_l) l = load_one<DT>(s.row, min(max(a.tokens[(size_t)s.b * a.K + s.i], 0), a.V - 1));
        slot_put(a.slot_l + rs, enc_f32(l >= fl ? l : -INFINITY));
    }
    if (s.rr == 0) {
        for (int c = t; c < C * kSlabsPerTile; c += stride)
            slot_put(a.slot_slab + (size_t)s.b * C * kSlabsPerTile + c, (uint64_t)0);
        for (int c = t; c < C; c += stride) slot_put(a.slot_tile + (size_t)s.b * C + c, (uint64_t)0);
    }
}

// The merge of one row of a small top-k (see floor_cands), by a group of
// four waves (256 threads, t the thread within the group).  Wave w takes the
// row's tiles w, w + 4, w + 8, ...; lane l holds entry l of each of them, in
// registers.  One histogram over 256 bins from the row's largest key down,
// shared by the waves, decides both cuts: bf16 bins are exact keys (every
// kept entry lies within 256 keys of the largest: the tile that holds it
// keeps its own top_k within its window); fp32 bins are the mass exponent at
// 8 per binade, and the bin holding a cut is resolved exactly by ranking its
// few entries.  Every wave reads the whole histogram and takes the same
// decisions.  A decided row gets its outputs here; a row left undecided goes
// to the full-row path.  The workgroup barriers are the same for every row
// (none depends on the row's data), so several groups share a workgroup.
constexpr int kMergeWaves = 4;                  // waves per row
constexpr int kMergeThreads = kMergeWaves * 64;
constexpr int kMergeTiles = 40;                 // tiles of a row the merge takes (more: the full-row path)
constexpr int kMergeHeld = kMergeTiles / kMergeWaves;   // tiles per wave
constexpr int kMergeList = 256;                 // fp32: entries of one bin ranked in LDS

struct MergeShared {
    uint32_t hist[256];
    uint64_t mhist[256];
    uint32_t lkey[kMergeList];
    uint64_t lmass[kMergeList];
    uint32_t nlist[2];                          // listed entries: the top-k bin, the top-p bin
    uint32_t best[2];                           // ranked keys: K*, the top-p cut
    double kept;                                // mass at and above the top-p cut
};

enum : int { kMergeNone = 0, kMergeDecided = 1, kMergeLeft = 2 };   // no row, decided, left

template <int DT>
__device__ __forceinline__ int merge_row(const FloorParams& a, int rs, MergeShared& ms, int t) {
    static_assert(kCandPerTile == 64, "lane l holds entry l of every tile");
    static_assert(kMergeThreads == 256 && kMergeHeld * kMergeWaves == kMergeTiles, "one bin per thread");
    const int lane = t & 63;
    const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
    const int rows = a.B * a.R;
    const int C = a.C;
    // A slot past the last one works on the last (and writes nothing).
    const int rsc = rs < rows ? rs : rows - 1;
    // One batch of loads: k_b (in row_slot_of), the heads (in every wave),
    // entry `lane` of the wave's tiles (checked against the counts
    // afterwards) and the draft token; then (wave 0) the logit at it.
    const size_t at0 = (size_t)rsc * C;
    const uint32_t* head = a.cand_head + at0 * 4;
    const uint32_t* ent = a.cand_ent + at0 * kCandPerTile;
    uint32_t h0 = 0u, h1 = 0u, h2 = 0u, h3 = 0u;
    if (lane < C) {
        h0 = head[4 * lane];
        h1 = head[4 * lane + 1];
        h2 = min(head[4 * lane + 2], (uint32_t)kCandPerTile);
        h3 = head[4 * lane + 3];
    }
    uint32_t ev[kMergeHeld];
#pragma unroll
    for (int j = 0; j < kMergeHeld; ++j) {
        const int c = wv + kMergeWaves * j;
        ev[j] = c < C ? ent[c * kCandPerTile + lane] : 0u;
    }
    const RowSlot s = row_slot_of<DT>(a, rsc);
    // A skipped row (past k_b) holds no candidates: its workspace is stale
    // but read within bounds, and nothing of it is written.
    const bool live = rs < rows && !s.skip;
    const bool gathers = live && wv == 0 && s.i < s.kb && a.tokens;
    const int tok = gathers ? min(max(a.tokens[(size_t)s.b * a.K + s.i], 0), a.V - 1) : 0;
    const float l_tok = gathers ? load_one<DT>(s.row, tok) : 0.0f;
    const uint32_t km = wave_max_u32(h0);
    const uint32_t lmax = wave_max_u32(h1);
    const uint32_t gmax = wave_max_u32(h3);
    auto val = [](uint32_t k) { return (DT == kBF16) ? value16_of(k) : value_of(k); };
    const float mx = val(km);
    const float M = offset_of(mx, a.sc);
    const float Dh = -exponent2(mx, M, a.sc);
    // Bin of a key: 0 (the largest) upward; >= 256 below the histogram.
    auto bin_of = [&](uint32_t k) -> uint32_t {
        if constexpr (DT == kBF16) {
            return km - k;
        } else {
            const float q = (-exponent2(value_of(k), M, a.sc) - Dh) * kCandBinsPerBinade;
            return q < 256.0f ? (uint32_t)(int)q : 256u;
        }
    };
    auto key_at = [&](int j) -> uint32_t { return (DT == kBF16) ? (ev[j] >> 16) : ev[j]; };
    auto cnt_at = [&](int j) -> uint32_t { return (DT == kBF16) ? (ev[j] & 0xFFFFu) : 1u; };
    auto mass_of = [&](uint32_t k) -> uint64_t { return fix_of(fast_exp2(exponent2(val(k), M, a.sc))); };
    // 0 where a tile has no entry `lane`, where it lies below gmax (below
    // every cut), or below the histogram: when the histogram still holds
    // top_k entries, those lie below the cut too; else the row is left to
    // the full-row path.  (The entry count of tile c is lane c of h2.)
#pragma unroll
    for (int j = 0; j < kMergeHeld; ++j) {
        const int c = wv + kMergeWaves * j;
        const uint32_t n = (uint32_t)__builtin_amdgcn_readlane((int)h2, min(c, 63));
        if (c >= C || (uint32_t)lane >= n || key_at(j) < gmax || bin_of(key_at(j)) >= 256u) ev[j] = 0u;
    }
    ms.hist[t] = 0u;
    ms.mhist[t] = 0ull;
    if (t < 2) {
        ms.nlist[t] = 0u;
        ms.best[t] = 0u;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kMergeHeld; ++j)
        if (ev[j] != 0u) atomicAdd(&ms.hist[bin_of(key_at(j))], cnt_at(j));
    __syncthreads();
    // Lane l holds the bins 4l .. 4l + 3 (descending keys); the first bin
    // where a running weight from the top reaches target, and the weight
    // above it (-1 when the bins' weights fall short of target).
    auto crossing = [&](const double (&wb)[4], double target, double& above_out) -> int {
        const double mine = (wb[0] + wb[1]) + (wb[2] + wb[3]);
        double run = wave_inclusive_scan(mine) - mine;          // the lanes before this one
        int pick = -1;
        double pa = 0.0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (pick < 0 && run < target && target <= run + wb[q]) {
                pick = 4 * lane + q;
                pa = run;
            }
            run += wb[q];
        }
        const uint64_t hit = __ballot(pick >= 0);
        if (!hit) return -1;
        const int src = __ffsll((unsigned long long)hit) - 1;
        above_out = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(pa), src),
                                     __builtin_amdgcn_readlane(__double2loint(pa), src));
        return __builtin_amdgcn_readlane(pick, src);
    };
    // The entries of one bin, listed in LDS (slot `which`), the wave's
    // ballot placed at an offset taken by its first lane.
    auto append = [&](int which, bool g, uint32_t key, bool with_mass) {
        const uint64_t mask = __ballot(g);
        if (mask == 0ull) return;
        uint32_t base = 0u;
        if (lane == 0) base = atomicAdd(&ms.nlist[which], (uint32_t)__popcll(mask));
        base = (uint32_t)__builtin_amdgcn_readlane((int)base, 0);
        const uint32_t i = base + lanes_below(mask);
        if (g && i < (uint32_t)kMergeList) {
            ms.lkey[i] = key;
            if (with_mass) ms.lmass[i] = mass_of(key);
        }
    };
    double wc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) wc[q] = (double)ms.hist[4 * lane + q];
    double cabove = 0.0;
    const int kbin = crossing(wc, (double)a.top_k, cabove);
    // ok: the row can still be decided here (uniform over the group; every
    // step below runs either way, so that the barriers stay the same).
    bool ok = live && kbin >= 0;                                // else fewer than top_k in the histogram
    // K*: the bin's key (bf16), or the (top_k - cabove)-th largest key of the
    // bin's entries (fp32).
    uint32_t kstar = 0u;
    if constexpr (DT == kBF16) {
        kstar = km - (uint32_t)kbin;
    } else {
#pragma unroll
        for (int j = 0; j < kMergeHeld; ++j)
            append(0, ok && ev[j] != 0u && bin_of(key_at(j)) == (uint32_t)kbin, key_at(j), false);
        __syncthreads();
        const uint32_t nl = ms.nlist[0];
        ok = ok && nl <= (uint32_t)kMergeList;
        const uint32_t need = (uint32_t)a.top_k - (uint32_t)cabove;
        uint32_t found = 0u;
        for (uint32_t i = t; ok && i < nl; i += kMergeThreads) {
            const uint32_t ki = ms.lkey[i];
            uint32_t gt = 0u, ge = 0u;
            for (uint32_t j = 0; j < nl; ++j) {
                const uint32_t kj = ms.lkey[j];
                gt += kj > ki;
                ge += kj >= ki;
            }
            if (gt < need && need <= ge) found = ki;                  // equal keys find the same
        }
        found = wave_max_u32(found);
        if (lane == 0 && found != 0u) atomicMax(&ms.best[0], found);
        __syncthreads();
        kstar = ms.best[0];
        ok = ok && kstar != 0u;
    }
    ok = ok && kstar >= lmax;                                    // else a tile's entries stop above the cut
    // The survivors' masses per bin (fp32: in bin kbin only keys >= K*).
#pragma unroll
    for (int j = 0; j < kMergeHeld; ++j) {
        if (ok && ev[j] != 0u && key_at(j) >= kstar) {
            const uint32_t k = key_at(j);
            atomicAdd(reinterpret_cast<unsigned long long*>(&ms.mhist[bin_of(k)]),
                      (unsigned long long)((uint64_t)cnt_at(j) * mass_of(k)));
        }
    }
    __syncthreads();
    double wm[4];
    uint64_t zs = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        zs += ms.mhist[4 * lane + q];
        wm[q] = (double)ms.mhist[4 * lane + q];
    }
    zs = wave_total_u64(zs);
    uint32_t fkey = kstar;
    double kept = (double)zs;
    if (a.top_p < 1.0) {
        const double target = a.top_p * (double)zs;
        double mabove = 0.0;
        const int pbin = crossing(wm, target, mabove);
        ok = ok && pbin >= 0;                                    // (top_p > 0 and the largest key's mass make one)
        if constexpr (DT == kBF16) {
            if (ok) {
                fkey = km - (uint32_t)pbin;
                kept = mabove + (double)ms.mhist[pbin];
            }
        } else {
            // The largest key of bin pbin whose weight from the top reaches
            // target: rank the bin's survivors.
#pragma unroll
            for (int j = 0; j < kMergeHeld; ++j)
                append(1, ok && ev[j] != 0u && key_at(j) >= kstar && bin_of(key_at(j)) == (uint32_t)pbin,
                       key_at(j), true);
            __syncthreads();
            const uint32_t nl = ms.nlist[1];
            ok = ok && nl <= (uint32_t)kMergeList;
            uint32_t found = 0u;
            double fkept = 0.0;
            for (uint32_t i = t; ok && i < nl; i += kMergeThreads) {
                const uint32_t ki = ms.lkey[i];
                uint64_t gt = 0, ge = 0;
                for (uint32_t j = 0; j < nl; ++j) {
                    const uint32_t kj = ms.lkey[j];
                    const uint64_t mj = ms.lmass[j];
                    gt += kj > ki ? mj : 0ull;
                    ge += kj >= ki ? mj : 0ull;
                }
                if (mabove + (double)gt < target && target <= mabove + (double)ge && ki >= found) {
                    found = ki;
                    fkept = mabove + (double)ge;
                }
            }
            const uint32_t wbest = wave_max_u32(found);
            if (lane == 0 && wbest != 0u) atomicMax(&ms.best[1], wbest);
            __syncthreads();
            const uint32_t best = ms.best[1];
            ok = ok && best != 0u;
            // Equal keys rank alike: whichever thread found it writes the same mass.
            if (ok && found == best) ms.kept = fkept;
            __syncthreads();
            if (ok) {
                fkey = best;
                kept = ms.kept;
            }
        }
    }
    if (!live) return kMergeNone;
    if (!ok) return kMergeLeft;
    write_outputs<DT>(a, s, mx, val(fkey), kept / kFix, t, kMergeThreads, true, l_tok);
    return kMergeDecided;
}

// floor_merge: one group (workgroup) per row slot; done[row] = 1 for a row
// it decides, 0 for one it leaves to floor_rows.
template <int DT>
__global__ __launch_bounds__(kMergeThreads) void floor_merge(FloorParams a) {
    __shared__ MergeShared ms;
    const int rs = blockIdx.x;
    if (a.C > kMergeTiles) {
        const RowSlot s = row_slot_of<DT>(a, rs);
        if (!s.skip && threadIdx.x == 0) a.cand_done[rs] = 0u;
        return;
    }
    const int st = merge_row<DT>(a, rs, ms, threadIdx.x);
    if (threadIdx.x == 0 && st != kMergeNone) a.cand_done[rs] = st == kMergeDecided ? 1u : 0u;
}

// Shared memory of the full-row path for one row.
template <int DT, bool VEC> struct RowSmem { using type = FloorShared; };
template <> struct RowSmem<kBF16, true> { using type = WinShared; };
template <> struct RowSmem<kFP32, true> { using type = Win32Shared; };

// The floor of one row and its outputs; nv is the row's length in 16-byte
// vectors.
template <int DT, bool VEC>
__device__ __forceinline__ void floor_row(const FloorParams& a, const RowSlot& s, int nv,
                                          typename RowSmem<DT, VEC>::type& sm) {
    RowRef r;
    r.row = s.row;
    r.V = a.V;
    r.NV = nv;
    r.sc = a.sc;
    float m, fl;
    double z;
    if constexpr (DT == kBF16 && VEC) {
        floor_by_window<VEC>(a, r, sm, m, fl, z);
    } else if constexpr (DT == kFP32 && VEC) {
        floor_by_window32<VEC>(a, r, sm, m, fl, z);
    } else {
        // Rows off 16-byte alignment (or of an odd length): the general
        // selection.
        floor_by_select<DT, VEC>(a, r, sm, m, fl, z);
    }
    write_outputs<DT>(a, s, m, fl, z);
}

// The row path for the rows listed in todo[0 .. n) (a workgroup-uniform
// count), one after another.
template <int DT, bool VEC>
__device__ __forceinline__ void floor_listed(const FloorParams& a, const int* todo, int n,
                                             typename RowSmem<DT, VEC>::type& sm) {
    for (int i = 0; i < n; ++i) {
        // The row length made opaque to the compiler, so that the loads'
        // offsets are formed where they are used rather than kept (spilled)
        // across the rows.
        int nv = a.NV;
        asm volatile("" : "+v"(nv));
        floor_row<DT, VEC>(a, row_slot_of<DT>(a, __builtin_amdgcn_readfirstlane(todo[i])),
                           __builtin_amdgcn_readfirstlane(nv), sm);
        __syncthreads();                                  // the shared memory is the next row's
    }
}

// Workgroups of floor_rows after floor_merge: one per compute unit of the
// chip (a workgroup of the full-row path fills one), each taking every
// kRowsGrid-th row slot that the merge left.
constexpr int kRowsGrid = 256;

template <int DT, bool VEC, bool LISTED>
__global__ __launch_bounds__(kFT) void floor_rows(FloorParams a) {
    __shared__ typename RowSmem<DT, VEC>::type sm;
    if constexpr (!LISTED) {
        // One workgroup per row slot.
        const RowSlot s = row_slot<DT>(a);
        if (s.skip) return;
        floor_row<DT, VEC>(a, s, a.NV, sm);
    } else {
        // After floor_merge: the flags of a batch of the workgroup's row
        // slots in one load per thread, then the undecided rows one after
        // another.  The first batch is listed before the loop, so that a
        // workgroup with nothing to do leaves before the row path's set-up.
        __shared__ int todo[kFT];
        __shared__ int ntodo;
        const int rows = a.B * a.R;
        const int step = (int)gridDim.x * kFT;
        auto list = [&](int first) -> int {
            if (threadIdx.x == 0) ntodo = 0;
            __syncthreads();
            const int rs = first + (int)threadIdx.x * (int)gridDim.x;
            if (rs < rows && a.cand_done[rs] == 0u && !row_slot_of<DT>(a, rs).skip)
                todo[atomicAdd(&ntodo, 1)] = rs;
            __syncthreads();
            return __builtin_amdgcn_readfirstlane(ntodo);
        };
        int first = blockIdx.x;
        int n = list(first);
        while (n > 0 || first + step < rows) {
            floor_listed<DT, VEC>(a, todo, n, sm);
            first += step;
            if (first >= rows) break;
            n = list(first);
        }
    }
}

// floor_finish: the merge and the full-row path in one kernel, for a call
// with few row slots (at most kFinishRows per compute unit: one round of
// workgroups).  A workgroup of 1,024 threads merges kFinishRows row slots,
// one per group of four waves, then takes the rows they left with all its
// threads; the merge's shared memory and the row path's overlap.
constexpr int kFinishRows = kFT / kMergeThreads;         // 4
constexpr int kFinishMaxRows = kFinishRows * kRowsGrid;

template <int DT>
union FinishShared {
    MergeShared m[kFinishRows];
    typename RowSmem<DT, true>::type r;
};

template <int DT>
__global__ __launch_bounds__(kFT) void floor_finish(FloorParams a) {
    __shared__ FinishShared<DT> sm;
    __shared__ int todo[kFinishRows];
    __shared__ int ntodo;
    const int g = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kMergeThreads);
    const int tl = (int)threadIdx.x % kMergeThreads;
    const int rs = (int)blockIdx.x * kFinishRows + g;
    const int rows = a.B * a.R;
    if (threadIdx.x == 0) ntodo = 0;
    __syncthreads();
    int st;
    if (a.C <= kMergeTiles) {
        st = merge_row<DT>(a, rs, sm.m[g], tl);
    } else {
        st = (rs < rows && !row_slot_of<DT>(a, rs).skip) ? kMergeLeft : kMergeNone;
    }
    if (tl == 0 && st == kMergeLeft) todo[atomicAdd(&ntodo, 1)] = rs;
    __syncthreads();
    floor_listed<DT, true>(a, todo, __builtin_amdgcn_readfirstlane(ntodo), sm.r);
}

template <int DT, bool VEC>
hipError_t launch_t(const FloorParams& p, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
    const size_t blocks = (size_t)p.B * p.R;
    if (blocks == 0) return hipSuccess;
    if constexpr (VEC) {
        if (cands_usable(p)) {
            // A small top-k: the tiles' candidates (the start event is this
            // dispatch's), their merge per row, then the full-row path for
            // the rows the merge left -- in one kernel when the row slots
            // fit one round of workgroups, else in two.
            hipExtLaunchKernelGGL(floor_cands<DT>, dim3((unsigned)p.C, (unsigned)p.R, (unsigned)p.B), dim3(kThreads),
                                  0, s, start, nullptr, 0, p);
            if (blocks <= (size_t)kFinishMaxRows) {
                hipExtLaunchKernelGGL(floor_finish<DT>, dim3((unsigned)((blocks + kFinishRows - 1) / kFinishRows)),
                                      dim3(kFT), 0, s, nullptr, stop, 0, p);
            } else {
                hipLaunchKernelGGL(floor_merge<DT>, dim3((unsigned)blocks), dim3(kMergeThreads), 0, s, p);
                hipExtLaunchKernelGGL((floor_rows<DT, true, true>), dim3((unsigned)kRowsGrid), dim3(kFT), 0, s,
                                      nullptr, stop, 0, p);
            }
            return hipGetLastError();
        }
    }
    FloorParams q = p;
    q.cand_head = nullptr;                                // the window paths alone
    q.cand_done = nullptr;
    hipExtLaunchKernelGGL((floor_rows<DT, VEC, false>), dim3((unsigned)blocks), dim3(kFT), 0, s, start, stop, 0, q);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_floors(const FloorParams& p, int dtype, bool vec, hipStream_t s, hipEvent_t start,
                         hipEvent_t stop) {
    if (dtype == kBF16) return vec ? launch_t<kBF16, true>(p, s, start, stop) : launch_t<kBF16, false>(p, s, start, stop);
    return vec ? launch_t<kFP32, true>(p, s, start, stop) : launch_t<kFP32, false>(p, s, start, stop);
}

}  // namespace specdec
