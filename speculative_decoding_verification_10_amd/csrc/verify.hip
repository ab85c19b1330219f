// Stochastic verify step on gfx950: three stream-ordered kernels, one
// workgroup per work item, and no waits inside any of them.
//
//  verify_rows    row item (request b, row, tile): tile max and sum of
//                 exponentials of target row i <= k_b or draft row i < k_b
//                 ("3.5 Speculative Decoding", "Notation": p and q are the
//                 temperature-processed distributions), and the logit at the
//                 draft token x_i when it lies in the tile.  Rows past k_b are
//                 skipped.
//  verify_final   final item (request b, tile): the decision of request b --
//                 the tile partials of every row merged, u_i < min(1,
//                 p_i(x_i)/q_i(x_i)) tested for every drafted position, the
//                 first rejection j taken with a ballot ("The algorithm (one
//                 step)", step 3) -- then the tile's slab sums of the
//                 unnormalised replacement masses max(0, p_j - q_j), or of
//                 p_{k_b} when every draft was accepted (step 4).  Tile 0
//                 stores the decision and the accept probabilities.  For
//                 long rows of many positions the decision is instead taken
//                 once per request by verify_decide, launched before it.
//  verify_search  one wave per request: the slab that holds u * S, a re-read
//                 of that one slab, the smallest token t with u * S < C_t,
//                 and the outputs.
//
// Each kernel reads only what the kernels before it wrote; the slots keep
// their self-validating encoding (slots.h) as a guard.
//
// Masses are kept unnormalised: the replacement is Z_p * max(0, p - q) =
// max(0, e_p - (Z_p/Z_q) e_q) with e = exp2(x * c - M) against each row's
// offset M, the bonus is e_p.  An inverse CDF only needs the masses up to a
// common factor.
#include "internal.h"
#include "slots.h"

namespace specdec {
namespace {

constexpr int kMaxRows = 2 * kMaxK + 1;
// Above this many partial loads per request (C tiles x R rows x C tiles), the
// decision is taken once per request by its own kernel.
constexpr int64_t kDecideOnceAbove = 8192;

__device__ __forceinline__ const void* row_ptr(const void* base, size_t row, int V, int S) {
    return static_cast<const char*>(base) + row * (size_t)V * (size_t)S;
}

// Draft token, clamped to [0, V) for addressing.
__device__ __forceinline__ int token_of(const VerifyParams& a, int b, int i) {
    return min(max(a.tokens[(size_t)b * a.K + i], 0), a.V - 1);
}

// Row slot of the rs-th row a request reads: target rows 0..kb, then draft
// rows 0..kb-1.
__device__ __forceinline__ int slot_of_rs(int rs, int kb, int K) {
    return rs <= kb ? rs : (K + 1) + (rs - kb - 1);
}

__device__ __forceinline__ int rows_of(int kb, int kinds) { return kb + 1 + (kinds == 2 ? kb : 0); }

struct StepShared {
    float m[kMaxRows];                  // row max, by row slot
    double z[kMaxRows];                 // row sum relative to offset_of(max)
    float ratio[kMaxK];
    unsigned long long rej[kWaves];
    Decision dec;
    float red_f[kWaves];
    double red_d[kWaves];
    double slab[kWaves][kUnroll];
};

// k_b, clamped to [0, K] so that a bad value can never address memory
// outside the caller's arrays.
__device__ __forceinline__ int kb_of(const VerifyParams& a, int b) {
    return a.kpr ? min(max(a.kpr[b], 0), a.K) : a.K;
}

// Unnormalised final-draw masses of one vector.
template <int DT>
__device__ __forceinline__ void final_masses(const u32x4& rp, const u32x4& rq, const Decision& d,
                                             int v, const Scale& sc, float (&r)[Elem<DT>::E]) {
    constexpr int E = Elem<DT>::E;
    float xp[E];
    decode<DT>(rp, xp);
    if (d.mode == kResidual) {
        float xq[E];
        decode<DT>(rq, xq);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float ep = fast_exp2(exponent2(xp[e], d.Mp, sc));
            const float eq = fast_exp2(exponent2(xq[e], d.Mq, sc));
            r[e] = fmaxf(__fsub_rn(ep, __fmul_rn(d.rho, eq)), 0.0f);
        }
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float ep = fast_exp2(exponent2(xp[e], d.Mp, sc));
            r[e] = (d.mode == kResidualOneHot && v * E + e == d.tok) ? 0.0f : ep;
        }
    }
}

// (m1, z1) <- merge of two partials (max, sum relative to offset_of(max)).
__device__ __forceinline__ void merge2(float& m1, double& z1, float m2, double z2, const Scale& sc) {
    if (m2 == -INFINITY) return;
    if (m1 == -INFINITY) {
        m1 = m2;
        z1 = z2;
        return;
    }
    const float m = fmaxf(m1, m2);
    const double M = (double)offset_of(m, sc);
    z1 = z1 * (double)fast_exp2((float)((double)offset_of(m1, sc) - M)) +
         z2 * (double)fast_exp2((float)((double)offset_of(m2, sc) - M));
    m1 = m;
}

// ---------------------------------------------------------------------------
// The decision of request b, by the whole workgroup, into sh.dec and
// sh.ratio.
//
// Rows are merged 16 lanes to a row, four rows per wave and two row groups
// per lane, so one pass covers 32 rows and every slot load of the pass goes
// out before any is used.  Lane `sub` of a row folds tiles sub, sub+16, ...:
// row max, row offset M = fp32(max * c), and the row sum relative to M, each
// tile rescaled by exp2(M_tile - M) -- the difference exact in fp64, the
// power in fp32 (relative error ~1e-7, exactly 1 for the tile that holds the
// max).  Thread i < k_b takes p_i and q_i at the draft token in fp64 and
// tests u_i < min(1, p_i/q_i); the first rejection j comes from a ballot.
// ---------------------------------------------------------------------------
constexpr int kRowGroups = 2;                         // row groups per lane
constexpr int kRowsPerPass = kRowGroups * kWaves * 4;  // 32
constexpr int kTilesPerLoad = 4;                      // tiles per lane per load batch

__device__ void decide(const VerifyParams& a, int b, int kb, StepShared& sh) {
    const int K = a.K, C = a.C, R = a.R;
    const bool one_hot = (a.draft == nullptr);
    const int nrs = rows_of(kb, a.kinds);
    const int t = threadIdx.x, w = t >> 6, lane = t & 63, sub = lane & 15;

    uint32_t rl = 0, rd = 0;
    float u = 0.0f;
    if (t < kb) {
        rl = slot_peek(a.slot_l + (size_t)b * R + t);
        if (!one_hot) rd = slot_peek(a.slot_l + (size_t)b * R + K + 1 + t);
        u = a.unif[(size_t)b * (K + 1) + t];
    }
    for (int base = 0; base < nrs; base += kRowsPerPass) {
        float lm[kRowGroups];
        double ls[kRowGroups];
        int rs[kRowGroups];
        size_t row0[kRowGroups];
#pragma unroll
        for (int g = 0; g < kRowGroups; ++g) {
            lm[g] = -INFINITY;
            ls[g] = 0.0;
            rs[g] = base + g * (kWaves * 4) + w * 4 + (lane >> 4);
            row0[g] = ((size_t)b * R + slot_of_rs(min(rs[g], nrs - 1), kb, K)) * C;
        }
        for (int c0 = 0; c0 < C; c0 += 16 * kTilesPerLoad) {
            uint32_t um[kRowGroups][kTilesPerLoad];
            uint64_t us[kRowGroups][kTilesPerLoad];
#pragma unroll
            for (int g = 0; g < kRowGroups; ++g) {
#pragma unroll
                for (int q = 0; q < kTilesPerLoad; ++q) {
                    const int c = c0 + sub + 16 * q;
                    um[g][q] = 0;
                    us[g][q] = 0;
                    if (rs[g] < nrs && c < C) {
                        um[g][q] = slot_peek(a.slot_m + row0[g] + c);
                        us[g][q] = slot_peek(a.slot_s + row0[g] + c);
                    }
                }
            }
#pragma unroll
            for (int g = 0; g < kRowGroups; ++g) {
#pragma unroll
                for (int q = 0; q < kTilesPerLoad; ++q) {
                    const int c = c0 + sub + 16 * q;
                    if (rs[g] < nrs && c < C) merge2(lm[g], ls[g], dec_f32(um[g][q]), dec_f64(us[g][q]), a.sc);
                }
            }
        }
#pragma unroll
        for (int g = 0; g < kRowGroups; ++g) {
            const float rmax = row16_max(lm[g]);
            double scaled = 0.0;
            if (lm[g] != -INFINITY)
                scaled = ls[g] * (double)fast_exp2(
                    (float)((double)offset_of(lm[g], a.sc) - (double)offset_of(rmax, a.sc)));
            const double zsum = row16_sum(scaled);
            if (sub == 0 && rs[g] < nrs) {
                const int slot = slot_of_rs(rs[g], kb, K);
                sh.m[slot] = rmax;
                sh.z[slot] = zsum;
            }
        }
    }
    __syncthreads();
    bool rej = false;
    if (t < kb) {
        const float l = dec_f32(rl);
        const double c = a.sc.c;
        const double p = exp2((double)l * c - (double)offset_of(sh.m[t], a.sc)) / sh.z[t];
        double q = 1.0;
        if (!one_hot) {
            const float dl = dec_f32(rd);
            const int qs = K + 1 + t;
            q = exp2((double)dl * c - (double)offset_of(sh.m[qs], a.sc)) / sh.z[qs];
        }
        const double ratio = (q == 0.0) ? 1.0 : fmin(1.0, p / q);
        sh.ratio[t] = (float)ratio;
        rej = !((double)u < ratio);
    }
    const unsigned long long mask = __ballot(rej);
    if (lane == 0) sh.rej[w] = mask;
    __syncthreads();
    if (t == 0) {
        int j = kb;
        for (int i = 0; i < kWaves; ++i) {
            if (sh.rej[i]) {
                j = i * 64 + __ffsll((long long)sh.rej[i]) - 1;
                break;
            }
        }
        Decision d;
        d.j = j;
        d.tok = -1;
        d.Mp = offset_of(sh.m[j], a.sc);
        d.Mq = 0.0f;
        d.rho = 0.0f;
        d.pad0 = d.pad1 = 0;
        if (j == kb) {
            d.mode = kBonus;
        } else if (one_hot) {
            d.mode = kResidualOneHot;
            d.tok = a.tokens[(size_t)b * K + j];
        } else {
            d.mode = kResidual;
            d.Mq = offset_of(sh.m[K + 1 + j], a.sc);
            d.rho = (float)(sh.z[j] / sh.z[K + 1 + j]);
        }
        sh.dec = d;
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// Row item: tile `tile` of row slot rr of request b (target rows 0..K, then
// draft rows 0..K-1).
// ---------------------------------------------------------------------------
template <int DT, bool VEC>
__device__ void row_item(const VerifyParams& a, int b, int rr, int tile, float* lds_f, double* lds_d) {
    constexpr int S = Elem<DT>::S;
    const int K = a.K;
    const int kb = kb_of(a, b);
    const bool draft = rr > K;
    const int i = draft ? rr - K - 1 : rr;
    if (draft ? i >= kb : i > kb) return;   // row past k_b: nothing to read
    const void* row = draft ? row_ptr(a.draft, (size_t)b * K + i, a.V, S)
                            : row_ptr(a.target, (size_t)b * (K + 1) + i, a.V, S);
    const int gx = (i < kb) ? token_of(a, b, i) : -1;
    float m, gval = 0.0f;
    double z;
    const bool held =
        tile_stats<DT, VEC>(row, a.V, a.NV, tile, a.sc, m, z, lds_f, lds_d, gx, &gval);
    if (held) slot_put(a.slot_l + (size_t)b * a.R + rr, enc_f32(gval));
    if (threadIdx.x == 0) {
        const size_t idx = ((size_t)b * a.R + rr) * a.C + tile;
        slot_put(a.slot_s + idx, enc_f64(z));
        slot_put(a.slot_m + idx, enc_f32(m));
    }
}

// Slab sums of one tile: the masses of each of the kUnroll vectors of every
// thread, summed over the workgroup per vector index (one slab each).
template <int DT>
__device__ void put_slabs(const VerifyParams& a, const u32x4 (&rp)[kUnroll], const u32x4 (&rq)[kUnroll],
                          const Decision& d, int v0, uint64_t* slabs_of_tile, StepShared& sh) {
    constexpr int E = Elem<DT>::E;
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        float r[E];
        final_masses<DT>(rp[u], rq[u], d, v0 + u * kThreads, a.sc, r);
        const double t = wave_sum((double)pairwise_sum<E>(r));
        if ((threadIdx.x & 63) == 0) sh.slab[w][u] = t;
    }
    __syncthreads();
    if (threadIdx.x < kUnroll) {
        double t = 0.0;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) t += sh.slab[i][threadIdx.x];
        slot_put(slabs_of_tile + threadIdx.x, enc_f64(t));
    }
}

// The decision of request b for the search kernel, and the accept
// probabilities.
__device__ void publish_decision(const VerifyParams& a, int b, int kb, const StepShared& sh) {
    if (threadIdx.x == 0) a.dec[b] = sh.dec;
    if (a.aprob)
        for (int i = threadIdx.x; i < a.K; i += kThreads)
            a.aprob[(size_t)b * a.K + i] = (i < kb) ? sh.ratio[i] : -1.0f;
}

// ---------------------------------------------------------------------------
// Final item: tile `tile` of the final row (pair) of request b.
// ---------------------------------------------------------------------------
template <int DT, bool VEC>
__device__ void final_item(const VerifyParams& a, int b, int tile, bool decided, StepShared& sh) {
    constexpr int E = Elem<DT>::E;
    constexpr int S = Elem<DT>::S;
    const int K = a.K;
    const int kb = kb_of(a, b);
    if (decided) {
        if (threadIdx.x == 0) sh.dec = a.dec[b];
        __syncthreads();
    } else {
        decide(a, b, kb, sh);
    }
    const Decision d = sh.dec;
    const void* rowp = row_ptr(a.target, (size_t)b * (K + 1) + d.j, a.V, S);
    const void* rowq = (d.mode == kResidual) ? row_ptr(a.draft, (size_t)b * K + d.j, a.V, S) : nullptr;
    const int v0 = tile * kTileVec + threadIdx.x;
    u32x4 rp[kUnroll], rq[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int v = v0 + u * kThreads;
        rp[u] = load_raw<DT, VEC, false>(rowp, a.V, a.NV, v);
        rq[u] = rowq ? load_raw<DT, VEC, false>(rowq, a.V, a.NV, v) : neg_inf_raw<DT>();
    }
    const size_t slab0 = (size_t)b * a.C * kUnroll;
    put_slabs<DT>(a, rp, rq, d, v0, a.slot_slab + slab0 + (size_t)tile * kUnroll, sh);
    if (tile == 0 && !decided) publish_decision(a, b, kb, sh);
}


// ---------------------------------------------------------------------------
// Token search of request b, by one wave (no workgroup barriers).
//
// The slab sums give S and the slab g that holds w = u * S: the first slab
// whose inclusive prefix exceeds w (the last slab with mass when rounding
// leaves w past the end).  Slab g is re-read, four vectors per lane in
// ascending token order, and the smallest token t with w < C_t is taken, C_t
// running from the mass before the slab (the last token with mass in the
// slab when rounding leaves w past every C_t).
// ---------------------------------------------------------------------------
constexpr int kSearchLanes = 64;
constexpr int kSlabPerLane = kSlab / kSearchLanes;   // vectors of a slab per lane

// Wave: first index in [0, n) of values v (read by get(i)) whose inclusive
// prefix exceeds w, and the mass before it; else the last index with mass.
template <class Get>
__device__ __forceinline__ int wave_locate(int n, double w, Get get, double* before_out) {
    const int lane = threadIdx.x & 63;
    double run = 0.0, last_before = 0.0;
    int last_nz = -1;
    for (int i0 = 0; i0 < n; i0 += 64) {
        const double v = (i0 + lane < n) ? get(i0 + lane) : 0.0;
        const double incl = run + wave_inclusive_scan(v);
        const double before = incl - v;
        const unsigned long long hit = __ballot(w < incl && i0 + lane < n);
        const unsigned long long nz = __ballot(v > 0.0);
        if (nz) {
            const int L = 63 - __clzll((long long)nz);
            last_nz = i0 + L;
            last_before = __shfl(before, L, 64);
        }
        if (hit) {
            const int L = __ffsll((long long)hit) - 1;
            *before_out = __shfl(before, L, 64);
            return i0 + L;
        }
        run = __shfl(incl, 63, 64);
    }
    *before_out = last_before;
    return last_nz < 0 ? 0 : last_nz;
}

template <int DT, bool VEC>
__device__ void search(const VerifyParams& a, int b) {
    constexpr int E = Elem<DT>::E;
    constexpr int S = Elem<DT>::S;
    const int K = a.K;
    const int lane = threadIdx.x;
    const int kb = kb_of(a, b);
    Decision d = a.dec[b];
    const void* rowp = row_ptr(a.target, (size_t)b * (K + 1) + d.j, a.V, S);
    const void* rowq = (d.mode == kResidual) ? row_ptr(a.draft, (size_t)b * K + d.j, a.V, S) : nullptr;
    const double u = (double)a.unif[(size_t)b * (K + 1) + kb];
    uint64_t* slabs = a.slot_slab + (size_t)b * a.C * kUnroll;
    const int NS = a.NS;

    // The slab sums, kept in registers for up to kHeld * 64 slabs (read
    // again from the slots beyond that).
    constexpr int kHeld = 4;
    double held[kHeld];
    double total = 0.0;
#pragma unroll
    for (int k = 0; k < kHeld; ++k) {
        held[k] = 0.0;
        if (k * 64 + lane < NS) held[k] = dec_f64(slot_wait(slabs + k * 64 + lane, a.err, enc_f64(0.0)));
        total += held[k];
    }
    for (int g0 = kHeld * 64; g0 < NS; g0 += 64)
        if (g0 + lane < NS) total += dec_f64(slot_wait(slabs + g0 + lane, a.err, enc_f64(0.0)));
    total = wave_sum(total);
    if (!(total > 0.0)) {
        // Every replacement mass is zero: draw from p_j itself.  Its slab
        // sums replace the residual ones (rare; one wave streams the row).
        d.mode = kBonus;
        rowq = nullptr;
        for (int g = 0; g < NS; ++g) {
            double t = 0.0;
            for (int k = 0; k < kSlabPerLane; ++k) {
                const int v = g * kSlab + k * 64 + lane;
                const u32x4 bp = load_raw<DT, VEC, false>(rowp, a.V, a.NV, v);
                float r[E];
                final_masses<DT>(bp, bp, d, v, a.sc, r);
                t += (double)pairwise_sum<E>(r);
            }
            t = wave_sum(t);
            if (lane == 0) slot_put(slabs + g, enc_f64(t));
        }
        total = 0.0;
#pragma unroll
        for (int k = 0; k < kHeld; ++k) {
            held[k] = 0.0;
            if (k * 64 + lane < NS) held[k] = dec_f64(slot_wait(slabs + k * 64 + lane, a.err, enc_f64(0.0)));
            total += held[k];
        }
        for (int g0 = kHeld * 64; g0 < NS; g0 += 64)
            if (g0 + lane < NS) total += dec_f64(slot_wait(slabs + g0 + lane, a.err, enc_f64(0.0)));
        total = wave_sum(total);
    }
    const double w = u * total;
    double base;
    const int g = wave_locate(NS, w,
                              [&](int i) {
                                  double x = 0.0;
#pragma unroll
                                  for (int k = 0; k < kHeld; ++k)
                                      if ((i >> 6) == k) x = held[k];
                                  return i < kHeld * 64 ? x : dec_f64(slot_peek(slabs + i));
                              },
                              &base);

    // Slab g: vector g * kSlab + k * 64 + lane for k = 0..3, in ascending order.
    float r[kSlabPerLane][E];
    double vs[kSlabPerLane];
#pragma unroll
    for (int k = 0; k < kSlabPerLane; ++k) {
        const int v = g * kSlab + k * 64 + lane;
        const u32x4 sp = load_raw<DT, VEC, false>(rowp, a.V, a.NV, v);
        const u32x4 sq = rowq ? load_raw<DT, VEC, false>(rowq, a.V, a.NV, v) : sp;
        final_masses<DT>(sp, sq, d, v, a.sc, r[k]);
        vs[k] = (double)pairwise_sum<E>(r[k]);
    }
    double vbase;
    const int vi = wave_locate(kSlabPerLane * 64, w - base,
                               [&](int i) {
                                   double x = 0.0;
#pragma unroll
                                   for (int k = 0; k < kSlabPerLane; ++k)
                                       if ((i >> 6) == k) x = vs[k];
                                   return x;
                               },
                               &vbase);
    // Lane vi & 63 holds vector vi (k = vi >> 6); scan its elements.
    int tok = -1;
    if (lane == (vi & 63)) {
        const int k = vi >> 6;
        float rr[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            float x = 0.0f;
#pragma unroll
            for (int kk = 0; kk < kSlabPerLane; ++kk)
                if (kk == k) x = r[kk][e];
            rr[e] = x;
        }
        const int v = g * kSlab + vi;
        double Cc = base + vbase;
        int lastpos = -1;
        for (int e = 0; e < E; ++e) {
            if (rr[e] > 0.0f) lastpos = v * E + e;
            Cc += (double)rr[e];
            if (tok < 0 && w < Cc) tok = v * E + e;
        }
        if (tok < 0) tok = lastpos;
    }
    tok = __shfl(tok, vi & 63, 64);
    if (tok < 0) tok = 0;
    const int j = d.j;
    for (int i = lane; i <= K; i += 64) {
        int32_t o = -1;
        if (i < j) o = a.tokens[(size_t)b * K + i];
        else if (i == j) o = tok;
        a.out[(size_t)b * (K + 1) + i] = o;
    }
    if (lane == 0) a.nacc[b] = j;
}

// Row items: workgroup (x, y, z) takes tile x of row slot y of request z
// (the grid is dispatched x fastest, so request-major).
template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void verify_rows(VerifyParams a) {
    __shared__ float lds_f[kWaves];
    __shared__ double lds_d[kWaves];
    row_item<DT, VEC>(a, blockIdx.z, blockIdx.y, blockIdx.x, lds_f, lds_d);
}

// Decisions, when taken once per request: workgroup x takes request x.
__global__ __launch_bounds__(kThreads) void verify_decide(VerifyParams a) {
    __shared__ StepShared sh;
    const int b = blockIdx.x;
    const int kb = kb_of(a, b);
    decide(a, b, kb, sh);
    publish_decision(a, b, kb, sh);
}

// Final items: workgroup (x, y) takes tile x of request y.
template <int DT, bool VEC, bool DECIDED>
__global__ __launch_bounds__(kThreads) void verify_final(VerifyParams a) {
    __shared__ StepShared sh;
    final_item<DT, VEC>(a, blockIdx.y, blockIdx.x, DECIDED, sh);
}

// Token search: one wave per request.
template <int DT, bool VEC>
__global__ __launch_bounds__(kSearchLanes) void verify_search(VerifyParams a) {
    search<DT, VEC>(a, blockIdx.x);
}

template <int DT, bool VEC>
hipError_t launch(const VerifyParams& p, hipStream_t s) {
    if (p.B == 0) return hipSuccess;
    hipLaunchKernelGGL((verify_rows<DT, VEC>), dim3(p.C, p.R, p.B), dim3(kThreads), 0, s, p);
    // Every final tile takes the decision itself (no extra launch) unless
    // that repeats much work: C tiles each merging R * C row-tile partials.
    if ((int64_t)p.C * p.R * p.C > kDecideOnceAbove) {
        hipLaunchKernelGGL(verify_decide, dim3(p.B), dim3(kThreads), 0, s, p);
        hipLaunchKernelGGL((verify_final<DT, VEC, true>), dim3(p.C, p.B), dim3(kThreads), 0, s, p);
    } else {
        hipLaunchKernelGGL((verify_final<DT, VEC, false>), dim3(p.C, p.B), dim3(kThreads), 0, s, p);
    }
    hipLaunchKernelGGL((verify_search<DT, VEC>), dim3(p.B), dim3(kSearchLanes), 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_verify(const VerifyParams& p, int dtype, bool vec, hipStream_t s) {
    if (dtype == kBF16) return vec ? launch<kBF16, true>(p, s) : launch<kBF16, false>(p, s);
    return vec ? launch<kFP32, true>(p, s) : launch<kFP32, false>(p, s);
}

}  // namespace specdec
