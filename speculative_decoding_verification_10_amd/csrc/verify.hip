// Stochastic verify step on gfx950: two stream-ordered kernels, one
// workgroup per work item.
//
//  verify_rows   row item (request b, row, tile): tile max and sum of
//                exponentials of target row i <= k_b or draft row i < k_b
//                ("3.5 Speculative Decoding", "Notation": p and q are the
//                temperature-processed distributions), and the logit at the
//                draft token x_i when it lies in the tile.  Rows past k_b are
//                skipped.  No item waits for another.  Items of target row 0
//                also clear the request's slab slots for the final kernel.
//  verify_final  final item (request b, tile): the decision of request b --
//                the tile partials of every row merged, u_i < min(1,
//                p_i(x_i)/q_i(x_i)) tested for every drafted position, the
//                first rejection j taken with a ballot ("The algorithm (one
//                step)", step 3) -- then the tile's slab sums of the
//                unnormalised replacement masses max(0, p_j - q_j), or of
//                p_{k_b} when every draft was accepted (step 4).  The
//                request's last tile then reads all of the request's slab
//                sums, finds the slab that holds u * S, re-reads that one
//                slab, takes the smallest token t with u * S < C_t and writes
//                the request's outputs.
//
// Results cross workgroups through self-validating slots (slots.h).  The
// kernel boundary orders every row slot before its readers.  The only wait
// is the last tile's, for the slab sums of its request's other tiles: those
// have lower workgroup indices, which the hardware dispatches no later, and
// they never wait themselves, so the wait ends.
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
    int g, found, lastpos, lastnz;
    double base, w, total;
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
    // Target row 0 is read by every request: its items clear the request's
    // slab slots for this call's final kernel.
    if (rr == 0 && threadIdx.x < kUnroll)
        slot_put(a.slot_slab + ((size_t)b * a.C + tile) * kUnroll + threadIdx.x, (uint64_t)0);
}

// ---------------------------------------------------------------------------
// Token search, by every final item of the request at once.
// ---------------------------------------------------------------------------

// Waits for the NS slab sums of the request; then (identically in every
// workgroup of the request) their total S, the slab g that holds w = u * S --
// the first slab whose inclusive prefix exceeds w -- and the mass before it;
// the last slab with mass when rounding leaves w past the end.
__device__ void find_slab(const VerifyParams& a, const uint64_t* slabs, double u, StepShared& sh) {
    const int t = threadIdx.x;
    const int NS = a.NS;
    double part = 0.0, v0 = 0.0;
    for (int s = t; s < NS; s += kThreads) {
        const double v = dec_f64(slot_wait(slabs + s, a.err, enc_f64(0.0)));
        part += v;
        if (s == t) v0 = v;
    }
    const double total = block_sum(part, sh.red_d);
    const double w = u * total;
    if (t == 0) {
        sh.g = 0x7FFFFFFF;
        sh.lastnz = -1;
    }
    __syncthreads();
    double run = 0.0;
    for (int s0 = 0; s0 < NS; s0 += kThreads) {
        const int s = s0 + t;
        const double v = (s0 == 0) ? v0 : (s < NS ? dec_f64(slot_peek(slabs + s)) : 0.0);
        double ctot;
        const double before = run + block_exclusive_scan(v, sh.red_d, &ctot);
        if (s < NS && w < before + v) atomicMin(&sh.g, s);
        if (s < NS && v > 0.0) atomicMax(&sh.lastnz, s);
        __syncthreads();
        const int g = sh.g;
        if (g == s) sh.base = before;
        if (g != 0x7FFFFFFF) break;
        run += ctot;
    }
    __syncthreads();
    if (t == 0) {
        if (sh.g == 0x7FFFFFFF) sh.g = -1;
        sh.w = w;
        sh.total = total;
    }
    __syncthreads();
    if (sh.g < 0) {
        // No slab reaches w: take the last slab with mass.
        const int L = sh.lastnz < 0 ? 0 : sh.lastnz;
        double run2 = 0.0;
        for (int s0 = 0; s0 < NS; s0 += kThreads) {
            const int s = s0 + t;
            const double v = s < NS ? dec_f64(slot_peek(slabs + s)) : 0.0;
            double ctot;
            const double before = run2 + block_exclusive_scan(v, sh.red_d, &ctot);
            if (s == L) sh.base = before;
            run2 += ctot;
        }
        __syncthreads();
        if (t == 0) sh.g = L;
        __syncthreads();
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

// The smallest token in slab g (held by this workgroup as vector index u)
// with w < C_t, C_t running from the mass before the slab; the last token
// with mass in the slab when rounding leaves w past every C_t.  Thread 0
// returns the token.
template <int DT>
__device__ int scan_slab(const VerifyParams& a, const u32x4& rp, const u32x4& rq, const Decision& d,
                         int v, double base, double w, StepShared& sh) {
    constexpr int E = Elem<DT>::E;
    float r[E];
    final_masses<DT>(rp, rq, d, v, a.sc, r);
    const double vs = (double)pairwise_sum<E>(r);
    if (threadIdx.x == 0) {
        sh.found = 0x7FFFFFFF;
        sh.lastpos = -1;
    }
    double slab_total;
    const double start = base + block_exclusive_scan(vs, sh.red_d, &slab_total);
    int lastpos = -1;
#pragma unroll
    for (int e = 0; e < E; ++e)
        if (r[e] > 0.0f) lastpos = v * E + e;
    if (lastpos >= 0) atomicMax(&sh.lastpos, lastpos);
    if (start <= w && vs > 0.0) {
        double Cc = start;
        for (int e = 0; e < E; ++e) {
            Cc += (double)r[e];
            if (w < Cc) {
                atomicMin(&sh.found, v * E + e);
                break;
            }
        }
    }
    __syncthreads();
    const int tok = sh.found != 0x7FFFFFFF ? sh.found : sh.lastpos;
    return tok < 0 ? 0 : tok;
}

// ---------------------------------------------------------------------------
// Final item: tile `tile` of the final row (pair) of request b.
// ---------------------------------------------------------------------------
template <int DT, bool VEC>
__device__ void final_item(const VerifyParams& a, int b, int tile, StepShared& sh) {
    constexpr int E = Elem<DT>::E;
    constexpr int S = Elem<DT>::S;
    const int K = a.K;
    const int kb = kb_of(a, b);
    decide(a, b, kb, sh);
    Decision d = sh.dec;
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
    if (tile != a.C - 1) return;

    // The request's last tile: every other tile of the request has a lower
    // workgroup index.
    const double u = (double)a.unif[(size_t)b * (K + 1) + kb];
    uint64_t* slabs = a.slot_slab + slab0;
    find_slab(a, slabs, u, sh);
    if (!(sh.total > 0.0)) {
        // Every replacement mass is zero: draw from p_j itself.  Its slab
        // sums replace the residual ones (rare; one workgroup streams the row).
        d.mode = kBonus;
        for (int g = 0; g < a.NS; ++g) {
            const int v = g * kSlab + threadIdx.x;
            const u32x4 bp = load_raw<DT, VEC, false>(rowp, a.V, a.NV, v);
            float r[E];
            final_masses<DT>(bp, bp, d, v, a.sc, r);
            const double t = block_sum((double)pairwise_sum<E>(r), sh.red_d);
            if (threadIdx.x == 0) slot_put(slabs + g, enc_f64(t));
        }
        __syncthreads();
        find_slab(a, slabs, u, sh);
    }
    // Re-read slab g (one vector per thread) and search it.
    const int v = sh.g * kSlab + threadIdx.x;
    const u32x4 sp = load_raw<DT, VEC, false>(rowp, a.V, a.NV, v);
    const u32x4 sq = (d.mode == kResidual) ? load_raw<DT, VEC, false>(rowq, a.V, a.NV, v) : sp;
    const int tok = scan_slab<DT>(a, sp, sq, d, v, sh.base, sh.w, sh);
    const int j = d.j;
    for (int i = threadIdx.x; i <= K; i += kThreads) {
        int32_t o = -1;
        if (i < j) o = a.tokens[(size_t)b * K + i];
        else if (i == j) o = tok;
        a.out[(size_t)b * (K + 1) + i] = o;
    }
    if (threadIdx.x == 0) a.nacc[b] = j;
    if (a.aprob)
        for (int i = threadIdx.x; i < K; i += kThreads)
            a.aprob[(size_t)b * K + i] = (i < kb) ? sh.ratio[i] : -1.0f;
}

// Row items: workgroup (x, y, z) takes tile x of row slot y of request z
// (the grid is dispatched x fastest, so request-major).
template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void verify_rows(VerifyParams a) {
    __shared__ float lds_f[kWaves];
    __shared__ double lds_d[kWaves];
    row_item<DT, VEC>(a, blockIdx.z, blockIdx.y, blockIdx.x, lds_f, lds_d);
}

// Final items: workgroup (x, y) takes tile x of request y; the request's last
// tile has the highest index of its row of the grid.
template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void verify_final(VerifyParams a) {
    __shared__ StepShared sh;
    final_item<DT, VEC>(a, blockIdx.y, blockIdx.x, sh);
}

template <int DT, bool VEC>
hipError_t launch(const VerifyParams& p, hipStream_t s) {
    if (p.B == 0) return hipSuccess;
    hipLaunchKernelGGL((verify_rows<DT, VEC>), dim3(p.C, p.R, p.B), dim3(kThreads), 0, s, p);
    hipLaunchKernelGGL((verify_final<DT, VEC>), dim3(p.C, p.B), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_verify(const VerifyParams& p, int dtype, bool vec, hipStream_t s) {
    if (dtype == kBF16) return vec ? launch<kBF16, true>(p, s) : launch<kBF16, false>(p, s);
    return vec ? launch<kFP32, true>(p, s) : launch<kFP32, false>(p, s);
}

}  // namespace specdec
