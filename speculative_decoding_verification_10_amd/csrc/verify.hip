// Stochastic verify step on gfx950: two stream-ordered kernels (three for
// long rows of many positions), one workgroup per work item.
//
//  verify_rows    row item (request b, row, tile): tile max and sum of
//                 exponentials of target row i <= k_b or draft row i < k_b
//                 ("3.5 Speculative Decoding", "Notation": p and q are the
//                 temperature-processed distributions), and the logit at the
//                 draft token x_i when it lies in the tile.  Rows past k_b are
//                 skipped.  Row 0 also empties the slab slots of the call.
//  verify_final   final item (request b, tile): the decision of request b --
//                 the tile partials of every row merged, u_i < min(1,
//                 p_i(x_i)/q_i(x_i)) tested for every drafted position, the
//                 first rejection j taken with a ballot ("The algorithm (one
//                 step)", step 3) -- then the tile's slab sums of the
//                 unnormalised replacement masses max(0, p_j - q_j), or of
//                 p_{k_b} when every draft was accepted (step 4).  Tile 0
//                 stores the accept probabilities.  The request's last tile
//                 then searches with one wave: the slab that holds u * S, a
//                 re-read of that one slab, the smallest token t with
//                 u * S < C_t, and the outputs; it empties the slab slots
//                 again.  For long rows of many positions the decision is
//                 instead taken once per request by verify_decide, launched
//                 before it.
//
// Only the search waits inside a kernel, on the slab and tile slots of its
// own request's other tiles (self-validating, slots.h); everything else
// reads what earlier kernels wrote.
//
// Masses are kept unnormalised: the replacement is Z_p * max(0, p - q) =
// max(0, e_p - rho e_q) with e = exp2(x * c - M) against each row's offset M
// and rho = Z_p / Z_q, the bonus is e_p.  An inverse CDF only needs the
// masses up to a common factor.  Where p and q nearly agree (a good drafter:
// "Speculative Decoding from First Principles", "What the numbers say") the
// replacement is a small difference of two large numbers, so it is formed
// without cancellation (-e_p expm1(z) from the exact logit difference) and
// rho, known from the row statistics only to ~1e-7, is refined inside the
// final pass from the signed sum of the replacement (see search_wave).
#include <hip/hip_ext.h>

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
    float red_f[kWaves];                // per wave: near-tie p mass of the tile
    double red_d[kWaves];               // per wave: signed replacement sum of the tile
    double slab[kSlabsPerTile];         // slab sums of the masses
    float slabq[kSlabsPerTile];         // slab sums of the q part (replacement with draft logits)
};

// k_b, clamped to [0, K] so that a bad value can never address memory
// outside the caller's arrays.
__device__ __forceinline__ int kb_of(const VerifyParams& a, int b) {
    return a.kpr ? min(max(a.kpr[b], 0), a.K) : a.K;
}

// expm1(z) for |z| < 1: z times a degree-8 polynomial in z, a weighted
// least-squares fit of expm1(z)/z on [-1, 1] (relative error 1e-8 in exact
// arithmetic, 1.2e-7 evaluated in fp32 by Horner's rule).
__device__ __forceinline__ float expm1_unit(float z) {
    float p = 2.7556084205571096e-06f;
    p = __fmaf_rn(z, p, 2.542029324104078e-05f);
    p = __fmaf_rn(z, p, 1.9848310330417007e-04f);
    p = __fmaf_rn(z, p, 1.3884315267205238e-03f);
    p = __fmaf_rn(z, p, 8.333275094628334e-03f);
    p = __fmaf_rn(z, p, 4.166679084300995e-02f);
    p = __fmaf_rn(z, p, 0.1666666865348816f);
    p = __fmaf_rn(z, p, 0.5f);
    p = __fmaf_rn(z, p, 1.0f);
    return __fmul_rn(z, p);
}

// |a| / e_p (~|z|) below which a token's replacement sign may flip between
// the ratio the tiles use and the refined one (|delta rho| / rho is checked
// against half of it in the search).
constexpr float kNearTie = 1.9073486328125e-06f;   // 2^-19

// Constants of the replacement with draft logits at one ratio rho:
// a = e_p - rho e_q = -e_p expm1(z), z = K0 + (x_q - x_p) / T.
struct ResConst {
    float Mp, Mq;
    float rho;          // rho rounded to fp32 (direct difference)
    double K0;          // ln(rho) + ln 2 (Mp - Mq)
};

__device__ __forceinline__ ResConst res_const(const Decision& d, double rho, double K0) {
    ResConst k;
    k.Mp = d.Mp;
    k.Mq = d.Mq;
    k.rho = (float)rho;
    k.K0 = K0;
    return k;
}

// Signed replacement a = e_p - rho e_q of one token, relative to Z_p.  Where
// |z| < 1 (p and q within a factor e) it is -e_p expm1(z) with z formed in
// fp64 from the exact logit difference, so it keeps the relative accuracy
// of e_p however closely p and q agree; elsewhere the direct difference
// loses at most a factor (1 + e) / (e - 1).  -inf logits give e = 0 and
// z = +-inf or NaN, which take the direct branch: a = -rho e_q, e_p or 0.
// Also returns e_q, and in xv the token's e_p when it is a near-tie
// (|a| <= 2^-19 e_p, i.e. |z| <= ~2^-19), else 0.
__device__ __forceinline__ float residual_exact(float xp, float xq, float ep, float eq, const ResConst& k,
                                                const Scale& sc, float& xv) {
    const float z = (float)__fma_rn((double)xq - (double)xp, sc.inv_t, k.K0);
    // Both forms are evaluated and one is selected (no branch per token).
    const float near = -__fmul_rn(ep, expm1_unit(z));
    const float far = __fmaf_rn(-k.rho, eq, ep);
    const bool in = fabsf(z) < 1.0f;
    xv = (in && fabsf(near) <= kNearTie * ep) ? ep : 0.0f;
    return in ? near : far;
}

__device__ __forceinline__ float residual_signed(float xp, float xq, const ResConst& k, const Scale& sc,
                                                 float& eq, float& xv) {
    const float ep = fast_exp2(exponent2(xp, k.Mp, sc));
    eq = fast_exp2(exponent2(xq, k.Mq, sc));
    return residual_exact(xp, xq, ep, eq, k, sc, xv);
}

// Final-draw masses (>= 0, relative to Z_p) of one vector: the replacement
// max(0, e_p - rho e_q) at the constants k, p without the rejected token
// (one-hot drafts), or the bonus e_p.
template <int DT>
__device__ __forceinline__ void final_masses(const u32x4& rp, const u32x4& rq, const Decision& d,
                                             const ResConst& k, int v, const Scale& sc,
                                             float (&r)[Elem<DT>::E]) {
    constexpr int E = Elem<DT>::E;
    float xp[E];
    decode<DT>(rp, xp);
    if (d.mode == kResidual) {
        float xq[E];
        decode<DT>(rq, xq);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            float eq, xv;
            r[e] = fmaxf(residual_signed(xp[e], xq[e], k, sc, eq, xv), 0.0f);
        }
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float ep = fast_exp2(exponent2(xp[e], d.Mp, sc));
            r[e] = (d.mode == kResidualOneHot && v * E + e == d.tok) ? 0.0f : ep;
        }
    }
}

// Processed rows: every logit below the row's floor reads as -inf (the
// top-k / top-p cut; the floor is -inf for an unprocessed row).
template <int DT>
__device__ __forceinline__ void apply_floor(u32x4& r, float fl) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if constexpr (DT == kFP32) {
            r[k] = (__uint_as_float(r[k]) >= fl) ? r[k] : 0xFF800000u;
        } else {
            const uint32_t lo = (__uint_as_float(r[k] << 16) >= fl) ? (r[k] & 0x0000FFFFu) : 0x0000FF80u;
            const uint32_t hi = (__uint_as_float(r[k] & 0xFFFF0000u) >= fl) ? (r[k] & 0xFFFF0000u) : 0xFF800000u;
            r[k] = hi | lo;
        }
    }
}

// Floors of the final row pair of request b (FL: processed rows).
template <bool FL>
__device__ __forceinline__ void final_floors(const VerifyParams& a, int b, const Decision& d, float& fp, float& fq) {
    fp = fq = -INFINITY;
    if constexpr (FL) {
        fp = a.floors[(size_t)b * a.R + d.j];
        if (d.mode == kResidual) fq = a.floors[(size_t)b * a.R + a.K + 1 + d.j];
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
// The decision of request b, by the whole workgroup: returned to every
// thread, the accept probabilities left in sh.ratio.
//
// Rows are merged 16 lanes to a row, four rows per wave and two row groups
// per lane, so one pass covers 32 rows and every slot load of the pass goes
// out before any is used.  Lane `sub` of a row folds tiles sub, sub+16, ...:
// row max, row offset M = fp32(max * c), and the row sum relative to M, each
// tile rescaled by exp2(M_tile - M) -- the difference exact in fp64, the
// power in fp32 (relative error ~1e-7, exactly 1 for the tile that holds the
// max).  Thread i < k_b forms p_i/q_i at the draft token in fp64 and tests
// u_i < min(1, p_i/q_i); the first rejection j comes from a ballot.
// ---------------------------------------------------------------------------
constexpr int kRowGroups = 2;                         // row groups per lane
constexpr int kRowsPerPass = kRowGroups * kWaves * 4;  // 32
constexpr int kTilesPerLoad = 4;                      // tiles per lane per load batch

__device__ Decision decide(const VerifyParams& a, int b, int kb, StepShared& sh) {
    const int K = a.K, C = a.C, R = a.R;
    const bool one_hot = (a.draft == nullptr);
    const int nrs = rows_of(kb, a.kinds);
    const int t = threadIdx.x, w = t >> 6, lane = t & 63, sub = lane & 15;

    // The gathered logits and the uniform of this thread's position,
    // branch-free (a thread past k_b reads position 0 and never uses it).
    const int tt = t < kb ? t : 0;
    uint32_t rl = a.slot_l[(size_t)b * R + tt];
    uint32_t rd = (one_hot || K == 0) ? 0u : a.slot_l[(size_t)b * R + K + 1 + tt];
    float u = a.unif[(size_t)b * (K + 1) + tt];
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
        // Groups and tile batches wholly past the end are skipped by the
        // whole workgroup (the conditions are uniform).
        for (int c0 = 0; c0 < C; c0 += 16 * kTilesPerLoad) {
            uint32_t um[kRowGroups][kTilesPerLoad];
            uint64_t us[kRowGroups][kTilesPerLoad];
            // Branch-free, so that every load goes out before any is waited
            // for: a lane past the end reads the request's first slot and
            // drops the value.
#pragma unroll
            for (int g = 0; g < kRowGroups; ++g) {
#pragma unroll
                for (int q = 0; q < kTilesPerLoad; ++q) {
                    const int c = c0 + sub + 16 * q;
                    const bool ok = rs[g] < nrs && c < C;
                    const size_t at = ok ? row0[g] + c : (size_t)b * R * C;
                    um[g][q] = a.slot_m[at];
                    us[g][q] = a.slot_s[at];
                }
            }
            // The values enter an empty asm statement here, so that the
            // compiler issues every load above before the first wait instead
            // of sinking each into the branch that merges it.
#pragma unroll
            for (int g = 0; g < kRowGroups; ++g)
#pragma unroll
                for (int q = 0; q < kTilesPerLoad; ++q) asm volatile("" : "+v"(um[g][q]), "+v"(us[g][q]));
#pragma unroll
            for (int g = 0; g < kRowGroups; ++g) {
                if (base + g * (kWaves * 4) >= nrs) continue;
#pragma unroll
                for (int q = 0; q < kTilesPerLoad; ++q) {
                    if (c0 + 16 * q >= C) continue;
                    const int c = c0 + sub + 16 * q;
                    if (rs[g] < nrs && c < C) merge2(lm[g], ls[g], dec_f32(um[g][q]), dec_f64(us[g][q]), a.sc);
                }
            }
        }
#pragma unroll
        for (int g = 0; g < kRowGroups; ++g) {
            if (base + g * (kWaves * 4) >= nrs) continue;
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
        // p_i/q_i = exp2((l - l_q) c - M_p + M_q) * Z_q / Z_p: one power of
        // two, the logit difference exact in fp64.  q_i = 0 (draft logit
        // -inf) counts as ratio 1.
        const float l = dec_f32(rl);
        const double c = a.sc.c;
        const double Mp = (double)offset_of(sh.m[t], a.sc);
        double ratio;
        if (one_hot) {
            ratio = fmin(1.0, exp2((double)l * c - Mp) / sh.z[t]);
        } else {
            const float dl = dec_f32(rd);
            const int qs = K + 1 + t;
            const double Mq = (double)offset_of(sh.m[qs], a.sc);
            ratio = (dl == -INFINITY)
                        ? 1.0
                        : fmin(1.0, exp2(((double)l - (double)dl) * c + (Mq - Mp)) * (sh.z[qs] / sh.z[t]));
        }
        sh.ratio[t] = (float)ratio;
        rej = !((double)u < ratio);
    }
    const unsigned long long mask = __ballot(rej);
    if (lane == 0) sh.rej[w] = mask;
    __syncthreads();
    // Every thread reads the first rejection and builds the same decision.
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
    d.pad = 0;
    d.Mp = offset_of(sh.m[j], a.sc);
    d.Mq = 0.0f;
    d.rho = 0.0;
    d.zq = 0.0;
    d.K0 = 0.0;
    if (j == kb) {
        d.mode = kBonus;
    } else if (one_hot) {
        d.mode = kResidualOneHot;
        d.tok = a.tokens[(size_t)b * K + j];
    } else {
        d.mode = kResidual;
        d.Mq = offset_of(sh.m[K + 1 + j], a.sc);
        d.zq = sh.z[K + 1 + j];
        d.rho = sh.z[j] / d.zq;
        d.K0 = log(d.rho) + 0.69314718055994530942 * ((double)d.Mp - (double)d.Mq);
    }
    return d;
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
    // The tile that holds the draft token x_i reads its logit (stored by
    // thread 0 after the reduction).  The token's id is a vector load issued
    // just before the tile's loads: waiting for it, to address the logit,
    // leaves the tile's loads in flight (a scalar load there made every tile
    // wait for it, and for the kernel arguments, before its loads went out).
    // Every lane of every tile issues the same-address logit load -- of the
    // row's first logit when the tile is not the holder -- so that no branch
    // sits among the loads.
    // (No branch: a row without a drafted token reads a uniform, dropped.)
    const int32_t* tp = (i < kb) ? a.tokens + (size_t)b * a.K + i : reinterpret_cast<const int32_t*>(a.unif);
    const int tok = __hip_atomic_load(const_cast<int32_t*>(tp), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    u32x4 raw[kUnroll];
    tile_load<DT, VEC>(row, a.V, a.NV, tile, raw);
    const int gx = (i < kb) ? min(max(tok, 0), a.V - 1) : -1;
    const bool holds = gx >= 0 && gx / (kTileVec * Elem<DT>::E) == tile;
    const bool holder = holds && threadIdx.x == 0;
    const float gval = load_one<DT>(row, holds ? gx : 0);
    float m;
    double z;
    tile_reduce<DT>(raw, a.sc, m, z, lds_f, lds_d);
    if (holder) slot_put(a.slot_l + (size_t)b * a.R + rr, enc_f32(gval));
    if (threadIdx.x == 0) {
        const size_t idx = ((size_t)b * a.R + rr) * a.C + tile;
        slot_put(a.slot_s + idx, enc_f64(z));
        slot_put(a.slot_m + idx, enc_f32(m));
    }
    // Row 0 (always read) empties the tile's slab and tile slots for the
    // final kernel.
    if (rr == 0 && threadIdx.x < kSlabsPerTile)
        slot_put(a.slot_slab + ((size_t)b * a.C + tile) * kSlabsPerTile + threadIdx.x, (uint64_t)0);
    if (rr == 0 && threadIdx.x == kSlabsPerTile) slot_put(a.slot_tile + (size_t)b * a.C + tile, (uint64_t)0);
}

// A slab's replacement terms (the 512 tokens one wave holds for one unroll
// step) are formed by the direct difference e_p - rho e_q when the slab's
// own cancellation is mild -- sum e_p at most kCheapRatio times sum |a|,
// i.e. p and q differ over the slab by a total variation of at least ~1/8
// -- where its rounding (~1e-7 of e_p + rho e_q per token, random in sign)
// moves C_t / S by under 1e-7; otherwise the wave re-forms the slab's terms
// in the cancellation-free form (residual_exact) from the same
// exponentials.  Rows with low acceptance, which reject often, take the
// direct form almost everywhere; rows where p and q nearly agree, which
// rarely reject, take both.
constexpr float kCheapRatio = 4.0f;

// The direct difference of one token; returns a and sets e_p, e_q.
__device__ __forceinline__ float residual_direct(float xp, float xq, const ResConst& k, const Scale& sc,
                                                 float& ep, float& eq) {
    ep = fast_exp2(exponent2(xp, k.Mp, sc));
    eq = fast_exp2(exponent2(xq, k.Mq, sc));
    return __fmaf_rn(-k.rho, eq, ep);
}

// The tile's replacement terms: per slab its mass and q part into LDS, per
// wave the signed sum and the near-tie p mass.  The slab test's two sums are
// reduced together per slab; the four slabs' masses and q parts together
// after the last.
template <int DT, bool ONE>
__device__ __forceinline__ void residual_slabs(const VerifyParams& a, const u32x4 (&rp)[kUnroll],
                                               const u32x4 (&rq)[kUnroll], const ResConst& k, int tile,
                                               StepShared& sh) {
    constexpr int E = Elem<DT>::E;
    static_assert(kUnroll == 4, "the four slabs of a wave are reduced together");
    const int w = threadIdx.x >> 6;
    const bool lead = (threadIdx.x & 63) == 0;
    const int wv0 = tile * kTileVec + w * kSlab;          // the wave's first vector of its first slab
    double dsum = 0.0;
    float xsum = 0.0f;
    double rs[kUnroll];                                   // per slab: the lane's mass
    float qs[kUnroll];                                    //           and q part
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        if (ONE && wv0 + u * kThreads >= a.NV) {
            // A one-tile row's slab wholly past the row's end (uniform over
            // the wave): its -inf padding sums to zero; the work is skipped.
            // (Short rows are mostly padding; a long row's last tile keeps
            // the unbranched loop, which measured faster there.)
            rs[u] = 0.0;
            qs[u] = 0.0f;
            continue;
        }
        float ep[E], eq[E], av[E];
        float cp = 0.0f, ca = 0.0f;
        {
            float xp[E], xq[E];
            decode<DT>(rp[u], xp);
            decode<DT>(rq[u], xq);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                av[e] = residual_direct(xp[e], xq[e], k, a.sc, ep[e], eq[e]);
                cp += ep[e];
                ca += fabsf(av[e]);
            }
        }
        float xv[E];
        wave_sum2(cp, ca);
        if (!(cp <= kCheapRatio * ca)) {
            // Strong cancellation in this slab (uniform over the wave): the
            // logits are decoded again rather than kept alive.
            u32x4 vp = rp[u], vq = rq[u];
            asm volatile("" : "+v"(vp), "+v"(vq));
            float xp[E], xq[E];
            decode<DT>(vp, xp);
            decode<DT>(vq, xq);
#pragma unroll
            for (int e = 0; e < E; ++e) av[e] = residual_exact(xp[e], xq[e], ep[e], eq[e], k, a.sc, xv[e]);
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) xv[e] = fabsf(av[e]) <= kNearTie * ep[e] ? ep[e] : 0.0f;
        }
        // The masses and signed values summed pairwise, the q part and
        // near-tie mass as running sums (they need only ~1e-6 relative
        // accuracy).
        float r[E];
        float sq = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            r[e] = fmaxf(av[e], 0.0f);
            sq += av[e] > 0.0f ? eq[e] : 0.0f;
            xsum += xv[e];
        }
        rs[u] = (double)pairwise_sum<E>(r);
        qs[u] = sq;
        dsum += (double)pairwise_sum<E>(av);
        // One vector at a time: the scheduler may not interleave the vectors
        // (their temporaries would not fit the registers of the occupancy
        // every final item needs to be resident at once).
        __builtin_amdgcn_sched_barrier(0);
    }
    double ts[kUnroll];
    float tq[kUnroll];
    wave_sum4(rs, ts);
    wave_sum4(qs, tq);
    dsum = wave_sum(dsum);
    xsum = wave_sum(xsum);
    if (lead) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            sh.slab[u * kWaves + w] = ts[u];
            sh.slabq[u * kWaves + w] = tq[u];
        }
        sh.red_d[w] = dsum;
        sh.red_f[w] = xsum;
    }
}

// Slab sums of one tile: slab u * kWaves + w of the tile holds the 64
// vectors that wave w loaded in unroll step u, summed by that wave; the
// tile's first nslabs slots (the slabs that start inside the row) leave in
// one batch of stores, each holding the slab's mass and, for a replacement
// with draft logits, its q part sum_{a > 0} e_q.  The tile's own slot holds
// the signed replacement sum sum_t (e_p - rho e_q) over the tile and the p
// mass of its near-ties (|z| <= ~2^-19), for the search's refinement of rho.
template <int DT, bool ONE>
__device__ void put_slabs(const VerifyParams& a, const u32x4 (&rp)[kUnroll], const u32x4 (&rq)[kUnroll],
                          const Decision& d, int v0, int b, int tile, int nslabs, StepShared& sh) {
    constexpr int E = Elem<DT>::E;
    const int w = threadIdx.x >> 6;
    const bool lead = (threadIdx.x & 63) == 0;
    if (d.mode == kResidual) {
        residual_slabs<DT, ONE>(a, rp, rq, res_const(d, d.rho, d.K0), tile, sh);
    } else {
        const ResConst k{};
        double rsd[kUnroll], ts[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            rsd[u] = 0.0;
            if (ONE && (threadIdx.x >> 6) * kSlab + u * kThreads >= a.NV) continue;   // (as above)
            float r[E];
            final_masses<DT>(rp[u], rq[u], d, k, v0 + u * kThreads, a.sc, r);
            rsd[u] = (double)pairwise_sum<E>(r);
        }
        wave_sum4(rsd, ts);
        if (lead) {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                sh.slab[u * kWaves + w] = ts[u];
                sh.slabq[u * kWaves + w] = 0.0f;
            }
            sh.red_d[w] = 0.0;
            sh.red_f[w] = 0.0f;
        }
    }
    __syncthreads();
    if (ONE) return;                                      // (a one-tile row: the search reads the LDS sums)
    if (tile == a.withhold_tile) return;                  // (error-path tests: sums never published)
    uint64_t* slabs = a.slot_slab + ((size_t)b * a.C + tile) * kSlabsPerTile;
    if (threadIdx.x < nslabs)
        slot_put(slabs + threadIdx.x, enc_f32x2((float)sh.slab[threadIdx.x], sh.slabq[threadIdx.x]));
    if (threadIdx.x == 64) {
        double ds = 0.0;
        float xs = 0.0f;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) {
            ds += sh.red_d[i];
            xs += sh.red_f[i];
        }
        slot_put(a.slot_tile + (size_t)b * a.C + tile, enc_f32x2((float)ds, xs));
    }
}

// The accept probabilities of request b.
__device__ void publish_aprob(const VerifyParams& a, int b, int kb, const StepShared& sh) {
    if (a.aprob)
        for (int i = threadIdx.x; i < a.K; i += kThreads)
            a.aprob[(size_t)b * a.K + i] = (i < kb) ? sh.ratio[i] : -1.0f;
}

constexpr int kSearchLanes = 64;

template <int DT, bool VEC, bool FL, bool ONE>
__device__ void search_wave(const VerifyParams& a, int b, int kb, Decision d, const StepShared& sh,
                            const u32x4* stage);

// The decision is the same in every lane: keep it in scalar registers.
__device__ __forceinline__ Decision to_scalar(const Decision& d) {
    static_assert(sizeof(Decision) % 4 == 0, "Decision is a whole number of words");
    constexpr int W = sizeof(Decision) / 4;
    uint32_t w[W];
    __builtin_memcpy(w, &d, sizeof(Decision));
#pragma unroll
    for (int i = 0; i < W; ++i) w[i] = __builtin_amdgcn_readfirstlane(w[i]);
    Decision r;
    __builtin_memcpy(&r, w, sizeof(Decision));
    return r;
}

// ---------------------------------------------------------------------------
// Final item: tile `tile` of the final row (pair) of request b.
// ---------------------------------------------------------------------------
// ONE: the row is a single tile (C = 1): the workgroup keeps the final
// row (pair) in LDS (stage: p at [0, kTileVec), q after it) and its search
// reads the slab sums and the final slab from there, not from the slots and
// the row again.
template <int DT, bool VEC, bool FL, bool ONE>
__device__ void final_item(const VerifyParams& a, int b, int tile, bool decided, StepShared& sh, u32x4* stage) {
    constexpr int S = Elem<DT>::S;
    const int K = a.K;
    const int kb = kb_of(a, b);
    const Decision d = to_scalar(decided ? a.dec[b] : decide(a, b, kb, sh));
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
    float fp, fq;
    final_floors<FL>(a, b, d, fp, fq);
    if constexpr (FL) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            apply_floor<DT>(rp[u], fp);
            apply_floor<DT>(rq[u], fq);
        }
    }
    if constexpr (ONE) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            stage[threadIdx.x + u * kThreads] = rp[u];
            if (rowq) stage[kTileVec + threadIdx.x + u * kThreads] = rq[u];
        }
    }
    put_slabs<DT, ONE>(a, rp, rq, d, v0, b, tile, min(kSlabsPerTile, a.NS - tile * kSlabsPerTile), sh);
    if (tile == 0 && !decided) publish_aprob(a, b, kb, sh);
    // The request's last tile -- dispatched after its other tiles, which
    // never wait -- searches, with its first wave, once every slab sum of
    // the request is in.
    if (tile == a.C - 1 && threadIdx.x < kSearchLanes) search_wave<DT, VEC, FL, ONE>(a, b, kb, d, sh, stage);
}


// ---------------------------------------------------------------------------
// Token search of request b, by the first wave of its last final tile (no
// workgroup barriers; the other waves have left).
//
// Refinement (replacement with draft logits).  The tiles used rho0 = Z_p/Z_q
// of the row statistics, accurate to ~1e-7; near p = q the replacement's
// total S is a small multiple TV of Z_p, so that error would move C_t / S by
// ~1e-7 / TV.  The tiles' signed sums give D = sum_t (e_p - rho0 e_q) =
// Z_p - rho0 Z_q with the relative accuracy of each term, hence the refined
// rho = rho0 + D / Z_q.  A slab's mass at rho is its mass at rho0 less
// (rho - rho0) times its q part, except for tokens whose sign flips between
// the two ratios; those have |z| <= |rho - rho0| / rho, so their error is
// at most |rho - rho0| / rho times the tiles' near-tie p mass X (e_p and
// rho e_q agree to 1e-6 there).  When that bound
// is not negligible (or rho moved by more than the near-tie band) every
// slab is recomputed exactly at rho instead.  The slab finally re-read is
// always evaluated exactly at rho.
//
// Slab g covers vectors [64 g, 64 g + 64).  Lane L owns the P = ceil(NS/64)
// consecutive slabs from L * P: one inclusive scan of the lanes' sums gives S
// (lane 63) and the lane whose range holds w = u * S; that lane walks its
// slabs to the first one whose running prefix exceeds w (the last slab with
// mass when rounding leaves w past the end).  Slab g is re-read, one vector
// per lane, a second scan finds the vector, and the smallest token t of it
// with w < C_t is taken (the last token with mass when rounding leaves w past
// every C_t).  Only entries with mass can be taken at any level, so a token
// of zero probability is never drawn, however the sums round.
//
// A wait that gives up (slots.h) leaves the request's outputs at -1
// (num_accepted and every token): a visibly invalid result, never a token
// drawn from missing sums.
// ---------------------------------------------------------------------------
constexpr int kHeld = 8;    // slab sums per lane kept in registers

// Bound on the crossing error of the corrected slab sums, relative to S,
// beyond which the slabs are recomputed exactly.
constexpr double kCrossingBound = 1e-7;

// Mass of slab g of the final row (pair), summed by one lane alone (the
// exact recomputation and the fallback draw from p_j).
template <int DT, bool VEC>
__device__ double lane_slab_mass(const VerifyParams& a, const void* rowp, const void* rowq, const Decision& d,
                                 const ResConst& k, int g, float fp, float fq) {
    constexpr int E = Elem<DT>::E;
    double t = 0.0;
#pragma unroll 1
    for (int i = 0; i < kSlab; ++i) {
        const int v = g * kSlab + i;
        u32x4 bp = load_raw<DT, VEC, false>(rowp, a.V, a.NV, v);
        apply_floor<DT>(bp, fp);
        u32x4 bq = bp;
        if (rowq) {
            bq = load_raw<DT, VEC, false>(rowq, a.V, a.NV, v);
            apply_floor<DT>(bq, fq);
        }
        float r[E];
        final_masses<DT>(bp, bq, d, k, v, a.sc, r);
        t += (double)pairwise_sum<E>(r);
    }
    return t;
}

template <int DT, bool VEC, bool FL, bool ONE>
__device__ void search_wave(const VerifyParams& a, int b, int kb, Decision d, const StepShared& sh,
                            const u32x4* stage) {
    constexpr int E = Elem<DT>::E;
    constexpr int S = Elem<DT>::S;
    const int K = a.K;
    const int lane = threadIdx.x & 63;
    const int NS = a.NS;
    const int P = (NS + 63) >> 6;             // slabs per lane
    const int g0 = lane * P;                  // this lane's first slab
    uint64_t* slabs = a.slot_slab + (size_t)b * a.C * kSlabsPerTile;
    uint64_t* tiles = a.slot_tile + (size_t)b * a.C;
    const uint64_t none = enc_f32x2(0.0f, 0.0f);
    bool lost = false;

    // Every slot this lane reads goes out in one batch of loads (its first
    // tile word and its first kHeld slab words); then each poll is finished.
    // The tiles' signed sums and near-tie masses come first: the refinement
    // needs them before any slab sum can be corrected.
    uint64_t tw = none;
    uint64_t hw[kHeld];
    if constexpr (ONE) {
        // The tile's own sums, in LDS (the words put_slabs would publish).
        if (lane == 0) {
            double ds = 0.0;
            float xs = 0.0f;
#pragma unroll
            for (int i = 0; i < kWaves; ++i) {
                ds += sh.red_d[i];
                xs += sh.red_f[i];
            }
            tw = enc_f32x2((float)ds, xs);
        }
#pragma unroll
        for (int k = 0; k < kHeld; ++k)
            hw[k] = (k < P && g0 + k < NS) ? enc_f32x2((float)sh.slab[g0 + k], sh.slabq[g0 + k]) : none;
    } else {
        tw = lane < a.C ? slot_peek(tiles + lane) : none;
#pragma unroll
        for (int k = 0; k < kHeld; ++k) hw[k] = (k < P && g0 + k < NS) ? slot_peek(slabs + g0 + k) : none;
    }
    if (!ONE) {
        // While any of these words is still empty: sleep, then reload every
        // empty one in one batch (one round trip per round, not per word).
        // The deadline is checked only after a reload that still found one
        // empty (slots.h).
        auto missing = [&]() {
            bool m = tw == 0;
#pragma unroll
            for (int k = 0; k < kHeld; ++k) m |= hw[k] == 0;
            return m;
        };
        uint64_t t0 = 0;
        while (missing()) {
            if (t0 == 0) t0 = __builtin_amdgcn_s_memrealtime();
            __builtin_amdgcn_s_sleep(2);
            if (tw == 0) tw = slot_peek(tiles + lane);
#pragma unroll
            for (int k = 0; k < kHeld; ++k)
                if (hw[k] == 0) hw[k] = slot_peek(slabs + g0 + k);
            if (missing() && __builtin_amdgcn_s_memrealtime() - t0 > a.wait_ticks) {
                atomicOr(a.err, 1u);
                lost = true;
                if (tw == 0) tw = none;
#pragma unroll
                for (int k = 0; k < kHeld; ++k)
                    if (hw[k] == 0) hw[k] = none;
            }
        }
    }
    double dsum = (double)dec_hi(tw);
    float xsum = dec_lo(tw);
    for (int c = lane + 64; c < a.C; c += 64) {
        const uint64_t t = slot_wait(tiles + c, a.err, none, lost, a.wait_ticks);
        dsum += (double)dec_hi(t);
        xsum += dec_lo(t);
    }
    dsum = wave_sum(dsum);
    xsum = wave_sum(xsum);

    // The refined ratio (uniform over the wave).
    double delta = 0.0;
    ResConst rk{};
    if (d.mode == kResidual) {
        if (d.zq > 0.0 && d.rho > 0.0) delta = dsum / d.zq;
        if (!(fabs(delta) < d.rho)) delta = 0.0;     // a broken row: keep rho0
        // ln(rho / rho0) = log1p(delta / rho0); |delta / rho0| is ~1e-7, where
        // two terms of the series are exact in fp64.
        const double e = delta / d.rho;
        rk = res_const(d, d.rho + delta, d.K0 + (fabs(e) < 1e-4 ? e * (1.0 - 0.5 * e) : log1p(e)));
    }
    auto corrected = [&](uint64_t word) { return fmax(0.0, (double)dec_hi(word) - delta * (double)dec_lo(word)); };

    double held[kHeld];
    double mine = 0.0;
#pragma unroll
    for (int k = 0; k < kHeld; ++k) {
        held[k] = corrected(hw[k]);
        mine += held[k];
    }
    for (int k = kHeld; k < P; ++k)
        if (g0 + k < NS) mine += corrected(slot_wait(slabs + g0 + k, a.err, none, lost, a.wait_ticks));

    const void* rowp = row_ptr(a.target, (size_t)b * (K + 1) + d.j, a.V, S);
    const void* rowq = (d.mode == kResidual) ? row_ptr(a.draft, (size_t)b * K + d.j, a.V, S) : nullptr;
    const double u = (double)a.unif[(size_t)b * (K + 1) + kb];
    float fp, fq;
    final_floors<FL>(a, b, d, fp, fq);

    double incl = wave_inclusive_scan(mine);
    double total = __shfl(incl, 63, 64);
    // Recompute every slab exactly at the refined ratio (exact), or from p_j
    // itself when every replacement mass is zero (rare; each lane sums its
    // own slabs).  The sums go back to the slots, rounded as the slots hold
    // them, and the registers reload from there, so that the walk below reads
    // the same values.
    int redo = d.mode == kResidual && (fabs(delta) > 0.5 * (double)kNearTie * d.rho ||
                                       fabs(delta / d.rho) * (double)xsum > kCrossingBound * total)
                   ? 1
                   : (total > 0.0 ? 0 : 2);
    while (redo) {
        if (redo == 2) {
            d.mode = kBonus;
            rowq = nullptr;
        }
        delta = 0.0;
        mine = 0.0;
#pragma unroll 1
        for (int k = 0; k < P; ++k)
            if (g0 + k < NS) {
                const float t = (float)lane_slab_mass<DT, VEC>(a, rowp, rowq, d, rk, g0 + k, fp, fq);
                slot_put(slabs + g0 + k, enc_f32x2(t, 0.0f));
                mine += (double)t;
            }
#pragma unroll
        for (int k = 0; k < kHeld; ++k) held[k] = (k < P && g0 + k < NS) ? corrected(slot_peek(slabs + g0 + k)) : 0.0;
        incl = wave_inclusive_scan(mine);
        total = __shfl(incl, 63, 64);
        // Every exact replacement mass is zero as well: draw from p_j.
        redo = (redo == 1 && !(total > 0.0)) ? 2 : 0;
    }
    const double w = u * total;

    // The lane whose slabs hold w, else the last lane with mass.
    int L;
    {
        const unsigned long long hit = __ballot(w < incl && mine > 0.0);
        const unsigned long long nz = __ballot(mine > 0.0);
        L = hit ? __ffsll((long long)hit) - 1 : (nz ? 63 - __clzll((long long)nz) : 0);
    }
    // Every lane walks its own slabs; lane L's answer is the one kept.
    int kk = -1, klast = -1;
    double kbefore = 0.0, klast_before = 0.0;
    {
        double c = incl - mine;
        auto visit = [&](int k, double x) {
            if (x > 0.0) {
                klast = k;
                klast_before = c;
            }
            if (kk < 0 && x > 0.0 && w < c + x) {
                kk = k;
                kbefore = c;
            }
            c += x;
        };
#pragma unroll
        for (int k = 0; k < kHeld; ++k) visit(k, held[k]);
        for (int k = kHeld; k < P; ++k)
            if (g0 + k < NS) visit(k, corrected(slot_peek(slabs + g0 + k)));
        if (kk < 0) {
            kk = max(klast, 0);
            kbefore = klast_before;
        }
    }
    const int g = __shfl(g0 + kk, L, 64);
    const double base = __shfl(kbefore, L, 64);
    // Every slab sum has been read: empty this lane's slots for the next call.
    for (int k = 0; k < P && g0 + k < NS; ++k) slot_put(slabs + g0 + k, (uint64_t)0);
    for (int c = lane; c < a.C; c += 64) slot_put(tiles + c, (uint64_t)0);

    // Slab g, one vector per lane in ascending order, exact at the refined
    // ratio.
    const int v = g * kSlab + lane;
    float r[E];
    {
        u32x4 sp, sq;
        if constexpr (ONE) {
            sp = stage[v];                                // (v < NS * kSlab <= kTileVec)
            sq = rowq ? stage[kTileVec + v] : sp;
        } else {
            sp = load_raw<DT, VEC, false>(rowp, a.V, a.NV, v);
            sq = rowq ? load_raw<DT, VEC, false>(rowq, a.V, a.NV, v) : sp;
        }
        if constexpr (FL) {
            apply_floor<DT>(sp, fp);
            apply_floor<DT>(sq, rowq ? fq : fp);
        }
        final_masses<DT>(sp, sq, d, rk, v, a.sc, r);
    }
    const double vs = (double)pairwise_sum<E>(r);
    const double vincl = base + wave_inclusive_scan(vs);
    int L2;
    {
        const unsigned long long hit = __ballot(w < vincl && vs > 0.0);
        const unsigned long long nz = __ballot(vs > 0.0);
        L2 = hit ? __ffsll((long long)hit) - 1 : (nz ? 63 - __clzll((long long)nz) : 0);
    }
    // Every lane scans its own elements; lane L2's answer is the one kept.
    int tok = -1, last = -1;
    {
        double Cc = vincl - vs;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if (r[e] > 0.0f) last = v * E + e;
            Cc += (double)r[e];
            if (tok < 0 && r[e] > 0.0f && w < Cc) tok = v * E + e;
        }
        if (tok < 0) tok = last;
    }
    tok = __shfl(tok, L2, 64);
    if (tok < 0) tok = 0;
    const bool invalid = __ballot(lost) != 0;
    const int j = d.j;
    for (int i = lane; i <= K; i += 64) {
        int32_t o = -1;
        if (!invalid) {
            if (i < j) o = a.tokens[(size_t)b * K + i];
            else if (i == j) o = tok;
        }
        a.out[(size_t)b * (K + 1) + i] = o;
    }
    if (lane == 0) a.nacc[b] = invalid ? -1 : j;
}

// Row items: workgroup (x, y, z) takes tile x of row slot y of request z
// (the grid is dispatched x fastest, so request-major).
template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void verify_rows(VerifyParams a) {
    __shared__ float lds_f[kWaves];
    __shared__ double lds_d[kWaves];
    row_item<DT, VEC>(a, blockIdx.z, blockIdx.y, blockIdx.x, lds_f, lds_d);
    // A call whose error word starts clear (the allocation-free entry point:
    // its scratch keeps the previous call's word): the first workgroup clears
    // it, after its loads (a store ahead of them would keep the compiler from
    // reading k_b and the draft tokens through the scalar cache); the only
    // writer of the word, the final kernel, runs after this one.
    if (a.clear_err && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0) *a.err = 0u;
}

// Decisions, when taken once per request: workgroup x takes request x.
__global__ __launch_bounds__(kThreads) void verify_decide(VerifyParams a) {
    __shared__ StepShared sh;
    const int b = blockIdx.x;
    const int kb = kb_of(a, b);
    const Decision d = decide(a, b, kb, sh);
    if (threadIdx.x == 0) a.dec[b] = d;
    publish_aprob(a, b, kb, sh);
}

// Final items: workgroup (x, y) takes tile x of request y.  FL: the rows are
// processed (top-k / top-p floors).
template <int DT, bool VEC, bool DECIDED, bool FL, bool ONE = false>
__global__ __launch_bounds__(kThreads) void verify_final(VerifyParams a) {
    __shared__ StepShared sh;
    __shared__ u32x4 stage[ONE ? 2 * kTileVec : 1];
    final_item<DT, VEC, FL, ONE>(a, blockIdx.y, blockIdx.x, DECIDED, sh, stage);
}

template <int DT, bool VEC>
hipError_t launch(const VerifyParams& p, hipStream_t s, hipEvent_t const* events) {
    if (p.B == 0) return hipSuccess;
    // Events, when given, are taken by the dispatches themselves (the
    // kernels' own start and end times), so no marker sits between kernels.
    hipEvent_t ev[3] = {nullptr, nullptr, nullptr};
    if (events)
        for (int k = 0; k < 3; ++k) ev[k] = events[k];
    hipExtLaunchKernelGGL((verify_rows<DT, VEC>), dim3(p.C, p.R, p.B), dim3(kThreads), 0, s, ev[0],
                          ev[1], 0, p);
    // Every final tile takes the decision itself (no extra launch) unless
    // that repeats much work: C tiles each merging R * C row-tile partials.
    if ((int64_t)p.C * p.R * p.C > kDecideOnceAbove) {
        hipLaunchKernelGGL(verify_decide, dim3(p.B), dim3(kThreads), 0, s, p);
        hipExtLaunchKernelGGL((verify_final<DT, VEC, true, false>), dim3(p.C, p.B), dim3(kThreads), 0, s,
                              nullptr, ev[2], 0, p);
    } else if (p.C == 1) {
        // Rows of one tile: the search works from LDS.
        hipExtLaunchKernelGGL((verify_final<DT, VEC, false, false, true>), dim3(1, p.B), dim3(kThreads), 0, s,
                              nullptr, ev[2], 0, p);
    } else {
        hipExtLaunchKernelGGL((verify_final<DT, VEC, false, false>), dim3(p.C, p.B), dim3(kThreads), 0, s,
                              nullptr, ev[2], 0, p);
    }
    return hipGetLastError();
}

// The processed step: the floor kernel takes the row kernel's place (it
// writes the same slots for the processed rows), then the same decision and
// final kernels read the rows through their floors.
template <int DT, bool VEC>
hipError_t launch_processed(const FloorParams& f, const VerifyParams& p, hipStream_t s,
                            hipEvent_t const* events) {
    if (p.B == 0) return hipSuccess;
    hipEvent_t ev[3] = {nullptr, nullptr, nullptr};
    if (events)
        for (int k = 0; k < 3; ++k) ev[k] = events[k];
    hipError_t e = launch_floors(f, DT, VEC, s, ev[0], ev[1]);
    if (e != hipSuccess) return e;
    if ((int64_t)p.C * p.R * p.C > kDecideOnceAbove) {
        hipLaunchKernelGGL(verify_decide, dim3(p.B), dim3(kThreads), 0, s, p);
        hipExtLaunchKernelGGL((verify_final<DT, VEC, true, true>), dim3(p.C, p.B), dim3(kThreads), 0, s,
                              nullptr, ev[2], 0, p);
    } else if (p.C == 1) {
        // Rows of one tile: the search works from LDS.
        hipExtLaunchKernelGGL((verify_final<DT, VEC, false, true, true>), dim3(1, p.B), dim3(kThreads), 0, s,
                              nullptr, ev[2], 0, p);
    } else {
        hipExtLaunchKernelGGL((verify_final<DT, VEC, false, true>), dim3(p.C, p.B), dim3(kThreads), 0, s,
                              nullptr, ev[2], 0, p);
    }
    return hipGetLastError();
}

// The workspace error word, copied to the caller and optionally cleared in
// one atomic step (one thread).
__global__ void workspace_errors_kernel(uint32_t* err, uint32_t* out, int clear) {
    out[0] = clear ? atomicExch(err, 0u)
                   : __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

hipError_t launch_workspace_errors(uint32_t* err, uint32_t* out, int clear, hipStream_t s) {
    hipLaunchKernelGGL(workspace_errors_kernel, dim3(1), dim3(1), 0, s, err, out, clear);
    return hipGetLastError();
}

hipError_t launch_verify(const VerifyParams& p, int dtype, bool vec, hipStream_t s,
                         hipEvent_t const* events) {
    if (dtype == kBF16) return vec ? launch<kBF16, true>(p, s, events) : launch<kBF16, false>(p, s, events);
    return vec ? launch<kFP32, true>(p, s, events) : launch<kFP32, false>(p, s, events);
}

hipError_t launch_verify_processed(const FloorParams& f, const VerifyParams& p, int dtype, bool vec,
                                   hipStream_t s, hipEvent_t const* events) {
    if (!p.floors) return hipErrorInvalidValue;
    if (dtype == kBF16)
        return vec ? launch_processed<kBF16, true>(f, p, s, events) : launch_processed<kBF16, false>(f, p, s, events);
    return vec ? launch_processed<kFP32, true>(f, p, s, events) : launch_processed<kFP32, false>(f, p, s, events);
}

}  // namespace specdec
