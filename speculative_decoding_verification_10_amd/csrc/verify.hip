// Stochastic verify step on gfx950: two stream-ordered kernels.
//
//  verify_rows   one workgroup per A item (position p, request b,
//                target|draft, tile c), position-major: tile max and sum of
//                exponentials of target row p <= k_b or draft row p < k_b
//                ("3.5 Speculative Decoding", "Notation": p and q are the
//                temperature-processed distributions).  Rows past k_b are
//                skipped.
//  verify_final  persistent (each workgroup takes items blockIdx.x,
//                blockIdx.x + gridDim.x, ...; the grid is sized so that every
//                workgroup is resident at once) over B items (request b,
//                tile c): the accept test of request b -- u_i < min(1,
//                p_i(x_i)/q_i(x_i)) left to right, first rejection j by a
//                ballot ("The algorithm (one step)", step 3) -- then tile c of
//                the final row (pair): slab sums of the unnormalised
//                replacement masses max(0, p_j - q_j), or of p_{k_b} when
//                every draft was accepted (step 4).  The workgroup that
//                completes a request's last tile then locates the token: the
//                slab that holds u * S (prefix over slab sums), a re-read of
//                that one slab, the smallest token t with u * S < C_t.
//
// Tile results travel through self-validating slots and a per-request
// completion counter (slots.h).  The kernel boundary orders A before B; the
// only wait inside verify_final is for slab slots of tiles whose workgroups
// have already counted themselves done, so it always ends.  The workgroup
// that locates a request's token also zeroes its slots, so the workspace is
// all zero again when the call ends.
//
// Masses are kept unnormalised: the replacement is Z_p * max(0, p - q) =
// max(0, e_p - (Z_p/Z_q) e_q) with e = exp2(x * c - M) against each row's
// offset M, the bonus is e_p.  An inverse CDF only needs the masses up to a
// common factor.
#include "internal.h"
#include "slots.h"

namespace specdec {
namespace {

__device__ __forceinline__ const void* row_ptr(const void* base, size_t row, int V, int S) {
    return static_cast<const char*>(base) + row * (size_t)V * (size_t)S;
}

// k_b, clamped to [0, K] so that a bad value can never address memory
// outside the caller's arrays.
__device__ __forceinline__ int k_of(const VerifyParams& a, int b) {
    return a.kpr ? min(max(a.kpr[b], 0), a.K) : a.K;
}

// Draft token, clamped to [0, V) for addressing.
__device__ __forceinline__ int token_of(const VerifyParams& a, int b, int i) {
    return min(max(a.tokens[(size_t)b * a.K + i], 0), a.V - 1);
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

// ---------------------------------------------------------------------------
// A: tile statistics of one row
// ---------------------------------------------------------------------------
template <int DT, bool VEC>
__device__ void a_item(const VerifyParams& a, int item, float* lds_f, double* lds_d) {
    constexpr int S = Elem<DT>::S;
    const int c = item % a.C;
    int t = item / a.C;
    const int kind = t % a.kinds;
    t /= a.kinds;
    const int b = t % a.B;
    const int p = t / a.B;
    const int kb = k_of(a, b);
    const void* row;
    int slot;
    if (kind == 0) {
        if (p > kb) return;
        row = row_ptr(a.target, (size_t)b * (a.K + 1) + p, a.V, S);
        slot = p;
    } else {
        if (p >= kb) return;
        row = row_ptr(a.draft, (size_t)b * a.K + p, a.V, S);
        slot = a.K + 1 + p;
    }
    float m;
    double z;
    tile_stats<DT, VEC>(row, a.V, a.NV, c, a.sc, m, z, lds_f, lds_d);
    if (threadIdx.x == 0) {
        const size_t idx = ((size_t)b * a.R + slot) * a.C + c;
        slot_put(&a.slot_s[idx], enc_f64(z));
        slot_put(&a.slot_m[idx], enc_f32(m));
    }
}

// ---------------------------------------------------------------------------
// The accept test of request b by the whole workgroup, once every row of the
// request is complete.
//
// Wave w merges the tile partials of row slots w, w+4, ... (lane l takes the
// tiles l, l+64, ...): row max, row offset M = fp32(max * c), and the row sum
// relative to M, rescaling each tile by exp2(M_tile - M) -- the difference
// exact in fp64, the power in fp32 (relative error ~1e-7 per tile, exactly 1
// for the tile that holds the max).  Thread i < k_b gathers p_i and q_i at
// the draft token in fp64 and tests u_i < min(1, p_i/q_i); the first
// rejection j comes from a ballot.  Every load is issued before any is
// consumed except the gathers, which need the token: two memory round trips.
// ---------------------------------------------------------------------------
constexpr int kMaxRows = 2 * kMaxK + 1;
constexpr int kRowBatch = 4;    // row slots per wave per batch of loads

struct DecideShared {
    float m[kMaxRows];          // row max
    double z[kMaxRows];         // row sum relative to offset_of(max)
    float ratio[kMaxK];         // min(1, p_i/q_i) per drafted position
    unsigned long long rej[kWaves];
    Decision dec;
};

// Row slot of the rs-th row in use: target rows 0..kb, then draft rows 0..kb-1.
__device__ __forceinline__ int slot_of_rs(int rs, int kb, int K) {
    return rs <= kb ? rs : (K + 1) + (rs - kb - 1);
}

template <int DT>
__device__ void decide_block(const VerifyParams& a, int b, DecideShared* sh) {
    constexpr int S = Elem<DT>::S;
    const int K = a.K;
    const int C = a.C;
    const int kb = k_of(a, b);
    const bool one_hot = (a.draft == nullptr);
    const int nrs = kb + 1 + (one_hot ? 0 : kb);
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = threadIdx.x;

    // Position t < kb: token and uniform now, the gathers once the token is in.
    int x = 0;
    float u = 0.0f;
    if (t < kb) {
        x = token_of(a, b, t);
        u = a.unif[(size_t)b * (K + 1) + t];
    }
    for (int base = 0; base < nrs; base += kWaves * kRowBatch) {
        float lm[kRowBatch];
        double ls[kRowBatch];
#pragma unroll
        for (int q = 0; q < kRowBatch; ++q) {
            lm[q] = -INFINITY;
            ls[q] = 0.0;
        }
        // Tiles lane, lane+64, ... of each row; rows with more than 64 tiles
        // are folded into (max, sum) per lane with an online rescale.
#pragma unroll
        for (int q = 0; q < kRowBatch; ++q) {
            const int rs = base + w + q * kWaves;
            if (rs < nrs) {
                const size_t idx = ((size_t)b * a.R + slot_of_rs(rs, kb, K)) * C;
                for (int c = lane; c < C; c += 64) {
                    const float mc = dec_f32(a.slot_m[idx + c]);
                    const double sc = dec_f64(a.slot_s[idx + c]);
                    if (mc == -INFINITY) continue;
                    if (mc > lm[q]) {
                        if (lm[q] != -INFINITY)
                            ls[q] *= (double)fast_exp2(
                                (float)((double)offset_of(lm[q], a.sc) - (double)offset_of(mc, a.sc)));
                        lm[q] = mc;
                    }
                    ls[q] += sc * (double)fast_exp2(
                        (float)((double)offset_of(mc, a.sc) - (double)offset_of(lm[q], a.sc)));
                }
            }
        }
#pragma unroll
        for (int q = 0; q < kRowBatch; ++q) {
            const int rs = base + w + q * kWaves;
            const float rmax = wave_max(lm[q]);
            double scaled = 0.0;
            if (lm[q] != -INFINITY)
                scaled = ls[q] * (double)fast_exp2(
                    (float)((double)offset_of(lm[q], a.sc) - (double)offset_of(rmax, a.sc)));
            const double zsum = __shfl(wave_sum(scaled), 0, 64);
            if (rs < nrs && lane == 0) {
                const int slot = slot_of_rs(rs, kb, K);
                sh->m[slot] = rmax;
                sh->z[slot] = zsum;
            }
        }
    }
    float l = 0.0f, dl = 0.0f;
    if (t < kb) {
        l = load_one<DT>(row_ptr(a.target, (size_t)b * (K + 1) + t, a.V, S), x);
        if (!one_hot) dl = load_one<DT>(row_ptr(a.draft, (size_t)b * K + t, a.V, S), x);
    }
    __syncthreads();
    bool rej = false;
    if (t < kb) {
        const double c = a.sc.c;
        const double p = exp2((double)l * c - (double)offset_of(sh->m[t], a.sc)) / sh->z[t];
        double q = 1.0;
        if (!one_hot) {
            const int qs = K + 1 + t;
            q = exp2((double)dl * c - (double)offset_of(sh->m[qs], a.sc)) / sh->z[qs];
        }
        const double ratio = (q == 0.0) ? 1.0 : fmin(1.0, p / q);
        sh->ratio[t] = (float)ratio;
        rej = !((double)u < ratio);
    }
    const unsigned long long mask = __ballot(rej);
    if (lane == 0) sh->rej[w] = mask;
    __syncthreads();
    if (t == 0) {
        int j = kb;
        for (int i = 0; i < kWaves; ++i) {
            if (sh->rej[i]) {
                j = i * 64 + __ffsll((long long)sh->rej[i]) - 1;
                break;
            }
        }
        Decision d;
        d.j = j;
        d.tok = -1;
        d.Mp = offset_of(sh->m[j], a.sc);
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
            d.Mq = offset_of(sh->m[K + 1 + j], a.sc);
            d.rho = (float)(sh->z[j] / sh->z[K + 1 + j]);
        }
        sh->dec = d;
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// B: one tile of the final row (pair), then (last tile only) the locate.
// ---------------------------------------------------------------------------
struct BShared {
    DecideShared dsh;
    double slab[kWaves][kUnroll];
    int last;
    int g, found, lastpos;
    double base, w, total;
    double red[kWaves];
};

// Wave 0: total mass over the slab slots of request b (waiting for each to be
// visible), then the slab g holding w = u * total and the mass before it.
// Falls back to the last slab with mass when rounding leaves w past the end.
__device__ void find_slab(const VerifyParams& a, const uint64_t* slabs, double u, int* g_out,
                          double* base_out, double* w_out, double* total_out) {
    const int lane = threadIdx.x;
    const int NS = a.NS;
    double total = 0.0;
    for (int g0 = 0; g0 < NS; g0 += 64) {
        double v = 0.0;
        if (g0 + lane < NS) v = dec_f64(slot_wait(slabs + g0 + lane, a.err, enc_f64(0.0)));
        total += __shfl(wave_sum(v), 0, 64);
    }
    const double w = u * total;
    double run = 0.0, base = 0.0, last_base = 0.0;
    int g = -1, last_nz = -1;
    for (int g0 = 0; g0 < NS; g0 += 64) {
        const double v = (g0 + lane < NS) ? dec_f64(slot_peek(slabs + g0 + lane)) : 0.0;
        const double incl = wave_inclusive_scan(v);
        const double up = __shfl_up(incl, 1, 64);
        const double before = run + (lane == 0 ? 0.0 : up);
        const unsigned long long hit = __ballot(w < run + incl);
        const unsigned long long nz = __ballot(v > 0.0);
        if (nz) {
            const int L = 63 - __clzll((long long)nz);
            last_nz = g0 + L;
            last_base = __shfl(before, L, 64);
        }
        if (hit) {
            const int L = __ffsll((long long)hit) - 1;
            g = g0 + L;
            base = __shfl(before, L, 64);
            break;
        }
        run += __shfl(incl, 63, 64);
    }
    if (g < 0) {
        g = last_nz < 0 ? 0 : last_nz;
        base = last_base;
    }
    if (lane == 0) {
        *g_out = g;
        *base_out = base;
        *w_out = w;
        *total_out = total;
    }
}

// The smallest token t with u * S < C_t, the outputs, and the reset of the
// request's slots.  Run by the workgroup that wrote the request's last tile:
// every other tile has counted itself done (its slab slots are awaited) and
// has finished reading the row slots.
template <int DT, bool VEC>
__device__ void locate(const VerifyParams& a, int b, Decision d, BShared* sh) {
    constexpr int E = Elem<DT>::E;
    constexpr int S = Elem<DT>::S;
    const int K = a.K;
    const int kb = k_of(a, b);
    const int nslab = a.C * kUnroll;
    uint64_t* slabs = a.slot_slab + (size_t)b * nslab;
    const double u = (double)a.unif[(size_t)b * (K + 1) + kb];
    const void* rowp = row_ptr(a.target, (size_t)b * (K + 1) + d.j, a.V, S);
    const void* rowq = (d.mode == kResidual) ? row_ptr(a.draft, (size_t)b * K + d.j, a.V, S) : nullptr;
    if (threadIdx.x < 64) {
        find_slab(a, slabs, u, &sh->g, &sh->base, &sh->w, &sh->total);
    } else {
        // Slab slots past the last slab of the row (zeros) must be in before
        // they are reset.
        for (int t = a.NS + threadIdx.x - 64; t < nslab; t += kThreads - 64)
            slot_wait(slabs + t, a.err, (uint64_t)1);
    }
    if (threadIdx.x == 0) {
        sh->found = 0x7FFFFFFF;
        sh->lastpos = -1;
    }
    __syncthreads();
    if (!(sh->total > 0.0)) {
        // Every replacement mass is zero: draw from p_j itself.
        d.mode = kBonus;
        rowq = nullptr;
        for (int g = 0; g < a.NS; ++g) {
            const int v = g * kSlab + threadIdx.x;
            const u32x4 rp = load_raw<DT, VEC, false>(rowp, a.V, a.NV, v);
            float r[E];
            final_masses<DT>(rp, rp, d, v, a.sc, r);
            const double t = block_sum((double)pairwise_sum<E>(r), sh->red);
            if (threadIdx.x == 0) slot_put(slabs + g, enc_f64(t));
        }
        __syncthreads();
        if (threadIdx.x < 64) find_slab(a, slabs, u, &sh->g, &sh->base, &sh->w, &sh->total);
        __syncthreads();
    }
    const int g = sh->g;
    const double base = sh->base, w = sh->w;

    // Re-read slab g and scan it in ascending token id.
    const int v = g * kSlab + threadIdx.x;
    const u32x4 rp = load_raw<DT, VEC, false>(rowp, a.V, a.NV, v);
    const u32x4 rq = rowq ? load_raw<DT, VEC, false>(rowq, a.V, a.NV, v) : neg_inf_raw<DT>();
    float r[E];
    final_masses<DT>(rp, rq, d, v, a.sc, r);
    const double vs = (double)pairwise_sum<E>(r);
    double slab_total;
    const double start = base + block_exclusive_scan(vs, sh->red, &slab_total);
    int lastpos = -1;
#pragma unroll
    for (int e = 0; e < E; ++e)
        if (r[e] > 0.0f) lastpos = v * E + e;
    if (lastpos >= 0) atomicMax(&sh->lastpos, lastpos);
    if (start <= w && vs > 0.0) {
        double Cc = start;
        for (int e = 0; e < E; ++e) {
            Cc += (double)r[e];
            if (w < Cc) {
                atomicMin(&sh->found, v * E + e);
                break;
            }
        }
    }
    __syncthreads();
    const int j = d.j;
    int tok = sh->found != 0x7FFFFFFF ? sh->found : sh->lastpos;
    if (tok < 0) tok = 0;
    for (int i = threadIdx.x; i <= K; i += kThreads) {
        int32_t o = -1;
        if (i < j) o = a.tokens[(size_t)b * K + i];
        else if (i == j) o = tok;
        a.out[(size_t)b * (K + 1) + i] = o;
        if (a.aprob && i < K) a.aprob[(size_t)b * K + i] = (i < kb) ? sh->dsh.ratio[i] : -1.0f;
    }
    if (threadIdx.x == 0) a.nacc[b] = j;

    // Reset the request's slots and counter for the next call.
    const int nrs = kb + 1 + (a.draft ? kb : 0);
    const int nrow = nrs * a.C;
    for (int t = threadIdx.x; t < nrow; t += kThreads) {
        const int rs = t / a.C, c = t % a.C;
        const size_t idx = ((size_t)b * a.R + slot_of_rs(rs, kb, K)) * a.C + c;
        slot_put(a.slot_m + idx, 0u);
        slot_put(a.slot_s + idx, (uint64_t)0);
    }
    for (int t = threadIdx.x; t < nslab; t += kThreads) slot_put(slabs + t, (uint64_t)0);
    if (threadIdx.x == 0) slot_put(a.req_done + b, 0u);
}

template <int DT, bool VEC>
__device__ void b_item(const VerifyParams& a, int item, BShared* sh) {
    constexpr int E = Elem<DT>::E;
    constexpr int S = Elem<DT>::S;
    const int b = item / a.C;
    const int tile = item % a.C;
    decide_block<DT>(a, b, &sh->dsh);
    const Decision d = sh->dsh.dec;
    const void* rowp = row_ptr(a.target, (size_t)b * (a.K + 1) + d.j, a.V, S);
    const void* rowq = (d.mode == kResidual) ? row_ptr(a.draft, (size_t)b * a.K + d.j, a.V, S) : nullptr;
    const int v0 = tile * kTileVec + threadIdx.x;
    const int w = threadIdx.x >> 6;
    u32x4 rp[kUnroll], rq[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int v = v0 + u * kThreads;
        rp[u] = load_raw<DT, VEC, false>(rowp, a.V, a.NV, v);
        rq[u] = rowq ? load_raw<DT, VEC, false>(rowq, a.V, a.NV, v) : neg_inf_raw<DT>();
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        float r[E];
        final_masses<DT>(rp[u], rq[u], d, v0 + u * kThreads, a.sc, r);
        const double t = wave_sum((double)pairwise_sum<E>(r));
        if ((threadIdx.x & 63) == 0) sh->slab[w][u] = t;
    }
    __syncthreads();
    if (threadIdx.x < kUnroll) {
        double t = 0.0;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) t += sh->slab[i][threadIdx.x];
        slot_put(&a.slot_slab[((size_t)b * a.C + tile) * kUnroll + threadIdx.x], enc_f64(t));
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t before = __hip_atomic_fetch_add(a.req_done + b, 1u, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT);
        sh->last = (before + 1u == (uint32_t)a.C);
    }
    __syncthreads();
    if (sh->last) locate<DT, VEC>(a, b, d, sh);
}

// Kernel 1: every A item in its own workgroup (no waits, full occupancy).
template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void verify_rows(VerifyParams a) {
    __shared__ float lds_f[kWaves];
    __shared__ double lds_d[kWaves];
    a_item<DT, VEC>(a, blockIdx.x, lds_f, lds_d);
}

// Kernel 2 (persistent): the B items; the one completing a request's tiles
// also locates its token.
template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void verify_final(VerifyParams a) {
    __shared__ BShared sh;
    for (int item = blockIdx.x; item < a.NB; item += gridDim.x) {
        b_item<DT, VEC>(a, item, &sh);
        __syncthreads();
    }
}

template <int DT, bool VEC>
hipError_t launch(const VerifyParams& p, hipStream_t s) {
    if (p.B == 0) return hipSuccess;
    static int resident[2][2] = {{0, 0}, {0, 0}};
    int& res = resident[DT][VEC ? 1 : 0];
    if (res == 0) {
        int dev = 0, cus = 0, per_cu = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e == hipSuccess)
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, verify_final<DT, VEC>, kThreads, 0);
        if (e != hipSuccess) return e;
        if (cus < 1 || per_cu < 1) return hipErrorInvalidConfiguration;
        res = cus * per_cu;
    }
    hipLaunchKernelGGL((verify_rows<DT, VEC>), dim3((unsigned)p.NA), dim3(kThreads), 0, s, p);
    const int grid = p.NB < res ? p.NB : res;
    hipLaunchKernelGGL((verify_final<DT, VEC>), dim3((unsigned)grid), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_verify(const VerifyParams& p, int dtype, bool vec, hipStream_t s) {
    if (dtype == kBF16) return vec ? launch<kBF16, true>(p, s) : launch<kBF16, false>(p, s);
    return vec ? launch<kFP32, true>(p, s) : launch<kFP32, false>(p, s);
}

}  // namespace specdec
