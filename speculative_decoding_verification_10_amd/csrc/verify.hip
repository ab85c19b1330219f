// Stochastic verify step on gfx950: two stream-ordered kernels over three
// kinds of work.  verify_rows runs every A item in its own workgroup;
// verify_final is persistent (each workgroup takes items blockIdx.x,
// blockIdx.x + gridDim.x, ...; the grid is sized so that every workgroup is
// resident at once) and runs the B items, the last of each request also
// doing its L step:
//
//  A  (position p, request b, target|draft, tile c), position-major: tile max
//     and sum of exponentials of target row p <= k_b or draft row p < k_b
//     ("3.5 Speculative Decoding", "Notation": p and q are the
//     temperature-processed distributions).  Rows past k_b are skipped.
//  B  (request b, tile c): the accept test of request b -- u_i < min(1,
//     p_i(x_i)/q_i(x_i)) left to right, first rejection j by a wavefront
//     ballot ("The algorithm (one step)", step 3) -- then tile c of the
//     final row (pair): slab sums of the unnormalised replacement masses
//     max(0, p_j - q_j), or of p_{k_b} when every draft was accepted (step 4).
//  L  (request b, by the workgroup that completes its last B item): the slab
//     that holds u * S (prefix over slab sums), a re-read of that one slab,
//     the smallest token t with u * S < C_t; then the outputs, and the reset
//     of the request's slots.
//
// A -> B -> L hand-offs go through self-validating slots and a per-request
// completion counter (slots.h).  The kernel boundary separates A from B; the
// only wait inside verify_final is for slab slots of tiles whose workgroups
// have already counted themselves done, so it always ends.
//
// Masses are kept unnormalised: the replacement is Z_p * max(0, p - q) =
// max(0, e_p - (Z_p/Z_q) e_q) with e = exp2((x - max) * c), the bonus is e_p.
// An inverse CDF only needs the masses up to a common factor.
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

// Row statistics from the tile slots of one row, read once.  Returns false
// when a tile has not been written yet (the values are then meaningless).
__device__ bool row_from_slots(const VerifyParams& a, size_t rid, float* m_out, double* z_out) {
    constexpr int G = 8;
    const uint32_t* sm = a.slot_m + rid * a.C;
    const uint64_t* ss = a.slot_s + rid * a.C;
    bool ok = true;
    float m = -INFINITY;
    double z = 0.0;
    for (int g0 = 0; g0 < a.C; g0 += G) {
        uint32_t um[G];
        uint64_t us[G];
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const bool in = g0 + i < a.C;
            um[i] = in ? slot_peek(sm + g0 + i) : enc_f32(-INFINITY);
            us[i] = in ? slot_peek(ss + g0 + i) : enc_f64(0.0);
        }
        float gm = m;
#pragma unroll
        for (int i = 0; i < G; ++i) {
            ok = ok && um[i] != 0u && us[i] != 0ull;
            gm = fmaxf(gm, dec_f32(um[i]));
        }
        if (!ok) break;
        if (gm != -INFINITY) {
            const double Mg = (double)offset_of(gm, a.sc);
            if (m != -INFINITY && gm > m) z *= exp2((double)offset_of(m, a.sc) - Mg);
#pragma unroll
            for (int i = 0; i < G; ++i) {
                const float mi = dec_f32(um[i]);
                if (mi != -INFINITY) z += dec_f64(us[i]) * exp2((double)offset_of(mi, a.sc) - Mg);
            }
            m = gm;
        }
    }
    *m_out = m;
    *z_out = z;
    return ok;
}

// ---------------------------------------------------------------------------
// The accept test of request b, by wave 0 of a workgroup.  Lane i handles
// draft position i (lane k_b the bonus row).  The gathers at the draft
// tokens are issued before any wait; then the tile slots are polled until
// the positions up to the first rejection (or all of them) are known.  With
// need_all (accept_prob requested) every drafted position is waited for and
// its ratio written to accept_prob.  Writes the decision to *dec.
// ---------------------------------------------------------------------------
template <int DT>
__device__ void decide(const VerifyParams& a, int b, bool need_all, Decision* dec) {
    constexpr int S = Elem<DT>::S;
    const int lane = threadIdx.x;
    const int K = a.K;
    const int kb = k_of(a, b);
    const bool one_hot = (a.draft == nullptr);
    const double c = a.sc.c;
    int j = -1;
    float fmp = 0.0f, fmq = 0.0f;
    double fzp = 1.0, fzq = 1.0;
    for (int base = 0; base <= kb; base += 64) {
        const int i = min(base + lane, K);
        const bool pos = (base + lane < kb);
        const bool need = (base + lane <= kb);
        const int x = (i < K) ? token_of(a, b, i) : 0;
        const float u = a.unif[(size_t)b * (K + 1) + i];
        const float l = load_one<DT>(row_ptr(a.target, (size_t)b * (K + 1) + i, a.V, S), x);
        float dl = 0.0f;
        if (!one_hot && K > 0)
            dl = load_one<DT>(row_ptr(a.draft, (size_t)b * K + min(i, K - 1), a.V, S), x);
        bool ready = !need, rej = false;
        double ratio = -1.0;
        float mp = 0.0f, mq = 0.0f;
        double zp = 1.0, zq = 1.0;
        int spins = 0;
        for (;;) {
            if (!ready) {
                bool ok = row_from_slots(a, (size_t)b * a.R + i, &mp, &zp);
                if (ok && pos && !one_hot) ok = row_from_slots(a, (size_t)b * a.R + K + 1 + i, &mq, &zq);
                if (ok) {
                    ready = true;
                    if (pos) {
                        const double p = exp2((double)l * c - (double)offset_of(mp, a.sc)) / zp;
                        const double q = one_hot ? 1.0
                                                 : exp2((double)dl * c - (double)offset_of(mq, a.sc)) / zq;
                        ratio = (q == 0.0) ? 1.0 : fmin(1.0, p / q);
                        rej = !((double)u < ratio);
                    }
                }
            }
            const unsigned long long rmask = __ballot(ready);
            const unsigned long long jmask = __ballot(ready && rej);
            const bool all_ready = (rmask == ~0ull);
            const int prefix = all_ready ? 64 : __ffsll((long long)~rmask) - 1;
            const int first = jmask ? __ffsll((long long)jmask) - 1 : 64;
            int src = -1;
            if (j < 0) {
                if (first < prefix) {
                    j = base + first;
                    src = first;
                } else if (all_ready && kb < base + 64) {
                    j = kb;
                    src = kb - base;
                }
            }
            if (src >= 0) {
                fmp = __shfl(mp, src, 64);
                fzp = __shfl(zp, src, 64);
                fmq = __shfl(mq, src, 64);
                fzq = __shfl(zq, src, 64);
            }
            if (need_all ? all_ready : (j >= 0 || all_ready)) break;
            if (++spins > kSpinLimit) {
                if (lane == 0) atomicOr(a.err, 1u);
                if (j < 0) j = kb;
                break;
            }
            poll_pause();
        }
        if (need_all && pos && a.aprob) a.aprob[(size_t)b * K + i] = (float)ratio;
        if (j >= 0 && !need_all) break;
    }
    if (j < 0) j = kb;
    if (lane == 0) {
        Decision d;
        d.j = j;
        d.tok = -1;
        d.Mp = offset_of(fmp, a.sc);
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
            d.Mq = offset_of(fmq, a.sc);
            d.rho = (float)(fzp / fzq);
        }
        *dec = d;
    }
}

// ---------------------------------------------------------------------------
// B: one tile of the final row (pair) of request b.  Writes the tile's 8 slab
// sums; the workgroup that completes the request's last tile then locates the
// token (L below).
// ---------------------------------------------------------------------------
struct BShared {
    Decision dec;
    double slab[kWaves][8];
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

// L: the smallest token t with u * S < C_t, the outputs, and the reset of the
// request's slots.  Run by the workgroup that wrote the request's last tile;
// every other tile of the request has been written (its slab slots are
// awaited) and has finished reading the row slots.
template <int DT, bool VEC>
__device__ void locate(const VerifyParams& a, int b, Decision d, BShared* sh) {
    constexpr int E = Elem<DT>::E;
    constexpr int S = Elem<DT>::S;
    const int K = a.K;
    const int kb = k_of(a, b);
    uint64_t* slabs = a.slot_slab + (size_t)b * a.C * kUnroll;
    const double u = (double)a.unif[(size_t)b * (K + 1) + kb];
    const void* rowp = row_ptr(a.target, (size_t)b * (K + 1) + d.j, a.V, S);
    const void* rowq = (d.mode == kResidual) ? row_ptr(a.draft, (size_t)b * K + d.j, a.V, S) : nullptr;
    if (threadIdx.x < 64) find_slab(a, slabs, u, &sh->g, &sh->base, &sh->w, &sh->total);
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
        if (a.aprob && i < K && i >= kb) a.aprob[(size_t)b * K + i] = -1.0f;
    }
    if (threadIdx.x == 0) a.nacc[b] = j;
    // accept_prob needs every drafted position (also past the rejection).
    if (a.aprob && threadIdx.x < 64) decide<DT>(a, b, true, &sh->dec);
    __syncthreads();

    // Reset the request's slots and counter for the next call.
    const int nrow_slots = kb + 1 + (a.draft ? kb : 0);
    const int nrow = nrow_slots * a.C;
    for (int t = threadIdx.x; t < nrow; t += kThreads) {
        const int rs = t / a.C, c = t % a.C;
        const int slot = rs <= kb ? rs : (K + 1) + (rs - kb - 1);
        const size_t idx = ((size_t)b * a.R + slot) * a.C + c;
        slot_put(a.slot_m + idx, 0u);
        slot_put(a.slot_s + idx, (uint64_t)0);
    }
    for (int t = threadIdx.x; t < a.C * kUnroll; t += kThreads) {
        slot_wait(slabs + t, a.err, (uint64_t)1);
        slot_put(slabs + t, (uint64_t)0);
    }
    if (threadIdx.x == 0) slot_put(a.req_done + b, 0u);
}

template <int DT, bool VEC>
__device__ void b_item(const VerifyParams& a, int item, BShared* sh) {
    constexpr int E = Elem<DT>::E;
    constexpr int S = Elem<DT>::S;
    const int b = item / a.C;
    const int tile = item % a.C;
    if (threadIdx.x < 64) decide<DT>(a, b, false, &sh->dec);
    __syncthreads();
    const Decision d = sh->dec;
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
// also locates its token.  Nothing waits except for slab slots that are
// already written.
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
