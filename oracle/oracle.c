/*
 * oracle.c -- plain, slow, fp64 CPU reference for the batched verify step of
 * speculative decoding.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or constant with the
 * GPU library.
 *
 * Sources (web pages; cited by title and section):
 *   [LP]  "3.5 Speculative Decoding" (LLM learning path)
 *   [AIA] "246 Speculative Decoding" (AI in Action)
 *   [MF]  "Speculative Decoding: Mathematical Foundations, Rejection Sampling
 *          Dynamics, Draft Architectures, and Serving Latency"
 *   [SS]  "Speculative Decoding from First Principles" (The Serving Stack)
 *
 * Every value is widened exactly to double before use; every sum runs
 * sequentially in ascending token id.  There is no blocking, fusion or
 * reordering.  Readings taken where the pages are silent or disagree:
 *   - accept iff u < min(1, p/q)  (strict; [LP] "The algorithm (one step)"
 *     writes "<", [AIA] 3.1 and [MF] write "<=").
 *   - q(x) == 0 gives ratio 1 ([AIA] 3.1 accept_or_resample).
 *   - an empty residual (sum <= 0) falls back to p ([AIA] 3.1
 *     residual_distribution).
 *   - the residual / bonus draw is an inverse CDF in ascending token id:
 *     the smallest t with u*S < C_t ([LP], [AIA] only say "sample").
 *   - uniforms[b, i] (i < k_b) drives the accept test of draft i;
 *     uniforms[b, k_b] drives the final draw (residual or bonus).
 *   - argmax ties resolve to the lowest token id.
 *   - p = softmax(l / T), q = softmax(d / T) with one T per call
 *     ([LP] "Notation"; [LP] "Common pitfalls": same processing for both).
 *
 * Parity pins for each function live in the CPU tests (exact enumeration,
 * closed forms, worked examples of the pages, library cross-checks).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_FP32 0
#define ORACLE_BF16 1

/* Exact widening of one stored logit to double.  bf16 is the top half of an
 * IEEE binary32, so shifting its 16 bits into the high half gives the same
 * value as a float. */
static double load_logit(const void *base, int dtype, size_t idx) {
    if (dtype == ORACLE_FP32) {
        return (double)((const float *)base)[idx];
    }
    uint32_t bits = ((uint32_t)((const uint16_t *)base)[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Row statistics of the temperature softmax p_t = exp((l_t - m)/T) / Z:
 * m = max_t l_t and Z = sum_t exp((l_t - m)/T).
 * [LP] "Notation": p is the next-token distribution after temperature. */
static void row_stats(const void *base, int dtype, size_t row_off, int32_t V,
                      double T, double *m_out, double *z_out) {
    double m = -INFINITY;
    for (int32_t t = 0; t < V; ++t) {
        double l = load_logit(base, dtype, row_off + (size_t)t);
        if (l > m) m = l;
    }
    double z = 0.0;
    for (int32_t t = 0; t < V; ++t) {
        double l = load_logit(base, dtype, row_off + (size_t)t);
        z += exp((l - m) / T);
    }
    *m_out = m;
    *z_out = z;
}

/* Probability of token t in a row with known statistics. */
static double row_prob(const void *base, int dtype, size_t row_off, int32_t t,
                       double m, double z, double T) {
    double l = load_logit(base, dtype, row_off + (size_t)t);
    return exp((l - m) / T) / z;
}

int oracle_softmax_stats(const void *logits, int dtype, int64_t rows, int32_t V,
                         double T, double *row_max, double *row_sumexp) {
    if (!logits || !row_max || !row_sumexp || rows < 0 || V <= 0 || !(T > 0.0))
        return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
        row_stats(logits, dtype, (size_t)r * (size_t)V, V, T, &row_max[r],
                  &row_sumexp[r]);
    }
    return 0;
}

/*
 * One batched verify step, request by request, following [LP] "The algorithm
 * (one step)", [AIA] 2.2 and 3.3, [MF] "The Modified Rejection Sampling
 * Algorithm".
 *
 * Layouts (row-major, contiguous):
 *   target      [B, K+1, V]   draft  [B, K, V] or NULL (one-hot drafts)
 *   draft_tokens[B, K] int32  k_per_req [B] or NULL (all K)
 *   uniforms    [B, K+1] fp32
 * Outputs:
 *   out_tokens  [B, K+1]: accepted drafts, then the final token, then -1
 *   num_accepted[B]
 *   accept_prob [B, K] (may be NULL): min(1, p_i/q_i) at every drafted
 *               position i < k_b (also past the first rejection), -1 beyond
 *   min_margin  [B] (may be NULL): smallest distance of a uniform to the
 *               threshold it was compared with, along the path taken
 *               (accept tests up to the first rejection, then the CDF
 *               boundaries around the drawn token, in normalised units)
 */
int oracle_verify(const void *target, const void *draft, int dtype,
                  const int32_t *draft_tokens, const int32_t *k_per_req,
                  const float *uniforms, double T, int32_t B, int32_t K,
                  int32_t V, int32_t *out_tokens, int32_t *num_accepted,
                  double *accept_prob, double *min_margin) {
    if (!target || !draft_tokens || !uniforms || !out_tokens || !num_accepted)
        return -1;
    if (B < 0 || K < 0 || V <= 0 || !(T > 0.0)) return -1;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
    for (int32_t b = 0; b < B; ++b) {
        int32_t k = k_per_req ? k_per_req[b] : K;
        if (k < 0 || k > K) { err |= 1; continue; }
        const int32_t *xt = draft_tokens + (size_t)b * K;
        const float *u = uniforms + (size_t)b * (K + 1);
        int32_t *out = out_tokens + (size_t)b * (K + 1);
        double *r = (double *)malloc(sizeof(double) * (size_t)V);
        if (!r) { err |= 1; continue; }

        /* Step 1 (processed distributions): row statistics of the k+1 target
         * rows and the k draft rows. */
        double pm[K + 1], pz[K + 1], qm[K + 1], qz[K + 1];
        for (int32_t i = 0; i <= k; ++i)
            row_stats(target, dtype, ((size_t)b * (K + 1) + i) * (size_t)V, V,
                      T, &pm[i], &pz[i]);
        if (draft)
            for (int32_t i = 0; i < k; ++i)
                row_stats(draft, dtype, ((size_t)b * K + i) * (size_t)V, V, T,
                          &qm[i], &qz[i]);

        /* Step 2 (accept / reject left to right): ratio_i = min(1, p_i/q_i)
         * at the drafted token; accept iff u_i < ratio_i; stop at the first
         * rejection.  The ratio is also reported past the stop. */
        double margin = INFINITY;
        int32_t j = k; /* index of the first rejection, k if none */
        for (int32_t i = 0; i < k; ++i) {
            int32_t x = xt[i];
            size_t prow = ((size_t)b * (K + 1) + i) * (size_t)V;
            double p = row_prob(target, dtype, prow, x, pm[i], pz[i], T);
            double q = draft ? row_prob(draft, dtype,
                                        ((size_t)b * K + i) * (size_t)V, x,
                                        qm[i], qz[i], T)
                             : 1.0;
            double ratio = (q == 0.0) ? 1.0 : fmin(1.0, p / q);
            if (accept_prob) accept_prob[(size_t)b * K + i] = ratio;
            if (j == k) { /* still on the path */
                double d = fabs((double)u[i] - ratio);
                if (d < margin) margin = d;
                if (!((double)u[i] < ratio)) j = i;
            }
        }
        if (accept_prob)
            for (int32_t i = k; i < K; ++i) accept_prob[(size_t)b * K + i] = -1.0;

        /* Step 3 (final draw).  On a rejection at j the draw is from
         * max(0, p_j - q_j) normalised ([LP] step 3, [AIA] 2.2, [MF]); if
         * every draft was accepted it is the bonus token from p_{k+1}
         * ([LP] step 4, [MF] step 4). */
        size_t prow = ((size_t)b * (K + 1) + j) * (size_t)V;
        for (int32_t t = 0; t < V; ++t) {
            double p = row_prob(target, dtype, prow, t, pm[j], pz[j], T);
            double q = 0.0;
            if (j < k) {
                if (draft)
                    q = row_prob(draft, dtype, ((size_t)b * K + j) * (size_t)V,
                                 t, qm[j], qz[j], T);
                else
                    q = (t == xt[j]) ? 1.0 : 0.0;
            }
            r[t] = (p - q > 0.0) ? (p - q) : 0.0;
        }
        double S = 0.0;
        for (int32_t t = 0; t < V; ++t) S += r[t];
        if (!(S > 0.0)) { /* [AIA] 3.1: p and q coincide, fall back to p */
            for (int32_t t = 0; t < V; ++t)
                r[t] = row_prob(target, dtype, prow, t, pm[j], pz[j], T);
            S = 0.0;
            for (int32_t t = 0; t < V; ++t) S += r[t];
        }
        double uf = (double)u[k];
        double target_mass = uf * S;
        double C = 0.0, C_prev = 0.0;
        int32_t tok = -1;
        for (int32_t t = 0; t < V; ++t) {
            C_prev = C;
            C += r[t];
            if (target_mass < C) { tok = t; break; }
        }
        if (tok < 0) { /* rounding left no t: take the last t with r_t > 0 */
            for (int32_t t = V - 1; t >= 0; --t)
                if (r[t] > 0.0) { tok = t; break; }
            C_prev = C = S;
        }
        double d0 = fabs(uf - C_prev / S), d1 = fabs(uf - C / S);
        double dmin = d0 < d1 ? d0 : d1;
        if (dmin < margin) margin = dmin;

        /* Step 4 (output): accepted prefix, then the final token. */
        for (int32_t i = 0; i < j; ++i) out[i] = xt[i];
        out[j] = tok;
        for (int32_t i = j + 1; i <= K; ++i) out[i] = -1;
        num_accepted[b] = j;
        if (min_margin) min_margin[b] = margin;
        free(r);
    }
    return err ? -1 : 0;
}

/*
 * Greedy verify: p and q are point masses, so a draft is kept iff it equals
 * the target argmax; at the first mismatch the target argmax is emitted; if
 * all k match, the argmax after the last draft is the extra token.
 * [LP] "Proof that the output distribution is exactly p" (last sentence) and
 * "Worked example"; [SS] "Draft, verify, keep what matches".
 * Ties resolve to the lowest token id.
 */
int oracle_verify_greedy(const void *target, int dtype,
                         const int32_t *draft_tokens, const int32_t *k_per_req,
                         int32_t B, int32_t K, int32_t V, int32_t *out_tokens,
                         int32_t *num_accepted, int32_t *argmax_out) {
    if (!target || !draft_tokens || !out_tokens || !num_accepted) return -1;
    if (B < 0 || K < 0 || V <= 0) return -1;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
    for (int32_t b = 0; b < B; ++b) {
        int32_t k = k_per_req ? k_per_req[b] : K;
        if (k < 0 || k > K) { err |= 1; continue; }
        const int32_t *xt = draft_tokens + (size_t)b * K;
        int32_t *out = out_tokens + (size_t)b * (K + 1);
        /* Target argmax of every row that the step may use. */
        int32_t a[K + 1];
        for (int32_t i = 0; i <= k; ++i) {
            size_t off = ((size_t)b * (K + 1) + i) * (size_t)V;
            int32_t best = 0;
            double bv = load_logit(target, dtype, off);
            for (int32_t t = 1; t < V; ++t) {
                double l = load_logit(target, dtype, off + (size_t)t);
                if (l > bv) { bv = l; best = t; }
            }
            a[i] = best;
        }
        if (argmax_out)
            for (int32_t i = 0; i <= K; ++i)
                argmax_out[(size_t)b * (K + 1) + i] = (i <= k) ? a[i] : -1;
        /* First draft that differs from the target argmax; k if none. */
        int32_t j = k;
        for (int32_t i = 0; i < k; ++i)
            if (xt[i] != a[i]) { j = i; break; }
        int32_t a_j = a[j];
        for (int32_t i = 0; i < j; ++i) out[i] = xt[i];
        out[j] = a_j;
        for (int32_t i = j + 1; i <= K; ++i) out[i] = -1;
        num_accepted[b] = j;
    }
    return err ? -1 : 0;
}

/*
 * Acceptance telemetry per drafted position i (0-based), over the requests
 * of one verify step, added to counters[3][K]:
 *   counters[0][i] (drafted)  += #{b : i < k_b}
 *   counters[1][i] (tested)   += #{b : i < k_b and i <= n_b}
 *   counters[2][i] (accepted) += #{b : i < n_b}
 * with n_b = num_accepted[b].  Position i is tested exactly when every
 * earlier draft was accepted.  The serving engine's counters of drafted and
 * accepted tokens ([SS] "What the numbers say", per-position acceptance
 * falling along the draft) and the acceptance rate measured over the tests
 * performed ([AIA] 3.4).
 */
int oracle_acceptance_counts(const int32_t *num_accepted, const int32_t *k_per_req,
                             int32_t B, int32_t K, uint64_t *counters) {
    if (!num_accepted || !counters || B < 0 || K < 0) return -1;
    for (int32_t b = 0; b < B; ++b) {
        const int32_t k = k_per_req ? k_per_req[b] : K;
        const int32_t n = num_accepted[b];
        if (k < 0 || k > K || n < 0 || n > k) return -1;
        for (int32_t i = 0; i < K; ++i) {
            if (i < k) counters[i] += 1;
            if (i < k && i <= n) counters[(size_t)K + i] += 1;
            if (i < n) counters[2 * (size_t)K + i] += 1;
        }
    }
    return 0;
}

/*
 * Draft length from the counters.  alpha_test = sum accepted / sum tested
 * (the per-draft acceptance probability of the independent-acceptance
 * model); alpha_draft = sum accepted / sum drafted (the engine counter
 * ratio).  Under independent acceptance with probability alpha a step emits
 * sum_{i=0..k} alpha^i tokens on average and costs 1 + c k target passes (c
 * = draft-to-target cost ratio), so the speedup over plain decoding is their
 * quotient ([LP] "Expected tokens per step", "Speedup" and the worked
 * example's table for choosing k; [AIA] 2.4, 3.5).  Returns the k in
 * [k_min, k_max] with the largest speedup at alpha = alpha_test (the
 * smallest such k on ties) and that speedup.  With no tested position
 * alpha_test is 0 (and k_min is chosen).
 */
int oracle_choose_k(const uint64_t *counters, int32_t K, double c, int32_t k_min,
                    int32_t k_max, double *alpha_test, double *alpha_draft, int32_t *k_out,
                    double *speedup_out) {
    if (!counters || !k_out || K < 0 || k_min < 0 || k_max < k_min || !(c >= 0.0)) return -1;
    double drafted = 0.0, tested = 0.0, accepted = 0.0;
    for (int32_t i = 0; i < K; ++i) {
        drafted += (double)counters[i];
        tested += (double)counters[(size_t)K + i];
        accepted += (double)counters[2 * (size_t)K + i];
    }
    const double a = tested > 0.0 ? accepted / tested : 0.0;
    if (alpha_test) *alpha_test = a;
    if (alpha_draft) *alpha_draft = drafted > 0.0 ? accepted / drafted : 0.0;
    int32_t best_k = k_min;
    double best = -1.0;
    for (int32_t k = k_min; k <= k_max; ++k) {
        double tokens = 0.0, power = 1.0;
        for (int32_t i = 0; i <= k; ++i) {
            tokens += power;
            power *= a;
        }
        const double speedup = tokens / (1.0 + c * (double)k);
        if (speedup > best) {
            best = speedup;
            best_k = k;
        }
    }
    *k_out = best_k;
    if (speedup_out) *speedup_out = best;
    return 0;
}

/*
 * n-gram (prompt-lookup) drafter: find the last few tokens earlier in the
 * context and propose what followed them there ([LP] "Choosing a draft",
 * n-gram / prompt lookup row; [MF] "Non-Parametric Drafters": match n-grams
 * in the prompt and speculate the tokens that followed; [SS] "Four kinds of
 * drafter", n-gram lookup).  Readings where the pages are silent:
 *   - the context is every token so far (prompt and output), c[0..L-1];
 *   - longer suffixes first: n from n_max down to n_min;
 *   - for a given n, the latest earlier occurrence: the largest end e < L-1
 *     with c[e-n+1..e] == c[L-n..L-1];
 *   - the proposal is c[e+1 .. e+K], cut at the end of the context (it may
 *     run into the suffix itself); k_b is its length;
 *   - no occurrence for any n: k_b = 0.
 * draft_tokens[b, i] = -1 for i >= k_b.
 */
int oracle_ngram_propose(const int32_t *context, const int32_t *context_len, int32_t B,
                         int32_t L_stride, int32_t n_min, int32_t n_max, int32_t K,
                         int32_t *draft_tokens, int32_t *k_per_req) {
    if (!context || !context_len || !draft_tokens || !k_per_req) return -1;
    if (B < 0 || K < 0 || n_min < 1 || n_max < n_min || L_stride < 0) return -1;
    for (int32_t b = 0; b < B; ++b) {
        const int32_t L = context_len[b];
        if (L < 0 || L > L_stride) return -1;
        const int32_t *c = context + (size_t)b * L_stride;
        int32_t found_e = -1;
        for (int32_t n = n_max; n >= n_min && found_e < 0; --n) {
            if (n > L - 1) continue;   /* the suffix needs an earlier occurrence */
            for (int32_t e = L - 2; e >= n - 1; --e) {
                int32_t m = 0;
                while (m < n && c[e - m] == c[L - 1 - m]) ++m;
                if (m == n) {
                    found_e = e;
                    break;
                }
            }
        }
        int32_t kb = 0;
        if (found_e >= 0) {
            kb = L - 1 - found_e;
            if (kb > K) kb = K;
        }
        for (int32_t i = 0; i < K; ++i)
            draft_tokens[(size_t)b * K + i] = (i < kb) ? c[found_e + 1 + i] : -1;
        k_per_req[b] = kb;
    }
    return 0;
}

/*
 * Greedy tree verification ([LP] "Tree verification": a tree of drafted
 * nodes flattened into one sequence, every node attending to its ancestors
 * only; one target pass scores all nodes; keep the longest root-to-leaf
 * path that passes verification; [MF] "Tree-Based Verification and Custom
 * Attention Masks").  Greedy acceptance (the chain rule applied along each
 * path, [LP] "Worked example"):
 *   - node n (flattened order, parent[n] < n, -1 = child of the root) is
 *     accepted iff its parent is accepted (the root always is) and its token
 *     equals the argmax of the parent's target row (row 0 = the root's,
 *     row p + 1 = the row after node p);
 *   - the kept path ends at the deepest accepted node, the lowest index on
 *     ties (only when siblings repeat a token);
 *   - the emitted tokens are the path's tokens, root side first, then the
 *     argmax of the row after the path's last node (row 0 when no node is
 *     accepted); num_accepted is the path length.
 * target [B, N+1, V]; node_tokens, parents [B, N]; n_nodes [B] or NULL (N).
 * out_tokens [B, N+1] (-1 padded); path_nodes [B, N] (node indices, root
 * side first, -1 padded); num_accepted [B].
 */
int oracle_tree_verify_greedy(const void *target, int dtype, const int32_t *node_tokens,
                              const int32_t *parents, const int32_t *n_nodes, int32_t B,
                              int32_t N, int32_t V, int32_t *out_tokens, int32_t *path_nodes,
                              int32_t *num_accepted) {
    if (!target || !out_tokens || !num_accepted || B < 0 || N < 0 || V <= 0) return -1;
    if (N > 0 && (!node_tokens || !parents)) return -1;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
    for (int32_t b = 0; b < B; ++b) {
        const int32_t n_b = n_nodes ? n_nodes[b] : N;
        if (n_b < 0 || n_b > N) { err |= 1; continue; }
        const int32_t *tok = node_tokens + (size_t)b * N;
        const int32_t *par = parents + (size_t)b * N;
        int32_t amax[N + 1], depth[N + 1], acc[N + 1];
        for (int32_t r = 0; r <= n_b; ++r) {
            size_t off = ((size_t)b * (N + 1) + r) * (size_t)V;
            int32_t best = 0;
            double bv = load_logit(target, dtype, off);
            for (int32_t t = 1; t < V; ++t) {
                double l = load_logit(target, dtype, off + (size_t)t);
                if (l > bv) { bv = l; best = t; }
            }
            amax[r] = best;
        }
        int32_t end = -1, end_depth = 0;
        for (int32_t n = 0; n < n_b; ++n) {
            const int32_t p = par[n];
            if (p < -1 || p >= n) { err |= 1; break; }
            const int32_t parent_ok = (p < 0) ? 1 : acc[p];
            acc[n] = parent_ok && tok[n] == amax[p + 1];
            depth[n] = (p < 0) ? 1 : depth[p] + 1;
            if (acc[n] && depth[n] > end_depth) { end = n; end_depth = depth[n]; }
        }
        int32_t *out = out_tokens + (size_t)b * (N + 1);
        int32_t *path = path_nodes ? path_nodes + (size_t)b * N : NULL;
        for (int32_t i = 0; i <= N; ++i) out[i] = -1;
        if (path) for (int32_t i = 0; i < N; ++i) path[i] = -1;
        for (int32_t n = end, d = end_depth - 1; n >= 0; n = par[n], --d) {
            out[d] = tok[n];
            if (path) path[d] = n;
        }
        out[end_depth] = amax[end + 1];
        num_accepted[b] = end_depth;
    }
    return err ? -1 : 0;
}

/*
 * Tree attention metadata ([LP] "Tree verification": each flattened node
 * attends to the context, its ancestors and itself, never to siblings or
 * cousins; nodes at equal depth share a position index; [MF] "Tree-Based
 * Verification and Custom Attention Masks": the mask admits j for i exactly
 * when j is an ancestor of i).  Reading: the diagonal is admitted, as in the
 * [LP] mask table.
 *   mask[b, i, j] = 1 iff j == i or j is an ancestor of i, else 0 (j < n_b);
 *                   rows and columns at or beyond n_b are 0;
 *   depth[b, i]   = 1 for a child of the root, depth of the parent + 1
 *                   otherwise; -1 at or beyond n_b.
 * parents [B, N] (parent[n] < n, -1 = root); n_nodes [B] or NULL (N).
 * mask [B, N, N] bytes; depth [B, N].
 */
int oracle_tree_mask(const int32_t *parents, const int32_t *n_nodes, int32_t B, int32_t N,
                     uint8_t *mask, int32_t *depth) {
    if (B < 0 || N < 0 || !mask || !depth || (N > 0 && !parents)) return -1;
    int err = 0;
    for (int32_t b = 0; b < B; ++b) {
        const int32_t n_b = n_nodes ? n_nodes[b] : N;
        const int32_t *par = parents + (size_t)b * N;
        uint8_t *m = mask + (size_t)b * N * N;
        int32_t *d = depth + (size_t)b * N;
        for (size_t i = 0; i < (size_t)N * N; ++i) m[i] = 0;
        for (int32_t i = 0; i < N; ++i) d[i] = -1;
        if (n_b < 0 || n_b > N) { err = 1; continue; }
        for (int32_t i = 0; i < n_b; ++i) {
            if (par[i] < -1 || par[i] >= i) { err = 1; break; }
            d[i] = par[i] < 0 ? 1 : d[par[i]] + 1;
            for (int32_t j = i; j >= 0; j = par[j]) m[(size_t)i * N + j] = 1;
        }
    }
    return err ? -1 : 0;
}

/*
 * Processed distributions: top-k, then top-p, after temperature ([LP]
 * "Notation": p is the target's distribution after temperature, top-p and
 * the like; [LP] "Common pitfalls" and [AIA] Key takeaways: the target and
 * the draft go through the same temperature / top-k / top-p pipeline, else
 * the guarantee breaks).  The pages name the two filters without defining
 * them; the plain readings taken:
 *   - top-k (0 < top_k < V): keep every token whose logit is at least the
 *     top_k-th largest logit of the row (counted with multiplicity; ties at
 *     that value are all kept); top_k <= 0 or >= V keeps every token;
 *   - top-p (0 < top_p < 1), applied to the top-k survivors renormalised:
 *     keep every token whose logit is at least tau, the largest logit value
 *     v for which the survivors with logit >= v hold at least top_p of the
 *     survivors' probability; top_p >= 1 keeps every survivor;
 *   - the processed distribution is softmax(l / T) restricted to the kept
 *     tokens and renormalised.
 * Both filters keep an upper set of logit values, so each row's processing
 * is one floor: the kept tokens are exactly those with l >= floor (-inf
 * when nothing is cut).  floor[r] is the floor of row r.  margin[r] (may be
 * NULL) is, when top-p decides the floor, the distance of top_p * Z_k from
 * the nearer of the two cumulative masses that bracket it (the mass at or
 * above tau and the mass strictly above it), relative to Z_k; +inf
 * otherwise.  A small margin marks a row whose kept set a rounding of the
 * masses could change.
 */
static int cmp_desc(const void *a, const void *b) {
    const double x = *(const double *)a, y = *(const double *)b;
    return (x < y) - (x > y);
}

int oracle_sampling_floor(const void *logits, int dtype, int64_t rows, int32_t V, double T,
                          int32_t top_k, double top_p, float *floor_out, double *margin) {
    if (!logits || !floor_out || rows < 0 || V <= 0 || !(T > 0.0) || !(top_p > 0.0))
        return -1;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
    for (int64_t r = 0; r < rows; ++r) {
        double *s = (double *)malloc(sizeof(double) * (size_t)V);
        if (!s) { err |= 1; continue; }
        for (int32_t t = 0; t < V; ++t) s[t] = load_logit(logits, dtype, (size_t)r * V + t);
        qsort(s, (size_t)V, sizeof(double), cmp_desc);       /* largest first */
        /* top-k: the top_k-th largest value, with multiplicity. */
        const double theta_k = (top_k > 0 && top_k < V) ? s[top_k - 1] : -INFINITY;
        double fl = theta_k, mg = INFINITY;
        if (top_p < 1.0) {
            /* Survivors' masses exp((l - m) / T), m the row max. */
            const double m = s[0];
            double zk = 0.0;
            for (int32_t i = 0; i < V && s[i] >= theta_k; ++i) zk += exp((s[i] - m) / T);
            const double w = top_p * zk;
            /* Walk the distinct values from the largest: tau is the first
             * value at which the mass at or above it reaches w. */
            double cum = 0.0;
            for (int32_t i = 0; i < V && s[i] >= theta_k;) {
                const double v = s[i];
                const double below = cum;
                while (i < V && s[i] == v) cum += exp((s[i++] - m) / T);
                if (cum >= w) {
                    fl = v;
                    mg = fmin(cum - w, w - below) / zk;
                    break;
                }
            }
        }
        floor_out[r] = (float)fl;
        if (margin) margin[r] = mg;
        free(s);
    }
    return err ? -1 : 0;
}
