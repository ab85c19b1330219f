/*
 * specdec.h -- C ABI of the batched verify step of speculative decoding on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (one step, every request b of a batch independently):
 *   p_i = softmax(target_logits[b, i, :] / T)       i = 0 .. k_b
 *   q_i = softmax(draft_logits[b, i, :] / T)        i = 0 .. k_b - 1
 *         (or the point mass on draft_tokens[b, i] when draft_logits is NULL)
 *   for i = 0 .. k_b-1: accept draft_tokens[b, i] iff u_i < min(1, p_i(x)/q_i(x));
 *   stop at the first rejection j; emit a replacement drawn from
 *   max(0, p_j - q_j) normalised; if every draft was accepted emit a bonus
 *   token drawn from p_{k_b}.
 * Sources: "3.5 Speculative Decoding" (LLM learning path), sections
 * "Notation" and "The algorithm (one step)"; "246 Speculative Decoding"
 * (AI in Action), sections 2.2 and 3.1-3.3; "Speculative Decoding:
 * Mathematical Foundations, ...", section "The Modified Rejection Sampling
 * Algorithm".  The greedy variant ("3.5 Speculative Decoding", section
 * "Proof that the output distribution is exactly p", last paragraph, and the
 * "Worked example"; "Speculative Decoding from First Principles", section
 * "Draft, verify, keep what matches") keeps a draft iff it equals the target
 * argmax and otherwise emits that argmax.
 *
 * Conventions shared by every entry point
 *   - All array pointers are DEVICE pointers (memory of the current HIP
 *     device), owned by the caller; the library keeps none of them after the
 *     call returns and allocates no memory.
 *   - Arrays are row-major and contiguous.  Logits are fp32 or bf16 (raw
 *     IEEE bfloat16, the top half of a binary32).
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream) and never synchronise with the host.  Outputs are valid once
 *     the stream has reached the call.
 *   - Return value: SPECDEC_OK (0) or a negative specdec_status_t.  Argument
 *     errors are detected on the host before anything is launched and leave
 *     every output untouched.  No C++ exception crosses the ABI.
 *   - Workspace: device memory of at least the size the matching
 *     *_workspace_bytes() function returns, 256-byte aligned.  The first 4
 *     bytes hold error bits: a call ORs in a bit when an internal bounded
 *     wait gives up, which a correct run on an unshared GPU never does (the
 *     affected outputs are then marked invalid); specdec_workspace_errors
 *     reads them, specdec_workspace_init clears them.  Every call sets each
 *     other scratch word it reads earlier in the same call, so a workspace
 *     needs no initialisation beyond a clear error word, may hold anything
 *     else, and may be shared by calls of different entry points and shapes
 *     that do not run concurrently.  Calls that may run concurrently need
 *     distinct workspaces.
 *   - Preconditions not checked on the fast path (a violation gives
 *     unspecified tokens, never an out-of-bounds access): logits finite or
 *     -inf (-inf = probability 0; a row may not be all -inf); 0 <=
 *     draft_tokens < V at the positions that are used; 0 <= uniforms < 1;
 *     0 <= k_per_req[b] <= K.  Rows past k_b (target rows i > k_b, draft
 *     rows i >= k_b) are never read.
 */
#ifndef SPECDEC_H
#define SPECDEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SPECDEC_FP32 = 0,
    SPECDEC_BF16 = 1
} specdec_dtype_t;

typedef enum {
    SPECDEC_OK = 0,
    SPECDEC_EINVAL = -1,     /* null pointer, bad size, bad temperature */
    SPECDEC_EDTYPE = -2,     /* unknown dtype */
    SPECDEC_EWORKSPACE = -3, /* workspace missing, too small or misaligned */
    SPECDEC_ELAUNCH = -4,    /* a kernel launch failed (HIP error) */
    SPECDEC_EDEVICE = -5,    /* no usable gfx950 device: a launch failed on a device of another
                                architecture (the library holds gfx950 code only), or the
                                allocation-free entry point found no current device */
    SPECDEC_ESCRATCH = -6    /* too large for the static scratch of specdec_verify_noalloc */
} specdec_status_t;

/* Size of the static scratch behind specdec_verify_noalloc, per GPU. */
#define SPECDEC_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/* Human-readable name of a status code (static storage). */
const char *specdec_status_string(int status);

/* Library version string (static storage). */
const char *specdec_version(void);

/* Zero-fill `bytes` of workspace on `stream` (asynchronous); clears the error bits. */
int specdec_workspace_init(void *workspace, size_t bytes, void *stream);

/*
 * The error word of a workspace: the bits that calls on it OR in when one of
 * their bounded in-kernel waits gives up (bit 0: the final draw of the
 * stochastic verify step, whose affected requests then read num_accepted = -1
 * and out_tokens = -1 throughout).  Copies the word to errors[0] (4 bytes of
 * DEVICE memory, owned by the caller) on `stream`, after every call enqueued
 * before it on that stream, and clears it in the same atomic step when
 * `clear` is non-zero.  Asynchronous like every call: errors[0] is valid once
 * the stream has reached it.  A call on a workspace also used on another
 * stream sees that stream's calls only as ordered by the caller.
 * SPECDEC_EINVAL for a NULL or misaligned workspace or a NULL errors.
 */
int specdec_workspace_errors(void *workspace, uint32_t *errors, int clear, void *stream);

/*
 * For tests of the error path above (callers that must see a wait give up
 * without a fault or a hang; not for production use).  Every stochastic
 * verify call issued after this one, from any thread, gives up a bounded
 * wait after `wait_ticks` ticks of the GPU's 100 MHz clock instead of the
 * library's 5,000,000 (50 ms), and, when `withhold_tile` >= 0, final tile
 * `withhold_tile` of every request publishes no slab sums, so that the
 * request's search waits for them and gives up: its outputs read -1 and bit
 * 0 of the workspace's error word is set, every kernel still exits.  Rows
 * of a single 16 KB tile (fp32 V <= 4,096, bf16 V <= 8,192) have no such
 * wait (their search reads its own workgroup's sums) and are not affected.
 * specdec_debug_bounded_wait(0, -1) restores the defaults.  SPECDEC_EINVAL
 * for withhold_tile < -1.
 */
int specdec_debug_bounded_wait(uint64_t wait_ticks, int32_t withhold_tile);

/*
 * Row statistics of the temperature softmax ("3.5 Speculative Decoding",
 * section "Notation": p is the distribution after temperature).
 *   logits      [rows, V]
 *   row_max     [rows] fp32 out: max_t l_t (raw logit units, exact)
 *   row_sumexp  [rows] fp32 out: sum_t exp((l_t - row_max) / T)
 * rows >= 0, V >= 1, T > 0 and finite.
 */
size_t specdec_softmax_stats_workspace_bytes(int64_t rows, int32_t V, specdec_dtype_t dtype);
int specdec_softmax_stats(const void *logits, specdec_dtype_t dtype, int64_t rows, int32_t V,
                          float temperature, float *row_max, float *row_sumexp,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * Stochastic verify step (the operation above).
 *   target_logits [B, K+1, V]
 *   draft_logits  [B, K, V], or NULL: drafts are point masses (n-gram /
 *                 prompt-lookup drafts), so the accept probability is
 *                 p_i(x) and the replacement is p_j with x removed,
 *                 renormalised.
 *   draft_tokens  [B, K] int32
 *   k_per_req     [B] int32, or NULL (every request has k_b = K)
 *   uniforms      [B, K+1] fp32 in [0, 1): uniforms[b, i] (i < k_b) drives
 *                 the accept test of draft i, uniforms[b, k_b] the final
 *                 draw (replacement or bonus); the others are ignored.
 *   temperature   one T > 0 for both distributions of every request.
 * Outputs:
 *   out_tokens    [B, K+1] int32: accepted drafts, then the final token,
 *                 then -1.  Emitted count = num_accepted[b] + 1.
 *   num_accepted  [B] int32
 *   accept_prob   [B, K] fp32, or NULL: min(1, p_i(x)/q_i(x)) at every
 *                 drafted position i < k_b (also past the first rejection),
 *                 -1 for i >= k_b.
 * The final draw is an inverse CDF in ascending token id: the smallest t
 * with u * S < C_t, C_t the running sum of the (unnormalised) replacement or
 * bonus masses and S their total.  0 <= B <= 65535, 0 <= K <= 255,
 * 1 <= V <= 2^28; larger values, or more than 2^24 row tiles (B * (2K+1)
 * rows of 16 KB tiles), give SPECDEC_EINVAL.
 */
size_t specdec_verify_workspace_bytes(int32_t B, int32_t K, int32_t V, specdec_dtype_t dtype,
                                      int one_hot_drafts);
int specdec_verify(const void *target_logits, const void *draft_logits, specdec_dtype_t dtype,
                   const int32_t *draft_tokens, const int32_t *k_per_req, const float *uniforms,
                   float temperature, int32_t B, int32_t K, int32_t V,
                   int32_t *out_tokens, int32_t *num_accepted, float *accept_prob,
                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * specdec_verify for callers that cannot allocate device memory -- code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc: the same operation, arguments, results and preconditions, with
 * no workspace argument.  Its scratch is a static array of
 * SPECDEC_NOALLOC_SCRATCH_BYTES (16 MiB) inside the library, one copy on
 * every GPU the library runs on, held until the process ends; the call
 * allocates nothing (its first call on a device only looks the array up).
 *   - It runs on the current HIP device, which must be the stream's.
 *   - Calls whose specdec_verify_workspace_bytes() exceeds the scratch
 *     return SPECDEC_ESCRATCH before anything is launched (at V = 128256
 *     bf16 with draft logits: up to B = 3,830 requests at K = 5; at
 *     V = 151936 fp32, K = 8: B = 1,286).
 *   - Every call on one GPU shares that GPU's scratch, which keeps the last
 *     call's contents: calls that may overlap on one GPU (other streams,
 *     other host threads) race and must be serialised by the caller.
 *   - The scratch's error word is cleared at the start of every call; a
 *     request whose bounded in-kernel wait gave up reads num_accepted = -1
 *     and out_tokens = -1 (specdec_workspace_errors does not apply: the
 *     scratch is not the caller's).
 */
int specdec_verify_noalloc(const void *target_logits, const void *draft_logits,
                           specdec_dtype_t dtype, const int32_t *draft_tokens,
                           const int32_t *k_per_req, const float *uniforms, float temperature,
                           int32_t B, int32_t K, int32_t V, int32_t *out_tokens,
                           int32_t *num_accepted, float *accept_prob, void *stream);

/*
 * specdec_verify with per-phase timing, for telemetry and benchmarks: the
 * same operation, arguments and results, and in addition the caller's HIP
 * events (hipEvent_t, created by the caller, owned by the caller), taken by
 * the kernel dispatches themselves on `stream` (no separate marker):
 *   events[0]  the start of the row-statistics kernel (the pass that reads
 *              every target and draft row once),
 *   events[1]  its end,
 *   events[2]  the end of the call's last kernel.
 * `events` may be NULL and any entry may be NULL (not recorded).
 * hipEventElapsedTime(events[0], events[1]) is then the row kernel's own
 * duration.  Nothing is recorded when B = 0 or the arguments are rejected.
 */
int specdec_verify_timed(const void *target_logits, const void *draft_logits,
                         specdec_dtype_t dtype, const int32_t *draft_tokens,
                         const int32_t *k_per_req, const float *uniforms, float temperature,
                         int32_t B, int32_t K, int32_t V, int32_t *out_tokens,
                         int32_t *num_accepted, float *accept_prob, void *workspace,
                         size_t workspace_bytes, void *stream, void *const *events);

/*
 * Greedy verify step: a_i = argmax_t target_logits[b, i, t] (lowest id on
 * ties); j = first i < k_b with draft_tokens[b, i] != a_i, else k_b;
 * out_tokens[b] = drafts 0..j-1, then a_j, then -1; num_accepted[b] = j.
 * No temperature (argmax does not depend on T > 0).
 *   target_logits [B, K+1, V]; draft_tokens [B, K]; k_per_req [B] or NULL.
 *   argmax_out    [B, K+1] int32, or NULL: a_i for i <= k_b, -1 beyond.
 * 0 <= B <= 65535, 0 <= K <= 255, 1 <= V <= 2^28; larger values, or more than
 * 2^24 row tiles, give SPECDEC_EINVAL.
 */
size_t specdec_verify_greedy_workspace_bytes(int32_t B, int32_t K, int32_t V,
                                             specdec_dtype_t dtype);
int specdec_verify_greedy(const void *target_logits, specdec_dtype_t dtype,
                          const int32_t *draft_tokens, const int32_t *k_per_req,
                          int32_t B, int32_t K, int32_t V,
                          int32_t *out_tokens, int32_t *num_accepted, int32_t *argmax_out,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * specdec_verify_greedy with per-phase timing, for telemetry and
 * benchmarks: the same operation, arguments and results; the caller's HIP
 * events (hipEvent_t, caller-created and caller-owned; `events` or any
 * entry may be NULL) are taken by the kernel dispatches on `stream`:
 * events[0] the start of the argmax pass over the target rows, events[1]
 * its end, events[2] the end of the call's last kernel.  Nothing is
 * recorded when B = 0 or the arguments are rejected.
 */
int specdec_verify_greedy_timed(const void *target_logits, specdec_dtype_t dtype,
                                const int32_t *draft_tokens, const int32_t *k_per_req,
                                int32_t B, int32_t K, int32_t V, int32_t *out_tokens,
                                int32_t *num_accepted, int32_t *argmax_out, void *workspace,
                                size_t workspace_bytes, void *stream, void *const *events);

/*
 * The verify step on processed distributions ("3.5 Speculative Decoding",
 * "Notation": p is the target's distribution after temperature, top-p and
 * the like; "Common pitfalls" and "246 Speculative Decoding", Key takeaways:
 * the target and the draft must go through the same temperature / top-k /
 * top-p processing, else the guarantee breaks).  Every target row i <= k_b
 * and draft row i < k_b is processed the same way, then specdec_verify's
 * step runs on the processed rows:
 *   top-k (0 < top_k < V): keep the tokens whose logit is at least the
 *          top_k-th largest logit of the row (ties at it are all kept);
 *          top_k <= 0 or >= V keeps every token;
 *   top-p (0 < top_p < 1), on the top-k survivors renormalised: keep the
 *          tokens whose logit is at least tau, the largest logit value whose
 *          upper set {l >= tau} holds at least top_p of the survivors'
 *          probability; top_p >= 1 keeps every survivor;
 *   the processed distribution is softmax(l / T) over the kept tokens,
 *          renormalised; a drafted token cut from the target row has
 *          p(x) = 0 and is rejected.
 * Arguments, outputs and preconditions as specdec_verify, plus top_k and
 * top_p (top_p <= 0 or NaN: SPECDEC_EINVAL).  Workspace:
 * specdec_verify_processed_workspace_bytes.  accept_prob is min(1, p/q) of
 * the processed rows.  B * (rows per request) <= 2^22.
 */
size_t specdec_verify_processed_workspace_bytes(int32_t B, int32_t K, int32_t V,
                                                specdec_dtype_t dtype, int one_hot_drafts);
int specdec_verify_processed(const void *target_logits, const void *draft_logits,
                             specdec_dtype_t dtype, const int32_t *draft_tokens,
                             const int32_t *k_per_req, const float *uniforms, float temperature,
                             int32_t top_k, float top_p, int32_t B, int32_t K, int32_t V,
                             int32_t *out_tokens, int32_t *num_accepted, float *accept_prob,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * specdec_verify_processed with per-phase timing: events[0] / events[1] are
 * taken at the start / end of the processing kernel (the pass that reads
 * every row and finds its cut), events[2] at the end of the call.
 */
int specdec_verify_processed_timed(const void *target_logits, const void *draft_logits,
                                   specdec_dtype_t dtype, const int32_t *draft_tokens,
                                   const int32_t *k_per_req, const float *uniforms,
                                   float temperature, int32_t top_k, float top_p, int32_t B,
                                   int32_t K, int32_t V, int32_t *out_tokens,
                                   int32_t *num_accepted, float *accept_prob, void *workspace,
                                   size_t workspace_bytes, void *stream, void *const *events);

/*
 * The processing alone: floors[r] of each row r of logits [rows, V] after
 * temperature T, top-k and top-p as in specdec_verify_processed -- the kept
 * tokens of row r are exactly those with logits[r, t] >= floors[r] (-inf
 * when nothing is cut).  floors: [rows] float, device.  0 <= rows <= 2^22,
 * else SPECDEC_EINVAL.  No workspace.
 */
int specdec_sampling_floors(const void *logits, specdec_dtype_t dtype, int64_t rows, int32_t V,
                            float temperature, int32_t top_k, float top_p, float *floors,
                            void *stream);

/*
 * Greedy tree verification ("3.5 Speculative Decoding", "Tree verification";
 * "Speculative Decoding: Mathematical Foundations ...", "Tree-Based
 * Verification and Custom Attention Masks"): a tree of drafted tokens,
 * flattened into N nodes, was scored by one target pass; keep the longest
 * root-to-leaf path that passes greedy verification.  For request b with
 * n = n_nodes[b] nodes (N when n_nodes is NULL):
 *   a_r       = argmax_t target_logits[b, r, t] (lowest id on ties), where
 *               row 0 follows the root (the last accepted token) and row
 *               i + 1 follows node i;
 *   node i    (parent p = parents[b, i], -1 = a child of the root) is
 *               accepted iff p is the root or accepted, and
 *               node_tokens[b, i] == a_{p+1};
 *   the path  ends at the deepest accepted node e (lowest index among equal
 *               depths; none: the empty path, e = -1) with depth D;
 *   out_tokens[b]   = the path's tokens from the root side, then a_{e+1},
 *                     then -1 (N + 1 entries);
 *   path_nodes[b]   = the path's node indices from the root side, then -1
 *                     (N entries), or NULL (not written);
 *   num_accepted[b] = D.
 * A chain (parents[b, i] = i - 1) gives specdec_verify_greedy's result.
 *   target_logits [B, N+1, V]; node_tokens, parents [B, N] int32;
 *   n_nodes [B] int32 or NULL.  Target rows past n are never read.
 * Preconditions not checked on the device: -1 <= parents[b, i] < i for
 * i < n (a node that breaks it is never accepted and no address comes from
 * it); 0 <= n_nodes[b] <= N (clamped).  0 <= B <= 65535, 0 <= N <= 255,
 * 1 <= V <= 2^28, else SPECDEC_EINVAL; more than 2^24 row tiles, likewise.
 * Workspace: specdec_tree_verify_greedy_workspace_bytes (the same layout as
 * specdec_verify_greedy with K = N).
 */
size_t specdec_tree_verify_greedy_workspace_bytes(int32_t B, int32_t N, int32_t V,
                                                  specdec_dtype_t dtype);
int specdec_tree_verify_greedy(const void *target_logits, specdec_dtype_t dtype,
                               const int32_t *node_tokens, const int32_t *parents,
                               const int32_t *n_nodes, int32_t B, int32_t N, int32_t V,
                               int32_t *out_tokens, int32_t *path_nodes, int32_t *num_accepted,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * specdec_tree_verify_greedy with per-phase timing: events[0] / events[1]
 * are taken at the start / end of the row kernel, events[2] at the end of
 * the call's last kernel, as for specdec_verify_timed.
 */
int specdec_tree_verify_greedy_timed(const void *target_logits, specdec_dtype_t dtype,
                                     const int32_t *node_tokens, const int32_t *parents,
                                     const int32_t *n_nodes, int32_t B, int32_t N, int32_t V,
                                     int32_t *out_tokens, int32_t *path_nodes,
                                     int32_t *num_accepted, void *workspace,
                                     size_t workspace_bytes, void *stream, void *const *events);

/*
 * Tree attention metadata for the target pass that scores a flattened draft
 * tree ("3.5 Speculative Decoding", "Tree verification": each node attends
 * to the context, its ancestors and itself, not to siblings; nodes of equal
 * depth share a position index; "Speculative Decoding: Mathematical
 * Foundations ...", "Tree-Based Verification and Custom Attention Masks").
 * For request b with n = n_nodes[b] nodes (N when NULL):
 *   mask[b, i, j]  = 1 if i, j < n and j is i or an ancestor of i, else 0
 *                    (uint8; the context columns, always open, are not
 *                    included);
 *   depth[b, i]    = 1 for a child of the root, the parent's depth + 1
 *                    otherwise; -1 for i >= n.  A node's position index is
 *                    the root's position plus its depth.
 *   parents [B, N] int32; n_nodes [B] int32 or NULL; mask [B, N, N] uint8;
 *   depth [B, N] int32 -- all device memory.
 * Preconditions not checked on the device: -1 <= parents[b, i] < i (a
 * broken link is read as -1); 0 <= n_nodes[b] <= N (clamped).
 * 0 <= B <= 65535 and 0 <= N <= 255, else SPECDEC_EINVAL.  No workspace.
 */
int specdec_tree_mask(const int32_t *parents, const int32_t *n_nodes, int32_t B, int32_t N,
                      uint8_t *mask, int32_t *depth, void *stream);

/*
 * Acceptance telemetry of one verify step ("Speculative Decoding from First
 * Principles", "What the numbers say": the engine's counters of drafted and
 * accepted tokens, acceptance per drafted position; "246 Speculative
 * Decoding", 3.4: acceptance measured over the tests performed).  For each
 * drafted position i < K it adds, on `stream`:
 *   counters[i]       += #{b : i < k_b}                    (drafted)
 *   counters[K + i]   += #{b : i < k_b and i <= n_b}       (tested: every
 *                                                          earlier draft kept)
 *   counters[2K + i]  += #{b : i < n_b}                    (accepted)
 * with n_b = num_accepted[b] and k_b = k_per_req[b] (K when NULL).
 *   num_accepted [B] int32, device (e.g. specdec_verify's output)
 *   k_per_req    [B] int32, device, or NULL
 *   counters     [3 * K] uint64, device, owned by the caller, zeroed by the
 *                caller once and accumulated across calls (atomic adds).
 * Preconditions not checked on the device: 0 <= n_b <= k_b <= K (values
 * outside are clamped, never used as addresses).  0 <= B <= 65535 and
 * 0 <= K <= 255, else SPECDEC_EINVAL.  No workspace.
 */
int specdec_acceptance_counts(const int32_t *num_accepted, const int32_t *k_per_req, int32_t B,
                              int32_t K, uint64_t *counters, void *stream);

/*
 * n-gram (prompt-lookup) drafter: find the last few tokens earlier in the
 * context and propose what followed them there ("3.5 Speculative
 * Decoding", "Choosing a draft": n-gram / prompt lookup; "Speculative
 * Decoding: Mathematical Foundations ...", "Non-Parametric Drafters";
 * "Speculative Decoding from First Principles", "Four kinds of drafter").
 * For request b with context c = context[b, 0 .. L-1] (L = context_len[b],
 * every token so far: prompt and output):
 *   - for n = n_max down to n_min, the suffix c[L-n .. L-1] is looked for
 *     earlier in the context; the first n that occurs is used, at its latest
 *     occurrence: the largest e < L-1 with c[e-n+1 .. e] = c[L-n .. L-1];
 *   - the proposal is c[e+1 .. e+K], cut at the end of the context;
 *     k_per_req[b] is its length (0 when no suffix of n_min or more tokens
 *     occurs earlier) and draft_tokens[b, i] = -1 for i >= k_per_req[b].
 *   context      [B, L_stride] int32, device, row-major (row stride L_stride)
 *   context_len  [B] int32, device, 0 <= context_len[b] <= L_stride (values
 *                outside are clamped)
 *   draft_tokens [B, K] int32, device (output)
 *   k_per_req    [B] int32, device (output), ready for
 *                specdec_verify_greedy's k_per_req
 * 0 <= B <= 65535, 0 <= K <= 255, 1 <= n_min <= n_max <= 64, L_stride >= 0,
 * else SPECDEC_EINVAL.  One workgroup per request; no workspace.
 */
int specdec_ngram_propose(const int32_t *context, const int32_t *context_len, int32_t B,
                          int32_t L_stride, int32_t n_min, int32_t n_max, int32_t K,
                          int32_t *draft_tokens, int32_t *k_per_req, void *stream);

/*
 * Draft length from the counters (host function, synchronous; `counters`
 * is HOST memory, [3 * K] as above).  alpha_test = sum accepted / sum
 * tested, the per-draft acceptance probability of the independent-
 * acceptance model; alpha_draft = sum accepted / sum drafted, the engine
 * ratio (0 when the denominator is 0).  Under independent acceptance a step
 * of block length k emits 1 + a + ... + a^k tokens on average and costs
 * 1 + c k target passes (c = draft-to-target cost ratio, >= 0), so its
 * speedup over plain decoding is their quotient ("3.5 Speculative
 * Decoding", "Expected tokens per step", "Speedup" and the worked example's
 * table for choosing k; "246 Speculative Decoding", 2.4 and 3.5).  *k_out is
 * the k in [k_min, k_max] with the largest speedup at a = alpha_test (the
 * smallest such k on ties), *speedup_out that speedup.  alpha_test,
 * alpha_draft and speedup_out may be NULL.  SPECDEC_EINVAL for a NULL
 * counters / k_out, K < 0, k_min < 0, k_max < k_min, or c negative or not
 * finite.
 */
int specdec_choose_k(const uint64_t *counters, int32_t K, double c, int32_t k_min, int32_t k_max,
                     double *alpha_test, double *alpha_draft, int32_t *k_out,
                     double *speedup_out);

/*
 * Measurement helper, not a step of the method: the read pattern of the row
 * pass alone -- one 256-thread workgroup per 16 KB tile of `data`, four
 * 16-byte nontemporal loads per thread issued before any use, no other work
 * -- over `bytes` of DEVICE memory (a multiple of 16, 16-byte aligned).  It
 * gives the read bandwidth this access pattern can reach on the device, the
 * ceiling the row pass is compared with.  sink: DEVICE uint32 array of
 * ceil(bytes / 16384) words, written only when a tile's bits fold to one
 * particular value (so that the loads are not dropped).  events: NULL or two
 * caller HIP events (either may be NULL) taken by the kernel's dispatch at
 * its start and end.  SPECDEC_EINVAL for a NULL pointer, a misaligned or
 * ragged size, or more than 2^24 tiles.
 */
int specdec_read_stream(const void *data, size_t bytes, uint32_t *sink, void *stream,
                        void *const *events);

#ifdef __cplusplus
}
#endif

#endif /* SPECDEC_H */
