// Host/device shared definitions of the specdec library (not part of the
// public ABI): kernel parameter blocks, the workspace layout and the
// launchers each kernel file provides.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "device_common.h"
#include "slots.h"

namespace specdec {

// Largest number of drafted positions per request: the accept test keeps one
// position per thread of a workgroup and every row's statistics in LDS.
constexpr int32_t kMaxK = kThreads - 1;

// How the final draw of one request is made.
enum FinalMode : int {
    kBonus = 0,       // every draft accepted: draw from p_{k_b}
    kResidual = 1,    // rejection at j with draft logits: max(0, p_j - q_j)
    kResidualOneHot = 2,  // rejection at j with a point-mass draft: p_j without x_j
};

// Decision of one request, computed from the row statistics.
struct Decision {
    int32_t j;        // position of the first rejection (k_b if none)
    int32_t mode;     // FinalMode
    int32_t tok;      // rejected draft token (one-hot residual), else -1
    int32_t pad;
    float Mp;         // offset fp32(max * c) of target row j
    float Mq;         // offset of draft row j (residual with draft logits)
    double rho;       // Z_p / Z_q of row pair j from the row statistics (residual with draft logits)
    double zq;        // Z_q, the draft row's sum relative to Mq
    double K0;        // ln(rho) + ln 2 (Mp - Mq): rho e_q / e_p = exp(K0 + (l_q - l_p) / T)
};

struct VerifyParams {
    const void* target;
    const void* draft;          // null: one-hot drafts
    const int32_t* tokens;
    const int32_t* kpr;         // null: every k_b = K
    const float* unif;
    int32_t* out;
    int32_t* nacc;
    float* aprob;               // may be null
    int B, K, V;
    int NV;                     // vectors per row
    int C;                      // tiles per row
    int R;                      // row slots per request: K+1 target (+K draft)
    int NS;                     // slabs per row
    int kinds;                  // 2 with draft logits, 1 for one-hot drafts
    Scale sc;
    uint32_t* err;              // workspace header: error bits
    uint32_t* slot_m;           // [B * R * C] tile max (self-validating)
    uint64_t* slot_s;           // [B * R * C] tile sum (self-validating)
    uint32_t* slot_l;           // [B * R] logit at the draft token of each row (self-validating)
    uint64_t* slot_slab;        // [B * C * kSlabsPerTile] slab sums of the final draw: the masses
                                // and, for a replacement with draft logits, their q part (self-validating)
    uint64_t* slot_tile;        // [B * C] per final tile: signed replacement sum and near-tie q mass
                                // (self-validating)
    Decision* dec;              // [B] decision of each request
    const float* floors;        // [B * R] processed-row floors, or null (plain rows)
    int clear_err;              // non-zero: the row kernel clears the error word first
    uint64_t wait_ticks = kWaitTicks;   // a bounded wait gives up after this many 100 MHz ticks
    int withhold_tile = -1;     // >= 0 (error-path tests only): that final tile publishes no sums
};

// Linear greedy verify (launch_greedy) or greedy tree verify
// (launch_tree_greedy): for a tree, K is the node count N, tokens the node
// tokens, kpr the node count of each request and amax unused.
struct GreedyParams {
    const void* target;
    const int32_t* tokens;
    const int32_t* kpr;
    const int32_t* parents;     // [B, K] tree parents (tree only)
    int32_t* out;
    int32_t* nacc;
    int32_t* amax;              // may be null
    int32_t* path;              // [B, K] tree path node indices, may be null
    int B, K, V, NV, C;
    uint32_t* err;              // workspace header: error bits
    uint64_t* slot;             // [B * (K+1) * C] tile (max, index) words
};

// Floors of the top-k / top-p processed distributions, one per row (the
// kept tokens are those with logit >= floor), and, when slot_m is set, the
// verify step's row statistics of the processed rows in its slot layout.
// Row slot rr of request b: target row b * (K + 1) + rr for rr <= K, draft
// row b * K + (rr - K - 1) otherwise; slots past k_b are skipped.
struct FloorParams {
    const void* target;         // [B, K+1, V]
    const void* draft;          // [B, K, V] or null
    const int32_t* tokens;      // [B, K] draft tokens (gathers), or null
    const int32_t* kpr;         // [B] or null (K)
    int B, K, V, NV, R, C;
    Scale sc;
    int top_k;                  // kept: the top_k largest (with ties); <= 0 or >= V: off
    double top_p;               // kept mass share of the survivors; >= 1: off
    float* floors;              // [B * R]
    uint32_t* err;              // workspace header, or null
    uint32_t* slot_m;           // verify slots (null: floors only)
    uint64_t* slot_s;
    uint32_t* slot_l;
    uint64_t* slot_slab;
    uint64_t* slot_tile;
    // Candidates of a small top-k (null: none), per (request, row slot, tile):
    // a head of four words (largest key, the key from which the candidates
    // are complete, their number, 0) and up to kCandPerTile entries.
    uint32_t* cand_head;        // [B * R * C * 4]
    uint32_t* cand_ent;         // [B * R * C * kCandPerTile]
    uint32_t* cand_done;        // [B * R]: 1 where the candidates decided the row
};

// Entries a tile leaves for a top-k of at most this size.
constexpr int kCandPerTile = 64;

// Ancestor masks and depths of flattened draft trees.
struct TreeMaskParams {
    const int32_t* parents;     // [B, N]
    const int32_t* nn;          // [B] node counts, or null (N)
    int B, N;
    uint8_t* mask;              // [B, N, N]
    int32_t* depth;             // [B, N]
};

struct StatsParams {
    const void* logits;
    int64_t rows;
    int V, NV, C;
    Scale sc;
    float* row_max;
    float* row_sumexp;
    float* part_m;              // [rows * C]
    double* part_s;             // [rows * C]
};

// events: null, or three events (each may be null) recorded on s before the
// row kernel, after it, and after the call's last kernel.
struct TelemetryParams {
    const int32_t* nacc;        // [B] accepted drafts per request
    const int32_t* kpr;         // [B] drafted positions per request, or null (K)
    int B, K;
    uint64_t* counters;         // [3 * K]: drafted, tested, accepted per position
};

// Longest n-gram the drafter matches.
constexpr int32_t kMaxNgram = 64;

struct NgramParams {
    const int32_t* ctx;         // [B, Ls] context tokens, row stride Ls
    const int32_t* len;         // [B] context lengths
    int B, Ls, n_min, n_max, K;
    int32_t* drafts;            // [B, K] proposals, -1 past k_b
    int32_t* kpr;               // [B] k_b: proposals per request
};

hipError_t launch_verify(const VerifyParams& p, int dtype, bool vec, hipStream_t s,
                         hipEvent_t const* events = nullptr);
// Copy the workspace error word at err to out[0], clearing it when clear.
hipError_t launch_workspace_errors(uint32_t* err, uint32_t* out, int clear, hipStream_t s);
// events: null, or three events (each may be null) taken by the dispatches:
// the row kernel's start and end, and the end of the call's last kernel.
hipError_t launch_greedy(const GreedyParams& p, int dtype, bool vec, hipStream_t s,
                         hipEvent_t const* events = nullptr);
// Tree variant of launch_greedy (same events).
hipError_t launch_tree_greedy(const GreedyParams& p, int dtype, bool vec, hipStream_t s,
                              hipEvent_t const* events = nullptr);
hipError_t launch_tree_mask(const TreeMaskParams& p, hipStream_t s);
// The floor kernel alone (standalone floors, or the first kernel of the
// processed verify step; events[0] / events[1] as for the row kernel).
hipError_t launch_floors(const FloorParams& p, int dtype, bool vec, hipStream_t s,
                         hipEvent_t start = nullptr, hipEvent_t stop = nullptr);
// The processed verify step: the floor kernel (which also writes the row
// statistics), then the verify step's decision and final kernels on the
// floored rows.  p.floors must be set.
hipError_t launch_verify_processed(const FloorParams& f, const VerifyParams& p, int dtype, bool vec,
                                   hipStream_t s, hipEvent_t const* events = nullptr);
hipError_t launch_stats(const StatsParams& p, int dtype, bool vec, hipStream_t s);
// The row pass's read pattern alone over `bytes` of data (a multiple of 16);
// sink holds one word per 16 KB tile; start / stop events may be null.
hipError_t launch_read_stream(const void* data, size_t bytes, uint32_t* sink, hipStream_t s,
                              hipEvent_t start, hipEvent_t stop);
hipError_t launch_acceptance_counts(const TelemetryParams& p, hipStream_t s);
hipError_t launch_ngram(const NgramParams& p, hipStream_t s);

}  // namespace specdec
