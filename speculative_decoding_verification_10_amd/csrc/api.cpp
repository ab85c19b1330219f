// C ABI of the specdec library: argument validation on the host, workspace
// layout, temperature scale, and dispatch to the kernel launchers.  Nothing
// here synchronises with the device.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/specdec.h"
#include "internal.h"

namespace specdec {
namespace {

constexpr int32_t kMaxV = 1 << 28;
constexpr size_t kAlign = 256;
constexpr size_t kMaxBlocks = (size_t)1 << 24;   // gridDim.x * 256 threads < 2^32
constexpr int32_t kMaxBatch = 65535;              // requests: a grid dimension other than x
constexpr size_t kMaxFloorRows = (size_t)1 << 22;  // 1,024-thread workgroups: gridDim.x * 1024 < 2^32

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int elem_size(specdec_dtype_t dt) { return dt == SPECDEC_BF16 ? 2 : 4; }
int elems_per_vec(specdec_dtype_t dt) { return dt == SPECDEC_BF16 ? 8 : 4; }

bool dtype_ok(int dt) { return dt == SPECDEC_FP32 || dt == SPECDEC_BF16; }

// Vectors per row and whether 16-byte loads can be used for every row.
void row_geometry(int32_t V, specdec_dtype_t dt, bool aligned, int* NV, bool* vec) {
    const size_t row_bytes = (size_t)V * elem_size(dt);
    *vec = aligned && (row_bytes % 16 == 0);
    *NV = *vec ? (int)(row_bytes / 16) : (V + elems_per_vec(dt) - 1) / elems_per_vec(dt);
}

int tiles_of(int NV) { return (NV + kTileVec - 1) / kTileVec; }

bool aligned16(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) % 16) == 0; }

// c = log2(e) / T as hi + lo with hi the largest float strictly below c, so
// that lo > 0.
bool make_scale(float temperature, Scale* s) {
    if (!(temperature > 0.0f) || !std::isfinite(temperature)) return false;
    const double c = 1.4426950408889634074 / (double)temperature;
    if (!std::isfinite(c) || c > 1e30) return false;
    float hi = (float)c;
    if ((double)hi >= c) hi = std::nextafter(hi, 0.0f);
    const float lo = (float)(c - (double)hi);
    if (!(hi > 0.0f) || !(lo > 0.0f)) return false;
    s->hi = hi;
    s->lo = lo;
    s->c = c;
    s->inv_t = 1.0 / (double)temperature;
    return true;
}

struct VerifyLayout {
    size_t err, slot_m, slot_s, slot_l, slot_slab, slot_tile, dec, floors, cand_head, cand_ent, cand_done, total;
};

// Header (error bits), self-validating slots -- tile max / tile sum of every
// row slot of every request, the logit at the draft token of every row, the
// slab sums and per-tile sums of every request's final row -- and each
// request's decision; for the processed step also the row floors and the
// tile candidates of a small top-k.
VerifyLayout verify_layout(int32_t B, int32_t K, int32_t V, specdec_dtype_t dt, bool one_hot,
                           bool processed = false) {
    int NV, NVv;
    bool vec;
    row_geometry(V, dt, false, &NV, &vec);        // scalar geometry >= vector geometry
    row_geometry(V, dt, true, &NVv, &vec);
    const size_t C = (size_t)tiles_of(NV > NVv ? NV : NVv);
    const size_t R = (size_t)K + 1 + (one_hot ? 0 : (size_t)K);
    const size_t parts = (size_t)B * R * C;
    VerifyLayout L;
    size_t off = 0;
    L.err = off;       off = align_up(off + sizeof(uint32_t));
    L.slot_m = off;    off = align_up(off + parts * sizeof(uint32_t));
    L.slot_s = off;    off = align_up(off + parts * sizeof(uint64_t));
    L.slot_l = off;    off = align_up(off + (size_t)B * R * sizeof(uint32_t));
    L.slot_slab = off; off = align_up(off + (size_t)B * C * kSlabsPerTile * sizeof(uint64_t));
    L.slot_tile = off; off = align_up(off + (size_t)B * C * sizeof(uint64_t));
    L.dec = off;       off = align_up(off + (size_t)B * sizeof(Decision));
    L.floors = off;    if (processed) off = align_up(off + (size_t)B * R * sizeof(float));
    L.cand_head = off; if (processed) off = align_up(off + parts * 4 * sizeof(uint32_t));
    L.cand_ent = off;  if (processed) off = align_up(off + parts * kCandPerTile * sizeof(uint32_t));
    L.cand_done = off; if (processed) off = align_up(off + (size_t)B * R * sizeof(uint32_t));
    L.total = off;
    return L;
}

struct GreedyLayout {
    size_t err, slot, total;
};

GreedyLayout greedy_layout(int32_t B, int32_t K, int32_t V, specdec_dtype_t dt) {
    int NV, NVv;
    bool vec;
    row_geometry(V, dt, false, &NV, &vec);
    row_geometry(V, dt, true, &NVv, &vec);
    const size_t C = (size_t)tiles_of(NV > NVv ? NV : NVv);
    const size_t parts = (size_t)B * ((size_t)K + 1) * C;
    GreedyLayout L;
    size_t off = 0;
    L.err = off;  off = align_up(off + sizeof(uint32_t));
    L.slot = off; off = align_up(off + parts * sizeof(uint64_t));
    L.total = off;
    return L;
}

struct StatsLayout {
    size_t part_m, part_s, total;
};

StatsLayout stats_layout(int64_t rows, int32_t V, specdec_dtype_t dt) {
    int NV, NVv;
    bool vec;
    row_geometry(V, dt, false, &NV, &vec);
    row_geometry(V, dt, true, &NVv, &vec);
    const size_t C = (size_t)tiles_of(NV > NVv ? NV : NVv);
    const size_t parts = (size_t)rows * C;
    StatsLayout L;
    size_t off = 0;
    L.part_m = off; off = align_up(off + parts * sizeof(float));
    L.part_s = off; off = align_up(off + parts * sizeof(double));
    L.total = off < kAlign ? kAlign : off;
    return L;
}

bool workspace_ok(const void* ws, size_t have, size_t need) {
    return ws != nullptr && have >= need && (reinterpret_cast<uintptr_t>(ws) % kAlign) == 0;
}

// The library holds gfx950 code only.  A launch that fails on a device of
// another architecture reports SPECDEC_EDEVICE; the check runs only after a
// failure, so a successful call pays nothing for it.
bool current_device_is_gfx950() {
    int dev = -1;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess) return false;
    return std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
}

int map_launch(hipError_t e) {
    if (e == hipSuccess) return SPECDEC_OK;
    return current_device_is_gfx950() ? SPECDEC_ELAUNCH : SPECDEC_EDEVICE;
}

// The bounded waits' limit and the withheld final tile of the next calls
// (specdec_debug_bounded_wait; the defaults outside tests of the error path).
std::atomic<uint64_t> g_wait_ticks{kWaitTicks};
std::atomic<int32_t> g_withhold_tile{-1};

// Scratch of the allocation-free entry point (specdec_verify_noalloc): a
// file-scope device array, one copy per GPU, held until the process ends.
// In host code its name is only a stand-in; its device address, found once
// per device with hipGetSymbolAddress, is what the kernels are given.
constexpr size_t kScratchBytes = SPECDEC_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];

// The current device's scratch address (found on the first call on that
// device, with that device current).
int scratch_on_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SPECDEC_EDEVICE;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return SPECDEC_EDEVICE;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return SPECDEC_OK;
}

// The stochastic verify step on a caller workspace, or (noalloc) on the
// library's static scratch.
int verify_impl(const void* target_logits, const void* draft_logits, specdec_dtype_t dtype,
                const int32_t* draft_tokens, const int32_t* k_per_req, const float* uniforms,
                float temperature, int32_t B, int32_t K, int32_t V, int32_t* out_tokens,
                int32_t* num_accepted, float* accept_prob, void* workspace, size_t workspace_bytes,
                void* stream, void* const* events, bool noalloc) {
    if (!dtype_ok(dtype)) return SPECDEC_EDTYPE;
    if (B < 0 || K < 0 || K > kMaxK || V < 1 || V > kMaxV) return SPECDEC_EINVAL;
    Scale sc;
    if (!make_scale(temperature, &sc)) return SPECDEC_EINVAL;
    if (B == 0) return SPECDEC_OK;
    if (!target_logits || !uniforms || !out_tokens || !num_accepted) return SPECDEC_EINVAL;
    if (K > 0 && !draft_tokens) return SPECDEC_EINVAL;
    const bool one_hot = (draft_logits == nullptr);
    const VerifyLayout L = verify_layout(B, K, V, dtype, one_hot);
    if (noalloc) {
        // The library's static scratch instead of a caller workspace.
        if (L.total > kScratchBytes) return SPECDEC_ESCRATCH;
        const int st = scratch_on_current_device(&workspace);
        if (st != SPECDEC_OK) return st;
        workspace_bytes = kScratchBytes;
    }
    if (!workspace_ok(workspace, workspace_bytes, L.total)) return SPECDEC_EWORKSPACE;
    VerifyParams p{};
    bool vec;
    row_geometry(V, dtype, aligned16(target_logits) && aligned16(draft_logits), &p.NV, &vec);
    p.C = tiles_of(p.NV);
    p.R = K + 1 + (one_hot ? 0 : K);
    p.NS = (p.NV + kSlab - 1) / kSlab;
    p.kinds = one_hot ? 1 : 2;
    p.clear_err = noalloc ? 1 : 0;
    p.wait_ticks = g_wait_ticks.load(std::memory_order_relaxed);
    p.withhold_tile = g_withhold_tile.load(std::memory_order_relaxed);
    // One workgroup per row item and per final item.
    if ((size_t)B * p.R * p.C > kMaxBlocks || B > kMaxBatch) return SPECDEC_EINVAL;
    p.target = target_logits;
    p.draft = draft_logits;
    p.tokens = draft_tokens;
    p.kpr = k_per_req;
    p.unif = uniforms;
    p.out = out_tokens;
    p.nacc = num_accepted;
    p.aprob = accept_prob;
    p.B = B;
    p.K = K;
    p.V = V;
    p.sc = sc;
    char* ws = static_cast<char*>(workspace);
    p.err = reinterpret_cast<uint32_t*>(ws + L.err);
    p.slot_m = reinterpret_cast<uint32_t*>(ws + L.slot_m);
    p.slot_s = reinterpret_cast<uint64_t*>(ws + L.slot_s);
    p.slot_l = reinterpret_cast<uint32_t*>(ws + L.slot_l);
    p.slot_slab = reinterpret_cast<uint64_t*>(ws + L.slot_slab);
    p.slot_tile = reinterpret_cast<uint64_t*>(ws + L.slot_tile);
    p.dec = reinterpret_cast<Decision*>(ws + L.dec);
    return map_launch(launch_verify(p, dtype, vec, (hipStream_t)stream,
                                    reinterpret_cast<hipEvent_t const*>(events)));
}
}  // namespace
}  // namespace specdec

using namespace specdec;

extern "C" {

const char* specdec_status_string(int status) {
    switch (status) {
        case SPECDEC_OK: return "ok";
        case SPECDEC_EINVAL: return "invalid argument";
        case SPECDEC_EDTYPE: return "unknown dtype";
        case SPECDEC_EWORKSPACE: return "workspace missing, too small or misaligned";
        case SPECDEC_ELAUNCH: return "kernel launch failed";
        case SPECDEC_EDEVICE: return "no usable gfx950 device";
        case SPECDEC_ESCRATCH: return "call too large for the library's static scratch (specdec_verify_noalloc)";
        default: return "unknown status";
    }
}

const char* specdec_version(void) { return "specdec 0.1 (gfx950)"; }

int specdec_workspace_init(void* workspace, size_t bytes, void* stream) {
    if (workspace == nullptr && bytes != 0) return SPECDEC_EINVAL;
    if (bytes == 0) return SPECDEC_OK;
    return map_launch(hipMemsetAsync(workspace, 0, bytes, (hipStream_t)stream));
}

int specdec_debug_bounded_wait(uint64_t wait_ticks, int32_t withhold_tile) {
    if (wait_ticks == 0) wait_ticks = kWaitTicks;
    if (withhold_tile < -1) return SPECDEC_EINVAL;
    g_wait_ticks.store(wait_ticks, std::memory_order_relaxed);
    g_withhold_tile.store(withhold_tile, std::memory_order_relaxed);
    return SPECDEC_OK;
}

int specdec_workspace_errors(void* workspace, uint32_t* errors, int clear, void* stream) {
    if (!workspace || !errors || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0) return SPECDEC_EINVAL;
    return map_launch(launch_workspace_errors(static_cast<uint32_t*>(workspace), errors, clear,
                                              (hipStream_t)stream));
}

size_t specdec_softmax_stats_workspace_bytes(int64_t rows, int32_t V, specdec_dtype_t dtype) {
    if (rows < 0 || V < 1 || V > kMaxV || !dtype_ok(dtype)) return 0;
    return stats_layout(rows, V, dtype).total;
}

int specdec_softmax_stats(const void* logits, specdec_dtype_t dtype, int64_t rows, int32_t V,
                          float temperature, float* row_max, float* row_sumexp, void* workspace,
                          size_t workspace_bytes, void* stream) {
    if (!dtype_ok(dtype)) return SPECDEC_EDTYPE;
    if (rows < 0 || V < 1 || V > kMaxV) return SPECDEC_EINVAL;
    Scale sc;
    if (!make_scale(temperature, &sc)) return SPECDEC_EINVAL;
    if (rows == 0) return SPECDEC_OK;
    if (!logits || !row_max || !row_sumexp) return SPECDEC_EINVAL;
    const StatsLayout L = stats_layout(rows, V, dtype);
    if (!workspace_ok(workspace, workspace_bytes, L.total)) return SPECDEC_EWORKSPACE;
    StatsParams p{};
    bool vec;
    row_geometry(V, dtype, aligned16(logits), &p.NV, &vec);
    p.C = tiles_of(p.NV);
    if ((size_t)rows * p.C > kMaxBlocks) return SPECDEC_EINVAL;
    p.logits = logits;
    p.rows = rows;
    p.V = V;
    p.sc = sc;
    p.row_max = row_max;
    p.row_sumexp = row_sumexp;
    char* ws = static_cast<char*>(workspace);
    p.part_m = reinterpret_cast<float*>(ws + L.part_m);
    p.part_s = reinterpret_cast<double*>(ws + L.part_s);
    return map_launch(launch_stats(p, dtype, vec, (hipStream_t)stream));
}

size_t specdec_verify_workspace_bytes(int32_t B, int32_t K, int32_t V, specdec_dtype_t dtype,
                                      int one_hot_drafts) {
    if (B < 0 || K < 0 || K > kMaxK || V < 1 || V > kMaxV || !dtype_ok(dtype)) return 0;
    return verify_layout(B, K, V, dtype, one_hot_drafts != 0).total;
}

int specdec_verify(const void* target_logits, const void* draft_logits, specdec_dtype_t dtype,
                   const int32_t* draft_tokens, const int32_t* k_per_req, const float* uniforms,
                   float temperature, int32_t B, int32_t K, int32_t V, int32_t* out_tokens,
                   int32_t* num_accepted, float* accept_prob, void* workspace,
                   size_t workspace_bytes, void* stream) {
    return specdec_verify_timed(target_logits, draft_logits, dtype, draft_tokens, k_per_req,
                                uniforms, temperature, B, K, V, out_tokens, num_accepted,
                                accept_prob, workspace, workspace_bytes, stream, nullptr);
}

int specdec_verify_noalloc(const void* target_logits, const void* draft_logits, specdec_dtype_t dtype,
                           const int32_t* draft_tokens, const int32_t* k_per_req, const float* uniforms,
                           float temperature, int32_t B, int32_t K, int32_t V, int32_t* out_tokens,
                           int32_t* num_accepted, float* accept_prob, void* stream) {
    return verify_impl(target_logits, draft_logits, dtype, draft_tokens, k_per_req, uniforms, temperature,
                       B, K, V, out_tokens, num_accepted, accept_prob, nullptr, 0, stream, nullptr, true);
}

int specdec_verify_timed(const void* target_logits, const void* draft_logits, specdec_dtype_t dtype,
                         const int32_t* draft_tokens, const int32_t* k_per_req, const float* uniforms,
                         float temperature, int32_t B, int32_t K, int32_t V, int32_t* out_tokens,
                         int32_t* num_accepted, float* accept_prob, void* workspace,
                         size_t workspace_bytes, void* stream, void* const* events) {
    return verify_impl(target_logits, draft_logits, dtype, draft_tokens, k_per_req, uniforms, temperature,
                       B, K, V, out_tokens, num_accepted, accept_prob, workspace, workspace_bytes, stream,
                       events, false);
}



size_t specdec_verify_processed_workspace_bytes(int32_t B, int32_t K, int32_t V,
                                                specdec_dtype_t dtype, int one_hot_drafts) {
    if (B < 0 || K < 0 || K > kMaxK || V < 1 || V > kMaxV || !dtype_ok(dtype)) return 0;
    return verify_layout(B, K, V, dtype, one_hot_drafts != 0, true).total;
}

int specdec_verify_processed(const void* target_logits, const void* draft_logits,
                             specdec_dtype_t dtype, const int32_t* draft_tokens,
                             const int32_t* k_per_req, const float* uniforms, float temperature,
                             int32_t top_k, float top_p, int32_t B, int32_t K, int32_t V,
                             int32_t* out_tokens, int32_t* num_accepted, float* accept_prob,
                             void* workspace, size_t workspace_bytes, void* stream) {
    return specdec_verify_processed_timed(target_logits, draft_logits, dtype, draft_tokens, k_per_req,
                                          uniforms, temperature, top_k, top_p, B, K, V, out_tokens,
                                          num_accepted, accept_prob, workspace, workspace_bytes,
                                          stream, nullptr);
}

int specdec_verify_processed_timed(const void* target_logits, const void* draft_logits,
                                   specdec_dtype_t dtype, const int32_t* draft_tokens,
                                   const int32_t* k_per_req, const float* uniforms,
                                   float temperature, int32_t top_k, float top_p, int32_t B,
                                   int32_t K, int32_t V, int32_t* out_tokens,
                                   int32_t* num_accepted, float* accept_prob, void* workspace,
                                   size_t workspace_bytes, void* stream, void* const* events) {
    if (!dtype_ok(dtype)) return SPECDEC_EDTYPE;
    if (B < 0 || K < 0 || K > kMaxK || V < 1 || V > kMaxV) return SPECDEC_EINVAL;
    if (!(top_p > 0.0f)) return SPECDEC_EINVAL;              // also rejects NaN
    Scale sc;
    if (!make_scale(temperature, &sc)) return SPECDEC_EINVAL;
    if (B == 0) return SPECDEC_OK;
    if (!target_logits || !uniforms || !out_tokens || !num_accepted) return SPECDEC_EINVAL;
    if (K > 0 && !draft_tokens) return SPECDEC_EINVAL;
    const bool one_hot = (draft_logits == nullptr);
    const VerifyLayout L = verify_layout(B, K, V, dtype, one_hot, true);
    if (!workspace_ok(workspace, workspace_bytes, L.total)) return SPECDEC_EWORKSPACE;
    VerifyParams p{};
    bool vec;
    row_geometry(V, dtype, aligned16(target_logits) && aligned16(draft_logits), &p.NV, &vec);
    p.C = tiles_of(p.NV);
    p.R = K + 1 + (one_hot ? 0 : K);
    p.NS = (p.NV + kSlab - 1) / kSlab;
    p.kinds = one_hot ? 1 : 2;
    p.wait_ticks = g_wait_ticks.load(std::memory_order_relaxed);
    p.withhold_tile = g_withhold_tile.load(std::memory_order_relaxed);
    if ((size_t)B * p.C > kMaxBlocks || (size_t)B * p.R > kMaxFloorRows || B > kMaxBatch)
        return SPECDEC_EINVAL;
    p.target = target_logits;
    p.draft = draft_logits;
    p.tokens = draft_tokens;
    p.kpr = k_per_req;
    p.unif = uniforms;
    p.out = out_tokens;
    p.nacc = num_accepted;
    p.aprob = accept_prob;
    p.B = B;
    p.K = K;
    p.V = V;
    p.sc = sc;
    char* ws = static_cast<char*>(workspace);
    p.err = reinterpret_cast<uint32_t*>(ws + L.err);
    p.slot_m = reinterpret_cast<uint32_t*>(ws + L.slot_m);
    p.slot_s = reinterpret_cast<uint64_t*>(ws + L.slot_s);
    p.slot_l = reinterpret_cast<uint32_t*>(ws + L.slot_l);
    p.slot_slab = reinterpret_cast<uint64_t*>(ws + L.slot_slab);
    p.slot_tile = reinterpret_cast<uint64_t*>(ws + L.slot_tile);
    p.dec = reinterpret_cast<Decision*>(ws + L.dec);
    p.floors = reinterpret_cast<float*>(ws + L.floors);
    FloorParams f{};
    f.target = target_logits;
    f.draft = draft_logits;
    f.tokens = draft_tokens;
    f.kpr = k_per_req;
    f.B = B;
    f.K = K;
    f.V = V;
    f.NV = p.NV;
    f.R = p.R;
    f.C = p.C;
    f.sc = sc;
    f.top_k = top_k;
    f.top_p = (double)top_p;
    f.floors = reinterpret_cast<float*>(ws + L.floors);
    f.err = p.err;
    f.slot_m = p.slot_m;
    f.slot_s = p.slot_s;
    f.slot_l = p.slot_l;
    f.slot_slab = p.slot_slab;
    f.slot_tile = p.slot_tile;
    f.cand_head = reinterpret_cast<uint32_t*>(ws + L.cand_head);
    f.cand_ent = reinterpret_cast<uint32_t*>(ws + L.cand_ent);
    f.cand_done = reinterpret_cast<uint32_t*>(ws + L.cand_done);
    return map_launch(launch_verify_processed(f, p, dtype, vec, (hipStream_t)stream,
                                              reinterpret_cast<hipEvent_t const*>(events)));
}

int specdec_sampling_floors(const void* logits, specdec_dtype_t dtype, int64_t rows, int32_t V,
                            float temperature, int32_t top_k, float top_p, float* floors,
                            void* stream) {
    if (!dtype_ok(dtype)) return SPECDEC_EDTYPE;
    if (rows < 0 || rows > (int64_t)kMaxFloorRows || V < 1 || V > kMaxV) return SPECDEC_EINVAL;
    if (!(top_p > 0.0f)) return SPECDEC_EINVAL;
    Scale sc;
    if (!make_scale(temperature, &sc)) return SPECDEC_EINVAL;
    if (rows == 0) return SPECDEC_OK;
    if (!logits || !floors) return SPECDEC_EINVAL;
    FloorParams f{};
    bool vec;
    row_geometry(V, dtype, aligned16(logits), &f.NV, &vec);
    f.target = logits;
    f.B = (int)rows;
    f.K = 0;
    f.R = 1;
    f.C = tiles_of(f.NV);
    f.V = V;
    f.sc = sc;
    f.top_k = top_k;
    f.top_p = (double)top_p;
    f.floors = floors;
    return map_launch(launch_floors(f, dtype, vec, (hipStream_t)stream));
}

size_t specdec_verify_greedy_workspace_bytes(int32_t B, int32_t K, int32_t V,
                                             specdec_dtype_t dtype) {
    if (B < 0 || K < 0 || K > kMaxK || V < 1 || V > kMaxV || !dtype_ok(dtype)) return 0;
    return greedy_layout(B, K, V, dtype).total;
}

int specdec_verify_greedy(const void* target_logits, specdec_dtype_t dtype,
                          const int32_t* draft_tokens, const int32_t* k_per_req, int32_t B,
                          int32_t K, int32_t V, int32_t* out_tokens, int32_t* num_accepted,
                          int32_t* argmax_out, void* workspace, size_t workspace_bytes,
                          void* stream) {
    return specdec_verify_greedy_timed(target_logits, dtype, draft_tokens, k_per_req, B, K, V,
                                       out_tokens, num_accepted, argmax_out, workspace,
                                       workspace_bytes, stream, nullptr);
}

int specdec_verify_greedy_timed(const void* target_logits, specdec_dtype_t dtype,
                                const int32_t* draft_tokens, const int32_t* k_per_req, int32_t B,
                                int32_t K, int32_t V, int32_t* out_tokens, int32_t* num_accepted,
                                int32_t* argmax_out, void* workspace, size_t workspace_bytes,
                                void* stream, void* const* events) {
    if (!dtype_ok(dtype)) return SPECDEC_EDTYPE;
    if (B < 0 || K < 0 || K > kMaxK || V < 1 || V > kMaxV) return SPECDEC_EINVAL;
    if (B == 0) return SPECDEC_OK;
    if (!target_logits || !out_tokens || !num_accepted) return SPECDEC_EINVAL;
    if (K > 0 && !draft_tokens) return SPECDEC_EINVAL;
    const GreedyLayout L = greedy_layout(B, K, V, dtype);
    if (!workspace_ok(workspace, workspace_bytes, L.total)) return SPECDEC_EWORKSPACE;
    GreedyParams p{};
    bool vec;
    row_geometry(V, dtype, aligned16(target_logits), &p.NV, &vec);
    p.C = tiles_of(p.NV);
    if ((size_t)B * (K + 1) * p.C > kMaxBlocks || B > kMaxBatch) return SPECDEC_EINVAL;
    p.target = target_logits;
    p.tokens = draft_tokens;
    p.kpr = k_per_req;
    p.out = out_tokens;
    p.nacc = num_accepted;
    p.amax = argmax_out;
    p.B = B;
    p.K = K;
    p.V = V;
    char* ws = static_cast<char*>(workspace);
    p.err = reinterpret_cast<uint32_t*>(ws + L.err);
    p.slot = reinterpret_cast<uint64_t*>(ws + L.slot);
    return map_launch(launch_greedy(p, dtype, vec, (hipStream_t)stream,
                                    reinterpret_cast<hipEvent_t const*>(events)));
}

size_t specdec_tree_verify_greedy_workspace_bytes(int32_t B, int32_t N, int32_t V,
                                                  specdec_dtype_t dtype) {
    return specdec_verify_greedy_workspace_bytes(B, N, V, dtype);
}

int specdec_tree_verify_greedy(const void* target_logits, specdec_dtype_t dtype,
                               const int32_t* node_tokens, const int32_t* parents,
                               const int32_t* n_nodes, int32_t B, int32_t N, int32_t V,
                               int32_t* out_tokens, int32_t* path_nodes, int32_t* num_accepted,
                               void* workspace, size_t workspace_bytes, void* stream) {
    return specdec_tree_verify_greedy_timed(target_logits, dtype, node_tokens, parents, n_nodes, B,
                                            N, V, out_tokens, path_nodes, num_accepted, workspace,
                                            workspace_bytes, stream, nullptr);
}

int specdec_tree_verify_greedy_timed(const void* target_logits, specdec_dtype_t dtype,
                                     const int32_t* node_tokens, const int32_t* parents,
                                     const int32_t* n_nodes, int32_t B, int32_t N, int32_t V,
                                     int32_t* out_tokens, int32_t* path_nodes,
                                     int32_t* num_accepted, void* workspace,
                                     size_t workspace_bytes, void* stream, void* const* events) {
    if (!dtype_ok(dtype)) return SPECDEC_EDTYPE;
    if (B < 0 || N < 0 || N > kMaxK || V < 1 || V > kMaxV) return SPECDEC_EINVAL;
    if (B == 0) return SPECDEC_OK;
    if (!target_logits || !out_tokens || !num_accepted) return SPECDEC_EINVAL;
    if (N > 0 && (!node_tokens || !parents)) return SPECDEC_EINVAL;
    const GreedyLayout L = greedy_layout(B, N, V, dtype);
    if (!workspace_ok(workspace, workspace_bytes, L.total)) return SPECDEC_EWORKSPACE;
    GreedyParams p{};
    bool vec;
    row_geometry(V, dtype, aligned16(target_logits), &p.NV, &vec);
    p.C = tiles_of(p.NV);
    if ((size_t)B * (N + 1) * p.C > kMaxBlocks || B > kMaxBatch) return SPECDEC_EINVAL;
    p.target = target_logits;
    p.tokens = node_tokens;
    p.kpr = n_nodes;
    p.parents = parents;
    p.out = out_tokens;
    p.nacc = num_accepted;
    p.path = path_nodes;
    p.B = B;
    p.K = N;
    p.V = V;
    char* ws = static_cast<char*>(workspace);
    p.err = reinterpret_cast<uint32_t*>(ws + L.err);
    p.slot = reinterpret_cast<uint64_t*>(ws + L.slot);
    return map_launch(launch_tree_greedy(p, dtype, vec, (hipStream_t)stream,
                                         reinterpret_cast<hipEvent_t const*>(events)));
}

int specdec_tree_mask(const int32_t* parents, const int32_t* n_nodes, int32_t B, int32_t N,
                      uint8_t* mask, int32_t* depth, void* stream) {
    if (B < 0 || B > kMaxBatch || N < 0 || N > kMaxK) return SPECDEC_EINVAL;
    if (B == 0 || N == 0) return SPECDEC_OK;
    if (!parents || !mask || !depth) return SPECDEC_EINVAL;
    TreeMaskParams p{};
    p.parents = parents;
    p.nn = n_nodes;
    p.B = B;
    p.N = N;
    p.mask = mask;
    p.depth = depth;
    return map_launch(launch_tree_mask(p, (hipStream_t)stream));
}

int specdec_acceptance_counts(const int32_t* num_accepted, const int32_t* k_per_req, int32_t B,
                              int32_t K, uint64_t* counters, void* stream) {
    if (B < 0 || B > kMaxBatch || K < 0 || K > kMaxK) return SPECDEC_EINVAL;
    if (B == 0 || K == 0) return SPECDEC_OK;
    if (!num_accepted || !counters) return SPECDEC_EINVAL;
    TelemetryParams p{};
    p.nacc = num_accepted;
    p.kpr = k_per_req;
    p.B = B;
    p.K = K;
    p.counters = counters;
    return map_launch(launch_acceptance_counts(p, (hipStream_t)stream));
}

int specdec_ngram_propose(const int32_t* context, const int32_t* context_len, int32_t B,
                          int32_t L_stride, int32_t n_min, int32_t n_max, int32_t K,
                          int32_t* draft_tokens, int32_t* k_per_req, void* stream) {
    if (B < 0 || B > kMaxBatch || K < 0 || K > kMaxK || L_stride < 0 || n_min < 1 ||
        n_max < n_min || n_max > kMaxNgram)
        return SPECDEC_EINVAL;
    if (B == 0) return SPECDEC_OK;
    if (!context_len || !k_per_req || (K > 0 && !draft_tokens) || (L_stride > 0 && !context))
        return SPECDEC_EINVAL;
    NgramParams p{};
    p.ctx = context;
    p.len = context_len;
    p.B = B;
    p.Ls = L_stride;
    p.n_min = n_min;
    p.n_max = n_max;
    p.K = K;
    p.drafts = draft_tokens;
    p.kpr = k_per_req;
    return map_launch(launch_ngram(p, (hipStream_t)stream));
}

int specdec_read_stream(const void* data, size_t bytes, uint32_t* sink, void* stream, void* const* events) {
    if (bytes == 0) return SPECDEC_OK;
    if (!data || !sink || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(data) % 16) != 0) return SPECDEC_EINVAL;
    if ((bytes / 16 + kTileVec - 1) / kTileVec > kMaxBlocks) return SPECDEC_EINVAL;
    hipEvent_t ev[2] = {nullptr, nullptr};
    if (events) {
        ev[0] = static_cast<hipEvent_t>(events[0]);
        ev[1] = static_cast<hipEvent_t>(events[1]);
    }
    return map_launch(launch_read_stream(data, bytes, sink, (hipStream_t)stream, ev[0], ev[1]));
}

int specdec_choose_k(const uint64_t* counters, int32_t K, double c, int32_t k_min, int32_t k_max,
                     double* alpha_test, double* alpha_draft, int32_t* k_out,
                     double* speedup_out) {
    if (!counters || !k_out || K < 0 || k_min < 0 || k_max < k_min || !(c >= 0.0) ||
        !std::isfinite(c))
        return SPECDEC_EINVAL;
    double n_drafted = 0.0, n_tested = 0.0, n_accepted = 0.0;
    for (int32_t i = 0; i < K; ++i) {
        n_drafted += (double)counters[i];
        n_tested += (double)counters[(size_t)K + i];
        n_accepted += (double)counters[2 * (size_t)K + i];
    }
    const double a = (n_tested > 0.0) ? n_accepted / n_tested : 0.0;
    if (alpha_test) *alpha_test = a;
    if (alpha_draft) *alpha_draft = (n_drafted > 0.0) ? n_accepted / n_drafted : 0.0;
    // Expected tokens for block length k: 1 + a + ... + a^k, grown one term
    // at a time; cost 1 + c k target passes.
    double tokens = 0.0, term = 1.0, best = -1.0;
    int32_t best_k = k_min;
    for (int32_t k = 0; k <= k_max; ++k) {
        tokens += term;
        term *= a;
        if (k < k_min) continue;
        const double speedup = tokens / (1.0 + c * (double)k);
        if (speedup > best) {
            best = speedup;
            best_k = k;
        }
    }
    *k_out = best_k;
    if (speedup_out) *speedup_out = best;
    return SPECDEC_OK;
}

}  // extern "C"
