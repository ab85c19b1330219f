// Work list of the fused verify kernel (host and device).
//
// The list is a sequence of groups g = 0 .. B + D - 1.  Group g holds
//   - the row items of request g (g < B): one per (row, tile) of every row the
//     request reads, rows(g) * C items, row-major;
//   - then the final items of request g - D (D <= g < B + D): one per tile of
//     the final row (pair), C items.
// A request's final items therefore come D groups after its row items, so a
// persistent grid that walks the list in order reaches them long after the
// rows they depend on.  Every dependency points to a lower index.
//
// rows_before(x) = sum over requests b < x of rows(b); any monotone prefix
// (a closed form, or a table in LDS) can be passed as a callable.
#pragma once

#include <stdint.h>

#ifdef __HIPCC__
#define SPECDEC_HD __host__ __device__ __forceinline__
#else
#define SPECDEC_HD inline
#endif

namespace specdec {

enum : int32_t { kItemRow = 0, kItemFinal = 1 };

struct WorkItem {
    int32_t kind;   // kItemRow or kItemFinal
    int32_t b;      // request
    int32_t rr;     // row index within the request (row items)
    int32_t tile;   // tile of that row, or of the final row (pair)
};

template <class Prefix>
SPECDEC_HD int64_t group_start(const Prefix& rows_before, int32_t g, int32_t B, int32_t D, int32_t C) {
    const int32_t gb = g < B ? g : B;
    int32_t gd = g - D;
    gd = gd < 0 ? 0 : (gd > B ? B : gd);
    return (int64_t)C * ((int64_t)rows_before(gb) + gd);
}

template <class Prefix>
SPECDEC_HD int64_t work_items(const Prefix& rows_before, int32_t B, int32_t C) {
    return (int64_t)C * ((int64_t)rows_before(B) + B);
}

// Item n of the list, 0 <= n < work_items(...).
template <class Prefix>
SPECDEC_HD WorkItem work_item(const Prefix& rows_before, int64_t n, int32_t B, int32_t D, int32_t C) {
    // Largest g with group_start(g) <= n: a non-empty group holding n.
    int32_t lo = 0, hi = B + D - 1;
    while (lo < hi) {
        const int32_t mid = (int32_t)(((int64_t)lo + hi + 1) >> 1);
        if (group_start(rows_before, mid, B, D, C) <= n) lo = mid;
        else hi = mid - 1;
    }
    const int64_t local = n - group_start(rows_before, lo, B, D, C);
    const int64_t na = lo < B ? (int64_t)C * ((int64_t)rows_before(lo + 1) - rows_before(lo)) : 0;
    WorkItem it;
    if (local < na) {
        it.kind = kItemRow;
        it.b = lo;
        it.rr = (int32_t)(local / C);
        it.tile = (int32_t)(local % C);
    } else {
        it.kind = kItemFinal;
        it.b = lo - D;
        it.rr = -1;
        it.tile = (int32_t)(local - na);
    }
    return it;
}

}  // namespace specdec
