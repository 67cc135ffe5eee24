// Key ranges of a 128-row query tile under the SSA rule, shared by the
// forward and the backward kernels.
//
// For query position i (block i / b), the attended keys are the sink range
// [0, min(s*b, i+1)) and the local range [max(s*b, (i/b - l + 1)*b), i+1):
// the first s blocks plus the l blocks ending at the query's own block,
// causal (LongCat ZigZag Attention digest, section 01 part (1), the SSA
// paragraph). Over a tile of rows [q0, q1) the union of the rows' key sets is
// still two ranges, walked in 64-key sub-tiles.
#pragma once

#include <stdint.h>

namespace ssa {

constexpr int kBM = 128;  // query rows per work-group
constexpr int kBN = 64;   // keys per sub-tile

// By-value min / max. A conditional between two struct fields is an lvalue,
// which clang lowers to a select of field addresses and can leave the struct
// in scratch memory; these keep every select on values.
__device__ __forceinline__ int imin(int a, int b) { return a < b ? a : b; }
__device__ __forceinline__ int imax(int a, int b) { return a > b ? a : b; }

// First key of the local window of query position q, clamped to [0, N].
// Args is any argument block with fields N, block, local.
template <class Args>
__device__ __forceinline__ int local_start(const Args &a, int64_t q) {
    const int64_t lo = (q / a.block - a.local + 1) * (int64_t)a.block;
    return (int)(lo < 0 ? 0 : (lo > a.N ? a.N : lo));
}

// A query tile's two key ranges and mask bounds. All positions fit in int32
// (the sequence length is an int32); bounds are clamped to [0, N].
struct TileRanges {
    int q0, q1, sb, sink_end, loc_begin, lo_last;
    int n_sink, n_total;  // sub-tiles in the sink range, in both ranges
    // The complement of the SSA keys within causal attention (full-attention
    // mode only): keys [sink_end, gap_end) with j < lo(i) for row i, where
    // gap_end = lo of the tile's last row. n_all counts all three ranges.
    int gap_end, n_all;
};

// The pattern and the sequence length a tile's ranges are computed against.
struct Geo {
    int N, block, sink, local;
};

template <class Args>
__device__ __forceinline__ Geo geo_of(const Args &a) {
    return Geo{a.N, a.block, a.sink, a.local};
}

// Ranges of the rows at positions [q0, q1) of a sequence of length g.N.
__device__ __forceinline__ TileRanges tile_ranges_at(const Geo &g, int q0, int q1) {
    TileRanges r;
    const int N = g.N;
    const int64_t sb = (int64_t)g.sink * g.block;
    r.sb = (int)(sb < N ? sb : N);
    r.q0 = q0;
    r.q1 = q1;
    const int lo_first = local_start(g, r.q0);
    r.lo_last = local_start(g, r.q1 - 1);
    r.sink_end = imin(r.sb, r.q1);
    r.loc_begin = imax(lo_first, r.sink_end);
    r.n_sink = (r.sink_end + kBN - 1) / kBN;
    r.n_total = r.n_sink + (r.q1 - r.loc_begin + kBN - 1) / kBN;
    r.gap_end = imax(r.lo_last, r.sink_end);
    r.n_all = r.n_total + (r.gap_end - r.sink_end + kBN - 1) / kBN;
    return r;
}

// Query tile qt (rows [128 qt, 128 qt + 128) clamped to a.N) of a whole sequence.
template <class Args>
__device__ __forceinline__ TileRanges tile_ranges(const Args &a, int qt) {
    return tile_ranges_at(geo_of(a), qt * kBM, imin(qt * kBM + kBM, a.N));
}

// Sub-tile t of a tile: first key, end of its range, and whether any pair in
// it can be masked (it crosses a range end, the diagonal of the tile's first
// row or, in the local range, the window start of the tile's last row).
struct SubTile {
    int j0, re;
    bool need_mask;
};

// With GAP, sub-tiles n_total .. n_all-1 walk the complement range.
template <bool GAP = false>
__device__ __forceinline__ SubTile sub_tile(const TileRanges &r, int t) {
    SubTile s;
    if constexpr (GAP) {
        if (t >= r.n_total) {
            // Uniform anyway; taken as a value (not a field load) so that the
            // three-way choice of re stays a select of values.
            s.j0 = r.sink_end + (t - r.n_total) * kBN;
            s.re = __builtin_amdgcn_readfirstlane(r.gap_end);
            s.need_mask = true;
            return s;
        }
    }
    const bool local = t >= r.n_sink;
    s.j0 = local ? r.loc_begin + (t - r.n_sink) * kBN : t * kBN;
    s.re = local ? (int)r.q1 : (int)r.sink_end;
    s.need_mask = !((s.j0 + kBN <= s.re) && (s.j0 + kBN - 1 <= r.q0) && (!local || s.j0 >= r.lo_last));
    return s;
}

}  // namespace ssa
