// attn_plan.h - window geometry and tile classification, shared by the host
// planner and the device kernels (header only, no HIP runtime calls).
//
// Mask reading (week-17 notes on efficient attention: local-window, Mistral
// sliding-window and global-token passages; "Sparse & sub-quadratic
// attention", "Escape 1"): row i sees the keys of one contiguous interval
// [row_lo(i), row_hi(i)] (the "band": window clipped to the sequence, causal
// folded in as a right bound of 0), plus the global columns, and a global row
// sees every key the causal limit allows. Because every row's band is one
// interval whose ends never decrease with i, a tile of rows [r0, r1] by keys
// [k0, k1] is
//   - empty (never visited) if k1 < row_lo(r0) or k0 > row_hi(r1),
//   - full  (no mask needed) if k0 >= row_lo(r1) and k1 <= row_hi(r0),
//   - an edge tile otherwise.
#pragma once

#if defined(__HIPCC__)
#define EEA_HD __host__ __device__ __forceinline__
#else
#define EEA_HD inline
#endif

namespace eea {

struct Band {
    int N;
    int wl;      // keys left of the diagonal, -1 = unbounded
    int wr;      // keys right of the diagonal, -1 = unbounded (0 under causal)
    int block;   // > 0: block-sparse rule instead of the window (own block and the previous one)
    int cap;     // block rule under causal: keys beyond the row are cut
};

EEA_HD int imin(int a, int b) { return a < b ? a : b; }
EEA_HD int imax(int a, int b) { return a > b ? a : b; }

// Fold causal into the right bound and drop bounds that cover the sequence,
// so that equivalent masks give the same band (and the same tile set).
EEA_HD Band make_band(int N, int causal, int win_left, int win_right) {
    Band b;
    b.N = N;
    b.wl = (win_left < 0 || win_left >= N - 1) ? -1 : win_left;
    int wr = causal ? 0 : win_right;
    b.wr = (wr < 0 || wr >= N - 1) ? -1 : wr;
    b.block = 0;
    b.cap = 0;
    return b;
}

// Block-sparse rule ("Sparse & sub-quadratic attention", "Escape 1": attend
// within your block and the previous one): row i sees keys
// [(i/block - 1) * block, (i/block + 1) * block - 1], cut at i under causal.
// A block covering the sequence is the unbounded window.
EEA_HD Band make_block_band(int N, int causal, int block) {
    if (block >= N) return make_band(N, causal, -1, -1);
    Band b;
    b.N = N;
    b.wl = -1;
    b.wr = -1;
    b.block = block;
    b.cap = causal;
    return b;
}

// First and last key of row i's local interval: both never decrease with i,
// which is what the tile classification below relies on.
EEA_HD int row_lo(const Band &b, int i) {
    if (b.block > 0) return imax(0, (i / b.block - 1) * b.block);
    return b.wl < 0 ? 0 : imax(0, i - b.wl);
}
EEA_HD int row_hi(const Band &b, int i) {
    if (b.block > 0) return b.cap ? imin(b.N - 1, i) : imin(b.N - 1, (i / b.block + 1) * b.block - 1);
    return b.wr < 0 ? b.N - 1 : imin(b.N - 1, i + b.wr);
}

// First and last row whose local interval holds key j (the same relation
// read column-wise; also never decreasing in j).
EEA_HD int col_lo(const Band &b, int j) {
    if (b.block > 0) return b.cap ? j : (j / b.block) * b.block;
    return b.wr < 0 ? 0 : imax(0, j - b.wr);
}
EEA_HD int col_hi(const Band &b, int j) {
    if (b.block > 0) return imin(b.N - 1, (j / b.block + 2) * b.block - 1);
    return b.wl < 0 ? b.N - 1 : imin(b.N - 1, j + b.wl);
}

// True when the band already holds every key a row may see under the causal
// rule, so global tokens add nothing.
EEA_HD bool band_is_everything(const Band &b, int causal) {
    return b.block == 0 && b.wl < 0 && (causal || b.wr < 0);
}

enum TileKind { TILE_SKIP = 0, TILE_EDGE = 1, TILE_FULL = 2 };

EEA_HD int classify(const Band &b, int r0, int r1, int k0, int k1) {
    if (k1 < row_lo(b, r0) || k0 > row_hi(b, r1)) return TILE_SKIP;
    if (k0 >= row_lo(b, r1) && k1 <= row_hi(b, r0)) return TILE_FULL;
    return TILE_EDGE;
}

// Key-tile interval [lo, hi] a query tile of rows [r0, r1] visits.
EEA_HD void key_tile_range(const Band &b, int r0, int r1, int bn, int *lo, int *hi) {
    *lo = row_lo(b, r0) / bn;
    *hi = row_hi(b, r1) / bn;
}

}  // namespace eea
