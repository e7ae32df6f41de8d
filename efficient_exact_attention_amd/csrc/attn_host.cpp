// attn_host.cpp - the host-side tile planner: workgroup tile shapes and the
// chunking of the split passes (forward global rows, backward global rows
// and columns, decoding over a long cache). Plain C++ with no HIP calls, so
// the C ABI and this planner also build for a CPU-only sanitizer run.
#include "attn_internal.h"

namespace eea {

// ---------------------------------------------------------------------------
// Forward.
// ---------------------------------------------------------------------------
int tile_bm(int d, int f32) { (void)d; return 32 * ((f32 ? kBandThreadsF32 : kBandThreadsBf16) / 64); }

// A bounded band of at most kNarrowBand keys per row: 256-row workgroups
// would carry several key tiles that some of their waves skip (a wave's 32
// rows see only a slice of the workgroup's key range), and a short loop
// leaves the copy-in of the first tiles exposed. Four-wave workgroups, two
// per CU (three at d = 64), lose less of both (measured: 11-19 % faster for
// bands of 128 to 1024 keys, even at 4096, 2.5 % slower on unbounded causal
// rows).
bool band_is_narrow(int wl, int wr, int dil) { return dil == 1 && wl >= 0 && wr >= 0 && wl + wr + 1 <= kNarrowBand; }

int band_tile_bm(int d, int f32, int block, int extra, int wl, int wr, int dil) {
    if (f32) return tile_bm(d, f32);
    if (block > 0 || extra) return 32 * (kBandThreadsBlock / 64);
    if (band_is_narrow(wl, wr, dil)) return 32 * (kBandThreadsNarrow / 64);
    return tile_bm(d, f32);
}

int tile_bn(int d, int f32) { (void)d; return f32 ? 32 : 64; }

int global_chunks(int BH, int N, int d, int f32, int *chunk_tiles) {
    const int bn = tile_bn(d, f32);
    const int num_kt = (N + bn - 1) / bn;
    // aim for a few hundred workgroups in the split-key pass (at most
    // kMaxGlobalChunks chunks: the merge keeps one weight per chunk in LDS)
    int target = (kMaxGlobalChunks + BH - 1) / BH;
    if (target < 1) target = 1;
    if (target > num_kt) target = num_kt;
    int ct = (num_kt + target - 1) / target;
    if (ct < 1) ct = 1;
    if (chunk_tiles) *chunk_tiles = ct;
    return (num_kt + ct - 1) / ct;
}

// The bf16 band pass of 128-row workgroups can take the global rows on: each
// workgroup computes their partials on the two key tiles under its own query
// rows (visited last, so they are still in LDS when its band loop ends), one
// partial per workgroup, so the split-key pass (which reads K and V once
// more) and its launch disappear. With the strided or random-block rules the
// phase runs before their extra tiles, which reuse the buffers. More than 32
// global rows at d = 128 stay with the split-key pass: one partial of d + 2
// floats per global row and query tile is then more to write and merge than
// the pass reads (measured 7-28 % slower fused; at d = 64 fused is 1-6 %
// faster on the narrow band, about even with the extra tiles).
bool fuse_global_rows(int f32, int d, int dil, int bm, int ng) {
    return !f32 && dil == 1 && bm == 128 && (ng <= 32 || d == 64);
}

// ---------------------------------------------------------------------------
// Backward.
// ---------------------------------------------------------------------------
int bwd_tile_q(int d, int band_only) { return 32 * ((d == 128 && band_only) ? 512 : kBwdThreads) / 64; }
int bwd_tile_k(int d) { (void)d; return 32 * (kBwdThreads / 64); }

// Chunks of the split passes: a few hundred workgroups in all.
void bwd_global_chunks(int units, int N, int *chunks, int *tiles_per_chunk) {
    const int tiles = (N + 63) / 64;
    int target = (512 + units - 1) / units;
    if (target < 1) target = 1;
    if (target > tiles) target = tiles;
    const int ct = (tiles + target - 1) / target;
    *tiles_per_chunk = ct;
    *chunks = (tiles + ct - 1) / ct;
}

// ---------------------------------------------------------------------------
// Decoding.
// ---------------------------------------------------------------------------
// Chunks per row group. Each CU runs one workgroup at a time, so the cost
// of a split is (rounds of kDecCUs workgroups) x (tiles per chunk + a
// pipeline fill of about kFillTiles tiles); take the cheapest split.
int decode_chunks(int B, int H_kv, int nrg, int S, int Nq, int win, int rolling) {
    constexpr int kFillTiles = 3;
    long long tiles = (S + 63) / 64;
    if (!rolling && win >= 0) {
        const long long span = ((long long)Nq + win + 63) / 64 + 1;   // window slots, any alignment
        tiles = tiles < span ? tiles : span;
    }
    const long long units = (long long)B * H_kv * nrg;
    const long long cmax = tiles < kDecMaxChunks ? tiles : kDecMaxChunks;
    long long best = 1, best_cost = -1;
    for (long long c = 1; c <= cmax; ++c) {
        const long long rounds = (units * c + kDecCUs - 1) / kDecCUs;
        const long long cost = rounds * ((tiles + c - 1) / c + kFillTiles);
        if (best_cost < 0 || cost < best_cost) {
            best = c;
            best_cost = cost;
        }
    }
    return (int)best;
}

}  // namespace eea
