// attn_internal.h - parameter blocks, workgroup shapes and launcher entry
// points shared between the C ABI (attn_api.cpp), the host planner
// (attn_host.cpp) and the HIP kernels (attn_fwd.hip, attn_bwd.hip,
// attn_decode.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace eea {

constexpr int kMaxGlobal = 64;       // one gathered key tile holds every global column
// Bytes of the file-scope device array attn_fwd_noalloc keeps its global-row
// partials in (one per device, for the life of the process).
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
constexpr int kMaxGlobalChunks = 512; // key chunks of the split-key pass over global rows

// Workgroup shapes. The kernels are instantiated with these, and the host
// planner (attn_host.cpp) derives tile sizes and grids from the same values.
constexpr int kBandThreadsBf16 = 512;   // 8 waves, 256 query rows
constexpr int kBandThreadsF32 = 256;    // 4 waves, 128 query rows
constexpr int kBandThreadsBlock = 256;  // bf16 with the block rule or extra tiles: 4 waves, 128 query rows
constexpr int kBandThreadsNarrow = 256; // bf16 narrow band: 4 waves, 128 query rows, two workgroups per CU
constexpr int kNarrowBand = 4096;       // widest band (keys per row) run by the narrow instance
constexpr int kBwdThreads = 256;        // backward: 4 waves, one per SIMD (up to 512 registers each) or two per SIMD
constexpr int kDecThreads = 256;        // decoding: four waves of 32 query rows each
constexpr int kDecLds = 163840;         // decoding uses the whole LDS of a CU: one workgroup per CU
constexpr int kDecCUs = 256;            // compute units of an MI355X

// Kernel arguments. Offsets are 64-bit throughout: one head at N=131072, d=128
// is 2^24 elements and B*H*N*d can exceed 2^31.
struct FwdParams {
    const void *q;
    const void *k;
    const void *v;
    void *out;
    float *lse;
    float *part;          // global-row partials [B*H][n_global][chunks][d + 2]
    long long head_stride;  // N * d elements
    int BH;               // B * H (query heads)
    int H;                // query heads per batch entry
    int group;            // query heads per K/V head (H / H_kv; 1 for plain multi-head)
    int N;
    int wl, wr;           // normalised band (see attn_plan.h)
    int block, cap;       // block-sparse rule (0: window rule)
    int dil;              // dilation: rows r, r+dil, ... form one sequence (1: plain)
    int causal;
    int n_global;         // 0 when the band already covers every visible key
    int num_qt;           // query tiles per head (per residue class when dil > 1)
    int chunks;           // key chunks per global row (split-key pass; with fuse_grows: query tiles)
    int chunk_tiles;      // key tiles per chunk (2 with fuse_grows: a band workgroup's own key tiles)
    int fuse_grows;       // 1: the bf16 band pass computes the global rows' partials on its own key tiles
    int xcd_remap;        // 1: group consecutive work items on one XCD; 2: heads per XCD, heaviest tiles first
    float scale_log2;     // score scale * log2(e)
    int stride;           // > 0: also the positions at distance stride * 2^m
    int rand_block;       // > 0: random-block rule, blocks of rand_block positions
    int n_rand;           // key blocks listed per query block
    const int *rand_idx;  // device [ceil(N / rand_block)][n_rand] key-block lists
    int gidx[kMaxGlobal]; // sorted global positions
};

// K/V head (over B * H_kv) read by query head bh (over B * H): query heads
// h = g*group .. g*group + group - 1 of one batch entry share K/V head g.
__host__ __device__ __forceinline__ long long kv_head(const FwdParams &p, int bh) {
    const int b = bh / p.H, h = bh - b * p.H;
    return (long long)b * (p.H / p.group) + h / p.group;
}

// Backward arguments (bf16 tensors, fp32 LSE and row terms).
struct BwdParams {
    const void *q, *k, *v, *out, *dout;
    const float *lse;       // forward LSE, natural log, [B*H][N]
    void *dq, *dk, *dv;
    float *delta;           // workspace: rowsum(dO * O), [B*H][N]
    float *lse2;            // workspace: LSE * log2(e) (the exponent offset of P), [B*H][N]
    long long head_stride;  // N * d elements
    int BH;                 // B * H
    int H, group;           // query heads per batch entry; per K/V head
    int N;
    int wl, wr;             // normalised band
    int block, cap;         // block-sparse rule (0: window rule)
    int dil;                // dilation: rows r, r+dil, ... form one sequence (1: plain)
    int causal;
    int num_qt;             // query tiles of the dQ pass (per residue class when dil > 1)
    int num_kt;             // key tiles of the dK/dV pass (per residue class when dil > 1)
    int xcd_remap_q, xcd_remap_k;
    float scale;            // score scale
    float scale_log2;       // scale * log2(e)
    // global tokens (n_global == 0: none)
    int n_global;
    int gchunks_q, gct_q;   // split pass over keys for the global rows: chunks, key tiles per chunk
    int gchunks_k, gct_k;   // split pass over query rows for the global columns
    float *part_q;          // workspace: [B*H][n_global][gchunks_q][d] fp32
    float *part_k;          // workspace: [B*H_kv][n_global][gchunks_k][2d] fp32
    int stride;             // > 0: also the positions at distance stride * 2^m
    int rand_block, n_rand; // random-block rule (rand_block 0: off)
    const int *rand_idx;    // device [ceil(N / rand_block)][n_rand] key-block lists
    int gidx[kMaxGlobal];   // sorted global positions
};

hipError_t launch_backward(const BwdParams &p, int d, hipStream_t stream);
// Chunks of a split pass over N positions shared by `units` workgroup rows.
void bwd_global_chunks(int units, int N, int *chunks, int *tiles_per_chunk);

// Decode arguments: the newest Nq queries of each sequence against a cache.
struct DecParams {
    const void *q;          // [B][H][Nq][d] bf16
    const void *kc, *vc;    // [B][H_kv][S][d] bf16
    void *out;              // [B][H][Nq][d] bf16
    float *lse;             // [B][H][Nq]
    float *part;            // workspace: [B*H*Nq][chunks][d + 2] partial (o, m, l)
    const int *seq_len;     // device [B]: total length of each sequence
    int B, H, H_kv, group, Nq, S;
    int win;                // positions i - win .. i are visible (-1: unbounded)
    int rolling;            // 1: position p lives in slot p % S
    int R;                  // query rows per K/V head: group * Nq
    int nrg;                // row groups of kDecRows per K/V head
    int chunks;             // cache chunks per row group (each sequence's tiles split evenly)
    float scale_log2;
};

constexpr int kDecRows = 128;        // query rows per decode workgroup (four waves)
constexpr int kDecMaxChunks = 256;   // most chunks one row is split into
hipError_t launch_decode(const DecParams &p, int d, hipStream_t stream);
int decode_chunks(int B, int H_kv, int nrg, int S, int Nq, int win, int rolling);
int bwd_tile_q(int d, int band_only);   // query rows per dQ workgroup (band_only: no global tokens, no extra rule)
int bwd_tile_k(int d);      // keys per dK/dV workgroup

// Tile shapes chosen per (d, dtype).
int tile_bm(int d, int f32);
int band_tile_bm(int d, int f32, int block, int extra, int wl, int wr, int dil);   // query rows per band workgroup
bool band_is_narrow(int wl, int wr, int dil);   // normalised band short enough for the four-wave band instance
int tile_bn(int d, int f32);

// Enqueue the band pass (every query tile), then, when n_global > 0, the
// split-key pass over global rows and the merge. Returns a hipError_t.
hipError_t launch_forward(const FwdParams &p, int d, int f32, hipStream_t stream);

// Number of key chunks the split-key pass uses for these sizes.
int global_chunks(int BH, int N, int d, int f32, int *chunk_tiles);
// Whether the band pass computes the global rows' partials itself (one per
// query tile of bm rows, over its own key tiles), instead of the split-key pass.
bool fuse_global_rows(int f32, int d, int dil, int bm, int ng);

// Device address, on the current device, of the allocation-free forward's
// scratch array (kNoAllocScratchBytes); looked up once per device.
hipError_t noalloc_scratch(void **ptr);

}  // namespace eea
