/*
 * attn.h - C ABI of the MI355X (gfx950) exact-attention forward library.
 *
 * The operation is exact scaled dot-product attention,
 *     out_i = sum_j softmax_j(q_i . k_j / sqrt(d)) v_j      (visible j only),
 * computed tile by tile with an online softmax so the N x N score matrix is
 * never stored ("Efficient Transformers: Sparse Attention, Linear Attention and
 * FlashAttention", sections "Family 3: exact attention, computed smarter" and
 * "The online softmax trick"; week-17 lecture notes on efficient attention,
 * FlashAttention tiling and online-softmax passages). Sparse masks follow the
 * week-17 notes (local window, Mistral sliding window, global tokens),
 * "Sparse & sub-quadratic attention" ("Escape 1") and "Module 9 - Quadratic
 * cost and efficient attention" ("Sparse and windowed attention").
 *
 * Conventions shared by every entry point:
 *   - Tensors q, k, v, out are dense row-major [B][H][N][d] (head-major, one
 *     row of d elements per token), element type bf16 (default) or fp32.
 *     lse is dense [B][H][N] fp32.
 *   - Every tensor pointer is a DEVICE pointer owned by the caller; the library
 *     never frees or retains it. Pointers must be 16-byte aligned (lse: 4).
 *     q, k and v may alias one another; out and lse must not overlap any input
 *     or each other.
 *   - global_idx is a HOST array of n_global int32 token positions, unique,
 *     each in [0, N), any order. It is copied before the call returns.
 *   - All device work is enqueued asynchronously on the chosen stream; the
 *     call does not synchronise. Execution errors surface at the caller's
 *     next synchronisation on that stream.
 *   - Every argument is validated before any HIP call. Functions return an
 *     attn_status; no exception crosses the ABI and the library never aborts.
 *     attn_last_error() gives a message for the last non-OK status of the
 *     calling thread.
 */
#ifndef EEA_ATTN_H
#define EEA_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_INVALID_ARG = 1,   /* bad pointer, size, index, alignment or overlap */
    ATTN_ERR_UNSUPPORTED = 2,   /* valid request this build does not implement */
    ATTN_ERR_DEVICE = 3         /* HIP runtime error; message in attn_last_error() */
} attn_status;

typedef enum { ATTN_BF16 = 0, ATTN_F32 = 1 } attn_dtype;

typedef struct attn_opts {
    int dtype;              /* attn_dtype of q, k, v and out */
    float scale;            /* score scale; 0 selects 1/sqrt(d) */
    void *stream;           /* hipStream_t to enqueue on; NULL = default stream */
    void *workspace;        /* device scratch for global-row partial results, or
                               NULL to use a library-owned buffer (see below) */
    size_t workspace_bytes; /* size of workspace; must be >= attn_workspace_bytes() */
} attn_opts;

/*
 * Library-owned scratch. A call that needs device scratch (forward with
 * global rows, backward, split decoding) and gets no opts->workspace uses a
 * buffer the library owns, one per device and per kind (forward, backward,
 * decoding). It is allocated on first use, grown when a call needs more
 * (the old buffer is freed once the last call that used it has finished)
 * and kept until the process ends. Calls that share it are ordered on the
 * device: each call's stream first waits for the work of the previous call
 * that used the buffer, whatever stream that was, so calls on different
 * streams run one after another where they share it. Callers that want
 * them to overlap pass a workspace of their own to each call.
 */

/*
 * attn_fwd - masked exact attention forward, bf16 in/out, scale 1/sqrt(d),
 * default stream. Equivalent to attn_fwd_ex(..., NULL).
 *
 *   q, k, v     [B][H][N][d] bf16 inputs.
 *   out         [B][H][N][d] bf16 output: softmax-weighted sum of value rows.
 *   lse         [B][H][N] fp32 output: natural log of the sum over visible
 *               keys of exp(scaled score), the per-row log-sum-exp that a
 *               recomputing backward pass needs.
 *   B, H, N     batch, heads, tokens (each >= 1). One head's K (or V) must
 *               stay below 2 GiB (N * d * element size < 2^31), else
 *               ATTN_ERR_UNSUPPORTED: tiles are addressed by 32-bit byte
 *               offsets from the head's base.
 *   d           head size, 64 or 128 (others: ATTN_ERR_UNSUPPORTED).
 *   causal      1: key j is visible from row i only if j <= i. 0: no such limit.
 *   win_left    keys strictly left of the diagonal that row i may see:
 *               j >= i - win_left. -1 = unbounded. A Mistral window of w
 *               tokens ending at i is win_left = w - 1.
 *   win_right   keys strictly right of the diagonal: j <= i + win_right.
 *               -1 = unbounded. Ignored (taken as 0) when causal = 1.
 *   global_idx  host array of global token positions (may be NULL when
 *               n_global = 0). A global row sees every key and a global
 *               column is seen by every row, the causal limit still applying.
 *   n_global    0..64 (more: ATTN_ERR_UNSUPPORTED).
 *
 * Visible(i, j) = [causal => j <= i] AND ( in_window(i, j) OR i in G OR j in G ).
 * Every row sees at least its diagonal key, so no row is empty.
 */
int attn_fwd(const void *q, const void *k, const void *v, void *out, float *lse,
             int B, int H, int N, int d, int causal, int win_left, int win_right,
             const int *global_idx, int n_global);

/*
 * attn_fwd_ex - as attn_fwd with options (opts may be NULL for defaults).
 * With opts->dtype = ATTN_F32, q, k, v and out are fp32 and both products run
 * in fp32 on the matrix cores. When n_global > 0 and the window does not
 * already cover every key, the global query rows are computed by a separate
 * split-key pass that needs attn_workspace_bytes() of device scratch: taken
 * from opts->workspace if given, else from a buffer the library owns (see
 * "Library-owned scratch" above).
 */
int attn_fwd_ex(const void *q, const void *k, const void *v, void *out, float *lse,
                int B, int H, int N, int d, int causal, int win_left, int win_right,
                const int *global_idx, int n_global, const attn_opts *opts);

/*
 * attn_fwd_noalloc - attn_fwd_ex that allocates no device memory, for callers
 * that cannot allocate: code being captured into a HIP graph, tight serving
 * loops, harnesses that forbid allocation. Arguments, outputs and errors are
 * those of attn_fwd_ex, except:
 *   - opts->workspace must be NULL (else ATTN_ERR_INVALID_ARG): the
 *     global-row partials go to a device array built into the library, one
 *     per device, ATTN_NOALLOC_SCRATCH_BYTES long, held from library load
 *     until the process ends;
 *   - a call whose global-row partials (attn_workspace_bytes) need more than
 *     ATTN_NOALLOC_SCRATCH_BYTES returns ATTN_ERR_UNSUPPORTED before any
 *     device work;
 *   - every call on one device uses the same array: calls that overlap on a
 *     device (different streams, no ordering between them) race and give
 *     wrong results. Order them, or use attn_fwd_ex with a workspace each.
 * Calls without global tokens need no scratch and are exactly attn_fwd_ex.
 * No hipMalloc, hipFree or other allocating call is made. The array is part
 * of the library's device code, which the HIP runtime loads (allocating it)
 * at the first launch of any of the library's kernels on a device, and the
 * first attn_fwd_noalloc call on a device looks up its address: make one
 * call (of any entry point, then of this one) before capturing a graph.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int attn_fwd_noalloc(const void *q, const void *k, const void *v, void *out, float *lse,
                     int B, int H, int N, int d, int causal, int win_left, int win_right,
                     const int *global_idx, int n_global, const attn_opts *opts);

/*
 * attn_mask - which (query row i, key j) pairs are visible, as one
 * descriptor. The local rule is one of
 *   window (block = 0, dilation <= 1): i - win_left <= j <= i + win_right,
 *       -1 for an unbounded side (the masks of attn_fwd);
 *   block-sparse (block > 0): j lies in the block of i or in the block just
 *       before it, blocks being runs of `block` positions ("Sparse &
 *       sub-quadratic attention", "Escape 1": attend within your block and
 *       the previous one). win_left and win_right must be -1;
 *   dilated (dilation = k > 1): j = i - m*k for whole m (week-17 lecture
 *       notes, dilated passage: i, i-k, i-2k, ...), with the window counted
 *       in those steps: -win_right <= m <= win_left. bf16 forward only, and
 *       not combined with global tokens.
 * causal (j <= i) is ANDed with the result, global tokens (rows that see
 * everything and columns seen by everyone) ORed with the local rule, and so
 * is at most one of two extra rules (window local rule only; bf16 only):
 *   strided (stride = s > 0): j is at distance s, 2s, 4s, ... from i ("Module
 *       9 - Quadratic cost and efficient attention", table in "Sparse and
 *       windowed attention": strides s, 2s, 4s with O(n log n) cost);
 *   random blocks (rand_block = b > 0): j lies in one of the key blocks listed
 *       for i's query block, blocks being runs of b positions (week-17 lecture
 *       notes, BigBird passage: global tokens + local window + random
 *       attention). The caller draws the lists: rand_idx is read on the
 *       device, row q of it lists the key blocks of query block q; entries
 *       outside [0, ceil(N / b)) are ignored and repeated entries count once.
 */
typedef struct attn_mask {
    int causal;             /* 0 or 1 */
    int win_left;           /* >= -1 */
    int win_right;          /* >= -1 */
    int block;              /* >= 0; 0 = no block rule */
    int dilation;           /* >= 0; 0 or 1 = no dilation */
    const int *global_idx;  /* host array of distinct positions in [0, N), or NULL */
    int n_global;           /* 0..64 */
    int stride;             /* >= 0; > 0: also the positions at distance stride * 2^m */
    int rand_block;         /* >= 0; > 0: random-block rule, blocks of rand_block positions (a multiple of 32) */
    int n_rand;             /* key blocks listed per query block: 1..16 (with rand_block > 0) */
    const int *rand_idx;    /* DEVICE int32 array [ceil(N / rand_block)][n_rand] of key-block indices */
} attn_mask;

/*
 * attn_fwd_masked - attn_fwd_gqa with the mask given as an attn_mask (which
 * adds the block-sparse and dilated rules). Arguments, outputs, workspace
 * and errors otherwise as attn_fwd_gqa; a NULL mask is ATTN_ERR_INVALID_ARG,
 * invalid combinations as described at attn_mask.
 */
int attn_fwd_masked(const void *q, const void *k, const void *v, void *out, float *lse,
                    int B, int H, int H_kv, int N, int d, const attn_mask *mask, const attn_opts *opts);

/*
 * attn_fwd_gqa - as attn_fwd_ex with fewer K/V heads than query heads:
 * grouped-query attention (H_kv groups of H/H_kv query heads, each group
 * sharing one K head and one V head) and, with H_kv = 1, multi-query
 * attention (one K/V head for every query head). Both are exact attention
 * with K and V shared, not an approximation (week-17 lecture notes on
 * efficient attention, the MQA / GQA passage on shrinking the KV cache).
 *
 *   q, out      [B][H][N][d]
 *   k, v        [B][H_kv][N][d]; query head h of batch entry b reads K/V
 *               head h / (H / H_kv) of the same b.
 *   H_kv        >= 1 and divides H (else ATTN_ERR_INVALID_ARG). H_kv = H is
 *               exactly attn_fwd_ex.
 * Every other argument, the outputs, the workspace and the error behaviour
 * are those of attn_fwd_ex (the workspace depends on B*H, not on H_kv).
 */
int attn_fwd_gqa(const void *q, const void *k, const void *v, void *out, float *lse,
                 int B, int H, int H_kv, int N, int d, int causal, int win_left, int win_right,
                 const int *global_idx, int n_global, const attn_opts *opts);

/*
 * attn_bwd - gradients of attn_fwd / attn_fwd_gqa with respect to q, k and v,
 * by recomputation: the scores are recomputed tile by tile and turned into
 * the exact softmax weights with the forward's lse, so no N x N matrix is
 * stored or built ("Efficient Transformers: Sparse Attention, Linear
 * Attention and FlashAttention", "Family 3": the tiled exact attention
 * recomputes what the backward pass needs). With P the softmax weights and
 * scale the score scale:
 *     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - rowsum(dO * out)),
 *     dQ = scale dS K,  dK = scale dS^T Q,
 * and a K/V head shared by a group of query heads receives the sum of their
 * contributions.
 *
 *   q, out, dout  [B][H][N][d] bf16: the forward's inputs, its output and the
 *                 gradient of the loss with respect to that output.
 *   k, v          [B][H_kv][N][d] bf16 (H_kv = H for plain multi-head).
 *   lse           [B][H][N] fp32: the forward's log-sum-exp output.
 *   dq            [B][H][N][d] bf16 output; dk, dv [B][H_kv][N][d] bf16
 *                 outputs. Every element is written; none may overlap an
 *                 input or another output.
 *   B, H, H_kv, N, d, causal, win_left, win_right: as in attn_fwd_gqa, and
 *                 they must be the forward call's values.
 *   global_idx, n_global: global tokens, as in attn_fwd (host array, at
 *                 most 64). Their pairs outside the band are handled by two
 *                 split passes whose fp32 partials live in the workspace.
 *   opts          as in attn_fwd_ex: only ATTN_BF16 (ATTN_F32 gives
 *                 ATTN_ERR_UNSUPPORTED), scale (must be the forward's),
 *                 stream, and a workspace of at least attn_bwd_workspace_bytes
 *                 (else the library-owned backward scratch is used).
 * Errors are reported as for attn_fwd_ex, before any launch.
 */
int attn_bwd(const void *q, const void *k, const void *v, const void *out, const void *dout,
             const float *lse, void *dq, void *dk, void *dv,
             int B, int H, int H_kv, int N, int d, int causal, int win_left, int win_right,
             const int *global_idx, int n_global, const attn_opts *opts);

/*
 * attn_bwd_masked - attn_bwd with the mask given as an attn_mask: window,
 * block-sparse and dilated rules, global tokens, the strided and random-block
 * rules (the combinations attn_fwd_masked accepts for bf16).
 */
int attn_bwd_masked(const void *q, const void *k, const void *v, const void *out, const void *dout,
                    const float *lse, void *dq, void *dk, void *dv,
                    int B, int H, int H_kv, int N, int d, const attn_mask *mask, const attn_opts *opts);

/*
 * attn_bwd_workspace_bytes - device scratch attn_bwd needs: two fp32 row terms
 * per query row (rowsum(dO * O) and the LSE in base 2; 2 * B*H*N*4 bytes, each
 * half rounded up to 256), plus, when n_global > 0,
 * the split passes' fp32 partials (O(n_global * d * N / 64) per head, never
 * O(N^2)). 0 for invalid sizes.
 */
size_t attn_bwd_workspace_bytes(int B, int H, int H_kv, int N, int d, int n_global);

/*
 * attn_decode - one decoding step over a key/value cache: the Nq newest
 * tokens of each sequence attend over the keys and values kept for every
 * earlier token and themselves (week-17 lecture notes: per-token inference
 * with a KV cache; "Beyond attention": a sliding window needs a rolling cache
 * of only W positions). Exact: the result equals the last Nq rows of the
 * causal (optionally windowed) forward over the whole sequence.
 *
 *   q           [B][H][Nq][d] bf16: queries of positions L_b-Nq .. L_b-1.
 *   k_cache,
 *   v_cache     [B][H_kv][S][d] bf16 caches of S slots (H_kv divides H;
 *               query head h reads K/V head h / (H / H_kv)).
 *   seq_len     DEVICE array of B int32: L_b, the length of sequence b
 *               including the Nq new tokens, whose keys and values must
 *               already be in the cache. Must satisfy Nq <= L_b, and
 *               L_b <= S for a contiguous cache; values outside are clamped
 *               into that range.
 *   out         [B][H][Nq][d] bf16 output; lse [B][H][Nq] fp32 (natural log).
 *   win_left    position i sees positions i - win_left .. i (-1: all earlier
 *               positions).
 *   rolling     0: position p is in slot p (contiguous cache). 1: position p
 *               is in slot p % S (the cache keeps the last S positions); needs
 *               win_left >= 0 and Nq + win_left <= S so every visible
 *               position is still cached.
 *   opts        bf16 only; scale, stream; workspace of at least
 *               attn_decode_workspace_bytes (else the library's scratch).
 * Errors are reported as for attn_fwd_ex, before any launch.
 */
int attn_decode(const void *q, const void *k_cache, const void *v_cache, const int *seq_len,
                void *out, float *lse, int B, int H, int H_kv, int Nq, int S, int d,
                int win_left, int rolling, const attn_opts *opts);

/*
 * attn_decode_workspace_bytes - device scratch attn_decode needs for its
 * per-chunk partial results: B*H*Nq*chunks*(d+2)*4 bytes, where the cache
 * is split into 1 <= chunks <= 256 parts; 0 when one chunk suffices (the
 * partials are not used) and for invalid sizes.
 */
size_t attn_decode_workspace_bytes(int B, int H, int H_kv, int Nq, int S, int d, int win_left,
                                   int rolling);

/*
 * attn_workspace_bytes - device scratch a call with these sizes needs for the
 * global-row partial results; 0 when n_global = 0. It grows with
 * B*H*n_global*d and a chunk count bounded by N/64, never with N*N.
 * Returns 0 for invalid sizes.
 */
size_t attn_workspace_bytes(int B, int H, int N, int d, int n_global);

/*
 * attn_plan_stats - host-only description of the work the tile scheduler
 * does for one head at a tile shape of bm query rows by bn keys: the number
 * of visible (i, j) pairs, and the number of band key tiles visited that need
 * no mask (tiles_full) or need one (tiles_edge), summed over the query tiles.
 * Tiles with no visible pair are never visited and not counted. Global
 * columns add ceil(n_global / bn) gathered tiles per query tile (counted in
 * tiles_edge);
 * global rows are counted as ceil(keys / bn) edge tiles each. Output
 * pointers are host pointers; any may be NULL. Makes no HIP call.
 */
int attn_plan_stats(int N, int causal, int win_left, int win_right,
                    const int *global_idx, int n_global, int bm, int bn,
                    long long *visible_pairs, long long *tiles_full,
                    long long *tiles_edge);

/*
 * attn_plan_stats_masked - attn_plan_stats for an attn_mask. With a dilated
 * mask the counts are summed over the residue classes, each planned as its
 * own band over its strided rows (the way the forward kernel visits them).
 * The strided rule's extra tiles are counted in tiles_edge (random blocks'
 * tiles are not); with the random-block rule the call reads the lists from
 * device memory with one blocking copy (the only HIP call of the planner)
 * and fails with ATTN_ERR_DEVICE if it cannot.
 */
int attn_plan_stats_masked(int N, const attn_mask *mask, int bm, int bn,
                           long long *visible_pairs, long long *tiles_full,
                           long long *tiles_edge);

/*
 * attn_tile_shape - the tile shape (query rows per workgroup, keys per tile)
 * of the forward band kernel for head size d and element type dtype, with an
 * unbounded window (plain or causal). bf16 calls whose band is bounded on
 * both sides and at most 4096 keys wide, or that use the block-sparse,
 * strided or random-block rules, run 128-row workgroups with the same key
 * tiles. Host-only, no HIP call.
 */
int attn_tile_shape(int d, int dtype, int *bm, int *bn);

/* attn_last_error - message for the calling thread's last non-OK status ("" if none). */
const char *attn_last_error(void);

/* attn_version - library version string. */
const char *attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EEA_ATTN_H */
