// attn_bwd.hip - gfx950 kernels for the backward pass of exact masked
// attention, by recomputation: no N x N matrix is kept from the forward pass;
// the scores are recomputed tile by tile and turned into exact softmax
// weights with the forward's per-row log-sum-exp ("Efficient Transformers:
// Sparse Attention, Linear Attention and FlashAttention", "Family 3": the
// tiled exact attention recomputes what the backward pass needs).
//
// Gradients (chain rule of O = softmax(scale Q K^T) V, masked entries out):
//   P  = exp(scale S - LSE)          dV = P^T dO          dP = dO V^T
//   dS = P * (dP - rowsum(dO * O))   dQ = scale dS K      dK = scale dS^T Q
//
// Three kernels:
//  * bwd_delta: rowsum(dO * O) per query row (fp32), into the workspace.
//  * bwd_dkdv: one workgroup per (K/V head, 128 keys); each wave keeps its 32
//    keys' K and V as MFMA operands and walks the visible 64-row query tiles
//    of every query head that reads this K/V head, accumulating
//    dV^T += dO^T P and dK^T += Q^T dS in registers: grouped-query heads are
//    summed here, with no atomics.
//  * bwd_dq: one workgroup per (query head, 128 rows; 256 for the d = 128
//    band instance); each wave keeps its 32 rows' Q and dO as operands and
//    walks the visible 64-key tiles, accumulating dQ^T += K^T dS^T.
// All products use v_mfma_f32_32x32x16_bf16 in the transposed forms of the
// forward pass, so each of them is one of the bf16 tile path's two operand
// patterns (row reads, transpose reads); the tiles read both ways (Q and dO
// in dK/dV, K in dQ) are copied into LDS once, in the tile path's unified
// layout, which serves both patterns without bank conflicts.
// Band masks (causal, windows, block-sparse), dilated masks (one band per
// residue class of rows) and global tokens (below) are handled.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_internal.h"
#include "attn_plan.h"
#include "attn_tiles.h"

namespace eea {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Row terms per query row: rowsum(dO * O), and LSE * log2(e) (so the
// score loops form P = exp2(S c - LSE log2 e) with one FMA per element);
// 8 lanes per row, 32 rows per workgroup.
template <int D>
__global__ void __launch_bounds__(kBwdThreads) bwd_delta(const BwdParams prm) {
    constexpr int PER = D / 8;   // elements per lane
    const long long rows = (long long)prm.BH * prm.N;
    const long long r = (long long)blockIdx.x * 32 + (threadIdx.x >> 3);
    const int sub = threadIdx.x & 7;
    float acc = 0.f;
    if (r < rows) {
        const uint16_t *o = static_cast<const uint16_t *>(prm.out) + r * D + sub * PER;
        const uint16_t *g = static_cast<const uint16_t *>(prm.dout) + r * D + sub * PER;
#pragma unroll
        for (int c = 0; c < PER / 8; ++c) {
            const u32x4 a = reinterpret_cast<const u32x4 *>(o)[c];
            const u32x4 b = reinterpret_cast<const u32x4 *>(g)[c];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc = __builtin_fmaf(bf16_to_f32(a[e] & 0xffffu), bf16_to_f32(b[e] & 0xffffu), acc);
                acc = __builtin_fmaf(bf16_to_f32(a[e] >> 16), bf16_to_f32(b[e] >> 16), acc);
            }
        }
    }
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    acc += __shfl_xor(acc, 4);
    if (sub == 0 && r < rows) {
        prm.delta[r] = acc;
        prm.lse2[r] = prm.lse[r] * kLog2e;
    }
}

// ---------------------------------------------------------------------------
// Global tokens. The visible pairs split into three disjoint sets:
//   S1  key in the row's band (every row, every column): the band loops,
//       unchanged;
//   S2  a global column outside a non-global row's band (causal cut): in
//       bwd_dq a gathered key tile of the global columns, in the dK/dV of the
//       global columns a split pass over query rows (BWD_GSET of bwd_dkdv);
//   S3  a global row's keys outside its band (causal cut): in bwd_dkdv a
//       gathered query tile of the global rows, in the dQ of the global rows
//       a split pass over keys (BWD_GSET of bwd_dq).
// The split passes leave fp32 partials that merge kernels add to the band
// kernels' outputs for those (at most 64) rows.
// ---------------------------------------------------------------------------
enum { BWD_BAND = 0, BWD_BAND_GL = 1, BWD_GSET = 2 };

// Waves per SIMD of an instance. At d = 64 the instances that fit 256
// registers run two per SIMD (two workgroups per CU), so one workgroup's
// copies and barriers overlap the other's products: every dQ instance, and
// the dK/dV band loop (in its unpipelined form: the pipelined one needs more
// registers), with or without the gathered tile of global rows, and split
// pass. Measured on d = 64: 36-40 % less time for a causal or banded
// backward than at one wave per SIMD with the pipelined loops, 20 % less for
// band 256 + 9 global tokens. d = 128 and the dK/dV extra-tile instances keep
// one wave per SIMD.
template <int D, int MODE, bool XT>
constexpr int dkdv_waves() { return (D == 64 && !XT) ? 2 : 1; }
template <int D>
constexpr int dq_waves() { return D == 64 ? 2 : 1; }
// Threads of a dQ instance. At d = 128 the band instance (no global tokens,
// no extra tiles) runs eight waves, 256 rows per workgroup, two per SIMD,
// with the unpipelined loop (it fits 256 registers; the pipelined one does
// not): 14 % less dQ time on a long causal head than four waves at one per
// SIMD with the pipelined loop.
template <int D, int MODE, bool XT>
constexpr int dq_threads() { return (D == 128 && MODE == BWD_BAND && !XT) ? 512 : kBwdThreads; }

// Bit r set when row q0 + r (r < 64) is a global position.
__device__ __forceinline__ unsigned long long global_rows_in(const int *g, int ng, int q0) {
    unsigned long long m = 0;
    for (int t = 0; t < ng; ++t) {
        const int r = g[t] - q0;
        if (r >= 0 && r < 64) m |= 1ull << r;
    }
    return m;
}

// ---------------------------------------------------------------------------
// Software pipeline of the dK/dV band loop, for the instances that run one
// wave per SIMD (nothing else then hides a wave's vector work). Iteration t runs S(t) and dP(t), then one
// region in which the 32 MFMAs of dV += dO(t-1)^T P(t-1) and
// dK += Q(t-1)^T dS(t-1) are issued in batches of four, each batch followed
// by the vector work of four elements of tile t: P = exp2(S c - LSE log2 e)
// and dS = P (dP - rowsum(dO O)). The A operands of a batch (transpose reads
// of tile t-1's dO and Q) are read one batch ahead; the row terms of the
// element group likewise.
// ---------------------------------------------------------------------------
// Both score products of one tile (S with the first B operand, dP with the
// second) as one stream of MFMAs that alternates between them, so the two
// accumulator chains hide each other's latency and are live together. The
// A operands (row layout, from LDS) are read one batch of four ahead.
template <class P>
struct ScorePair {
    static constexpr int MB = P::MB, KS = P::KS;
    static constexpr int kB = 4, kSlots = 8;
    static constexpr int NM = 2 * KS * MB;   // MFMAs (32 at d=128, 16 at d=64)
    static_assert(NM % kB == 0, "whole batches");

    template <int J>
    static __device__ __forceinline__ void fetch(bf16x8 (&op)[kSlots], const typename P::Lane &L, const char *ba,
                                                 const char *bb) {
        if constexpr (J < NM) {
            constexpr int I = J / 2, ks = I / MB, mb = I % MB;
            op[J % kSlots] = *reinterpret_cast<const bf16x8 *>(((J & 1) ? bb : ba) + L.krd[ks] + mb * 32 * P::ROWB);
        }
    }
    template <int B>
    static __device__ __forceinline__ void run(f32x16 (&sa)[MB], f32x16 (&sb)[MB], const typename P::QFrag &fa,
                                               const typename P::QFrag &fb, const typename P::Lane &L, const char *ba,
                                               const char *bb, bf16x8 (&op)[kSlots]) {
        if constexpr (B < NM / kB) {
            if constexpr (B + 1 < NM / kB) {
                fetch<kB * (B + 1) + 0>(op, L, ba, bb);
                fetch<kB * (B + 1) + 1>(op, L, ba, bb);
                fetch<kB * (B + 1) + 2>(op, L, ba, bb);
                fetch<kB * (B + 1) + 3>(op, L, ba, bb);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int u = 0; u < kB; ++u) {
                const int J = kB * B + u, I = J / 2, ks = I / MB, mb = I % MB;
                if (J & 1) sb[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[J % kSlots], fb.x[ks], sb[mb], 0, 0, 0);
                else sa[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[J % kSlots], fa.x[ks], sa[mb], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            run<B + 1>(sa, sb, fa, fb, L, ba, bb, op);
        }
    }
    static __device__ __forceinline__ void scores(f32x16 (&sa)[MB], f32x16 (&sb)[MB], const typename P::QFrag &fa,
                                                  const typename P::QFrag &fb, const typename P::Lane &L,
                                                  const char *ba, const char *bb) {
        bf16x8 op[kSlots];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            sa[mb] = f32x16{};
            sb[mb] = f32x16{};
        }
        fetch<0>(op, L, ba, bb);
        fetch<1>(op, L, ba, bb);
        fetch<2>(op, L, ba, bb);
        fetch<3>(op, L, ba, bb);
        __builtin_amdgcn_sched_barrier(0);
        run<0>(sa, sb, fa, fb, L, ba, bb, op);
    }
};

template <class P>
struct BwdPipe {
    static constexpr int MB = P::MB, DB = P::DB, PVS = P::PVS;
    static constexpr int kB = 4, kSlots = 8;
    static constexpr int NHALF = PVS * DB;        // MFMAs per product (16 at d=128, 8 at d=64)
    static constexpr int NB = 2 * NHALF / kB;     // batches
    static constexpr int GPB = 4 * MB / NB;       // element groups (4 of a 32-row block) per batch
    static_assert(GPB * NB == 4 * MB, "whole element groups per batch");

    template <int I>
    static __device__ __forceinline__ void fetch(bf16x8 (&op)[kSlots], const typename P::Lane &L, const char *ov,
                                                 const char *qv) {
        if constexpr (I < 2 * NHALF) {
            constexpr int J = I % NHALF;
            op[I % kSlots] = P::v_operand(L, I < NHALF ? ov : qv, J % DB, J / DB);
        }
    }

    // row terms (LSE log2 e, rowsum(dO O)) of the element groups of batch B
    template <int B>
    static __device__ __forceinline__ void terms(f32x4 (&l4)[GPB], f32x4 (&d4)[GPB], const float *lse, const float *dl,
                                                 int h) {
#pragma unroll
        for (int j = 0; j < GPB; ++j) {
            const int gi = B * GPB + j, mb = gi / 4, g = gi % 4;
            l4[j] = *reinterpret_cast<const f32x4 *>(&lse[32 * mb + 8 * g + 4 * h]);
            d4[j] = *reinterpret_cast<const f32x4 *>(&dl[32 * mb + 8 * g + 4 * h]);
        }
    }

    template <bool MM, bool VA, bool EDGE, int B>
    static __device__ __forceinline__ void run(f32x16 (&dv)[DB], f32x16 (&dk)[DB], const typename P::PFrag &pp,
                                               const typename P::PFrag &pd, f32x16 (&s)[MB], f32x16 (&dp)[MB],
                                               const typename P::Lane &L, const char *ov, const char *qv,
                                               bf16x8 (&op)[kSlots], f32x4 (&l4)[GPB], f32x4 (&d4)[GPB],
                                               const float *lse, const float *dl, float c, int h, int q0, int qlo,
                                               int qhi) {
        if constexpr (B < NB) {
            f32x4 nl4[GPB], nd4[GPB];
            if constexpr (MM && B + 1 < NB) {
                fetch<kB * (B + 1) + 0>(op, L, ov, qv);
                fetch<kB * (B + 1) + 1>(op, L, ov, qv);
                fetch<kB * (B + 1) + 2>(op, L, ov, qv);
                fetch<kB * (B + 1) + 3>(op, L, ov, qv);
            }
            if constexpr (VA && B + 1 < NB) terms<B + 1>(nl4, nd4, lse, dl, h);
            if constexpr ((MM || VA) && B + 1 < NB) __builtin_amdgcn_sched_barrier(0);
            if constexpr (MM) {
#pragma unroll
                for (int u = 0; u < kB; ++u) {
                    const int I = kB * B + u, J = I % NHALF, st = J / DB, db = J % DB;
                    if (I < NHALF) dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[I % kSlots], pp.x[st], dv[db], 0, 0, 0);
                    else dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[I % kSlots], pd.x[st], dk[db], 0, 0, 0);
                }
            }
            if constexpr (VA) {
#pragma unroll
                for (int j = 0; j < GPB; ++j) {
                    const int gi = B * GPB + j, mb = gi / 4, g = gi % 4;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * g + e;
                        float p = fast_exp2(__builtin_fmaf(s[mb][r], c, -l4[j][e]));
                        if constexpr (EDGE) {
                            const int i = q0 + 32 * mb + acc_row(r, h);
                            p = ((i >= qlo) & (i <= qhi)) ? p : 0.f;
                        }
                        s[mb][r] = p;
                        dp[mb][r] = p * (dp[mb][r] - d4[j][e]);
                    }
                }
            }
            if constexpr (MM && VA) {
                constexpr int NV = GPB * 4 * (EDGE ? 7 : 4) / kB;   // per element: fma, exp, sub, mul (+ mask)
#pragma unroll
                for (int u = 0; u < kB; ++u) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x402, NV, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (VA && B + 1 < NB) {
#pragma unroll
                for (int j = 0; j < GPB; ++j) {
                    l4[j] = nl4[j];
                    d4[j] = nd4[j];
                }
            }
            run<MM, VA, EDGE, B + 1>(dv, dk, pp, pd, s, dp, L, ov, qv, op, l4, d4, lse, dl, c, h, q0, qlo, qhi);
        }
    }

    // MM: the dV/dK MFMAs of the previous tile; VA: the vector work of this
    // tile (S, dP in s, dp become P, dS in place).
    template <bool MM, bool VA, bool EDGE>
    static __device__ __forceinline__ void region(f32x16 (&dv)[DB], f32x16 (&dk)[DB], const typename P::PFrag &pp,
                                                  const typename P::PFrag &pd, f32x16 (&s)[MB], f32x16 (&dp)[MB],
                                                  const typename P::Lane &L, const char *ov, const char *qv,
                                                  const float *lse, const float *dl, float c, int h, int q0, int qlo,
                                                  int qhi) {
        bf16x8 op[kSlots];
        f32x4 l4[GPB], d4[GPB];
        if constexpr (MM) {
            fetch<0>(op, L, ov, qv);
            fetch<1>(op, L, ov, qv);
            fetch<2>(op, L, ov, qv);
            fetch<3>(op, L, ov, qv);
        }
        if constexpr (VA) terms<0>(l4, d4, lse, dl, h);
        __builtin_amdgcn_sched_barrier(0);
        run<MM, VA, EDGE, 0>(dv, dk, pp, pd, s, dp, L, ov, qv, op, l4, d4, lse, dl, c, h, q0, qlo, qhi);
    }
};

// ---------------------------------------------------------------------------
// dK, dV: keys stationary, query tiles streamed.
// BWD_BAND / BWD_BAND_GL: one workgroup per (K/V head, [residue class,] key
//   tile); BWD_BAND_GL adds, per query head, the gathered tile of global rows
//   (set S3).
// BWD_GSET: the global columns as the keys (one workgroup per (K/V head,
//   chunk of query tiles)), rows of set S2, fp32 partials out.
// ---------------------------------------------------------------------------
// XT (with BWD_BAND_GL): the rows that see this workgroup's keys by the
// log-spaced strided or the random-block rule, as extra query tiles.
template <int D, bool DIL, int MODE, bool XT = false>
__global__ void __launch_bounds__(kBwdThreads, (dkdv_waves<D, MODE, XT>())) bwd_dkdv(const BwdParams prm) {
    // Q and dO tiles are read both ways (row reads for S and dP, transpose
    // reads for dK and dV): the unified LDS layout serves both from one copy.
    typedef Bf16Path<D, kBwdThreads, true> P;
    constexpr int BQ = P::BN;               // query rows per streamed tile
    constexpr int BK = 32 * P::NW;          // keys per workgroup
    constexpr int MB = P::MB, DB = P::DB;
    static_assert(!(DIL && MODE != BWD_BAND), "dilation is not combined with global tokens");
    // the software-pipelined band loop (below) reads a tile's rows in one
    // iteration and its transposed operands in the next: three buffer sets
    constexpr bool PIPE = !(MODE == BWD_GSET || XT || dkdv_waves<D, MODE, XT>() == 2);

    // Q and dO of one query tile, one copy each; two sets (three for the
    // pipelined loop), distinct objects, the loops unrolled to match.
    __shared__ __attribute__((aligned(1024))) char qb0[P::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char ob0[P::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char qb1[P::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char ob1[P::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char qb2[PIPE ? P::TILE_BYTES : 16];
    __shared__ __attribute__((aligned(1024))) char ob2[PIPE ? P::TILE_BYTES : 16];
    __shared__ __attribute__((aligned(16))) float s_lse[2][BQ];   // LSE * log2(e)
    __shared__ __attribute__((aligned(16))) float s_dl[2][BQ];    // rowsum(dO * O)
    __shared__ int s_g[kMaxGlobal];                               // sorted global positions
    __shared__ int s_hit[XT ? kBwdThreads : 1];                    // random-block list hits of one scan chunk
    __shared__ int s_nhit[XT ? kBwdThreads / 64 : 1];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ln = lane & 31, h = lane >> 5;
    const int H_kv = prm.H / prm.group;
    const int ng = MODE == BWD_BAND ? 0 : prm.n_global;
    if constexpr (MODE != BWD_BAND) {
        if (tid < kMaxGlobal) s_g[tid] = tid < ng ? prm.gidx[tid] : -1;
        __syncthreads();
    }

    // work item
    const int G = gridDim.x, bid = blockIdx.x;
    const int Lw = prm.xcd_remap_k ? (bid & 7) * (G >> 3) + (bid >> 3) : bid;
    const int dil = DIL ? prm.dil : 1;
    int bkv, rcls = 0, kt = 0, chunk = 0;
    if constexpr (MODE == BWD_GSET) {
        bkv = Lw / prm.gchunks_k;
        chunk = Lw - bkv * prm.gchunks_k;
    } else {
        const int per_kv = dil * prm.num_kt;
        bkv = Lw / per_kv;
        rcls = (Lw - bkv * per_kv) / prm.num_kt;
        kt = Lw - bkv * per_kv - rcls * prm.num_kt;
    }
    const int N = DIL ? (prm.N - rcls + dil - 1) / dil : prm.N;   // rows of this residue class
    if (MODE != BWD_GSET && kt * BK >= N) return;                  // whole workgroup: a shorter class
    const Band band{N, prm.wl, prm.wr, prm.block, prm.cap};
    const int b = bkv / H_kv, kvh = bkv - b * H_kv;
    const long long cls_off = (long long)rcls * D;   // first row of the class
    const uint16_t *kh = static_cast<const uint16_t *>(prm.k) + (long long)bkv * prm.head_stride + cls_off;
    const uint16_t *vh = static_cast<const uint16_t *>(prm.v) + (long long)bkv * prm.head_stride + cls_off;

    typename P::Lane L;
    P::init_lane(L, lane, wave, dil);

    // this lane's key: a band key, or (BWD_GSET) a global column
    const int K0 = kt * BK;
    int key, k0w, k1w;
    bool kvalid, wave_active;
    if constexpr (MODE == BWD_GSET) {
        const int r = wave * 32 + ln;
        kvalid = r < ng;
        key = kvalid ? s_g[r] : 0;
        wave_active = wave * 32 < ng;
        k0w = 0;
        k1w = N - 1;
    } else {
        key = K0 + wave * 32 + ln;
        kvalid = key < N;
        k0w = K0 + wave * 32;
        k1w = imin(N - 1, k0w + 31);
        wave_active = k0w < N;
    }
    // rows whose local interval holds this lane's key, and the query tiles
    // this workgroup streams
    const int qlo = col_lo(band, key), qhi = col_hi(band, key);
    int qt_lo, nqt;
    if constexpr (MODE == BWD_GSET) {
        const int ntot = (N + BQ - 1) / BQ;
        qt_lo = chunk * prm.gct_k;
        nqt = imax(0, imin(prm.gct_k, ntot - qt_lo));
    } else {
        const int glo = col_lo(band, K0), ghi = col_hi(band, imin(N - 1, K0 + BK - 1));
        qt_lo = glo / BQ;
        nqt = ghi / BQ - qt_lo + 1;
    }
    const int T = prm.group * nqt;   // (query head, query tile) pairs

    // this wave's keys as the B operands of S = Q K^T and dP = dO V^T
    typename P::QFrag kf, vf;
    P::load_q(kf, kh, key * dil, kvalid, h);
    P::load_q(vf, vh, key * dil, kvalid, h);

    f32x16 dk[DB], dv[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) { dk[db] = f32x16{}; dv[db] = f32x16{}; }
    const float c = prm.scale_log2;

    auto head_of = [&](int t) { return b * prm.H + kvh * prm.group + t / nqt; };
    auto tile_of = [&](int t) { return qt_lo + t % nqt; };
    auto issue = [&](int t, char *qb, char *ob) __attribute__((always_inline)) {
        const long long bh = head_of(t);
        const int q0 = tile_of(t) * BQ;
        const uint16_t *qh = static_cast<const uint16_t *>(prm.q) + bh * prm.head_stride + cls_off;
        const uint16_t *gh = static_cast<const uint16_t *>(prm.dout) + bh * prm.head_stride + cls_off;
        P::issue_k(L, qh, N, qb, q0, dil);
        P::issue_k(L, gh, N, ob, q0, dil);
    };
    // per-row terms of tile t (LSE and rowsum(dO * O)) copied straight into
    // LDS by one wave, like the tiles (rows past the sequence read as 0): a
    // load into registers made the compiler wait for it, and with it for
    // every tile copy issued before it, ahead of the next score MFMAs
    auto issue_terms = [&](int t, float *lse_dst, float *dl_dst) __attribute__((always_inline)) {
        if (wave == 0) {
            const long long bh = head_of(t);
            const int i = tile_of(t) * BQ + lane;
            const unsigned off = (unsigned)(rcls + i * dil) * 4u;   // row in the stored sequence
            const __amdgpu_buffer_rsrc_t lr =
                __builtin_amdgcn_make_buffer_rsrc(prm.lse2 + bh * prm.N, 0, prm.N * 4, 0x00020000);
            const __amdgpu_buffer_rsrc_t dr =
                __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(prm.delta + bh * prm.N), 0, prm.N * 4, 0x00020000);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(lr, (EEA_LDS void *)lse_dst, 4, off, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(dr, (EEA_LDS void *)dl_dst, 4, off, 0, 0, 0);
        }
    };

    // the four products of one staged query tile; row(r) gives the sequence
    // row of tile slot r (or -1), vis(i) the extra test of an edge tile. The
    // edge mask is a pass of its own under a wave-uniform branch: folded
    // into the element loop, the compiler had turned it into selects that
    // every tile executed (about as many vector instructions as the rest).
    auto tile_products = [&](const char *qb, const char *ob, int sb, int cl, auto row, auto vis)
        __attribute__((always_inline)) {
        f32x16 s[MB], dp[MB];
        P::scores(s, kf, L, qb);    // S  = Q K^T : lane = key, registers = query rows
        P::scores(dp, vf, L, ob);   // dP = dO V^T
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 l4 = *reinterpret_cast<const f32x4 *>(&s_lse[sb][32 * mb + 8 * g + 4 * h]);
#pragma unroll
                for (int e = 0; e < 4; ++e) s[mb][4 * g + e] = fast_exp2(__builtin_fmaf(s[mb][4 * g + e], c, -l4[e]));
            }
        if (cl == TILE_EDGE) {
            asm volatile("");   // keeps this a branch (no speculation into selects)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[mb][r] = vis(row(32 * mb + acc_row(r, h))) ? s[mb][r] : 0.f;
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 d4 = *reinterpret_cast<const f32x4 *>(&s_dl[sb][32 * mb + 8 * g + 4 * h]);
#pragma unroll
                for (int e = 0; e < 4; ++e) dp[mb][4 * g + e] = s[mb][4 * g + e] * (dp[mb][4 * g + e] - d4[e]);
            }
        typename P::PFrag pp, pd;
        P::pack_p(pp, s);
        P::pack_p(pd, dp);
        P::pv(dv, pp, L, ob);   // dV^T += dO^T P
        P::pv(dk, pd, L, qb);   // dK^T += Q^T dS
    };

    // The split pass over global columns and the extra-rule instance (whose
    // extra code does not fit beside the pipeline's registers) keep the
    // unpipelined loop.
    if constexpr (!PIPE) {
        auto step = [&](int t, const char *qb, const char *ob, char *nqb, char *nob, int sb)
            __attribute__((always_inline)) {
            const bool more = t + 1 < T;
            debug_sync();
            if (more) {
                issue(t + 1, nqb, nob);
                issue_terms(t + 1, s_lse[sb ^ 1], s_dl[sb ^ 1]);
            }
            debug_sync();
            const int q0 = tile_of(t) * BQ;
            if constexpr (MODE == BWD_GSET) {
                // set S2: rows outside the key's band, not global, causal cut
                if (wave_active) {
                    const unsigned long long gm = global_rows_in(s_g, ng, q0);
                    tile_products(qb, ob, sb, TILE_EDGE, [&](int r) { return q0 + r; },
                                  [&](int i) {
                                      return kvalid & (i < N) & ((i < qlo) | (i > qhi)) &
                                             ((prm.causal == 0) | (i >= key)) & !((gm >> (i - q0)) & 1ull);
                                  });
                }
            } else {
                const int q1 = imin(N - 1, q0 + BQ - 1);
                int cl = wave_active ? classify(band, q0, q1, k0w, k1w) : TILE_SKIP;
                if (cl == TILE_FULL && q0 + BQ - 1 >= N) cl = TILE_EDGE;
                if (cl != TILE_SKIP)
                    tile_products(qb, ob, sb, cl, [&](int r) { return q0 + r; },
                                  [&](int i) { return (i >= qlo) & (i <= qhi); });
            }
            wait_vmem();
            __syncthreads();
        };
        if (T > 0) {
            issue(0, qb0, ob0);
            issue_terms(0, s_lse[0], s_dl[0]);
            wait_vmem();
            __syncthreads();
        }
        for (int t = 0; t < T; t += 2) {
            step(t, qb0, ob0, qb1, ob1, 0);
            if (t + 1 >= T) break;
            step(t + 1, qb1, ob1, qb0, ob0, 1);
        }
    } else {
        // band tiles, software-pipelined (BwdPipe). Iteration t copies tile
        // t+1, reads tile t's rows (S, dP) and tile t-1's transposed operands
        // (dV, dK of tile t-1): three buffer sets in rotation, the loop
        // unrolled by three so every buffer is a named object.
        typedef BwdPipe<P> BP;
        typename P::PFrag pp, pd;   // P and dS of the previous active tile
        bool act_prev = false;
        auto pstep = [&](int t, const char *qb, const char *ob, char *nqb, char *nob, const char *qb_p,
                         const char *ob_p, int sb) __attribute__((always_inline)) {
            const bool more = t + 1 < T;
            debug_sync();
            if (more) {
                issue(t + 1, nqb, nob);
                issue_terms(t + 1, s_lse[sb ^ 1], s_dl[sb ^ 1]);
            }
            debug_sync();
            const int q0 = tile_of(t) * BQ;
            const int q1 = imin(N - 1, q0 + BQ - 1);
            int cl = wave_active ? classify(band, q0, q1, k0w, k1w) : TILE_SKIP;
            if (cl == TILE_FULL && q0 + BQ - 1 >= N) cl = TILE_EDGE;
            const bool act = cl != TILE_SKIP;
            f32x16 s[MB], dp[MB];
            // S = Q K^T and dP = dO V^T (lane = key, registers = query rows);
            // one after the other with global tokens, where the registers
            // for both chains at once run out
            if (act) {
                if constexpr (MODE == BWD_BAND_GL) {
                    P::scores(s, kf, L, qb);
                    P::scores(dp, vf, L, ob);
                } else {
                    ScorePair<P>::scores(s, dp, kf, vf, L, qb, ob);
                }
            }
            const float *lr = s_lse[sb], *dr = s_dl[sb];
            if (act_prev) {
                if (act) {
                    if (cl == TILE_EDGE)
                        BP::template region<true, true, true>(dv, dk, pp, pd, s, dp, L, ob_p, qb_p, lr, dr, c, h, q0, qlo, qhi);
                    else
                        BP::template region<true, true, false>(dv, dk, pp, pd, s, dp, L, ob_p, qb_p, lr, dr, c, h, q0, qlo, qhi);
                } else {
                    BP::template region<true, false, false>(dv, dk, pp, pd, s, dp, L, ob_p, qb_p, lr, dr, c, h, q0, qlo, qhi);
                }
            } else if (act) {
                if (cl == TILE_EDGE)
                    BP::template region<false, true, true>(dv, dk, pp, pd, s, dp, L, ob_p, qb_p, lr, dr, c, h, q0, qlo, qhi);
                else
                    BP::template region<false, true, false>(dv, dk, pp, pd, s, dp, L, ob_p, qb_p, lr, dr, c, h, q0, qlo, qhi);
            }
            if (act) {
                P::pack_p(pp, s);
                P::pack_p(pd, dp);
            }
            act_prev = act;
            wait_vmem();
            __syncthreads();
        };
        if (T > 0) {
            issue(0, qb0, ob0);
            issue_terms(0, s_lse[0], s_dl[0]);
            wait_vmem();
            __syncthreads();
        }
        // tile x sits in set x % 3; its row terms in slot x & 1
        for (int t = 0; t < T; t += 3) {
            pstep(t, qb0, ob0, qb1, ob1, qb2, ob2, t & 1);
            if (t + 1 >= T) break;
            pstep(t + 1, qb1, ob1, qb2, ob2, qb0, ob0, (t + 1) & 1);
            if (t + 2 >= T) break;
            pstep(t + 2, qb2, ob2, qb0, ob0, qb1, ob1, t & 1);
        }
        // the last active tile's dV/dK products (its operands are still in
        // the set of tile T-1)
        if (act_prev) {
            f32x16 s[MB], dp[MB];
            const int r = (T - 1) % 3;
            if (r == 0)
                BP::template region<true, false, false>(dv, dk, pp, pd, s, dp, L, ob0, qb0, s_lse[0], s_dl[0], c, h, 0, 0, 0);
            else if (r == 1)
                BP::template region<true, false, false>(dv, dk, pp, pd, s, dp, L, ob1, qb1, s_lse[0], s_dl[0], c, h, 0, 0, 0);
            else
                BP::template region<true, false, false>(dv, dk, pp, pd, s, dp, L, ob2, qb2, s_lse[0], s_dl[0], c, h, 0, 0, 0);
        }
        __syncthreads();   // every wave is done with the tile buffers
    }

    if constexpr (MODE == BWD_BAND_GL) {
        // set S3: per query head, the gathered tile of the global rows; a
        // global row counts here for the keys outside its own band
        for (int hq = 0; hq < (ng > 0 ? prm.group : 0); ++hq) {
            const long long bh = (long long)b * prm.H + kvh * prm.group + hq;
            const uint16_t *qh = static_cast<const uint16_t *>(prm.q) + bh * prm.head_stride;
            const uint16_t *gh = static_cast<const uint16_t *>(prm.dout) + bh * prm.head_stride;
            const TileSrc src{0, 1, N, ng, s_g};
            P::issue_one(L, qh, qb0, src, s_g[0]);
            P::issue_one(L, gh, ob0, src, s_g[0]);
            if (tid < BQ) {
                const bool gv = tid < ng;
                s_lse[0][tid] = gv ? prm.lse2[bh * N + s_g[tid]] : 0.f;
                s_dl[0][tid] = gv ? prm.delta[bh * N + s_g[tid]] : 0.f;
            }
            wait_vmem();
            __syncthreads();
            if (wave_active)
                tile_products(qb0, ob0, 0, TILE_EDGE, [&](int r) { return r < ng ? s_g[r] : -1; },
                              [&](int i) {   // row i's band holds the key iff qlo <= i <= qhi
                                  return kvalid & (i >= 0) & ((prm.causal == 0) | (key <= i)) &
                                         ((i < qlo) | (i > qhi));
                              });
            __syncthreads();
        }
    }

    if constexpr (XT) {
        // extra query tiles of the strided / random-block rules: a pair
        // counts outside the key's band, off the global rows and columns
        // (their pairs are in S2 and S3) and within the causal limit
        bool key_is_g = false;
        for (int t = 0; t < ng; ++t) key_is_g |= s_g[t] == key;
        auto extra_qtile = [&](int q0, auto vis) __attribute__((always_inline)) {
            for (int hq = 0; hq < prm.group; ++hq) {
                const long long bh = (long long)b * prm.H + kvh * prm.group + hq;
                const uint16_t *qh = static_cast<const uint16_t *>(prm.q) + bh * prm.head_stride;
                const uint16_t *gh = static_cast<const uint16_t *>(prm.dout) + bh * prm.head_stride;
                P::issue_k(L, qh, N, qb0, q0);
                P::issue_k(L, gh, N, ob0, q0);
                if (tid < BQ) {
                    const int i = q0 + tid;
                    s_lse[0][tid] = i < N ? prm.lse2[bh * N + i] : 0.f;
                    s_dl[0][tid] = i < N ? prm.delta[bh * N + i] : 0.f;
                }
                wait_vmem();
                __syncthreads();
                if (wave_active) {
                    const unsigned long long gm = global_rows_in(s_g, ng, q0);
                    tile_products(qb0, ob0, 0, TILE_EDGE, [&](int r) { return q0 + r; }, [&](int i) {
                        return kvalid & !key_is_g & (i < N) & ((i < qlo) | (i > qhi)) &
                               ((prm.causal == 0) | (i >= key)) & !((gm >> (i - q0)) & 1ull) && vis(i);
                    });
                }
                __syncthreads();
            }
        };
        const int K1 = imin(N - 1, K0 + BK - 1);
        if (prm.stride > 0) {
            // rows at distance o = stride * 2^m from the keys: [K0 - o, K1 - o]
            // (farthest first, without the causal cut only) then
            // [K0 + o, K1 + o] (nearest first), visited once each
            const int st = prm.stride;
            int mtop = -1;
            while (mtop < 30 && ((long long)st << (mtop + 1)) < N) ++mtop;
            int next = 0;
            auto strided = [&](int i) {
                const int dist = i > key ? i - key : key - i;
                if (dist == 0 || dist % st) return false;
                const int m = dist / st;
                return (m & (m - 1)) == 0;
            };
            auto visit = [&](int rlo, int rhi) __attribute__((always_inline)) {
                rlo = imax(rlo, 0);
                rhi = imin(rhi, N - 1);
                if (rlo > rhi) return;
                const int t1 = rhi / BQ;
                for (int t = imax(rlo / BQ, next); t <= t1; ++t) extra_qtile(t * BQ, strided);
                next = imax(next, t1 + 1);
            };
            if (!prm.causal)
                for (int m = mtop; m >= 0; --m) visit(K0 - (st << m), K1 - (st << m));
            for (int m = 0; m <= mtop; ++m) visit(K0 + (st << m), K1 + (st << m));
        }
        if (prm.rand_block > 0) {
            // the query blocks whose lists name a key block of this
            // workgroup (out-of-range entries skipped, repeats once). The
            // lists are scanned a workgroup-width of entries at a time, one
            // entry per thread, and the hits compacted in list order through
            // LDS (a serial scan of every list by one wave waited on each
            // load in turn)
            const int rb = prm.rand_block, nr = prm.n_rand, nb = (N + rb - 1) / rb;
            const int total = nb * nr;
            for (int base = 0; base < total; base += kBwdThreads) {
                const int idx = base + tid;
                bool hit = false;
                if (idx < total) {
                    const int qb = idx / nr, e = idx - qb * nr;
                    const int *lst = prm.rand_idx + (long long)qb * nr;
                    const int kb = lst[e];
                    hit = kb >= 0 && kb < nb && kb * rb <= K1 && kb * rb + rb - 1 >= K0;
                    for (int e2 = 0; e2 < e && hit; ++e2) hit = lst[e2] != kb;
                    if (prm.causal && imin(N - 1, qb * rb + rb - 1) < kb * rb) hit = false;
                }
                const unsigned long long bal = __ballot(hit);
                if (lane == 0) s_nhit[wave] = __popcll(bal);
                __syncthreads();
                int off = 0, nhit = 0;
                for (int w2 = 0; w2 < P::NW; ++w2) {
                    off += w2 < wave ? s_nhit[w2] : 0;
                    nhit += s_nhit[w2];
                }
                if (hit) s_hit[off + __popcll(bal & ((1ull << lane) - 1ull))] = idx;
                __syncthreads();
                for (int x = 0; x < nhit; ++x) {
                    const int idx2 = __builtin_amdgcn_readfirstlane(s_hit[x]);
                    const int qb = idx2 / nr, kb = prm.rand_idx[idx2];
                    const int rlo = qb * rb, rhi = imin(N - 1, rlo + rb - 1);
                    const int klo = kb * rb, khi = kb * rb + rb - 1;
                    for (int t = rlo / BQ; t <= rhi / BQ; ++t)
                        extra_qtile(t * BQ, [&](int i) { return i >= rlo && i <= rhi && key >= klo && key <= khi; });
                }
                __syncthreads();   // every wave has read s_hit before the next chunk
            }
        }
    }

    if (!kvalid) return;
    if constexpr (MODE == BWD_GSET) {   // fp32 partials: [B*H_kv][ng][chunks][2 D] (dK^T unscaled, dV^T)
        float *dst = prm.part_k + (((long long)bkv * ng + (wave * 32 + ln)) * prm.gchunks_k + chunk) * (2 * D);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int d = db * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
                dst[d] = dk[db][e];
                dst[D + d] = dv[db][e];
            }
        return;
    }
    uint16_t *dkh = static_cast<uint16_t *>(prm.dk) + (long long)bkv * prm.head_stride + cls_off;
    uint16_t *dvh = static_cast<uint16_t *>(prm.dv) + (long long)bkv * prm.head_stride + cls_off;
    P::store_out(dkh, key * dil, dk, prm.scale, h);
    P::store_out(dvh, key * dil, dv, 1.f, h);
}

// ---------------------------------------------------------------------------
// Software pipeline of the dQ band loop, as for dK/dV: iteration t runs
// S^T(t) and dP^T(t), then a region in which the MFMAs of
// dQ^T += K(t-1)^T dS^T(t-1) are issued in batches of four, each followed by
// the vector work of a share of tile t's elements (the row's LSE and row
// term are per lane here).
// ---------------------------------------------------------------------------
template <class P>
struct DqPipe {
    static constexpr int MB = P::MB, DB = P::DB, PVS = P::PVS;
    static constexpr int kB = 4, kSlots = 8;
    static constexpr int NM = PVS * DB;           // MFMAs (16 at d=128, 8 at d=64)
    static constexpr int NB = NM / kB;            // batches
    static constexpr int EPB = 16 * MB / NB;      // elements per batch
    static_assert(EPB * NB == 16 * MB, "whole element shares per batch");

    template <int I>
    static __device__ __forceinline__ void fetch(bf16x8 (&op)[kSlots], const typename P::Lane &L, const char *kv) {
        if constexpr (I < NM) op[I % kSlots] = P::v_operand(L, kv, I % DB, I / DB);
    }

    template <bool MM, bool VA, bool EDGE, int B>
    static __device__ __forceinline__ void run(f32x16 (&dq)[DB], const typename P::PFrag &pd, f32x16 (&s)[MB],
                                               f32x16 (&dp)[MB], const typename P::Lane &L, const char *kv,
                                               bf16x8 (&op)[kSlots], float c, float l2, float dl, int h, int k0,
                                               int lo, int hi) {
        if constexpr (B < NB) {
            if constexpr (MM && B + 1 < NB) {
                fetch<kB * (B + 1) + 0>(op, L, kv);
                fetch<kB * (B + 1) + 1>(op, L, kv);
                fetch<kB * (B + 1) + 2>(op, L, kv);
                fetch<kB * (B + 1) + 3>(op, L, kv);
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (MM) {
#pragma unroll
                for (int u = 0; u < kB; ++u) {
                    const int I = kB * B + u, st = I / DB, db = I % DB;
                    dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[I % kSlots], pd.x[st], dq[db], 0, 0, 0);
                }
            }
            if constexpr (VA) {
#pragma unroll
                for (int e = B * EPB; e < (B + 1) * EPB; ++e) {
                    const int mb = e / 16, r = e % 16;
                    float p = fast_exp2(__builtin_fmaf(s[mb][r], c, -l2));
                    if constexpr (EDGE) {
                        const int j = k0 + mb * 32 + acc_row(r, h);
                        p = ((j >= lo) & (j <= hi)) ? p : 0.f;
                    }
                    dp[mb][r] = p * (dp[mb][r] - dl);
                }
            }
            if constexpr (MM && VA) {
                constexpr int NV = EPB * (EDGE ? 7 : 4) / kB;
#pragma unroll
                for (int u = 0; u < kB; ++u) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x402, NV, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            run<MM, VA, EDGE, B + 1>(dq, pd, s, dp, L, kv, op, c, l2, dl, h, k0, lo, hi);
        }
    }

    template <bool MM, bool VA, bool EDGE>
    static __device__ __forceinline__ void region(f32x16 (&dq)[DB], const typename P::PFrag &pd, f32x16 (&s)[MB],
                                                  f32x16 (&dp)[MB], const typename P::Lane &L, const char *kv, float c,
                                                  float l2, float dl, int h, int k0, int lo, int hi) {
        bf16x8 op[kSlots];
        if constexpr (MM) {
            fetch<0>(op, L, kv);
            fetch<1>(op, L, kv);
            fetch<2>(op, L, kv);
            fetch<3>(op, L, kv);
            __builtin_amdgcn_sched_barrier(0);
        }
        run<MM, VA, EDGE, 0>(dq, pd, s, dp, L, kv, op, c, l2, dl, h, k0, lo, hi);
    }
};

// ---------------------------------------------------------------------------
// dQ: query rows stationary, key tiles streamed.
// BWD_BAND / BWD_BAND_GL: one workgroup per (query head, [residue class,]
//   query tile); BWD_BAND_GL adds the gathered tile of global columns (set S2).
// BWD_GSET: the global rows as the query rows (one workgroup per (query head,
//   chunk of key tiles)), keys of set S3, fp32 partials out.
// ---------------------------------------------------------------------------
// XT (with BWD_BAND_GL): the keys this workgroup's rows see by the
// log-spaced strided or the random-block rule, as extra key tiles.
template <int D, bool DIL, int MODE, bool XT = false>
__global__ void __launch_bounds__((dq_threads<D, MODE, XT>()), dq_waves<D>()) bwd_dq(const BwdParams prm) {
    // K tiles are read both ways (row reads for S^T, transpose reads for
    // dQ): the unified LDS layout serves both from one copy.
    typedef Bf16Path<D, dq_threads<D, MODE, XT>(), true> P;
    constexpr int BN = P::BN;                 // keys per streamed tile
    constexpr int BM = 32 * P::NW;            // query rows per workgroup
    constexpr int MB = P::MB, DB = P::DB;
    static_assert(!(DIL && MODE != BWD_BAND), "dilation is not combined with global tokens");
    // the software-pipelined band loop (below) reads a K tile's rows in one
    // iteration and its transposed operands in the next: three buffer sets
    constexpr bool PIPE = !(MODE == BWD_GSET || XT || dq_threads<D, MODE, XT>() == 512);

    // K and V of one key tile, one copy each; two sets (three for the
    // pipelined loop), distinct objects, the loops unrolled to match
    __shared__ __attribute__((aligned(1024))) char kb0[P::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char vb0[P::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char kb1[P::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char vb1[P::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char kb2[PIPE ? P::TILE_BYTES : 16];
    __shared__ __attribute__((aligned(1024))) char vb2[PIPE ? P::TILE_BYTES : 16];
    __shared__ int s_g[kMaxGlobal];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: the row bounds stay scalar
    const int ln = lane & 31, h = lane >> 5;
    const int ng = MODE == BWD_BAND ? 0 : prm.n_global;
    if constexpr (MODE != BWD_BAND) {
        if (tid < kMaxGlobal) s_g[tid] = tid < ng ? prm.gidx[tid] : -1;
        __syncthreads();
    }

    // work item
    const int G = gridDim.x, bid = blockIdx.x;
    const int Lw = prm.xcd_remap_q ? (bid & 7) * (G >> 3) + (bid >> 3) : bid;
    const int dil = DIL ? prm.dil : 1;
    int bh, rcls = 0, unit = 0, chunk = 0;
    if constexpr (MODE == BWD_GSET) {
        bh = Lw / prm.gchunks_q;
        chunk = Lw - bh * prm.gchunks_q;
    } else {
        const int per_head = dil * prm.num_qt;
        bh = Lw / per_head;
        rcls = (Lw - bh * per_head) / prm.num_qt;
        const int qi = Lw - bh * per_head - rcls * prm.num_qt;
        unit = prm.causal ? prm.num_qt - 1 - qi : qi;
    }
    const int N = DIL ? (prm.N - rcls + dil - 1) / dil : prm.N;   // rows of this residue class
    if (MODE != BWD_GSET && unit * BM >= N) return;                // whole workgroup: a shorter class
    const Band band{N, prm.wl, prm.wr, prm.block, prm.cap};
    const long long cls_off = (long long)rcls * D;
    const long long kvb = (long long)(bh / prm.H) * (prm.H / prm.group) + (bh % prm.H) / prm.group;
    const uint16_t *qh = static_cast<const uint16_t *>(prm.q) + (long long)bh * prm.head_stride + cls_off;
    const uint16_t *gh = static_cast<const uint16_t *>(prm.dout) + (long long)bh * prm.head_stride + cls_off;
    const uint16_t *kh = static_cast<const uint16_t *>(prm.k) + kvb * prm.head_stride + cls_off;
    const uint16_t *vh = static_cast<const uint16_t *>(prm.v) + kvb * prm.head_stride + cls_off;

    typename P::Lane L;
    P::init_lane(L, lane, wave, dil);

    // this lane's row: a band row, or (BWD_GSET) a global row
    const int q0 = unit * BM;
    int row, wr0, wr1, kt_lo, kt_hi;
    bool valid, wave_active;
    if constexpr (MODE == BWD_GSET) {
        const int r = wave * 32 + ln;
        valid = r < ng;
        row = valid ? s_g[r] : 0;
        wave_active = wave * 32 < ng;
        wr0 = 0;
        wr1 = N - 1;
        const int ntot = (N + BN - 1) / BN;
        kt_lo = chunk * prm.gct_q;
        kt_hi = imin(ntot, kt_lo + prm.gct_q) - 1;
    } else {
        row = q0 + wave * 32 + ln;
        valid = row < N;
        wr0 = q0 + wave * 32;
        wr1 = imin(N - 1, wr0 + 31);
        wave_active = wr0 < N;
        key_tile_range(band, q0, imin(N - 1, q0 + BM - 1), BN, &kt_lo, &kt_hi);
    }
    const int lo = row_lo(band, row), hi = row_hi(band, row);

    typename P::QFrag qf, gf;   // this wave's Q and dO rows: B operands of S^T and dP^T
    P::load_q(qf, qh, row * dil, valid, h);
    P::load_q(gf, gh, row * dil, valid, h);
    const long long grow = (long long)bh * prm.N + rcls + (long long)row * dil;   // row in the stored sequence
    const float l2 = valid ? prm.lse2[grow] : 0.f;
    const float dl = valid ? prm.delta[grow] : 0.f;
    const float c = prm.scale_log2;

    f32x16 dq[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) dq[db] = f32x16{};

    // dS^T of one staged key tile into dQ^T; col(r) gives the key of tile
    // slot r (or -1), vis(j) the extra test of an edge tile
    auto tile_products = [&](const char *kb, const char *vb, int cl, auto col, auto vis)
        __attribute__((always_inline)) {
        f32x16 s[MB], dp[MB];
        P::scores(s, qf, L, kb);    // S^T  = K Q^T  : lane = query row, registers = keys
        P::scores(dp, gf, L, vb);   // dP^T = V dO^T
        // (the edge mask a pass of its own under a uniform branch, as in bwd_dkdv)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[mb][r] = fast_exp2(__builtin_fmaf(s[mb][r], c, -l2));
        if (cl == TILE_EDGE) {
            asm volatile("");   // keeps this a branch (no speculation into selects)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[mb][r] = vis(col(mb * 32 + acc_row(r, h))) ? s[mb][r] : 0.f;
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) dp[mb][r] = s[mb][r] * (dp[mb][r] - dl);
        typename P::PFrag pd;
        P::pack_p(pd, dp);
        P::pv(dq, pd, L, kb);       // dQ^T += K^T dS^T
    };

    auto issue = [&](int kt, char *kb, char *vb) __attribute__((always_inline)) {
        P::issue_k(L, kh, N, kb, kt * BN, dil);
        P::issue_k(L, vh, N, vb, kt * BN, dil);
    };
    auto step = [&](int kt, const char *kb, const char *vb, char *nkb, char *nvb) __attribute__((always_inline)) {
        debug_sync();
        if (kt < kt_hi) issue(kt + 1, nkb, nvb);
        debug_sync();
        const int k0 = kt * BN;
        if constexpr (MODE == BWD_GSET) {
            // set S3: keys outside the global row's band, causal cut
            if (wave_active)
                tile_products(kb, vb, TILE_EDGE, [&](int r) { return k0 + r; }, [&](int j) {
                    return valid & (j < N) & ((j < lo) | (j > hi)) & ((prm.causal == 0) | (j <= row));
                });
        } else {
            const int cl = wave_active ? classify(band, wr0, wr1, k0, k0 + BN - 1) : TILE_SKIP;
            if (cl != TILE_SKIP)
                tile_products(kb, vb, cl, [&](int r) { return k0 + r; },
                              [&](int j) { return (j >= lo) & (j <= hi); });
        }
        wait_vmem();
        __syncthreads();
    };

    if constexpr (!PIPE) {
        if (kt_lo <= kt_hi) {
            issue(kt_lo, kb0, vb0);
            wait_vmem();
            __syncthreads();
            for (int kt = kt_lo; kt <= kt_hi; kt += 2) {
                step(kt, kb0, vb0, kb1, vb1);
                if (kt + 1 > kt_hi) break;
                step(kt + 1, kb1, vb1, kb0, vb0);
            }
        }
    } else if (kt_lo <= kt_hi) {
        // band tiles, software-pipelined (DqPipe). Iteration t copies tile
        // t+1, reads tile t's K and V rows (S^T, dP^T) and tile t-1's K
        // transposed (dQ of tile t-1): three buffer sets in rotation, the
        // loop unrolled by three so every buffer is a named object.
        typedef DqPipe<P> QP;
        typename P::PFrag pd;   // dS of the previous active tile
        bool act_prev = false;
        auto pstep = [&](int kt, const char *kb, const char *vb, char *nkb, char *nvb, const char *kb_p)
            __attribute__((always_inline)) {
            debug_sync();
            if (kt < kt_hi) issue(kt + 1, nkb, nvb);
            debug_sync();
            const int k0 = kt * BN;
            const int cl = wave_active ? classify(band, wr0, wr1, k0, k0 + BN - 1) : TILE_SKIP;
            const bool act = cl != TILE_SKIP;
            f32x16 s[MB], dp[MB];
            // S^T = K Q^T and dP^T = V dO^T (lane = query row, registers = keys)
            if (act) ScorePair<P>::scores(s, dp, qf, gf, L, kb, vb);
            if (act_prev) {
                if (act) {
                    if (cl == TILE_EDGE) QP::template region<true, true, true>(dq, pd, s, dp, L, kb_p, c, l2, dl, h, k0, lo, hi);
                    else QP::template region<true, true, false>(dq, pd, s, dp, L, kb_p, c, l2, dl, h, k0, lo, hi);
                } else {
                    QP::template region<true, false, false>(dq, pd, s, dp, L, kb_p, c, l2, dl, h, k0, lo, hi);
                }
            } else if (act) {
                if (cl == TILE_EDGE) QP::template region<false, true, true>(dq, pd, s, dp, L, kb_p, c, l2, dl, h, k0, lo, hi);
                else QP::template region<false, true, false>(dq, pd, s, dp, L, kb_p, c, l2, dl, h, k0, lo, hi);
            }
            if (act) P::pack_p(pd, dp);
            act_prev = act;
            wait_vmem();
            __syncthreads();
        };
        issue(kt_lo, kb0, vb0);
        wait_vmem();
        __syncthreads();
        // tile kt_lo + x sits in set x % 3
        for (int kt = kt_lo; kt <= kt_hi; kt += 3) {
            pstep(kt, kb0, vb0, kb1, vb1, kb2);
            if (kt + 1 > kt_hi) break;
            pstep(kt + 1, kb1, vb1, kb2, vb2, kb0);
            if (kt + 2 > kt_hi) break;
            pstep(kt + 2, kb2, vb2, kb0, vb0, kb1);
        }
        if (act_prev) {   // the last active tile's dQ products
            f32x16 s[MB], dp[MB];
            const int r = (kt_hi - kt_lo) % 3;
            if (r == 0) QP::template region<true, false, false>(dq, pd, s, dp, L, kb0, c, l2, dl, h, 0, 0, 0);
            else if (r == 1) QP::template region<true, false, false>(dq, pd, s, dp, L, kb1, c, l2, dl, h, 0, 0, 0);
            else QP::template region<true, false, false>(dq, pd, s, dp, L, kb2, c, l2, dl, h, 0, 0, 0);
        }
        __syncthreads();   // every wave is done with the tile buffers
    }

    bool row_is_g = false;
    if constexpr (MODE == BWD_BAND_GL)
        for (int t = 0; t < ng; ++t) row_is_g |= s_g[t] == row;
    if (MODE == BWD_BAND_GL && ng > 0) {
        // set S2: the gathered tile of the global columns; a global column
        // counts here for non-global rows outside whose band it lies
        const TileSrc src{0, 1, N, ng, s_g};
        P::issue_one(L, kh, kb0, src, s_g[0]);
        P::issue_one(L, vh, vb0, src, s_g[0]);
        wait_vmem();
        __syncthreads();
        if (wave_active)
            tile_products(kb0, vb0, TILE_EDGE, [&](int r) { return r < ng ? s_g[r] : -1; }, [&](int j) {
                return valid & !row_is_g & (j >= 0) & ((prm.causal == 0) | (j <= row)) & ((j < lo) | (j > hi));
            });
        __syncthreads();
    }

    if constexpr (XT) {
        // extra key tiles of the strided / random-block rules (as in the
        // forward): a pair counts outside the row's band, off the global rows
        // and columns and within the causal limit
        const int q1 = imin(N - 1, q0 + BM - 1);
        auto extra_ktile = [&](int k0, bool take, auto vis) __attribute__((always_inline)) {
            P::issue_k(L, kh, N, kb0, k0);
            P::issue_k(L, vh, N, vb0, k0);
            wait_vmem();
            __syncthreads();
            if (take) {
                const unsigned long long gm = global_rows_in(s_g, ng, k0);   // global columns of the tile
                tile_products(kb0, vb0, TILE_EDGE, [&](int r) { return k0 + r; }, [&](int j) {
                    return valid & !row_is_g & (j < N) & ((j < lo) | (j > hi)) & ((prm.causal == 0) | (j <= row)) &
                           !((gm >> (j - k0)) & 1ull) && vis(j);
                });
            }
            __syncthreads();
        };
        if (prm.stride > 0) {
            // a row's keys at distance s * 2^m, one pair at a time on the
            // vector ALU (as in the forward): S and dP by dot products of the
            // lane's halves, dS, then dQ^T += dS K_j
            const int st = prm.stride;
            int mtop = -1;
            while (mtop < 30 && ((long long)st << (mtop + 1)) < N) ++mtop;
            for (int side = 0; side < (prm.causal ? 1 : 2); ++side)
                for (int m = 0; m <= mtop; ++m) {
                    const int o = st << m;
                    const int j = side ? row + o : row - o;
                    bool ok = valid & !row_is_g & (j >= 0) & (j < N) & ((j < lo) | (j > hi));
                    for (int t = 0; t < ng; ++t) ok &= s_g[t] != j;   // pairs of the gathered global tile
                    if (!__any(ok)) continue;
                    const int jj = ok ? j : 0;   // a row that exists; its result is dropped
                    const uint16_t *kr = kh + (long long)jj * D, *vr = vh + (long long)jj * D;
                    const float sc = sum_across_halves(dot_row_half(kr, qf.x, h));
                    const float dpv = sum_across_halves(dot_row_half(vr, gf.x, h));
                    const float p = ok ? fast_exp2(__builtin_fmaf(sc, c, -l2)) : 0.f;
                    axpy_row_half(dq, p * (dpv - dl), kr, h);
                }
        }
        if (prm.rand_block > 0) {
            const int rb = prm.rand_block, nr = prm.n_rand, nkb = (N + rb - 1) / rb;
            const int my_qb = wr0 / rb;
            for (int qb = q0 / rb; qb <= q1 / rb; ++qb) {
                const int *lst = prm.rand_idx + (long long)qb * nr;
                for (int e = 0; e < nr; ++e) {
                    const int kb = lst[e];
                    bool skip = kb < 0 || kb >= nkb;
                    for (int e2 = 0; e2 < e && !skip; ++e2) skip = lst[e2] == kb;
                    if (skip) continue;
                    const int klo = kb * rb, khi = imin(N - 1, klo + rb - 1);
                    if (prm.causal && klo > imin(q1, qb * rb + rb - 1)) continue;
                    for (int t = klo / BN; t <= khi / BN; ++t)
                        extra_ktile(t * BN, wave_active && my_qb == qb, [&](int j) { return j >= klo && j <= khi; });
                }
            }
        }
    }

    if constexpr (MODE == BWD_BAND) {
        // the row again, from the lane id and the wave-uniform wave index:
        // keeping row and valid live across the tile loop costs registers
        // the eight-wave instance does not have
        const int lane2 = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
        const int row2 = q0 + wave * 32 + (lane2 & 31);
        if (row2 >= N) return;
        uint16_t *dqh = static_cast<uint16_t *>(prm.dq) + (long long)bh * prm.head_stride + cls_off;
        P::store_out(dqh, row2 * dil, dq, prm.scale, lane2 >> 5);
        return;
    }
    if (!valid) return;
    if constexpr (MODE == BWD_GSET) {   // fp32 partials: [B*H][ng][chunks][D] (dQ^T unscaled)
        float *dst = prm.part_q + (((long long)bh * ng + (wave * 32 + ln)) * prm.gchunks_q + chunk) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) dst[db * 32 + 8 * (e >> 2) + 4 * h + (e & 3)] = dq[db][e];
        return;
    }
    uint16_t *dqh = static_cast<uint16_t *>(prm.dq) + (long long)bh * prm.head_stride + cls_off;
    P::store_out(dqh, row * dil, dq, prm.scale, h);
}

// Add the split passes' partials to the band kernels' outputs for the global
// rows (dQ) and global columns (dK, dV): one workgroup of 64 lanes per row.
template <int D>
__global__ void __launch_bounds__(64) bwd_merge_dq(const BwdParams prm) {
    const int ng = prm.n_global;
    const long long bh = blockIdx.x / ng;
    const int r = blockIdx.x - (int)(bh * ng);
    const float *src = prm.part_q + ((long long)bh * ng + r) * prm.gchunks_q * D;
    __bf16 *dst = static_cast<__bf16 *>(prm.dq) + bh * prm.head_stride + (long long)prm.gidx[r] * D;
    for (int d = threadIdx.x; d < D; d += 64) {
        float acc = 0.f;
#pragma unroll 8
        for (int ci = 0; ci < prm.gchunks_q; ++ci) acc += src[ci * D + d];
        dst[d] = (__bf16)((float)dst[d] + acc * prm.scale);
    }
}

template <int D>
__global__ void __launch_bounds__(64) bwd_merge_dkdv(const BwdParams prm) {
    const int ng = prm.n_global;
    const long long bkv = blockIdx.x / ng;
    const int r = blockIdx.x - (int)(bkv * ng);
    const float *src = prm.part_k + ((long long)bkv * ng + r) * prm.gchunks_k * (2 * D);
    __bf16 *dk = static_cast<__bf16 *>(prm.dk) + bkv * prm.head_stride + (long long)prm.gidx[r] * D;
    __bf16 *dv = static_cast<__bf16 *>(prm.dv) + bkv * prm.head_stride + (long long)prm.gidx[r] * D;
    for (int d = threadIdx.x; d < D; d += 64) {
        float ak = 0.f, av = 0.f;
#pragma unroll 8
        for (int ci = 0; ci < prm.gchunks_k; ++ci) {
            ak += src[ci * 2 * D + d];
            av += src[ci * 2 * D + D + d];
        }
        dk[d] = (__bf16)((float)dk[d] + ak * prm.scale);
        dv[d] = (__bf16)((float)dv[d] + av);
    }
}

template <int D>
static hipError_t launch_bwd_impl(const BwdParams &p0, hipStream_t stream) {
    BwdParams p = p0;
    const long long rows = (long long)p.BH * p.N;
    hipLaunchKernelGGL((bwd_delta<D>), dim3((unsigned)((rows + 31) / 32)), dim3(kBwdThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int BKV = p.BH / p.group;
    const int kgrid = BKV * p.dil * p.num_kt;
    p.xcd_remap_k = kgrid % 8 == 0;
    if (p.stride > 0 || p.rand_block > 0)
        hipLaunchKernelGGL((bwd_dkdv<D, false, BWD_BAND_GL, true>), dim3(kgrid), dim3(kBwdThreads), 0, stream, p);
    else if (p.n_global > 0)
        hipLaunchKernelGGL((bwd_dkdv<D, false, BWD_BAND_GL>), dim3(kgrid), dim3(kBwdThreads), 0, stream, p);
    else if (p.dil > 1)
        hipLaunchKernelGGL((bwd_dkdv<D, true, BWD_BAND>), dim3(kgrid), dim3(kBwdThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((bwd_dkdv<D, false, BWD_BAND>), dim3(kgrid), dim3(kBwdThreads), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int qgrid = p.BH * p.dil * p.num_qt;
    p.xcd_remap_q = qgrid % 8 == 0;
    if (p.stride > 0 || p.rand_block > 0)
        hipLaunchKernelGGL((bwd_dq<D, false, BWD_BAND_GL, true>), dim3(qgrid), dim3(kBwdThreads), 0, stream, p);
    else if (p.n_global > 0)
        hipLaunchKernelGGL((bwd_dq<D, false, BWD_BAND_GL>), dim3(qgrid), dim3(kBwdThreads), 0, stream, p);
    else if (p.dil > 1)
        hipLaunchKernelGGL((bwd_dq<D, true, BWD_BAND>), dim3(qgrid), dim3(dq_threads<D, BWD_BAND, false>()), 0, stream, p);
    else
        hipLaunchKernelGGL((bwd_dq<D, false, BWD_BAND>), dim3(qgrid), dim3(dq_threads<D, BWD_BAND, false>()), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess || p.n_global == 0) return e;
    // split passes over the global rows and columns, then their merges
    const int g1 = p.BH * p.gchunks_q;
    p.xcd_remap_q = g1 % 8 == 0;
    hipLaunchKernelGGL((bwd_dq<D, false, BWD_GSET>), dim3(g1), dim3(kBwdThreads), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int g2 = BKV * p.gchunks_k;
    p.xcd_remap_k = g2 % 8 == 0;
    hipLaunchKernelGGL((bwd_dkdv<D, false, BWD_GSET>), dim3(g2), dim3(kBwdThreads), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_merge_dq<D>), dim3(p.BH * p.n_global), dim3(64), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_merge_dkdv<D>), dim3(BKV * p.n_global), dim3(64), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_backward(const BwdParams &p, int d, hipStream_t stream) {
    return d == 64 ? launch_bwd_impl<64>(p, stream) : launch_bwd_impl<128>(p, stream);
}

}  // namespace eea
