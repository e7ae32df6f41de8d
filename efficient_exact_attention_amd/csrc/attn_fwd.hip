// attn_fwd.hip - gfx950 (CDNA4) kernels for exact masked attention forward.
//
// Method: exact softmax(Q K^T / sqrt(d)) V computed tile by tile with an
// online softmax (running row max and normaliser), so the N x N score matrix
// never reaches HBM ("Efficient Transformers: Sparse Attention, Linear
// Attention and FlashAttention", "Family 3" and "The online softmax trick";
// week-17 lecture notes on efficient attention, FlashAttention tiling and
// online-softmax passages). Tiles whose every pair is masked are never
// visited ("Sparse & sub-quadratic attention", "Escape 1": only the lit cells
// are paid for, and block patterns map onto tiles).
//
// Layout of the work on gfx950 (our design, not the pages'):
//  * bf16: one workgroup = 8 wave64s = 256 query rows (two waves per SIMD, so
//    one wave's softmax arithmetic overlaps the other's matrix-core work);
//    each wave owns 32 rows.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: K rows are the A operand (from LDS), the
//    wave's 32 queries are the B operand (kept in registers for the whole
//    kernel). In the 32x32 accumulator layout a lane then holds ONE query and
//    16 keys, so the row max and row sum are in-lane reductions plus a single
//    exchange between the two half-waves (v_permlane32_swap).
//  * The output is accumulated transposed, O^T += V^T P^T, so the fp32
//    accumulators of a lane also belong to its one query: the online-softmax
//    rescale is a per-lane scalar multiply. The exponentiated scores, rounded
//    to bf16, are already in the B-operand layout of this product.
//  * K and V tiles go straight from HBM into LDS (global_load_lds_dwordx4,
//    no register staging), double-buffered, one barrier per tile. Each lane
//    fetches the 16-byte chunk that lands at its LDS slot, so the XOR
//    swizzle of chunks within a row is applied on the global side. K is read
//    with ds_read_b128; V^T operands are produced by the LDS transpose read
//    ds_read_b64_tr_b16 straight from row-major V.
//  * Softmax runs in the exp2 domain with scale*log2(e) folded into one FMA.
//    The running max is only moved (and the accumulators rescaled) when it
//    grows by more than 2^8; otherwise the stale max keeps every weight below
//    256, which is exact once divided by the same running normaliser.
//  * Work items are ordered heaviest-first for causal masks, and consecutive
//    work items are grouped onto one XCD so the workgroups that share a
//    head's K/V stream share that XCD's L2.
//  * fp32 inputs use v_mfma_f32_32x32x2_f32 with the same transposed scheme
//    and register-staged tile loads.
//
// Global tokens: global COLUMNS are gathered into extra key tiles per query
// tile (masked where the column already lies in the row's window); global
// ROWS see every key, so they are computed by a split-key pass that writes
// partial (o, m, l) per key chunk and a merge kernel that combines them with
// the same rescaling identity the online softmax uses.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <vector>

#include "attn_internal.h"
#include "attn_plan.h"
#include "attn_tiles.h"

namespace eea {

// ---------------------------------------------------------------------------
// fp32 inputs: both products on v_mfma_f32_32x32x2_f32 (true fp32 products).
// The contraction index of QK^T is split between half-waves as d = h*D/2 + s.
// Tiles are staged through registers (global loads issued before the
// current tile's work, written to LDS after it).
// ---------------------------------------------------------------------------
template <int D_, int NT_>
struct F32Path {
    static constexpr int D = D_, BN = 32, NT = NT_;
    static constexpr bool F32 = true;
    static constexpr int KS = D / 2;
    static constexpr int MB = BN / 32;
    static constexpr int DB = D / 32;
    static constexpr int ROW = D * 4;
    static constexpr int CH = D / 4;          // 16-byte chunks per row
    static constexpr int TILE_BYTES = BN * D * 4;
    static constexpr int CHUNKS = BN * CH;
    static constexpr int PER_T = (CHUNKS + NT - 1) / NT;
    static constexpr int LDS_BYTES = 4 * TILE_BYTES;

    typedef float elem_t;
    struct QFrag { float x[KS]; };
    struct Stage { u32x4 k[PER_T]; u32x4 v[PER_T]; };
    struct PFrag { float x[MB][16]; };
    struct Lane { int ln, h, tid; };

    static __device__ __forceinline__ void init_lane(Lane &L, int lane, int wave) {
        L.ln = lane & 31;
        L.h = lane >> 5;
        L.tid = wave * 64 + lane;
    }

    static __device__ __forceinline__ int k_off(int row, int chunk) {
        return row * ROW + ((chunk ^ (row & 7)) << 4);
    }

    static __device__ __forceinline__ void load_q(QFrag &qf, const elem_t *qh, int row, bool valid, int h) {
        const f32x4 *src = reinterpret_cast<const f32x4 *>(qh + (long long)row * D + h * (D / 2));
#pragma unroll
        for (int c = 0; c < D / 8; ++c) {
            f32x4 w = valid ? src[c] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 4; ++e) qf.x[4 * c + e] = w[e];
        }
    }

    static __device__ __forceinline__ void issue(Stage &st, const Lane &L, const elem_t *kh, const elem_t *vh,
                                                 char *, char *, const TileSrc &src, int) {
#pragma unroll
        for (int i = 0; i < PER_T; ++i) {
            int c = L.tid + i * NT;
            st.k[i] = u32x4{0, 0, 0, 0};
            st.v[i] = u32x4{0, 0, 0, 0};
            if (c < CHUNKS) {
                int row = c / CH, ch = c % CH;
                int key = src.key(row);
                if (key >= 0) {
                    st.k[i] = *reinterpret_cast<const u32x4 *>(kh + (long long)key * D + ch * 4);
                    st.v[i] = *reinterpret_cast<const u32x4 *>(vh + (long long)key * D + ch * 4);
                }
            }
        }
    }

    static __device__ __forceinline__ void finish(const Stage &st, char *kbuf, char *vbuf, int tid) {
#pragma unroll
        for (int i = 0; i < PER_T; ++i) {
            int c = tid + i * NT;
            if (c < CHUNKS) {
                int row = c / CH, ch = c % CH;
                *reinterpret_cast<u32x4 *>(kbuf + k_off(row, ch)) = st.k[i];
                *reinterpret_cast<u32x4 *>(vbuf + row * ROW + ch * 16) = st.v[i];
            }
        }
    }

    static __device__ __forceinline__ void scores(f32x16 (&s)[MB], const QFrag &qf, const Lane &L,
                                                  const char *kbuf) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            f32x16 acc = {};
#pragma unroll
            for (int c = 0; c < D / 8; ++c) {
                f32x4 a = *reinterpret_cast<const f32x4 *>(kbuf + k_off(mb * 32 + L.ln, L.h * (D / 8) + c));
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], qf.x[4 * c + e], acc, 0, 0, 0);
            }
            s[mb] = acc;
        }
    }

    static __device__ __forceinline__ void pack_p(PFrag &pf, const f32x16 (&s)[MB]) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) pf.x[mb][r] = s[mb][r];
    }

    static __device__ __forceinline__ void pv(f32x16 (&o)[DB], const PFrag &pf, const Lane &L,
                                              const char *vbuf) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = mb * 32 + acc_row(r, L.h);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    float a = *reinterpret_cast<const float *>(vbuf + key * ROW + (db * 32 + L.ln) * 4);
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, pf.x[mb][r], o[db], 0, 0, 0);
                }
            }
    }

    static __device__ __forceinline__ void store_out(elem_t *oh, int row, const f32x16 (&o)[DB],
                                                     float inv, int h) {
        elem_t *dst = oh + (long long)row * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 x = {o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv,
                           o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv};
                *reinterpret_cast<f32x4 *>(dst + db * 32 + 8 * g + 4 * h) = x;
            }
    }
};

// ---------------------------------------------------------------------------
// Per-lane online-softmax state and one tile step.
// ---------------------------------------------------------------------------
template <class P>
struct RowState {
    float m;        // running max of scaled scores, log2 domain
    float lpart;    // this half-wave's share of the running normaliser
    f32x16 o[P::DB];
};


template <class P>
__device__ __forceinline__ void softmax_pv_step(RowState<P> &rs, f32x16 (&s)[P::MB], float c,
                                                const typename P::Lane &L, const char *vbuf) {
    float mx = EEA_NEG_INF;
#pragma unroll
    for (int mb = 0; mb < P::MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mb][r]);
    mx = max_across_halves(mx);
    const float mnew = fmaxf(rs.m, mx * c);
    const bool need = mnew > rs.m + kRescaleLog2;
    if (__any(need)) {
        const float alpha = (mnew == EEA_NEG_INF) ? 1.f : fast_exp2(rs.m - mnew);
        rs.m = mnew;
        rs.lpart *= alpha;
#pragma unroll
        for (int db = 0; db < P::DB; ++db) rs.o[db] *= alpha;
    }
    const float mu = (rs.m == EEA_NEG_INF) ? 0.f : rs.m;
    float sum = 0.f;
#pragma unroll
    for (int mb = 0; mb < P::MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float p = fast_exp2(__builtin_fmaf(s[mb][r], c, -mu));
            s[mb][r] = p;
            sum += p;
        }
    rs.lpart += sum;
    typename P::PFrag pf;
    P::pack_p(pf, s);
    P::pv(rs.o, pf, L, vbuf);
}

// ---------------------------------------------------------------------------
// Forward kernel. MODE_BAND: one query tile of 32*NT/64 consecutive rows.
// MODE_GROWS: the global rows (gathered) against one chunk of keys, writing
// unnormalised partials for the merge kernel.
// ---------------------------------------------------------------------------
template <class P, int MODE>
__global__ void __launch_bounds__(P::NT) fwd_kernel(const FwdParams prm) {
    constexpr int D = P::D, BN = P::BN, NT = P::NT;
    constexpr int BM = 32 * (NT / 64);
    typedef typename P::elem_t elem_t;

    // Two LDS buffers (K tile then V tile each) as distinct objects, so that
    // reads of one are never made to wait for the DMA into the other.
    __shared__ __attribute__((aligned(1024))) char smem0[P::LDS_BYTES / 2];
    __shared__ __attribute__((aligned(1024))) char smem1[P::LDS_BYTES / 2];
    __shared__ int s_gidx[kMaxGlobal];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ln = lane & 31, h = lane >> 5;
    const int N = prm.N;
    const int ng = prm.n_global;
    const Band band{N, prm.wl, prm.wr, prm.block, prm.cap};

    if (tid < kMaxGlobal) s_gidx[tid] = tid < ng ? prm.gidx[tid] : -1;

    // --- which work item
    const int G = gridDim.x;
    const int bid = blockIdx.x;
    const int Lw = prm.xcd_remap ? (bid & 7) * (G >> 3) + (bid >> 3) : bid;
    int bh, unit;
    if (MODE == MODE_BAND) {
        bh = Lw / prm.num_qt;
        const int qi = Lw - bh * prm.num_qt;
        unit = prm.causal ? prm.num_qt - 1 - qi : qi;
    } else {
        bh = Lw / prm.chunks;
        unit = Lw - bh * prm.chunks;
    }
    const elem_t *qh = static_cast<const elem_t *>(prm.q) + (long long)bh * prm.head_stride;
    const elem_t *kh = static_cast<const elem_t *>(prm.k) + kv_head(prm, bh) * prm.head_stride;
    const elem_t *vh = static_cast<const elem_t *>(prm.v) + kv_head(prm, bh) * prm.head_stride;

    typename P::Lane L;
    P::init_lane(L, lane, wave);

    __syncthreads();   // s_gidx visible

    // --- this lane's query row and its visible key interval [lo, hi]
    int row, lo, hi, kt_lo, kt_hi, wave_hi;
    bool valid, wave_active;
    int wr0 = 0, wr1 = 0;
    if (MODE == MODE_BAND) {
        const int q0 = unit * BM;
        row = q0 + wave * 32 + ln;
        valid = row < N;
        lo = row_lo(band, row);
        hi = row_hi(band, row);
        wr0 = q0 + wave * 32;
        wr1 = imin(N - 1, wr0 + 31);
        wave_active = wr0 < N;
        key_tile_range(band, q0, imin(N - 1, q0 + BM - 1), BN, &kt_lo, &kt_hi);
        wave_hi = 0;
    } else {
        const int t = wave * 32 + ln;
        valid = t < ng;
        row = valid ? s_gidx[t] : 0;
        lo = 0;
        hi = prm.causal ? row : N - 1;
        wave_active = wave * 32 < ng;
        const int num_kt = (N + BN - 1) / BN;
        kt_lo = unit * prm.chunk_tiles;
        kt_hi = imin(num_kt - 1, kt_lo + prm.chunk_tiles - 1);
        if (prm.causal) kt_hi = imin(kt_hi, s_gidx[ng - 1] / BN);
        wave_hi = wave_active ? (prm.causal ? s_gidx[imin(ng - 1, wave * 32 + 31)] : N - 1) : -1;
    }

    typename P::QFrag qf;
    P::load_q(qf, qh, row, valid, h);

    RowState<P> rs;
    rs.m = EEA_NEG_INF;
    rs.lpart = 0.f;
#pragma unroll
    for (int db = 0; db < P::DB; ++db) rs.o[db] = f32x16{};

    const float c = prm.scale_log2;
    char *const k0buf = smem0, *const v0buf = smem0 + P::TILE_BYTES;
    char *const k1buf = smem1, *const v1buf = smem1 + P::TILE_BYTES;

    // --- gathered tiles of global columns (one per BN globals)
    if (MODE == MODE_BAND && ng > 0) {
        for (int g0 = 0; g0 < ng; g0 += BN) {
            typename P::Stage st;
            const TileSrc src{g0, 1, N, ng, s_gidx};
            P::issue(st, L, kh, vh, k0buf, v0buf, src, s_gidx[0]);
            P::finish(st, k0buf, v0buf, tid);
            __syncthreads();
            if (wave_active) {
                f32x16 s[P::MB];
                P::scores(s, qf, L, k0buf);
                // branch-free mask: a global column counts here only when it is
                // outside the row's window (inside, the band tiles count it)
#pragma unroll
                for (int mb = 0; mb < P::MB; ++mb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int col = g0 + mb * 32 + acc_row(r, h);
                        const int g = s_gidx[col < kMaxGlobal ? col : 0];
                        const bool vis = (col < ng) & ((prm.causal == 0) | (g <= row)) & ((g < lo) | (g > hi));
                        s[mb][r] = vis ? s[mb][r] : EEA_NEG_INF;
                    }
                softmax_pv_step<P>(rs, s, c, L, v0buf);
            }
            __syncthreads();
        }
    }

    // --- band tiles, double-buffered; the loop is unrolled by two so that
    // each step reads one named buffer while the next tile streams into the
    // other one.
    auto step = [&](int kt, char *kr, char *vr, char *kw, char *vw) {
        const bool more = kt < kt_hi;
        typename P::Stage st;
        debug_sync();
        if (more) {
            const TileSrc src{(kt + 1) * BN, 0, N, ng, s_gidx};
            P::issue(st, L, kh, vh, kw, vw, src, N - 1);
            if constexpr (kDebugSync) P::finish(st, kw, vw, tid);
        }
        debug_sync();
        const int k0 = kt * BN;
        int kind;   // -1 skip, 0 full, 1 edge
        if (MODE == MODE_BAND) {
            const int cl = classify(band, wr0, wr1, k0, k0 + BN - 1);
            kind = (cl == TILE_SKIP || !wave_active) ? -1 : (cl == TILE_FULL ? 0 : 1);
        } else {
            kind = (!wave_active || k0 > wave_hi) ? -1 : 1;
        }
        if (kind >= 0) {
            f32x16 s[P::MB];
            P::scores(s, qf, L, kr);
            if (kind == 1) {
#pragma unroll
                for (int mb = 0; mb < P::MB; ++mb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int j = k0 + mb * 32 + acc_row(r, h);
                        s[mb][r] = ((j >= lo) & (j <= hi)) ? s[mb][r] : EEA_NEG_INF;
                    }
            }
            softmax_pv_step<P>(rs, s, c, L, vr);
        }
        if (more && !kDebugSync) P::finish(st, kw, vw, tid);
        __syncthreads();
    };
    if (kt_lo <= kt_hi) {
        {
            typename P::Stage st;
            const TileSrc src{kt_lo * BN, 0, N, ng, s_gidx};
            P::issue(st, L, kh, vh, k0buf, v0buf, src, N - 1);
            P::finish(st, k0buf, v0buf, tid);
        }
        __syncthreads();
        for (int kt = kt_lo; kt <= kt_hi; kt += 2) {
            step(kt, k0buf, v0buf, k1buf, v1buf);
            if (kt + 1 > kt_hi) break;
            step(kt + 1, k1buf, v1buf, k0buf, v0buf);
        }
    }

    // --- epilogue
    const float l = sum_across_halves(rs.lpart);
    if (MODE == MODE_BAND) {
        if (!valid) return;
        if (ng > 0) {
            for (int t = 0; t < ng; ++t)
                if (s_gidx[t] == row) return;   // global rows are written by the merge
        }
        const float inv = l > 0.f ? 1.f / l : 0.f;
        elem_t *oh = static_cast<elem_t *>(prm.out) + (long long)bh * prm.head_stride;
        P::store_out(oh, row, rs.o, inv, h);
        if (h == 0)
            prm.lse[(long long)bh * N + row] = l > 0.f ? (rs.m + __log2f(l)) * kLn2 : EEA_NEG_INF;
    } else {
        if (!valid) return;
        const int t = wave * 32 + ln;
        float *dst = prm.part + (((long long)bh * ng + t) * prm.chunks + unit) * (D + 2);
#pragma unroll
        for (int db = 0; db < P::DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float *p = dst + db * 32 + 8 * g + 4 * h;
                p[0] = rs.o[db][4 * g + 0];
                p[1] = rs.o[db][4 * g + 1];
                p[2] = rs.o[db][4 * g + 2];
                p[3] = rs.o[db][4 * g + 3];
            }
        if (h == 0) {
            dst[D] = rs.m;
            dst[D + 1] = l;
        }
    }
}

// ---------------------------------------------------------------------------
// bf16 band pass, software-pipelined inside each wave.
//
// Iteration j of the key-tile loop gives the matrix cores and the vector ALU
// of one wave independent work at the same time:
//   region A: S(j+1) = K(j+1) Q^T on the matrix cores, while the vector ALU
//             exponentiates S(j) against the running max and packs the
//             weights to bf16;
//   region B: O^T += V(j)^T P(j)^T on the matrix cores, while the vector ALU
//             adds the fp32 weights of tile j to the normaliser and masks
//             (edge tiles) and reduces the row max of S(j+1);
//   then the running max moves, and O and the normaliser are rescaled, if
//   S(j+1) raised it by more than 2^8.
// K runs one tile ahead of V: iteration j reads K(j+1) and V(j) and copies
// K(j+2) and V(j+1) into the buffers iteration j-1 finished reading.
// Within a region, sched_group_barrier lays the stream out as one MFMA
// followed by a share of the vector work, so the vector instructions issue
// while the MFMA before them is still in the matrix pipe.
// ---------------------------------------------------------------------------
// Materialise wave-uniform values in scalar registers at this point (an
// empty asm per value, no instruction of its own).
template <class T>
__device__ __forceinline__ void scalar_ready1(const T &x) {
    asm volatile("" ::"s"(x));
}
template <class... T>
__device__ __forceinline__ void scalar_ready(const T &...x) {
    (scalar_ready1(x), ...);
}

// Edge-tile mask: key k0 + mb*32 + acc_row(r, h) is visible to the lane's row
// iff it lies in [lo, hi]; the half-wave offset 4h is folded into the bounds
// (lo4 = lo - 4h, hi4 = hi - 4h), so h need not stay live in the loop.
struct EdgeMask {
    int k0, lo4, hi4;   // first key of the tile; the lane's row interval less 4h
};

template <class P>
struct BandPipe {
    static constexpr int MB = P::MB, KS = P::KS, DB = P::DB, PVS = P::PVS;
    static constexpr int NE = 16 * MB;                    // scores per lane per tile
    // MFMAs per batch and operand slots; at d = 64 batches of two, whose
    // operand slots (half as many) let the narrow instance fit 168 registers
    static constexpr int kB = P::D == 64 ? 2 : 4, kSlots = 2 * kB;
    static constexpr int BQK = KS * MB / kB, BPV = PVS * DB / kB;
    static constexpr int EA = NE / BQK, EB = NE / BPV;    // scores handled per batch
    static_assert(EA % 8 == 0 && EB % 2 == 0, "whole packed groups per batch");
    typedef typename P::QFrag QF;
    typedef typename P::PFrag PF;
    typedef typename P::Lane LN;

    template <int I>
    static __device__ __forceinline__ void k_fetch(bf16x8 (&op)[kSlots], const LN &L, const char *kbuf) {
        if constexpr (I < KS * MB) {
            constexpr int ks = I / MB, mb = I % MB;
            op[I % kSlots] = *reinterpret_cast<const bf16x8 *>(kbuf + L.krd[ks] + mb * 32 * P::ROWB);
        }
    }
    template <int I>
    static __device__ __forceinline__ void v_fetch(bf16x8 (&op)[kSlots], const LN &L, const char *vbuf) {
        if constexpr (I < PVS * DB) op[I % kSlots] = P::v_operand(L, vbuf, I % DB, I / DB);
    }
    // The kB operand reads of batch B.
    template <int B>
    static __device__ __forceinline__ void k_batch(bf16x8 (&op)[kSlots], const LN &L, const char *kbuf) {
        k_fetch<kB * B + 0>(op, L, kbuf);
        k_fetch<kB * B + 1>(op, L, kbuf);
        if constexpr (kB == 4) {
            k_fetch<kB * B + 2>(op, L, kbuf);
            k_fetch<kB * B + 3>(op, L, kbuf);
        }
    }
    template <int B>
    static __device__ __forceinline__ void v_batch(bf16x8 (&op)[kSlots], const LN &L, const char *vbuf) {
        v_fetch<kB * B + 0>(op, L, vbuf);
        v_fetch<kB * B + 1>(op, L, vbuf);
        if constexpr (kB == 4) {
            v_fetch<kB * B + 2>(op, L, vbuf);
            v_fetch<kB * B + 3>(op, L, vbuf);
        }
    }

    // Region A, batch B: the reads of batch B+1, four QK MFMAs, and the
    // exponentials of scores [B*EA, (B+1)*EA) of the previous tile.
    template <bool QK, bool EXP, int B>
    static __device__ __forceinline__ void a_run(f32x16 (&sn)[MB], f32x16 (&s)[MB], PF &pf, const QF &qf,
                                                 const LN &L, const char *kbuf, bf16x8 (&op)[kSlots], float c,
                                                 float nmu) {
        if constexpr (B < BQK) {
            if constexpr (QK && B + 1 < BQK) {
                k_batch<B + 1>(op, L, kbuf);
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (QK) {
#pragma unroll
                for (int u = 0; u < kB; ++u) {
                    const int I = kB * B + u, ks = I / MB, mb = I % MB;
                    sn[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[I % kSlots], qf.x[ks], sn[mb], 0, 0, 0);
                }
            }
            if constexpr (EXP) {
                // The scaling FMAs stay beside this region's MFMAs: the scores
                // are redefined here (an empty asm, no instruction); both
                // region A variants exponentiate the same scores, and the
                // compiler would otherwise compute all of them ahead of the
                // branch between the variants, in one block with no MFMA.
                if constexpr ((B * EA) % 16 == 0) asm volatile("" : "+v"(s[(B * EA) / 16]));
#pragma unroll
                for (int e = B * EA; e < (B + 1) * EA; ++e)
                    s[e / 16][e % 16] = fast_exp2(__builtin_fmaf(s[e / 16][e % 16], c, nmu));
#pragma unroll
                for (int st = B * EA / 8; st < (B + 1) * EA / 8; ++st) {
                    const int mb = st >> 1, r0 = 8 * (st & 1);
                    f32x8 x = {s[mb][r0 + 0], s[mb][r0 + 1], s[mb][r0 + 2], s[mb][r0 + 3],
                               s[mb][r0 + 4], s[mb][r0 + 5], s[mb][r0 + 6], s[mb][r0 + 7]};
                    pf.x[st] = __builtin_convertvector(x, bf16x8);
                }
            }
            if constexpr (QK && EXP) {
                constexpr int NV = (5 * EA / 2) / kB;   // fma + exp per score, one cvt per two
#pragma unroll
                for (int u = 0; u < kB; ++u) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x402, NV, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            a_run<QK, EXP, B + 1>(sn, s, pf, qf, L, kbuf, op, c, nmu);
        }
    }
    template <bool QK, bool EXP>
    static __device__ __forceinline__ void region_a(f32x16 (&sn)[MB], f32x16 (&s)[MB], PF &pf, const QF &qf,
                                                    const LN &L, const char *kbuf, float c, float nmu) {
        bf16x8 op[kSlots];
        if constexpr (QK) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) sn[mb] = f32x16{};
            k_batch<0>(op, L, kbuf);
            __builtin_amdgcn_sched_barrier(0);
        }
        // Raised wave priority while the QK^T MFMAs are issued: with the
        // other wave of the SIMD in the same region, the arbiter then favours
        // the wave that feeds the matrix pipe (measured +1.7 % on the causal
        // N=32768 workload; raising it in region B instead gave nothing).
        if constexpr (QK) __builtin_amdgcn_s_setprio(1);
        a_run<QK, EXP, 0>(sn, s, pf, qf, L, kbuf, op, c, nmu);
        if constexpr (QK) __builtin_amdgcn_s_setprio(0);
    }

    // Region B, batch B: the reads of batch B+1, four PV MFMAs, the sum of
    // weights [B*EB, (B+1)*EB) of this tile, and mask + max of the same
    // scores of the next tile.
    template <bool PV, bool NEXT, bool EDGE, int B>
    static __device__ __forceinline__ void b_run(f32x16 (&o)[DB], const PF &pf, const f32x16 (&s)[MB],
                                                 float (&sum)[2], f32x16 (&sn)[MB], float (&mx)[2], const LN &L,
                                                 const char *vbuf, bf16x8 (&op)[kSlots], const EdgeMask &em) {
        if constexpr (B < BPV) {
            if constexpr (PV && B + 1 < BPV) {
                v_batch<B + 1>(op, L, vbuf);
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (PV) {
#pragma unroll
                for (int u = 0; u < kB; ++u) {
                    const int I = kB * B + u, st = I / DB, db = I % DB;
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[I % kSlots], pf.x[st], o[db], 0, 0, 0);
                }
#pragma unroll
                for (int e = B * EB; e < (B + 1) * EB; ++e) sum[e & 1] += s[e / 16][e % 16];
            }
            if constexpr (NEXT) {
#pragma unroll
                for (int e = B * EB; e < (B + 1) * EB; ++e) {
                    const int mb = e / 16, r = e % 16;
                    if constexpr (EDGE) {
                        const int j = em.k0 + mb * 32 + acc_row(r, 0);
                        sn[mb][r] = ((j >= em.lo4) & (j <= em.hi4)) ? sn[mb][r] : EEA_NEG_INF;
                    }
                    mx[e & 1] = fmaxf(mx[e & 1], sn[mb][r]);
                }
            }
            if constexpr (PV && NEXT) {
                constexpr int NV = (EDGE ? 6 * EB : 2 * EB) / kB;
#pragma unroll
                for (int u = 0; u < kB; ++u) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            b_run<PV, NEXT, EDGE, B + 1>(o, pf, s, sum, sn, mx, L, vbuf, op, em);
        }
    }
    template <bool PV, bool NEXT, bool EDGE>
    static __device__ __forceinline__ float region_b(f32x16 (&o)[DB], const PF &pf, const f32x16 (&s)[MB],
                                                     float &lpart, f32x16 (&sn)[MB], const LN &L, const char *vbuf,
                                                     const EdgeMask &em) {
        bf16x8 op[kSlots];
        float sum[2] = {0.f, 0.f}, mx[2] = {EEA_NEG_INF, EEA_NEG_INF};
        if constexpr (PV) {
            v_batch<0>(op, L, vbuf);
            __builtin_amdgcn_sched_barrier(0);
        }
        b_run<PV, NEXT, EDGE, 0>(o, pf, s, sum, sn, mx, L, vbuf, op, em);
        if constexpr (PV) lpart += sum[0] + sum[1];
        return fmaxf(mx[0], mx[1]);
    }
};

// Move the running max to cover a new tile whose lane max is mx (raw score
// units); rescale O and the normaliser only when some row's max grew by more
// than 2^kRescaleLog2.
template <class P>
__device__ __forceinline__ void raise_max(RowState<P> &rs, float mx, float c) {
    mx = max_across_halves(mx);
    const float mnew = fmaxf(rs.m, mx * c);
    if (__any(mnew > rs.m + kRescaleLog2)) {
        const float alpha = (mnew == EEA_NEG_INF) ? 1.f : fast_exp2(rs.m - mnew);
        rs.m = mnew;
        rs.lpart *= alpha;
#pragma unroll
        for (int db = 0; db < P::DB; ++db) rs.o[db] *= alpha;
    }
}

// DIL: dilation is live; BLK: the block-sparse rule is live; XT: the extra
// tiles of the log-spaced strided and random-block rules follow the band.
// Each is folded to a constant where off, since at 512 threads (two waves
// per SIMD, 256 registers each) the kernel has almost no registers to spare;
// the block-rule and extra-tile instances run 256 threads for that reason:
// the block-rule one at one wave per SIMD, the extra-tile one with two
// workgroups per CU (its unpipelined extra tiles wait on their copies, which
// the other workgroup's waves fill; 30 % faster on the strided rule than one
// workgroup per CU). NAR (narrow bands, band_is_narrow) is the plain
// kernel at 256 threads with the two-waves-per-SIMD budget, so two
// workgroups share a CU; at d = 64 it fits 168 registers and three share a
// CU (three waves per SIMD), which hides the copy-in, epilogue and global-row
// phases of its short loops behind the other workgroups' loops (c. 15 % on a
// band of 513 keys).
template <int D, bool DIL, bool BLK, bool XT = false, bool NAR = false, bool FUS = false>
__global__ void __launch_bounds__((BLK || XT || NAR) ? 256 : 512, NAR ? (D == 64 ? 3 : 2) : XT ? 2 : 1)
    fwd_band_bf16(const FwdParams prm) {
    constexpr bool GEN = BLK;
    typedef Bf16Path<D, (BLK || XT || NAR) ? 256 : 512> P;
    typedef BandPipe<P> BP;
    constexpr int BN = P::BN, BM = 32 * P::NW, MB = P::MB;

    // Every scalar parameter is read here, in one batch: left to itself the
    // compiler loads each from the kernel-argument segment where it is first
    // needed and waits for it there, about ten memory round trips one after
    // another before the first tile. Later uses reuse these loads.
    scalar_ready(prm.q, prm.k, prm.v, prm.out, prm.lse, prm.part, prm.head_stride, prm.BH, prm.H, prm.group, prm.N,
                 prm.wl, prm.wr, prm.block, prm.cap, prm.dil, prm.causal, prm.n_global, prm.num_qt, prm.chunks,
                 prm.fuse_grows, prm.xcd_remap, prm.scale_log2, gridDim.x);

    // Two K and two V buffers as distinct objects: the copy into one is never
    // mistaken for a hazard of the reads from another.
    __shared__ __attribute__((aligned(1024))) char kb0[P::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char kb1[P::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char vb0[P::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char vb1[P::TILE_BYTES];
    // GSEP: the gathered tile of global columns has buffers of its own, so
    // its copy goes out with the band's first copies (one wait for both).
    // Only in the four-wave d=64 instance, whose short loops make the extra
    // wait a large share; elsewhere it costs registers (d=128 at 256) or the
    // LDS two workgroups share.
    constexpr bool GSEP = FUS && NAR && D == 64;
    __shared__ __attribute__((aligned(1024))) char kgb[GSEP ? P::TILE_BYTES : 16];
    __shared__ __attribute__((aligned(1024))) char vgb[GSEP ? P::TILE_BYTES : 16];
    __shared__ int s_gidx[kMaxGlobal];
    __shared__ float s_gml[FUS ? 2 : 1][2][64];   // global-row exchange: max, normaliser

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ln = lane & 31, h = lane >> 5;
    const int ng = prm.n_global;

    // --- work item: (head, residue class, query tile); heaviest query tiles
    // first under a causal mask, runs of consecutive items on one XCD. With a
    // dilated mask (dilation k) the rows r, r+k, r+2k, ... of residue class r
    // see only each other, so each class is a band attention over a strided
    // sequence of its own (the window counted in its steps); k = 1 is the
    // plain sequence.
    const int G = gridDim.x;
    const int bid = blockIdx.x;
    const int dil = DIL ? prm.dil : 1;
    int bh, rcls, qi;
    if (!DIL && prm.xcd_remap == 2) {
        // workgroups are dispatched round-robin over the 8 XCDs (bid % 8):
        // each XCD owns BH/8 consecutive heads (their K/V share its L2) and
        // takes their query tiles heaviest first across all of them, so the
        // light causal tiles fill the tail
        const int hx = prm.BH >> 3;
        const int k = bid >> 3;
        bh = (bid & 7) * hx + k % hx;
        rcls = 0;
        qi = k / hx;
    } else {
        const int Lw = prm.xcd_remap ? (bid & 7) * (G >> 3) + (bid >> 3) : bid;
        const int per_head = dil * prm.num_qt;
        bh = Lw / per_head;
        rcls = (Lw - bh * per_head) / prm.num_qt;
        qi = Lw - bh * per_head - rcls * prm.num_qt;
    }
    const int unit = prm.causal ? prm.num_qt - 1 - qi : qi;
    const int N = (prm.N - rcls + dil - 1) / dil;   // rows of this residue class
    if (unit * BM >= N) return;                      // whole workgroup: a shorter class
    const Band band{N, prm.wl, prm.wr, BLK ? prm.block : 0, BLK ? prm.cap : 0};

    if (tid < kMaxGlobal) s_gidx[tid] = tid < ng ? prm.gidx[tid] : -1;

    const uint16_t *qh = static_cast<const uint16_t *>(prm.q) + (long long)bh * prm.head_stride + (long long)rcls * D;
    const uint16_t *kh =
        static_cast<const uint16_t *>(prm.k) + kv_head(prm, bh) * prm.head_stride + (long long)rcls * D;
    const uint16_t *vh =
        static_cast<const uint16_t *>(prm.v) + kv_head(prm, bh) * prm.head_stride + (long long)rcls * D;

    typename P::Lane L;
    // the wave index in a scalar register: the epilogue and the global-row
    // phase take it from here, so no lane register stays live across the loop
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    P::init_lane(L, lane, wave_u, dil);

    __syncthreads();   // s_gidx visible

    const int q0 = unit * BM;
    const int row = q0 + wave * 32 + ln;
    const bool valid = row < N;
    const int lo = row_lo(band, row);
    const int hi = row_hi(band, row);
    const int lo4 = lo - 4 * h, hi4 = hi - 4 * h;
    const int wr0 = q0 + wave * 32;
    const int wr1 = imin(N - 1, wr0 + 31);
    const bool wave_active = wr0 < N;
    int kt_lo, kt_hi;
    key_tile_range(band, q0, imin(N - 1, q0 + BM - 1), BN, &kt_lo, &kt_hi);
    int w_lo = kt_hi + 1, w_hi = kt_hi;   // this wave's key tiles (none if inactive)
    if (wave_active) key_tile_range(band, wr0, wr1, BN, &w_lo, &w_hi);

    typename P::QFrag qf;
    P::load_q(qf, qh, row * dil, valid, h);

    RowState<P> rs;
    rs.m = EEA_NEG_INF;
    rs.lpart = 0.f;
#pragma unroll
    for (int db = 0; db < P::DB; ++db) rs.o[db] = f32x16{};
    const float c = prm.scale_log2;

    // --- the gathered tile of global columns (at most kMaxGlobal = BN of
    // them: one tile), unpipelined (global tokens are not combined with a
    // dilated mask). A global column counts here only outside the row's
    // window.
    static_assert(kMaxGlobal <= BN, "the global columns fit one gathered tile");
    auto gathered = [&](const char *kbuf, const char *vbuf) __attribute__((always_inline)) {
        if (ng <= 32) {
            // every global column in the tile's first 32 columns: the second
            // row block of scores would be all masked, so only the first one
            // is computed (its products, exponentials and PV steps; the
            // skipped ones would add exact zeros, so the bits are the same)
            f32x16 s0 = f32x16{};
#pragma unroll
            for (int ks = 0; ks < P::KS; ++ks)
                s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8 *>(kbuf + L.krd[ks]),
                                                             qf.x[ks], s0, 0, 0, 0);
            float mx = EEA_NEG_INF;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int col = acc_row(r, h);
                const int g = s_gidx[col];
                const bool vis = (col < ng) & ((prm.causal == 0) | (g <= row)) & ((g < lo) | (g > hi));
                s0[r] = vis ? s0[r] : EEA_NEG_INF;
                mx = fmaxf(mx, s0[r]);
            }
            mx = max_across_halves(mx);
            const float mnew = fmaxf(rs.m, mx * c);
            if (__any(mnew > rs.m + kRescaleLog2)) {
                const float alpha = (mnew == EEA_NEG_INF) ? 1.f : fast_exp2(rs.m - mnew);
                rs.m = mnew;
                rs.lpart *= alpha;
#pragma unroll
                for (int db = 0; db < P::DB; ++db) rs.o[db] *= alpha;
            }
            const float mu = (rs.m == EEA_NEG_INF) ? 0.f : rs.m;
            float sum = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float pr = fast_exp2(__builtin_fmaf(s0[r], c, -mu));
                s0[r] = pr;
                sum += pr;
            }
            rs.lpart += sum;
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                const int r0 = 8 * st;
                f32x8 x = {s0[r0 + 0], s0[r0 + 1], s0[r0 + 2], s0[r0 + 3],
                           s0[r0 + 4], s0[r0 + 5], s0[r0 + 6], s0[r0 + 7]};
                const bf16x8 pw = __builtin_convertvector(x, bf16x8);
#pragma unroll
                for (int db = 0; db < P::DB; ++db)
                    rs.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(P::v_operand(L, vbuf, db, st), pw, rs.o[db],
                                                                       0, 0, 0);
            }
            return;
        }
        // clean: every global column passes for every row of the wave (all
        // rows exist, no global position lies in any row's band, and under a
        // causal mask every one precedes every row); only the columns past
        // the last global are then masked. The positions are sorted, and
        // the band ends never decrease with the row. (Wave-uniform: a scalar
        // branch.)
        const int gmin = __builtin_amdgcn_readfirstlane(s_gidx[0]);
        const int gmax = __builtin_amdgcn_readfirstlane(s_gidx[ng - 1]);
        const int w0 = q0 + wave_u * 32;
        const bool clean = (w0 + 31 < N) & ((gmax < row_lo(band, w0)) | (gmin > row_hi(band, w0 + 31))) &
                           ((prm.causal == 0) | (gmax <= w0));
        f32x16 s[MB];
        P::scores(s, qf, L, kbuf);
        if (!clean || ng < kMaxGlobal) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int col = mb * 32 + acc_row(r, h);
                    bool vis = col < ng;
                    if (!clean) {
                        const int g = s_gidx[col < kMaxGlobal ? col : 0];
                        vis &= ((prm.causal == 0) | (g <= row)) & ((g < lo) | (g > hi));
                    }
                    s[mb][r] = vis ? s[mb][r] : EEA_NEG_INF;
                }
        }
        softmax_pv_step<P>(rs, s, c, L, vbuf);
    };
    if (ng > 0) {
        typename P::Stage st;
        const TileSrc src{0, 1, N, ng, s_gidx};
        if constexpr (GSEP) {
            P::issue(st, L, kh, vh, kgb, vgb, src, s_gidx[0]);   // waited for with the band's first tiles
        } else {
            P::issue(st, L, kh, vh, kb0, vb0, src, s_gidx[0]);
            P::finish(st, kb0, vb0, tid);
            __syncthreads();
            if (wave_active) gathered(kb0, vb0);
            __syncthreads();
        }
    }

    // --- band tiles
    auto in_w = [&](int kt) { return kt >= w_lo && kt <= w_hi; };
    // a tile of the wave's range needs the mask unless every key of it lies
    // in every row's interval: [row_lo(last row), row_hi(first row)]. Under
    // the block rule these bounds take divisions, so they are computed once
    // (wave-uniform, scalar registers); the window form is cheap inline.
    const int full_lo = GEN ? __builtin_amdgcn_readfirstlane(row_lo(band, wr1)) : 0;
    const int full_hi = GEN ? __builtin_amdgcn_readfirstlane(row_hi(band, wr0)) : 0;
    auto is_edge = [&](int kt) {
        if constexpr (GEN) return !(kt * BN >= full_lo && kt * BN + BN - 1 <= full_hi);
        else return classify(band, wr0, wr1, kt * BN, kt * BN + BN - 1) != TILE_FULL;
    };

    // Order of the band tiles: positions 0 .. nt-1. When the global rows are
    // fused into this pass (four-wave instances), the workgroup's own key
    // tiles (the keys under its query rows, two tiles) come last, so they are
    // still in the two buffers when the loop ends; otherwise the order is
    // kt_lo .. kt_hi. Position nt and beyond map past kt_hi (no wave's tile).
    // The online softmax does not depend on the order of the tiles.
    // Only the FUS instances (128-row workgroups with global tokens: the
    // narrow, block-rule and extra-tile ones) fuse; in the others the order
    // is the plain one at compile time.
    constexpr bool CANFUSE = FUS;
    static_assert(!FUS || ((BLK || NAR || XT) && !DIL), "fusion needs 128-row workgroups");
    const bool fuse = CANFUSE && ng > 0 && prm.fuse_grows;
    const int nt = kt_hi - kt_lo + 1;
    const int own_lo = fuse ? imax(unit * 2, kt_lo) : kt_hi + 1;
    const int nown = fuse ? imax(0, imin(imin(unit * 2 + 1, kt_hi), (N - 1) / BN) - own_lo + 1) : 0;
    const int npre = nt - nown;
    auto tile_at = [&](int pos) {
        if constexpr (!CANFUSE) return kt_lo + pos;
        if (pos < npre) {
            const int t = kt_lo + pos;
            return t >= own_lo ? t + nown : t;
        }
        return pos < nt ? own_lo + (pos - npre) : kt_hi + 1;
    };

    P::issue_k(L, kh, N, kb0, tile_at(0) * BN, dil);
    P::issue_v(L, vh, N, vb0, tile_at(0) * BN, dil);
    if (1 < nt) P::issue_k(L, kh, N, kb1, tile_at(1) * BN, dil);
    wait_vmem();
    __syncthreads();
    if constexpr (GSEP) {
        if (ng > 0 && wave_active) gathered(kgb, vgb);
    }

    f32x16 sa[MB], sb[MB];
    typename P::PFrag pf;
    if (in_w(tile_at(0))) {
        P::scores(sa, qf, L, kb0);
        const EdgeMask em{tile_at(0) * BN, lo4, hi4};
        const float mx = is_edge(tile_at(0))
                             ? BP::template region_b<false, true, true>(rs.o, pf, sb, rs.lpart, sa, L, vb0, em)
                             : BP::template region_b<false, true, false>(rs.o, pf, sb, rs.lpart, sa, L, vb0, em);
        raise_max<P>(rs, mx, c);
    }
    __syncthreads();   // every wave is done with kb0

    // One iteration at position j; s holds S(tile j), sn receives S(tile j+1).
    auto iter = [&](int j, f32x16 (&s)[MB], f32x16 (&sn)[MB], const char *kr, const char *vr, char *kw, char *vw)
        __attribute__((always_inline)) {
        const int tn = tile_at(j + 1);
        debug_sync();
        if (j + 2 < nt) P::issue_k(L, kh, N, kw, tile_at(j + 2) * BN, dil);
        if (j + 1 < nt) P::issue_v(L, vh, N, vw, tn * BN, dil);
        debug_sync();
        const bool cur = in_w(tile_at(j)), nxt = in_w(tn);
        const EdgeMask em{tn * BN, lo4, hi4};
        const float nmu = rs.m == EEA_NEG_INF ? 0.f : -rs.m;
        if (cur) {
            if (nxt) {
                BP::template region_a<true, true>(sn, s, pf, qf, L, kr, c, nmu);
                const float mx = is_edge(tn)
                                     ? BP::template region_b<true, true, true>(rs.o, pf, s, rs.lpart, sn, L, vr, em)
                                     : BP::template region_b<true, true, false>(rs.o, pf, s, rs.lpart, sn, L, vr, em);
                raise_max<P>(rs, mx, c);
            } else {
                BP::template region_a<false, true>(sn, s, pf, qf, L, kr, c, nmu);
                BP::template region_b<true, false, false>(rs.o, pf, s, rs.lpart, sn, L, vr, em);
            }
        } else if (nxt) {
            BP::template region_a<true, false>(sn, s, pf, qf, L, kr, c, nmu);
            const float mx = is_edge(tn)
                                 ? BP::template region_b<false, true, true>(rs.o, pf, s, rs.lpart, sn, L, vr, em)
                                 : BP::template region_b<false, true, false>(rs.o, pf, s, rs.lpart, sn, L, vr, em);
            raise_max<P>(rs, mx, c);
        }
        wait_vmem();
        __syncthreads();
    };
    // The tiles of positions x sit in kb[x & 1] and vb[x & 1]; the loop is
    // unrolled by two so every buffer is a named object.
    for (int j = 0; j < nt; j += 2) {
        iter(j, sa, sb, kb1, vb0, kb0, vb1);
        if (j + 1 >= nt) break;
        iter(j + 1, sb, sa, kb0, vb1, kb1, vb0);
    }

    // The fused global-row phase runs right after the band loop when the
    // extra-tile rules follow (their tiles reuse the band buffers), else
    // after the epilogue.
    auto global_rows = [&]() __attribute__((always_inline)) {
        // --- the global rows against this workgroup's own key tiles (the
        // keys under its 128 query rows, positions npre and npre + 1 of the
        // loop, still in the buffers of those positions). Over all query
        // tiles every key tile is some workgroup's own exactly once, so the
        // partials (output, max, normaliser) of the global rows cover every
        // key once, without a pass of their own over K and V: partial `unit`
        // of each global row, combined by merge_kernel. Two waves per row
        // block of 32 global rows, one own tile each (a last query tile may
        // own one tile only); the second wave's state is folded into the
        // first's through LDS (the K buffers, free once both own tiles are
        // read), so each workgroup still writes one partial. A global row
        // sees every key up to the causal limit.
        // Lane and wave indices are taken afresh (mbcnt, and the wave index
        // in a scalar register): keeping the entry ones live across the band
        // loop costs registers the loop needs.
        const int glane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
        const int gh = glane >> 5;
        const int rb = wave_u >> 1, ot = wave_u & 1;   // row block, own tile
        const bool rows = rb * 32 < ng;                // wave-uniform
        const int gt = rb * 32 + (glane & 31);
        RowState<P> gs;
        gs.m = EEA_NEG_INF;
        gs.lpart = 0.f;
#pragma unroll
        for (int db = 0; db < P::DB; ++db) gs.o[db] = f32x16{};
        if (rows && ot < nown) {
            const int grow = gt < ng ? s_gidx[gt] : 0;
            typename P::QFrag gq;
            P::load_q(gq, qh, grow, gt < ng, gh);
            typename P::Lane GL;   // lane offsets taken afresh as well
            P::init_lane(GL, glane, wave_u, 1);
            // own tile ot sits at position npre + ot, in buffer (npre + ot) & 1
            const bool second = ((npre + ot) & 1) != 0;
            const char *kbuf = second ? kb1 : kb0;
            const char *vbuf = second ? vb1 : vb0;
            const int kt = own_lo + ot;
            f32x16 s[MB];
            P::scores(s, gq, GL, kbuf);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int jk = kt * BN + mb * 32 + acc_row(r, gh);
                    const bool vis = (gt < ng) & (jk < N) & ((prm.causal == 0) | (jk <= grow));
                    s[mb][r] = vis ? s[mb][r] : EEA_NEG_INF;
                }
            softmax_pv_step<P>(gs, s, c, GL, vbuf);
        }
        __syncthreads();   // both own tiles read: the K buffers take the exchange
        static_assert(P::DB * 16 * 64 * 4 <= P::TILE_BYTES, "one wave's output fits a K buffer");
        float *xo = reinterpret_cast<float *>(rb ? kb1 : kb0);
        if (rows && ot == 1) {
#pragma unroll
            for (int db = 0; db < P::DB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) xo[(db * 16 + i) * 64 + glane] = gs.o[db][i];
            s_gml[rb][0][glane] = gs.m;
            s_gml[rb][1][glane] = gs.lpart;
        }
        __syncthreads();
        if (rows && ot == 0) {
            const float m1 = s_gml[rb][0][glane], l1 = s_gml[rb][1][glane];
            const float m = fmaxf(gs.m, m1);
            const float w0 = gs.m == EEA_NEG_INF ? 0.f : fast_exp2(gs.m - m);
            const float w1 = m1 == EEA_NEG_INF ? 0.f : fast_exp2(m1 - m);
            gs.m = m;
            gs.lpart = w0 * gs.lpart + w1 * l1;
#pragma unroll
            for (int db = 0; db < P::DB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) gs.o[db][i] = w0 * gs.o[db][i] + w1 * xo[(db * 16 + i) * 64 + glane];
            if (gt < ng) {
                const float l = sum_across_halves(gs.lpart);
                float *dst = prm.part + (((long long)bh * ng + gt) * prm.chunks + unit) * (D + 2);
#pragma unroll
                for (int db = 0; db < P::DB; ++db)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        float *pp = dst + db * 32 + 8 * g + 4 * gh;
                        pp[0] = gs.o[db][4 * g + 0];
                        pp[1] = gs.o[db][4 * g + 1];
                        pp[2] = gs.o[db][4 * g + 2];
                        pp[3] = gs.o[db][4 * g + 3];
                    }
                if (gh == 0) {
                    dst[D] = gs.m;
                    dst[D + 1] = l;
                }
            }
        }
    };

    if constexpr (XT) {
        if (fuse) {
            global_rows();
            __syncthreads();   // the own tiles and the exchange buffers are free again
        }
    }
    if constexpr (XT) {
        // --- pairs of the strided and random-block rules beyond the band:
        // the random-block rule as unpipelined extra key tiles, the strided
        // rule pair by pair (below). A pair counts here only outside the
        // row's band, off the global columns (the gathered tile has those)
        // and within the causal limit; every tile is visited once per
        // pattern entry.
        const int q1 = imin(N - 1, q0 + BM - 1);
        // whether position j is a global token: a scan of the few, else a
        // binary search of the sorted positions in s_gidx (seven reads at
        // most, each lane its own j)
        auto is_global = [&](int j) __attribute__((always_inline)) {
            if (ng <= 6) {
                bool g = false;
                for (int t = 0; t < ng; ++t) g |= s_gidx[t] == j;
                return g;
            }
            int pos = 0;   // entries below j
#pragma unroll
            for (int step = 32; step > 0; step >>= 1)
                if (pos + step <= ng && s_gidx[pos + step - 1] < j) pos += step;
            return pos < ng && s_gidx[pos] == j;
        };
        static_assert(kMaxGlobal == 64 && BN == 64, "the search covers 64 positions, one tile row per lane");
        auto extra_tile = [&](int k0, bool take, auto vis) __attribute__((always_inline)) {
            P::issue_k(L, kh, N, kb0, k0);
            P::issue_v(L, vh, N, vb0, k0);
            wait_vmem();
            __syncthreads();
            if (take) {
                // global columns of this tile, one bit per key: lane l tests
                // key k0 + l
                const unsigned long long gm = __ballot(is_global(k0 + lane));
                f32x16 s[MB];
                P::scores(s, qf, L, kb0);
                // no mask needed when every key of the tile passes for every
                // row of the wave (all rows exist, the tile lies inside the
                // listed block, outside every row's band, holds no global
                // column and, under a causal mask, precedes every row)
                const int k1 = k0 + BN - 1;
                const bool full = (wr0 + 31 < N) & vis(k0) & vis(k1) & (gm == 0) &
                                  (classify(band, wr0, wr0 + 31, k0, k1) == TILE_SKIP) &
                                  ((prm.causal == 0) | (k1 <= wr0));
                if (!full) {
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int jr = mb * 32 + acc_row(r, h), j = k0 + jr;
                            const bool ok = valid & (j < N) & ((j < lo) | (j > hi)) & ((prm.causal == 0) | (j <= row)) &
                                            !((gm >> jr) & 1ull) && vis(j);
                            s[mb][r] = ok ? s[mb][r] : EEA_NEG_INF;
                        }
                }
                softmax_pv_step<P>(rs, s, c, L, vb0);
            }
            __syncthreads();
        };
        if (prm.stride > 0) {
            // offsets o = stride * 2^m < N. A row sees at most one key per
            // offset and side, so each such pair is one dot product on the
            // vector ALU (each lane takes its half of d, as its Q operand
            // holds it; the halves are summed across the wave halves)
            // instead of a 64-key tile of which one key per row is used.
            // The weight is kept in fp32 for the output as for the
            // normaliser.
            const int st = prm.stride;
            int mtop = -1;
            while (mtop < 30 && ((long long)st << (mtop + 1)) < N) ++mtop;
            for (int side = 0; side < (prm.causal ? 1 : 2); ++side)
                for (int m = 0; m <= mtop; ++m) {
                    const int o = st << m;
                    const int j = side ? row + o : row - o;
                    bool ok = valid & (j >= 0) & (j < N) & ((j < lo) | (j > hi));
                    if (ng > 0) ok &= !is_global(j);   // pairs of the gathered global tile
                    if (!__any(ok)) continue;
                    const int jj = ok ? j : 0;   // a row that exists; its result is dropped
                    const float part = dot_row_half(kh + (long long)jj * D, qf.x, h);
                    const float sl = ok ? sum_across_halves(part) * c : EEA_NEG_INF;   // log2 domain
                    const float mnew = fmaxf(rs.m, sl);
                    if (__any(mnew > rs.m + kRescaleLog2)) {
                        const float alpha = (mnew == EEA_NEG_INF) ? 1.f : fast_exp2(rs.m - mnew);
                        rs.m = mnew;
                        rs.lpart *= alpha;
#pragma unroll
                        for (int db = 0; db < P::DB; ++db) rs.o[db] *= alpha;
                    }
                    const float pw = ok ? fast_exp2(sl - rs.m) : 0.f;
                    if (h == 0) rs.lpart += pw;   // one half counts the key in the normaliser
                    axpy_row_half(rs.o, pw, vh + (long long)jj * D, h);   // O^T += p V_j
                }
        }
        if (prm.rand_block > 0) {
            // each query block's listed key blocks (out-of-range entries
            // skipped, repeats taken once); rows of one wave share a block
            const int b = prm.rand_block, nr = prm.n_rand, nkb = (N + b - 1) / b;
            const int my_qb = wr0 / b;
            for (int qb = q0 / b; qb <= q1 / b; ++qb) {
                const int *lst = prm.rand_idx + (long long)qb * nr;
                for (int e = 0; e < nr; ++e) {
                    const int kb = lst[e];
                    bool skip = kb < 0 || kb >= nkb;
                    for (int e2 = 0; e2 < e; ++e2) skip |= lst[e2] == kb;
                    if (skip) continue;
                    const int klo = kb * b, khi = imin(N - 1, klo + b - 1);
                    if (prm.causal && klo > imin(q1, qb * b + b - 1)) continue;
                    for (int t = klo / BN; t <= khi / BN; ++t)
                        extra_tile(t * BN, wave_active && my_qb == qb, [&](int j) { return j >= klo && j <= khi; });
                }
            }
        }
    }

    // --- epilogue (the row taken afresh from the lane index, as in the
    // global-row phase below)
    {
        const int elane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
        const int eh = elane >> 5;
        const int erow = q0 + wave_u * 32 + (elane & 31);
        const int orow = rcls + erow * dil;   // row index in the stored sequence
        bool store = erow < N;
        for (int t = 0; t < ng; ++t) store &= s_gidx[t] != orow;   // global rows are written by the merge
        if (store) {
            const float l = sum_across_halves(rs.lpart);
            const float inv = l > 0.f ? 1.f / l : 0.f;
            uint16_t *oh = static_cast<uint16_t *>(prm.out) + (long long)bh * prm.head_stride;
            P::store_out(oh, orow, rs.o, inv, eh);
            if (eh == 0) prm.lse[(long long)bh * prm.N + orow] = l > 0.f ? (rs.m + __log2f(l)) * kLn2 : EEA_NEG_INF;
        }
    }

    if constexpr (!XT) {
        if (fuse) global_rows();
    }
}

// Merge of the split-key partials of one global row: the same rescaling
// identity as the online softmax, applied across chunks.
template <int D, bool F32>
__global__ void __launch_bounds__(256) merge_kernel(const FwdParams prm) {
    // One workgroup per (head, global row); its four waves take every fourth
    // partial. Per wave: the largest partial max, then the weights
    // exp2(m_c - M) and the weighted normalisers and outputs of its partials
    // (lanes over d); the four waves' results are combined through LDS.
    __shared__ float wm[4], wl[4];
    __shared__ float wo[4][D];
    const int ng = prm.n_global, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int bh = blockIdx.x / ng, t = blockIdx.x - bh * ng;
    const int g = prm.gidx[t];
    const int C = prm.chunks;
    const float *src = prm.part + ((long long)bh * ng + t) * C * (D + 2);
    float M = EEA_NEG_INF;
    for (int ci = wave + 4 * lane; ci < C; ci += 256) M = fmaxf(M, src[ci * (D + 2) + D]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    constexpr int PER = D / 64;
    float acc[PER], Lsum = 0.f;
#pragma unroll
    for (int j = 0; j < PER; ++j) acc[j] = 0.f;
#pragma unroll 4
    for (int ci = wave; ci < C; ci += 4) {
        const float *pc = src + ci * (D + 2);
        const float mc = pc[D];
        const float w = mc == EEA_NEG_INF ? 0.f : fast_exp2(mc - M);
        Lsum += w * pc[D + 1];
#pragma unroll
        for (int j = 0; j < PER; ++j) acc[j] += pc[lane + 64 * j] * w;
    }
    if (lane == 0) {
        wm[wave] = M;
        wl[wave] = Lsum;
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) wo[wave][lane + 64 * j] = acc[j];
    __syncthreads();
    if (wave != 0) return;
    const float Mt = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
    float sc[4], Lt = 0.f;
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4) {
        sc[w4] = wm[w4] == EEA_NEG_INF ? 0.f : fast_exp2(wm[w4] - Mt);
        Lt += sc[w4] * wl[w4];
    }
    const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int dd = lane + 64 * j;
        const float o = (sc[0] * wo[0][dd] + sc[1] * wo[1][dd] + sc[2] * wo[2][dd] + sc[3] * wo[3][dd]) * inv;
        const long long oi = ((long long)bh * prm.N + g) * D + dd;
        if (F32) {
            static_cast<float *>(prm.out)[oi] = o;
        } else {
            static_cast<__bf16 *>(prm.out)[oi] = (__bf16)o;
        }
    }
    if (lane == 0) prm.lse[(long long)bh * prm.N + g] = Lt > 0.f ? (Mt + __log2f(Lt)) * kLn2 : EEA_NEG_INF;
}

// ---------------------------------------------------------------------------
// Host-side launch.
// ---------------------------------------------------------------------------
template <class PB, class PG64, class PG128, int D, bool F32>
static hipError_t launch_impl(const FwdParams &p0, hipStream_t stream) {
    FwdParams p = p0;
    const int grid = p.BH * p.dil * p.num_qt;
    p.xcd_remap = (grid % 8 == 0) ? 1 : 0;
    // short causal sequences: heads per XCD, heaviest tiles first across
    // them (the tail is a large share of the call). Long ones keep one head
    // at a time per XCD, whose K/V stream the XCD's L2 then serves to every
    // workgroup (measured: 872 -> 930 TFLOP/s at N=4096, B*H=128; 1161 ->
    // 1114 at N=32768, B*H=32 with the head-interleaved order)
    if (!F32 && p.dil == 1 && p.causal && p.BH % 8 == 0 && p.num_qt <= 32) p.xcd_remap = 2;
    if constexpr (F32)
        hipLaunchKernelGGL((fwd_kernel<PB, MODE_BAND>), dim3(grid), dim3(PB::NT), 0, stream, p);
    else if ((p.stride > 0 || p.rand_block > 0) && p.fuse_grows)
        hipLaunchKernelGGL((fwd_band_bf16<D, false, false, true, false, true>), dim3(grid), dim3(kBandThreadsBlock), 0,
                           stream, p);
    else if (p.stride > 0 || p.rand_block > 0)
        hipLaunchKernelGGL((fwd_band_bf16<D, false, false, true>), dim3(grid), dim3(kBandThreadsBlock), 0, stream, p);
    else if (p.block > 0 && p.fuse_grows)
        hipLaunchKernelGGL((fwd_band_bf16<D, false, true, false, false, true>), dim3(grid), dim3(kBandThreadsBlock), 0,
                           stream, p);
    else if (p.block > 0)
        hipLaunchKernelGGL((fwd_band_bf16<D, false, true>), dim3(grid), dim3(kBandThreadsBlock), 0, stream, p);
    else if (p.dil > 1)
        hipLaunchKernelGGL((fwd_band_bf16<D, true, false>), dim3(grid), dim3(PB::NT), 0, stream, p);
    else if (band_is_narrow(p.wl, p.wr, p.dil) && p.fuse_grows)
        hipLaunchKernelGGL((fwd_band_bf16<D, false, false, false, true, true>), dim3(grid), dim3(kBandThreadsNarrow), 0,
                           stream, p);
    else if (band_is_narrow(p.wl, p.wr, p.dil))
        hipLaunchKernelGGL((fwd_band_bf16<D, false, false, false, true>), dim3(grid), dim3(kBandThreadsNarrow), 0, stream, p);
    else
        hipLaunchKernelGGL((fwd_band_bf16<D, false, false>), dim3(grid), dim3(PB::NT), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.n_global == 0) return e;
    if (p.fuse_grows) {   // the band pass wrote the global rows' partials
        hipLaunchKernelGGL((merge_kernel<D, F32>), dim3(p.BH * p.n_global), dim3(256), 0, stream, p);
        return hipGetLastError();
    }
    const int ggrid = p.BH * p.chunks;
    p.xcd_remap = (ggrid % 8 == 0) ? 1 : 0;
    if (p.n_global <= 32)
        hipLaunchKernelGGL((fwd_kernel<PG64, MODE_GROWS>), dim3(ggrid), dim3(64), 0, stream, p);
    else
        hipLaunchKernelGGL((fwd_kernel<PG128, MODE_GROWS>), dim3(ggrid), dim3(128), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((merge_kernel<D, F32>), dim3(p.BH * p.n_global), dim3(256), 0, stream, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free forward (attn_fwd_noalloc): the global-row
// partials of callers that cannot allocate device memory. One copy of the
// array per device, from module load to the end of the process; every call
// on a device uses the same memory, so calls that overlap on one device race.
// Host code uses the address hipGetSymbolAddress returns for the current
// device, never the array's name.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void **ptr) {
    static std::mutex mu;
    static std::vector<void *> addr;   // per device, looked up once
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lk(mu);
    if ((int)addr.size() <= dev) addr.resize(dev + 1, nullptr);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_forward(const FwdParams &p, int d, int f32, hipStream_t stream) {
    if (f32) {
        if (d == 64)
            return launch_impl<F32Path<64, kBandThreadsF32>, F32Path<64, 64>, F32Path<64, 128>, 64, true>(p, stream);
        return launch_impl<F32Path<128, kBandThreadsF32>, F32Path<128, 64>, F32Path<128, 128>, 128, true>(p, stream);
    }
    if (d == 64)
        return launch_impl<Bf16Path<64, kBandThreadsBf16>, Bf16Path<64, 64>, Bf16Path<64, 128>, 64, false>(p, stream);
    return launch_impl<Bf16Path<128, kBandThreadsBf16>, Bf16Path<128, 64>, Bf16Path<128, 128>, 128, false>(p, stream);
}

}  // namespace eea
