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
//  * One workgroup = 4 wave64s = 128 query rows; each wave owns 32 rows.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: K rows are the A operand (from LDS), the
//    wave's 32 queries are the B operand (kept in registers for the whole
//    kernel). In the 32x32 accumulator layout a lane then holds ONE query and
//    16 keys, so the row max and row sum are in-lane reductions plus a single
//    exchange between the two half-waves.
//  * The output is accumulated transposed, O^T += V^T P^T, so the fp32
//    accumulators of a lane also belong to its one query: the online-softmax
//    rescale is a per-lane scalar multiply. The exponentiated scores, rounded
//    to bf16, are already in the B-operand layout of this product; the key
//    order inside each 16-key step is permuted to match, and V^T is stored in
//    LDS in that permuted order.
//  * K and V^T tiles are double-buffered in LDS: the next tile's global loads
//    are issued before the current tile's matrix work and written to the
//    other buffer after it, one barrier per tile. 16-byte LDS chunks are XOR
//    swizzled so the MFMA operand reads are free of bank conflicts.
//  * Softmax runs in the exp2 domain with scale*log2(e) folded into one FMA.
//    The running max is only moved (and the accumulators rescaled) when it
//    grows by more than 2^8; otherwise the stale max keeps every weight below
//    256, which is exact once divided by the same running normaliser.
//  * Work items are ordered heaviest-first for causal masks, and consecutive
//    work items are grouped onto one XCD so the workgroups that share a
//    head's K/V stream share that XCD's L2.
//  * fp32 inputs use v_mfma_f32_32x32x2_f32 with the same transposed scheme.
//
// Global tokens: global COLUMNS are gathered into one extra key tile per
// query tile (masked where the column already lies in the row's window);
// global ROWS see every key, so they are computed by a split-key pass that
// writes partial (o, m, l) per key chunk and a merge kernel that combines
// them with the same rescaling identity the online softmax uses.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_internal.h"
#include "attn_plan.h"

namespace eea {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleLog2 = 8.0f;
#define EEA_NEG_INF (-__builtin_huge_valf())

enum { MODE_BAND = 0, MODE_GROWS = 1 };
enum { KIND_FULL = 0, KIND_EDGE = 1, KIND_GATHER = 2 };

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Key offset (within its 32-key block) of accumulator register r of a lane in
// half-wave h, for the 32x32 MFMA output layout.
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// ---------------------------------------------------------------------------
// bf16 inputs: QK^T and PV on v_mfma_f32_32x32x16_bf16.
// ---------------------------------------------------------------------------
template <int D_, int BN_, int NT_>
struct Bf16Path {
    static constexpr int D = D_, BN = BN_, NT = NT_;
    static constexpr bool F32 = false;
    static constexpr int KS = D / 16;     // k-steps of QK^T
    static constexpr int MB = BN / 32;    // 32-key blocks per tile
    static constexpr int DB = D / 32;     // 32-wide blocks of d in O^T
    static constexpr int PVS = BN / 16;   // 16-key steps of PV
    static constexpr int KROW = D * 2;    // bytes per K row in LDS
    static constexpr int VROW = BN * 2;   // bytes per V^T row in LDS
    static constexpr int TILE_BYTES = BN * D * 2;
    static constexpr int K_CHUNKS = BN * D / 8;
    static constexpr int K_PER_T = (K_CHUNKS + NT - 1) / NT;
    static constexpr int V_BLOCKS = (BN / 4) * (D / 8);   // 4 keys x 8 d
    static constexpr int V_PER_T = (V_BLOCKS + NT - 1) / NT;
    static constexpr int LDS_BYTES = 4 * TILE_BYTES;     // K, V^T, two buffers each
    static_assert(D % 64 == 0 && BN % 64 == 0, "tile shape");

    typedef uint16_t elem_t;
    struct QFrag { bf16x8 x[KS]; };
    struct Stage { u32x4 k[K_PER_T]; u32x4 v[V_PER_T][4]; };
    struct PFrag { bf16x8 x[PVS]; };

    static __device__ __forceinline__ int k_off(int row, int chunk) {
        return row * KROW + ((chunk ^ (row & 7)) << 4);
    }
    static __device__ __forceinline__ int v_off(int d, int chunk) {
        return d * VROW + ((chunk ^ ((d ^ (d >> 3)) & 7)) << 4);
    }

    static __device__ __forceinline__ void load_q(QFrag &qf, const elem_t *qh, int row, bool valid, int h) {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(qh + (long long)row * D);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 w = valid ? src[2 * ks + h] : u32x4{0, 0, 0, 0};
            qf.x[ks] = __builtin_bit_cast(bf16x8, w);
        }
    }

    // Global -> registers for one key tile. key_of(row) gives the source key
    // of tile row `row`, or -1 for a zero row.
    template <class KeyOf>
    static __device__ __forceinline__ void load_stage(Stage &st, const elem_t *kh, const elem_t *vh,
                                                      KeyOf key_of, int tid) {
#pragma unroll
        for (int i = 0; i < K_PER_T; ++i) {
            int c = tid + i * NT;
            st.k[i] = u32x4{0, 0, 0, 0};
            if (c < K_CHUNKS) {
                int row = c / (D / 8), ch = c % (D / 8);
                int key = key_of(row);
                if (key >= 0)
                    st.k[i] = *reinterpret_cast<const u32x4 *>(kh + (long long)key * D + ch * 8);
            }
        }
#pragma unroll
        for (int i = 0; i < V_PER_T; ++i) {
            int b = tid + i * NT;
#pragma unroll
            for (int r = 0; r < 4; ++r) st.v[i][r] = u32x4{0, 0, 0, 0};
            if (b < V_BLOCKS) {
                int kg = b / (D / 8), dc = b % (D / 8);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    int key = key_of(4 * kg + r);
                    if (key >= 0)
                        st.v[i][r] = *reinterpret_cast<const u32x4 *>(vh + (long long)key * D + dc * 8);
                }
            }
        }
    }

    // Registers -> LDS. K rows go in as they are (swizzled 16-byte chunks);
    // each 4-key x 8-d block of V is transposed in registers and written as
    // eight 8-byte runs of V^T, in the permuted key order of the PV operand.
    static __device__ __forceinline__ void store_stage(const Stage &st, char *kbuf, char *vbuf, int tid) {
#pragma unroll
        for (int i = 0; i < K_PER_T; ++i) {
            int c = tid + i * NT;
            if (c < K_CHUNKS) {
                int row = c / (D / 8), ch = c % (D / 8);
                *reinterpret_cast<u32x4 *>(kbuf + k_off(row, ch)) = st.k[i];
            }
        }
#pragma unroll
        for (int i = 0; i < V_PER_T; ++i) {
            int b = tid + i * NT;
            if (b < V_BLOCKS) {
                int kg = b / (D / 8), dc = b % (D / 8);
                int ko = 4 * kg;
                int in16 = ko & 15;
                int pos = (ko & ~15) | ((in16 & 4) << 1) | ((in16 & 8) >> 1);
                int chunk = pos >> 3, within = (pos & 7) * 2;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    int p = e >> 1;
                    unsigned w0, w1;
                    if (e & 1) {
                        w0 = (st.v[i][0][p] >> 16) | (st.v[i][1][p] & 0xffff0000u);
                        w1 = (st.v[i][2][p] >> 16) | (st.v[i][3][p] & 0xffff0000u);
                    } else {
                        w0 = (st.v[i][0][p] & 0xffffu) | (st.v[i][1][p] << 16);
                        w1 = (st.v[i][2][p] & 0xffffu) | (st.v[i][3][p] << 16);
                    }
                    int d = dc * 8 + e;
                    *reinterpret_cast<u32x2 *>(vbuf + v_off(d, chunk) + within) = u32x2{w0, w1};
                }
            }
        }
    }

    static __device__ __forceinline__ void scores(f32x16 (&s)[MB], const QFrag &qf, const char *kbuf,
                                                  int ln, int h) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            f32x16 acc = {};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                bf16x8 a = *reinterpret_cast<const bf16x8 *>(kbuf + k_off(mb * 32 + ln, 2 * ks + h));
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf.x[ks], acc, 0, 0, 0);
            }
            s[mb] = acc;
        }
    }

    static __device__ __forceinline__ void pack_p(PFrag &pf, const f32x16 (&s)[MB]) {
#pragma unroll
        for (int st = 0; st < PVS; ++st) {
            const int mb = st >> 1, r0 = 8 * (st & 1);
            f32x8 x = {s[mb][r0 + 0], s[mb][r0 + 1], s[mb][r0 + 2], s[mb][r0 + 3],
                       s[mb][r0 + 4], s[mb][r0 + 5], s[mb][r0 + 6], s[mb][r0 + 7]};
            pf.x[st] = __builtin_convertvector(x, bf16x8);
        }
    }

    static __device__ __forceinline__ void pv(f32x16 (&o)[DB], const PFrag &pf, const char *vbuf,
                                              int ln, int h) {
#pragma unroll
        for (int st = 0; st < PVS; ++st) {
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                bf16x8 a = *reinterpret_cast<const bf16x8 *>(vbuf + v_off(db * 32 + ln, 2 * st + h));
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf.x[st], o[db], 0, 0, 0);
            }
        }
    }

    static __device__ __forceinline__ void store_out(elem_t *oh, int row, const f32x16 (&o)[DB],
                                                     float inv, int h) {
        elem_t *dst = oh + (long long)row * D;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 x = {o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv,
                           o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv};
                typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
                bf16x4 y = __builtin_convertvector(x, bf16x4);
                *reinterpret_cast<bf16x4 *>(dst + db * 32 + 8 * g + 4 * h) = y;
            }
        }
    }
};

// ---------------------------------------------------------------------------
// fp32 inputs: both products on v_mfma_f32_32x32x2_f32 (true fp32 products).
// The contraction index of QK^T is split between half-waves as d = h*D/2 + s.
// ---------------------------------------------------------------------------
template <int D_, int BN_, int NT_>
struct F32Path {
    static constexpr int D = D_, BN = BN_, NT = NT_;
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
    static_assert(D % 32 == 0 && BN % 32 == 0, "tile shape");

    typedef float elem_t;
    struct QFrag { float x[KS]; };
    struct Stage { u32x4 k[PER_T]; u32x4 v[PER_T]; };
    struct PFrag { float x[MB][16]; };

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

    template <class KeyOf>
    static __device__ __forceinline__ void load_stage(Stage &st, const elem_t *kh, const elem_t *vh,
                                                      KeyOf key_of, int tid) {
#pragma unroll
        for (int i = 0; i < PER_T; ++i) {
            int c = tid + i * NT;
            st.k[i] = u32x4{0, 0, 0, 0};
            st.v[i] = u32x4{0, 0, 0, 0};
            if (c < CHUNKS) {
                int row = c / CH, ch = c % CH;
                int key = key_of(row);
                if (key >= 0) {
                    st.k[i] = *reinterpret_cast<const u32x4 *>(kh + (long long)key * D + ch * 4);
                    st.v[i] = *reinterpret_cast<const u32x4 *>(vh + (long long)key * D + ch * 4);
                }
            }
        }
    }

    static __device__ __forceinline__ void store_stage(const Stage &st, char *kbuf, char *vbuf, int tid) {
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

    static __device__ __forceinline__ void scores(f32x16 (&s)[MB], const QFrag &qf, const char *kbuf,
                                                  int ln, int h) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            f32x16 acc = {};
#pragma unroll
            for (int c = 0; c < D / 8; ++c) {
                f32x4 a = *reinterpret_cast<const f32x4 *>(kbuf + k_off(mb * 32 + ln, h * (D / 8) + c));
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

    static __device__ __forceinline__ void pv(f32x16 (&o)[DB], const PFrag &pf, const char *vbuf,
                                              int ln, int h) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = mb * 32 + acc_row(r, h);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    float a = *reinterpret_cast<const float *>(vbuf + key * ROW + (db * 32 + ln) * 4);
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
                                                const char *vbuf, int ln, int h) {
    float mx = EEA_NEG_INF;
#pragma unroll
    for (int mb = 0; mb < P::MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
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
    P::pv(rs.o, pf, vbuf, ln, h);
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

    __shared__ __attribute__((aligned(16))) char smem[P::LDS_BYTES];
    __shared__ int s_gidx[kMaxGlobal];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ln = lane & 31, h = lane >> 5;
    const int N = prm.N;
    const int ng = prm.n_global;
    const Band band{N, prm.wl, prm.wr};

    if (tid < kMaxGlobal) s_gidx[tid] = tid < ng ? prm.gidx[tid] : -1;

    // --- which work item
    const int G = gridDim.x;
    const int bid = blockIdx.x;
    const int L = prm.xcd_remap ? (bid & 7) * (G >> 3) + (bid >> 3) : bid;
    int bh, unit;
    if (MODE == MODE_BAND) {
        bh = L / prm.num_qt;
        const int qi = L - bh * prm.num_qt;
        unit = prm.causal ? prm.num_qt - 1 - qi : qi;
    } else {
        bh = L / prm.chunks;
        unit = L - bh * prm.chunks;
    }
    const elem_t *qh = static_cast<const elem_t *>(prm.q) + (long long)bh * prm.head_stride;
    const elem_t *kh = static_cast<const elem_t *>(prm.k) + (long long)bh * prm.head_stride;
    const elem_t *vh = static_cast<const elem_t *>(prm.v) + (long long)bh * prm.head_stride;

    __syncthreads();   // s_gidx visible

    // --- this lane's query row and its visible key interval [lo, hi]
    int row, lo, hi, kt_lo, kt_hi, wave_lo, wave_hi;
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
        wave_lo = row_lo(band, wr0);
        wave_hi = row_hi(band, wr1);
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
        wave_lo = 0;
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
    // buffer b: K at smem + 2*b*TILE, V^T right after it
    auto kbuf = [&](int b) { return smem + 2 * b * P::TILE_BYTES; };
    auto vbuf = [&](int b) { return smem + (2 * b + 1) * P::TILE_BYTES; };

    // --- gathered tiles of global columns (one per BN globals)
    if (MODE == MODE_BAND && ng > 0) {
        for (int g0 = 0; g0 < ng; g0 += BN) {
            typename P::Stage st;
            P::load_stage(st, kh, vh, [&](int r) { return g0 + r < ng ? s_gidx[g0 + r] : -1; }, tid);
            P::store_stage(st, kbuf(0), vbuf(0), tid);
            __syncthreads();
            if (wave_active) {
                f32x16 s[P::MB];
                P::scores(s, qf, kbuf(0), ln, h);
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
                softmax_pv_step<P>(rs, s, c, vbuf(0), ln, h);
            }
            __syncthreads();
        }
    }

    // --- band tiles, double-buffered
    if (kt_lo <= kt_hi) {
        {
            typename P::Stage st;
            const int k0 = kt_lo * BN;
            P::load_stage(st, kh, vh, [&](int r) { return k0 + r < N ? k0 + r : -1; }, tid);
            P::store_stage(st, kbuf(0), vbuf(0), tid);
        }
        __syncthreads();
        int cur = 0;
        for (int kt = kt_lo; kt <= kt_hi; ++kt) {
            const bool more = kt < kt_hi;
            typename P::Stage st;
            if (more) {
                const int k1 = (kt + 1) * BN;
                P::load_stage(st, kh, vh, [&](int r) { return k1 + r < N ? k1 + r : -1; }, tid);
            }
            const int k0 = kt * BN;
            int kind;
            if (MODE == MODE_BAND) {
                const int cl = classify(band, wr0, wr1, k0, k0 + BN - 1);
                kind = (cl == TILE_SKIP || !wave_active) ? -1 : (cl == TILE_FULL ? KIND_FULL : KIND_EDGE);
            } else {
                kind = (!wave_active || k0 > wave_hi) ? -1 : KIND_EDGE;
            }
            if (kind >= 0) {
                f32x16 s[P::MB];
                P::scores(s, qf, kbuf(cur), ln, h);
                if (kind == KIND_EDGE) {
#pragma unroll
                    for (int mb = 0; mb < P::MB; ++mb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int j = k0 + mb * 32 + acc_row(r, h);
                            s[mb][r] = ((j >= lo) & (j <= hi)) ? s[mb][r] : EEA_NEG_INF;
                        }
                }
                softmax_pv_step<P>(rs, s, c, vbuf(cur), ln, h);
            }
            if (more) P::store_stage(st, kbuf(cur ^ 1), vbuf(cur ^ 1), tid);
            __syncthreads();
            cur ^= 1;
        }
    }
    (void)wave_lo;

    // --- epilogue
    const float l = rs.lpart + __shfl_xor(rs.lpart, 32, 64);
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
                f32x4 x = {rs.o[db][4 * g + 0], rs.o[db][4 * g + 1], rs.o[db][4 * g + 2], rs.o[db][4 * g + 3]};
                float *p = dst + db * 32 + 8 * g + 4 * h;
                p[0] = x[0]; p[1] = x[1]; p[2] = x[2]; p[3] = x[3];
            }
        if (h == 0) {
            dst[D] = rs.m;
            dst[D + 1] = l;
        }
    }
}

// Merge of the split-key partials of one global row: the same rescaling
// identity as the online softmax, applied across chunks.
template <int D, bool F32>
__global__ void __launch_bounds__(64) merge_kernel(const FwdParams prm) {
    const int ng = prm.n_global;
    const int bh = blockIdx.x / ng, t = blockIdx.x - bh * ng;
    __shared__ int s_g;
    if (threadIdx.x == 0) s_g = prm.gidx[t];
    __syncthreads();
    const int g = s_g;
    const float *src = prm.part + ((long long)bh * ng + t) * prm.chunks * (D + 2);
    float M = EEA_NEG_INF;
    for (int ci = 0; ci < prm.chunks; ++ci) M = fmaxf(M, src[ci * (D + 2) + D]);
    float Lsum = 0.f;
    for (int ci = 0; ci < prm.chunks; ++ci) {
        const float mc = src[ci * (D + 2) + D];
        if (mc != EEA_NEG_INF) Lsum += src[ci * (D + 2) + D + 1] * fast_exp2(mc - M);
    }
    const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
    for (int dd = threadIdx.x; dd < D; dd += 64) {
        float acc = 0.f;
        for (int ci = 0; ci < prm.chunks; ++ci) {
            const float mc = src[ci * (D + 2) + D];
            if (mc != EEA_NEG_INF) acc += src[ci * (D + 2) + dd] * fast_exp2(mc - M);
        }
        const long long o = ((long long)bh * prm.N + g) * D + dd;
        if (F32) {
            static_cast<float *>(prm.out)[o] = acc * inv;
        } else {
            static_cast<__bf16 *>(prm.out)[o] = (__bf16)(acc * inv);
        }
    }
    if (threadIdx.x == 0)
        prm.lse[(long long)bh * prm.N + g] = Lsum > 0.f ? (M + __log2f(Lsum)) * kLn2 : EEA_NEG_INF;
}

// ---------------------------------------------------------------------------
// Host-side launch.
// ---------------------------------------------------------------------------
template <int D> using BandBf16 = Bf16Path<D, 64, 256>;
template <int D> using BandF32 = F32Path<D, 32, 256>;

int tile_bm(int d, int f32) { (void)d; (void)f32; return 128; }
int tile_bn(int d, int f32) { (void)d; return f32 ? 32 : 64; }

int global_chunks(int BH, int N, int d, int f32, int *chunk_tiles) {
    const int bn = tile_bn(d, f32);
    const int num_kt = (N + bn - 1) / bn;
    // aim for a few hundred workgroups in the split-key pass
    int target = (512 + BH - 1) / BH;
    if (target < 1) target = 1;
    if (target > num_kt) target = num_kt;
    int ct = (num_kt + target - 1) / target;
    if (ct < 1) ct = 1;
    if (chunk_tiles) *chunk_tiles = ct;
    return (num_kt + ct - 1) / ct;
}

template <class PB, class PG64, class PG128, int D, bool F32>
static hipError_t launch_impl(const FwdParams &p0, hipStream_t stream) {
    FwdParams p = p0;
    const int grid = p.BH * p.num_qt;
    p.xcd_remap = (grid % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((fwd_kernel<PB, MODE_BAND>), dim3(grid), dim3(PB::NT), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.n_global == 0) return e;
    const int ggrid = p.BH * p.chunks;
    p.xcd_remap = (ggrid % 8 == 0) ? 1 : 0;
    if (p.n_global <= 32)
        hipLaunchKernelGGL((fwd_kernel<PG64, MODE_GROWS>), dim3(ggrid), dim3(64), 0, stream, p);
    else
        hipLaunchKernelGGL((fwd_kernel<PG128, MODE_GROWS>), dim3(ggrid), dim3(128), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((merge_kernel<D, F32>), dim3(p.BH * p.n_global), dim3(64), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_forward(const FwdParams &p, int d, int f32, hipStream_t stream) {
    if (f32) {
        if (d == 64) return launch_impl<F32Path<64, 32, 256>, F32Path<64, 32, 64>, F32Path<64, 32, 128>, 64, true>(p, stream);
        return launch_impl<F32Path<128, 32, 256>, F32Path<128, 32, 64>, F32Path<128, 32, 128>, 128, true>(p, stream);
    }
    if (d == 64) return launch_impl<Bf16Path<64, 64, 256>, Bf16Path<64, 64, 64>, Bf16Path<64, 64, 128>, 64, false>(p, stream);
    return launch_impl<Bf16Path<128, 64, 256>, Bf16Path<128, 64, 64>, Bf16Path<128, 64, 128>, 128, false>(p, stream);
}

}  // namespace eea
