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
//  * bwd_dq: one workgroup per (query head, 128 rows); each wave keeps its 32
//    rows' Q and dO as operands and walks the visible 64-key tiles,
//    accumulating dQ^T += K^T dS^T.
// All products use v_mfma_f32_32x32x16_bf16 in the transposed forms of the
// forward pass, so each of them is one of the bf16 tile path's two operand
// patterns (row reads with the K swizzle, transpose reads with the V
// swizzle); a tile needed in both forms is copied into LDS in both layouts.
// Only band masks (causal, sliding and symmetric windows) are handled;
// the C ABI rejects global tokens for the backward pass.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_internal.h"
#include "attn_plan.h"
#include "attn_tiles.h"

namespace eea {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kBwdThreads = 256;   // 4 waves, one per SIMD (up to 512 registers each)

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// rowsum(dO * O) per query row: 8 lanes per row, 32 rows per workgroup.
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
    if (sub == 0 && r < rows) prm.delta[r] = acc;
}

// ---------------------------------------------------------------------------
// dK, dV: keys stationary, query tiles streamed.
// ---------------------------------------------------------------------------
// DIL: a dilated mask, run as one band attention per residue class of rows
// (the forward's decomposition); folded to 1 otherwise.
template <int D, bool DIL>
__global__ void __launch_bounds__(kBwdThreads) bwd_dkdv(const BwdParams prm) {
    typedef Bf16Path<D, kBwdThreads> P;
    constexpr int BQ = P::BN;               // query rows per streamed tile
    constexpr int BK = 32 * P::NW;          // keys per workgroup
    constexpr int MB = P::MB, DB = P::DB;

    // Q and dO of one query tile, each in both layouts, double-buffered; the
    // eight buffers are distinct objects and the loop is unrolled by two.
    __shared__ __attribute__((aligned(1024))) char qk0[P::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char qv0[P::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char ok0[P::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char ov0[P::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char qk1[P::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char qv1[P::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char ok1[P::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char ov1[P::TILE_BYTES];
    __shared__ __attribute__((aligned(16))) float s_lse[2][BQ];   // LSE * log2(e)
    __shared__ __attribute__((aligned(16))) float s_dl[2][BQ];    // rowsum(dO * O)

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ln = lane & 31, h = lane >> 5;
    const int H_kv = prm.H / prm.group;

    // work item: (K/V head, residue class, key tile)
    const int G = gridDim.x, bid = blockIdx.x;
    const int Lw = prm.xcd_remap_k ? (bid & 7) * (G >> 3) + (bid >> 3) : bid;
    const int dil = DIL ? prm.dil : 1;
    const int per_kv = dil * prm.num_kt;
    const int bkv = Lw / per_kv;
    const int rcls = (Lw - bkv * per_kv) / prm.num_kt;
    const int kt = Lw - bkv * per_kv - rcls * prm.num_kt;
    const int N = DIL ? (prm.N - rcls + dil - 1) / dil : prm.N;   // rows of this residue class
    if (kt * BK >= N) return;                                      // whole workgroup: a shorter class
    const Band band{N, prm.wl, prm.wr, prm.block, prm.cap};
    const int b = bkv / H_kv, kvh = bkv - b * H_kv;
    const long long cls_off = (long long)rcls * D;   // first row of the class
    const uint16_t *kh = static_cast<const uint16_t *>(prm.k) + (long long)bkv * prm.head_stride + cls_off;
    const uint16_t *vh = static_cast<const uint16_t *>(prm.v) + (long long)bkv * prm.head_stride + cls_off;

    typename P::Lane L;
    P::init_lane(L, lane, wave, dil);

    const int K0 = kt * BK;
    const int key = K0 + wave * 32 + ln;
    const bool kvalid = key < N;
    const int k0w = K0 + wave * 32, k1w = imin(N - 1, k0w + 31);
    const bool wave_active = k0w < N;
    // rows whose local interval holds this lane's key, and the query tiles
    // of the workgroup's keys (both bounds never decrease with the key)
    const int qlo = col_lo(band, key), qhi = col_hi(band, key);
    const int glo = col_lo(band, K0), ghi = col_hi(band, imin(N - 1, K0 + BK - 1));
    const int qt_lo = glo / BQ, nqt = ghi / BQ - qt_lo + 1;
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
    auto issue = [&](int t, char *qk, char *qv, char *ok, char *ov) __attribute__((always_inline)) {
        const long long bh = head_of(t);
        const int q0 = tile_of(t) * BQ;
        const uint16_t *qh = static_cast<const uint16_t *>(prm.q) + bh * prm.head_stride + cls_off;
        const uint16_t *gh = static_cast<const uint16_t *>(prm.dout) + bh * prm.head_stride + cls_off;
        P::issue_k(L, qh, N, qk, q0, dil);
        P::issue_v(L, qh, N, qv, q0, dil);
        P::issue_k(L, gh, N, ok, q0, dil);
        P::issue_v(L, gh, N, ov, q0, dil);
    };
    // per-row terms of tile t, loaded into registers now and stored to LDS later
    auto row_terms = [&](int t, float &l2, float &dl) __attribute__((always_inline)) {
        l2 = 0.f;
        dl = 0.f;
        if (tid < BQ) {
            const long long bh = head_of(t);
            const int i = tile_of(t) * BQ + tid;
            if (i < N) {
                const long long gi = bh * prm.N + rcls + (long long)i * dil;   // row in the stored sequence
                l2 = prm.lse[gi] * kLog2e;
                dl = prm.delta[gi];
            }
        }
    };

    auto step = [&](int t, const char *qk, const char *qv, const char *ok, const char *ov, char *nqk, char *nqv,
                    char *nok, char *nov, int sb) __attribute__((always_inline)) {
        const bool more = t + 1 < T;
        float nl2 = 0.f, ndl = 0.f;
        if (more) {
            issue(t + 1, nqk, nqv, nok, nov);
            row_terms(t + 1, nl2, ndl);
        }
        const int q0 = tile_of(t) * BQ;
        const int q1 = imin(N - 1, q0 + BQ - 1);
        int cl = wave_active ? classify(band, q0, q1, k0w, k1w) : TILE_SKIP;
        if (cl == TILE_FULL && q0 + BQ - 1 >= N) cl = TILE_EDGE;
        if (cl != TILE_SKIP) {
            f32x16 s[MB], dp[MB];
            P::scores(s, kf, L, qk);    // S  = Q K^T : lane = key, registers = query rows
            P::scores(dp, vf, L, ok);   // dP = dO V^T
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4 l4 = *reinterpret_cast<const f32x4 *>(&s_lse[sb][32 * mb + 8 * g + 4 * h]);
                    const f32x4 d4 = *reinterpret_cast<const f32x4 *>(&s_dl[sb][32 * mb + 8 * g + 4 * h]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * g + e;
                        float p = fast_exp2(__builtin_fmaf(s[mb][r], c, -l4[e]));
                        if (cl == TILE_EDGE) {
                            const int i = q0 + 32 * mb + acc_row(r, h);
                            p = ((i >= qlo) & (i <= qhi)) ? p : 0.f;
                        }
                        s[mb][r] = p;
                        dp[mb][r] = p * (dp[mb][r] - d4[e]);
                    }
                }
            typename P::PFrag pp, pd;
            P::pack_p(pp, s);
            P::pack_p(pd, dp);
            P::pv(dv, pp, L, ov);   // dV^T += dO^T P
            P::pv(dk, pd, L, qv);   // dK^T += Q^T dS
        }
        if (more && tid < BQ) {
            s_lse[sb ^ 1][tid] = nl2;
            s_dl[sb ^ 1][tid] = ndl;
        }
        wait_vmem();
        __syncthreads();
    };

    {
        issue(0, qk0, qv0, ok0, ov0);
        float l2, dl;
        row_terms(0, l2, dl);
        if (tid < BQ) {
            s_lse[0][tid] = l2;
            s_dl[0][tid] = dl;
        }
        wait_vmem();
        __syncthreads();
    }
    for (int t = 0; t < T; t += 2) {
        step(t, qk0, qv0, ok0, ov0, qk1, qv1, ok1, ov1, 0);
        if (t + 1 >= T) break;
        step(t + 1, qk1, qv1, ok1, ov1, qk0, qv0, ok0, ov0, 1);
    }

    if (!kvalid) return;
    uint16_t *dkh = static_cast<uint16_t *>(prm.dk) + (long long)bkv * prm.head_stride + cls_off;
    uint16_t *dvh = static_cast<uint16_t *>(prm.dv) + (long long)bkv * prm.head_stride + cls_off;
    P::store_out(dkh, key * dil, dk, prm.scale, h);
    P::store_out(dvh, key * dil, dv, 1.f, h);
}

// ---------------------------------------------------------------------------
// dQ: query rows stationary, key tiles streamed.
// ---------------------------------------------------------------------------
template <int D, bool DIL>
__global__ void __launch_bounds__(kBwdThreads) bwd_dq(const BwdParams prm) {
    typedef Bf16Path<D, kBwdThreads> P;
    constexpr int BN = P::BN;                 // keys per streamed tile
    constexpr int BM = 32 * P::NW;            // query rows per workgroup
    constexpr int MB = P::MB, DB = P::DB;

    __shared__ __attribute__((aligned(1024))) char kk0[P::TILE_BYTES];   // K, row-read layout
    __shared__ __attribute__((aligned(1024))) char kv0[P::TILE_BYTES];   // K, transpose-read layout
    __shared__ __attribute__((aligned(1024))) char vk0[P::TILE_BYTES];   // V, row-read layout
    __shared__ __attribute__((aligned(1024))) char kk1[P::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char kv1[P::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char vk1[P::TILE_BYTES];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ln = lane & 31, h = lane >> 5;
    // work item: (query head, residue class, query tile)
    const int G = gridDim.x, bid = blockIdx.x;
    const int Lw = prm.xcd_remap_q ? (bid & 7) * (G >> 3) + (bid >> 3) : bid;
    const int dil = DIL ? prm.dil : 1;
    const int per_head = dil * prm.num_qt;
    const int bh = Lw / per_head;
    const int rcls = (Lw - bh * per_head) / prm.num_qt;
    const int qi = Lw - bh * per_head - rcls * prm.num_qt;
    const int unit = prm.causal ? prm.num_qt - 1 - qi : qi;
    const int N = DIL ? (prm.N - rcls + dil - 1) / dil : prm.N;   // rows of this residue class
    if (unit * BM >= N) return;                                    // whole workgroup: a shorter class
    const Band band{N, prm.wl, prm.wr, prm.block, prm.cap};
    const long long cls_off = (long long)rcls * D;
    const long long kvb = (long long)(bh / prm.H) * (prm.H / prm.group) + (bh % prm.H) / prm.group;
    const uint16_t *qh = static_cast<const uint16_t *>(prm.q) + (long long)bh * prm.head_stride + cls_off;
    const uint16_t *gh = static_cast<const uint16_t *>(prm.dout) + (long long)bh * prm.head_stride + cls_off;
    const uint16_t *kh = static_cast<const uint16_t *>(prm.k) + kvb * prm.head_stride + cls_off;
    const uint16_t *vh = static_cast<const uint16_t *>(prm.v) + kvb * prm.head_stride + cls_off;

    typename P::Lane L;
    P::init_lane(L, lane, wave, dil);

    const int q0 = unit * BM;
    const int row = q0 + wave * 32 + ln;
    const bool valid = row < N;
    const int lo = row_lo(band, row), hi = row_hi(band, row);
    const int wr0 = q0 + wave * 32, wr1 = imin(N - 1, wr0 + 31);
    const bool wave_active = wr0 < N;
    int kt_lo, kt_hi;
    key_tile_range(band, q0, imin(N - 1, q0 + BM - 1), BN, &kt_lo, &kt_hi);

    typename P::QFrag qf, gf;   // this wave's Q and dO rows: B operands of S^T and dP^T
    P::load_q(qf, qh, row * dil, valid, h);
    P::load_q(gf, gh, row * dil, valid, h);
    const long long grow = (long long)bh * prm.N + rcls + (long long)row * dil;   // row in the stored sequence
    const float l2 = valid ? prm.lse[grow] * kLog2e : 0.f;
    const float dl = valid ? prm.delta[grow] : 0.f;
    const float c = prm.scale_log2;

    f32x16 dq[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) dq[db] = f32x16{};

    auto issue = [&](int kt, char *kk, char *kv, char *vk) __attribute__((always_inline)) {
        P::issue_k(L, kh, N, kk, kt * BN, dil);
        P::issue_v(L, kh, N, kv, kt * BN, dil);
        P::issue_k(L, vh, N, vk, kt * BN, dil);
    };
    auto step = [&](int kt, const char *kk, const char *kv, const char *vk, char *nkk, char *nkv, char *nvk)
        __attribute__((always_inline)) {
        if (kt < kt_hi) issue(kt + 1, nkk, nkv, nvk);
        const int k0 = kt * BN;
        const int cl = wave_active ? classify(band, wr0, wr1, k0, k0 + BN - 1) : TILE_SKIP;
        if (cl != TILE_SKIP) {
            f32x16 s[MB], dp[MB];
            P::scores(s, qf, L, kk);    // S^T  = K Q^T  : lane = query row, registers = keys
            P::scores(dp, gf, L, vk);   // dP^T = V dO^T
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float p = fast_exp2(__builtin_fmaf(s[mb][r], c, -l2));
                    if (cl == TILE_EDGE) {
                        const int j = k0 + mb * 32 + acc_row(r, h);
                        p = ((j >= lo) & (j <= hi)) ? p : 0.f;
                    }
                    dp[mb][r] = p * (dp[mb][r] - dl);
                }
            typename P::PFrag pd;
            P::pack_p(pd, dp);
            P::pv(dq, pd, L, kv);       // dQ^T += K^T dS^T
        }
        wait_vmem();
        __syncthreads();
    };

    if (kt_lo <= kt_hi) {
        issue(kt_lo, kk0, kv0, vk0);
        wait_vmem();
        __syncthreads();
        for (int kt = kt_lo; kt <= kt_hi; kt += 2) {
            step(kt, kk0, kv0, vk0, kk1, kv1, vk1);
            if (kt + 1 > kt_hi) break;
            step(kt + 1, kk1, kv1, vk1, kk0, kv0, vk0);
        }
    }
    if (!valid) return;
    uint16_t *dqh = static_cast<uint16_t *>(prm.dq) + (long long)bh * prm.head_stride + cls_off;
    P::store_out(dqh, row * dil, dq, prm.scale, h);
}

int bwd_tile_q(int d) { (void)d; return 32 * (kBwdThreads / 64); }
int bwd_tile_k(int d) { (void)d; return 32 * (kBwdThreads / 64); }

template <int D>
static hipError_t launch_bwd_impl(const BwdParams &p0, hipStream_t stream) {
    BwdParams p = p0;
    const long long rows = (long long)p.BH * p.N;
    hipLaunchKernelGGL((bwd_delta<D>), dim3((unsigned)((rows + 31) / 32)), dim3(kBwdThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int kgrid = (p.BH / p.group) * p.dil * p.num_kt;
    p.xcd_remap_k = kgrid % 8 == 0;
    if (p.dil > 1)
        hipLaunchKernelGGL((bwd_dkdv<D, true>), dim3(kgrid), dim3(kBwdThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((bwd_dkdv<D, false>), dim3(kgrid), dim3(kBwdThreads), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int qgrid = p.BH * p.dil * p.num_qt;
    p.xcd_remap_q = qgrid % 8 == 0;
    if (p.dil > 1)
        hipLaunchKernelGGL((bwd_dq<D, true>), dim3(qgrid), dim3(kBwdThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((bwd_dq<D, false>), dim3(qgrid), dim3(kBwdThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_backward(const BwdParams &p, int d, hipStream_t stream) {
    return d == 64 ? launch_bwd_impl<64>(p, stream) : launch_bwd_impl<128>(p, stream);
}

}  // namespace eea
