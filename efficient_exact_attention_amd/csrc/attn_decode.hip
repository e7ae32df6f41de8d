// attn_decode.hip - gfx950 kernels for decoding with a key/value cache: the
// newest tokens' queries attend over the keys and values kept for every
// earlier token (week-17 lecture notes, per-token inference cost with a KV
// cache; "Beyond attention", the rolling cache of a sliding window).
//
// The work is bound by reading the cache from HBM, so it is split over the
// cache ("split-KV"): a workgroup takes every query row that reads one K/V
// head (a group of query heads times the Nq newest tokens, up to 64 rows)
// against one chunk of cache slots, streams the chunk's K and V tiles into
// LDS, and leaves an unnormalised partial (output, running max, normaliser)
// per row; a merge kernel combines the chunks with the same rescaling
// identity as the online softmax. Slots map to positions either directly
// (contiguous cache) or modulo the cache size (rolling cache: the last S
// positions, a newer one overwriting the oldest).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <climits>
#include <type_traits>
#include <utility>

#include "attn_internal.h"
#include "attn_plan.h"
#include "attn_tiles.h"

namespace eea {


// s_waitcnt vmcnt(C) leaving the other counters alone (gfx9 encoding).
template <int C>
__device__ __forceinline__ void wait_vm() {
    static_assert(C >= 0 && C < 64, "vmcnt holds 6 bits");
    __builtin_amdgcn_s_waitcnt((C & 15) | ((C >> 4) << 14) | 0x0F70);
}

// Wait until at most `younger` tiles of LPT loads each are still in flight
// (younger is wave-uniform, 0 .. N).
template <int LPT, int N>
__device__ __forceinline__ void wait_tiles(int younger) {
    if constexpr (N == 0) {
        wait_vm<0>();
    } else {
        if (younger >= N) wait_vm<N * LPT>();
        else wait_tiles<LPT, N - 1>(younger);
    }
}

// f(integral_constant<int, 0>) .. f(integral_constant<int, N-1>), unrolled.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Slot -> position. With sl = (L-1) mod S the slot of the newest position,
// a rolling cache holds position s + off in slots s <= sl and s + off - S
// in slots s > sl, where off = L-1-sl (a negative result: the slot holds
// no position yet). A contiguous cache is the case off = 0, sl >= every s.
struct SlotMap {
    int off, sl, S;
    __device__ __forceinline__ int pos(int s) const { return s + off - (s > sl ? S : 0); }
};

// KS2 (for at most 64 query rows): waves 2w and 2w+1 hold the same 32 rows
// and take the first and the second 32-key block of every tile, each with an
// online softmax of its own, combined at the end; every wave then computes.
// Otherwise each wave holds 32 rows of its own against whole tiles.
template <int D, bool KS2>
__global__ void __launch_bounds__(kDecThreads) decode_kernel(const DecParams prm) {
    typedef Bf16Path<D, kDecThreads> P;
    constexpr int BN = P::BN, MB = P::MB, DB = P::DB, TB = P::TILE_BYTES;
    constexpr int NB = KS2 ? 1 : MB;   // 32-key blocks a wave takes per tile
    // Pipeline stages, each one K tile and one V tile: 5 (d=128) or 8
    // (d=64). Every stage is an LDS variable of its own and the loop below
    // names stages by constants, so the compiler can tell that a read of one
    // stage does not alias the copies in flight to the others (it would
    // otherwise wait for every copy before each LDS read).
    constexpr int NS = kDecLds / (2 * TB) < 8 ? kDecLds / (2 * TB) : 8;
    constexpr int LPT = 2 * P::SPW;          // copies per wave per tile (K and V)
    static_assert((NS - 2) * LPT < 64, "in-flight copies must fit the vmcnt counter");
    __shared__ __attribute__((aligned(1024))) char st0[2 * TB];
    __shared__ __attribute__((aligned(1024))) char st1[2 * TB];
    __shared__ __attribute__((aligned(1024))) char st2[2 * TB];
    __shared__ __attribute__((aligned(1024))) char st3[2 * TB];
    __shared__ __attribute__((aligned(1024))) char st4[2 * TB];
    __shared__ __attribute__((aligned(1024))) char st5[2 * TB];
    __shared__ __attribute__((aligned(1024))) char st6[2 * TB];
    __shared__ __attribute__((aligned(1024))) char st7[2 * TB];
    auto stage = [&](auto I) __attribute__((always_inline)) -> char * {
        constexpr int i = decltype(I)::value % NS;
        if constexpr (i == 0) return st0;
        else if constexpr (i == 1) return st1;
        else if constexpr (i == 2) return st2;
        else if constexpr (i == 3) return st3;
        else if constexpr (i == 4) return st4;
        else if constexpr (i == 5) return st5;
        else if constexpr (i == 6) return st6;
        else return st7;
    };

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ln = lane & 31, h = lane >> 5;

    // work item: (batch entry, K/V head, row group, chunk)
    const int c = blockIdx.x % prm.chunks;
    const int rest = blockIdx.x / prm.chunks;
    const int rg = rest % prm.nrg;
    const int bkv = rest / prm.nrg;
    const int b = bkv / prm.H_kv, kvh = bkv - b * prm.H_kv;
    const int S = prm.S, Nq = prm.Nq;
    int L = prm.seq_len[b];
    L = L < Nq ? Nq : L;
    if (!prm.rolling && L > S) L = S;

    // this lane's query row (rows past R compute nothing and store nothing)
    const int rw = KS2 ? wave >> 1 : wave;   // which 32 rows
    const int kb = KS2 ? wave & 1 : 0;       // first key block taken
    const int r = rg * kDecRows + rw * 32 + ln;
    const bool valid = r < prm.R;
    const bool active = rg * kDecRows + rw * 32 < prm.R;   // wave-uniform
    const int hq = kvh * prm.group + (valid ? r / Nq : 0);
    const int t = valid ? r % Nq : 0;
    const int pos = L - Nq + t;
    const int lo = prm.win < 0 ? 0 : imax(0, pos - prm.win);   // oldest visible position
    const long long grow = ((long long)b * prm.H + hq) * Nq + t;   // row of out / lse
    const uint16_t *qrow = static_cast<const uint16_t *>(prm.q) + grow * D;
    // slots >= min(S, L) hold no position of this sequence (a cache that is
    // not yet full may hold anything there, NaN included): the copies treat
    // them as past the end of the buffer, which reads zeros
    const int Nb = imin(S, L);
    const uint16_t *kh = static_cast<const uint16_t *>(prm.kc) + (long long)bkv * S * D;
    const uint16_t *vh = static_cast<const uint16_t *>(prm.vc) + (long long)bkv * S * D;

    SlotMap map;
    if (prm.rolling) {
        map.sl = (L - 1) % S;
        map.off = L - 1 - map.sl;
    } else {
        map.sl = INT_MAX;
        map.off = 0;
    }
    map.S = S;
    // every row of the workgroup sees positions [wlo, whi] at least
    const int whi = L - Nq;
    const int wlo = prm.win < 0 ? 0 : imax(0, L - 1 - prm.win);

    // tiles this chunk visits: a contiguous cache holds positions 0..L-1
    // in slots 0..L-1, of which the rows see at most the last Nq + win; a
    // rolling cache may hold a visible position in any of its min(S, L)
    // filled slots. The chunks split this sequence's tiles evenly.
    const int s_lo = (!prm.rolling && prm.win >= 0) ? imax(0, L - Nq - prm.win) : 0;
    const int f_lo = s_lo / BN, f_n = (Nb - 1) / BN - f_lo + 1;
    const int per = (f_n + prm.chunks - 1) / prm.chunks;
    const int t_lo = f_lo + c * per, t_hi = imin(f_lo + f_n, t_lo + per) - 1;

    typename P::Lane Ln;
    P::init_lane(Ln, lane, wave);
    typename P::QFrag qf;
    P::load_q(qf, qrow, 0, valid, h);

    const float cl2 = prm.scale_log2;
    float m = EEA_NEG_INF, lpart = 0.f;
    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x16{};

    auto issue = [&](int tile, char *buf) __attribute__((always_inline)) {
        P::issue_k(Ln, kh, Nb, buf, tile * BN);
        P::issue_v(Ln, vh, Nb, buf + TB, tile * BN);
    };

    auto compute = [&](int tile, const char *kr, const char *vr) __attribute__((always_inline)) {
        f32x16 s[NB];
        if constexpr (KS2) {
            s[0] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < P::KS; ++ks) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(kr + Ln.krd[ks] + kb * 32 * P::ROWB);
                s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf.x[ks], s[0], 0, 0, 0);
            }
        } else {
            P::scores(s, qf, Ln, kr);
        }
        // interior tile: one run of positions (no wrap inside), all of them
        // seen by every row of the workgroup
        const int s0 = tile * BN, p0 = map.pos(s0);
        const bool interior = s0 + BN <= S && !(s0 <= map.sl && map.sl < s0 + BN - 1) && p0 >= wlo &&
                              p0 + BN - 1 <= whi;
        float mx = EEA_NEG_INF;
        if (interior) {   // rows past R score zeros here: finite, never stored
#pragma unroll
            for (int mb = 0; mb < NB; ++mb)
#pragma unroll
                for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[mb][e]);
        } else {
#pragma unroll
            for (int mb = 0; mb < NB; ++mb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int slot = s0 + (kb + mb) * 32 + acc_row(e, h);
                    const int p = map.pos(slot);
                    const bool vis = valid & (slot < S) & (p >= lo) & (p <= pos);
                    s[mb][e] = vis ? s[mb][e] : EEA_NEG_INF;
                    mx = fmaxf(mx, s[mb][e]);
                }
        }
        mx = max_across_halves(mx);
        const float mnew = fmaxf(m, mx * cl2);
        const float alpha = (mnew == EEA_NEG_INF) ? 1.f : fast_exp2(m - mnew);   // m = -inf gives 0
        m = mnew;
        const float mu = (m == EEA_NEG_INF) ? 0.f : m;
        float sum = 0.f;
#pragma unroll
        for (int mb = 0; mb < NB; ++mb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float pw = fast_exp2(__builtin_fmaf(s[mb][e], cl2, -mu));
                s[mb][e] = pw;
                sum += pw;
            }
        lpart = lpart * alpha + sum;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= alpha;
        if constexpr (KS2) {   // the block's two 16-key steps of P V
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                f32x8 x = {s[0][8 * j + 0], s[0][8 * j + 1], s[0][8 * j + 2], s[0][8 * j + 3],
                           s[0][8 * j + 4], s[0][8 * j + 5], s[0][8 * j + 6], s[0][8 * j + 7]};
                const bf16x8 pj = __builtin_convertvector(x, bf16x8);
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(P::v_operand(Ln, vr, db, 2 * kb + j), pj, o[db],
                                                                    0, 0, 0);
            }
        } else {
            typename P::PFrag pf;
            P::pack_p(pf, s);
            P::pv(o, pf, Ln, vr);
        }
    };

    // NS-stage pipeline: tiles t_lo .. t_lo+NS-2 are in flight before the
    // loop; each iteration waits for its tile, then refills the stage the
    // previous iteration computed on (every wave has left it: barrier)
    static_for<NS - 1>([&](auto I) __attribute__((always_inline)) {
        if (t_lo + I <= t_hi) issue(t_lo + I, stage(I));
    });
    for (int tile0 = t_lo; tile0 <= t_hi; tile0 += NS) {
        static_for<NS>([&](auto I) __attribute__((always_inline)) {
            const int tile = tile0 + I;
            if (tile <= t_hi) {
                wait_tiles<LPT, NS - 2>(imin(NS - 2, t_hi - tile));
                __syncthreads();
                if (tile + NS - 1 <= t_hi)
                    issue(tile + NS - 1, stage(std::integral_constant<int, I + NS - 1>{}));
                debug_sync();
                if (active) compute(tile, stage(I), stage(I) + TB);
            }
        });
    }

    float l = sum_across_halves(lpart);
    if constexpr (KS2) {   // fold the second key block's state into the first's
        __syncthreads();   // every wave is done with the stages
        float *xs = reinterpret_cast<float *>(rw == 0 ? st0 : st1);
        constexpr int NO = DB * 16;
        if (kb == 1 && active) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) xs[(db * 16 + e) * 64 + lane] = o[db][e];
            xs[NO * 64 + lane] = m;
            xs[(NO + 1) * 64 + lane] = l;
        }
        __syncthreads();
        if (kb == 1 || !active) return;
        const float m1 = xs[NO * 64 + lane], l1 = xs[(NO + 1) * 64 + lane];
        const float M = fmaxf(m, m1);
        const float a0 = m == EEA_NEG_INF ? 0.f : fast_exp2(m - M);
        const float a1 = m1 == EEA_NEG_INF ? 0.f : fast_exp2(m1 - M);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[db][e] = o[db][e] * a0 + xs[(db * 16 + e) * 64 + lane] * a1;
        l = l * a0 + l1 * a1;
        m = M;
    }
    if (!valid) return;
    if (prm.chunks == 1) {   // the only chunk: finish the row here
        P::store_out(static_cast<uint16_t *>(prm.out) + grow * D, 0, o, l > 0.f ? 1.f / l : 0.f, h);
        if (h == 0) prm.lse[grow] = l > 0.f ? (m + __log2f(l)) * kLn2 : EEA_NEG_INF;
        return;
    }
    float *dst = prm.part + (grow * prm.chunks + c) * (D + 2);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            float *pp = dst + db * 32 + 8 * g + 4 * h;
            pp[0] = o[db][4 * g + 0];
            pp[1] = o[db][4 * g + 1];
            pp[2] = o[db][4 * g + 2];
            pp[3] = o[db][4 * g + 3];
        }
    if (h == 0) {
        dst[D] = m;
        dst[D + 1] = l;
    }
}

// One wave per output row: weight each chunk's partial by exp2(m_c - M)
// (M the largest m_c), sum, and divide by the weighted normalisers.
template <int D>
__global__ void __launch_bounds__(64) decode_merge(const DecParams prm) {
    __shared__ float wsh[kDecMaxChunks];
    const int lane = threadIdx.x;
    const long long grow = blockIdx.x;   // over B * H * Nq
    const int C = prm.chunks;
    const float *src = prm.part + grow * C * (D + 2);
    float M = EEA_NEG_INF;
    for (int ci = lane; ci < C; ci += 64) M = fmaxf(M, src[ci * (D + 2) + D]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    float Ls = 0.f;
    for (int ci = lane; ci < C; ci += 64) {
        const float mc = src[ci * (D + 2) + D];
        const float w = mc == EEA_NEG_INF ? 0.f : fast_exp2(mc - M);
        wsh[ci] = w;
        Ls += w * src[ci * (D + 2) + D + 1];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) Ls += __shfl_xor(Ls, off);
    __syncthreads();
    const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
    constexpr int PER = D / 64;
    float acc[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) acc[j] = 0.f;
#pragma unroll 4
    for (int ci = 0; ci < C; ++ci) {
        const float w = wsh[ci];
#pragma unroll
        for (int j = 0; j < PER; ++j) acc[j] += src[ci * (D + 2) + lane + 64 * j] * w;
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) static_cast<__bf16 *>(prm.out)[grow * D + lane + 64 * j] = (__bf16)(acc[j] * inv);
    if (lane == 0) prm.lse[grow] = Ls > 0.f ? (M + __log2f(Ls)) * kLn2 : EEA_NEG_INF;
}

template <int D>
static hipError_t launch_dec_impl(const DecParams &p, hipStream_t stream) {
    const long long grid = (long long)p.B * p.H_kv * p.nrg * p.chunks;
    if (p.R <= 64)
        hipLaunchKernelGGL((decode_kernel<D, true>), dim3((unsigned)grid), dim3(kDecThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((decode_kernel<D, false>), dim3((unsigned)grid), dim3(kDecThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.chunks == 1) return e;
    hipLaunchKernelGGL((decode_merge<D>), dim3((unsigned)((long long)p.B * p.H * p.Nq)), dim3(64), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_decode(const DecParams &p, int d, hipStream_t stream) {
    return d == 64 ? launch_dec_impl<64>(p, stream) : launch_dec_impl<128>(p, stream);
}

}  // namespace eea
