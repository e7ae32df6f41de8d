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

#include "attn_internal.h"
#include "attn_plan.h"
#include "attn_tiles.h"

namespace eea {

constexpr int kDecThreads = 128;   // two waves, kDecRows query rows

// Position held by cache slot s when the sequence has length L (negative:
// the slot holds no position of this sequence). A rolling cache keeps
// position p in slot p % S, so slot s holds the newest p <= L-1 with
// p = s (mod S).
__device__ __forceinline__ int slot_position(int s, int L, int S, int rolling) {
    if (s >= S) return -1;
    if (!rolling) return s < L ? s : -1;
    const int x = L - 1 - s;
    return L - 1 - ((x % S) + S) % S;
}

template <int D>
__global__ void __launch_bounds__(kDecThreads) decode_kernel(const DecParams prm) {
    typedef Bf16Path<D, kDecThreads> P;
    constexpr int BN = P::BN, MB = P::MB, DB = P::DB;
    __shared__ __attribute__((aligned(1024))) char kb0[P::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char kb1[P::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char vb0[P::TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char vb1[P::TILE_BYTES];

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

    // this lane's query row
    const int r = rg * kDecRows + wave * 32 + ln;
    const bool valid = r < prm.R;
    const int hq = kvh * prm.group + (valid ? r / Nq : 0);
    const int t = valid ? r % Nq : 0;
    const int pos = L - Nq + t;
    const long long grow = ((long long)b * prm.H + hq) * Nq + t;   // row of out / lse
    const uint16_t *qrow = static_cast<const uint16_t *>(prm.q) + grow * D;
    // the waves whose 32 rows are all past the last query row still share
    // the tile copies and barriers but skip the arithmetic
    const bool active = rg * kDecRows + wave * 32 < prm.R;
    // slots >= min(S, L) hold no position of this sequence (a cache that
    // is not yet full may hold anything there, NaN included): the copies
    // treat them as past the end of the buffer, which reads zeros
    const int Nb = imin(S, L);
    const uint16_t *kh = static_cast<const uint16_t *>(prm.kc) + (long long)bkv * S * D;
    const uint16_t *vh = static_cast<const uint16_t *>(prm.vc) + (long long)bkv * S * D;

    // slots this chunk must visit: a contiguous cache holds positions
    // 0..L-1 in slots 0..L-1, of which the rows see at most the last
    // Nq + win; a rolling cache may hold a visible position in any slot
    int s_lo = 0, s_hi = prm.rolling ? imin(S, L) - 1 : L - 1;
    if (!prm.rolling && prm.win >= 0) s_lo = imax(0, L - Nq - prm.win);
    const int c0 = c * prm.chunk_tiles * BN;
    s_lo = imax(s_lo, c0);
    s_hi = imin(s_hi, imin(S - 1, c0 + prm.chunk_tiles * BN - 1));
    const int t_lo = s_lo / BN, t_hi = s_hi >= s_lo ? s_hi / BN : t_lo - 1;

    typename P::Lane Ln;
    P::init_lane(Ln, lane, wave);
    typename P::QFrag qf;
    P::load_q(qf, qrow, 0, valid, h);

    const float cl2 = prm.scale_log2;
    float m = EEA_NEG_INF, lpart = 0.f;
    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x16{};

    auto step = [&](int tile, const char *kr, const char *vr, char *kw, char *vw) __attribute__((always_inline)) {
        if (tile < t_hi) {
            P::issue_k(Ln, kh, Nb, kw, (tile + 1) * BN);
            P::issue_v(Ln, vh, Nb, vw, (tile + 1) * BN);
        }
        if (active) {
            f32x16 s[MB];
            P::scores(s, qf, Ln, kr);
            float mx = EEA_NEG_INF;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int slot = tile * BN + mb * 32 + acc_row(e, h);
                    const int p = slot_position(slot, L, S, prm.rolling);
                    const bool vis = valid & (p >= 0) & (p <= pos) & ((prm.win < 0) | (p >= pos - prm.win));
                    s[mb][e] = vis ? s[mb][e] : EEA_NEG_INF;
                    mx = fmaxf(mx, s[mb][e]);
                }
            mx = max_across_halves(mx);
            const float mnew = fmaxf(m, mx * cl2);
            const float alpha = (mnew == EEA_NEG_INF) ? 1.f : fast_exp2(m - mnew);   // m = -inf gives 0
            m = mnew;
            const float mu = (m == EEA_NEG_INF) ? 0.f : m;
            float sum = 0.f;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float pw = fast_exp2(__builtin_fmaf(s[mb][e], cl2, -mu));
                    s[mb][e] = pw;
                    sum += pw;
                }
            lpart = lpart * alpha + sum;
#pragma unroll
            for (int db = 0; db < DB; ++db) o[db] *= alpha;
            typename P::PFrag pf;
            P::pack_p(pf, s);
            P::pv(o, pf, Ln, vr);
        }
        wait_vmem();
        __syncthreads();
    };

    if (t_lo <= t_hi) {
        P::issue_k(Ln, kh, Nb, kb0, t_lo * BN);
        P::issue_v(Ln, vh, Nb, vb0, t_lo * BN);
        wait_vmem();
        __syncthreads();
        for (int tile = t_lo; tile <= t_hi; tile += 2) {
            step(tile, kb0, vb0, kb1, vb1);
            if (tile + 1 > t_hi) break;
            step(tile + 1, kb1, vb1, kb0, vb0);
        }
    }

    const float l = sum_across_halves(lpart);
    if (!valid) return;
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

// One wave per output row: combine the chunks' partials.
template <int D>
__global__ void __launch_bounds__(64) decode_merge(const DecParams prm) {
    const long long grow = blockIdx.x;   // over B * H * Nq
    const float *src = prm.part + grow * prm.chunks * (D + 2);
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
        static_cast<__bf16 *>(prm.out)[grow * D + dd] = (__bf16)(acc * inv);
    }
    if (threadIdx.x == 0) prm.lse[grow] = Lsum > 0.f ? (M + __log2f(Lsum)) * kLn2 : EEA_NEG_INF;
}

int decode_chunks(int B, int H_kv, int nrg, int S, int *chunk_tiles) {
    const int tiles = (S + 63) / 64;
    const long long units = (long long)B * H_kv * nrg;
    long long target = (2048 + units - 1) / units;   // a few thousand workgroups
    if (target < 1) target = 1;
    if (target > tiles) target = tiles;
    int ct = (int)((tiles + target - 1) / target);
    if (ct < 1) ct = 1;
    if (chunk_tiles) *chunk_tiles = ct;
    return (tiles + ct - 1) / ct;
}

template <int D>
static hipError_t launch_dec_impl(const DecParams &p, hipStream_t stream) {
    const long long grid = (long long)p.B * p.H_kv * p.nrg * p.chunks;
    hipLaunchKernelGGL((decode_kernel<D>), dim3((unsigned)grid), dim3(kDecThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_merge<D>), dim3((unsigned)((long long)p.B * p.H * p.Nq)), dim3(64), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_decode(const DecParams &p, int d, hipStream_t stream) {
    return d == 64 ? launch_dec_impl<64>(p, stream) : launch_dec_impl<128>(p, stream);
}

}  // namespace eea
