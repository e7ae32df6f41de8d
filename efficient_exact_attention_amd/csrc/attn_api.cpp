// attn_api.cpp - the C ABI of include/attn.h: argument validation, error
// reporting, workspace handling and the host-side tile planner.
//
// Every argument is checked before the first HIP call, so every error path
// can be exercised on a machine without a GPU.
#include "attn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "attn_internal.h"
#include "attn_plan.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

// Library-owned device scratch, one buffer per device and kind (the
// forward's global-row partials, the backward's row terms and split-pass
// partials, decoding's per-chunk partials). A call without a caller
// workspace runs under the mutex: its stream first waits on the event that
// the previous user of the buffer recorded, then its kernels are enqueued,
// then it records the event itself. Calls on different streams therefore
// use the buffer one after another, never at the same time.
enum ScratchKind { SCR_FWD = 0, SCR_BWD = 1, SCR_DEC = 2, SCR_KINDS = 3 };

struct DeviceSlot {
    int arch_checked = 0;
    int arch_ok = 0;
    void *scratch[SCR_KINDS] = {nullptr, nullptr, nullptr};
    size_t scratch_bytes[SCR_KINDS] = {0, 0, 0};
    hipEvent_t last_use[SCR_KINDS] = {nullptr, nullptr, nullptr};
};
std::mutex g_mu;
std::vector<DeviceSlot> g_dev;

DeviceSlot &slot(int dev) {
    if ((int)g_dev.size() <= dev) g_dev.resize(dev + 1);
    return g_dev[dev];
}

// Current device, checked to be gfx950 once. Caller holds g_mu.
int current_device_locked(DeviceSlot **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(ATTN_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
    DeviceSlot &s = slot(dev);
    if (!s.arch_checked) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return fail(ATTN_ERR_DEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
        s.arch_ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        s.arch_checked = 1;
    }
    if (!s.arch_ok) return fail(ATTN_ERR_UNSUPPORTED, "device %d is not gfx950 (MI355X)", dev);
    *out = &s;
    return ATTN_OK;
}

// Enqueue launch(buf) on `stream`. With caller_ws set (or need == 0) the
// kernels run on that memory and no library state is touched beyond the
// device check. Otherwise buf is the library scratch of `kind`, grown to at
// least `need` bytes (the old buffer is freed only after its last user's
// event has completed) and ordered against its previous user as described
// at DeviceSlot. launch returns a hipError_t.
template <class F>
int run_on_device(int kind, size_t need, void *caller_ws, hipStream_t stream, F &&launch) {
    std::unique_lock<std::mutex> lk(g_mu);
    DeviceSlot *s = nullptr;
    int rc = current_device_locked(&s);
    if (rc != ATTN_OK) return rc;
    hipError_t e;
    if (caller_ws || need == 0) {
        lk.unlock();
        e = launch(caller_ws);
        if (e != hipSuccess) return fail(ATTN_ERR_DEVICE, "kernel launch: %s", hipGetErrorString(e));
        return ATTN_OK;
    }
    hipEvent_t &ev = s->last_use[kind];
    if (!ev) {
        e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
        if (e != hipSuccess) {
            ev = nullptr;
            return fail(ATTN_ERR_DEVICE, "hipEventCreateWithFlags: %s", hipGetErrorString(e));
        }
    }
    void *&ptr = s->scratch[kind];
    size_t &bytes = s->scratch_bytes[kind];
    if (bytes < need) {
        if (ptr) {
            e = hipEventSynchronize(ev);   // the last call that used the old buffer is done
            if (e == hipSuccess) e = hipFree(ptr);
            ptr = nullptr;
            bytes = 0;
            if (e != hipSuccess) return fail(ATTN_ERR_DEVICE, "releasing the old scratch: %s", hipGetErrorString(e));
        }
        e = hipMalloc(&ptr, need);
        if (e != hipSuccess) {
            ptr = nullptr;
            return fail(ATTN_ERR_DEVICE, "hipMalloc(%zu): %s", need, hipGetErrorString(e));
        }
        bytes = need;
    }
    e = hipStreamWaitEvent(stream, ev, 0);   // after the previous user (a no-op the first time)
    if (e != hipSuccess) return fail(ATTN_ERR_DEVICE, "hipStreamWaitEvent: %s", hipGetErrorString(e));
    e = launch(ptr);
    if (e != hipSuccess) return fail(ATTN_ERR_DEVICE, "kernel launch: %s", hipGetErrorString(e));
    e = hipEventRecord(ev, stream);
    if (e != hipSuccess) return fail(ATTN_ERR_DEVICE, "hipEventRecord: %s", hipGetErrorString(e));
    return ATTN_OK;
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

// Largest split-key workspace over both element types.
size_t workspace_for(int BH, int N, int d, int ng) {
    size_t best = 0;
    for (int f32 = 0; f32 < 2; ++f32) {
        int ct = 0;
        int chunks = eea::global_chunks(BH, N, d, f32, &ct);
        size_t b = (size_t)BH * ng * chunks * (d + 2) * sizeof(float);
        best = std::max(best, b);
    }
    // global rows fused into the bf16 band pass: one partial per query tile
    // of 128 rows
    const int nqt = (N + 127) / 128;
    best = std::max(best, (size_t)BH * ng * (size_t)nqt * (d + 2) * sizeof(float));
    return best;
}

}  // namespace

extern "C" {

const char *attn_version(void) { return "efficient_exact_attention_amd 0.1.0 (gfx950)"; }

const char *attn_last_error(void) { return g_err.c_str(); }

int attn_tile_shape(int d, int dtype, int *bm, int *bn) {
    if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "head size d=%d is not supported (64 or 128)", d);
    if (dtype != ATTN_BF16 && dtype != ATTN_F32) return fail(ATTN_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    if (bm) *bm = eea::tile_bm(d, dtype == ATTN_F32);
    if (bn) *bn = eea::tile_bn(d, dtype == ATTN_F32);
    return ATTN_OK;
}

size_t attn_workspace_bytes(int B, int H, int N, int d, int n_global) {
    if (B <= 0 || H <= 0 || N <= 0 || n_global <= 0 || n_global > eea::kMaxGlobal) return 0;
    if (d != 64 && d != 128) return 0;
    if ((long long)B * H > INT_MAX) return 0;
    return workspace_for(B * H, N, d, n_global);
}

static int check_globals(const int *global_idx, int n_global, int N, std::vector<int> &sorted) {
    if (n_global < 0) return fail(ATTN_ERR_INVALID_ARG, "n_global=%d is negative", n_global);
    if (n_global > eea::kMaxGlobal)
        return fail(ATTN_ERR_UNSUPPORTED, "n_global=%d exceeds the supported maximum of %d", n_global,
                    eea::kMaxGlobal);
    if (n_global > 0 && !global_idx) return fail(ATTN_ERR_INVALID_ARG, "global_idx is NULL with n_global=%d", n_global);
    sorted.assign(global_idx, global_idx + n_global);
    std::sort(sorted.begin(), sorted.end());
    for (int t = 0; t < n_global; ++t) {
        if (sorted[t] < 0 || sorted[t] >= N)
            return fail(ATTN_ERR_INVALID_ARG, "global index %d is outside [0, %d)", sorted[t], N);
        if (t > 0 && sorted[t] == sorted[t - 1])
            return fail(ATTN_ERR_INVALID_ARG, "global index %d is listed twice", sorted[t]);
    }
    return ATTN_OK;
}

}  // extern "C"

namespace {

// A validated, normalised mask.
struct MaskSpec {
    int causal = 0;
    int dil = 1;          // dilation (1: off)
    eea::Band band{};     // window or block rule; with dil > 1 the window counts steps
    std::vector<int> G;   // sorted global positions
    int ng = 0;           // globals in use (0 when the band already holds every visible key)
    int stride = 0;       // log-spaced strided rule (0: off)
    int rand_block = 0;   // random-block rule (0: off)
    int n_rand = 0;
    const int *rand_idx = nullptr;   // device key-block lists
    bool extra() const { return stride > 0 || rand_block > 0; }
};

constexpr int kMaxRand = 16;   // key blocks listed per query block

// The strided and random-block fields of an attn_mask, validated against the
// already resolved local rule.
int resolve_extras(int N, const attn_mask *mask, MaskSpec &m) {
    if (!mask) return ATTN_OK;
    if (mask->stride < 0) return fail(ATTN_ERR_INVALID_ARG, "stride=%d must be >= 0", mask->stride);
    if (mask->rand_block < 0) return fail(ATTN_ERR_INVALID_ARG, "rand_block=%d must be >= 0", mask->rand_block);
    if (mask->stride == 0 && mask->rand_block == 0) return ATTN_OK;
    if (mask->stride > 0 && mask->rand_block > 0)
        return fail(ATTN_ERR_UNSUPPORTED, "the strided and random-block rules cannot be combined");
    if (m.band.block > 0 || m.dil > 1)
        return fail(ATTN_ERR_UNSUPPORTED, "the strided and random-block rules combine with a window only");
    if (mask->rand_block > 0) {
        if (mask->rand_block % 32 != 0)
            return fail(ATTN_ERR_UNSUPPORTED, "rand_block=%d must be a multiple of 32", mask->rand_block);
        if (mask->n_rand < 1 || mask->n_rand > kMaxRand)
            return fail(ATTN_ERR_INVALID_ARG, "n_rand=%d must be in [1, %d]", mask->n_rand, kMaxRand);
        if (!mask->rand_idx) return fail(ATTN_ERR_INVALID_ARG, "rand_idx is NULL");
        if ((uintptr_t)mask->rand_idx & 3) return fail(ATTN_ERR_INVALID_ARG, "rand_idx must be 4-byte aligned");
    }
    // a band that already holds every visible key leaves nothing to add
    if (eea::band_is_everything(m.band, m.causal)) return ATTN_OK;
    if (mask->stride > 0 && mask->stride < N) m.stride = mask->stride;
    if (mask->rand_block > 0) {
        m.rand_block = mask->rand_block;
        m.n_rand = mask->n_rand;
        m.rand_idx = mask->rand_idx;
    }
    return ATTN_OK;
}

int resolve_mask(int N, int causal, int win_left, int win_right, int block, int dilation, const int *global_idx,
                 int n_global, MaskSpec &m) {
    if (causal != 0 && causal != 1) return fail(ATTN_ERR_INVALID_ARG, "causal=%d must be 0 or 1", causal);
    if (win_left < -1 || win_right < -1)
        return fail(ATTN_ERR_INVALID_ARG, "window (%d, %d) must be >= -1", win_left, win_right);
    if (block < 0) return fail(ATTN_ERR_INVALID_ARG, "block=%d must be >= 0", block);
    if (dilation < 0) return fail(ATTN_ERR_INVALID_ARG, "dilation=%d must be >= 0", dilation);
    if (block > 0 && (win_left != -1 || win_right != -1))
        return fail(ATTN_ERR_INVALID_ARG, "the block rule replaces the window: win_left and win_right must be -1");
    if (block > 0 && dilation > 1)
        return fail(ATTN_ERR_UNSUPPORTED, "block-sparse and dilated rules cannot be combined");
    int rc = check_globals(global_idx, n_global, N, m.G);
    if (rc != ATTN_OK) return rc;
    m.causal = causal;
    m.dil = dilation > 1 ? dilation : 1;
    if (m.dil > 1 && n_global > 0)
        return fail(ATTN_ERR_UNSUPPORTED, "global tokens cannot be combined with a dilated mask");
    m.band = block > 0 ? eea::make_block_band(N, causal, block) : eea::make_band(N, causal, win_left, win_right);
    m.ng = (m.dil == 1 && eea::band_is_everything(m.band, causal)) ? 0 : n_global;
    return ATTN_OK;
}

int plan_impl(int N, const MaskSpec &m, int bm, int bn, long long *visible_pairs, long long *tiles_full,
              long long *tiles_edge) {
    if (bm <= 0 || bn <= 0) return fail(ATTN_ERR_INVALID_ARG, "tile shape %dx%d must be positive", bm, bn);
    const bool use_g = m.ng > 0;
    const int causal = m.causal;
    std::vector<char> is_g(N, 0);
    if (use_g)
        for (int g : m.G) is_g[g] = 1;
    // the random-block lists live on the device: one blocking copy
    std::vector<int> lists;
    const int rb = m.rand_block, nkb = rb > 0 ? (N + rb - 1) / rb : 0;
    if (rb > 0) {
        lists.resize((size_t)nkb * m.n_rand);
        hipError_t e = hipMemcpy(lists.data(), m.rand_idx, lists.size() * sizeof(int), hipMemcpyDeviceToHost);
        if (e != hipSuccess) return fail(ATTN_ERR_DEVICE, "reading rand_idx: %s", hipGetErrorString(e));
    }
    long long pairs = 0, full = 0, edge = 0;
    // every residue class (one class unless dilated) is a band of its own
    for (int r = 0; r < m.dil && r < N; ++r) {
        eea::Band band = m.band;
        band.N = (N - r + m.dil - 1) / m.dil;
        const int Nr = band.N;
        for (int i = 0; i < Nr; ++i) {
            const int lo = eea::row_lo(band, i), hi = eea::row_hi(band, i);
            if (use_g && is_g[i]) {
                pairs += causal ? (long long)i + 1 : (long long)N;
                continue;
            }
            pairs += hi - lo + 1;
            if (use_g)
                for (int g : m.G)
                    if ((g < lo || g > hi) && (!causal || g <= i)) ++pairs;
            if (rb > 0) {   // keys of each distinct listed block outside the band, off the globals
                const int *lst = &lists[(size_t)(i / rb) * m.n_rand];
                for (int e = 0; e < m.n_rand; ++e) {
                    const int kb = lst[e];
                    bool skip = kb < 0 || kb >= nkb;
                    for (int e2 = 0; e2 < e && !skip; ++e2) skip = lst[e2] == kb;
                    if (skip) continue;
                    const int j1 = std::min(Nr - 1, kb * rb + rb - 1);
                    for (int j = kb * rb; j <= j1; ++j) {
                        if ((causal && j > i) || (j >= lo && j <= hi) || (use_g && is_g[j])) continue;
                        ++pairs;
                    }
                }
            }
            if (m.stride > 0)   // positions at distance stride * 2^k outside the band, off the globals
                for (long long o = m.stride; o < Nr; o *= 2)
                    for (int sgn = -1; sgn <= 1; sgn += 2) {
                        if (sgn > 0 && causal) continue;
                        const long long j = i + sgn * o;
                        if (j < 0 || j >= Nr || (j >= lo && j <= hi)) continue;
                        if (use_g && is_g[j]) continue;
                        ++pairs;
                    }
        }
        const int nqt = (Nr + bm - 1) / bm;
        for (int qt = 0; qt < nqt; ++qt) {
            const int r0 = qt * bm, r1 = std::min(Nr - 1, r0 + bm - 1);
            int klo, khi;
            eea::key_tile_range(band, r0, r1, bn, &klo, &khi);
            for (int kt = klo; kt <= khi; ++kt) {
                const int cl = eea::classify(band, r0, r1, kt * bn, kt * bn + bn - 1);
                if (cl == eea::TILE_FULL) ++full;
                else if (cl == eea::TILE_EDGE) ++edge;
            }
            if (use_g) edge += (m.ng + bn - 1) / bn;   // gathered tiles of global columns
            if (m.stride > 0) {   // the strided rule's extra tiles, each visited once
                long long next = 0;
                auto visit = [&](long long klo, long long khi) {
                    klo = std::max(klo, 0LL);
                    khi = std::min(khi, (long long)Nr - 1);
                    if (klo > khi) return;
                    const long long t1 = khi / bn, t0 = std::max(klo / bn, next);
                    if (t1 >= t0) edge += t1 - t0 + 1;
                    next = std::max(next, t1 + 1);
                };
                std::vector<long long> offs;
                for (long long o = m.stride; o < Nr; o *= 2) offs.push_back(o);
                for (int a = (int)offs.size() - 1; a >= 0; --a) visit(r0 - offs[a], r1 - offs[a]);
                if (!causal)
                    for (long long o : offs) visit(r0 + o, r1 + o);
            }
        }
    }
    if (use_g)
        for (int g : m.G) {
            const long long keys = causal ? (long long)g + 1 : (long long)N;
            edge += (keys + bn - 1) / bn;
        }
    if (visible_pairs) *visible_pairs = pairs;
    if (tiles_full) *tiles_full = full;
    if (tiles_edge) *tiles_edge = edge;
    return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_plan_stats(int N, int causal, int win_left, int win_right, const int *global_idx, int n_global,
                    int bm, int bn, long long *visible_pairs, long long *tiles_full, long long *tiles_edge) {
    g_err.clear();
    if (N <= 0) return fail(ATTN_ERR_INVALID_ARG, "N=%d must be positive", N);
    MaskSpec m;
    int rc = resolve_mask(N, causal, win_left, win_right, 0, 1, global_idx, n_global, m);
    if (rc != ATTN_OK) return rc;
    return plan_impl(N, m, bm, bn, visible_pairs, tiles_full, tiles_edge);
}

int attn_plan_stats_masked(int N, const attn_mask *mask, int bm, int bn, long long *visible_pairs,
                           long long *tiles_full, long long *tiles_edge) {
    g_err.clear();
    if (N <= 0) return fail(ATTN_ERR_INVALID_ARG, "N=%d must be positive", N);
    if (!mask) return fail(ATTN_ERR_INVALID_ARG, "mask is NULL");
    MaskSpec m;
    int rc = resolve_mask(N, mask->causal, mask->win_left, mask->win_right, mask->block, mask->dilation,
                          mask->global_idx, mask->n_global, m);
    if (rc != ATTN_OK) return rc;
    rc = resolve_extras(N, mask, m);
    if (rc != ATTN_OK) return rc;
    return plan_impl(N, m, bm, bn, visible_pairs, tiles_full, tiles_edge);
}

}  // extern "C"

namespace {

// The forward call with H_kv K/V heads per batch entry (H_kv == H: plain
// multi-head attention).
int fwd_impl(const void *q, const void *k, const void *v, void *out, float *lse, int B, int H, int H_kv, int N,
             int d, int causal, int win_left, int win_right, int block, int dilation, const int *global_idx,
             int n_global, const attn_opts *opts, const attn_mask *extras = nullptr, bool noalloc = false) {
    g_err.clear();
    const int dtype = opts ? opts->dtype : ATTN_BF16;
    if (!q || !k || !v || !out || !lse) return fail(ATTN_ERR_INVALID_ARG, "a tensor pointer is NULL");
    if (B <= 0 || H <= 0 || N <= 0)
        return fail(ATTN_ERR_INVALID_ARG, "sizes B=%d H=%d N=%d must be positive", B, H, N);
    if (H_kv <= 0 || H % H_kv != 0)
        return fail(ATTN_ERR_INVALID_ARG, "H_kv=%d must be positive and divide H=%d", H_kv, H);
    if (dtype != ATTN_BF16 && dtype != ATTN_F32) return fail(ATTN_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    MaskSpec m;
    int rc = resolve_mask(N, causal, win_left, win_right, block, dilation, global_idx, n_global, m);
    if (rc != ATTN_OK) return rc;
    if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "head size d=%d is not supported (64 or 128)", d);
    if (m.dil > 1 && dtype == ATTN_F32)
        return fail(ATTN_ERR_UNSUPPORTED, "dilated masks are supported for bf16 tensors only");
    rc = resolve_extras(N, extras, m);
    if (rc != ATTN_OK) return rc;
    if (m.extra() && dtype == ATTN_F32)
        return fail(ATTN_ERR_UNSUPPORTED, "the strided and random-block rules are supported for bf16 tensors only");
    const std::vector<int> &G = m.G;

    const long long BH = (long long)B * H;
    const int bm = eea::band_tile_bm(d, dtype == ATTN_F32, m.band.block, m.extra(), m.band.wl, m.band.wr, m.dil);
    // query tiles per residue class (the longest class: ceil(N / dil) rows)
    const long long nqt = ((N + (long long)m.dil - 1) / m.dil + bm - 1) / bm;
    if (BH > INT_MAX || BH * m.dil * nqt > INT_MAX)
        return fail(ATTN_ERR_INVALID_ARG, "B*H=%lld with N=%d exceeds the launch grid", BH, N);
    const size_t esize = dtype == ATTN_F32 ? 4 : 2;
    if ((long long)N * d * (long long)esize > INT_MAX)
        return fail(ATTN_ERR_UNSUPPORTED, "one head's K of N=%d x d=%d elements exceeds 2 GiB", N, d);
    const size_t tbytes = (size_t)BH * N * d * esize;   // < 2^31 * 2^31 * 128 * 4: fits in 64 bits
    const size_t kvbytes = (size_t)B * H_kv * N * d * esize;
    const size_t lbytes = (size_t)BH * N * sizeof(float);

    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15)
        return fail(ATTN_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
    if ((uintptr_t)lse & 3) return fail(ATTN_ERR_INVALID_ARG, "lse must be 4-byte aligned");
    if (overlaps(out, tbytes, q, tbytes) || overlaps(out, tbytes, k, kvbytes) || overlaps(out, tbytes, v, kvbytes))
        return fail(ATTN_ERR_INVALID_ARG, "out overlaps an input tensor");
    if (overlaps(lse, lbytes, q, tbytes) || overlaps(lse, lbytes, k, kvbytes) || overlaps(lse, lbytes, v, kvbytes) ||
        overlaps(lse, lbytes, out, tbytes))
        return fail(ATTN_ERR_INVALID_ARG, "lse overlaps another tensor");

    float scale = (opts && opts->scale != 0.f) ? opts->scale : 1.0f / std::sqrt((float)d);
    if (!(scale > 0.f) || !std::isfinite(scale))
        return fail(ATTN_ERR_INVALID_ARG, "scale must be positive and finite");

    const eea::Band band = m.band;
    const int ng = m.ng;

    eea::FwdParams p;
    std::memset(&p, 0, sizeof p);
    p.q = q;
    p.k = k;
    p.v = v;
    p.out = out;
    p.lse = lse;
    p.head_stride = (long long)N * d;
    p.BH = (int)BH;
    p.H = H;
    p.group = H / H_kv;
    p.N = N;
    p.wl = band.wl;
    p.wr = band.wr;
    p.block = band.block;
    p.cap = band.cap;
    p.dil = m.dil;
    p.causal = causal;
    p.n_global = ng;
    p.num_qt = (int)nqt;
    p.scale_log2 = scale * 1.4426950408889634f;
    p.stride = m.stride;
    p.rand_block = m.rand_block;
    p.n_rand = m.n_rand;
    p.rand_idx = m.rand_idx;
    for (int t = 0; t < ng; ++t) p.gidx[t] = G[t];

    size_t need = 0;
    if (ng > 0) {
        if (eea::fuse_global_rows(dtype == ATTN_F32, d, m.dil, bm, ng)) {
            p.fuse_grows = 1;
            p.chunks = (int)nqt;
            p.chunk_tiles = 2;
        } else {
            int ct = 0;
            p.chunks = eea::global_chunks((int)BH, N, d, dtype == ATTN_F32, &ct);
            p.chunk_tiles = ct;
        }
        need = (size_t)BH * ng * p.chunks * (d + 2) * sizeof(float);
        if (noalloc && need > eea::kNoAllocScratchBytes)
            return fail(ATTN_ERR_UNSUPPORTED,
                        "attn_fwd_noalloc: the global-row partials need %zu bytes, more than its %zu-byte scratch", need,
                        eea::kNoAllocScratchBytes);
        if (opts && opts->workspace) {
            if (opts->workspace_bytes < need)
                return fail(ATTN_ERR_INVALID_ARG, "workspace of %zu bytes is smaller than the %zu needed",
                            opts->workspace_bytes, need);
            if ((uintptr_t)opts->workspace & 15)
                return fail(ATTN_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
            p.part = static_cast<float *>(opts->workspace);
        }
    }

    if (noalloc && opts && opts->workspace)
        return fail(ATTN_ERR_INVALID_ARG, "attn_fwd_noalloc takes no workspace (opts->workspace must be NULL)");

    // ---- first HIP call
    hipStream_t stream = opts ? static_cast<hipStream_t>(opts->stream) : nullptr;
    const int f32 = dtype == ATTN_F32;
    if (noalloc && ng > 0) {
        void *buf = nullptr;
        hipError_t e = eea::noalloc_scratch(&buf);
        if (e != hipSuccess) return fail(ATTN_ERR_DEVICE, "scratch address: %s", hipGetErrorString(e));
        p.part = static_cast<float *>(buf);
    }
    return run_on_device(SCR_FWD, need, p.part, stream, [&](void *buf) {
        p.part = static_cast<float *>(buf);
        return eea::launch_forward(p, d, f32, stream);
    });
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Backward workspace: the row terms rowsum(dO * O) and LSE * log2(e), each
// [B*H][N], then, with global tokens, the split passes' partials (dQ of the
// global rows per key chunk, dK and dV of the global columns per row chunk).
struct BwdLayout {
    size_t delta = 0, lse2 = 0, part_q = 0, part_k = 0, total = 0;
    int gchunks_q = 0, gct_q = 0, gchunks_k = 0, gct_k = 0;
};

BwdLayout bwd_layout(long long BH, long long BKV, int N, int d, int ng) {
    BwdLayout w;
    w.delta = 0;
    w.lse2 = align256((size_t)BH * N * sizeof(float));
    w.total = 2 * w.lse2;
    if (ng > 0) {
        eea::bwd_global_chunks((int)BH, N, &w.gchunks_q, &w.gct_q);
        eea::bwd_global_chunks((int)BKV, N, &w.gchunks_k, &w.gct_k);
        w.part_q = w.total;
        w.total += align256((size_t)BH * ng * w.gchunks_q * d * sizeof(float));
        w.part_k = w.total;
        w.total += align256((size_t)BKV * ng * w.gchunks_k * 2 * d * sizeof(float));
    }
    return w;
}

int bwd_impl(const void *q, const void *k, const void *v, const void *out, const void *dout, const float *lse,
             void *dq, void *dk, void *dv, int B, int H, int H_kv, int N, int d, int causal, int win_left,
             int win_right, int block, int dilation, const int *global_idx, int n_global, const attn_opts *opts,
             const attn_mask *extras = nullptr) {
    g_err.clear();
    const int dtype = opts ? opts->dtype : ATTN_BF16;
    if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv)
        return fail(ATTN_ERR_INVALID_ARG, "a tensor pointer is NULL");
    if (B <= 0 || H <= 0 || N <= 0)
        return fail(ATTN_ERR_INVALID_ARG, "sizes B=%d H=%d N=%d must be positive", B, H, N);
    if (H_kv <= 0 || H % H_kv != 0)
        return fail(ATTN_ERR_INVALID_ARG, "H_kv=%d must be positive and divide H=%d", H_kv, H);
    if (dtype != ATTN_BF16 && dtype != ATTN_F32) return fail(ATTN_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    if (dtype == ATTN_F32) return fail(ATTN_ERR_UNSUPPORTED, "the backward pass supports bf16 tensors only");
    MaskSpec m;
    int rc = resolve_mask(N, causal, win_left, win_right, block, dilation, global_idx, n_global, m);
    if (rc != ATTN_OK) return rc;
    if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "head size d=%d is not supported (64 or 128)", d);
    rc = resolve_extras(N, extras, m);
    if (rc != ATTN_OK) return rc;
    const eea::Band band = m.band;

    const long long BH = (long long)B * H;
    const int bq = eea::bwd_tile_q(d, m.ng == 0 && !m.extra()), bk = eea::bwd_tile_k(d);
    // tiles per residue class (the longest class: ceil(N / dil) rows)
    const long long Nc = (N + (long long)m.dil - 1) / m.dil;
    const long long nqt = (Nc + bq - 1) / bq, nkt = (Nc + bk - 1) / bk;
    if (BH > INT_MAX || BH * m.dil * nqt > INT_MAX || (long long)B * H_kv * m.dil * nkt > INT_MAX)
        return fail(ATTN_ERR_INVALID_ARG, "B*H=%lld with N=%d exceeds the launch grid", BH, N);
    if ((long long)N * d * 2 > INT_MAX)
        return fail(ATTN_ERR_UNSUPPORTED, "one head's K of N=%d x d=%d elements exceeds 2 GiB", N, d);
    const size_t qbytes = (size_t)BH * N * d * 2;
    const size_t kvbytes = (size_t)B * H_kv * N * d * 2;
    const size_t lbytes = (size_t)BH * N * sizeof(float);
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out | (uintptr_t)dout | (uintptr_t)dq |
         (uintptr_t)dk | (uintptr_t)dv) & 15)
        return fail(ATTN_ERR_INVALID_ARG, "q, k, v, out, dout, dq, dk and dv must be 16-byte aligned");
    if ((uintptr_t)lse & 3) return fail(ATTN_ERR_INVALID_ARG, "lse must be 4-byte aligned");
    const void *ins[6] = {q, k, v, out, dout, lse};
    const size_t insz[6] = {qbytes, kvbytes, kvbytes, qbytes, qbytes, lbytes};
    void *outs[3] = {dq, dk, dv};
    const size_t outsz[3] = {qbytes, kvbytes, kvbytes};
    for (int a = 0; a < 3; ++a) {
        for (int i = 0; i < 6; ++i)
            if (overlaps(outs[a], outsz[a], ins[i], insz[i]))
                return fail(ATTN_ERR_INVALID_ARG, "gradient output %d overlaps an input tensor", a);
        for (int o = 0; o < a; ++o)
            if (overlaps(outs[a], outsz[a], outs[o], outsz[o]))
                return fail(ATTN_ERR_INVALID_ARG, "gradient outputs %d and %d overlap", o, a);
    }
    const float scale = (opts && opts->scale != 0.f) ? opts->scale : 1.0f / std::sqrt((float)d);
    if (!(scale > 0.f) || !std::isfinite(scale))
        return fail(ATTN_ERR_INVALID_ARG, "scale must be positive and finite");

    const BwdLayout lay = bwd_layout(BH, (long long)B * H_kv, N, d, m.ng);
    const size_t need = lay.total;
    void *ws = nullptr;
    if (opts && opts->workspace) {
        if (opts->workspace_bytes < need)
            return fail(ATTN_ERR_INVALID_ARG, "workspace of %zu bytes is smaller than the %zu needed",
                        opts->workspace_bytes, need);
        if ((uintptr_t)opts->workspace & 15) return fail(ATTN_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
        ws = opts->workspace;
        const void *all[9] = {q, k, v, out, dout, lse, dq, dk, dv};
        const size_t allsz[9] = {qbytes, kvbytes, kvbytes, qbytes, qbytes, lbytes, qbytes, kvbytes, kvbytes};
        for (int i = 0; i < 9; ++i)
            if (overlaps(ws, need, all[i], allsz[i]))
                return fail(ATTN_ERR_INVALID_ARG, "workspace overlaps a tensor");
    }

    eea::BwdParams p;
    std::memset(&p, 0, sizeof p);
    p.q = q;
    p.k = k;
    p.v = v;
    p.out = out;
    p.dout = dout;
    p.lse = lse;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.head_stride = (long long)N * d;
    p.BH = (int)BH;
    p.H = H;
    p.group = H / H_kv;
    p.N = N;
    p.wl = band.wl;
    p.wr = band.wr;
    p.block = band.block;
    p.cap = band.cap;
    p.dil = m.dil;
    p.causal = causal;
    p.num_qt = (int)nqt;
    p.num_kt = (int)nkt;
    p.scale = scale;
    p.scale_log2 = scale * 1.4426950408889634f;
    p.n_global = m.ng;
    for (int t = 0; t < m.ng; ++t) p.gidx[t] = m.G[t];
    p.gchunks_q = lay.gchunks_q;
    p.gct_q = lay.gct_q;
    p.gchunks_k = lay.gchunks_k;
    p.gct_k = lay.gct_k;
    p.stride = m.stride;
    p.rand_block = m.rand_block;
    p.n_rand = m.n_rand;
    p.rand_idx = m.rand_idx;

    // ---- first HIP call
    hipStream_t stream = opts ? static_cast<hipStream_t>(opts->stream) : nullptr;
    return run_on_device(SCR_BWD, need, ws, stream, [&](void *buf) {
        p.delta = static_cast<float *>(buf);
        p.lse2 = reinterpret_cast<float *>(static_cast<char *>(buf) + lay.lse2);
        if (m.ng > 0) {
            p.part_q = reinterpret_cast<float *>(static_cast<char *>(buf) + lay.part_q);
            p.part_k = reinterpret_cast<float *>(static_cast<char *>(buf) + lay.part_k);
        }
        return eea::launch_backward(p, d, stream);
    });
}

size_t decode_workspace(int B, int H, int H_kv, int Nq, int S, int d, int win_left, int rolling) {
    const int group = H / H_kv;
    const long long R = (long long)group * Nq;
    const int nrg = (int)((R + eea::kDecRows - 1) / eea::kDecRows);
    const int chunks = eea::decode_chunks(B, H_kv, nrg, S, Nq, win_left, rolling);
    return chunks == 1 ? 0 : (size_t)B * H * Nq * chunks * (d + 2) * sizeof(float);
}

int decode_impl(const void *q, const void *kc, const void *vc, const int *seq_len, void *out, float *lse, int B,
                int H, int H_kv, int Nq, int S, int d, int win_left, int rolling, const attn_opts *opts) {
    g_err.clear();
    const int dtype = opts ? opts->dtype : ATTN_BF16;
    if (!q || !kc || !vc || !seq_len || !out || !lse) return fail(ATTN_ERR_INVALID_ARG, "a pointer is NULL");
    if (B <= 0 || H <= 0 || Nq <= 0 || S <= 0)
        return fail(ATTN_ERR_INVALID_ARG, "sizes B=%d H=%d Nq=%d S=%d must be positive", B, H, Nq, S);
    if (H_kv <= 0 || H % H_kv != 0)
        return fail(ATTN_ERR_INVALID_ARG, "H_kv=%d must be positive and divide H=%d", H_kv, H);
    if (dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "decoding supports bf16 tensors only");
    if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "head size d=%d is not supported (64 or 128)", d);
    if (win_left < -1) return fail(ATTN_ERR_INVALID_ARG, "win_left=%d must be >= -1", win_left);
    if (rolling != 0 && rolling != 1) return fail(ATTN_ERR_INVALID_ARG, "rolling=%d must be 0 or 1", rolling);
    if (Nq > S) return fail(ATTN_ERR_INVALID_ARG, "Nq=%d new tokens do not fit a cache of S=%d slots", Nq, S);
    if (rolling && (win_left < 0 || (long long)Nq + win_left > S))
        return fail(ATTN_ERR_INVALID_ARG,
                    "a rolling cache of S=%d slots needs a window with Nq + win_left <= S (Nq=%d, win_left=%d)", S,
                    Nq, win_left);
    if ((long long)S * d * 2 > INT_MAX)
        return fail(ATTN_ERR_UNSUPPORTED, "one head's cache of S=%d x d=%d elements exceeds 2 GiB", S, d);
    const long long BH = (long long)B * H;
    const long long R = (long long)(H / H_kv) * Nq;
    const int nrg = (int)((R + eea::kDecRows - 1) / eea::kDecRows);
    const int chunks = eea::decode_chunks(B, H_kv, nrg, S, Nq, win_left, rolling);
    if (BH * Nq > INT_MAX || (long long)B * H_kv * nrg * chunks > INT_MAX)
        return fail(ATTN_ERR_INVALID_ARG, "sizes exceed the launch grid");
    const size_t qbytes = (size_t)BH * Nq * d * 2;
    const size_t cbytes = (size_t)B * H_kv * S * d * 2;
    const size_t lbytes = (size_t)BH * Nq * sizeof(float);
    if (((uintptr_t)q | (uintptr_t)kc | (uintptr_t)vc | (uintptr_t)out) & 15)
        return fail(ATTN_ERR_INVALID_ARG, "q, k_cache, v_cache and out must be 16-byte aligned");
    if (((uintptr_t)lse | (uintptr_t)seq_len) & 3) return fail(ATTN_ERR_INVALID_ARG, "lse and seq_len must be 4-byte aligned");
    if (overlaps(out, qbytes, q, qbytes) || overlaps(out, qbytes, kc, cbytes) || overlaps(out, qbytes, vc, cbytes) ||
        overlaps(out, qbytes, seq_len, (size_t)B * 4))
        return fail(ATTN_ERR_INVALID_ARG, "out overlaps an input");
    if (overlaps(lse, lbytes, q, qbytes) || overlaps(lse, lbytes, kc, cbytes) || overlaps(lse, lbytes, vc, cbytes) ||
        overlaps(lse, lbytes, out, qbytes) || overlaps(lse, lbytes, seq_len, (size_t)B * 4))
        return fail(ATTN_ERR_INVALID_ARG, "lse overlaps another tensor");
    const float scale = (opts && opts->scale != 0.f) ? opts->scale : 1.0f / std::sqrt((float)d);
    if (!(scale > 0.f) || !std::isfinite(scale))
        return fail(ATTN_ERR_INVALID_ARG, "scale must be positive and finite");
    const size_t need = decode_workspace(B, H, H_kv, Nq, S, d, win_left, rolling);
    void *ws = nullptr;
    if (opts && opts->workspace) {
        if (opts->workspace_bytes < need)
            return fail(ATTN_ERR_INVALID_ARG, "workspace of %zu bytes is smaller than the %zu needed",
                        opts->workspace_bytes, need);
        if ((uintptr_t)opts->workspace & 15) return fail(ATTN_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
        ws = opts->workspace;
    }

    eea::DecParams p;
    std::memset(&p, 0, sizeof p);
    p.q = q;
    p.kc = kc;
    p.vc = vc;
    p.out = out;
    p.lse = lse;
    p.seq_len = seq_len;
    p.B = B;
    p.H = H;
    p.H_kv = H_kv;
    p.group = H / H_kv;
    p.Nq = Nq;
    p.S = S;
    p.win = win_left;
    p.rolling = rolling;
    p.R = (int)R;
    p.nrg = nrg;
    p.chunks = chunks;
    p.scale_log2 = scale * 1.4426950408889634f;

    hipStream_t stream = opts ? static_cast<hipStream_t>(opts->stream) : nullptr;
    return run_on_device(SCR_DEC, need, ws, stream, [&](void *buf) {
        p.part = static_cast<float *>(buf);
        return eea::launch_decode(p, d, stream);
    });
}

}  // namespace

extern "C" {

int attn_decode(const void *q, const void *k_cache, const void *v_cache, const int *seq_len, void *out,
                float *lse, int B, int H, int H_kv, int Nq, int S, int d, int win_left, int rolling,
                const attn_opts *opts) {
    return decode_impl(q, k_cache, v_cache, seq_len, out, lse, B, H, H_kv, Nq, S, d, win_left, rolling, opts);
}

size_t attn_decode_workspace_bytes(int B, int H, int H_kv, int Nq, int S, int d, int win_left, int rolling) {
    if (B <= 0 || H <= 0 || H_kv <= 0 || H % H_kv != 0 || Nq <= 0 || S <= 0 || (d != 64 && d != 128) ||
        win_left < -1)
        return 0;
    return decode_workspace(B, H, H_kv, Nq, S, d, win_left, rolling != 0);
}

int attn_bwd(const void *q, const void *k, const void *v, const void *out, const void *dout, const float *lse,
             void *dq, void *dk, void *dv, int B, int H, int H_kv, int N, int d, int causal, int win_left,
             int win_right, const int *global_idx, int n_global, const attn_opts *opts) {
    return bwd_impl(q, k, v, out, dout, lse, dq, dk, dv, B, H, H_kv, N, d, causal, win_left, win_right, 0, 1,
                    global_idx, n_global, opts);
}

int attn_bwd_masked(const void *q, const void *k, const void *v, const void *out, const void *dout,
                    const float *lse, void *dq, void *dk, void *dv, int B, int H, int H_kv, int N, int d,
                    const attn_mask *mask, const attn_opts *opts) {
    if (!mask) {
        g_err.clear();
        return fail(ATTN_ERR_INVALID_ARG, "mask is NULL");
    }
    return bwd_impl(q, k, v, out, dout, lse, dq, dk, dv, B, H, H_kv, N, d, mask->causal, mask->win_left,
                    mask->win_right, mask->block, mask->dilation, mask->global_idx, mask->n_global, opts, mask);
}

size_t attn_bwd_workspace_bytes(int B, int H, int H_kv, int N, int d, int n_global) {
    if (B <= 0 || H <= 0 || N <= 0 || (d != 64 && d != 128)) return 0;
    if (H_kv <= 0 || H % H_kv != 0 || n_global < 0 || n_global > eea::kMaxGlobal) return 0;
    if ((long long)B * H > INT_MAX) return 0;
    return bwd_layout((long long)B * H, (long long)B * H_kv, N, d, n_global).total;
}

int attn_fwd_ex(const void *q, const void *k, const void *v, void *out, float *lse, int B, int H, int N, int d,
                int causal, int win_left, int win_right, const int *global_idx, int n_global,
                const attn_opts *opts) {
    return fwd_impl(q, k, v, out, lse, B, H, H, N, d, causal, win_left, win_right, 0, 1, global_idx, n_global,
                    opts);
}

int attn_fwd_gqa(const void *q, const void *k, const void *v, void *out, float *lse, int B, int H, int H_kv,
                 int N, int d, int causal, int win_left, int win_right, const int *global_idx, int n_global,
                 const attn_opts *opts) {
    return fwd_impl(q, k, v, out, lse, B, H, H_kv, N, d, causal, win_left, win_right, 0, 1, global_idx,
                    n_global, opts);
}

int attn_fwd_masked(const void *q, const void *k, const void *v, void *out, float *lse, int B, int H, int H_kv,
                    int N, int d, const attn_mask *mask, const attn_opts *opts) {
    if (!mask) {
        g_err.clear();
        return fail(ATTN_ERR_INVALID_ARG, "mask is NULL");
    }
    return fwd_impl(q, k, v, out, lse, B, H, H_kv, N, d, mask->causal, mask->win_left, mask->win_right,
                    mask->block, mask->dilation, mask->global_idx, mask->n_global, opts, mask);
}

int attn_fwd_noalloc(const void *q, const void *k, const void *v, void *out, float *lse, int B, int H, int N,
                     int d, int causal, int win_left, int win_right, const int *global_idx, int n_global,
                     const attn_opts *opts) {
    return fwd_impl(q, k, v, out, lse, B, H, H, N, d, causal, win_left, win_right, 0, 1, global_idx, n_global,
                    opts, nullptr, true);
}

int attn_fwd(const void *q, const void *k, const void *v, void *out, float *lse, int B, int H, int N, int d,
             int causal, int win_left, int win_right, const int *global_idx, int n_global) {
    return fwd_impl(q, k, v, out, lse, B, H, H, N, d, causal, win_left, win_right, 0, 1, global_idx, n_global,
                    nullptr);
}

}  // extern "C"
