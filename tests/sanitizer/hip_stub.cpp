// The HIP runtime calls and kernel launchers of the library, replaced for a
// CPU-only build of its host code (attn_api.cpp, attn_host.cpp) under
// AddressSanitizer and UndefinedBehaviorSanitizer. Test infrastructure: never
// part of the shipped library.
//
// Two modes, switched by eea_stub_simulate_device():
//   - no device (the default): hipGetDevice fails as on a machine without a
//     GPU, so every valid call ends in ATTN_ERR_DEVICE;
//   - a simulated gfx950: "device memory" is host memory (hipMalloc is
//     malloc, hipMemcpy is memcpy), events and streams are no-ops, and each
//     launcher touches every byte its kernels would read or write, with the
//     extents the kernels index by (the part/delta offsets in the kernel
//     sources). A launch plan or workspace size that disagrees with those
//     extents then shows up as a heap overflow in the sanitizer report.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "attn_internal.h"

namespace {

int g_simulate = 0;
std::mutex g_mu;
long long g_malloc_calls = 0;
long long g_live_bytes = 0;
long long g_launches = 0;

struct ihipEventStub {
    int recorded;
};

volatile unsigned char g_sink;

void read_all(const void *p, size_t bytes) {
    const unsigned char *b = static_cast<const unsigned char *>(p);
    unsigned char acc = 0;
    for (size_t i = 0; i < bytes; ++i) acc ^= b[i];
    g_sink = acc;
}

void write_all(void *p, size_t bytes) { std::memset(p, 0, bytes); }

// Every launch must see sorted, distinct, in-range global positions.
bool globals_ok(const int *g, int n, int N) {
    for (int t = 0; t < n; ++t) {
        if (g[t] < 0 || g[t] >= N) return false;
        if (t > 0 && g[t] <= g[t - 1]) return false;
    }
    return true;
}

bool rand_lists_ok(const int *lists, int N, int rand_block, int n_rand) {
    if (rand_block <= 0) return true;
    const long long nb = (N + rand_block - 1) / rand_block;
    read_all(lists, (size_t)nb * n_rand * sizeof(int));
    for (long long i = 0; i < nb * n_rand; ++i)
        if (lists[i] < 0 || lists[i] >= nb) return false;
    return true;
}

}  // namespace

extern "C" {

void eea_stub_simulate_device(int on) { g_simulate = on; }

long long eea_stub_malloc_calls() {
    std::lock_guard<std::mutex> lk(g_mu);
    return g_malloc_calls;
}

long long eea_stub_live_bytes() {
    std::lock_guard<std::mutex> lk(g_mu);
    return g_live_bytes;
}

long long eea_stub_launches() {
    std::lock_guard<std::mutex> lk(g_mu);
    return g_launches;
}

}  // extern "C"

hipError_t hipGetDevice(int *dev) {
    if (!g_simulate) return hipErrorNoDevice;
    *dev = 0;
    return hipSuccess;
}

hipError_t hipGetDeviceProperties(hipDeviceProp_t *prop, int dev) {
    if (!g_simulate || dev != 0) return hipErrorNoDevice;
    std::memset(prop, 0, sizeof *prop);
    std::snprintf(prop->name, sizeof prop->name, "simulated");
    std::snprintf(prop->gcnArchName, sizeof prop->gcnArchName, "gfx950:sramecc+:xnack-");
    prop->totalGlobalMem = (size_t)288 << 30;
    prop->multiProcessorCount = 256;
    return hipSuccess;
}

const char *hipGetErrorString(hipError_t e) {
    switch (e) {
        case hipSuccess: return "no error";
        case hipErrorInvalidValue: return "invalid argument";
        case hipErrorOutOfMemory: return "out of memory";
        case hipErrorNoDevice: return "no ROCm-capable device is detected";
    }
    return "unknown error";
}

// The allocation size lives in a 64-byte header so that hipFree can keep
// the live-byte count; the returned pointer stays 64-byte aligned.
hipError_t hipMalloc(void **ptr, size_t bytes) {
    if (!g_simulate) return hipErrorNoDevice;
    void *raw = std::aligned_alloc(64, 64 + ((bytes + 63) / 64) * 64);
    if (!raw) return hipErrorOutOfMemory;
    *static_cast<size_t *>(raw) = bytes;
    *ptr = static_cast<char *>(raw) + 64;
    std::lock_guard<std::mutex> lk(g_mu);
    ++g_malloc_calls;
    g_live_bytes += (long long)bytes;
    return hipSuccess;
}

hipError_t hipFree(void *ptr) {
    if (!g_simulate) return hipErrorNoDevice;
    if (!ptr) return hipSuccess;
    void *raw = static_cast<char *>(ptr) - 64;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        g_live_bytes -= (long long)*static_cast<size_t *>(raw);
    }
    std::free(raw);
    return hipSuccess;
}

hipError_t hipMemcpy(void *dst, const void *src, size_t bytes, hipMemcpyKind) {
    if (!g_simulate) return hipErrorNoDevice;
    std::memcpy(dst, src, bytes);
    return hipSuccess;
}

hipError_t hipEventCreateWithFlags(hipEvent_t *ev, unsigned) {
    if (!g_simulate) return hipErrorNoDevice;
    *ev = reinterpret_cast<hipEvent_t>(new ihipEventStub{0});
    return hipSuccess;
}

hipError_t hipEventRecord(hipEvent_t ev, hipStream_t) {
    if (!g_simulate || !ev) return hipErrorInvalidValue;
    reinterpret_cast<ihipEventStub *>(ev)->recorded = 1;
    return hipSuccess;
}

hipError_t hipEventSynchronize(hipEvent_t ev) { return (g_simulate && ev) ? hipSuccess : hipErrorInvalidValue; }

hipError_t hipStreamWaitEvent(hipStream_t, hipEvent_t ev, unsigned) {
    return (g_simulate && ev) ? hipSuccess : hipErrorInvalidValue;
}

namespace eea {

hipError_t launch_forward(const FwdParams &p, int d, int f32, hipStream_t) {
    const size_t es = f32 ? 4 : 2;
    const long long BKV = (long long)p.BH / p.group;
    read_all(p.q, (size_t)p.BH * p.N * d * es);
    read_all(p.k, (size_t)BKV * p.N * d * es);
    read_all(p.v, (size_t)BKV * p.N * d * es);
    if (!globals_ok(p.gidx, p.n_global, p.N)) return hipErrorInvalidValue;
    if (!rand_lists_ok(p.rand_idx, p.N, p.rand_block, p.n_rand)) return hipErrorInvalidValue;
    if (p.n_global > 0) {
        if (p.chunks < 1 || p.chunks > kMaxGlobalChunks || (long long)p.chunks * p.chunk_tiles * tile_bn(d, f32) < p.N)
            return hipErrorInvalidValue;
        // split-key pass: row (bh, t), chunk c at ((bh * ng + t) * chunks + c) * (d + 2)
        write_all(p.part, (size_t)p.BH * p.n_global * p.chunks * (d + 2) * sizeof(float));
        read_all(p.part, (size_t)p.BH * p.n_global * p.chunks * (d + 2) * sizeof(float));
    }
    write_all(p.out, (size_t)p.BH * p.N * d * es);
    write_all(p.lse, (size_t)p.BH * p.N * sizeof(float));
    std::lock_guard<std::mutex> lk(g_mu);
    ++g_launches;
    return hipSuccess;
}

hipError_t launch_backward(const BwdParams &p, int d, hipStream_t) {
    const long long BKV = (long long)p.BH / p.group;
    const size_t act = (size_t)p.BH * p.N * d * 2, kv = (size_t)BKV * p.N * d * 2;
    read_all(p.q, act);
    read_all(p.k, kv);
    read_all(p.v, kv);
    read_all(p.out, act);
    read_all(p.dout, act);
    read_all(p.lse, (size_t)p.BH * p.N * sizeof(float));
    if (!globals_ok(p.gidx, p.n_global, p.N)) return hipErrorInvalidValue;
    if (!rand_lists_ok(p.rand_idx, p.N, p.rand_block, p.n_rand)) return hipErrorInvalidValue;
    write_all(p.delta, (size_t)p.BH * p.N * sizeof(float));
    write_all(p.lse2, (size_t)p.BH * p.N * sizeof(float));
    if (p.n_global > 0) {
        if ((long long)p.gchunks_q * p.gct_q * 64 < p.N || (long long)p.gchunks_k * p.gct_k * 64 < p.N)
            return hipErrorInvalidValue;
        write_all(p.part_q, (size_t)p.BH * p.n_global * p.gchunks_q * d * sizeof(float));
        write_all(p.part_k, (size_t)BKV * p.n_global * p.gchunks_k * 2 * d * sizeof(float));
    }
    write_all(p.dq, act);
    write_all(p.dk, kv);
    write_all(p.dv, kv);
    std::lock_guard<std::mutex> lk(g_mu);
    ++g_launches;
    return hipSuccess;
}

hipError_t launch_decode(const DecParams &p, int d, hipStream_t) {
    read_all(p.q, (size_t)p.B * p.H * p.Nq * d * 2);
    read_all(p.kc, (size_t)p.B * p.H_kv * p.S * d * 2);
    read_all(p.vc, (size_t)p.B * p.H_kv * p.S * d * 2);
    read_all(p.seq_len, (size_t)p.B * sizeof(int));
    if (p.chunks < 1 || p.chunks > kDecMaxChunks || p.R != p.group * p.Nq ||
        (long long)p.nrg * kDecRows < p.R)
        return hipErrorInvalidValue;
    if (p.chunks > 1) {
        // chunk c of query row grow at (grow * chunks + c) * (d + 2)
        write_all(p.part, (size_t)p.B * p.H * p.Nq * p.chunks * (d + 2) * sizeof(float));
    }
    write_all(p.out, (size_t)p.B * p.H * p.Nq * d * 2);
    write_all(p.lse, (size_t)p.B * p.H * p.Nq * sizeof(float));
    std::lock_guard<std::mutex> lk(g_mu);
    ++g_launches;
    return hipSuccess;
}

// The allocation-free forward's array: a static host array of the same size.
hipError_t noalloc_scratch(void **ptr) {
    if (!g_simulate) return hipErrorNoDevice;
    alignas(256) static char scratch[kNoAllocScratchBytes];
    *ptr = scratch;
    return hipSuccess;
}

}  // namespace eea
