// attn_tiles.h - device-side pieces shared by the forward and backward
// kernels: vector types, the 32x32 MFMA accumulator layout, and the bf16 tile
// path (LDS swizzles, operand reads, tile copies HBM -> LDS, Q-style operand
// loads and row stores). Included by the .hip sources only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace eea {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(8))) short s16x8;
typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

#define EEA_LDS __attribute__((address_space(3)))

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleLog2 = 8.0f;
#define EEA_NEG_INF (-__builtin_huge_valf())

enum { MODE_BAND = 0, MODE_GROWS = 1 };

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Key offset (within its 32-key block) of accumulator register r of a lane in
// half-wave h, for the 32x32 MFMA output layout.
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// s_waitcnt with vmcnt(0) and the other counters left alone (gfx9 encoding:
// vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt_hi[15:14]).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Debug-sync build (-DATTN_DEBUG_SYNC): every pipelined copy into an LDS
// buffer is fenced on both sides. Before the copy, every wave has finished
// with all earlier LDS reads (the barrier waits for them); after it, the copy
// has landed before any wave goes on. Copies and compute then never overlap,
// so the build's results must equal the optimised build's bit for bit; a
// missing wait or barrier in the pipelined order would show as a difference.
// Call sites are points that every wave of the workgroup reaches. The
// optimised build compiles this to nothing.
#ifdef ATTN_DEBUG_SYNC
constexpr bool kDebugSync = true;
#else
constexpr bool kDebugSync = false;
#endif
__device__ __forceinline__ void debug_sync() {
    if constexpr (kDebugSync) {
        wait_vmem();
        __syncthreads();
    }
}

// Source rows of one key tile: keys k0.. for a band tile, or the global
// positions g[k0..] for a gathered tile. Returns -1 for a row with no key.
struct TileSrc {
    int k0;
    int gather;     // 0: band tile at key k0; 1: gathered tile from global slot k0
    int N;
    int ng;
    const int *g;   // LDS copy of the sorted global positions
    __device__ __forceinline__ int key(int r) const {
        if (gather) return k0 + r < ng ? g[k0 + r] : -1;
        return k0 + r < N ? k0 + r : -1;
    }
};

// ---------------------------------------------------------------------------
// bf16 inputs: QK^T and PV on v_mfma_f32_32x32x16_bf16; tiles loaded
// global -> LDS directly, V operands through the LDS transpose read.
// ---------------------------------------------------------------------------
// UNI_: one LDS layout per tile for both operand patterns (row reads and
// transpose reads), so a tile that is read both ways is copied once (see ux).
template <int D_, int NT_, bool UNI_ = false>
struct Bf16Path {
    static constexpr int D = D_, BN = 64, NT = NT_, NW = NT / 64;
    static constexpr bool UNI = UNI_;
    static constexpr bool F32 = false;
    static constexpr int KS = D / 16;     // k-steps of QK^T
    static constexpr int MB = BN / 32;    // 32-key blocks per tile
    static constexpr int DB = D / 32;     // 32-wide blocks of d in O^T
    static constexpr int PVS = BN / 16;   // 16-key steps of PV
    static constexpr int ROWB = D * 2;    // bytes per K or V row
    static constexpr int TILE_BYTES = BN * ROWB;
    static constexpr int SEGS = TILE_BYTES / 1024;   // one wave-wide 16-byte load = 1 KiB
    static constexpr int SPW = SEGS / NW;            // loads per wave per tile (each of K, V)
    static constexpr int LDS_BYTES = 4 * TILE_BYTES; // K and V, two buffers each
    static_assert(SEGS % NW == 0, "tile loads must split evenly over the waves");
    static_assert(D == 64 || D == 128, "head size");

    typedef uint16_t elem_t;
    struct QFrag { bf16x8 x[KS]; };
    struct PFrag { bf16x8 x[PVS]; };
    struct Stage {};

    // LDS layouts (gfx950 LDS serves 256 bytes per clock: 64 banks of 4 B).
    // K rows: 16-byte chunk c of row r is stored at chunk c ^ kx(r). A
    // ds_read_b128 serves 16 lanes per pass and the 16 lanes of a pass read
    // the same logical chunk of 16 consecutive rows, so kx must map those
    // rows onto 16 distinct 16-byte slots of the 256-byte bank window.
    // (the swizzles and the per-lane offsets are host-callable too, so a CPU
    // test can replay the copies and reads of a tile)
    static __host__ __device__ __forceinline__ int kx(int r) {
        return D == 128 ? (r & 15) : ((r >> 1) & 7);   // d=64: two rows per window
    }
    // V rows: the transpose read of a half-wave touches 4 consecutive key
    // rows over one 64-byte d-block, so vx moves those 4 rows onto the 4
    // distinct 64-byte quarters of the bank window.
    static __host__ __device__ __forceinline__ int vx(int r) {
        return D == 128 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2);
    }
    // One layout for both patterns: ux gives 16 distinct chunk slots to the
    // 16 rows of a row-read pass (d = 128: its low two bits take r >> 2, its
    // high two bits r & 3; d = 64: 8 distinct slots to each row parity) and
    // sends the 4 rows of a transpose-read pass to 4 distinct 64-byte
    // quarters (its bit 2, and at d = 128 bit 3, follow the row within its
    // aligned quad). Rows 8 apart differ by ux ^ 2 (r >> 2 moves by 2).
    static __host__ __device__ __forceinline__ int ux(int r) {
        return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
    }
    static __host__ __device__ __forceinline__ int kxs(int r) { return UNI ? ux(r) : kx(r); }
    static __host__ __device__ __forceinline__ int vxs(int r) { return UNI ? ux(r) : vx(r); }

    // Per-lane constants, computed once.
    struct Lane {
        int krd[KS];       // K operand: byte offset in a K tile for (mb=0, ks)
        int vrd[DB];       // V operand: byte offset in a V tile for (st=0, db)
        int vrdh[UNI ? DB : 1];   // UNI: the same for the second read, 8 key rows on
        int ldrow[SPW];    // tile row this lane fetches in load i
        int ldkcol[SPW];   // element offset of its K chunk within that row
        int ldvcol[SPW];   // element offset of its V chunk within that row
        int ldlds[SPW];    // LDS byte offset (within a tile) of this wave's load i
        int ldk[SPW];      // byte offset of load i's K chunk from the tile's first row
        int ldv[SPW];      // byte offset of load i's V chunk from the tile's first row
    };

    // dil: distance in rows of the stored tensor between consecutive tile
    // rows (1 for contiguous rows; k for one residue class of a dilated mask).
    static __host__ __device__ __forceinline__ void init_lane(Lane &L, int lane, int wave, int dil = 1) {
        const int ln = lane & 31, h = lane >> 5;
        // K row ln, logical chunk 2ks + h
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) L.krd[ks] = ln * ROWB + 16 * ((2 * ks + h) ^ kxs(ln));
        // transpose read: lane j of 16-lane group g loads 4 elements of key
        // row 4h + j/4 at d = 32db + 16(g&1) + 4(j&3); lane i of the group then
        // holds d = 32db + 16(g&1) + i for the keys 4h + e, e = 0..3
        const int g = lane >> 4, j = lane & 15;
        const int krow = 4 * h + (j >> 2);
        const int t = 2 * (g & 1) + ((j >> 1) & 1);
#pragma unroll
        for (int db = 0; db < DB; ++db) L.vrd[db] = krow * ROWB + 16 * ((4 * db + t) ^ vxs(krow)) + 8 * (j & 1);
        if constexpr (UNI) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
                L.vrdh[db] = (krow + 8) * ROWB + 16 * ((4 * db + t) ^ ux(krow + 8)) + 8 * (j & 1);
        }
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int o = (wave * SPW + i) * 1024 + lane * 16;
            const int row = o / ROWB, phys = (o % ROWB) / 16;
            L.ldrow[i] = row;
            L.ldkcol[i] = (phys ^ kxs(row)) * 8;
            L.ldvcol[i] = (phys ^ vxs(row)) * 8;
            L.ldlds[i] = (wave * SPW + i) * 1024;
            L.ldk[i] = row * dil * ROWB + 2 * L.ldkcol[i];
            L.ldv[i] = row * dil * ROWB + 2 * L.ldvcol[i];
        }
    }

    static __device__ __forceinline__ void load_q(QFrag &qf, const elem_t *qh, int row, bool valid, int h) {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(qh + (long long)row * D);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 w = valid ? src[2 * ks + h] : u32x4{0, 0, 0, 0};
            qf.x[ks] = __builtin_bit_cast(bf16x8, w);
        }
    }

    // Start the global -> LDS copy of one K tile and one V tile. Rows with no
    // key fetch row `fallback` (a valid row); the caller masks them.
    //
    // The copies are MUBUF buffer loads with the LDS-destination bit (one
    // buffer resource per head, byte offsets below 2^31). Unlike the FLAT
    // form of the same copy, a buffer load only counts on vmcnt, so the
    // compiler can still wait for an exact number of the LDS reads that
    // follow it while the copy is in flight.
    static __device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const elem_t *base, int N) {
        // dword3 0x00020000: raw 32-bit data format, the usual gfx9 setting
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<elem_t *>(base), 0, N * ROWB, 0x00020000);
    }
    static __device__ __forceinline__ void issue(Stage &, const Lane &L, const elem_t *kh, const elem_t *vh,
                                                 char *kbuf, char *vbuf, const TileSrc &src, int fallback) {
        const __amdgpu_buffer_rsrc_t kr = head_rsrc(kh, src.N), vr = head_rsrc(vh, src.N);
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            int key = src.key(L.ldrow[i]);
            key = key < 0 ? fallback : key;
            const unsigned off = (unsigned)key * ROWB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (EEA_LDS void *)(kbuf + L.ldlds[i]), 16,
                                                     off + 2 * L.ldkcol[i], 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (EEA_LDS void *)(vbuf + L.ldlds[i]), 16,
                                                     off + 2 * L.ldvcol[i], 0, 0, 0);
        }
    }
    // UNI: the one copy of a gathered tile that serves both read patterns.
    static __device__ __forceinline__ void issue_one(const Lane &L, const elem_t *h, char *buf, const TileSrc &src,
                                                     int fallback) {
        static_assert(UNI, "one copy serves both patterns only in the unified layout");
        const __amdgpu_buffer_rsrc_t r = head_rsrc(h, src.N);
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            int key = src.key(L.ldrow[i]);
            key = key < 0 ? fallback : key;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (EEA_LDS void *)(buf + L.ldlds[i]), 16,
                                                     (unsigned)key * ROWB + 2 * L.ldkcol[i], 0, 0, 0);
        }
    }

    // Band tiles: the copy of the K (or V) tile whose first key is k0. Rows
    // past the end of the sequence lie past the buffer's last record, so the
    // copy fills them with zeros (finite values that the edge mask drops).
    // With dil > 1 (init_lane given the same dil), tile row r is stored row
    // (k0 + r) * dil of the tensor at kh, and N counts the rows of that
    // strided sequence; rows past it still read as zeros.
    // At d = 64 a wave's loads are 8 tile rows apart, and kx(r + 8) =
    // kx(r) ^ 4 while vx(r + 8) = vx(r) (ux(r + 8) = ux(r) ^ 2): load i's
    // offsets follow from load 0's (the row part is a multiple of ROWB, the
    // chunk part below it), so only load 0's stay live.
    static __device__ __forceinline__ int k_off(const Lane &L, int i, int dil) {
        if constexpr (D == 64) return ((L.ldk[0] ^ ((UNI ? 32 : 64) * (i & 1))) + 8 * i * dil * ROWB);
        else return L.ldk[i];
    }
    static __device__ __forceinline__ int v_off(const Lane &L, int i, int dil) {
        if constexpr (D == 64 && UNI) return k_off(L, i, dil);
        else if constexpr (D == 64) return L.ldv[0] + 8 * i * dil * ROWB;
        else return L.ldv[i];
    }
    static __device__ __forceinline__ void issue_k(const Lane &L, const elem_t *kh, int N, char *kbuf, int k0,
                                                   int dil = 1) {
        const __amdgpu_buffer_rsrc_t kr = head_rsrc(kh, (N - 1) * dil + 1);
        const unsigned base = (unsigned)k0 * dil * ROWB;
#pragma unroll
        for (int i = 0; i < SPW; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (EEA_LDS void *)(kbuf + L.ldlds[i]), 16,
                                                     base + k_off(L, i, dil), 0, 0, 0);
    }
    static __device__ __forceinline__ void issue_v(const Lane &L, const elem_t *vh, int N, char *vbuf, int k0,
                                                   int dil = 1) {
        const __amdgpu_buffer_rsrc_t vr = head_rsrc(vh, (N - 1) * dil + 1);
        const unsigned base = (unsigned)k0 * dil * ROWB;
#pragma unroll
        for (int i = 0; i < SPW; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (EEA_LDS void *)(vbuf + L.ldlds[i]), 16,
                                                     base + v_off(L, i, dil), 0, 0, 0);
    }

    static __device__ __forceinline__ void finish(Stage &, char *, char *, int) { wait_vmem(); }

    // Operand pipeline of one matrix phase. The LDS reads of batch b+1 (four
    // operands) are issued before the four MFMAs of batch b, each group fenced
    // by sched_barrier, so every MFMA finds its operand a whole batch after
    // the read was issued instead of waiting out the LDS latency. Operands
    // are taken in an order whose consecutive MFMAs write different
    // accumulators. The recursion keeps every index a compile-time constant.
    static constexpr int kBatch = 4, kSlots = 2 * kBatch;

    template <int I>
    static __device__ __forceinline__ void qk_fetch(bf16x8 (&op)[kSlots], const Lane &L, const char *kbuf) {
        if constexpr (I < KS * MB) {
            constexpr int ks = I / MB, mb = I % MB;
            op[I % kSlots] = *reinterpret_cast<const bf16x8 *>(kbuf + L.krd[ks] + mb * 32 * ROWB);
        }
    }
    template <int B>
    static __device__ __forceinline__ void qk_run(f32x16 (&s)[MB], const QFrag &qf, const Lane &L,
                                                  const char *kbuf, bf16x8 (&op)[kSlots]) {
        constexpr int NB = KS * MB / kBatch;
        if constexpr (B < NB) {
            if constexpr (B + 1 < NB) {
                qk_fetch<kBatch * (B + 1) + 0>(op, L, kbuf);
                qk_fetch<kBatch * (B + 1) + 1>(op, L, kbuf);
                qk_fetch<kBatch * (B + 1) + 2>(op, L, kbuf);
                qk_fetch<kBatch * (B + 1) + 3>(op, L, kbuf);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int I = kBatch * B + u, ks = I / MB, mb = I % MB;
                s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[I % kSlots], qf.x[ks], s[mb], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            qk_run<B + 1>(s, qf, L, kbuf, op);
        }
    }

    static __device__ __forceinline__ void scores(f32x16 (&s)[MB], const QFrag &qf, const Lane &L,
                                                  const char *kbuf) {
        static_assert((KS * MB) % kBatch == 0, "whole batches");
        bf16x8 op[kSlots];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) s[mb] = f32x16{};
        qk_fetch<0>(op, L, kbuf);
        qk_fetch<1>(op, L, kbuf);
        qk_fetch<2>(op, L, kbuf);
        qk_fetch<3>(op, L, kbuf);
        __builtin_amdgcn_sched_barrier(0);
        qk_run<0>(s, qf, L, kbuf, op);
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

    static __device__ __forceinline__ bf16x8 v_operand(const Lane &L, const char *vbuf, int db, int st) {
        const char *p = vbuf + L.vrd[db] + 16 * st * ROWB;
        const char *q = UNI ? vbuf + L.vrdh[db] + 16 * st * ROWB : p + 8 * ROWB;
        s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((EEA_LDS s16x4 *)(p));
        s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((EEA_LDS s16x4 *)(q));
        s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return __builtin_bit_cast(bf16x8, v);
    }

    template <int I>
    static __device__ __forceinline__ void pv_fetch(bf16x8 (&op)[kSlots], const Lane &L, const char *vbuf) {
        if constexpr (I < PVS * DB) op[I % kSlots] = v_operand(L, vbuf, I % DB, I / DB);
    }
    template <int B>
    static __device__ __forceinline__ void pv_run(f32x16 (&o)[DB], const PFrag &pf, const Lane &L,
                                                  const char *vbuf, bf16x8 (&op)[kSlots]) {
        constexpr int NB = PVS * DB / kBatch;
        if constexpr (B < NB) {
            if constexpr (B + 1 < NB) {
                pv_fetch<kBatch * (B + 1) + 0>(op, L, vbuf);
                pv_fetch<kBatch * (B + 1) + 1>(op, L, vbuf);
                pv_fetch<kBatch * (B + 1) + 2>(op, L, vbuf);
                pv_fetch<kBatch * (B + 1) + 3>(op, L, vbuf);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int I = kBatch * B + u, st = I / DB, db = I % DB;
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[I % kSlots], pf.x[st], o[db], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            pv_run<B + 1>(o, pf, L, vbuf, op);
        }
    }

    static __device__ __forceinline__ void pv(f32x16 (&o)[DB], const PFrag &pf, const Lane &L,
                                              const char *vbuf) {
        static_assert((PVS * DB) % kBatch == 0, "whole batches");
        bf16x8 op[kSlots];
        pv_fetch<0>(op, L, vbuf);
        pv_fetch<1>(op, L, vbuf);
        pv_fetch<2>(op, L, vbuf);
        pv_fetch<3>(op, L, vbuf);
        __builtin_amdgcn_sched_barrier(0);
        pv_run<0>(o, pf, L, vbuf, op);
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
                bf16x4 y = __builtin_convertvector(x, bf16x4);
                *reinterpret_cast<bf16x4 *>(dst + db * 32 + 8 * g + 4 * h) = y;
            }
        }
    }
};

// Single (row, key) pairs on the vector ALU, for rules that give a row a
// handful of scattered keys (no dense tile to contract). A lane's operand
// fragment holds the 16-byte chunks 2 ks + h of its row (as load_q reads
// them); its transposed accumulators hold d = 32 db + 8 g + 4 h + e.
// dot_row_half: this lane's half of row . fragment (the other half is in
// lane ^ 32); axpy_row_half: acc += w * row over this lane's accumulator d.
template <int KS>
__device__ __forceinline__ float dot_row_half(const uint16_t *rowp, const bf16x8 (&x)[KS], int h) {
    const u32x4 *r = reinterpret_cast<const u32x4 *>(rowp);
    float part = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 v = __builtin_bit_cast(bf16x8, r[2 * ks + h]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bf16x2 a = {v[2 * e], v[2 * e + 1]};
            const bf16x2 b = {x[ks][2 * e], x[ks][2 * e + 1]};
            part = __builtin_amdgcn_fdot2_f32_bf16(a, b, part, false);
        }
    }
    return part;
}
template <int DB>
__device__ __forceinline__ void axpy_row_half(f32x16 (&acc)[DB], float w, const uint16_t *rowp, int h) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const uint2 v = *reinterpret_cast<const uint2 *>(rowp + db * 32 + 8 * g + 4 * h);
            acc[db][4 * g + 0] += w * __uint_as_float(v.x << 16);
            acc[db][4 * g + 1] += w * __uint_as_float(v.x & 0xffff0000u);
            acc[db][4 * g + 2] += w * __uint_as_float(v.y << 16);
            acc[db][4 * g + 3] += w * __uint_as_float(v.y & 0xffff0000u);
        }
}

// Lane l and lane l^32 hold the same row of a 32x32 accumulator column:
// combine their values.
__device__ __forceinline__ float max_across_halves(float x) {
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

__device__ __forceinline__ float sum_across_halves(float x) {
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

}  // namespace eea
