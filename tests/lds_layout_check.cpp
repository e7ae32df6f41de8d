// Host replay of the bf16 tile path's LDS layouts (attn_tiles.h): for each
// layout, the per-lane copy offsets of init_lane place a tile in a simulated
// LDS image, and every operand read of the kernels (row reads of 16 bytes,
// transpose reads of 8 bytes, at the per-lane offsets of init_lane) must
// find the element it is meant to read and, within each hardware pass, hit
// distinct banks. Exit status 0 when every check holds.
#include "attn_tiles.h"

#include <cstdio>
#include <set>
#include <vector>

using namespace eea;

static int g_fail = 0;
#define CHECK(cond, ...)                 \
    do {                                 \
        if (!(cond)) {                   \
            if (g_fail < 20) {           \
                std::printf(__VA_ARGS__); \
                std::printf("\n");       \
            }                            \
            ++g_fail;                    \
        }                                \
    } while (0)

// One tile of BN rows x D bf16 elements; element (r, e) is tagged r * D + e.
// kind 0: the K copy (ldkcol), 1: the V copy (ldvcol).
template <class P>
static std::vector<int> place(int kind) {
    std::vector<int> lds(P::TILE_BYTES / 2, -1);   // one tag per 2-byte LDS slot
    for (int wave = 0; wave < P::NW; ++wave)
        for (int lane = 0; lane < 64; ++lane) {
            typename P::Lane L;
            P::init_lane(L, lane, wave);
            for (int i = 0; i < P::SPW; ++i) {
                const int row = L.ldrow[i];
                const int col = kind == 0 ? L.ldkcol[i] : L.ldvcol[i];   // element offset of the 16-byte chunk read
                const int dst = L.ldlds[i] + lane * 16;                    // byte offset written (buffer_load ... lds)
                for (int e = 0; e < 8; ++e) {
                    int &slot = lds[dst / 2 + e];
                    CHECK(slot == -1, "D=%d NT=%d UNI=%d kind %d: LDS byte %d written twice", P::D, P::NT, P::UNI,
                          kind, dst + 2 * e);
                    slot = row * P::D + col + e;
                }
            }
        }
    for (size_t x = 0; x < lds.size(); ++x) CHECK(lds[x] >= 0, "D=%d: LDS slot %zu never written", P::D, x);
    return lds;
}

// Row reads (the K operand of S = K Q^T): lane reads 16 bytes at krd[ks] +
// mb * 32 * ROWB = row ln + 32 mb, elements 8 (2 ks + h) .. +7. A pass of a
// 16-byte read serves 16 consecutive lanes, whose chunks must fall on 16
// distinct 16-byte slots of the 256-byte bank window.
template <class P>
static void row_reads(const std::vector<int> &lds) {
    for (int ks = 0; ks < P::KS; ++ks)
        for (int mb = 0; mb < P::MB; ++mb)
            for (int pass = 0; pass < 4; ++pass) {
                std::set<int> slots;
                for (int lane = 16 * pass; lane < 16 * pass + 16; ++lane) {
                    typename P::Lane L;
                    P::init_lane(L, lane, 0);
                    const int ln = lane & 31, h = lane >> 5;
                    const int addr = L.krd[ks] + mb * 32 * P::ROWB;
                    for (int e = 0; e < 8; ++e)
                        CHECK(lds[addr / 2 + e] == (ln + 32 * mb) * P::D + 8 * (2 * ks + h) + e,
                              "D=%d UNI=%d row read ks=%d mb=%d lane %d elem %d: wrong element", P::D, P::UNI, ks, mb,
                              lane, e);
                    slots.insert((addr % 256) / 16);
                }
                CHECK(slots.size() == 16, "D=%d UNI=%d row read ks=%d mb=%d pass %d: %zu distinct slots (bank conflict)",
                      P::D, P::UNI, ks, mb, pass, slots.size());
            }
}

// Transpose reads (the V operand of O^T += V^T P^T): v_operand's two
// 8-byte reads, at vrd[db] + 16 st ROWB and (UNI) vrdh[db] + 16 st ROWB or
// (otherwise) 8 rows further. Lane j of 16-lane group g reads 4 elements of
// key row 16 st + 4 h + j / 4 (+ 8 for the second read) at d = 32 db + 16 (g
// & 1) + 4 (j & 3). A pass serves 32 lanes, whose 8-byte pieces must fall on
// 32 distinct 8-byte slots of the bank window.
template <class P>
static void transpose_reads(const std::vector<int> &lds) {
    for (int db = 0; db < P::DB; ++db)
        for (int st = 0; st < P::PVS; ++st)
            for (int second = 0; second < 2; ++second)
                for (int pass = 0; pass < 2; ++pass) {
                    std::set<int> slots;
                    for (int lane = 32 * pass; lane < 32 * pass + 32; ++lane) {
                        typename P::Lane L;
                        P::init_lane(L, lane, 0);
                        const int g = lane >> 4, j = lane & 15, h = lane >> 5;
                        int addr = L.vrd[db] + 16 * st * P::ROWB;
                        if (second) {
                            if constexpr (P::UNI) addr = L.vrdh[db] + 16 * st * P::ROWB;
                            else addr += 8 * P::ROWB;
                        }
                        const int krow = 16 * st + 4 * h + j / 4 + 8 * second;
                        const int d0 = 32 * db + 16 * (g & 1) + 4 * (j & 3);
                        for (int e = 0; e < 4; ++e)
                            CHECK(lds[addr / 2 + e] == krow * P::D + d0 + e,
                                  "D=%d UNI=%d transpose read db=%d st=%d second=%d lane %d elem %d: wrong element",
                                  P::D, P::UNI, db, st, second, lane, e);
                        slots.insert((addr % 256) / 8);
                    }
                    CHECK(slots.size() == 32,
                          "D=%d UNI=%d transpose read db=%d st=%d second=%d pass %d: %zu distinct slots (bank conflict)",
                          P::D, P::UNI, db, st, second, pass, slots.size());
                }
}

template <int D, int NT, bool UNI>
static void check_layout() {
    typedef Bf16Path<D, NT, UNI> P;
    if constexpr (UNI) {
        const std::vector<int> t = place<P>(0);   // one copy, read both ways
        row_reads<P>(t);
        transpose_reads<P>(t);
        const std::vector<int> tv = place<P>(1);   // the V copy offsets coincide with the K ones
        CHECK(t == tv, "D=%d NT=%d: unified K and V copies differ", D, NT);
    } else {
        row_reads<P>(place<P>(0));         // K tiles are read by rows
        transpose_reads<P>(place<P>(1));   // V tiles are read transposed
    }
}

int main() {
    check_layout<128, 512, false>();
    check_layout<128, 256, false>();
    check_layout<64, 512, false>();
    check_layout<64, 256, false>();
    check_layout<128, 512, true>();
    check_layout<128, 256, true>();
    check_layout<64, 256, true>();
    check_layout<64, 512, true>();
    std::printf("%s: %d failed checks\n", g_fail ? "FAIL" : "ok", g_fail);
    return g_fail ? 1 : 0;
}
