"""The C ABI on the CPU: exported symbols, host-side validation and the tile
planner. No call here reaches a kernel launch."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import efficient_exact_attention_amd as ea
from efficient_exact_attention_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(ea.library_path()),
                                reason="libattn.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(attn_\w+)\s*\(", src, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"attn_fwd", "attn_fwd_ex", "attn_fwd_gqa", "attn_fwd_masked", "attn_bwd", "attn_bwd_masked",
            "attn_plan_stats_masked", "attn_bwd_workspace_bytes", "attn_decode", "attn_decode_workspace_bytes",
            "attn_workspace_bytes", "attn_plan_stats",
            "attn_last_error", "attn_version", "attn_tile_shape"} <= set(names)
    L = ctypes.CDLL(ea.library_path())
    for n in names:
        assert hasattr(L, n), n


def test_version():
    assert "gfx950" in ea.attn_version()


# ---- validation: every case returns before any HIP call --------------------------

FAKE = 0x7f0000000000          # 16-byte aligned, never dereferenced on the host


def _call(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE + (1 << 32), lse=FAKE + (2 << 32),
             B=1, H=2, N=100, d=128, causal=1, win_left=-1, win_right=-1, global_idx=None)
    opts = {}
    for key in ("dtype", "scale", "workspace", "workspace_bytes"):
        if key in over:
            opts[key] = over.pop(key)
    a.update(over)
    with pytest.raises(ea.AttnError) as ei:
        ea.attn_fwd_ex(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["H"], a["N"], a["d"],
                       a["causal"], a["win_left"], a["win_right"], a["global_idx"], **opts)
    return ei.value


@pytest.mark.parametrize("over,status,text", [
    (dict(q=0), ea.ATTN_ERR_INVALID_ARG, "NULL"),
    (dict(lse=0), ea.ATTN_ERR_INVALID_ARG, "NULL"),
    (dict(B=0), ea.ATTN_ERR_INVALID_ARG, "positive"),
    (dict(N=-3), ea.ATTN_ERR_INVALID_ARG, "positive"),
    (dict(d=96), ea.ATTN_ERR_UNSUPPORTED, "head size"),
    (dict(d=256), ea.ATTN_ERR_UNSUPPORTED, "head size"),
    (dict(causal=2), ea.ATTN_ERR_INVALID_ARG, "causal"),
    (dict(win_left=-2), ea.ATTN_ERR_INVALID_ARG, "window"),
    (dict(win_right=-5), ea.ATTN_ERR_INVALID_ARG, "window"),
    (dict(dtype=7), ea.ATTN_ERR_INVALID_ARG, "dtype"),
    (dict(global_idx=[3, 3], win_left=4), ea.ATTN_ERR_INVALID_ARG, "twice"),
    (dict(global_idx=[100], win_left=4), ea.ATTN_ERR_INVALID_ARG, "outside"),
    (dict(global_idx=[-1], win_left=4), ea.ATTN_ERR_INVALID_ARG, "outside"),
    (dict(global_idx=list(range(65)), win_left=4), ea.ATTN_ERR_UNSUPPORTED, "maximum"),
    (dict(q=FAKE + 8), ea.ATTN_ERR_INVALID_ARG, "aligned"),
    (dict(out=FAKE + (1 << 32) + 2), ea.ATTN_ERR_INVALID_ARG, "aligned"),
    (dict(lse=FAKE + (2 << 32) + 2), ea.ATTN_ERR_INVALID_ARG, "aligned"),
    (dict(out=FAKE + 256), ea.ATTN_ERR_INVALID_ARG, "overlaps"),
    (dict(lse=FAKE + (1 << 32) + 64), ea.ATTN_ERR_INVALID_ARG, "overlaps"),
    (dict(v=FAKE + (1 << 32) + 4096), ea.ATTN_ERR_INVALID_ARG, "overlaps"),
    (dict(N=8388608, d=128), ea.ATTN_ERR_UNSUPPORTED, "2 GiB"),
    (dict(N=4194304, d=128, dtype=ea.ATTN_F32), ea.ATTN_ERR_UNSUPPORTED, "2 GiB"),
    (dict(scale=-1.0), ea.ATTN_ERR_INVALID_ARG, "scale"),
    (dict(scale=float("inf")), ea.ATTN_ERR_INVALID_ARG, "scale"),
    (dict(global_idx=[0, 50], win_left=4, workspace=FAKE + (3 << 32), workspace_bytes=16),
     ea.ATTN_ERR_INVALID_ARG, "workspace"),
])
def test_validation(over, status, text):
    err = _call(**over)
    assert err.status == status
    assert text in err.message


def _call_gqa(H, H_kv, scale=0.0, **over):
    a = dict(q=FAKE, k=FAKE + (3 << 32), v=FAKE + (4 << 32), out=FAKE + (1 << 32), lse=FAKE + (2 << 32),
             B=2, N=100, d=128)
    a.update(over)
    with pytest.raises(ea.AttnError) as ei:
        ea.attn_fwd_gqa(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], H, H_kv, a["N"], a["d"],
                        1, -1, -1, None, scale=scale)
    return ei.value


@pytest.mark.parametrize("H,H_kv", [(8, 0), (8, -1), (8, 3), (6, 4), (4, 8)])
def test_gqa_head_counts(H, H_kv):
    err = _call_gqa(H, H_kv)
    assert err.status == ea.ATTN_ERR_INVALID_ARG
    assert "H_kv" in err.message


def test_gqa_overlap_uses_kv_size():
    """k holds B*H_kv heads (here 2): an out buffer inside them is rejected,
    one starting right after them passes the overlap check (the call is
    then stopped by the invalid scale, which is checked after it, so no case
    reaches the device)."""
    head = 100 * 128 * 2
    kv = FAKE + (3 << 32)
    err = _call_gqa(8, 1, k=kv, out=kv + head)
    assert "overlaps" in err.message
    err = _call_gqa(8, 1, scale=-1.0, k=kv, v=kv + (1 << 30), out=kv + 2 * head, lse=kv + (1 << 31))
    assert "scale" in err.message


def _call_bwd(**over):
    base = FAKE
    a = dict(q=base, k=base + (1 << 32), v=base + (2 << 32), out=base + (3 << 32), dout=base + (4 << 32),
             lse=base + (5 << 32), dq=base + (6 << 32), dk=base + (7 << 32), dv=base + (8 << 32),
             B=1, H=4, H_kv=2, N=100, d=128, causal=1, win_left=-1, win_right=-1, global_idx=None)
    opts = {}
    for key in ("dtype", "scale", "workspace", "workspace_bytes"):
        if key in over:
            opts[key] = over.pop(key)
    a.update(over)
    with pytest.raises(ea.AttnError) as ei:
        ea.attn_bwd(a["q"], a["k"], a["v"], a["out"], a["dout"], a["lse"], a["dq"], a["dk"], a["dv"],
                    a["B"], a["H"], a["H_kv"], a["N"], a["d"], a["causal"], a["win_left"], a["win_right"],
                    a["global_idx"], **opts)
    return ei.value


@pytest.mark.parametrize("over,status,text", [
    (dict(dout=0), ea.ATTN_ERR_INVALID_ARG, "NULL"),
    (dict(dv=0), ea.ATTN_ERR_INVALID_ARG, "NULL"),
    (dict(H_kv=3), ea.ATTN_ERR_INVALID_ARG, "H_kv"),
    (dict(d=96), ea.ATTN_ERR_UNSUPPORTED, "head size"),
    (dict(dtype=ea.ATTN_F32), ea.ATTN_ERR_UNSUPPORTED, "bf16"),
    (dict(global_idx=[0, 50, 50], win_left=4, causal=0, win_right=4), ea.ATTN_ERR_INVALID_ARG, "twice"),
    (dict(global_idx=list(range(65)), win_left=4), ea.ATTN_ERR_UNSUPPORTED, "maximum"),
    (dict(dq=FAKE + (1 << 32) + 64), ea.ATTN_ERR_INVALID_ARG, "overlaps an input"),
    (dict(dk=FAKE + (6 << 32) + 1024), ea.ATTN_ERR_INVALID_ARG, "overlap"),
    (dict(dk=FAKE + (7 << 32) + 8), ea.ATTN_ERR_INVALID_ARG, "aligned"),
    (dict(scale=-2.0), ea.ATTN_ERR_INVALID_ARG, "scale"),
    (dict(workspace=FAKE + (9 << 32), workspace_bytes=64), ea.ATTN_ERR_INVALID_ARG, "workspace"),
    (dict(workspace=FAKE + (6 << 32), workspace_bytes=1 << 20), ea.ATTN_ERR_INVALID_ARG, "workspace overlaps"),
])
def test_bwd_validation(over, status, text):
    err = _call_bwd(**over)
    assert err.status == status, err.message
    assert text in err.message, err.message


def test_bwd_globals_are_accepted():
    """Global tokens with a window pass validation (the call then stops on
    the invalid scale, before the device)."""
    err = _call_bwd(global_idx=[0, 50], win_left=4, causal=0, win_right=4, scale=-1.0)
    assert err.status == ea.ATTN_ERR_INVALID_ARG and "scale" in err.message


def test_bwd_globals_covered_by_window_are_accepted():
    """Global tokens add nothing when the window already covers every visible
    key (causal, unbounded left): validation passes them (the call then stops
    on the invalid scale, before the device)."""
    err = _call_bwd(global_idx=[0, 7], causal=1, win_left=-1, scale=-1.0)
    assert "scale" in err.message


def test_bwd_workspace_bytes():
    assert ea.attn_bwd_workspace_bytes(2, 8, 1000, 128) == 2 * ((2 * 8 * 1000 * 4 + 255) // 256 * 256)
    assert ea.attn_bwd_workspace_bytes(0, 8, 1000, 128) == 0
    assert ea.attn_bwd_workspace_bytes(1, 1, 16, 96) == 0
    # global tokens add the split passes' partials: O(n_global d N / 64) per head
    base = ea.attn_bwd_workspace_bytes(2, 12, 16384, 64)
    with_g = ea.attn_bwd_workspace_bytes(2, 12, 16384, 64, H_kv=4, n_global=9)
    assert base < with_g < base + 2 * 12 * 9 * 64 * 4 * (16384 // 64) * 3
    assert ea.attn_bwd_workspace_bytes(2, 12, 16384, 64, H_kv=5, n_global=9) == 0
    assert ea.attn_bwd_workspace_bytes(2, 12, 16384, 64, n_global=65) == 0


def _call_masked(mask=None, dtype=ea.ATTN_BF16, **m):
    with pytest.raises(ea.AttnError) as ei:
        if mask is False:
            L = ea.lib()
            opts = ea._Opts(dtype, 0.0, None, None, 0)
            ea._check(L.attn_fwd_masked(FAKE, FAKE + (1 << 32), FAKE + (2 << 32), FAKE + (3 << 32),
                                        FAKE + (4 << 32), 1, 2, 2, 100, 128, None, ctypes.byref(opts)))
        else:
            ea.attn_fwd_masked(FAKE, FAKE + (1 << 32), FAKE + (2 << 32), FAKE + (3 << 32), FAKE + (4 << 32),
                               1, 2, 2, 100, 128, dtype=dtype, **m)
    return ei.value


@pytest.mark.parametrize("m,status,text", [
    (dict(block=16, win_left=3), ea.ATTN_ERR_INVALID_ARG, "replaces the window"),
    (dict(block=16, dilation=2), ea.ATTN_ERR_UNSUPPORTED, "cannot be combined"),
    (dict(dilation=3, global_idx=[5]), ea.ATTN_ERR_UNSUPPORTED, "dilated"),
    (dict(block=-1), ea.ATTN_ERR_INVALID_ARG, "block"),
    (dict(dilation=-2), ea.ATTN_ERR_INVALID_ARG, "dilation"),
    (dict(dilation=2, dtype=ea.ATTN_F32), ea.ATTN_ERR_UNSUPPORTED, "bf16"),
    (dict(dilation=2, causal=1, scale=-1.0), ea.ATTN_ERR_INVALID_ARG, "scale"),
])
def test_masked_validation(m, status, text):
    dtype = m.pop("dtype", ea.ATTN_BF16)
    err = _call_masked(dtype=dtype, **m)
    assert err.status == status, err.message
    assert text in err.message, err.message


def test_masked_null_mask():
    err = _call_masked(mask=False)
    assert err.status == ea.ATTN_ERR_INVALID_ARG and "mask" in err.message


def test_bwd_rejects_dilation_with_globals():
    err = _call_bwd_masked(dilation=2, global_idx=[0, 50])
    assert err.status == ea.ATTN_ERR_UNSUPPORTED and "dilated" in err.message


def test_bwd_accepts_dilation():
    """A dilated mask passes validation (the call then stops on the invalid
    scale, before the device)."""
    err = _call_bwd_masked(dilation=2, causal=1, scale=-1.0)
    assert err.status == ea.ATTN_ERR_INVALID_ARG and "scale" in err.message


def _call_bwd_masked(**m):
    base = FAKE
    with pytest.raises(ea.AttnError) as ei:
        ea.attn_bwd_masked(base, base + (1 << 32), base + (2 << 32), base + (3 << 32), base + (4 << 32),
                           base + (5 << 32), base + (6 << 32), base + (7 << 32), base + (8 << 32),
                           1, 4, 2, 100, 128, **m)
    return ei.value


@pytest.mark.parametrize("N", [1, 63, 64, 300, 1000])
@pytest.mark.parametrize("m", [dict(block=64), dict(block=64, causal=1), dict(block=100, causal=1),
                               dict(block=7), dict(block=3000), dict(dilation=2, causal=1),
                               dict(dilation=3), dict(dilation=5, win_left=7, win_right=2),
                               dict(dilation=4, causal=1, win_left=20, win_right=0),
                               dict(block=50, causal=1, global_idx=[0, 17])])
def test_masked_plan_pairs_match_oracle(N, m):
    G = tuple(g for g in m.get("global_idx", ()) if g < N)
    mm = dict(m, global_idx=list(G))
    pairs = ea.attn_plan_stats_masked(N, 256, 64, **mm)[0]
    ref = oracle.visible_pairs_bruteforce(N, m.get("causal", 0), m.get("win_left", -1), m.get("win_right", -1),
                                          G, block=m.get("block", 0), dilation=m.get("dilation", 1))
    assert pairs == ref


@pytest.mark.parametrize("N,b", [(300, 64), (1000, 100), (513, 7)])
@pytest.mark.parametrize("causal", [0, 1])
def test_block_tiles_match_bruteforce(N, b, causal):
    """Tile classes of the block rule against the oracle's mask, tile by tile."""
    vis = oracle.mask_rows(np.arange(N), N, causal, -1, -1, (), b, 1)
    full = edge = 0
    for q0 in range(0, N, 256):
        for k0 in range(0, N, 64):
            blk = vis[q0:q0 + 256, k0:k0 + 64]
            if not blk.any():
                continue
            if blk.all() and blk.shape == (min(256, N - q0), 64):
                full += 1
            else:
                edge += 1
    _, f, e = ea.attn_plan_stats_masked(N, 256, 64, causal=causal, block=b)
    assert (f, e) == (full, edge)


def test_inputs_may_alias():
    """q = k = v is allowed; with a valid request the call proceeds to the device
    (on a machine without a GPU that is a DEVICE error, never a crash)."""
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("would launch on fake pointers")
    except ImportError:
        pass
    err = _call(q=FAKE, k=FAKE, v=FAKE)
    assert err.status == ea.ATTN_ERR_DEVICE


def test_tile_shape():
    assert ea.attn_tile_shape(128) == (256, 64)
    assert ea.attn_tile_shape(64) == (256, 64)
    assert ea.attn_tile_shape(64, ea.ATTN_F32) == (128, 32)
    with pytest.raises(ea.AttnError):
        ea.attn_tile_shape(80)


def test_workspace_bytes():
    assert ea.attn_workspace_bytes(2, 12, 16384, 64, 0) == 0
    a = ea.attn_workspace_bytes(2, 12, 16384, 64, 9)
    b = ea.attn_workspace_bytes(2, 12, 16384, 64, 18)
    assert a > 0 and b == 2 * a
    # bounded by B*H*n_global*(N/32)*(d+2) floats: linear in N, never N^2
    assert a <= 2 * 12 * 9 * (16384 // 32) * 66 * 4
    assert ea.attn_workspace_bytes(0, 12, 16384, 64, 9) == 0
    assert ea.attn_workspace_bytes(1, 1, 16, 96, 1) == 0


# ---- planner: pair counts and tile classes against brute force ---------------------

def brute_tiles(N, m, bm, bn):
    """Classify every (query tile, key tile) of the band by evaluating the
    oracle's mask (global columns and rows excluded: they have their own passes)."""
    vis = oracle.mask_rows(np.arange(N), N, m["causal"], m["win_left"], m["win_right"], ())
    full = edge = 0
    for q0 in range(0, N, bm):
        for k0 in range(0, N, bn):
            blk = vis[q0:q0 + bm, k0:k0 + bn]
            if not blk.any():
                continue
            if blk.all() and blk.shape == (min(bm, N - q0), bn):
                full += 1
            else:
                edge += 1
    return full, edge


MASKS = [
    dict(causal=1, win_left=-1, win_right=-1),
    dict(causal=0, win_left=-1, win_right=-1),
    dict(causal=1, win_left=40, win_right=-1),
    dict(causal=1, win_left=0, win_right=-1),
    dict(causal=0, win_left=17, win_right=17),
    dict(causal=0, win_left=3, win_right=70),
    dict(causal=0, win_left=0, win_right=0),
]


@pytest.mark.parametrize("m", MASKS)
@pytest.mark.parametrize("N", [1, 37, 128, 300, 517])
@pytest.mark.parametrize("bm,bn", [(128, 64), (64, 32), (16, 16)])
def test_plan_matches_bruteforce(m, N, bm, bn):
    pairs, full, edge = ea.attn_plan_stats(N, m["causal"], m["win_left"], m["win_right"], None, bm, bn)
    assert pairs == oracle.visible_pairs_bruteforce(N, m["causal"], m["win_left"], m["win_right"])
    assert (full, edge) == brute_tiles(N, m, bm, bn)


@pytest.mark.parametrize("N,m,G", [
    (300, dict(causal=0, win_left=10, win_right=10), (0, 1, 150, 299)),
    (300, dict(causal=1, win_left=10, win_right=-1), (0, 5, 200)),
    (97, dict(causal=0, win_left=0, win_right=3), (50,)),
    (64, dict(causal=1, win_left=-1, win_right=-1), (3, 9)),       # band covers all
    (64, dict(causal=0, win_left=-1, win_right=-1), (3, 9)),
])
def test_plan_pairs_with_globals(N, m, G):
    pairs, _, _ = ea.attn_plan_stats(N, m["causal"], m["win_left"], m["win_right"], G, 128, 64)
    assert pairs == oracle.visible_pairs_bruteforce(N, m["causal"], m["win_left"], m["win_right"], G)


def test_plan_workloads():
    """Pairs per head of the benchmark workloads and their tile counts at 128x64."""
    got = {k: ea.attn_plan_stats(w.N, w.causal, w.win_left, w.win_right, w.global_idx, 128, 64)
           for k, w in W.WORKLOADS.items()}
    assert got["causal_4k_b4"] == (8_390_656, 992, 64)
    assert got["swa4096_32k"] == (125_831_168, 14_880, 960)
    assert got["causal_131k"][0] == 8_590_000_128
    assert got["causal_32k"] == (536_887_296, 65_280, 512)
    pairs, full, edge = got["band256_globals_16k"]
    assert pairs == 8_625_830
    # band-only tiles (global columns are handled by the gathered tile, so they
    # do not turn band tiles into edge tiles): 764 full + 504 edge, the same
    # as brute force over the band mask; plus one gathered tile per query tile
    # (128) and one 64-key tile run per global row (9 x 256)
    assert full == 764 and edge == 504 + 128 + 9 * 256


def test_window_equivalence_gives_same_plan():
    a = ea.attn_plan_stats(1000, 1, -1, -1, None, 128, 64)
    for wl in (999, 5000):
        assert ea.attn_plan_stats(1000, 1, wl, 0, None, 128, 64) == a


# ---- decoding: validation only (no call reaches the device) -----------------------

def _call_decode(**over):
    a = dict(q=FAKE, k=FAKE + (1 << 32), v=FAKE + (2 << 32), seq=FAKE + (3 << 32), out=FAKE + (4 << 32),
             lse=FAKE + (5 << 32), B=2, H=8, H_kv=2, Nq=1, S=1000, d=128, win_left=-1, rolling=0)
    opts = {}
    for key in ("dtype", "scale", "workspace", "workspace_bytes"):
        if key in over:
            opts[key] = over.pop(key)
    a.update(over)
    with pytest.raises(ea.AttnError) as ei:
        ea.attn_decode(a["q"], a["k"], a["v"], a["seq"], a["out"], a["lse"], a["B"], a["H"], a["H_kv"],
                       a["Nq"], a["S"], a["d"], a["win_left"], a["rolling"], **opts)
    return ei.value


@pytest.mark.parametrize("over,status,text", [
    (dict(q=0), ea.ATTN_ERR_INVALID_ARG, "NULL"),
    (dict(seq=0), ea.ATTN_ERR_INVALID_ARG, "NULL"),
    (dict(B=0), ea.ATTN_ERR_INVALID_ARG, "positive"),
    (dict(Nq=0), ea.ATTN_ERR_INVALID_ARG, "positive"),
    (dict(S=-1), ea.ATTN_ERR_INVALID_ARG, "positive"),
    (dict(H_kv=3), ea.ATTN_ERR_INVALID_ARG, "divide"),
    (dict(H_kv=0), ea.ATTN_ERR_INVALID_ARG, "divide"),
    (dict(dtype=ea.ATTN_F32), ea.ATTN_ERR_UNSUPPORTED, "bf16"),
    (dict(d=96), ea.ATTN_ERR_UNSUPPORTED, "head size"),
    (dict(win_left=-2), ea.ATTN_ERR_INVALID_ARG, "win_left"),
    (dict(rolling=2), ea.ATTN_ERR_INVALID_ARG, "rolling"),
    (dict(Nq=1001), ea.ATTN_ERR_INVALID_ARG, "do not fit"),
    (dict(rolling=1), ea.ATTN_ERR_INVALID_ARG, "rolling cache"),
    (dict(rolling=1, win_left=1000), ea.ATTN_ERR_INVALID_ARG, "rolling cache"),
    (dict(rolling=1, Nq=4, win_left=997), ea.ATTN_ERR_INVALID_ARG, "rolling cache"),
    (dict(q=FAKE + 8), ea.ATTN_ERR_INVALID_ARG, "aligned"),
    (dict(seq=FAKE + (3 << 32) + 2), ea.ATTN_ERR_INVALID_ARG, "aligned"),
    (dict(out=FAKE + 512), ea.ATTN_ERR_INVALID_ARG, "overlaps"),
    (dict(lse=FAKE + (4 << 32) + 64), ea.ATTN_ERR_INVALID_ARG, "overlaps"),
    (dict(scale=-1.0), ea.ATTN_ERR_INVALID_ARG, "scale"),
    (dict(workspace=FAKE + (9 << 32), workspace_bytes=64), ea.ATTN_ERR_INVALID_ARG, "workspace"),
    # a valid rolling configuration passes every check and stops at the scale
    (dict(rolling=1, Nq=4, win_left=996, scale=-1.0), ea.ATTN_ERR_INVALID_ARG, "scale"),
])
def test_decode_validation(over, status, text):
    err = _call_decode(**over)
    assert err.status == status, err.message
    assert text in err.message, err.message


def test_decode_workspace_bytes():
    for (B, H, Hkv, Nq, S, d, wl, roll) in [(1, 32, 8, 1, 32768, 128, -1, 0), (4, 8, 8, 4, 1000, 64, -1, 0),
                                            (2, 64, 1, 1, 4096, 128, -1, 0), (1, 8, 8, 1, 32768, 128, 4095, 0),
                                            (1, 8, 2, 1, 4096, 128, 4095, 1)]:
        n = ea.attn_decode_workspace_bytes(B, H, Hkv, Nq, S, d, wl, roll)
        chunks = n // (B * H * Nq * (d + 2) * 4)
        assert n == B * H * Nq * (d + 2) * 4 * chunks
        assert 2 <= chunks <= min(256, (S + 63) // 64)      # one partial per chunk
    # a window bounds the chunks of a contiguous cache by the window's tiles
    assert ea.attn_decode_workspace_bytes(1, 8, 8, 1, 32768, 128, 127, 0) // (8 * 130 * 4) <= 4
    # thousands of sequences: one chunk each, no partials
    assert ea.attn_decode_workspace_bytes(512, 64, 8, 1, 4096, 128, 4095, 1) == 0
    assert ea.attn_decode_workspace_bytes(1, 6, 4, 1, 100, 128) == 0
    assert ea.attn_decode_workspace_bytes(1, 8, 8, 1, 100, 96) == 0


# ---- strided and random-block rules: validation and planning ---------------------

@pytest.mark.parametrize("m,dtype,status,text", [
    (dict(stride=-1), ea.ATTN_BF16, ea.ATTN_ERR_INVALID_ARG, "stride"),
    (dict(rand_block=-1), ea.ATTN_BF16, ea.ATTN_ERR_INVALID_ARG, "rand_block"),
    (dict(stride=2, rand_block=64, n_rand=1, rand_idx=FAKE), ea.ATTN_BF16, ea.ATTN_ERR_UNSUPPORTED, "combined"),
    (dict(stride=2, block=16), ea.ATTN_BF16, ea.ATTN_ERR_UNSUPPORTED, "window only"),
    (dict(stride=2, dilation=2), ea.ATTN_BF16, ea.ATTN_ERR_UNSUPPORTED, "window only"),
    (dict(rand_block=48, n_rand=1, rand_idx=FAKE), ea.ATTN_BF16, ea.ATTN_ERR_UNSUPPORTED, "multiple of 32"),
    (dict(rand_block=64, n_rand=0, rand_idx=FAKE), ea.ATTN_BF16, ea.ATTN_ERR_INVALID_ARG, "n_rand"),
    (dict(rand_block=64, n_rand=17, rand_idx=FAKE), ea.ATTN_BF16, ea.ATTN_ERR_INVALID_ARG, "n_rand"),
    (dict(rand_block=64, n_rand=2, rand_idx=None), ea.ATTN_BF16, ea.ATTN_ERR_INVALID_ARG, "NULL"),
    (dict(rand_block=64, n_rand=2, rand_idx=FAKE + 2), ea.ATTN_BF16, ea.ATTN_ERR_INVALID_ARG, "aligned"),
    (dict(stride=3, win_left=2, win_right=2), ea.ATTN_F32, ea.ATTN_ERR_UNSUPPORTED, "bf16"),
    # valid configurations pass every check and stop at the scale
    (dict(stride=3, win_left=2, win_right=2, scale=-1.0), ea.ATTN_BF16, ea.ATTN_ERR_INVALID_ARG, "scale"),
    (dict(rand_block=32, n_rand=3, rand_idx=FAKE, causal=1, win_left=31, scale=-1.0), ea.ATTN_BF16,
     ea.ATTN_ERR_INVALID_ARG, "scale"),
])
def test_extra_rule_validation(m, dtype, status, text):
    err = _call_masked(dtype=dtype, **m)
    assert err.status == status, err.message
    assert text in err.message, err.message


def test_extra_rules_accepted_by_backward():
    """The strided and random-block rules pass the backward's validation
    (the call then stops on the invalid scale, before the device)."""
    err = _call_bwd_masked(stride=2, win_left=3, win_right=3, scale=-1.0)
    assert err.status == ea.ATTN_ERR_INVALID_ARG and "scale" in err.message
    err = _call_bwd_masked(rand_block=48, n_rand=1, rand_idx=FAKE, win_left=3, win_right=3)
    assert err.status == ea.ATTN_ERR_UNSUPPORTED and "multiple of 32" in err.message


def test_random_plan_stats_validation_before_the_copy():
    """Invalid random-block fields are reported before the planner reads the
    device lists."""
    with pytest.raises(ea.AttnError) as ei:
        ea.attn_plan_stats_masked(100, 128, 64, rand_block=48, n_rand=1, rand_idx=FAKE, win_left=2, win_right=2)
    assert ei.value.status == ea.ATTN_ERR_UNSUPPORTED


@pytest.mark.parametrize("N", [1, 63, 300, 1000, 4097])
@pytest.mark.parametrize("m", [dict(stride=1, causal=1, win_left=0, win_right=0),
                               dict(stride=3, causal=0, win_left=5, win_right=5),
                               dict(stride=16, causal=1, win_left=40, win_right=0, global_idx=[0, 7, 999]),
                               dict(stride=2, causal=0, win_left=0, win_right=0, global_idx=[10]),
                               dict(stride=5000, causal=1, win_left=3, win_right=0)])
def test_strided_plan_pairs_match_oracle(N, m):
    G = [g for g in m.get("global_idx", []) if g < N]
    mm = dict(m, global_idx=G)
    pairs = ea.attn_plan_stats_masked(N, 128, 64, **mm)[0]
    ref = oracle.visible_pairs_bruteforce(N, m["causal"], m["win_left"], m["win_right"], tuple(G), stride=m["stride"])
    assert pairs == ref


# ---- the allocation-free forward: its own limits, checked before any HIP call ---------

def test_noalloc_rejects_a_workspace():
    L = ea.lib()
    opts = ea._Opts(ea.ATTN_BF16, 0.0, None, FAKE + (3 << 32), 1 << 20)
    g = (ctypes.c_int * 1)(5)
    rc = L.attn_fwd_noalloc(FAKE, FAKE, FAKE, FAKE + (1 << 32), FAKE + (2 << 32), 1, 2, 100, 128, 0, 3, 3, g, 1,
                            ctypes.byref(opts))
    assert rc == ea.ATTN_ERR_INVALID_ARG and "workspace" in ea.attn_last_error()


def test_noalloc_rejects_more_partials_than_its_array():
    """4096 heads x 64 global rows of partials: far beyond the built-in array."""
    L = ea.lib()
    B, H, N, d = 64, 64, 640, 128
    need = ea.attn_workspace_bytes(B, H, N, d, 64)
    assert need > ea.ATTN_NOALLOC_SCRATCH_BYTES
    g = (ctypes.c_int * 64)(*range(0, 640, 10))
    big = 1 << 36   # tensors of this call are ~1.3 GB: keep the fake ranges apart
    rc = L.attn_fwd_noalloc(FAKE, FAKE, FAKE, FAKE + big, FAKE + 2 * big, B, H, N, d, 0, 3, 3, g, 64, None)
    assert rc == ea.ATTN_ERR_UNSUPPORTED, ea.attn_last_error()
    assert "attn_fwd_noalloc" in ea.attn_last_error()


def test_noalloc_limit_matches_header():
    src = open(HEADER).read()
    m = re.search(r"#define ATTN_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == ea.ATTN_NOALLOC_SCRATCH_BYTES
