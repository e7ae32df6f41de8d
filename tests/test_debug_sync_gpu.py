"""The LDS double buffers checked against a fenced build.

libattn_debugsync.so is the same sources compiled with -DATTN_DEBUG_SYNC:
every pipelined copy into LDS is preceded by a full wait and a workgroup
barrier (every wave has finished its earlier reads) and followed by the same
(the copy has landed before any wave goes on), so copies and compute never
overlap. The arithmetic is unchanged, so the optimised library must give the
same bits on every kernel family that pipelines its copies: the bf16 band
forward (512- and 256-thread instances, block rule, dilation, extra tiles,
global rows), the register-staged fp32 forward, the backward passes and
split-cache decoding. Each optimised call is also repeated and must
reproduce its own bits."""
import ctypes

import numpy as np
import pytest

from efficient_exact_attention_amd import workloads as W
from gpu_common import say, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def libs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import efficient_exact_attention_amd as ea
    return ea.lib(), ea.open_library(ea.DEBUG_SYNC_LIB_PATH)


def _mask(m, rand_idx=None):
    import efficient_exact_attention_amd as ea
    return ea._mask(m.get("causal", 0), m.get("win_left", -1), m.get("win_right", -1), m.get("block", 0),
                    m.get("dilation", 1), m.get("global_idx") or None, m.get("stride", 0), m.get("rand_block", 0),
                    m.get("n_rand", 0), rand_idx)


def _opts(dtype):
    import efficient_exact_attention_amd as ea
    return ea._Opts(dtype, 0.0, None, None, 0)


def _check(L, rc):
    assert rc == 0, L.attn_last_error().decode()


def _fwd(L, q, k, v, B, H, H_kv, N, d, m, dtype, lists):
    out = torch.empty_like(q)
    lse = torch.empty(B, H, N, dtype=torch.float32, device="cuda")
    mk = _mask(m, lists.data_ptr() if lists is not None else None)
    op = _opts(dtype)
    _check(L, L.attn_fwd_masked(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, H_kv,
                                N, d, ctypes.byref(mk), ctypes.byref(op)))
    torch.cuda.synchronize()
    return out, lse


def _lists(N, m, seed):
    if not m.get("rand_block"):
        return None
    nb = (N + m["rand_block"] - 1) // m["rand_block"]
    rng = np.random.default_rng(seed)
    return torch.from_numpy(rng.integers(0, nb, size=(nb, m["n_rand"]), dtype=np.int32)).cuda()


FWD = {
    "causal-4096-d128": (1, 8, 8, 4096, 128, dict(causal=1), "bf16"),
    "causal-3000-d64-gqa": (2, 8, 2, 3000, 64, dict(causal=1), "bf16"),
    "narrow-band-d64": (2, 4, 4, 5000, 64, dict(win_left=128, win_right=128), "bf16"),
    "swa-d128": (1, 4, 4, 6000, 128, dict(causal=1, win_left=2047), "bf16"),
    "band-globals-d64": (2, 6, 6, 4097, 64, dict(win_left=256, win_right=256, global_idx=[0, 1, 2, 900, 4000]),
                         "bf16"),
    "block-rule": (1, 4, 4, 2500, 128, dict(block=100, causal=1, global_idx=[5, 1999]), "bf16"),
    "dilation": (1, 4, 4, 3000, 64, dict(dilation=3, causal=1, win_left=300), "bf16"),
    "strided": (1, 4, 4, 3000, 64, dict(stride=16, causal=1, win_left=40, win_right=0, global_idx=[0, 7]), "bf16"),
    "random-block": (1, 4, 4, 3000, 128, dict(rand_block=64, n_rand=3, win_left=64, win_right=64), "bf16"),
    "f32-causal": (1, 4, 4, 1000, 64, dict(causal=1), "f32"),
    "f32-band-globals": (1, 2, 2, 1500, 128, dict(win_left=30, win_right=30, global_idx=[3, 1400]), "f32"),
}


@pytest.mark.parametrize("name", list(FWD))
def test_forward_matches_fenced_build(libs, name):
    import efficient_exact_attention_amd as ea
    opt, dbg = libs
    B, H, H_kv, N, d, m, dt = FWD[name]
    w = W.random_workload(name, B, H, N, d, dtype=dt, causal=m.get("causal", 0), seed=61)
    q, k, v = (to_device(x, dt) for x in W.make_qkv(w))
    k, v = k[:, :H_kv].contiguous(), v[:, :H_kv].contiguous()
    lists = _lists(N, m, 62)
    dtype = ea.ATTN_F32 if dt == "f32" else ea.ATTN_BF16
    say(f"  fenced vs optimised forward {name}: B={B} H={H} H_kv={H_kv} N={N} d={d} {dt} {m}")
    o1, l1 = _fwd(opt, q, k, v, B, H, H_kv, N, d, m, dtype, lists)
    o2, l2 = _fwd(dbg, q, k, v, B, H, H_kv, N, d, m, dtype, lists)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for _ in range(2):
        o3, l3 = _fwd(opt, q, k, v, B, H, H_kv, N, d, m, dtype, lists)
        assert torch.equal(o1, o3) and torch.equal(l1, l3)


BWD = {
    "causal-2048-d128": (1, 4, 4, 2048, 128, dict(causal=1)),
    "band-d64": (2, 4, 4, 3000, 64, dict(win_left=100, win_right=100)),
    "swa-globals-d128": (1, 4, 2, 2500, 128, dict(causal=1, win_left=255, global_idx=[0, 1000, 2400])),
    "random-block": (1, 2, 2, 2000, 64, dict(rand_block=64, n_rand=2, causal=1, win_left=63)),
}


@pytest.mark.parametrize("name", list(BWD))
def test_backward_matches_fenced_build(libs, name):
    import efficient_exact_attention_amd as ea
    opt, dbg = libs
    B, H, H_kv, N, d, m = BWD[name]
    w = W.random_workload(name, B, H, N, d, causal=m.get("causal", 0), seed=63)
    q, k, v = (to_device(x, "bf16") for x in W.make_qkv(w))
    k, v = k[:, :H_kv].contiguous(), v[:, :H_kv].contiguous()
    do = to_device(W.make_tensor(w.with_(seed=64), 0), "bf16")
    lists = _lists(N, m, 65)
    out, lse = _fwd(opt, q, k, v, B, H, H_kv, N, d, m, ea.ATTN_BF16, lists)
    say(f"  fenced vs optimised backward {name}: B={B} H={H} H_kv={H_kv} N={N} d={d} {m}")

    def grads(L):
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        mk = _mask(m, lists.data_ptr() if lists is not None else None)
        op = _opts(ea.ATTN_BF16)
        _check(L, L.attn_bwd_masked(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), do.data_ptr(),
                                    lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, H_kv, N, d,
                                    ctypes.byref(mk), ctypes.byref(op)))
        torch.cuda.synchronize()
        return dq, dk, dv

    g1, g2, g3 = grads(opt), grads(dbg), grads(opt)
    for a, b, c in zip(g1, g2, g3):
        assert torch.equal(a, b) and torch.equal(a, c)


DEC = [
    W.DecodeWorkload("dbg-dec-full", 2, 16, 4, 1, 20000, 128, -1, 0, (20000, 13001), 66),
    W.DecodeWorkload("dbg-dec-multi", 1, 8, 8, 4, 9000, 64, -1, 0, (9000,), 67),
    W.DecodeWorkload("dbg-dec-rolling", 4, 8, 2, 1, 4096, 128, 4095, 1, (30000, 4096, 5000, 100), 68),
]


@pytest.mark.parametrize("w", DEC, ids=[w.name for w in DEC])
def test_decode_matches_fenced_build(libs, w):
    import efficient_exact_attention_amd as ea
    opt, dbg = libs
    q, kc, vc, seq = W.make_decode(w)
    q, kc, vc = (to_device(x, "bf16") for x in (q, kc, vc))
    seq = torch.from_numpy(seq).cuda()
    say(f"  fenced vs optimised decode {w.name}: B={w.B} H={w.H}/{w.H_kv} Nq={w.Nq} S={w.S} d={w.d} "
        f"win={w.win_left} rolling={w.rolling}")

    def run(L):
        out = torch.empty_like(q)
        lse = torch.empty(w.B, w.H, w.Nq, dtype=torch.float32, device="cuda")
        op = _opts(ea.ATTN_BF16)
        _check(L, L.attn_decode(q.data_ptr(), kc.data_ptr(), vc.data_ptr(), seq.data_ptr(), out.data_ptr(),
                                lse.data_ptr(), w.B, w.H, w.H_kv, w.Nq, w.S, w.d, w.win_left, w.rolling,
                                ctypes.byref(op)))
        torch.cuda.synchronize()
        return out, lse

    (o1, l1), (o2, l2), (o3, l3) = run(opt), run(dbg), run(opt)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)
