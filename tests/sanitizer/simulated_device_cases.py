"""Cases for the host-sanitizer run (not collected by a plain pytest run: the
host-sanitizer test names this file explicitly, in a child process whose
binding points at the ASan/UBSan build of the host code with the simulated
device of hip_stub.cpp).

Every call goes through the C ABI with host buffers of exactly the sizes the
header states, standing in for device memory; the stub launchers then touch
every byte the kernels would read or write. A workspace-size formula, a
planner or a pointer offset that disagrees with what the kernels index is
reported by AddressSanitizer as a heap overflow; the C ABI code itself runs
under UndefinedBehaviorSanitizer."""
import ctypes
import os

import numpy as np
import pytest

import efficient_exact_attention_amd as ea

pytestmark = pytest.mark.skipif(not os.environ.get("EEA_SANITIZER_LIB"),
                                reason="runs only against the host-sanitizer build")


@pytest.fixture(autouse=True, scope="module")
def _simulated_device():
    L = ea.lib()
    assert ea.library_path() == os.environ["EEA_SANITIZER_LIB"]
    L.eea_stub_simulate_device(1)
    for f in ("eea_stub_malloc_calls", "eea_stub_live_bytes", "eea_stub_launches"):
        getattr(L, f).restype = ctypes.c_longlong
    yield
    L.eea_stub_simulate_device(0)


def _stub(name):
    return int(getattr(ea.lib(), name)())


def buf(nbytes):
    """A host buffer of exactly nbytes standing in for device memory."""
    return np.zeros(max(int(nbytes), 1), np.uint8)


def ptr(a):
    return a.ctypes.data if a is not None else None


def tensors(B, H, H_kv, N, d, es=2):
    q = buf(B * H * N * d * es)
    k = buf(B * H_kv * N * d * es)
    v = buf(B * H_kv * N * d * es)
    out = buf(B * H * N * d * es)
    lse = buf(B * H * N * 4)
    return q, k, v, out, lse


def rand_lists(N, rand_block, n_rand, seed):
    nb = (N + rand_block - 1) // rand_block
    rng = np.random.default_rng(seed)
    return np.ascontiguousarray(rng.integers(0, nb, size=(nb, n_rand), dtype=np.int32))


FWD = [
    dict(B=2, H=3, H_kv=3, N=1000, d=128, causal=1),
    dict(B=1, H=4, H_kv=4, N=3000, d=64, causal=1, win_left=300),
    dict(B=2, H=3, H_kv=3, N=2500, d=64, win_left=40, win_right=40, global_idx=[0, 1, 1024, 2049]),
    dict(B=1, H=8, H_kv=2, N=777, d=128, causal=1, global_idx=[3, 500]),
    dict(B=3, H=2, H_kv=2, N=4097, d=128, win_left=7, win_right=7, global_idx=list(range(0, 4097, 65))),
    dict(B=1, H=2, H_kv=2, N=1000, d=64, block=100, causal=1, global_idx=[5, 999]),
    dict(B=1, H=2, H_kv=2, N=1000, d=128, dilation=3, win_left=7, win_right=2),
    dict(B=1, H=2, H_kv=2, N=1000, d=64, stride=16, causal=1, win_left=40, win_right=0, global_idx=[0, 7, 999]),
    dict(B=1, H=2, H_kv=2, N=1000, d=128, rand_block=64, n_rand=3, causal=1, win_left=63),
    dict(B=1, H=2, H_kv=2, N=1, d=64, causal=1),
    dict(B=1, H=1, H_kv=1, N=500, d=64, causal=1, dtype=ea.ATTN_F32),
    dict(B=1, H=1, H_kv=1, N=300, d=128, win_left=3, win_right=3, global_idx=[299], dtype=ea.ATTN_F32),
]


def _mask_args(c, lists):
    m = {k: c[k] for k in ("causal", "win_left", "win_right", "block", "dilation", "global_idx", "stride",
                           "rand_block", "n_rand") if k in c}
    if lists is not None:
        m["rand_idx"] = lists.ctypes.data
    return m


@pytest.mark.parametrize("c", FWD, ids=[str(i) for i in range(len(FWD))])
@pytest.mark.parametrize("scratch", ["caller", "library"])
def test_forward(c, scratch):
    dtype = c.get("dtype", ea.ATTN_BF16)
    B, H, H_kv, N, d = c["B"], c["H"], c["H_kv"], c["N"], c["d"]
    q, k, v, out, lse = tensors(B, H, H_kv, N, d, 4 if dtype == ea.ATTN_F32 else 2)
    lists = rand_lists(N, c["rand_block"], c["n_rand"], 7) if c.get("rand_block") else None
    ng = len(c.get("global_idx", []))
    ws = None
    if scratch == "caller" and ng:
        ws = buf(ea.attn_workspace_bytes(B, H, N, d, ng))
    launches = _stub("eea_stub_launches")
    ea.attn_fwd_masked(ptr(q), ptr(k), ptr(v), ptr(out), ptr(lse), B, H, H_kv, N, d, dtype=dtype,
                       workspace=ptr(ws), workspace_bytes=0 if ws is None else ws.size, **_mask_args(c, lists))
    assert _stub("eea_stub_launches") == launches + 1


def test_library_scratch_grows_and_is_reused():
    """A larger call replaces the library buffer, a smaller one reuses it."""
    # the middle call (d = 64, 40 global rows fused into the band pass: one
    # partial per query tile) needs all of attn_workspace_bytes
    sizes = [(1, 1, 600, 64, [3]), (3, 8, 4000, 64, list(range(0, 4000, 100))), (1, 2, 900, 64, [0, 1])]
    for B, H, N, d, g in sizes:
        q, k, v, out, lse = tensors(B, H, H, N, d)
        ea.attn_fwd(ptr(q), ptr(k), ptr(v), ptr(out), ptr(lse), B, H, N, d, 0, 8, 8, g)
    big = ea.attn_workspace_bytes(3, 8, 4000, 64, 40)
    assert _stub("eea_stub_live_bytes") >= big


def test_noalloc_allocates_nothing():
    """attn_fwd_noalloc makes no hipMalloc: two calls, the second smaller."""
    before = _stub("eea_stub_malloc_calls")
    for B, H, N, d, g in [(2, 4, 3000, 128, [0, 777, 2999]), (1, 2, 500, 64, [7])]:
        q, k, v, out, lse = tensors(B, H, H, N, d)
        ea.attn_fwd_noalloc(ptr(q), ptr(k), ptr(v), ptr(out), ptr(lse), B, H, N, d, 0, 30, 30, g)
    assert _stub("eea_stub_malloc_calls") == before


def test_noalloc_at_its_limit():
    """The largest global-row partial set that still fits the array."""
    d, ng, N = 128, 64, 4096
    B, H = 1, 1
    while ea.attn_workspace_bytes(B, H * 2, N, d, ng) <= ea.ATTN_NOALLOC_SCRATCH_BYTES:
        H *= 2
    assert ea.attn_workspace_bytes(B, H, N, d, ng) <= ea.ATTN_NOALLOC_SCRATCH_BYTES
    q, k, v, out, lse = tensors(B, H, H, N, d)
    ea.attn_fwd_noalloc(ptr(q), ptr(k), ptr(v), ptr(out), ptr(lse), B, H, N, d, 0, 3, 3, list(range(0, N, 64)))


BWD = [
    dict(B=2, H=4, H_kv=4, N=1000, d=128, causal=1),
    dict(B=1, H=4, H_kv=2, N=3000, d=64, win_left=30, win_right=30, global_idx=[0, 777, 2999]),
    dict(B=2, H=2, H_kv=2, N=2049, d=128, causal=1, win_left=100, global_idx=list(range(0, 2049, 33))),
    dict(B=1, H=2, H_kv=2, N=1000, d=64, block=64, causal=1, global_idx=[0, 130, 777]),
    dict(B=1, H=2, H_kv=2, N=1000, d=128, dilation=2, causal=1),
    dict(B=1, H=2, H_kv=2, N=1000, d=64, stride=3, win_left=5, win_right=5),
    dict(B=1, H=2, H_kv=2, N=999, d=128, rand_block=32, n_rand=3, causal=1, win_left=31, global_idx=[4]),
]


@pytest.mark.parametrize("c", BWD, ids=[str(i) for i in range(len(BWD))])
@pytest.mark.parametrize("scratch", ["caller", "library"])
def test_backward(c, scratch):
    B, H, H_kv, N, d = c["B"], c["H"], c["H_kv"], c["N"], c["d"]
    q, k, v, out, lse = tensors(B, H, H_kv, N, d)
    do, dq = buf(q.size), buf(q.size)
    dk, dv = buf(k.size), buf(v.size)
    lists = rand_lists(N, c["rand_block"], c["n_rand"], 8) if c.get("rand_block") else None
    ng = len(c.get("global_idx", []))
    ws = buf(ea.attn_bwd_workspace_bytes(B, H, N, d, H_kv=H_kv, n_global=ng)) if scratch == "caller" else None
    launches = _stub("eea_stub_launches")
    ea.attn_bwd_masked(ptr(q), ptr(k), ptr(v), ptr(out), ptr(do), ptr(lse), ptr(dq), ptr(dk), ptr(dv), B, H, H_kv,
                       N, d, workspace=ptr(ws), workspace_bytes=0 if ws is None else ws.size,
                       **_mask_args(c, lists))
    assert _stub("eea_stub_launches") == launches + 1


DEC = [
    dict(B=1, H=8, H_kv=8, Nq=1, S=32768, d=128, win=-1, rolling=0),
    dict(B=2, H=32, H_kv=8, Nq=4, S=9000, d=128, win=-1, rolling=0),
    dict(B=3, H=6, H_kv=2, Nq=2, S=5000, d=64, win=1023, rolling=0),
    dict(B=2, H=8, H_kv=1, Nq=1, S=4096, d=128, win=4095, rolling=1),
    dict(B=1, H=4, H_kv=4, Nq=16, S=100, d=64, win=-1, rolling=0),
    dict(B=1, H=64, H_kv=2, Nq=8, S=20000, d=128, win=-1, rolling=0),
]


@pytest.mark.parametrize("c", DEC, ids=[str(i) for i in range(len(DEC))])
@pytest.mark.parametrize("scratch", ["caller", "library"])
def test_decode(c, scratch):
    B, H, H_kv, Nq, S, d = c["B"], c["H"], c["H_kv"], c["Nq"], c["S"], c["d"]
    q, out = buf(B * H * Nq * d * 2), buf(B * H * Nq * d * 2)
    kc, vc = buf(B * H_kv * S * d * 2), buf(B * H_kv * S * d * 2)
    lse = buf(B * H * Nq * 4)
    seq = np.full(B, S if not c["rolling"] else 3 * S, np.int32)
    need = ea.attn_decode_workspace_bytes(B, H, H_kv, Nq, S, d, c["win"], c["rolling"])
    ws = buf(need) if scratch == "caller" and need else None
    ea.attn_decode(ptr(q), ptr(kc), ptr(vc), seq.ctypes.data, ptr(out), ptr(lse), B, H, H_kv, Nq, S, d, c["win"],
                   c["rolling"], workspace=ptr(ws), workspace_bytes=0 if ws is None else ws.size)


def test_random_plan_reads_the_lists():
    """The planner copies the key-block lists from the device (hipMemcpy)."""
    N, rb, nr = 1000, 64, 2
    lists = rand_lists(N, rb, nr, 9)
    pairs, full, edge = ea.attn_plan_stats_masked(N, 128, 64, rand_block=rb, n_rand=nr, rand_idx=lists.ctypes.data,
                                                  causal=1, win_left=63)
    assert pairs > 0 and full + edge > 0
