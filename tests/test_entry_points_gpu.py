"""The plain entry points attn_fwd and attn_fwd_ex, called through ctypes
with torch device pointers: the default (NULL) stream, NULL options and the
library-owned global-row scratch. Their results must equal attn_fwd_masked's
bit for bit (the same kernels run), and the fp32 N=256 workload must match
the oracle."""
import ctypes

import numpy as np
import pytest

from efficient_exact_attention_amd import workloads as W
from gpu_common import all_heads, check, host_f64, say, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import efficient_exact_attention_amd as ea
    ea.lib()


def _gidx(g):
    if not g:
        return None, 0
    return (ctypes.c_int * len(g))(*g), len(g)


def _masked(w, q, k, v):
    """attn_fwd_masked on torch's stream with a caller workspace."""
    import efficient_exact_attention_amd as ea
    ws = None
    if w.global_idx:
        ws = torch.empty(ea.attn_workspace_bytes(w.B, w.H, w.N, w.d, len(w.global_idx)), dtype=torch.uint8,
                         device="cuda")
    o, l = ea.fwd(q, k, v, causal=w.causal, win_left=w.win_left, win_right=w.win_right,
                  global_idx=w.global_idx or None, workspace=ws)
    torch.cuda.synchronize()
    return o, l


CASES = [
    W.random_workload("ep-causal", 2, 3, 1000, 128, causal=1, seed=41),
    W.random_workload("ep-swa", 1, 4, 3000, 64, causal=1, win_left=300, seed=42),
    W.random_workload("ep-band-g", 2, 3, 2500, 64, causal=0, win_left=40, win_right=40,
                      global_idx=(0, 1, 1024, 2049), seed=43),
    W.random_workload("ep-causal-g", 1, 2, 1800, 128, causal=1, win_left=100, global_idx=(5, 900), seed=44),
]


@pytest.mark.parametrize("w", CASES, ids=[c.name for c in CASES])
def test_attn_fwd_null_stream_matches_masked(w):
    """attn_fwd: bf16, default scale, NULL stream, library scratch for the
    global rows; bitwise the attn_fwd_masked result."""
    import efficient_exact_attention_amd as ea
    qkv = W.make_qkv(w)
    q, k, v = (to_device(x, w.dtype) for x in qkv)
    out = torch.empty_like(q)
    lse = torch.empty(w.B, w.H, w.N, dtype=torch.float32, device="cuda")
    g, ng = _gidx(list(w.global_idx))
    say(f"  attn_fwd {w.name}: B={w.B} H={w.H} N={w.N} d={w.d} causal={w.causal} wl={w.win_left} "
        f"wr={w.win_right} globals={ng}")
    torch.cuda.synchronize()
    rc = ea.lib().attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                           w.B, w.H, w.N, w.d, w.causal, w.win_left, w.win_right, g, ng)
    assert rc == ea.ATTN_OK, ea.attn_last_error()
    torch.cuda.synchronize()
    o2, l2 = _masked(w, q, k, v)
    assert torch.equal(out, o2) and torch.equal(lse, l2)
    check(w, out, lse, all_heads(w), np.arange(w.N), qkv)


@pytest.mark.parametrize("w", CASES[2:], ids=[c.name for c in CASES[2:]])
def test_attn_fwd_ex_null_opts_matches_masked(w):
    """attn_fwd_ex with opts = NULL (every default) gives the same bits."""
    import efficient_exact_attention_amd as ea
    qkv = W.make_qkv(w)
    q, k, v = (to_device(x, w.dtype) for x in qkv)
    out = torch.empty_like(q)
    lse = torch.empty(w.B, w.H, w.N, dtype=torch.float32, device="cuda")
    g, ng = _gidx(list(w.global_idx))
    say(f"  attn_fwd_ex(opts=NULL) {w.name}")
    torch.cuda.synchronize()
    rc = ea.lib().attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                              w.B, w.H, w.N, w.d, w.causal, w.win_left, w.win_right, g, ng, None)
    assert rc == ea.ATTN_OK, ea.attn_last_error()
    torch.cuda.synchronize()
    o2, l2 = _masked(w, q, k, v)
    assert torch.equal(out, o2) and torch.equal(lse, l2)


def test_attn_fwd_ex_f32_workload_against_oracle():
    """The fp32 N=256 workload through attn_fwd_ex (dtype ATTN_F32, NULL
    stream, no workspace) against the oracle, and bitwise against
    attn_fwd_masked."""
    import efficient_exact_attention_amd as ea
    w = W.WORKLOADS["f32_causal_256"]
    qkv = W.make_qkv(w)
    q, k, v = (to_device(x, w.dtype) for x in qkv)
    out = torch.empty_like(q)
    lse = torch.empty(w.B, w.H, w.N, dtype=torch.float32, device="cuda")
    say(f"  attn_fwd_ex fp32 {w.name}")
    torch.cuda.synchronize()
    ea.attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), w.B, w.H, w.N, w.d,
                   w.causal, w.win_left, w.win_right, None, dtype=ea.ATTN_F32, stream=None)
    torch.cuda.synchronize()
    check(w, out, lse, all_heads(w), np.arange(w.N), qkv, tol=(1e-4, 1e-5, 1e-4), strict=True)
    o2, l2 = _masked(w, q, k, v)
    assert torch.equal(out, o2) and torch.equal(lse, l2)


def test_library_scratch_grows_between_calls():
    """A call needing more global-row scratch than an earlier one grows the
    library buffer; the second result must still equal the masked call's."""
    import efficient_exact_attention_amd as ea
    small = W.random_workload("ep-small", 1, 1, 600, 64, causal=0, win_left=8, win_right=8, global_idx=(3,),
                              seed=45)
    big = W.random_workload("ep-big", 3, 8, 4000, 128, causal=0, win_left=8, win_right=8,
                            global_idx=tuple(range(0, 4000, 100)), seed=46)
    assert ea.attn_workspace_bytes(big.B, big.H, big.N, big.d, len(big.global_idx)) > \
        ea.attn_workspace_bytes(small.B, small.H, small.N, small.d, 1)
    for w in (small, big):
        qkv = W.make_qkv(w)
        q, k, v = (to_device(x, w.dtype) for x in qkv)
        out = torch.empty_like(q)
        lse = torch.empty(w.B, w.H, w.N, dtype=torch.float32, device="cuda")
        g, ng = _gidx(list(w.global_idx))
        say(f"  attn_fwd {w.name}: globals={ng}")
        rc = ea.lib().attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                               w.B, w.H, w.N, w.d, w.causal, w.win_left, w.win_right, g, ng)
        assert rc == ea.ATTN_OK, ea.attn_last_error()
        torch.cuda.synchronize()
        o2, l2 = _masked(w, q, k, v)
        assert torch.equal(out, o2) and torch.equal(lse, l2)
        assert np.isfinite(host_f64(out)).all()


def test_library_scratch_shared_by_two_streams():
    """Calls on two streams that both use the library-owned scratch (no
    workspace) are ordered on the device: each result equals the same call
    made alone with a workspace of its own. Forward with global rows, and
    backward (row terms in the scratch)."""
    import efficient_exact_attention_amd as ea
    ws_a = W.random_workload("ep-two-a", 2, 4, 3000, 64, causal=0, win_left=30, win_right=30,
                             global_idx=(0, 777, 2999), seed=47)
    ws_b = ws_a.with_(name="ep-two-b", seed=48)
    devs = [tuple(to_device(x, "bf16") for x in W.make_qkv(w)) for w in (ws_a, ws_b)]
    refs = [_masked(w, *t) for w, t in zip((ws_a, ws_b), devs)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [(torch.empty_like(t[0]), torch.empty(w.B, w.H, w.N, dtype=torch.float32, device="cuda"))
            for w, t in zip((ws_a, ws_b), devs)]
    g = list(ws_a.global_idx)
    say("  two streams, forward with global rows, library scratch")
    torch.cuda.synchronize()
    for rep in range(3):
        for w, (q, k, v), (o, l), s in zip((ws_a, ws_b), devs, outs, streams):
            ea.attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr(), w.B, w.H, w.N,
                           w.d, w.causal, w.win_left, w.win_right, g, stream=s.cuda_stream)
    torch.cuda.synchronize()
    for (o, l), (ro, rl) in zip(outs, refs):
        assert torch.equal(o, ro) and torch.equal(l, rl)

    # backward: both calls put their row terms in the library's backward scratch
    say("  two streams, backward, library scratch")
    grads_ref, grads = [], []
    for w, (q, k, v), (ro, rl) in zip((ws_a, ws_b), devs, refs):
        do = to_device(W.make_tensor(w.with_(seed=w.seed + 100), 0), "bf16")
        grads_ref.append((do, ea.bwd(q, k, v, ro, do, rl, global_idx=g, win_left=w.win_left,
                                     win_right=w.win_right)))
    torch.cuda.synchronize()
    for rep in range(3):
        grads = []
        for w, (q, k, v), (ro, rl), (do, _), s in zip((ws_a, ws_b), devs, refs, grads_ref, streams):
            dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
            ea.attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), ro.data_ptr(), do.data_ptr(), rl.data_ptr(),
                        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), w.B, w.H, w.H, w.N, w.d, w.causal,
                        w.win_left, w.win_right, g, stream=s.cuda_stream)
            grads.append((dq, dk, dv))
        torch.cuda.synchronize()
        for got, (_, want) in zip(grads, grads_ref):
            for a, b in zip(got, want):
                assert torch.equal(a, b)
