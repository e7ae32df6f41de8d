"""attn_fwd_noalloc: the allocation-free forward, through the C ABI.

Two calls in a row (the second with a smaller input) must give, bit for bit,
what attn_fwd_ex gives with a caller workspace (the same kernels run), the
smaller one must match the oracle, and the free device memory must not change
across the calls once the library's device code is loaded (the global-row
partials live in its built-in array)."""
import numpy as np
import pytest

from efficient_exact_attention_amd import workloads as W
from gpu_common import all_heads, check, say, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import efficient_exact_attention_amd as ea
    ea.lib()


def _with_workspace(w, q, k, v):
    import efficient_exact_attention_amd as ea
    ws = torch.empty(max(1, ea.attn_workspace_bytes(w.B, w.H, w.N, w.d, len(w.global_idx))), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty(w.B, w.H, w.N, dtype=torch.float32, device="cuda")
    ea.attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), w.B, w.H, w.N, w.d,
                   w.causal, w.win_left, w.win_right, list(w.global_idx) or None,
                   stream=torch.cuda.current_stream().cuda_stream, workspace=ws.data_ptr(),
                   workspace_bytes=ws.numel())
    torch.cuda.synchronize()
    return out, lse


def test_noalloc_matches_workspace_call_twice():
    import efficient_exact_attention_amd as ea
    big = W.random_workload("na-big", 2, 6, 3000, 128, causal=0, win_left=40, win_right=40,
                            global_idx=(0, 1, 777, 2048, 2999), seed=61)
    small = W.random_workload("na-small", 1, 3, 1500, 64, causal=1, win_left=100, global_idx=(3, 700, 1499),
                              seed=62)
    for w in (big, small):
        nbytes = ea.attn_workspace_bytes(w.B, w.H, w.N, w.d, len(w.global_idx))
        assert 0 < nbytes <= ea.ATTN_NOALLOC_SCRATCH_BYTES
    inputs = []
    for w in (big, small):
        qkv = W.make_qkv(w)
        dev = tuple(to_device(x, w.dtype) for x in qkv)
        out = torch.empty_like(dev[0])
        lse = torch.empty(w.B, w.H, w.N, dtype=torch.float32, device="cuda")
        inputs.append((w, qkv, dev, out, lse))
    # one ordinary call first: the runtime loads the library's device code
    # (its built-in array included) at the first launch of any of its kernels
    tiny = W.random_workload("na-warm", 1, 1, 64, 64, causal=1, seed=60)
    _with_workspace(tiny, *(to_device(x, "bf16") for x in W.make_qkv(tiny)))
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for w, qkv, (q, k, v), out, lse in inputs:
        say(f"  attn_fwd_noalloc {w.name}: B={w.B} H={w.H} N={w.N} d={w.d} globals={len(w.global_idx)}")
        ea.attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), w.B, w.H,
                            w.N, w.d, w.causal, w.win_left, w.win_right, list(w.global_idx),
                            stream=torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert abs(free1 - free0) < (1 << 20), (free0, free1)
    for w, qkv, (q, k, v), out, lse in inputs:
        o2, l2 = _with_workspace(w, q, k, v)
        assert torch.equal(out, o2) and torch.equal(lse, l2), w.name
    w, qkv, _, out, lse = inputs[1]
    check(w, out, lse, all_heads(w), np.arange(w.N), qkv)


def test_noalloc_without_globals_is_attn_fwd_ex():
    import efficient_exact_attention_amd as ea
    w = W.random_workload("na-plain", 1, 4, 2000, 128, causal=1, seed=63)
    qkv = W.make_qkv(w)
    q, k, v = (to_device(x, w.dtype) for x in qkv)
    out = torch.empty_like(q)
    lse = torch.empty(w.B, w.H, w.N, dtype=torch.float32, device="cuda")
    say(f"  attn_fwd_noalloc {w.name} (no globals)")
    ea.attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), w.B, w.H, w.N,
                        w.d, w.causal, w.win_left, w.win_right, None)
    torch.cuda.synchronize()
    o2, l2 = _with_workspace(w, q, k, v)
    assert torch.equal(out, o2) and torch.equal(lse, l2)
