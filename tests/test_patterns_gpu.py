"""GPU parity of the block-sparse and dilated masks (attn_fwd_masked and
attn_bwd_masked through the C ABI) against the oracle on seeded inputs."""
import numpy as np
import pytest

import oracle
from efficient_exact_attention_amd import workloads as W
from gpu_common import errors, host_f64, say, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import efficient_exact_attention_amd as ea
    ea.lib()


def _inputs(B, H, H_kv, N, d, dtype, seed):
    wq = W.random_workload("pq", B, H, N, d, dtype=dtype, seed=seed)
    wk = W.random_workload("pkv", B, H_kv, N, d, dtype=dtype, seed=seed + 1)
    return W.make_tensor(wq, 0), W.make_tensor(wk, 1), W.make_tensor(wk, 2)


def run_fwd(B, H, H_kv, N, d, m, dtype="bf16", seed=0, rows=None):
    import efficient_exact_attention_amd as ea
    q, k, v = _inputs(B, H, H_kv, N, d, dtype, seed)
    say(f"  launch masked fwd: B={B} H={H} H_kv={H_kv} N={N} d={d} {dtype} mask={m} seed={seed}")
    o, l = ea.fwd(to_device(q, dtype), to_device(k, dtype), to_device(v, dtype), **m)
    torch.cuda.synchronize()
    rows = np.arange(N) if rows is None else rows
    mo = dict(causal=m.get("causal", 0), win_left=m.get("win_left", -1), win_right=m.get("win_right", -1),
              global_idx=tuple(m.get("global_idx", ()) or ()), block=m.get("block", 0),
              dilation=m.get("dilation", 1))
    ref_o, ref_l = oracle.attention(W.as_f64(q, dtype), W.as_f64(k, dtype), W.as_f64(v, dtype), rows=rows, **mo)
    go, gl = host_f64(o[:, :, rows]), host_f64(l[:, :, rows])
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl))
    e = errors(go, gl, ref_o, ref_l, bf16_out=dtype == "bf16")
    say(f"    raw max-abs {e[3]:.3e} (beyond bf16 rounding {e[0]:.3e}) rel-L2 {e[1]:.3e} lse {e[2]:.3e}")
    tol = (1e-2, 5e-3, 1e-3) if dtype == "bf16" else (1e-4, 1e-5, 1e-4)
    assert e[0] <= tol[0] and e[1] <= tol[1] and e[2] <= tol[2], e


BLOCK = [dict(block=64), dict(block=64, causal=1), dict(block=100, causal=1), dict(block=7),
         dict(block=300, causal=1, global_idx=[0, 5, 777]), dict(block=37, global_idx=[1, 500])]
DIL = [dict(dilation=2, causal=1), dict(dilation=3), dict(dilation=5, win_left=7, win_right=2),
       dict(dilation=4, causal=1, win_left=40, win_right=0), dict(dilation=2, win_left=0, win_right=0)]


@pytest.mark.parametrize("m", BLOCK, ids=str)
@pytest.mark.parametrize("d", [64, 128])
def test_block_fwd(m, d):
    run_fwd(2, 3, 3, 1000, d, m, seed=d + m["block"])


@pytest.mark.parametrize("m", DIL, ids=str)
@pytest.mark.parametrize("N,d", [(1000, 128), (777, 64), (3, 64)])
def test_dilated_fwd(m, N, d):
    run_fwd(2, 2, 2, N, d, m, seed=N + m["dilation"])


def test_block_fwd_fp32_gqa():
    run_fwd(1, 4, 2, 500, 64, dict(block=50, causal=1), dtype="f32", seed=3)


def test_dilated_gqa_long():
    rows = np.unique(np.concatenate([np.arange(0, 16384, 97), [1, 2, 3, 16381, 16382, 16383]]))
    run_fwd(1, 8, 2, 16384, 128, dict(dilation=4, causal=1, win_left=1023, win_right=0), seed=4, rows=rows)


def test_dilation_one_is_the_window_bitwise():
    import efficient_exact_attention_amd as ea
    q, k, v = (to_device(x, "bf16") for x in _inputs(1, 4, 4, 1500, 128, "bf16", 9))
    o1, l1 = ea.fwd(q, k, v, causal=1, win_left=200)
    o2, l2 = ea.fwd(q, k, v, causal=1, win_left=200, dilation=1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("m", [dict(block=64), dict(block=64, causal=1), dict(block=90, causal=1),
                               dict(block=13)], ids=str)
def test_block_bwd(m):
    import efficient_exact_attention_amd as ea
    from test_bwd_gpu import check_bwd
    B, H, H_kv, N, d = 1, 4, 2, 700, 128
    q, k, v = _inputs(B, H, H_kv, N, d, "bf16", 11)
    do = W.make_tensor(W.random_workload("pdo", B, H, N, d, seed=12), 0)
    qd, kd, vd, dod = (to_device(x, "bf16") for x in (q, k, v, do))
    say(f"  launch masked bwd: B={B} H={H} H_kv={H_kv} N={N} d={d} mask={m}")
    out, lse = ea.fwd(qd, kd, vd, **m)
    grads = ea.bwd(qd, kd, vd, out, dod, lse, **m)
    torch.cuda.synchronize()
    check_bwd((q, k, v, do), grads, dict(causal=m.get("causal", 0), win_left=-1, win_right=-1, global_idx=(),
                                          block=m["block"]))


@pytest.mark.parametrize("m", DIL, ids=str)
@pytest.mark.parametrize("N,d,H,H_kv", [(700, 128, 4, 2), (333, 64, 2, 2), (3, 64, 2, 1)])
def test_dilated_bwd(m, N, d, H, H_kv):
    """Backward of a dilated mask: every residue class is a band attention
    of its own (strided rows), GQA heads summed."""
    import efficient_exact_attention_amd as ea
    from test_bwd_gpu import check_bwd
    B = 1
    q, k, v = _inputs(B, H, H_kv, N, d, "bf16", 21 + N)
    do = W.make_tensor(W.random_workload("pdo", B, H, N, d, seed=22 + N), 0)
    qd, kd, vd, dod = (to_device(x, "bf16") for x in (q, k, v, do))
    say(f"  launch dilated bwd: B={B} H={H} H_kv={H_kv} N={N} d={d} mask={m}")
    out, lse = ea.fwd(qd, kd, vd, **m)
    grads = ea.bwd(qd, kd, vd, out, dod, lse, **m)
    torch.cuda.synchronize()
    check_bwd((q, k, v, do), grads, dict(causal=m.get("causal", 0), win_left=m.get("win_left", -1),
                                          win_right=m.get("win_right", -1), global_idx=(),
                                          dilation=m["dilation"]))


def test_dilation_one_bwd_is_the_window_bitwise():
    import efficient_exact_attention_amd as ea
    q, k, v, do = (to_device(x, "bf16") for x in (*_inputs(1, 4, 2, 900, 128, "bf16", 31),
                                                   W.make_tensor(W.random_workload("pdo", 1, 4, 900, 128, seed=32), 0)))
    out, lse = ea.fwd(q, k, v, causal=1, win_left=77)
    g1 = ea.bwd(q, k, v, out, do, lse, causal=1, win_left=77)
    g2 = ea.bwd(q, k, v, out, do, lse, causal=1, win_left=77, dilation=1)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
