"""GPU parity of grouped-query and multi-query attention (K/V heads shared by
groups of consecutive query heads) through attn_fwd_gqa, against the oracle
on the same seeded inputs."""
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
    """q from one seeded workload of H heads, k and v from another of H_kv
    heads (same generator, distinct seed)."""
    wq = W.random_workload("gqa-q", B, H, N, d, dtype=dtype, seed=seed)
    wk = W.random_workload("gqa-kv", B, H_kv, N, d, dtype=dtype, seed=seed + 1)
    q = W.make_tensor(wq, 0)
    k = W.make_tensor(wk, 1)
    v = W.make_tensor(wk, 2)
    return q, k, v


def _run(B, H, H_kv, N, d, mask, dtype="bf16", seed=1, rows=None):
    import efficient_exact_attention_amd as ea
    q, k, v = _inputs(B, H, H_kv, N, d, dtype, seed)
    say(f"  launch gqa: B={B} H={H} H_kv={H_kv} N={N} d={d} {dtype} mask={mask} seed={seed}")
    o, l = ea.fwd(to_device(q, dtype), to_device(k, dtype), to_device(v, dtype),
                  causal=mask["causal"], win_left=mask["win_left"], win_right=mask["win_right"],
                  global_idx=mask["global_idx"] or None)
    torch.cuda.synchronize()
    rows = np.arange(N) if rows is None else rows
    ref_o, ref_l = oracle.attention(W.as_f64(q, dtype), W.as_f64(k, dtype), W.as_f64(v, dtype),
                                    rows=rows, **mask)
    go, gl = host_f64(o[:, :, rows]), host_f64(l[:, :, rows])
    e = errors(go, gl, ref_o, ref_l, bf16_out=dtype == "bf16")
    say(f"    raw max-abs {e[3]:.3e} (beyond bf16 rounding {e[0]:.3e}) rel-L2 {e[1]:.3e} lse {e[2]:.3e}")
    tol = (1e-2, 5e-3, 1e-3) if dtype == "bf16" else (1e-4, 1e-5, 1e-4)
    assert e[0] <= tol[0] and e[1] <= tol[1] and e[2] <= tol[2], e
    return o, l


MASKS = {
    "causal": dict(causal=1, win_left=-1, win_right=-1, global_idx=()),
    "swa": dict(causal=1, win_left=300, win_right=0, global_idx=()),
    "band_g": dict(causal=0, win_left=40, win_right=40, global_idx=(0, 513, 1111)),
}


@pytest.mark.parametrize("mask", list(MASKS))
@pytest.mark.parametrize("H,H_kv", [(8, 2), (8, 1), (6, 3)])
@pytest.mark.parametrize("d", [64, 128])
def test_gqa_bf16(mask, H, H_kv, d):
    _run(2, H, H_kv, 1200, d, MASKS[mask], seed=H * 10 + H_kv + d)


@pytest.mark.parametrize("H,H_kv", [(4, 2), (4, 1)])
def test_gqa_fp32(H, H_kv):
    _run(1, H, H_kv, 333, 64, dict(MASKS["band_g"], global_idx=(0, 100, 300)), dtype="f32", seed=7 + H_kv)


def test_gqa_equals_repeated_heads_bitwise():
    """A grouped call and a multi-head call on K/V repeated over each group
    run the same kernels on the same operands: identical bits."""
    import efficient_exact_attention_amd as ea
    B, H, H_kv, N, d = 1, 8, 2, 2048, 128
    q, k, v = _inputs(B, H, H_kv, N, d, "bf16", 21)
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    o1, l1 = ea.fwd(qd, kd, vd, causal=1)
    kr = kd.repeat_interleave(H // H_kv, dim=1).contiguous()
    vr = vd.repeat_interleave(H // H_kv, dim=1).contiguous()
    o2, l2 = ea.fwd(qd, kr, vr, causal=1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_gqa_long_sampled_rows():
    """Llama-like shape: 32 query heads on 8 K/V heads, N=8192, sampled rows."""
    rows = np.unique(np.concatenate([np.arange(0, 8192, 257), [1, 255, 256, 4095, 8191]]))
    _run(1, 32, 8, 8192, 128, MASKS["causal"], seed=31, rows=rows)
