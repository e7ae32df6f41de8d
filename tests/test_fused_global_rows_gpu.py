"""The global rows computed inside the band pass of 128-row workgroups: each
workgroup takes its own key tiles (the keys under its query rows) for every
global row, one partial per workgroup, merged afterwards. Every row of every
head against the oracle, on the shapes that exercise that path's edges:

* a ragged last query tile that owns one key tile only (N = 7*128 + 50);
* N = 64 and N = 1 (a single query tile, a single partial);
* d = 64 and d = 128 (the four-wave band instances of both head sizes);
* a causal sliding window (global rows then see keys up to themselves);
* the block rule with globals (the block-rule instance);
* 64 global tokens (two row blocks of global rows, two waves);
* grouped-query heads (K/V head of each query head);
* global tokens at the first and last positions and next to each other.
"""
import numpy as np
import pytest

import oracle
from efficient_exact_attention_amd import workloads as W
from gpu_common import errors, host_f64, say, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TOL = (1e-2, 5e-3, 1e-3)   # max-abs beyond the bf16 output rounding, rel-L2, LSE


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import efficient_exact_attention_amd as ea
    ea.lib()


CASES = {
    "d64-ragged-one-own-tile": dict(B=1, H=3, H_kv=3, N=946, d=64, causal=0, wl=100, wr=100, g=(0, 5, 945)),
    "d128-ragged-one-own-tile": dict(B=1, H=2, H_kv=2, N=946, d=128, causal=0, wl=100, wr=100, g=(0, 400, 945)),
    "d64-n64": dict(B=1, H=2, H_kv=2, N=64, d=64, causal=0, wl=8, wr=8, g=(0, 63)),
    "d128-n1": dict(B=2, H=2, H_kv=2, N=1, d=128, causal=0, wl=0, wr=0, g=(0,)),
    "d64-causal-window": dict(B=2, H=2, H_kv=2, N=2000, d=64, causal=1, wl=200, wr=0, g=(3, 500, 1999)),
    "d128-causal-window": dict(B=1, H=2, H_kv=2, N=1500, d=128, causal=1, wl=300, wr=0, g=(0, 1, 2, 777)),
    "d64-64-globals": dict(B=1, H=2, H_kv=2, N=3000, d=64, causal=0, wl=64, wr=64, g=tuple(range(0, 3000, 47))[:64]),
    "d128-block-rule": dict(B=1, H=2, H_kv=2, N=2000, d=128, causal=1, block=100, g=(5, 1999)),
    "d64-block-rule": dict(B=1, H=2, H_kv=2, N=1300, d=64, causal=0, block=64, g=(0, 640, 641)),
    "d64-gqa": dict(B=2, H=8, H_kv=2, N=1200, d=64, causal=0, wl=128, wr=128, g=(10, 1100)),
    "d128-gqa-causal": dict(B=1, H=4, H_kv=1, N=1100, d=128, causal=1, wl=511, wr=0, g=(0, 1099)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_fused_global_rows_every_row(name):
    import efficient_exact_attention_amd as ea
    c = CASES[name]
    B, H, H_kv, N, d = c["B"], c["H"], c["H_kv"], c["N"], c["d"]
    block = c.get("block", 0)
    wl, wr = (c["wl"], c["wr"]) if not block else (-1, -1)
    w = W.random_workload(name, B, H, N, d, causal=c["causal"], win_left=wl, win_right=wr,
                          global_idx=c["g"], seed=71)
    qkv = W.make_qkv(w)
    q, k, v = (to_device(x, "bf16") for x in qkv)
    k, v = k[:, :H_kv].contiguous(), v[:, :H_kv].contiguous()
    say(f"  fused global rows {name}: B={B} H={H} H_kv={H_kv} N={N} d={d} causal={c['causal']} "
        f"wl={wl} wr={wr} block={block} globals={len(c['g'])}")
    o, l = ea.fwd(q, k, v, causal=c["causal"], win_left=wl, win_right=wr, global_idx=c["g"], block=block)
    torch.cuda.synchronize()
    q64, k64, v64 = (W.as_f64(x, "bf16") for x in qkv)
    ref_o, ref_l = oracle.attention(q64, k64[:, :H_kv], v64[:, :H_kv], causal=c["causal"], win_left=wl,
                                    win_right=wr, global_idx=c["g"], block=block)
    got_o, got_l = host_f64(o), host_f64(l)
    assert np.all(np.isfinite(got_o)) and np.all(np.isfinite(got_l))
    e = errors(got_o, got_l, ref_o, ref_l, bf16_out=True)
    say(f"    raw max-abs {e[3]:.3e} (beyond bf16 rounding {e[0]:.3e})  rel-L2 {e[1]:.3e}  lse {e[2]:.3e}")
    assert e[0] <= TOL[0] and e[1] <= TOL[1] and e[2] <= TOL[2], e
    # the global rows alone: these come from the merged partials
    gi = list(c["g"])
    eg = errors(got_o[:, :, gi], got_l[:, :, gi], ref_o[:, :, gi], ref_l[:, :, gi], bf16_out=True)
    assert eg[0] <= TOL[0] and eg[2] <= TOL[2], eg


def test_fused_global_rows_repeat_bitwise():
    """Repeated calls give the same bits (the merge order is fixed)."""
    import efficient_exact_attention_amd as ea
    c = CASES["d64-causal-window"]
    w = W.random_workload("rep", c["B"], c["H"], c["N"], c["d"], causal=1, win_left=c["wl"], win_right=0,
                          global_idx=c["g"], seed=72)
    q, k, v = (to_device(x, "bf16") for x in W.make_qkv(w))
    o1, l1 = ea.fwd(q, k, v, causal=1, win_left=c["wl"], win_right=0, global_idx=c["g"])
    o2, l2 = ea.fwd(q, k, v, causal=1, win_left=c["wl"], win_right=0, global_idx=c["g"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
