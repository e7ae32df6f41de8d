"""GPU parity of the log-spaced strided and random-block (BigBird) rules
(attn_fwd_masked through the C ABI) against the oracle on seeded inputs;
the random key-block lists are seeded inputs too, read by the kernel from
device memory."""
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


def _inputs(B, H, H_kv, N, d, seed):
    wq = W.random_workload("xq", B, H, N, d, seed=seed)
    wk = W.random_workload("xkv", B, H_kv, N, d, seed=seed + 1)
    return W.make_tensor(wq, 0), W.make_tensor(wk, 1), W.make_tensor(wk, 2)


def rand_lists(N, b, r, seed, extra=()):
    """Seeded key-block lists [ceil(N / b), r] (values may repeat), with
    (query block, entry, value) overrides for repeats and out-of-range
    entries."""
    nb = (N + b - 1) // b
    lists = np.random.default_rng(seed).integers(0, nb, size=(nb, r)).astype(np.int32)
    for qb, e, val in extra:
        if qb < nb:
            lists[qb, e] = val
    return lists


def run(B, H, H_kv, N, d, m, seed, rows=None, lists=None):
    import efficient_exact_attention_amd as ea
    q, k, v = _inputs(B, H, H_kv, N, d, seed)
    say(f"  launch extra-rule fwd: B={B} H={H} H_kv={H_kv} N={N} d={d} mask={m} seed={seed}")
    kw = dict(m)
    if lists is not None:
        kw["rand_idx"] = torch.from_numpy(lists).cuda()
    o, l = ea.fwd(to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16"), **kw)
    torch.cuda.synchronize()
    rows = np.arange(N) if rows is None else rows
    mo = dict(causal=m.get("causal", 0), win_left=m.get("win_left", -1), win_right=m.get("win_right", -1),
              global_idx=tuple(m.get("global_idx", ()) or ()), stride=m.get("stride", 0),
              rand_block=m.get("rand_block", 0), rand_idx=lists)
    ref_o, ref_l = oracle.attention(W.as_f64(q, "bf16"), W.as_f64(k, "bf16"), W.as_f64(v, "bf16"), rows=rows, **mo)
    go, gl = host_f64(o[:, :, rows]), host_f64(l[:, :, rows])
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl))
    e = errors(go, gl, ref_o, ref_l, bf16_out=True)
    say(f"    raw max-abs {e[3]:.3e} (beyond bf16 rounding {e[0]:.3e}) rel-L2 {e[1]:.3e} lse {e[2]:.3e}")
    assert e[0] <= 1e-2 and e[1] <= 5e-3 and e[2] <= 1e-3, e


STRIDED = [dict(stride=1, causal=1, win_left=0, win_right=0),
           dict(stride=3, causal=0, win_left=5, win_right=5),
           dict(stride=16, causal=1, win_left=40, win_right=0, global_idx=(0, 7, 999)),
           dict(stride=2, causal=0, win_left=0, win_right=0, global_idx=(10,)),
           dict(stride=64, causal=1, win_left=63, win_right=0)]


@pytest.mark.parametrize("m", STRIDED, ids=str)
@pytest.mark.parametrize("N,d,H,H_kv", [(1000, 128, 4, 2), (777, 64, 2, 2), (5, 64, 1, 1)])
def test_strided(m, N, d, H, H_kv):
    mm = dict(m, global_idx=tuple(g for g in m.get("global_idx", ()) if g < N))
    run(1, H, H_kv, N, d, mm, seed=N + d + m["stride"])


def test_strided_long_sampled():
    N = 16384
    rows = np.unique(np.concatenate([np.arange(0, N, 61), [1, 2, 255, 256, N - 2, N - 1]]))
    run(1, 4, 2, N, 128, dict(stride=8, causal=1, win_left=255, win_right=0, global_idx=(0, 4096)), seed=5,
        rows=rows)


RANDOM = [(dict(rand_block=64, causal=0, win_left=64, win_right=64), 3, ()),
          (dict(rand_block=64, causal=1, win_left=127, win_right=0), 2, ((1, 0, 0), (1, 1, 0), (3, 0, 999))),
          (dict(rand_block=32, causal=0, win_left=0, win_right=0, global_idx=(0, 1, 500)), 4, ((2, 3, -5),)),
          (dict(rand_block=96, causal=1, win_left=10, win_right=0), 1, ()),
          (dict(rand_block=128, causal=0, win_left=31, win_right=31, global_idx=(900,)), 2, ())]


@pytest.mark.parametrize("ci", range(len(RANDOM)))
@pytest.mark.parametrize("N,d,H,H_kv", [(1000, 128, 4, 2), (700, 64, 2, 1), (40, 64, 2, 2)])
def test_random_blocks(ci, N, d, H, H_kv):
    m, r, extra = RANDOM[ci]
    mm = dict(m, global_idx=tuple(g for g in m.get("global_idx", ()) if g < N))
    lists = rand_lists(N, m["rand_block"], r, seed=ci + N, extra=extra)
    run(1, H, H_kv, N, d, mm, seed=N + ci, lists=lists)


def test_random_blocks_bigbird_long_sampled():
    """BigBird-style: window of one block each side, 2 global tokens, 3
    random blocks of 64 per query block, N = 16384."""
    N, b = 16384, 64
    rows = np.unique(np.concatenate([np.arange(0, N, 53), [1, 63, 64, N - 1]]))
    lists = rand_lists(N, b, 3, seed=77)
    run(1, 4, 4, N, 128, dict(rand_block=b, causal=0, win_left=b, win_right=b, global_idx=(0, 1)), seed=6,
        rows=rows, lists=lists)


def test_every_block_listed_is_full_attention():
    """Listing every key block for every query block gives plain (dense)
    attention; compared with the HIP forward's own dense result."""
    import efficient_exact_attention_amd as ea
    N, b = 512, 64
    nb = N // b
    q, k, v = (to_device(x, "bf16") for x in _inputs(1, 2, 2, N, 128, 8))
    lists = torch.from_numpy(np.tile(np.arange(nb, dtype=np.int32), (nb, 1))).cuda()
    o1, l1 = ea.fwd(q, k, v, win_left=0, win_right=0, rand_block=b, rand_idx=lists)
    o2, l2 = ea.fwd(q, k, v)
    torch.cuda.synchronize()
    assert (o1.float() - o2.float()).abs().max().item() <= 1e-2
    assert (l1 - l2).abs().max().item() <= 1e-3


@pytest.mark.parametrize("ci", range(len(RANDOM)))
@pytest.mark.parametrize("N", [40, 700, 1000])
def test_random_plan_pairs_match_oracle(ci, N):
    """The planner's visible-pair count for random blocks (lists read from
    the device) against the oracle's mask."""
    import efficient_exact_attention_amd as ea
    m, r, extra = RANDOM[ci]
    G = tuple(g for g in m.get("global_idx", ()) if g < N)
    lists = rand_lists(N, m["rand_block"], r, seed=ci + N, extra=extra)
    dl = torch.from_numpy(lists).cuda()
    pairs = ea.attn_plan_stats_masked(N, 128, 64, causal=m["causal"], win_left=m["win_left"],
                                      win_right=m["win_right"], global_idx=list(G), rand_block=m["rand_block"],
                                      n_rand=r, rand_idx=dl.data_ptr())[0]
    ref = oracle.visible_pairs_bruteforce(N, m["causal"], m["win_left"], m["win_right"], G,
                                          rand_block=m["rand_block"], rand_idx=lists)
    assert pairs == ref


# ---- backward of the strided and random-block rules ----------------------------

def run_bwd_extra(B, H, H_kv, N, d, m, seed, lists=None):
    import efficient_exact_attention_amd as ea
    from test_bwd_gpu import check_bwd
    q, k, v = _inputs(B, H, H_kv, N, d, seed)
    do = W.make_tensor(W.random_workload("xdo", B, H, N, d, seed=seed + 5), 0)
    qd, kd, vd, dod = (to_device(x, "bf16") for x in (q, k, v, do))
    kw = dict(m)
    if lists is not None:
        kw["rand_idx"] = torch.from_numpy(lists).cuda()
    say(f"  launch extra-rule bwd: B={B} H={H} H_kv={H_kv} N={N} d={d} mask={m} seed={seed}")
    out, lse = ea.fwd(qd, kd, vd, **kw)
    grads = ea.bwd(qd, kd, vd, out, dod, lse, **kw)
    torch.cuda.synchronize()
    mo = dict(causal=m.get("causal", 0), win_left=m.get("win_left", -1), win_right=m.get("win_right", -1),
              global_idx=tuple(m.get("global_idx", ()) or ()), stride=m.get("stride", 0),
              rand_block=m.get("rand_block", 0), rand_idx=lists)
    check_bwd((q, k, v, do), grads, mo)


@pytest.mark.parametrize("m", STRIDED, ids=str)
@pytest.mark.parametrize("N,d,H,H_kv", [(700, 128, 4, 2), (333, 64, 2, 2), (5, 64, 1, 1)])
def test_strided_bwd(m, N, d, H, H_kv):
    mm = dict(m, global_idx=tuple(g for g in m.get("global_idx", ()) if g < N))
    run_bwd_extra(1, H, H_kv, N, d, mm, seed=N + d + m["stride"] + 1)


@pytest.mark.parametrize("ci", range(len(RANDOM)))
@pytest.mark.parametrize("N,d,H,H_kv", [(700, 128, 4, 2), (333, 64, 2, 1), (40, 64, 2, 2)])
def test_random_blocks_bwd(ci, N, d, H, H_kv):
    m, r, extra = RANDOM[ci]
    mm = dict(m, global_idx=tuple(g for g in m.get("global_idx", ()) if g < N))
    lists = rand_lists(N, m["rand_block"], r, seed=ci + N + 3, extra=extra)
    run_bwd_extra(1, H, H_kv, N, d, mm, seed=N + ci + 2, lists=lists)


def test_random_blocks_bwd_many_list_entries_deterministic():
    """More list entries than one scan chunk of the dK/dV kernel (128 query
    blocks x 4 entries = 512 > 256 threads): the hits of every chunk are
    taken, against the oracle, and two calls give identical bits."""
    import efficient_exact_attention_amd as ea
    N, d, b, r = 4096, 64, 32, 4
    m = dict(rand_block=b, causal=0, win_left=16, win_right=16, global_idx=(0, 2047))
    lists = rand_lists(N, b, r, seed=77, extra=((5, 1, -1), (9, 3, 4096)))
    run_bwd_extra(1, 2, 2, N, d, m, seed=78, lists=lists)
    q, k, v = _inputs(1, 2, 2, N, d, 79)
    do = W.make_tensor(W.random_workload("xdo", 1, 2, N, d, seed=84), 0)
    qd, kd, vd, dod = (to_device(x, "bf16") for x in (q, k, v, do))
    kw = dict(m, rand_idx=torch.from_numpy(lists).cuda())
    say(f"  launch random-block bwd twice: N={N} d={d} b={b} r={r}")
    out, lse = ea.fwd(qd, kd, vd, **kw)
    g1 = [x.clone() for x in ea.bwd(qd, kd, vd, out, dod, lse, **kw)]
    g2 = ea.bwd(qd, kd, vd, out, dod, lse, **kw)
    torch.cuda.synchronize()
    for a, c in zip(g1, g2):
        assert torch.equal(a.view(torch.int16), c.view(torch.int16))
