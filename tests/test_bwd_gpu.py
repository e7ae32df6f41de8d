"""GPU parity of the backward pass (attn_bwd through the C ABI) against the
fp64 backward oracle on the same seeded bf16 inputs. The forward output and
LSE fed to the backward are the HIP forward's own."""
import numpy as np
import pytest

import oracle
from efficient_exact_attention_amd import workloads as W
from gpu_common import host_f64, say, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# Tolerances for bf16 gradients, relative to each tensor's largest exact
# magnitude: the kernels round P and dS to bf16 for the matrix cores (2^-9
# relative), read rowsum(dO * O) from the forward's bf16 output, and round
# the gradients themselves to bf16.
# Where the exact gradient is zero (one visible key: P = 1 and dS = 0), the
# kernels return only the fp32 rounding of dP - rowsum(dO * O): an absolute
# floor of 1e-5 covers it.
TOL_RELL2 = 1e-2
TOL_MAXREL = 3e-2
TOL_ABS = 1e-5


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import efficient_exact_attention_amd as ea
    ea.lib()


def _inputs(B, H, H_kv, N, d, seed):
    wq = W.random_workload("bq", B, H, N, d, seed=seed)
    wk = W.random_workload("bkv", B, H_kv, N, d, seed=seed + 1)
    return W.make_tensor(wq, 0), W.make_tensor(wk, 1), W.make_tensor(wk, 2), W.make_tensor(wq, 2)


def run_bwd(B, H, H_kv, N, d, mask, seed):
    import efficient_exact_attention_amd as ea
    q, k, v, do = _inputs(B, H, H_kv, N, d, seed)
    say(f"  launch bwd: B={B} H={H} H_kv={H_kv} N={N} d={d} mask={mask} seed={seed}")
    qd, kd, vd, dod = (to_device(x, "bf16") for x in (q, k, v, do))
    out, lse = ea.fwd(qd, kd, vd, **mask)
    dq, dk, dv = ea.bwd(qd, kd, vd, out, dod, lse, **mask)
    torch.cuda.synchronize()
    return (q, k, v, do), (dq, dk, dv)


def check_bwd(inputs, grads, mask, tol=(TOL_RELL2, TOL_MAXREL)):
    q, k, v, do = (W.as_f64(x, "bf16") for x in inputs)
    ref = oracle.attention_backward(q, k, v, do, **mask)
    worst = []
    for name, g, r in zip(("dq", "dk", "dv"), grads, ref):
        g = host_f64(g)
        assert np.all(np.isfinite(g)), name
        scale = float(np.max(np.abs(r)))
        err = float(np.max(np.abs(g - r)))
        rel = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300))
        say(f"    {name}: rel-L2 {rel:.3e}  max-abs {err:.3e}  max|ref| {scale:.3e}")
        worst.append((name, rel, err, scale))
    for name, rel, err, scale in worst:
        if scale < TOL_ABS:   # exact gradient (numerically) zero
            assert err <= TOL_ABS, (name, err)
            continue
        assert rel <= tol[0], (name, rel)
        assert err <= tol[1] * scale + TOL_ABS, (name, err, scale)


MASKS = {
    "causal": dict(causal=1, win_left=-1, win_right=-1),
    "full": dict(causal=0, win_left=-1, win_right=-1),
    "swa100": dict(causal=1, win_left=100, win_right=0),
    "band50": dict(causal=0, win_left=50, win_right=50),
    "asym": dict(causal=0, win_left=3, win_right=90),
}


@pytest.mark.parametrize("mask", list(MASKS))
@pytest.mark.parametrize("N", [1, 37, 200, 1000])
@pytest.mark.parametrize("d", [64, 128])
def test_bwd_small(mask, N, d):
    m = MASKS[mask]
    inputs, grads = run_bwd(2, 3, 3, N, d, m, seed=N * 3 + d)
    check_bwd(inputs, grads, dict(m, global_idx=()))


@pytest.mark.parametrize("H,H_kv", [(8, 2), (8, 1), (6, 3)])
@pytest.mark.parametrize("mask", ["causal", "band50"])
@pytest.mark.parametrize("d", [64, 128])
def test_bwd_gqa(H, H_kv, mask, d):
    m = MASKS[mask]
    inputs, grads = run_bwd(1, H, H_kv, 700, d, m, seed=H + H_kv + d)
    check_bwd(inputs, grads, dict(m, global_idx=()))


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_causal_long(d):
    m = MASKS["causal"]
    inputs, grads = run_bwd(1, 2, 2, 4097, d, m, seed=5 + d)
    check_bwd(inputs, grads, dict(m, global_idx=()))


def test_bwd_sliding_window_long():
    m = dict(causal=1, win_left=511, win_right=0)
    inputs, grads = run_bwd(1, 4, 2, 3000, 64, m, seed=6)
    check_bwd(inputs, grads, dict(m, global_idx=()))


def test_bwd_deterministic():
    import efficient_exact_attention_amd as ea
    m = MASKS["band50"]
    (q, k, v, do), (dq, dk, dv) = run_bwd(1, 4, 2, 900, 128, m, seed=8)
    qd, kd, vd, dod = (to_device(x, "bf16") for x in (q, k, v, do))
    out, lse = ea.fwd(qd, kd, vd, **m)
    dq2, dk2, dv2 = ea.bwd(qd, kd, vd, out, dod, lse, **m)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)


def test_bwd_workspace_and_stream():
    import efficient_exact_attention_amd as ea
    m = MASKS["causal"]
    q, k, v, do = _inputs(1, 2, 2, 600, 64, 9)
    qd, kd, vd, dod = (to_device(x, "bf16") for x in (q, k, v, do))
    out, lse = ea.fwd(qd, kd, vd, **m)
    g1 = ea.bwd(qd, kd, vd, out, dod, lse, **m)
    ws = torch.empty(ea.attn_bwd_workspace_bytes(1, 2, 600, 64), dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g2 = ea.bwd(qd, kd, vd, out, dod, lse, workspace=ws, stream=s, **m)
    s.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


# ---- global tokens ------------------------------------------------------------

GMASKS = {
    "band_g": dict(causal=0, win_left=20, win_right=20, global_idx=(0, 1, 100, 511, 700, 999)),
    "swa_g": dict(causal=1, win_left=50, win_right=0, global_idx=(0, 3, 64, 500, 999)),
    "diag_g63": dict(causal=0, win_left=0, win_right=0, global_idx=tuple(range(0, 1000, 16))),
    "block_g": dict(causal=1, block=64, global_idx=(0, 130, 777)),
    "left_only_g": dict(causal=0, win_left=7, win_right=0, global_idx=(5, 998)),
}


@pytest.mark.parametrize("mask", list(GMASKS))
@pytest.mark.parametrize("N,d,H,H_kv", [(1000, 128, 4, 2), (1000, 64, 2, 2), (77, 64, 3, 1)])
def test_bwd_globals(mask, N, d, H, H_kv):
    """Global rows and columns: the band loops plus the gathered tiles and
    the split passes over the global rows and columns."""
    m = dict(GMASKS[mask])
    m["global_idx"] = tuple(g for g in m["global_idx"] if g < N)
    inputs, grads = run_bwd(1, H, H_kv, N, d, m, seed=N + d + H)
    check_bwd(inputs, grads, dict(dict(win_left=-1, win_right=-1), **m))


def test_bwd_globals_max_count():
    m = dict(causal=1, win_left=30, win_right=0, global_idx=tuple(range(3, 3 + 64 * 37, 37)))
    inputs, grads = run_bwd(1, 2, 1, 2500, 128, m, seed=41)
    check_bwd(inputs, grads, m)


def test_bwd_globals_band256_every_2048th():
    """The non-causal band +-256 with global tokens {0, 1} and every 2048th
    position, at N = 4096 (the oracle's fp64 backward is O(N^2) per head)."""
    N = 4096
    m = dict(causal=0, win_left=256, win_right=256, global_idx=W.every_2048th(N))
    inputs, grads = run_bwd(2, 2, 2, N, 64, m, seed=42)
    check_bwd(inputs, grads, m)


def test_bwd_globals_deterministic_and_workspace():
    import efficient_exact_attention_amd as ea
    m = GMASKS["band_g"]
    (q, k, v, do), g1 = run_bwd(1, 4, 2, 1000, 128, m, seed=43)
    qd, kd, vd, dod = (to_device(x, "bf16") for x in (q, k, v, do))
    out, lse = ea.fwd(qd, kd, vd, **m)
    nbytes = ea.attn_bwd_workspace_bytes(1, 4, 1000, 128, H_kv=2, n_global=len(m["global_idx"]))
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    g2 = ea.bwd(qd, kd, vd, out, dod, lse, workspace=ws, **m)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
