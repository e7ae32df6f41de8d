"""Helpers for the GPU parity tests: upload seeded inputs, run the HIP path
through the C ABI, and compare with the CPU oracle."""
from __future__ import annotations

import math
import sys

import numpy as np

import oracle
from efficient_exact_attention_amd import workloads as W

# Pass criteria (all configurations): max-abs and relative L2 over every checked
# output element, max-abs over checked LSE values; compared in fp64.
# A bf16 output cannot hold a value of magnitude >= 2.56 to within 1e-2 (half
# an ulp there exceeds 1e-2: 1.56e-2 in [4, 8)), so for bf16 outputs each
# element's max-abs bound is 1e-2 plus half a bf16 ulp of the exact value
# (at most |O| * 2^-8). Only peaked rows with large outputs ever use it.
TOL_MAXABS = 1e-2
TOL_RELL2 = 5e-3
TOL_LSE = 1e-3


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(arr: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.cuda()


def run_gpu(w: W.Workload, qkv=None, *, out=None, lse=None, stream=None, workspace=None,
            same_tensor=False):
    """Run the HIP path on workload w; returns (out, lse) as torch tensors."""
    import torch
    import efficient_exact_attention_amd as ea
    if qkv is None:
        qkv = W.make_qkv(w)
    if same_tensor:
        q = k = v = to_device(qkv[0], w.dtype)
    else:
        q, k, v = (to_device(x, w.dtype) for x in qkv)
    say(f"  launch {w.name}: B={w.B} H={w.H} N={w.N} d={w.d} {w.dtype} causal={w.causal} "
        f"wl={w.win_left} wr={w.win_right} globals={len(w.global_idx)} seed={w.seed}")
    o, l = ea.fwd(q, k, v, causal=w.causal, win_left=w.win_left, win_right=w.win_right,
                  global_idx=w.global_idx or None, out=out, lse=lse, stream=stream,
                  workspace=workspace)
    torch.cuda.synchronize()
    return o, l


def host_f64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def oracle_heads(w: W.Workload, heads, rows, qkv=None):
    """Oracle output for the listed (b, h) heads and query rows."""
    outs, lses = [], []
    for (b, h) in heads:
        if qkv is not None:
            q, k, v = (W.as_f64(x[b, h], w.dtype) for x in qkv)
        else:
            q, k, v = (W.head_values(w, t, b, h).astype(np.float64) for t in range(3))
        O, L = oracle.attention(q[None, None], k[None, None], v[None, None], causal=w.causal,
                                win_left=w.win_left, win_right=w.win_right,
                                global_idx=w.global_idx, rows=rows)
        outs.append(O[0, 0])
        lses.append(L[0, 0])
    return np.stack(outs), np.stack(lses)


def errors(got_o, got_l, ref_o, ref_l, bf16_out=False):
    """(max-abs excess over the bf16 output's own rounding, rel-L2, LSE max-abs).
    For fp32 outputs the first value is the plain max-abs error."""
    diff = got_o - ref_o
    widen = np.abs(ref_o) * 2.0 ** -8 if bf16_out else 0.0
    maxabs = float(np.max(np.abs(diff) - widen))
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref_o), 1e-300))
    lse = float(np.max(np.abs(got_l - ref_l)))
    return maxabs, rel, lse


def check(w: W.Workload, o, l, heads, rows, qkv=None, tol=(TOL_MAXABS, TOL_RELL2, TOL_LSE)):
    ref_o, ref_l = oracle_heads(w, heads, rows, qkv)
    go = np.stack([host_f64(o[b, h, rows]) for (b, h) in heads])
    gl = np.stack([host_f64(l[b, h, rows]) for (b, h) in heads])
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl)), "non-finite output"
    e = errors(go, gl, ref_o, ref_l, bf16_out=w.dtype == "bf16")
    raw = float(np.max(np.abs(go - ref_o)))
    say(f"    {w.name}: max-abs {raw:.3e} (beyond bf16 output rounding {e[0]:.3e})  "
        f"rel-L2 {e[1]:.3e}  lse {e[2]:.3e}  ({len(heads)} heads x {len(rows)} rows)")
    assert e[0] <= tol[0], e
    assert e[1] <= tol[1], e
    assert e[2] <= tol[2], e
    return e


def all_heads(w):
    return [(b, h) for b in range(w.B) for h in range(w.H)]


def some_heads(w, n, seed=0):
    hs = all_heads(w)
    if len(hs) <= n:
        return hs
    rng = np.random.default_rng(w.seed + seed)
    idx = sorted(rng.choice(len(hs), size=n, replace=False))
    return [hs[i] for i in idx]
