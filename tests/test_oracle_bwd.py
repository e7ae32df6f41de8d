"""Pins of the fp64 backward oracle (CPU): torch autograd on the same masked
definition, central finite differences, and invariants the gradient of a
softmax attention must satisfy. Planted mistakes in copies of the oracle are
caught by at least one pin."""
import math

import numpy as np
import pytest

import oracle
import oracle.masked_attention_bwd as OB
from oracle_pins import loop_visible

torch = pytest.importorskip("torch")

MASKS = [
    dict(causal=1, win_left=-1, win_right=-1, global_idx=()),
    dict(causal=1, win_left=5, win_right=-1, global_idx=()),
    dict(causal=0, win_left=4, win_right=2, global_idx=()),
    dict(causal=0, win_left=3, win_right=3, global_idx=(0, 17)),
    dict(causal=0, win_left=-1, win_right=-1, global_idx=()),
]


def _qkv(seed, B, H, H_kv, N, d):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, N, d)), rng.standard_normal((B, H_kv, N, d)),
            rng.standard_normal((B, H_kv, N, d)), rng.standard_normal((B, H, N, d)))


def _torch_grads(q, k, v, do, m):
    N = q.shape[2]
    mask = torch.from_numpy(np.array([[loop_visible(i, j, N, m) for j in range(N)] for i in range(N)]))
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask,
                                                           enable_gqa=q.shape[1] != k.shape[1])
    out.backward(torch.from_numpy(do))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def pin_autograd(bwd):
    for t, m in enumerate(MASKS):
        for (H, H_kv) in ((2, 2), (4, 2), (3, 1)):
            q, k, v, do = _qkv(100 + t, 2, H, H_kv, 29 + 3 * t, 8)
            got = bwd(q, k, v, do, **m)
            ref = _torch_grads(q, k, v, do, m)
            for g, r in zip(got, ref):
                assert np.max(np.abs(g - r)) <= 1e-10, (m, H, H_kv)


def pin_finite_differences(bwd):
    m = dict(causal=0, win_left=2, win_right=1, global_idx=(4,))
    q, k, v, do = _qkv(7, 1, 2, 1, 7, 3)
    got = bwd(q, k, v, do, **m)
    eps = 1e-5

    def loss(q_, k_, v_):
        O, _ = oracle.attention(q_, k_, v_, **m)
        return float((O * do).sum())
    for which, x in enumerate((q, k, v)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        assert np.max(np.abs(num - got[which])) <= 1e-7, which


def pin_invariants(bwd):
    """Adding one vector to every key moves each row's scores by a constant:
    no gradient changes. Adding one vector to every value moves each row's dP
    by a constant: no gradient changes either. Every row's dS sums to zero,
    so the key gradients of a head sum to zero over the keys."""
    m = dict(causal=1, win_left=9, win_right=-1, global_idx=())
    q, k, v, do = _qkv(11, 1, 4, 2, 40, 6)
    g0 = bwd(q, k, v, do, **m)
    u = np.random.default_rng(3).standard_normal(6)
    g1 = bwd(q, k + u, v, do, **m)
    g2 = bwd(q, k, v + u, do, **m)
    for a, b in zip(g0, g1):
        assert np.max(np.abs(a - b)) <= 1e-11
    for a, b in zip(g0, g2):
        assert np.max(np.abs(a - b)) <= 1e-11
    assert np.max(np.abs(g0[1].sum(axis=2))) <= 1e-11


def pin_delta(bwd):
    """rowsum(dO * O) equals rowsum(dP * P) (both forms of the Jacobian term)."""
    m = dict(causal=0, win_left=6, win_right=6, global_idx=())
    q, k, v, do = _qkv(13, 1, 2, 2, 30, 5)
    O, _ = oracle.attention(q, k, v, **m)
    P = oracle.probabilities(q, k, **m)
    dP = np.einsum("bhnd,bhmd->bhnm", do, v)
    assert np.max(np.abs(oracle.delta_rows(O, do) - (dP * P).sum(-1))) <= 1e-12


BWD_PINS = [pin_autograd, pin_finite_differences, pin_invariants, pin_delta]


@pytest.mark.parametrize("pin", BWD_PINS, ids=lambda f: f.__name__)
def test_backward_pin(pin):
    pin(oracle.attention_backward)


# ---- planted mistakes ---------------------------------------------------------------

def _mutant(edit):
    """A copy of the oracle's backward with one line of its arithmetic changed."""
    import inspect
    src = inspect.getsource(OB.attention_backward)
    assert edit[0] in src
    ns = dict(OB.__dict__)
    exec(src.replace(edit[0], edit[1]), ns)
    return ns["attention_backward"]


MUTANT_EDITS = [
    ("ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))", "ds = p * (dp + (dp * p).sum(axis=1, keepdims=True))"),
    ("ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))", "ds = p * dp"),
    ("dq[b, h] = scale * (ds @ k[b, kh])", "dq[b, h] = ds @ k[b, kh]"),
    ("dk[b, kh] += scale * (ds.T @ q[b, h])", "dk[b, kh] += scale * (ds @ q[b, h])"),
    ("dv[b, kh] += p.T @ do", "dv[b, kh] += p @ do"),
    ("dv[b, kh] += p.T @ do", "dv[b, kh] = p.T @ do"),
    ("dp = do @ v[b, kh].T", "dp = do @ k[b, kh].T"),
]


@pytest.mark.parametrize("edit", MUTANT_EDITS, ids=lambda e: e[1][:40])
def test_backward_mutant_is_caught(edit):
    bad = _mutant(edit)
    caught = []
    for pin in BWD_PINS:
        try:
            pin(bad)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught: {edit[1]}"
