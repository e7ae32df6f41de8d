"""Checks that pin the oracle to facts other than itself.

Each ``pin_*`` function takes an attention callable with the oracle's
signature (``attn(q, k, v, causal=, win_left=, win_right=, global_idx=,
rows=, scale=) -> (O, LSE)``) and raises AssertionError when it disagrees
with what the mathematics or the pages fix. ``tests/test_oracle_pins.py`` runs
them on the oracle; ``tests/test_oracle_mutants.py`` runs them on copies of the
oracle with planted mistakes to show each mistake is caught.

The pins (brute force, closed forms, invariants, library special cases) are
chosen so that a dropped term, a wrong sign or index, or a transposed operand
anywhere in the oracle breaks at least one of them.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

MASKS = [
    dict(causal=0, win_left=-1, win_right=-1, global_idx=()),
    dict(causal=1, win_left=-1, win_right=-1, global_idx=()),
    dict(causal=1, win_left=3, win_right=-1, global_idx=()),
    dict(causal=1, win_left=0, win_right=-1, global_idx=()),
    dict(causal=0, win_left=2, win_right=2, global_idx=()),
    dict(causal=0, win_left=2, win_right=1, global_idx=(0, 5)),
    dict(causal=1, win_left=2, win_right=-1, global_idx=(1, 7)),
    dict(causal=0, win_left=0, win_right=0, global_idx=(3,)),
]


def _rng_qkv(seed, B, H, N, d, scale=1.0):
    rng = np.random.default_rng(seed)
    return tuple(rng.standard_normal((B, H, N, d)) * scale for _ in range(3))


# ---- P1: brute force, pure Python loops ------------------------------------

def brute_attention(q, k, v, causal, win_left, win_right, global_idx):
    """Straight loops with math.exp over one head: q, k, v nested lists."""
    N, d = len(q), len(q[0])
    G = set(global_idx)
    out, lse = [], []
    for i in range(N):
        scores = []
        for j in range(N):
            ok = True
            if causal and j > i:
                ok = False
            elif not (i in G or j in G):
                if win_left >= 0 and j < i - win_left:
                    ok = False
                if win_right >= 0 and j > i + win_right:
                    ok = False
            if ok:
                scores.append((j, sum(q[i][c] * k[j][c] for c in range(d)) / math.sqrt(d)))
        mx = max(s for _, s in scores)
        w = [(j, math.exp(s - mx)) for j, s in scores]
        tot = sum(x for _, x in w)
        out.append([sum(x * v[j][c] for j, x in w) / tot for c in range(len(v[0]))])
        lse.append(mx + math.log(tot))
    return out, lse


def pin_bruteforce(attn):
    for t, m in enumerate(MASKS):
        for N, d in ((1, 3), (9, 4), (17, 8)):
            q, k, v = _rng_qkv(1000 + 17 * t + N, 1, 1, N, d)
            mm = dict(m, global_idx=tuple(g for g in m["global_idx"] if g < N))
            O, L = attn(q, k, v, **mm)
            bo, bl = brute_attention(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(),
                                     mm["causal"], mm["win_left"], mm["win_right"],
                                     mm["global_idx"])
            assert np.max(np.abs(O[0, 0] - np.array(bo))) <= 1e-12, (m, N)
            assert np.max(np.abs(L[0, 0] - np.array(bl))) <= 1e-12, (m, N)


# ---- golden closed forms ----------------------------------------------------

def load_closed_forms():
    with open(os.path.join(GOLDEN, "closed_forms.json")) as f:
        return json.load(f)["cases"]


def closed_form_inputs(case):
    N, d = case["N"], case["d"]
    q = np.zeros((1, 1, N, d))
    q[..., 0] = 1.0
    k = np.zeros((1, 1, N, d))
    k[0, 0, :, 0] = [math.sqrt(d) * math.log(a) for a in case["a"]]
    if case["v"] == "one-hot":
        v = np.eye(N, d)[None, None]
    else:
        v = np.array(case["v"], dtype=np.float64)[None, None]
    return q, k, v


def pin_closed_forms(attn):
    for case in load_closed_forms():
        q, k, v = closed_form_inputs(case)
        O, L = attn(q, k, v, causal=case["causal"], win_left=case["win_left"],
                    win_right=case["win_right"], global_idx=tuple(case["global_idx"]))
        want = np.array([[float(Fraction(x)) for x in row] for row in case["out"]])
        want_lse = np.array([math.log(float(Fraction(x))) for x in case["lse_of"]])
        assert np.max(np.abs(O[0, 0] - want)) <= 1e-13, case["name"]
        assert np.max(np.abs(L[0, 0] - want_lse)) <= 1e-13, case["name"]


# ---- P4 constant V, P5 identical keys ---------------------------------------

def pin_constant_v(attn):
    for m in MASKS:
        q, k, _ = _rng_qkv(7, 2, 2, 13, 5)
        c = np.array([0.5, -1.25, 3.0, 0.0, 7.5])
        v = np.broadcast_to(c, (2, 2, 13, 5)).copy()
        O, _ = attn(q, k, v, **m)
        assert np.max(np.abs(O - c)) <= 1e-12, m


def pin_identical_keys(attn, mask_fn):
    """All keys equal: output = mean of visible value rows, LSE = q.k/sqrt(d) +
    ln(count). ``mask_fn(rows, N, **mask)`` is an independent visibility
    evaluation (the brute-force loop predicate)."""
    for m in MASKS:
        q, _, v = _rng_qkv(11, 1, 2, 15, 6)
        kk = np.random.default_rng(3).standard_normal(6)
        k = np.broadcast_to(kk, q.shape).copy()
        O, L = attn(q, k, v, **m)
        for h in range(2):
            for i in range(15):
                vis = [j for j in range(15) if mask_fn(i, j, 15, m)]
                want = v[0, h, vis].mean(axis=0)
                assert np.max(np.abs(O[0, h, i] - want)) <= 1e-12, (m, i)
                wl = q[0, h, i] @ kk / math.sqrt(6) + math.log(len(vis))
                assert abs(L[0, h, i] - wl) <= 1e-12, (m, i)


def loop_visible(i, j, N, m):
    """Visibility written out as in the brute-force loop above."""
    if m["causal"] and j > i:
        return False
    if i in m["global_idx"] or j in m["global_idx"]:
        return True
    if m["win_left"] >= 0 and j < i - m["win_left"]:
        return False
    if m["win_right"] >= 0 and j > i + m["win_right"]:
        return False
    return True


# ---- P6 window >= N-1 is plain causal ---------------------------------------

def pin_window_covers_causal(attn):
    q, k, v = _rng_qkv(21, 1, 3, 40, 8)
    Oc, Lc = attn(q, k, v, causal=1, win_left=-1, win_right=-1, global_idx=())
    for wl in (39, 40, 1000):
        Ow, Lw = attn(q, k, v, causal=1, win_left=wl, win_right=0, global_idx=())
        assert np.array_equal(Oc, Ow) and np.array_equal(Lc, Lw)
    Ow, Lw = attn(q, k, v, causal=1, win_left=38, win_right=0, global_idx=())
    assert not np.allclose(Lc, Lw)   # one key fewer for the last row


# ---- P7 key shift ------------------------------------------------------------

def pin_key_shift(attn):
    for m in MASKS:
        q, k, v = _rng_qkv(31, 1, 2, 12, 4)
        for mag in (1.0, 1e3):
            u = np.array([1.0, -2.0, 0.5, 3.0]) * mag
            O0, L0 = attn(q, k, v, **m)
            O1, L1 = attn(q, k + u, v, **m)
            shift = (q @ u) / 2.0          # sqrt(d) = 2
            assert np.all(np.isfinite(O1)), m
            assert np.max(np.abs(O1 - O0)) <= 1e-9 * max(1.0, mag / 100), (m, mag)
            assert np.max(np.abs(L1 - (L0 + shift))) <= 1e-9 * mag, (m, mag)


# ---- P10 permutations ----------------------------------------------------------

def pin_permutation(attn):
    q, k, v = _rng_qkv(41, 1, 2, 23, 6)
    perm = np.random.default_rng(5).permutation(23)
    m = dict(causal=0, win_left=-1, win_right=-1, global_idx=())
    O0, L0 = attn(q, k, v, **m)
    O1, L1 = attn(q, k[:, :, perm], v[:, :, perm], **m)
    assert np.max(np.abs(O0 - O1)) <= 1e-12 and np.max(np.abs(L0 - L1)) <= 1e-12
    O2, L2 = attn(q[:, :, perm], k, v, **m)
    assert np.max(np.abs(O0[:, :, perm] - O2)) <= 1e-12
    assert np.max(np.abs(L0[:, :, perm] - L2)) <= 1e-12


# ---- P11 special cases ---------------------------------------------------------

def pin_special_cases(attn):
    q, k, v = _rng_qkv(51, 1, 1, 1, 7)
    for m in MASKS:
        O, L = attn(q, k, v, **dict(m, global_idx=tuple(g for g in m["global_idx"] if g < 1)))
        assert np.max(np.abs(O[0, 0, 0] - v[0, 0, 0])) <= 1e-15
        assert abs(L[0, 0, 0] - q[0, 0, 0] @ k[0, 0, 0] / math.sqrt(7)) <= 1e-14
    # a row whose only visible key is the diagonal: output is exactly that value row
    q, k, v = _rng_qkv(52, 1, 1, 10, 4)
    O, L = attn(q, k, v, causal=1, win_left=0, win_right=0, global_idx=())
    assert np.max(np.abs(O[0, 0] - v[0, 0])) <= 1e-15
    assert np.max(np.abs(L[0, 0] - np.einsum("nd,nd->n", q[0, 0], k[0, 0]) / 2.0)) <= 1e-14


# ---- P9 library special case: torch SDPA on CPU fp64 with an explicit mask -----

def pin_torch_sdpa(attn):
    import torch
    import torch.nn.functional as F
    for t, m in enumerate(MASKS):
        N = 200 + 37 * t
        q, k, v = _rng_qkv(61 + t, 1, 2, N, 16)
        O, _ = attn(q, k, v, **m)
        mask = np.array([[loop_visible(i, j, N, m) for j in range(N)] for i in range(N)])
        ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k),
                                             torch.from_numpy(v),
                                             attn_mask=torch.from_numpy(mask))
        assert np.max(np.abs(O - ref.numpy())) <= 1e-12, m
    # the library's own causal flag, no explicit mask
    q, k, v = _rng_qkv(71, 2, 2, 300, 32)
    O, _ = attn(q, k, v, causal=1, win_left=-1, win_right=-1, global_idx=())
    ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k),
                                         torch.from_numpy(v), is_causal=True)
    assert np.max(np.abs(O - ref.numpy())) <= 1e-12


def pin_grouped_heads(attn):
    """Grouped-query and multi-query attention (week-17 notes, the MQA / GQA
    passage: groups of query heads share one K and one V head) against
    torch's SDPA with enable_gqa, which repeats each K/V head over a run of
    consecutive query heads: H = 6 query heads with H_kv = 6, 3, 2 and 1, under
    a causal and a windowed mask."""
    import torch
    import torch.nn.functional as F
    masks = [dict(causal=1, win_left=-1, win_right=-1, global_idx=()),
             dict(causal=0, win_left=9, win_right=4, global_idx=(0, 77))]
    for t, H_kv in enumerate((6, 3, 2, 1)):
        rng = np.random.default_rng(81 + t)
        N, d = 150 + 11 * t, 16
        q = rng.standard_normal((2, 6, N, d))
        k = rng.standard_normal((2, H_kv, N, d))
        v = rng.standard_normal((2, H_kv, N, d))
        for m in masks:
            O, _ = attn(q, k, v, **m)
            mask = np.array([[loop_visible(i, j, N, m) for j in range(N)] for i in range(N)])
            ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                                 attn_mask=torch.from_numpy(mask), enable_gqa=True)
            assert O.shape == (2, 6, N, d)
            assert np.max(np.abs(O - ref.numpy())) <= 1e-12, (H_kv, m)


ALL_PINS = ["pin_bruteforce", "pin_closed_forms", "pin_constant_v", "pin_identical_keys",
            "pin_window_covers_causal", "pin_key_shift", "pin_permutation",
            "pin_special_cases", "pin_torch_sdpa", "pin_grouped_heads"]


def run_pin(name, attn):
    fn = globals()[name]
    if name == "pin_identical_keys":
        return fn(attn, loop_visible)
    return fn(attn)
