"""The CPU oracle checked against facts other than itself (CPU only)."""
import math

import numpy as np
import pytest

import oracle
import oracle_pins as P
from efficient_exact_attention_amd import workloads as W


@pytest.mark.parametrize("name", P.ALL_PINS)
def test_pin(name):
    P.run_pin(name, oracle.attention)


# ---- visible-pair counts: closed forms from the pages' complexity terms -------
# causal: triangle; sliding window of w keys: O(n w); symmetric band: O(n w);
# band plus g global tokens: O(n g + n w) ("Module 9", table in "Sparse and
# windowed attention"; week-17 notes, local-window passage).

def causal_pairs(N):
    return N * (N + 1) // 2


def swa_pairs(N, w):
    """Causal window of w keys including the diagonal (win_left = w - 1)."""
    if N <= w:
        return causal_pairs(N)
    return w * (w + 1) // 2 + (N - w) * w


def band_pairs(N, r):
    """Symmetric band i-r..i+r clipped, N >= r."""
    return N * (2 * r + 1) - r * (r + 1)


def band_global_pairs(N, r, G):
    """Non-causal band plus global rows/columns, by inclusion-exclusion."""
    G = sorted(set(G))
    g = len(G)

    def row_band(i):
        return min(i, r) + min(N - 1 - i, r) + 1
    inter_r = sum(row_band(i) for i in G)                 # band & global rows
    inter_rc = sum(1 for a in G for b in G if abs(a - b) <= r)
    return band_pairs(N, r) + 2 * g * N - g * g - 2 * inter_r + inter_rc


@pytest.mark.parametrize("N", [1, 2, 7, 64, 129, 300])
def test_pair_counts_small(N):
    assert oracle.visible_pairs_bruteforce(N, 1, -1, -1) == causal_pairs(N)
    assert oracle.visible_pairs_bruteforce(N, 0, -1, -1) == N * N
    for w in (1, 2, 5, 64, 400):
        assert oracle.visible_pairs_bruteforce(N, 1, w - 1, 0) == swa_pairs(N, w)
        assert oracle.visible_pairs_bruteforce(N, 1, w - 1, -1) == swa_pairs(N, w)
    for r in (0, 1, 3, 17):
        if N >= r:
            assert oracle.visible_pairs_bruteforce(N, 0, r, r) == band_pairs(N, r)
            G = [x for x in (0, 1, N // 3, N - 1) if x < N]
            assert oracle.visible_pairs_bruteforce(N, 0, r, r, tuple(sorted(set(G)))) == \
                band_global_pairs(N, r, G)


def test_pair_counts_workloads():
    """Per-head visible pairs of the benchmark workloads: closed form and, for
    the sizes that finish quickly, the oracle's own mask."""
    assert causal_pairs(4096) == 8_390_656
    assert swa_pairs(32768, 4096) == 125_831_168
    assert causal_pairs(131072) == 8_590_000_128
    assert causal_pairs(32768) == 536_887_296
    G = W.WORKLOADS["band256_globals_16k"].global_idx
    assert len(G) == 9
    assert band_global_pairs(16384, 256, G) == 8_625_830
    assert oracle.visible_pairs_bruteforce(16384, 0, 256, 256, G) == 8_625_830
    assert oracle.visible_pairs_bruteforce(4096, 1, -1, -1) == 8_390_656
    # the alternative reading of the Mistral window (w+1 keys) differs
    assert oracle.visible_pairs_bruteforce(4096, 1, 512, 0) == swa_pairs(4096, 513)


def test_mask_matches_scalar_predicate():
    rng = np.random.default_rng(0)
    for _ in range(30):
        N = int(rng.integers(1, 40))
        m = dict(causal=int(rng.integers(0, 2)), win_left=int(rng.integers(-1, 6)),
                 win_right=int(rng.integers(-1, 6)))
        G = tuple(sorted(set(int(x) for x in rng.integers(0, N, size=int(rng.integers(0, 4))))))
        vis = oracle.mask_rows(np.arange(N), N, global_idx=G, **m)
        for i in range(N):
            for j in range(N):
                assert vis[i, j] == P.loop_visible(i, j, N, dict(m, global_idx=G))
                assert vis[i, j] == oracle.visible(i, j, N, m["causal"], m["win_left"],
                                                   m["win_right"], set(G))


# ---- P3 probabilities sum to one; masked weights are exactly zero ----------------

@pytest.mark.parametrize("m", P.MASKS)
def test_probabilities_sum_to_one(m):
    q, k, _ = P._rng_qkv(5, 1, 2, 31, 8)
    p = oracle.probabilities(q, k, **m)
    assert np.max(np.abs(p.sum(-1) - 1.0)) <= 1e-12
    vis = np.array([[P.loop_visible(i, j, 31, m) for j in range(31)] for i in range(31)])
    assert np.all(p[:, :, ~vis] == 0.0)
    assert np.all(p[:, :, vis] > 0.0)


# ---- P8 attention over key blocks, merged, equals the two-pass definition --------

@pytest.mark.parametrize("m", P.MASKS)
def test_blockwise_merge(m):
    q, k, v = P._rng_qkv(9, 1, 1, 37, 8, scale=2.0)
    O, L = oracle.attention(q, k, v, **m)
    vis = oracle.mask_rows(np.arange(37), 37, global_idx=m["global_idx"],
                           **{x: m[x] for x in ("causal", "win_left", "win_right")})
    rng = np.random.default_rng(10)
    splits = [[], list(range(1, 37)), list(range(16, 37, 16))]   # one block, single keys, 16-key tiles
    splits += [sorted(rng.choice(np.arange(1, 37), size=n, replace=False)) for n in (1, 2, 5, 11, 20) for _ in range(3)]
    for cuts in splits:
        Ob, Lb = oracle.blockwise_attention_rows(q[0, 0], k[0, 0], v[0, 0], vis, cuts)
        assert np.max(np.abs(Ob - O[0, 0])) <= 1e-12
        assert np.max(np.abs(Lb - L[0, 0])) <= 1e-12


def test_blockwise_merge_survives_large_scores():
    """Scores near 700 (exp overflows fp64 beyond 709): the block summaries
    must keep everything relative to their own maxima."""
    q, k, v = P._rng_qkv(11, 1, 1, 23, 4)
    q = q * 0 + 1.0
    k = k.copy()
    k[0, 0, :, :] = 350.0 + np.arange(23)[:, None] * 0.25   # scaled scores 700..711
    vis = np.ones((23, 23), bool)
    O, L = oracle.attention(q, k, v, causal=0, win_left=-1, win_right=-1)
    Ob, Lb = oracle.blockwise_attention_rows(q[0, 0], k[0, 0], v[0, 0], vis, [4, 9, 17])
    assert np.all(np.isfinite(Ob)) and np.all(np.isfinite(Lb))
    assert np.max(np.abs(Ob - O[0, 0])) <= 1e-12
    assert np.max(np.abs(Lb - L[0, 0])) <= 1e-9


def test_row_subset_matches_full():
    q, k, v = P._rng_qkv(13, 2, 2, 90, 8)
    rows = np.array([0, 5, 44, 89])
    for m in P.MASKS:
        O, L = oracle.attention(q, k, v, **m)
        Os, Ls = oracle.attention(q, k, v, rows=rows, row_block=3, **m)
        # BLAS may block differently for other row counts: agree to rounding
        assert np.max(np.abs(O[:, :, rows] - Os)) <= 1e-14
        assert np.max(np.abs(L[:, :, rows] - Ls)) <= 1e-14


def test_useful_flops():
    # 4 d per visible pair: two flops per multiply-add in each of the two products
    assert oracle.useful_flops(1, 32, 128, causal_pairs(32768)) == 4 * 128 * 536_887_296 * 32
    assert math.isclose(oracle.useful_flops(1, 32, 128, causal_pairs(32768)), 8.796e12, rel_tol=1e-3)
