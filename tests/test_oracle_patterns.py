"""Pins of the oracle's block-sparse and dilated masks (CPU): the scalar
predicate against the vectorised mask, closed-form pair counts, the residue
class identity of dilated attention, and torch SDPA under the explicit
boolean mask."""
import math

import numpy as np
import pytest

import oracle
from oracle.masked_attention import visible

torch = pytest.importorskip("torch")


def _scalar_mask(N, causal, wl, wr, G=(), block=0, dilation=1):
    gs = set(G)
    return np.array([[visible(i, j, N, causal, wl, wr, gs, block, dilation) for j in range(N)]
                     for i in range(N)])


CASES = [
    dict(causal=0, win_left=-1, win_right=-1, block=8),
    dict(causal=1, win_left=-1, win_right=-1, block=8),
    dict(causal=1, win_left=-1, win_right=-1, block=5, global_idx=(3, 40)),
    dict(causal=0, win_left=-1, win_right=-1, block=64),
    dict(causal=1, win_left=-1, win_right=-1, dilation=3),
    dict(causal=0, win_left=-1, win_right=-1, dilation=4),
    dict(causal=1, win_left=5, win_right=0, dilation=3),
    dict(causal=0, win_left=2, win_right=3, dilation=2),
    dict(causal=0, win_left=4, win_right=4, dilation=5, global_idx=(0, 7, 33)),
]


@pytest.mark.parametrize("N", [1, 13, 50, 67])
@pytest.mark.parametrize("m", CASES)
def test_vector_mask_matches_scalar(N, m):
    G = tuple(g for g in m.get("global_idx", ()) if g < N)
    ref = _scalar_mask(N, m["causal"], m["win_left"], m["win_right"], G, m.get("block", 0), m.get("dilation", 1))
    got = oracle.mask_rows(np.arange(N), N, m["causal"], m["win_left"], m["win_right"], G,
                           m.get("block", 0), m.get("dilation", 1))
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("b,nb", [(1, 7), (4, 5), (16, 3), (32, 1)])
def test_block_pair_counts(b, nb):
    N = b * nb
    # non-causal: every row sees its block and the one before (2b keys), rows
    # of the first block only their own (b keys)
    assert oracle.visible_pairs_bruteforce(N, 0, -1, -1, block=b) == (2 * N - b) * b
    # causal: the whole previous block, and its own block up to itself
    assert oracle.visible_pairs_bruteforce(N, 1, -1, -1, block=b) == (nb - 1) * b * b + nb * b * (b + 1) // 2


@pytest.mark.parametrize("k,m", [(1, 9), (2, 8), (3, 7), (5, 4)])
def test_dilated_pair_counts(k, m):
    N = k * m
    # causal, unbounded: row i sees i, i-k, ... down to i mod k: floor(i/k) + 1 keys
    assert oracle.visible_pairs_bruteforce(N, 1, -1, -1, dilation=k) == k * m * (m - 1) // 2 + N
    # non-causal, unbounded: every row sees the m positions of its residue class
    assert oracle.visible_pairs_bruteforce(N, 0, -1, -1, dilation=k) == N * m
    # causal with a window of w dilated steps: min(floor(i/k), w) + 1 keys
    w = 2
    assert oracle.visible_pairs_bruteforce(N, 1, w, 0, dilation=k) == sum(min(i // k, w) + 1 for i in range(N))


def test_pattern_special_cases():
    N = 40
    # dilation 1 is the plain window; a block covering the sequence is full
    for c, wl, wr in [(1, 5, 0), (0, 3, 9), (0, -1, -1)]:
        assert np.array_equal(oracle.mask_rows(np.arange(N), N, c, wl, wr, (), 0, 1),
                              oracle.mask_rows(np.arange(N), N, c, wl, wr))
    assert oracle.mask_rows(np.arange(N), N, 0, -1, -1, (), N, 1).all()


@pytest.mark.parametrize("k", [2, 3, 4])
@pytest.mark.parametrize("c,wl,wr", [(1, -1, -1), (1, 3, 0), (0, 2, 5)])
def test_dilated_is_windowed_attention_on_residue_classes(k, c, wl, wr):
    """Rows i = r + m*k of a dilated attention see exactly the keys of their
    residue class within the window (counted in steps), so their outputs and
    LSE equal a plain windowed attention over the subsequence x[r::k]."""
    rng = np.random.default_rng(k * 10 + wl)
    N, d = 61, 8
    q, kk, v = (rng.standard_normal((1, 2, N, d)) for _ in range(3))
    O, L = oracle.attention(q, kk, v, causal=c, win_left=wl, win_right=wr, dilation=k)
    for r in range(k):
        Os, Ls = oracle.attention(q[:, :, r::k], kk[:, :, r::k], v[:, :, r::k], causal=c,
                                  win_left=wl, win_right=wr, scale=1 / math.sqrt(d))
        assert np.max(np.abs(O[:, :, r::k] - Os)) <= 1e-12
        assert np.max(np.abs(L[:, :, r::k] - Ls)) <= 1e-12


@pytest.mark.parametrize("m", CASES)
def test_patterns_against_torch_sdpa(m):
    N, d = 70, 16
    rng = np.random.default_rng(5)
    q, k, v = (rng.standard_normal((2, 2, N, d)) for _ in range(3))
    G = tuple(g for g in m.get("global_idx", ()) if g < N)
    kw = dict(causal=m["causal"], win_left=m["win_left"], win_right=m["win_right"], global_idx=G,
              block=m.get("block", 0), dilation=m.get("dilation", 1))
    O, _ = oracle.attention(q, k, v, **kw)
    mask = _scalar_mask(N, m["causal"], m["win_left"], m["win_right"], G, kw["block"], kw["dilation"])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=torch.from_numpy(mask))
    assert np.max(np.abs(O - ref.numpy())) <= 1e-12
