"""Pins of the decode oracle (CPU): the last rows of a forward attention, a
rolling cache against the contiguous cache of the same sequence, the
single-key and constant-value cases, and torch SDPA on the unrolled
sequence."""
import math

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")


def _seq(seed, B, H, H_kv, L, d):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, L, d)), rng.standard_normal((B, H_kv, L, d)),
            rng.standard_normal((B, H_kv, L, d)))


def _roll(x, S):
    """Rolling cache of S slots after writing positions 0..L-1 in order."""
    B, H, L, d = x.shape
    c = np.zeros((B, H, S, d))
    for p in range(L):
        c[:, :, p % S] = x[:, :, p]
    return c


@pytest.mark.parametrize("Nq", [1, 3])
@pytest.mark.parametrize("wl", [-1, 9])
def test_decode_is_the_last_rows_of_forward(Nq, wl):
    q, k, v = _seq(1, 2, 4, 2, 40, 8)
    O, L = oracle.attention(q, k, v, causal=1, win_left=wl, win_right=0)
    Od, Ld = oracle.decode(q[:, :, 40 - Nq:], k, v, [40, 40], win_left=wl)
    assert np.max(np.abs(Od - O[:, :, 40 - Nq:])) <= 1e-12
    assert np.max(np.abs(Ld - L[:, :, 40 - Nq:])) <= 1e-12


def test_variable_lengths():
    q, k, v = _seq(2, 3, 2, 2, 50, 8)
    lens = [50, 17, 31]
    Od, Ld = oracle.decode(q[:, :, :2], k, v, lens)
    for b, Lb in enumerate(lens):
        qs = q[b:b + 1].copy()
        qs[:, :, Lb - 2:Lb] = q[b:b + 1, :, :2]
        O, L = oracle.attention(qs[:, :, :Lb], k[b:b + 1, :, :Lb], v[b:b + 1, :, :Lb], causal=1,
                                rows=np.arange(Lb - 2, Lb))
        assert np.max(np.abs(Od[b] - O[0])) <= 1e-12


@pytest.mark.parametrize("W,Nq,S", [(8, 1, 8), (8, 2, 9), (5, 3, 12)])
def test_rolling_cache_matches_contiguous(W, Nq, S):
    """A rolling cache that still holds every window gives the same result as
    the contiguous cache of the whole sequence."""
    q, k, v = _seq(3, 1, 2, 1, 37, 8)
    Oc, Lc = oracle.decode(q[:, :, :Nq], k, v, [37], win_left=W - 1)
    Or, Lr = oracle.decode(q[:, :, :Nq], _roll(k, S), _roll(v, S), [37], win_left=W - 1, rolling=True)
    assert np.max(np.abs(Oc - Or)) <= 1e-12 and np.max(np.abs(Lc - Lr)) <= 1e-12


def test_single_visible_key_and_constant_values():
    q, k, v = _seq(4, 1, 2, 2, 20, 8)
    # window 0: the newest token sees only itself
    O, L = oracle.decode(q[:, :, :1], k, v, [20], win_left=0)
    assert np.max(np.abs(O[0, :, 0] - v[0, :, 19])) <= 1e-12
    assert np.max(np.abs(L[0, :, 0] - (q[0, :, 0] * k[0, :, 19]).sum(-1) / math.sqrt(8))) <= 1e-12
    vc = np.broadcast_to(np.linspace(-1, 1, 8), v.shape).copy()
    O, _ = oracle.decode(q[:, :, :2], k, vc, [20])
    assert np.max(np.abs(O - np.linspace(-1, 1, 8))) <= 1e-12


def test_decode_against_torch():
    q, k, v = _seq(5, 1, 4, 2, 30, 16)
    Od, _ = oracle.decode(q[:, :, :2], k, v, [30], win_left=12)
    N = 30
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    mask = (j <= i) & (j >= i - 12)
    qs = torch.from_numpy(q).clone()
    qs[:, :, 28:30] = torch.from_numpy(q[:, :, :2])
    ref = torch.nn.functional.scaled_dot_product_attention(qs, torch.from_numpy(k), torch.from_numpy(v),
                                                           attn_mask=torch.from_numpy(mask), enable_gqa=True)
    assert np.max(np.abs(Od - ref.numpy()[:, :, 28:30])) <= 1e-12
