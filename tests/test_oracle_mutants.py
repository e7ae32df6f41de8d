"""Plant plausible mistakes in copies of the oracle (CPU only) and show that
the pins in ``oracle_pins`` catch every one of them."""
import math

import numpy as np
import pytest

import oracle
import oracle.masked_attention as OA
import oracle_pins as P


def _fails(attn, monkey=None):
    failed = []
    for name in P.ALL_PINS:
        try:
            P.run_pin(name, attn)
        except (AssertionError, ValueError):   # a pin the mutant cannot even run also catches it
            failed.append(name)
    return failed


def no_scale(q, k, v, **kw):
    kw.pop("scale", None)
    return oracle.attention(q, k, v, scale=1.0, **kw)


def swapped_kv(q, k, v, **kw):
    return oracle.attention(q, v, k, **kw)


def transposed_scores(q, k, v, **kw):
    # uses keys where queries belong (scores transposed)
    return oracle.attention(k, q, v, **kw)


def lse_log2(q, k, v, **kw):
    O, L = oracle.attention(q, k, v, **kw)
    return O, L / math.log(2.0)


def lse_unscaled(q, k, v, **kw):
    O, L = oracle.attention(q, k, v, **kw)
    d = q.shape[-1]
    return O, L * math.sqrt(d)


def sign_flip(q, k, v, **kw):
    return oracle.attention(-q, k, v, **kw)


def globals_dropped(q, k, v, **kw):
    kw = dict(kw, global_idx=())
    return oracle.attention(q, k, v, **kw)


def window_shift_left(q, k, v, **kw):
    wl = kw.get("win_left", -1)
    return oracle.attention(q, k, v, **dict(kw, win_left=wl + 1 if wl >= 0 else wl))


def window_right_ignored(q, k, v, **kw):
    return oracle.attention(q, k, v, **dict(kw, win_right=-1))


def causal_ignored(q, k, v, **kw):
    return oracle.attention(q, k, v, **dict(kw, causal=0))


def groups_interleaved(q, k, v, **kw):
    # query head h reads K/V head h % H_kv instead of h // (H / H_kv)
    H, H_kv = q.shape[1], k.shape[1]
    idx = [h % H_kv for h in range(H)]
    return oracle.attention(q, k[:, idx], v[:, idx], **kw)


def first_kv_head_only(q, k, v, **kw):
    # every query head reads K/V head 0
    H = q.shape[1]
    return oracle.attention(q, k[:, [0] * H], v[:, [0] * H], **kw)


MUTANTS = [no_scale, swapped_kv, transposed_scores, lse_log2, lse_unscaled, sign_flip,
           globals_dropped, window_shift_left, window_right_ignored, causal_ignored,
           groups_interleaved, first_kv_head_only]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda f: f.__name__)
def test_mutant_is_caught(mutant):
    assert _fails(mutant), f"no pin caught {mutant.__name__}"


def _mask_global_rows_only(rows, N, causal, win_left, win_right, global_idx=(), block=0, dilation=1, *extra):
    """Mask with the global-column term dropped (globals see all, but are not seen)."""
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(N, dtype=np.int64)[None, :]
    band = np.ones((i.shape[0], N), dtype=bool)
    if win_left >= 0:
        band &= j >= i - win_left
    if win_right >= 0:
        band &= j <= i + win_right
    g = np.zeros(N, dtype=bool)
    if len(global_idx):
        g[np.asarray(global_idx)] = True
    vis = band | g[i]
    if causal:
        vis &= j <= i
    return vis


def _mask_strict_window(rows, N, causal, win_left, win_right, global_idx=(), block=0, dilation=1, *extra):
    """Window bounds taken as strict (off by one on both sides)."""
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(N, dtype=np.int64)[None, :]
    band = np.ones((i.shape[0], N), dtype=bool)
    if win_left >= 0:
        band &= j > i - win_left
    if win_right >= 0:
        band &= j < i + win_right
    band |= (j == i)
    g = np.zeros(N, dtype=bool)
    if len(global_idx):
        g[np.asarray(global_idx)] = True
    vis = band | g[i] | g[j]
    if causal:
        vis &= j <= i
    return vis


@pytest.mark.parametrize("bad_mask", [_mask_global_rows_only, _mask_strict_window],
                         ids=lambda f: f.__name__)
def test_mask_mutant_is_caught(monkeypatch, bad_mask):
    monkeypatch.setattr(OA, "mask_rows", bad_mask)
    assert _fails(oracle.attention)


def test_missing_max_subtraction_is_caught(monkeypatch):
    real_where = np.where

    def attention_nomax(q, k, v, **kw):
        # exp of raw scores: overflows for the large key shifts of the key-shift pin
        q = np.asarray(q, np.float64); k = np.asarray(k, np.float64); v = np.asarray(v, np.float64)
        B, H, N, d = q.shape
        scale = 1.0 / math.sqrt(d)
        vis = OA.mask_rows(np.arange(N), N, kw["causal"], kw.get("win_left", -1),
                           kw.get("win_right", -1), kw.get("global_idx", ()))
        with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
            s = np.einsum("bhnd,bhmd->bhnm", q, k) * scale
            p = real_where(vis, np.exp(s), 0.0)
            l = p.sum(-1, keepdims=True)
            return p @ v / l, np.log(l[..., 0])
    assert "pin_key_shift" in _fails(attention_nomax)
