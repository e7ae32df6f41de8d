"""CPU fp64 oracle for decoding with a key/value cache.

TEST INFRASTRUCTURE. Only the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import or call this module. The product path
never does, and this module imports nothing from the product package.

Decoding keeps the keys and values of every earlier token instead of
recomputing them, and the newest tokens' queries attend over that cache, one
step per generated token (week-17 lecture notes, inference cost per token
with a KV cache; "Beyond attention", the rolling cache of a sliding window:
at n = 32,768 with W = 4,096 it keeps 4,096 positions). What it computes is
the ordinary masked attention of the newest rows over the whole sequence
(``masked_attention.attention``); this module only says where each position's
key and value sit in the cache:

* contiguous cache: position p is slot p;
* rolling cache of S slots: position p is slot p mod S, so the cache holds
  the last S positions and a newer position overwrites the oldest.

Readings (the pages give no layout): the Nq newest tokens of a sequence of
length L are positions L-Nq .. L-1, causal among themselves, and a window of
win_left lets position i see positions i - win_left .. i.
"""
from __future__ import annotations

import numpy as np

from .masked_attention import attention


def slot_of(p: int, S: int, rolling: bool) -> int:
    return p % S if rolling else p


def cache_to_sequence(cache, L: int, rolling: bool):
    """[B?, H, S, d] cache rows of positions 0..L-1, in position order. With a
    rolling cache only the last S positions are present; earlier ones come
    back as NaN (a correct decode never reads them)."""
    cache = np.asarray(cache)
    S = cache.shape[-2]
    seq = np.full(cache.shape[:-2] + (L, cache.shape[-1]), np.nan)
    for p in range(max(0, L - S) if rolling else 0, L):
        seq[..., p, :] = cache[..., slot_of(p, S, rolling), :]
    return seq


def decode(q, k_cache, v_cache, seq_len, *, win_left: int = -1, rolling: bool = False,
           scale: float | None = None):
    """Outputs and LSE of the newest Nq queries of each sequence.

    q: [B, H, Nq, d]; k_cache, v_cache: [B, H_kv, S, d]; seq_len: [B] total
    lengths L_b (including the Nq new tokens). Returns (O [B, H, Nq, d],
    LSE [B, H, Nq]) in fp64."""
    q = np.asarray(q, dtype=np.float64)
    B, H, Nq, d = q.shape
    O = np.zeros((B, H, Nq, d))
    LSE = np.zeros((B, H, Nq))
    for b in range(B):
        L = int(seq_len[b])
        k = cache_to_sequence(np.asarray(k_cache[b], np.float64), L, rolling)
        v = cache_to_sequence(np.asarray(v_cache[b], np.float64), L, rolling)
        if rolling:   # positions before the cache's reach must not be visible
            oldest = max(0, L - k_cache.shape[-2])
            assert win_left >= 0 and L - Nq - win_left >= oldest or L <= k_cache.shape[-2], \
                "rolling cache shorter than the window"
            k = np.nan_to_num(k, nan=0.0)
            v = np.nan_to_num(v, nan=0.0)
        rows = np.arange(L - Nq, L)
        qs = np.zeros((1, H, L, d))
        qs[0, :, L - Nq:L] = q[b]
        Ob, Lb = attention(qs, k[None], v[None], causal=1, win_left=win_left, win_right=0, rows=rows,
                           scale=scale)
        O[b] = Ob[0]
        LSE[b] = Lb[0]
    return O, LSE
