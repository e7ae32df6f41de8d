"""CPU fp64 oracle for the backward pass of exact masked attention.

TEST INFRASTRUCTURE. Only the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import or call this module. The product path
never does, and this module imports nothing from the product package.

The pages say only that an exact, tiled attention keeps no N x N matrix and
"recomputes what is needed in the backward pass" ("Efficient Transformers:
Sparse Attention, Linear Attention and FlashAttention", "Family 3"). The
gradient itself is the plain derivative of the forward definition (the
masked softmax attention of ``masked_attention.attention``), written out here
with the usual chain rule, no tiling:

    S  = scale * Q K^T, masked entries -inf      P = softmax_rows(S)
    O  = P V
    dV = P^T dO
    dP = dO V^T
    dS = P * (dP - rowsum(dP * P))               (softmax Jacobian, per row)
    dQ = scale * dS K
    dK = scale * dS^T Q

rowsum(dP * P) equals rowsum(dO * O), the form a recomputing kernel uses.
With H_kv < H K/V heads (grouped-query attention) a K/V head's gradient is
the sum over the query heads that read it. Masked pairs have P = 0 and so
contribute nothing. Readings: gradients are taken with respect to the inputs
as given (the scale is a constant), and a row with no visible key (not
possible under the argument rules) contributes nothing.
"""
from __future__ import annotations

import math

import numpy as np

from .masked_attention import mask_rows


def attention_backward(q, k, v, dout, *, causal: int, win_left: int = -1, win_right: int = -1,
                       global_idx=(), scale: float | None = None, block: int = 0, dilation: int = 1,
                       stride: int = 0, rand_block: int = 0, rand_idx=None):
    """(dQ [B, H, N, d], dK [B, H_kv, N, d], dV [B, H_kv, N, d]) in fp64 for
    O = attention(q, k, v) and upstream gradient dout [B, H, N, d]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    if H_kv < 1 or H % H_kv or v.shape[1] != H_kv:
        raise ValueError(f"K/V heads {H_kv} must divide query heads {H}")
    group = H // H_kv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    vis = mask_rows(np.arange(N), N, causal, win_left, win_right, global_idx, block, dilation, stride,
                    rand_block, rand_idx)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            kh = h // group
            s = (q[b, h] @ k[b, kh].T) * scale
            s = np.where(vis, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            m = np.where(np.isfinite(m), m, 0.0)
            e = np.exp(s - m)
            l = e.sum(axis=1, keepdims=True)
            p = e / np.where(l > 0, l, 1.0)                # masked -> 0
            do = dout[b, h]
            dv[b, kh] += p.T @ do
            dp = do @ v[b, kh].T
            ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))
            dq[b, h] = scale * (ds @ k[b, kh])
            dk[b, kh] += scale * (ds.T @ q[b, h])
    return dq, dk, dv


def delta_rows(out, dout):
    """rowsum(dO * O) per query row, [B, H, N] fp64: the per-row term of the
    softmax Jacobian that a recomputing backward pass reads instead of
    rowsum(dP * P)."""
    return (np.asarray(out, np.float64) * np.asarray(dout, np.float64)).sum(axis=-1)
