"""CPU fp64 oracle for exact scaled dot-product attention with sparse masks.

TEST INFRASTRUCTURE. Only the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import or call this module. The product path
never does, and this module imports nothing from the product package.

What it computes (plain definition, no tiling, no fusion):

* Attention: each output row is the softmax-weighted sum of value rows, the
  weights being the softmax over keys of the query-key dot products divided by
  the square root of the head size. Sources: "Week 17 lecture notes on
  efficient attention" (neelsoumya.github.io), opening recap of scaled
  dot-product attention and its cost table; "Module 9 - Quadratic cost and
  efficient attention", section "Where the n^2 hides".
* Masking: invisible pairs get a score of minus infinity before the softmax,
  as in the masked naive attention of "Efficient Transformers: Sparse
  Attention, Linear Attention and FlashAttention" (section "Family 3") and the
  sliding-window mask code of the week-17 notes.
* Mask sets:
    - local window, row i sees i-wl .. i+wr clipped to the sequence (week-17
      notes, local-window passage; "Module 9", table in "Sparse and windowed
      attention");
    - Mistral-style causal sliding window (week-17 notes, Mistral passage;
      "Sparse & sub-quadratic attention", section "Escape 1");
    - global tokens that see every position and are seen by every position
      (week-17 notes, global-token passage; "Efficient Transformers",
      "Family 1"; "Sparse & sub-quadratic attention", "Escape 1");
    - log-spaced strides: row i also sees the positions at distance s, 2s,
      4s, ... ("Module 9", table in "Sparse and windowed attention": the
      strided / dilated family at strides s, 2s, 4s with O(n log n) cost);
    - random blocks: row i also sees every key of the key blocks listed for
      its query block (week-17 notes, BigBird passage: global tokens + local
      window + random attention; "Efficient Transformers", "Family 1"). The
      random draw is an input (the list), so the definition is deterministic.
  Readings used where the pages leave a choice open:
    - ``win_left``/``win_right`` count keys strictly left/right of the
      diagonal; -1 means unbounded on that side;
    - ``causal`` is combined with everything else by AND;
    - a pair is visible if it is in the window band OR its row is global OR
      its column is global OR (with a stride s) the distance |i - j| is s
      times a power of two OR (with random blocks of size b) block j // b is
      in the list of block i // b; each pair counted once. Random-list
      entries outside the block range are ignored and repeated entries count
      once;
    - LSE is the natural log of the sum over visible keys of exp(scaled
      score), one value per query row;
    - a row with no visible key (impossible under the argument rules, since
      the diagonal is always visible) yields output 0 and LSE -inf.

``blockwise_attention_rows`` computes the same rows over arbitrary key blocks
whose summaries (log-sum-exp and block-normalised output) are merged, the
decomposition behind the FlashAttention passage of the week-17 notes, so that
the algebra the GPU kernel relies on is itself checked against the two-pass
definition above.
"""
from __future__ import annotations

import math

import numpy as np


def _is_log_stride(dist: int, stride: int) -> bool:
    """dist = stride * 2^m for some whole m >= 0 (scalar form)."""
    if stride <= 0 or dist <= 0 or dist % stride:
        return False
    m = dist // stride
    while m % 2 == 0:
        m //= 2
    return m == 1


def visible(i: int, j: int, N: int, causal: int, win_left: int, win_right: int,
            global_set, block: int = 0, dilation: int = 1, stride: int = 0,
            rand_block: int = 0, rand_idx=None) -> bool:
    """Scalar visibility predicate: may query row i attend to key j?

    The local part of the mask is one of
      * the window: j in [i - win_left, i + win_right] (-1: unbounded side);
      * block-sparse (block > 0): j lies in the block of i or in the block
        just before it, blocks being runs of `block` positions ("Sparse &
        sub-quadratic attention", "Escape 1": attend within your block and
        the previous one); win_left / win_right are not used;
      * dilated (dilation k > 1): j = i - m*k for whole m ("Week 17 lecture
        notes", dilated passage: i, i-k, i-2k, ...), with the window counted
        in dilated steps: -win_right <= m <= win_left.
    Causal (j <= i) is ANDed with everything; global rows and columns, the
    log-spaced strides and the random blocks are ORed with the local part."""
    if not (0 <= i < N and 0 <= j < N):
        return False
    if causal and j > i:
        return False
    if block > 0:
        local = (j // block) in (i // block, i // block - 1)
    elif dilation > 1:
        diff = i - j
        local = (diff % dilation == 0 and (win_left < 0 or diff <= win_left * dilation)
                 and (win_right < 0 or -diff <= win_right * dilation))
    else:
        local = (win_left < 0 or j >= i - win_left) and (win_right < 0 or j <= i + win_right)
    strided = _is_log_stride(abs(i - j), stride)
    rand = False
    if rand_block > 0 and rand_idx is not None:
        rand = (j // rand_block) in set(int(x) for x in rand_idx[i // rand_block])
    return bool(local or (i in global_set) or (j in global_set) or strided or rand)


def mask_rows(rows, N: int, causal: int, win_left: int, win_right: int,
              global_idx=(), block: int = 0, dilation: int = 1, stride: int = 0,
              rand_block: int = 0, rand_idx=None) -> np.ndarray:
    """Boolean visibility matrix [len(rows), N]: the predicate of `visible`
    evaluated for every (row, key) pair. rand_idx: [ceil(N / rand_block), r]
    key-block lists, one row per query block."""
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(N, dtype=np.int64)[None, :]
    if block > 0:
        band = (j // block == i // block) | (j // block == i // block - 1)
    else:
        k = max(int(dilation), 1)
        band = ((i - j) % k == 0) if k > 1 else np.ones((i.shape[0], N), dtype=bool)
        if win_left >= 0:
            band = band & (j >= i - win_left * k)
        if win_right >= 0:
            band = band & (j <= i + win_right * k)
    is_global = np.zeros(N, dtype=bool)
    if len(global_idx):
        is_global[np.asarray(global_idx, dtype=np.int64)] = True
    vis = band | is_global[i] | is_global[j]
    if stride > 0:   # |i - j| in {s, 2s, 4s, ...}
        dist = np.abs(i - j)
        m = np.where(dist % stride == 0, dist // stride, 0)
        vis = vis | ((m > 0) & ((m & (m - 1)) == 0))
    if rand_block > 0 and rand_idx is not None:
        lists = np.asarray(rand_idx, dtype=np.int64)
        qb = (i[:, 0] // rand_block)
        kb = j[0] // rand_block
        for e in range(lists.shape[1]):
            vis = vis | (kb[None, :] == lists[qb, e][:, None])
    if causal:
        vis &= j <= i
    return vis


def attention(q, k, v, *, causal: int, win_left: int = -1, win_right: int = -1,
              global_idx=(), rows=None, scale: float | None = None,
              row_block: int = 256, block: int = 0, dilation: int = 1, stride: int = 0,
              rand_block: int = 0, rand_idx=None):
    """Masked softmax attention in fp64.

    q:       [B, H, N, d]; k, v: [B, H_kv, N, d] with H_kv dividing H (any
             real dtype; upcast to float64). H_kv < H is grouped-query
             attention and H_kv = 1 multi-query attention (week-17 notes, the
             MQA / GQA passage: groups of query heads share one K and one V
             head). Reading: the groups are runs of consecutive query heads,
             query head h using K/V head h // (H // H_kv).
    rows:    optional 1-D array of query rows to compute (default: all).
    Returns (O [B, H, R, d] float64, LSE [B, H, R] float64).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    if H_kv < 1 or H % H_kv or v.shape[1] != H_kv:
        raise ValueError(f"K/V heads {H_kv} must divide query heads {H}")
    group = H // H_kv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    out = np.zeros((B, H, R, v.shape[-1]), dtype=np.float64)
    lse = np.full((B, H, R), -np.inf, dtype=np.float64)
    for r0 in range(0, R, row_block):
        rb = rows[r0:r0 + row_block]
        vis = mask_rows(rb, N, causal, win_left, win_right, global_idx, block, dilation, stride,
                        rand_block, rand_idx)
        any_vis = vis.any(axis=1)
        for b in range(B):
            for h in range(H):
                kh = h // group                                # shared K/V head
                s = (q[b, h, rb] @ k[b, kh].T) * scale         # full score rows
                s = np.where(vis, s, -np.inf)
                m = s.max(axis=1, keepdims=True)
                m = np.where(np.isfinite(m), m, 0.0)
                p = np.exp(s - m)                              # masked -> 0
                l = p.sum(axis=1, keepdims=True)
                safe_l = np.where(l > 0, l, 1.0)
                out[b, h, r0:r0 + len(rb)] = np.where(any_vis[:, None], (p @ v[b, kh]) / safe_l, 0.0)
                lse[b, h, r0:r0 + len(rb)] = np.where(any_vis, m[:, 0] + np.log(safe_l[:, 0]), -np.inf)
    return out, lse


def probabilities(q, k, *, causal: int, win_left: int = -1, win_right: int = -1,
                  global_idx=(), rows=None, scale: float | None = None, block: int = 0,
                  dilation: int = 1, stride: int = 0, rand_block: int = 0, rand_idx=None):
    """Softmax weights [B, H, R, N] (fp64) of the same definition; used to
    check that visible weights sum to one and masked weights are zero."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    vis = mask_rows(rows, N, causal, win_left, win_right, global_idx, block, dilation, stride,
                    rand_block, rand_idx)
    s = np.einsum("bhrd,bhnd->bhrn", q[:, :, rows], k) * scale
    s = np.where(vis[None, None], s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    p = np.exp(s - m)
    l = p.sum(axis=-1, keepdims=True)
    return p / np.where(l > 0, l, 1.0)


def blockwise_attention_rows(q_rows, k, v, vis, cuts, scale: float | None = None):
    """Attention of each query row computed over key blocks and merged, the
    decomposition the FlashAttention passage of the week-17 notes rests on
    (softmax over the keys taken one block at a time, never holding a full
    row of scores).

    Here every block is first reduced on its own to a summary: the natural
    log of its visible mass (its log-sum-exp) and its output normalised
    within the block. The summaries are then folded left to right, each merge
    weighting the two outputs by their shares of the combined mass. The
    blocks are arbitrary: `cuts` lists the interior boundaries (sorted key
    indices in 1..N-1), so the tests can split the keys at random places.
    q_rows: [R, d]; k, v: [N, d]; vis: bool [R, N]. Returns (O [R, d], LSE [R]).
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    R, d = q_rows.shape
    N = k.shape[0]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    edges = [0] + [int(c) for c in cuts] + [N]
    O = np.zeros((R, v.shape[1]))
    LSE = np.full(R, -np.inf)
    for r in range(R):
        total, out = -np.inf, np.zeros(v.shape[1])
        for a, b in zip(edges[:-1], edges[1:]):
            if b <= a:
                continue
            s = np.where(vis[r, a:b], (k[a:b] @ q_rows[r]) * scale, -np.inf)
            top = s.max()
            if top == -np.inf:            # no visible key in this block
                continue
            w = np.exp(s - top)
            mass = w.sum()
            blk_lse = top + math.log(mass)
            blk_out = (w @ v[a:b]) / mass
            merged = np.logaddexp(total, blk_lse)
            out = math.exp(total - merged) * out + math.exp(blk_lse - merged) * blk_out
            total = merged
        O[r] = out
        LSE[r] = total
    return O, LSE


# ---- visible-pair counting -------------------------------------------------

def visible_pairs_bruteforce(N: int, causal: int, win_left: int, win_right: int,
                             global_idx=(), row_block: int = 4096, block: int = 0,
                             dilation: int = 1, stride: int = 0, rand_block: int = 0,
                             rand_idx=None) -> int:
    """Count of visible (i, j) pairs of one head by evaluating the mask."""
    total = 0
    for r0 in range(0, N, row_block):
        rows = np.arange(r0, min(N, r0 + row_block))
        total += int(mask_rows(rows, N, causal, win_left, win_right, global_idx, block, dilation, stride,
                               rand_block, rand_idx).sum())
    return total


def useful_flops(B: int, H: int, d: int, pairs_per_head: int) -> int:
    """Useful FLOPs of one forward call: 2*d for the score of each visible
    pair plus 2*d for its contribution to the output (cost table of the
    week-17 notes: QK^T and weights-times-V each O(n^2 d))."""
    return 4 * d * pairs_per_head * B * H
