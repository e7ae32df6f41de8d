"""Pins of the oracle's log-spaced strided and random-block masks (CPU): the
scalar predicate against the vectorised mask, closed-form pair counts,
reductions to masks with a plain definition, and torch SDPA under a boolean
mask built here with plain loops."""
import math

import numpy as np
import pytest

import oracle
from oracle.masked_attention import visible

torch = pytest.importorskip("torch")


def _rand_lists(N, b, r, seed, extra=()):
    """Seeded key-block lists [ceil(N / b), r], with optional (qb, e, value)
    overrides (duplicates, out-of-range entries)."""
    nb = (N + b - 1) // b
    lists = np.random.default_rng(seed).integers(0, nb, size=(nb, r))
    for qb, e, val in extra:
        if qb < nb:
            lists[qb, e] = val
    return lists


def _scalar(N, m):
    gs = set(m.get("global_idx", ()))
    return np.array([[visible(i, j, N, m["causal"], m["win_left"], m["win_right"], gs,
                              stride=m.get("stride", 0), rand_block=m.get("rand_block", 0),
                              rand_idx=m.get("rand_idx")) for j in range(N)] for i in range(N)])


def _vector(N, m):
    return oracle.mask_rows(np.arange(N), N, m["causal"], m["win_left"], m["win_right"], m.get("global_idx", ()),
                            stride=m.get("stride", 0), rand_block=m.get("rand_block", 0),
                            rand_idx=m.get("rand_idx"))


def _cases(N):
    return [
        dict(causal=1, win_left=0, win_right=0, stride=1),
        dict(causal=0, win_left=0, win_right=0, stride=3),
        dict(causal=1, win_left=4, win_right=0, stride=2, global_idx=tuple(g for g in (0, 9) if g < N)),
        dict(causal=0, win_left=2, win_right=2, stride=5),
        dict(causal=0, win_left=0, win_right=0, rand_block=4, rand_idx=_rand_lists(N, 4, 2, 1)),
        dict(causal=1, win_left=3, win_right=0, rand_block=8, rand_idx=_rand_lists(N, 8, 3, 2, [(1, 0, 99), (1, 1, 0), (1, 2, 0)])),
        dict(causal=0, win_left=1, win_right=1, rand_block=5, rand_idx=_rand_lists(N, 5, 2, 3),
             global_idx=tuple(g for g in (2, 30) if g < N)),
    ]


@pytest.mark.parametrize("N", [1, 17, 40, 65])
@pytest.mark.parametrize("ci", range(7))
def test_vector_mask_matches_scalar(N, ci):
    m = _cases(N)[ci]
    assert np.array_equal(_vector(N, m), _scalar(N, m))


@pytest.mark.parametrize("N,s", [(1, 1), (50, 1), (100, 3), (257, 4), (1000, 7), (64, 64)])
def test_strided_pair_counts(N, s):
    """Window 0: row i sees itself and the rows at distance s * 2^m. Causal:
    N + sum over m of (N - s 2^m); both sides: twice that sum."""
    offs = []
    o = s
    while o < N:
        offs.append(o)
        o *= 2
    one_side = sum(N - o for o in offs)
    assert oracle.visible_pairs_bruteforce(N, 1, 0, 0, stride=s) == N + one_side
    assert oracle.visible_pairs_bruteforce(N, 0, 0, 0, stride=s) == N + 2 * one_side


def test_strided_offsets_are_doublings_not_multiples():
    """Distance 3s is not on the strided pattern; 4s is."""
    m = oracle.mask_rows(np.array([40]), 41, 1, 0, 0, stride=2)[0]
    seen = sorted(40 - j for j in np.nonzero(m)[0])
    assert seen == [0, 2, 4, 8, 16, 32]


@pytest.mark.parametrize("N,b,r", [(64, 8, 2), (100, 10, 3), (37, 4, 1)])
def test_random_pair_counts(N, b, r):
    """Window 0 and lists that never name the query's own block: each row
    sees itself plus every key of each distinct listed block (a short last
    block counts its own size); entries outside the block range are
    ignored."""
    nb = (N + b - 1) // b
    rng = np.random.default_rng(N)
    lists = np.zeros((nb, r + 1), np.int64)
    expect = N
    for qb in range(nb):
        others = [x for x in range(nb) if x != qb]
        pick = rng.choice(others, size=min(r, len(others)), replace=True)
        lists[qb, :len(pick)] = pick
        lists[qb, len(pick):] = nb + 5   # out of range: ignored
        rows = min(N, (qb + 1) * b) - qb * b
        expect += rows * sum(min(N, (x + 1) * b) - x * b for x in set(int(y) for y in pick))
    assert oracle.visible_pairs_bruteforce(N, 0, 0, 0, rand_block=b, rand_idx=lists) == expect


def test_random_every_block_is_full_attention():
    N, b = 50, 7
    nb = (N + b - 1) // b
    lists = np.tile(np.arange(nb), (nb, 1))
    assert oracle.mask_rows(np.arange(N), N, 0, 0, 0, rand_block=b, rand_idx=lists).all()
    causal = oracle.mask_rows(np.arange(N), N, 1, 0, 0, rand_block=b, rand_idx=lists)
    assert np.array_equal(causal, np.tril(np.ones((N, N), bool)))


def test_stride_beyond_sequence_is_the_window():
    N = 60
    a = oracle.mask_rows(np.arange(N), N, 1, 5, 0, stride=N)
    b = oracle.mask_rows(np.arange(N), N, 1, 5, 0)
    assert np.array_equal(a, b)


def _loop_mask(N, causal, wl, wr, G, stride, rb, lists):
    """The same visibility written out with plain loops and sets."""
    M = np.zeros((N, N), bool)
    gs = set(G)
    offs = set()
    if stride > 0:
        o = stride
        while o < N:
            offs.add(o)
            o *= 2
    for i in range(N):
        listed = set(int(x) for x in lists[i // rb]) if rb else set()
        for j in range(N):
            ok = (wl < 0 or j >= i - wl) and (wr < 0 or j <= i + wr)
            ok = ok or i in gs or j in gs or abs(i - j) in offs or (rb > 0 and j // rb in listed)
            M[i, j] = ok and (not causal or j <= i)
    return M


@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("kind", ["strided", "random"])
def test_matches_torch_sdpa_with_explicit_mask(causal, kind):
    N, d = 96, 16
    rng = np.random.default_rng(7 + causal)
    q, k, v = (rng.standard_normal((1, 2, N, d)) for _ in range(3))
    if kind == "strided":
        m = dict(causal=causal, win_left=3, win_right=3, global_idx=(5,), stride=2)
        M = _loop_mask(N, causal, 3, 3, (5,), 2, 0, None)
    else:
        lists = _rand_lists(N, 16, 2, 9)
        m = dict(causal=causal, win_left=3, win_right=3, global_idx=(5,), rand_block=16, rand_idx=lists)
        M = _loop_mask(N, causal, 3, 3, (5,), 0, 16, lists)
    O, _ = oracle.attention(q, k, v, **m)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=torch.from_numpy(M))
    assert np.max(np.abs(O - ref.numpy())) < 1e-12


# ---- planted mistakes in a copy of the mask (CPU): each must break a pin above

def _mutant_mask(kind):
    real = oracle.mask_rows

    def bad(rows, N, causal, wl, wr, G=(), block=0, dilation=1, stride=0, rand_block=0, rand_idx=None):
        if kind == "multiples" and stride > 0:   # s, 2s, 3s, ... instead of s, 2s, 4s
            base = real(rows, N, causal, wl, wr, G, block, dilation)
            i = np.asarray(rows)[:, None]
            j = np.arange(N)[None, :]
            dist = np.abs(i - j)
            extra = (dist > 0) & (dist % stride == 0)
            if causal:
                extra &= j <= i
            return base | extra
        if kind == "key_block_list" and rand_block > 0:   # list looked up by the key's block
            vis = real(rows, N, causal, wl, wr, G, block, dilation, stride)
            i = np.asarray(rows)[:, None]
            j = np.arange(N)[None, :]
            lists = np.asarray(rand_idx)
            for e in range(lists.shape[1]):
                hit = lists[j[0] // rand_block, e][None, :] == (i // rand_block)
                vis = vis | (hit & ((j <= i) if causal else True))
            return vis
        if kind == "one_sided" and stride > 0:   # strides to the left only, also without causal
            base = real(rows, N, causal, wl, wr, G, block, dilation)
            i = np.asarray(rows)[:, None]
            j = np.arange(N)[None, :]
            dist = i - j
            m = np.where((dist > 0) & (dist % stride == 0), dist // stride, 0)
            return base | ((m > 0) & ((m & (m - 1)) == 0))
        return real(rows, N, causal, wl, wr, G, block, dilation, stride, rand_block, rand_idx)
    return bad


@pytest.mark.parametrize("kind", ["multiples", "key_block_list", "one_sided"])
def test_planted_mask_mistakes_are_caught(monkeypatch, kind):
    import oracle.masked_attention as OA
    monkeypatch.setattr(OA, "mask_rows", _mutant_mask(kind))
    monkeypatch.setattr(oracle, "mask_rows", OA.mask_rows)
    caught = 0
    for fn in (lambda: test_strided_pair_counts(100, 3),
               lambda: test_strided_offsets_are_doublings_not_multiples(),
               lambda: test_random_pair_counts(100, 10, 3),
               lambda: test_matches_torch_sdpa_with_explicit_mask(0, "strided"),
               lambda: test_matches_torch_sdpa_with_explicit_mask(1, "random"),
               lambda: test_matches_torch_sdpa_with_explicit_mask(0, "random")):
        try:
            fn()
        except AssertionError:
            caught += 1
    assert caught > 0, kind
