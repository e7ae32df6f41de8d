"""Seeded synthetic workloads shared by the tests, the bench and the oracle checks.

This module only draws and rounds numbers; it holds none of the attention
arithmetic. Both the HIP path and the CPU oracle take their inputs from here.

Recipe (stated once, used everywhere):
  * Each of Q, K, V is drawn head by head. Stream ``t*B*H + b*H + h`` of
    ``numpy.random.SeedSequence(seed).spawn(3*B*H)`` (t = 0, 1, 2 for Q, K, V)
    feeds ``default_rng(...).standard_normal((N, d), float32)``, multiplied by
    ``sigma``. Any one head can therefore be regenerated on its own.
  * For bf16 workloads every value is rounded once to bf16 with
    round-to-nearest-even; the same 16-bit patterns go to the GPU and, upcast
    exactly, to the oracle.

The shapes and mask arguments are the five workloads of the exact-attention
pages (causal, Mistral-style sliding window, long-context causal,
Longformer/BigBird-style local+global) plus the causal N=32768 d=128 shape the
throughput target is quoted on.

Decoding workloads (``DecodeWorkload``) draw the Nq new queries [B][H][Nq][d]
and the K and V caches [B][H_kv][S][d] with the same per-head recipe (Q from
one seed, the caches from seed + 1); cache slots that hold no position of a
sequence (slot >= min(S, L_b)) are set to bf16 NaN, so a kernel that reads
them shows it.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "bf16" or "f32"
    sigma: float
    causal: int
    win_left: int
    win_right: int
    global_idx: tuple = field(default_factory=tuple)
    seed: int = 0
    desc: str = ""

    @property
    def n_global(self) -> int:
        return len(self.global_idx)

    def mask_args(self) -> dict:
        return dict(causal=self.causal, win_left=self.win_left,
                    win_right=self.win_right, global_idx=tuple(self.global_idx))

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


def every_2048th(N: int) -> tuple:
    """Global tokens {0, 1} plus every multiple of 2048 below N (0 listed once)."""
    return tuple(sorted({0, 1} | set(range(0, N, 2048))))


WORKLOADS = {
    "f32_causal_256": Workload("f32_causal_256", 1, 1, 256, 64, "f32", 1.0, 1, -1, -1, (), 101,
                   "single-head causal, fp32 inputs"),
    "causal_4k_b4": Workload("causal_4k_b4", 4, 32, 4096, 128, "bf16", 1.0, 1, -1, -1, (), 102,
                   "full causal"),
    "swa4096_32k": Workload("swa4096_32k", 1, 32, 32768, 128, "bf16", 1.0, 1, 4095, 0, (), 103,
                   "sliding-window causal, w=4096 (row i sees i-4095..i)"),
    "causal_131k": Workload("causal_131k", 1, 8, 131072, 128, "bf16", 0.5, 1, -1, -1, (), 104,
                   "long-context causal, sigma 0.5"),
    "band256_globals_16k": Workload("band256_globals_16k", 2, 12, 16384, 64, "bf16", 1.0, 0, 256, 256,
                   every_2048th(16384), 105,
                   "non-causal band +-256 plus 9 global tokens"),
    "causal_32k": Workload("causal_32k", 1, 32, 32768, 128, "bf16", 1.0, 1, -1, -1, (), 106,
                    "full causal"),
}


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _streams(seed: int, B: int, H: int):
    return np.random.SeedSequence(seed).spawn(3 * B * H)


def head_values(w: Workload, t: int, b: int, h: int, streams=None) -> np.ndarray:
    """One head of tensor t (0=Q, 1=K, 2=V) as float32 values exactly as the
    GPU sees them (already rounded to bf16 for bf16 workloads)."""
    ss = (streams or _streams(w.seed, w.B, w.H))[t * w.B * w.H + b * w.H + h]
    x = np.random.default_rng(ss).standard_normal((w.N, w.d), dtype=np.float32)
    if w.sigma != 1.0:
        x *= np.float32(w.sigma)
    if w.dtype == "bf16":
        x = bf16_bits_to_f32(round_to_bf16_bits(x))
    return x


def make_tensor(w: Workload, t: int, threads: int | None = None) -> np.ndarray:
    """Full [B][H][N][d] tensor t. bf16 workloads return uint16 bit patterns,
    f32 workloads return float32."""
    streams = _streams(w.seed, w.B, w.H)
    dt = np.uint16 if w.dtype == "bf16" else np.float32
    out = np.empty((w.B, w.H, w.N, w.d), dtype=dt)

    def fill(bh):
        b, h = divmod(bh, w.H)
        x = np.random.default_rng(streams[t * w.B * w.H + bh]).standard_normal(
            (w.N, w.d), dtype=np.float32)
        if w.sigma != 1.0:
            x *= np.float32(w.sigma)
        out[b, h] = round_to_bf16_bits(x) if w.dtype == "bf16" else x

    n = threads or min(16, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(n) as ex:
        list(ex.map(fill, range(w.B * w.H)))
    return out


def make_qkv(w: Workload):
    return tuple(make_tensor(w, t) for t in range(3))


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact upcast of stored inputs (bf16 bits or float32) to float64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return x.astype(np.float64)


def sample_rows(w: Workload, per_head: int, bm: int = 128, seed_offset: int = 7) -> np.ndarray:
    """Seeded query-row subset used where the oracle cannot cover every row:
    fixed edge rows (tile boundaries, the middle, the end) plus seeded random
    rows, sorted and unique."""
    N = w.N
    edge = {0, 1, bm - 1, bm, 2 * bm - 1, 2 * bm, N // 2, N - 2, N - 1}
    edge |= set(int(g) for g in w.global_idx)
    edge = {r for r in edge if 0 <= r < N}
    rng = np.random.default_rng(w.seed + seed_offset)
    extra = max(0, per_head - len(edge))
    rnd = rng.choice(N, size=min(extra, N), replace=False) if extra else []
    return np.array(sorted(edge | set(int(r) for r in rnd)), dtype=np.int64)


def random_workload(name: str, B: int, H: int, N: int, d: int, *, dtype="bf16",
                    sigma=1.0, causal=1, win_left=-1, win_right=-1,
                    global_idx=(), seed=0) -> Workload:
    return Workload(name, B, H, N, d, dtype, sigma, causal, win_left, win_right,
                    tuple(global_idx), seed, "ad-hoc")


@dataclass(frozen=True)
class DecodeWorkload:
    """One decoding step: Nq new tokens per sequence against a cache of S
    slots per K/V head; seq_len[b] counts the sequence's tokens, new ones
    included."""
    name: str
    B: int
    H: int
    H_kv: int
    Nq: int
    S: int
    d: int
    win_left: int
    rolling: int
    seq_len: tuple
    seed: int = 0
    desc: str = ""

    def cache_bytes(self) -> int:
        """Bytes of K and V cache slots that hold a position of some sequence."""
        used = sum(min(self.S, L) for L in self.seq_len)
        return 2 * used * self.H_kv * self.d * 2


DECODE_WORKLOADS = {
    # 64 query heads over 8 K/V heads (the grouped-query shape of the GQA
    # passage), one new token, a full 32768-token contiguous cache
    "dec_full": DecodeWorkload("dec_full", 8, 64, 8, 1, 32768, 128, -1, 0, (32768,) * 8, 201,
                               "GQA 64/8, contiguous cache, L=32768"),
    # the same heads over a rolling sliding-window cache of 4096 positions at
    # L=32768 (each cache 8x smaller than the full one)
    "dec_swa": DecodeWorkload("dec_swa", 64, 64, 8, 1, 4096, 128, 4095, 1, (32768,) * 64, 202,
                              "GQA 64/8, rolling cache W=4096, L=32768"),
}

_BF16_NAN = np.uint16(0x7FC0)


def make_decode(w: DecodeWorkload, b_list=None):
    """(q, k_cache, v_cache, seq_len) host arrays: bf16 bit patterns and int32
    lengths. b_list restricts the draw to those batch entries (the others
    stay zero), for checks that read a few entries of a large workload."""
    sq = np.random.SeedSequence(w.seed).spawn(w.B * w.H)
    sk = np.random.SeedSequence(w.seed + 1).spawn(2 * w.B * w.H_kv)
    q = np.zeros((w.B, w.H, w.Nq, w.d), np.uint16)
    kc = np.zeros((w.B, w.H_kv, w.S, w.d), np.uint16)
    vc = np.zeros((w.B, w.H_kv, w.S, w.d), np.uint16)
    bs = range(w.B) if b_list is None else b_list

    def fill(job):
        t, b, h = job
        if t == 0:
            x = np.random.default_rng(sq[b * w.H + h]).standard_normal((w.Nq, w.d), dtype=np.float32)
            q[b, h] = round_to_bf16_bits(x)
            return
        dst = kc if t == 1 else vc
        x = np.random.default_rng(sk[(t - 1) * w.B * w.H_kv + b * w.H_kv + h]).standard_normal(
            (w.S, w.d), dtype=np.float32)
        dst[b, h] = round_to_bf16_bits(x)
        dst[b, h, min(w.S, w.seq_len[b]):] = _BF16_NAN

    jobs = [(0, b, h) for b in bs for h in range(w.H)] + \
        [(t, b, h) for t in (1, 2) for b in bs for h in range(w.H_kv)]
    with ThreadPoolExecutor(min(16, len(os.sched_getaffinity(0)))) as ex:
        list(ex.map(fill, jobs))
    return q, kc, vc, np.asarray(w.seq_len, np.int32)


# Workloads of the strided and random-block rules (forward only).
PATTERN_WORKLOADS = {
    # BigBird-style: window of one 64-token block each side, the first block
    # as global tokens, 3 random key blocks of 64 per query block
    "bigbird": dict(workload=Workload("bigbird", 1, 16, 16384, 64, "bf16", 1.0, 0, 64, 64, tuple(range(64)), 301,
                                      "BigBird-style: window +-64, 64 global tokens, 3 random blocks of 64"),
                    rand_block=64, n_rand=3, stride=0),
    # strided rule with a local window: row i sees i-255..i and i - 256 * 2^m
    "strided": dict(workload=Workload("strided", 1, 16, 16384, 128, "bf16", 1.0, 1, 255, 0, (), 302,
                                      "causal window 256 + positions at distance 256, 512, 1024, ..."),
                    rand_block=0, n_rand=0, stride=256),
}


def random_block_lists(N: int, b: int, r: int, seed: int) -> np.ndarray:
    """Seeded key-block lists [ceil(N / b), r] (int32): uniform draws over the
    blocks, repeats allowed (they count once)."""
    nb = (N + b - 1) // b
    return np.random.default_rng(seed).integers(0, nb, size=(nb, r)).astype(np.int32)
