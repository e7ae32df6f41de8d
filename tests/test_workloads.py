"""Seeded input generation (CPU only)."""
import numpy as np
import torch

from efficient_exact_attention_amd import workloads as W


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 3,
                        np.array([1.00390625, 1.01171875, -1.00390625, 0.0, -0.0,
                                  65504.0, 1e-30], np.float32)])
    ours = W.round_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_head_values_match_full_tensor():
    w = W.random_workload("t", 2, 3, 50, 16, seed=9, sigma=0.5)
    full = W.make_tensor(w, 1)
    for b in range(2):
        for h in range(3):
            got = W.head_values(w, 1, b, h)
            assert np.array_equal(W.bf16_bits_to_f32(full[b, h]), got)


def test_seeds_reproducible_and_distinct():
    w = W.WORKLOADS["f32_causal_256"]
    a = W.make_qkv(w)
    b = W.make_qkv(w)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    assert not np.array_equal(a[0], a[1])
    assert a[0].dtype == np.float32 and a[0].shape == (1, 1, 256, 64)


def test_sample_rows():
    w = W.WORKLOADS["causal_131k"]
    r = W.sample_rows(w, 256)
    assert len(r) == 256 and np.all(np.diff(r) > 0)
    for e in (0, 1, 127, 128, 255, 256, w.N // 2, w.N - 2, w.N - 1):
        assert e in r


def test_workload_table():
    band = W.WORKLOADS["band256_globals_16k"]
    assert band.global_idx == (0, 1, 2048, 4096, 6144, 8192, 10240, 12288, 14336)
    assert W.WORKLOADS["swa4096_32k"].win_left == 4095 and W.WORKLOADS["swa4096_32k"].win_right == 0
