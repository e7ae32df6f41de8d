"""Every kernel fits its register budget: no VGPR spills to scratch memory.

A spill inside a hot loop turns each iteration's register traffic into
memory traffic; the band kernel sits a few registers under its 256-register
budget at 512 threads, so a small change to shared code can push it over
(its throughput then drops about threefold while every result stays right).
This check compiles the device code to assembly on the CPU and reads the
code-object metadata, so it catches that before any GPU run."""
import re
import shutil

import pytest

from efficient_exact_attention_amd import build

pytestmark = pytest.mark.skipif(shutil.which(build.HIPCC) is None and not __import__("os").path.exists(build.HIPCC),
                                reason="hipcc not available")


@pytest.fixture(scope="module")
def resources():
    return build.kernel_resources()


def test_kernels_found(resources):
    names = " ".join(resources)
    for k in ("fwd_band_bf16", "fwd_kernel", "merge_kernel", "bwd_dkdv", "bwd_dq", "bwd_delta",
              "decode_kernel", "decode_merge"):
        assert k in names, k


def test_no_vector_register_spills(resources):
    bad = {k: v for k, v in resources.items() if v["vgpr_spill"] > 0 or v["scratch_bytes"] > 0}
    assert not bad, bad


def _band_flags(name):
    """(DIL, BLK, XT, NAR, FUS) of a mangled fwd_band_bf16<D, DIL, BLK, XT, NAR, FUS> name."""
    args = name.split("fwd_band_bf16I", 1)[1]
    return tuple(f == "1" for f in re.findall(r"Lb([01])E", args)[:5])


def test_band_kernel_fits_two_waves_per_simd(resources):
    """The band instances that run two waves per SIMD (plain and dilated at
    512 threads; narrow, with and without the fused global rows, and the
    strided/random-block instances, with and without the fused global rows,
    at 256 threads with two workgroups per CU)
    keep within 256 registers."""
    seen = 0
    for k, v in resources.items():
        if "fwd_band_bf16" not in k:
            continue
        dil, blk, xt, nar, fus = _band_flags(k)
        if not blk:
            seen += 1
            assert v["vgpr"] + v["agpr"] <= 256, (k, v)
    assert seen == 12   # d = 64, 128 x (plain, dilated, narrow, narrow and extra tiles with and without fused global rows)


def test_narrow_d64_fits_three_workgroups_per_cu(resources):
    """The d = 64 narrow band instances (with and without the fused global
    rows) run three four-wave workgroups per CU, three waves per SIMD: at
    most 168 registers each (512 / 3, in granules of 8)."""
    seen = 0
    for k, v in resources.items():
        if "fwd_band_bf16ILi64E" not in k:
            continue
        dil, blk, xt, nar, fus = _band_flags(k)
        if nar:
            seen += 1
            assert v["vgpr"] + v["agpr"] <= 168, (k, v)
    assert seen == 2


def test_two_wave_backward_instances_fit(resources):
    """Backward instances that run two waves per SIMD keep within 256
    registers: at d = 64 every dQ instance and the dK/dV instances other than
    the one with gathered global rows (mode 1, with or without extra tiles);
    at d = 128 the eight-wave dQ band instances (mode 0, plain and dilated)."""
    seen = 0
    for k, v in resources.items():
        m = re.search(r"bwd_(dq|dkdv)ILi(64|128)ELb([01])ELi([012])ELb([01])E", k)
        if not m:
            continue
        kind, d, mode = m.group(1), int(m.group(2)), int(m.group(4))
        two = (kind == "dq" or mode != 1) if d == 64 else (kind == "dq" and mode == 0)
        if two:
            seen += 1
            assert v["vgpr"] + v["agpr"] <= 256, (k, v)
    assert seen == 10   # d=64 dq x5, d=64 dkdv x3, d=128 dq band x2
