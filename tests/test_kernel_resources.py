"""Every kernel fits its register budget: no VGPR spills to scratch memory.

A spill inside a hot loop turns each iteration's register traffic into
memory traffic; the band kernel sits a few registers under its 256-register
budget at 512 threads, so a small change to shared code can push it over
(its throughput then drops about threefold while every result stays right).
This check compiles the device code to assembly on the CPU and reads the
code-object metadata, so it catches that before any GPU run."""
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


def test_band_kernel_fits_two_waves_per_simd(resources):
    """The 512-thread band instances (plain and dilated) keep within 256
    registers, the budget of two waves per SIMD."""
    for k, v in resources.items():
        if "fwd_band_bf16" in k and "Lb0ELb0EEE" in k:   # BLK = XT = false: the 512-thread instances
            assert v["vgpr"] + v["agpr"] <= 256, (k, v)
