"""The LDS tile layouts of the bf16 path, replayed on the CPU.

`lds_layout_check.cpp` takes the per-lane offsets that the kernels compute
(`Bf16Path::init_lane` in attn_tiles.h, host-callable), places one tile in a
simulated LDS image the way the tile copies do, and replays every operand
read: the 16-byte row reads (K operands) and the 8-byte transpose reads (V
operands, and in the backward the transposed Q, dO and K operands). Each read
must find the element it stands for, and the lanes of one hardware pass must
hit distinct banks (16 lanes of 16-byte reads on 16 distinct 16-byte slots of
the 256-byte bank window; 32 lanes of 8-byte reads on 32 distinct 8-byte
slots). Checked for the forward's two layouts (K swizzle for row reads, V
swizzle for transpose reads) and for the unified layout the backward uses,
where one copy serves both kinds of read, at d = 64 and d = 128."""
import os
import shutil
import subprocess

import pytest

from efficient_exact_attention_amd import build

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

pytestmark = pytest.mark.skipif(shutil.which(build.HIPCC) is None and not os.path.exists(build.HIPCC),
                                reason="hipcc not available")


def test_tile_layouts_read_right_elements_without_bank_conflicts(tmp_path):
    exe = tmp_path / "lds_layout_check"
    subprocess.run([build.HIPCC, "-x", "hip", "--cuda-host-only", "-std=c++17", "-O1",
                    "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "efficient_exact_attention_amd", "csrc"),
                    os.path.join(HERE, "lds_layout_check.cpp"), "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("ok: 0 failed checks")
