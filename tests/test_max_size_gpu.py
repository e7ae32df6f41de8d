"""The largest head the C ABI accepts (N * d * 2 bytes just under 2 GiB:
N = 8,388,607 at d = 128, bf16), forward and backward under a causal sliding
window, against the oracle on slices of the sequence. Inputs are drawn on
the device with a seeded torch generator (four 2 GiB tensors would take a
long time to draw and upload from the host); the oracle reads the same
values back."""
import numpy as np
import pytest

import oracle
from gpu_common import errors, host_f64, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

N_MAX = 8388607     # (N_MAX * 128 * 2) < 2^31 <= ((N_MAX + 1) * 128 * 2)
D = 128
WIN = 255


@pytest.fixture(scope="module")
def tensors():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import efficient_exact_attention_amd as ea
    ea.lib()
    g = torch.Generator(device="cuda")
    g.manual_seed(2024)
    say(f"  drawing 4 x [1, 1, {N_MAX}, {D}] bf16 on the device")
    q, k, v, do = (torch.randn((1, 1, N_MAX, D), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
                   for _ in range(4))
    return q, k, v, do


SLICES = [0, 1234567, 4194000, N_MAX - 1000]


def test_forward_at_max_length(tensors):
    import efficient_exact_attention_amd as ea
    q, k, v, _ = tensors
    say(f"  launch fwd: B=1 H=1 N={N_MAX} d={D} causal win_left={WIN}")
    out, lse = ea.fwd(q, k, v, causal=True, win_left=WIN)
    torch.cuda.synchronize()
    for a in SLICES:
        lo = max(0, a - WIN)
        b = min(N_MAX, a + 1000)
        rows = np.arange(a - lo, b - lo)
        sl = lambda t: host_f64(t[:, :, lo:b])
        ref_o, ref_l = oracle.attention(sl(q), sl(k), sl(v), causal=1, win_left=WIN, win_right=0, rows=rows)
        go, gl = host_f64(out[:, :, a:b]), host_f64(lse[:, :, a:b])
        e = errors(go, gl, ref_o, ref_l, bf16_out=True)
        say(f"    rows {a}..{b - 1}: raw max-abs {e[3]:.3e} rel-L2 {e[1]:.3e} lse {e[2]:.3e}")
        assert e[0] <= 1e-2 and e[1] <= 5e-3 and e[2] <= 1e-3, e


def test_backward_at_max_length(tensors):
    """Gradients of interior positions of each slice depend only on the
    slice (every row that sees a key lies within WIN after it)."""
    import efficient_exact_attention_amd as ea
    q, k, v, do = tensors
    out, lse = ea.fwd(q, k, v, causal=True, win_left=WIN)
    say(f"  launch bwd: B=1 H=1 N={N_MAX} d={D} causal win_left={WIN}")
    dq, dk, dv = ea.bwd(q, k, v, out, do, lse, causal=True, win_left=WIN)
    torch.cuda.synchronize()
    for a in SLICES:
        lo = max(0, a - WIN)
        b = min(N_MAX, a + 1200)
        sl = lambda t: host_f64(t[:, :, lo:b])
        rq, rk, rv = oracle.attention_backward(sl(q), sl(k), sl(v), sl(do), causal=1, win_left=WIN, win_right=-1)
        # rows of the slice see their whole window only from lo + WIN on (or
        # from 0); a key's gradient needs every row within WIN after it to be
        # whole: keys from lo + WIN (or 0) up to b - 1 - WIN (or the end)
        r0 = WIN if lo > 0 else 0
        k1 = (b - lo) - WIN if b < N_MAX else b - lo
        for name, got, ref, s0, s1 in (("dq", dq, rq, r0, b - lo), ("dk", dk, rk, r0, k1), ("dv", dv, rv, r0, k1)):
            g = host_f64(got[:, :, lo + s0:lo + s1])
            r = ref[:, :, s0:s1]
            rel = float(np.linalg.norm(g - r) / np.linalg.norm(r))
            say(f"    {name} positions {lo + s0}..{lo + s1 - 1}: rel-L2 {rel:.3e}")
            assert rel <= 1e-2, (name, rel)
