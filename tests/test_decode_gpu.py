"""GPU parity of decoding with a key/value cache (attn_decode): the newest
Nq queries of each sequence against contiguous and rolling caches, against
the CPU oracle on the same seeded inputs. Cache slots that hold no position
of a sequence are NaN, so a kernel that reads them fails the check."""
import numpy as np
import pytest

import oracle
from efficient_exact_attention_amd import workloads as W
from gpu_common import TOL_LSE, TOL_MAXABS, TOL_RELL2, errors, host_f64, say, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import efficient_exact_attention_amd as ea
    ea.lib()


def _device(q, kc, vc, seq):
    return (to_device(q, "bf16"), to_device(kc, "bf16"), to_device(vc, "bf16"),
            torch.from_numpy(seq).cuda())


def _check(w, b_list=None, out=None, lse=None, scale=None):
    import efficient_exact_attention_amd as ea
    q, kc, vc, seq = W.make_decode(w, b_list)
    say(f"  launch decode {w.name}: B={w.B} H={w.H} H_kv={w.H_kv} Nq={w.Nq} S={w.S} d={w.d} "
        f"win={w.win_left} rolling={w.rolling} L={list(w.seq_len)[:6]} seed={w.seed}")
    dq, dk, dv, ds = _device(q, kc, vc, seq)
    o, l = ea.decode(dq, dk, dv, ds, win_left=w.win_left, rolling=bool(w.rolling), out=out, lse=lse,
                     scale=scale)
    torch.cuda.synchronize()
    bs = list(range(w.B)) if b_list is None else list(b_list)
    f = lambda x: W.as_f64(x, "bf16")
    ref_o, ref_l = [], []
    for b in bs:
        ro, rl = oracle.decode(f(q[b:b + 1]), f(kc[b:b + 1]), f(vc[b:b + 1]), seq[b:b + 1],
                               win_left=w.win_left, rolling=bool(w.rolling), scale=scale)
        ref_o.append(ro[0])
        ref_l.append(rl[0])
    ref_o, ref_l = np.stack(ref_o), np.stack(ref_l)
    go, gl = host_f64(o[bs]), host_f64(l[bs])
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl)), "non-finite output"
    e = errors(go, gl, ref_o, ref_l, bf16_out=True)
    say(f"    raw max-abs {e[3]:.3e} (beyond bf16 rounding {e[0]:.3e}) "
        f"rel-L2 {e[1]:.3e} lse {e[2]:.3e}")
    assert e[0] <= TOL_MAXABS and e[1] <= TOL_RELL2 and e[2] <= TOL_LSE, e
    return o, l


def dw(name, B, H, H_kv, Nq, S, d, win, rolling, seq, seed=7):
    return W.DecodeWorkload(name, B, H, H_kv, Nq, S, d, win, rolling, tuple(seq), seed)


CASES = [
    # contiguous caches: ragged lengths (one slot, a tile and a bit, full)
    dw("mha_nq1", 3, 4, 4, 1, 1000, 128, -1, 0, (1, 65, 1000)),
    dw("gqa_nq1", 3, 8, 2, 1, 1000, 128, -1, 0, (517, 64, 999)),
    dw("gqa_win", 3, 8, 2, 1, 1000, 128, 100, 0, (1000, 101, 7)),
    dw("gqa_nq4_d64", 3, 16, 4, 4, 700, 64, -1, 0, (4, 300, 700)),
    dw("gqa_nq4_win_d64", 2, 16, 4, 4, 700, 64, 63, 0, (700, 130)),
    dw("mqa_nq2", 2, 64, 1, 2, 513, 128, -1, 0, (513, 200)),        # 128 rows: two row groups
    dw("mqa_nq3_d64", 1, 40, 1, 3, 300, 64, 17, 0, (250,)),          # 120 rows, ragged group
    # rolling caches of S slots: L below, at and far beyond S
    dw("roll_nq1", 4, 8, 2, 1, 256, 128, 255, 1, (10, 256, 257, 3000)),
    dw("roll_nq3", 3, 8, 8, 3, 256, 128, 200, 1, (3, 700, 259)),
    dw("roll_d64_short_win", 2, 16, 4, 2, 192, 64, 5, 1, (1000, 190)),
    dw("roll_ragged_S", 2, 8, 2, 1, 100, 128, 99, 1, (100, 12345)),
]


@pytest.mark.parametrize("w", CASES, ids=[c.name for c in CASES])
def test_decode_parity(w):
    _check(w)


def test_decode_custom_scale():
    _check(dw("scale", 2, 8, 2, 1, 300, 128, -1, 0, (300, 77)), scale=0.3)


def test_decode_matches_forward_last_rows():
    """A contiguous decode equals the last rows of the causal forward over
    the whole sequence (same kernels' rounding aside): the HIP forward is
    itself pinned to the oracle, so this checks the two paths agree."""
    import efficient_exact_attention_amd as ea
    w = dw("vs_fwd", 1, 8, 2, 1, 2048, 128, 300, 0, (2048,))
    q1, kc, vc, seq = W.make_decode(w)
    qf = torch.randn(1, 8, 2048, 128, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    qf[:, :, -1:] = torch.from_numpy(q1.view(np.int16)).view(torch.bfloat16)
    dq, dk, dv, ds = _device(q1, kc, vc, seq)
    o_dec, l_dec = ea.decode(dq, dk, dv, ds, win_left=300)
    o_f, l_f = ea.fwd(qf.cuda(), dk, dv, causal=True, win_left=300, win_right=0)
    torch.cuda.synchronize()
    d = (o_dec.float() - o_f[:, :, -1:].float()).abs().max().item()
    say(f"    decode vs forward last row: max-abs {d:.3e}")
    assert d <= 2e-2
    assert (l_dec - l_f[:, :, -1:]).abs().max().item() <= 1e-3


@pytest.mark.parametrize("name", ["dec_full", "dec_swa"])
def test_decode_full_size_sampled(name):
    """The benchmarked decode workloads at full size; the oracle checks two
    sampled sequences (first and last) in full."""
    w = W.DECODE_WORKLOADS[name]
    _check(w, b_list=[0, w.B - 1])


def test_decode_workspace_argument():
    """A caller-supplied workspace gives the same result as the library's."""
    import efficient_exact_attention_amd as ea
    w = dw("ws", 2, 8, 2, 1, 1000, 128, -1, 0, (1000, 333))
    q, kc, vc, seq = W.make_decode(w)
    dq, dk, dv, ds = _device(q, kc, vc, seq)
    o1, l1 = ea.decode(dq, dk, dv, ds)
    nbytes = ea.attn_decode_workspace_bytes(w.B, w.H, w.H_kv, w.Nq, w.S, w.d)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    o2, l2 = ea.decode(dq, dk, dv, ds, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
