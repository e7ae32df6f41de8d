"""Python binding of the gfx950 exact-attention library (include/attn.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libattn.so``. PyTorch supplies device memory and the stream.
If the library has not been built, every entry point raises.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["AttnError", "attn_fwd", "attn_fwd_ex", "attn_fwd_noalloc", "ATTN_NOALLOC_SCRATCH_BYTES", "attn_fwd_gqa", "attn_fwd_masked", "attn_bwd", "attn_bwd_masked",
           "attn_bwd_workspace_bytes", "attn_plan_stats_masked", "bwd", "attn_decode",
           "attn_decode_workspace_bytes", "decode", "attn_workspace_bytes", "attn_plan_stats",
           "attn_tile_shape", "attn_last_error", "attn_version", "fwd", "library_path", "open_library",
           "DEBUG_SYNC_LIB_PATH",
           "ATTN_OK", "ATTN_ERR_INVALID_ARG", "ATTN_ERR_UNSUPPORTED", "ATTN_ERR_DEVICE",
           "ATTN_BF16", "ATTN_F32"]

ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_DEVICE = 0, 1, 2, 3
ATTN_BF16, ATTN_F32 = 0, 1
ATTN_NOALLOC_SCRATCH_BYTES = 16 << 20   # include/attn.h

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libattn.so")
# The same sources built with -DATTN_DEBUG_SYNC (copies and compute never
# overlap); only the tests load it, to compare with libattn.so bit for bit.
DEBUG_SYNC_LIB_PATH = os.path.join(_HERE, "libattn_debugsync.so")
_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"attn status {status}: {message}")
        self.status = status
        self.message = message


class _Opts(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("scale", ctypes.c_float), ("stream", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class _Mask(ctypes.Structure):
    _fields_ = [("causal", ctypes.c_int), ("win_left", ctypes.c_int), ("win_right", ctypes.c_int),
                ("block", ctypes.c_int), ("dilation", ctypes.c_int),
                ("global_idx", ctypes.POINTER(ctypes.c_int)), ("n_global", ctypes.c_int),
                ("stride", ctypes.c_int), ("rand_block", ctypes.c_int), ("n_rand", ctypes.c_int),
                ("rand_idx", ctypes.c_void_p)]


def _mask(causal, win_left, win_right, block, dilation, global_idx, stride=0, rand_block=0, n_rand=0,
          rand_idx=None):
    """rand_idx: device address (int) of the int32 key-block lists, or None."""
    g, ng = _gidx(global_idx)
    m = _Mask(int(bool(causal)), int(win_left), int(win_right), int(block), int(dilation),
              ctypes.cast(g, ctypes.POINTER(ctypes.c_int)) if g is not None else None, ng,
              int(stride), int(rand_block), int(n_rand), rand_idx)
    m._keep = g   # the index array must outlive the call
    return m


def library_path() -> str:
    return _LIB_PATH


def lib():
    """Load libattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = open_library(_LIB_PATH)
    return _lib


def open_library(path):
    """Load a build of the library at `path` with the argument types of
    include/attn.h (raises if the file is missing). lib() uses it for the
    shipped libattn.so; the debug-sync build opens through it too."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m efficient_exact_attention_amd.build`")
    L = ctypes.CDLL(path)
    vp, ci = ctypes.c_void_p, ctypes.c_int
    fwd_args = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, ctypes.POINTER(ci), ci]
    L.attn_fwd.argtypes = fwd_args
    L.attn_fwd.restype = ci
    L.attn_fwd_ex.argtypes = fwd_args + [ctypes.POINTER(_Opts)]
    L.attn_fwd_ex.restype = ci
    L.attn_fwd_noalloc.argtypes = fwd_args + [ctypes.POINTER(_Opts)]
    L.attn_fwd_noalloc.restype = ci
    L.attn_fwd_gqa.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, ci, ctypes.POINTER(ci), ci,
                               ctypes.POINTER(_Opts)]
    L.attn_fwd_gqa.restype = ci
    L.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, ci,
                           ctypes.POINTER(ci), ci, ctypes.POINTER(_Opts)]
    L.attn_bwd.restype = ci
    L.attn_fwd_masked.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ctypes.POINTER(_Mask),
                                  ctypes.POINTER(_Opts)]
    L.attn_fwd_masked.restype = ci
    L.attn_bwd_masked.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ctypes.POINTER(_Mask),
                                  ctypes.POINTER(_Opts)]
    L.attn_bwd_masked.restype = ci
    L.attn_decode.argtypes = [vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, ci, ctypes.POINTER(_Opts)]
    L.attn_decode.restype = ci
    L.attn_decode_workspace_bytes.argtypes = [ci, ci, ci, ci, ci, ci, ci, ci]
    L.attn_decode_workspace_bytes.restype = ctypes.c_size_t
    L.attn_bwd_workspace_bytes.argtypes = [ci, ci, ci, ci, ci, ci]
    L.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.attn_workspace_bytes.argtypes = [ci, ci, ci, ci, ci]
    L.attn_workspace_bytes.restype = ctypes.c_size_t
    ll = ctypes.POINTER(ctypes.c_longlong)
    L.attn_plan_stats_masked.argtypes = [ci, ctypes.POINTER(_Mask), ci, ci, ll, ll, ll]
    L.attn_plan_stats_masked.restype = ci
    L.attn_plan_stats.argtypes = [ci, ci, ci, ci, ctypes.POINTER(ci), ci, ci, ci, ll, ll, ll]
    L.attn_plan_stats.restype = ci
    L.attn_tile_shape.argtypes = [ci, ci, ctypes.POINTER(ci), ctypes.POINTER(ci)]
    L.attn_tile_shape.restype = ci
    L.attn_last_error.argtypes = []
    L.attn_last_error.restype = ctypes.c_char_p
    L.attn_version.argtypes = []
    L.attn_version.restype = ctypes.c_char_p
    return L


def attn_last_error() -> str:
    return lib().attn_last_error().decode()


def attn_version() -> str:
    return lib().attn_version().decode()


def _check(status: int):
    if status != ATTN_OK:
        raise AttnError(status, attn_last_error())


def _gidx(global_idx):
    if global_idx is None or len(global_idx) == 0:
        return None, 0
    arr = (ctypes.c_int * len(global_idx))(*[int(g) for g in global_idx])
    return arr, len(global_idx)


def attn_fwd(q, k, v, out, lse, B, H, N, d, causal, win_left, win_right, global_idx=None):
    """Raw entry point: q, k, v, out, lse are integer device addresses."""
    g, ng = _gidx(global_idx)
    _check(lib().attn_fwd(q, k, v, out, lse, B, H, N, d, causal, win_left, win_right, g, ng))


def attn_fwd_ex(q, k, v, out, lse, B, H, N, d, causal, win_left, win_right, global_idx=None,
                *, dtype=ATTN_BF16, scale=0.0, stream=None, workspace=None, workspace_bytes=0):
    """Raw entry point with options: pointers and stream are integers."""
    g, ng = _gidx(global_idx)
    opts = _Opts(dtype, float(scale), stream, workspace, workspace_bytes)
    _check(lib().attn_fwd_ex(q, k, v, out, lse, B, H, N, d, causal, win_left, win_right, g, ng,
                             ctypes.byref(opts)))


def attn_fwd_noalloc(q, k, v, out, lse, B, H, N, d, causal, win_left, win_right, global_idx=None,
                     *, dtype=ATTN_BF16, scale=0.0, stream=None):
    """Raw allocation-free entry point (no workspace): pointers and stream are integers."""
    g, ng = _gidx(global_idx)
    opts = _Opts(dtype, float(scale), stream, None, 0)
    _check(lib().attn_fwd_noalloc(q, k, v, out, lse, B, H, N, d, causal, win_left, win_right, g, ng,
                                  ctypes.byref(opts)))


def attn_fwd_gqa(q, k, v, out, lse, B, H, H_kv, N, d, causal, win_left, win_right, global_idx=None,
                 *, dtype=ATTN_BF16, scale=0.0, stream=None, workspace=None, workspace_bytes=0):
    """Raw grouped-query entry point: k and v hold H_kv heads per batch entry."""
    g, ng = _gidx(global_idx)
    opts = _Opts(dtype, float(scale), stream, workspace, workspace_bytes)
    _check(lib().attn_fwd_gqa(q, k, v, out, lse, B, H, H_kv, N, d, causal, win_left, win_right, g, ng,
                              ctypes.byref(opts)))


def attn_bwd(q, k, v, out, dout, lse, dq, dk, dv, B, H, H_kv, N, d, causal, win_left, win_right,
             global_idx=None, *, dtype=ATTN_BF16, scale=0.0, stream=None, workspace=None, workspace_bytes=0):
    """Raw backward entry point: every tensor is an integer device address."""
    g, ng = _gidx(global_idx)
    opts = _Opts(dtype, float(scale), stream, workspace, workspace_bytes)
    _check(lib().attn_bwd(q, k, v, out, dout, lse, dq, dk, dv, B, H, H_kv, N, d, causal, win_left, win_right,
                          g, ng, ctypes.byref(opts)))


def attn_fwd_masked(q, k, v, out, lse, B, H, H_kv, N, d, *, causal=0, win_left=-1, win_right=-1, block=0,
                    dilation=1, global_idx=None, dtype=ATTN_BF16, scale=0.0, stream=None, workspace=None,
                    workspace_bytes=0, stride=0, rand_block=0, n_rand=0, rand_idx=None):
    """Raw forward entry point with an attn_mask descriptor (rand_idx: device address)."""
    m = _mask(causal, win_left, win_right, block, dilation, global_idx, stride, rand_block, n_rand, rand_idx)
    opts = _Opts(dtype, float(scale), stream, workspace, workspace_bytes)
    _check(lib().attn_fwd_masked(q, k, v, out, lse, B, H, H_kv, N, d, ctypes.byref(m), ctypes.byref(opts)))


def attn_bwd_masked(q, k, v, out, dout, lse, dq, dk, dv, B, H, H_kv, N, d, *, causal=0, win_left=-1,
                    win_right=-1, block=0, dilation=1, global_idx=None, dtype=ATTN_BF16, scale=0.0, stream=None,
                    workspace=None, workspace_bytes=0, stride=0, rand_block=0, n_rand=0, rand_idx=None):
    """Raw backward entry point with an attn_mask descriptor."""
    m = _mask(causal, win_left, win_right, block, dilation, global_idx, stride, rand_block, n_rand, rand_idx)
    opts = _Opts(dtype, float(scale), stream, workspace, workspace_bytes)
    _check(lib().attn_bwd_masked(q, k, v, out, dout, lse, dq, dk, dv, B, H, H_kv, N, d, ctypes.byref(m),
                                 ctypes.byref(opts)))


def attn_plan_stats_masked(N, bm, bn, *, causal=0, win_left=-1, win_right=-1, block=0, dilation=1,
                           global_idx=None, stride=0, rand_block=0, n_rand=0, rand_idx=None):
    """(visible_pairs, tiles_full, tiles_edge) of one head for an attn_mask."""
    m = _mask(causal, win_left, win_right, block, dilation, global_idx, stride, rand_block, n_rand, rand_idx)
    a, b, c = ctypes.c_longlong(), ctypes.c_longlong(), ctypes.c_longlong()
    _check(lib().attn_plan_stats_masked(N, ctypes.byref(m), bm, bn, ctypes.byref(a), ctypes.byref(b),
                                        ctypes.byref(c)))
    return a.value, b.value, c.value


def attn_decode(q, k_cache, v_cache, seq_len, out, lse, B, H, H_kv, Nq, S, d, win_left=-1, rolling=0, *,
                dtype=ATTN_BF16, scale=0.0, stream=None, workspace=None, workspace_bytes=0):
    """Raw decoding entry point (seq_len is a device int32 array of B)."""
    opts = _Opts(dtype, float(scale), stream, workspace, workspace_bytes)
    _check(lib().attn_decode(q, k_cache, v_cache, seq_len, out, lse, B, H, H_kv, Nq, S, d, win_left, rolling,
                             ctypes.byref(opts)))


def attn_decode_workspace_bytes(B, H, H_kv, Nq, S, d, win_left=-1, rolling=0) -> int:
    return int(lib().attn_decode_workspace_bytes(B, H, H_kv, Nq, S, d, win_left, int(bool(rolling))))


def attn_bwd_workspace_bytes(B, H, N, d, *, H_kv=None, n_global=0) -> int:
    return int(lib().attn_bwd_workspace_bytes(B, H, H if H_kv is None else H_kv, N, d, n_global))


def attn_workspace_bytes(B, H, N, d, n_global) -> int:
    return int(lib().attn_workspace_bytes(B, H, N, d, n_global))


def attn_plan_stats(N, causal, win_left, win_right, global_idx, bm, bn):
    """(visible_pairs, tiles_full, tiles_edge) of one head."""
    g, ng = _gidx(global_idx)
    a, b, c = ctypes.c_longlong(), ctypes.c_longlong(), ctypes.c_longlong()
    _check(lib().attn_plan_stats(N, causal, win_left, win_right, g, ng, bm, bn,
                                 ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
    return a.value, b.value, c.value


def attn_tile_shape(d, dtype=ATTN_BF16):
    bm, bn = ctypes.c_int(), ctypes.c_int()
    _check(lib().attn_tile_shape(d, dtype, ctypes.byref(bm), ctypes.byref(bn)))
    return bm.value, bn.value


def _ws(workspace):
    """(device address, bytes) of a workspace tensor, or (None, 0)."""
    if workspace is None:
        return None, 0
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def fwd(q, k, v, *, causal=False, win_left=-1, win_right=-1, global_idx=None, scale=None,
        out=None, lse=None, workspace=None, stream=None, block=0, dilation=1, stride=0, rand_block=0,
        rand_idx=None):
    """Attention forward on torch CUDA tensors: q [B, H, N, d], k and v
    [B, H_kv, N, d] with H_kv dividing H (H_kv = H: multi-head; H_kv < H:
    grouped-query; H_kv = 1: multi-query), bf16 or fp32. ``rand_idx`` (with
    ``rand_block``) is a contiguous int32 device tensor [ceil(N / rand_block),
    r] of key-block lists.

    Allocates ``out`` (input dtype) and ``lse`` (fp32 [B, H, N]) with torch
    unless given, and with global tokens a workspace for the global-row
    partials (so concurrent calls on different streams share no memory),
    enqueues the kernels on torch's current stream (or ``stream``) and
    returns (out, lse) without synchronising.
    """
    import torch
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(f"unsupported dtype {q.dtype}")
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("tensors must be [B, H, N, d]")
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != q.dtype or (t.shape[0], t.shape[2], t.shape[3]) != (B, N, d):
            raise ValueError(f"{name} must match q in dtype, batch, length and head size")
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if v.shape != k.shape:
        raise ValueError("k and v must have the same shape")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 tensor [B, H, N]")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    if workspace is None and global_idx is not None and len(global_idx) > 0:
        # a workspace of this call's own (torch's caching allocator), so that
        # calls on different streams never share the library's scratch
        nb = attn_workspace_bytes(B, H, N, d, len(global_idx))
        if nb > 0:
            workspace = torch.empty(nb, dtype=torch.uint8, device=q.device)
    ws, wsb = _ws(workspace)
    n_rand, rptr = 0, None
    if rand_block:
        if rand_idx is None or rand_idx.dtype != torch.int32 or not rand_idx.is_cuda or rand_idx.dim() != 2 \
                or not rand_idx.is_contiguous() or rand_idx.shape[0] != (N + rand_block - 1) // rand_block:
            raise ValueError("rand_idx must be a contiguous int32 device tensor [ceil(N / rand_block), r]")
        n_rand, rptr = rand_idx.shape[1], rand_idx.data_ptr()
    attn_fwd_masked(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                    B, H, H_kv, N, d, causal=causal, win_left=win_left, win_right=win_right, block=block,
                    dilation=dilation, global_idx=global_idx,
                    dtype=ATTN_F32 if q.dtype == torch.float32 else ATTN_BF16,
                    scale=0.0 if scale is None else float(scale), stream=stream,
                    workspace=ws, workspace_bytes=wsb, stride=stride, rand_block=rand_block, n_rand=n_rand,
                    rand_idx=rptr)
    return out, lse


def bwd(q, k, v, out, dout, lse, *, causal=False, win_left=-1, win_right=-1, global_idx=None, scale=None,
        dq=None, dk=None, dv=None, workspace=None, stream=None, block=0, dilation=1, stride=0, rand_block=0,
        rand_idx=None):
    """Gradients (dq, dk, dv) of ``fwd`` on torch CUDA bf16 tensors: q, out,
    dout [B, H, N, d], k, v [B, H_kv, N, d], lse fp32 [B, H, N] from the
    forward call with the same mask and scale. Allocates the gradients and
    the workspace with torch unless given and enqueues the kernels without
    synchronising."""
    import torch
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("tensors must be [B, H, N, d]")
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    for name, t, shape in (("q", q, q.shape), ("out", out, q.shape), ("dout", dout, q.shape),
                           ("k", k, k.shape), ("v", v, k.shape)):
        if t.dtype != torch.bfloat16 or t.shape != shape or (t.shape[0], t.shape[2], t.shape[3]) != (B, N, d):
            raise ValueError(f"{name} must be bf16 and shaped consistently with q")
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 tensor [B, H, N]")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    if workspace is None:
        nb = attn_bwd_workspace_bytes(B, H, N, d, H_kv=H_kv,
                                      n_global=0 if global_idx is None else len(global_idx))
        if nb > 0:
            workspace = torch.empty(nb, dtype=torch.uint8, device=q.device)
    ws, wsb = _ws(workspace)
    n_rand, rptr = 0, None
    if rand_block:
        if rand_idx is None or rand_idx.dtype != torch.int32 or not rand_idx.is_cuda or rand_idx.dim() != 2 \
                or not rand_idx.is_contiguous() or rand_idx.shape[0] != (N + rand_block - 1) // rand_block:
            raise ValueError("rand_idx must be a contiguous int32 device tensor [ceil(N / rand_block), r]")
        n_rand, rptr = rand_idx.shape[1], rand_idx.data_ptr()
    attn_bwd_masked(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                    dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, H_kv, N, d, causal=causal,
                    win_left=win_left, win_right=win_right, block=block, dilation=dilation,
                    global_idx=global_idx, scale=0.0 if scale is None else float(scale), stream=stream,
                    workspace=ws, workspace_bytes=wsb, stride=stride, rand_block=rand_block, n_rand=n_rand,
                    rand_idx=rptr)
    return dq, dk, dv


def decode(q, k_cache, v_cache, seq_len, *, win_left=-1, rolling=False, scale=None, out=None, lse=None,
           workspace=None, stream=None):
    """One decoding step on torch CUDA bf16 tensors: q [B, H, Nq, d] holds the
    queries of each sequence's Nq newest positions, k_cache and v_cache
    [B, H_kv, S, d] the cached keys and values (the new positions included),
    seq_len a device int32 tensor [B] of sequence lengths. ``rolling`` keeps
    position p in slot p % S. Returns (out [B, H, Nq, d], lse fp32 [B, H, Nq])
    without synchronising."""
    import torch
    if q.dim() != 4 or k_cache.dim() != 4:
        raise ValueError("q must be [B, H, Nq, d] and the caches [B, H_kv, S, d]")
    B, H, Nq, d = q.shape
    H_kv, S = k_cache.shape[1], k_cache.shape[2]
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 device tensor")
    if v_cache.shape != k_cache.shape or k_cache.shape[0] != B or k_cache.shape[3] != d:
        raise ValueError("caches must be [B, H_kv, S, d] matching q")
    if seq_len.dtype != torch.int32 or seq_len.shape != (B,) or not seq_len.is_cuda or not seq_len.is_contiguous():
        raise ValueError("seq_len must be a contiguous int32 device tensor [B]")
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if lse is None else lse
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    if lse.shape != (B, H, Nq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 tensor [B, H, Nq]")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    if workspace is None:
        nb = attn_decode_workspace_bytes(B, H, H_kv, Nq, S, d, win_left, rolling)
        if nb > 0:
            workspace = torch.empty(nb, dtype=torch.uint8, device=q.device)
    ws, wsb = _ws(workspace)
    attn_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seq_len.data_ptr(), out.data_ptr(),
                lse.data_ptr(), B, H, H_kv, Nq, S, d, win_left, int(bool(rolling)),
                scale=0.0 if scale is None else float(scale), stream=stream, workspace=ws, workspace_bytes=wsb)
    return out, lse
