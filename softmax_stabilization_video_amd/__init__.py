"""CLiS attention forward on AMD MI355X (gfx950): Python binding.

Thin ctypes layer over ``libclis.so`` (the C ABI declared in
``include/clis.h``).  It only marshals torch tensors (device memory) and the
current HIP stream into the C calls; every step of the computation runs in
the library's HIP kernels.  There is no CPU fallback: importing this package
without a built library raises.

Entry points (same names as the C ABI):
    clis_certify(q, k, v, scale)       -> (mu, cert[, stats, kbar])
    clis_attn_fwd(q, k, v, ...)        -> o[, route][, lse]
                                          (mode auto/fixed/online/online_lazy)
    clis_attn_fwd_noalloc(q, k, v, out=o, ...) -> o   (no workspace, no allocation)
    online_attn_fwd(q, k, v, ...)      -> o            (optionally with lse)
    clis_attn_fwd_partial(q, k_shard, v_shard, mu, o_acc, l_acc, ...)
    clis_attn_combine(o_acc, l_acc, ...) -> o        (optionally with lse)
Tensors are [B, H, N, d], contiguous, bf16 or fp32, on the GPU.
The library is loaded on first use; a missing build raises ImportError.

Method: "CLiS: Plug-and-Play Attention Acceleration for Video Diffusion on
TPUs via Certified Stabilization" (abstract; Algorithm 1).
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libclis.so")

CLIS_BF16, CLIS_FP32 = 0, 1
MODES = {"auto": 0, "fixed": 1, "online": 2, "online_lazy": 3}
STATUS = {0: "CLIS_OK", 1: "CLIS_ERR_NULL", 2: "CLIS_ERR_SHAPE", 3: "CLIS_ERR_UNSUPPORTED",
          4: "CLIS_ERR_ALIGN", 5: "CLIS_ERR_WORKSPACE", 6: "CLIS_ERR_HIP"}
EXPORTS = ["clis_workspace_bytes", "clis_certify", "clis_attn_fwd", "clis_attn_fwd_noalloc", "online_attn_fwd",
           "clis_attn_fwd_partial", "clis_attn_combine", "clis_status_string", "clis_last_error",
           "clis_abi_version"]
NOALLOC_SCRATCH_BYTES = 128 << 20  # CLIS_NOALLOC_SCRATCH_BYTES of include/clis.h

# clis_head_stats_t: 4 doubles, 6 int32
STATS_DTYPE = np.dtype([("kappa", "<f8"), ("qnorm_max", "<f8"), ("bound", "<f8"), ("maxabs_v", "<f8"),
                        ("G", "<i4"), ("L", "<i4"), ("A", "<i4"), ("C", "<i4"), ("cert", "<i4"),
                        ("reserved", "<i4")])
STATS_BYTES = STATS_DTYPE.itemsize


class ClisError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libclis.so and declare its signatures (raises if it is missing)."""
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m softmax_stabilization_video_amd.build`")
    L = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.clis_workspace_bytes.argtypes = [i, i, i, i, i]
    L.clis_workspace_bytes.restype = sz
    L.clis_certify.argtypes = [vp, vp, vp, i, i, i, i, i, f, i, vp, vp, vp, vp, vp, sz, vp]
    L.clis_attn_fwd.argtypes = [vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp, vp, vp, vp, vp, sz, vp]
    L.clis_attn_fwd_noalloc.argtypes = [vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp, vp, vp, vp, vp]
    L.online_attn_fwd.argtypes = [vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp, vp, sz, vp]
    L.clis_attn_fwd_partial.argtypes = [vp, vp, vp, i, i, i, i, i, f, i, i, vp, i, i, vp, vp, vp, sz, vp]
    L.clis_attn_combine.argtypes = [vp, vp, vp, i, i, i, i, i, vp, vp, vp]
    for fn in (L.clis_certify, L.clis_attn_fwd, L.clis_attn_fwd_noalloc, L.online_attn_fwd, L.clis_attn_fwd_partial,
               L.clis_attn_combine, L.clis_abi_version):
        fn.restype = ctypes.c_int
    L.clis_abi_version.argtypes = []
    L.clis_status_string.argtypes = [i]
    L.clis_status_string.restype = ctypes.c_char_p
    L.clis_last_error.argtypes = []
    L.clis_last_error.restype = ctypes.c_char_p
    return L


_lib = None


def get_lib() -> ctypes.CDLL:
    """The loaded library (loaded on first use; raises if it is not built)."""
    global _lib
    if _lib is None:
        _lib = load_library()
    return _lib


def __getattr__(name):  # module attribute `lib`, loaded on first access
    if name == "lib":
        return get_lib()
    raise AttributeError(name)


def _check(status: int):
    if status != 0:
        raise ClisError(status, get_lib().clis_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return CLIS_BF16
    if t.dtype == torch.float32:
        return CLIS_FP32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _shapes(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, H, Nq, d = q.shape
    if k.shape[:2] != (B, H) or v.shape != k.shape or k.shape[3] != d:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    for t in (q, k, v):
        if not t.is_contiguous() or not t.is_cuda or t.dtype != q.dtype:
            raise ValueError("q, k, v must be contiguous GPU tensors of one dtype")
    return B, H, Nq, k.shape[2], d


def workspace_bytes(B: int, H: int, Nq: int, Nk: int, d: int) -> int:
    return int(get_lib().clis_workspace_bytes(B, H, Nq, Nk, d))


def new_workspace(B: int, H: int, Nq: int, Nk: int, d: int, device=None):
    """A workspace tensor for these shapes (torch allocations are 256-byte aligned)."""
    import torch
    return torch.empty(workspace_bytes(B, H, Nq, Nk, d), dtype=torch.uint8, device=device or "cuda")


def clis_certify(q, k, v, scale: float | None = None, *, want_stats: bool = False, workspace=None,
                 stream=None):
    """Certify every head and compute its fixed stabilizers (clis_certify).

    Returns (mu [B,H,Nq] fp32, cert [B,H] int32), plus (stats uint8
    [B*H, 56] device bytes, kbar [B,H,d] fp64) when want_stats.
    """
    import torch
    B, H, Nq, Nk, d = _shapes(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    mu = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    cert = torch.empty((B, H), dtype=torch.int32, device=q.device)
    stats = kbar = None
    if want_stats:
        stats = torch.empty((B * H, STATS_BYTES), dtype=torch.uint8, device=q.device)
        kbar = torch.empty((B, H, d), dtype=torch.float64, device=q.device)
    ws = workspace if workspace is not None else new_workspace(B, H, Nq, Nk, d, q.device)
    _check(get_lib().clis_certify(_ptr(q), _ptr(k), _ptr(v), B, H, Nq, Nk, d, scale, _dtype_code(q),
                            _ptr(mu), _ptr(cert), _ptr(stats), _ptr(kbar), _ptr(ws), ws.numel(),
                            _stream(stream)))
    return (mu, cert, stats, kbar) if want_stats else (mu, cert)


def decode_stats(stats) -> np.ndarray:
    """Device stats bytes -> numpy structured array (one record per head)."""
    return np.frombuffer(stats.cpu().numpy().tobytes(), dtype=STATS_DTYPE)


def clis_attn_fwd(q, k, v, scale: float | None = None, causal: bool = False, mode: str = "auto",
                  mu=None, cert=None, out=None, want_route: bool = False, want_lse: bool = False,
                  workspace=None, stream=None):
    """CLiS attention forward (clis_attn_fwd).  Returns o, plus route [B,H]
    int32 and/or lse [B,H,Nq] fp32 when asked: o, (o, route), (o, lse) or
    (o, route, lse)."""
    import torch
    B, H, Nq, Nk, d = _shapes(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    if o.shape != q.shape or o.dtype != q.dtype or not o.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    route = torch.empty((B, H), dtype=torch.int32, device=q.device) if want_route else None
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if want_lse else None
    ws = workspace
    if ws is None and (mode != "online" or want_route or q.dtype != torch.float32):
        ws = new_workspace(B, H, Nq, Nk, d, q.device)
    _check(get_lib().clis_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, Nq, Nk, d, scale, int(causal),
                             _dtype_code(q), MODES[mode], _ptr(mu), _ptr(cert), _ptr(route), _ptr(lse),
                             _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))
    res = (o,) + ((route,) if want_route else ()) + ((lse,) if want_lse else ())
    return res if len(res) > 1 else o


def clis_attn_fwd_noalloc(q, k, v, scale: float | None = None, causal: bool = False, mode: str = "auto",
                          mu=None, cert=None, out=None, route=None, lse=None, stream=None):
    """clis_attn_fwd without a workspace (clis_attn_fwd_noalloc): the library's
    static per-GPU scratch instead.  The caller passes every output tensor it
    wants (out is required; route [B,H] int32 and lse [B,H,Nq] fp32 are
    optional), so this call allocates nothing.  Returns out."""
    B, H, Nq, Nk, d = _shapes(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None or out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    _check(get_lib().clis_attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, Nq, Nk, d, scale,
                                           int(causal), _dtype_code(q), MODES[mode], _ptr(mu), _ptr(cert),
                                           _ptr(route), _ptr(lse), _stream(stream)))
    return out


def online_attn_fwd(q, k, v, scale: float | None = None, causal: bool = False, out=None, want_lse: bool = False,
                    workspace=None, stream=None):
    """Online-softmax attention forward for every head (online_attn_fwd).
    Returns o, or (o, lse)."""
    import torch
    B, H, Nq, Nk, d = _shapes(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if want_lse else None
    ws = workspace
    if ws is None and q.dtype != torch.float32:
        ws = new_workspace(B, H, Nq, Nk, d, q.device)
    _check(get_lib().online_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, Nq, Nk, d, scale, int(causal),
                                     _dtype_code(q), _ptr(lse), _ptr(ws), 0 if ws is None else ws.numel(),
                                     _stream(stream)))
    return (o, lse) if want_lse else o


def clis_attn_fwd_partial(q, k, v, mu, o_acc, l_acc, scale: float | None = None, causal: bool = False,
                          kv_offset: int = 0, accumulate: bool = False, workspace=None, stream=None):
    """One key shard of fixed-stabilizer attention (clis_attn_fwd_partial):
    writes (accumulate=False) or adds to (True) the unnormalized fp32 sums
    o_acc [B,H,Nq,d] and l_acc [B,H,Nq].  k, v hold global keys
    kv_offset .. kv_offset + Nk - 1."""
    import torch
    B, H, Nq, Nk, d = _shapes(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    for t, shape in ((o_acc, (B, H, Nq, d)), (l_acc, (B, H, Nq))):
        if t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"accumulators must be contiguous fp32 of shape {shape}")
    ws = workspace
    if ws is None and q.dtype != torch.float32:
        ws = new_workspace(B, H, Nq, Nk, d, q.device)
    _check(get_lib().clis_attn_fwd_partial(_ptr(q), _ptr(k), _ptr(v), B, H, Nq, Nk, d, scale, int(causal),
                                           _dtype_code(q), _ptr(mu), int(kv_offset), int(accumulate),
                                           _ptr(o_acc), _ptr(l_acc), _ptr(ws), 0 if ws is None else ws.numel(),
                                           _stream(stream)))
    return o_acc, l_acc


def clis_attn_combine(o_acc, l_acc, dtype=None, mu=None, want_lse: bool = False, out=None, stream=None):
    """o = o_acc / l (clis_attn_combine) in `dtype` (default bf16); with
    want_lse also each row's log-sum-exp ln 2 (mu + log2 l).  Returns o, or
    (o, lse)."""
    import torch
    if o_acc.dim() != 4:
        raise ValueError("o_acc must be [B, H, Nq, d]")
    B, H, Nq, d = o_acc.shape
    for t, shape in ((o_acc, (B, H, Nq, d)), (l_acc, (B, H, Nq))) + (((mu, (B, H, Nq)),) if mu is not None else ()):
        if t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"o_acc, l_acc and mu must be contiguous fp32 GPU tensors; expected shape {shape}")
    dtype = torch.bfloat16 if dtype is None else dtype
    o = torch.empty((B, H, Nq, d), dtype=dtype, device=o_acc.device) if out is None else out
    if tuple(o.shape) != (B, H, Nq, d) or not o.is_contiguous():
        raise ValueError(f"out must be contiguous with shape {(B, H, Nq, d)}")
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=o_acc.device) if want_lse else None
    code = CLIS_BF16 if o.dtype == torch.bfloat16 else CLIS_FP32 if o.dtype == torch.float32 else None
    if code is None:
        raise ValueError("output dtype must be bf16 or fp32")
    _check(get_lib().clis_attn_combine(_ptr(o_acc), _ptr(l_acc), _ptr(o), B, H, Nq, d, code, _ptr(mu), _ptr(lse),
                                       _stream(stream)))
    return (o, lse) if want_lse else o


certify = clis_certify
attn_fwd = clis_attn_fwd
