"""fp64 CPU oracle for CLiS attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library and its Python binding
never import, link or call it, and it shares no code with them; the only
module both sides read is ``workloads`` (seeded inputs, no method arithmetic).

The arithmetic lives in ``oracle.c`` (plain C, fp64).  This wrapper only
decodes inputs to fp64 exactly (bf16 bit patterns or fp32), hands one
(batch, head) pair at a time to the C functions, and spreads independent row
ranges over threads (ctypes releases the GIL), which changes no result.

Source pages: "CLiS: Plug-and-Play Attention Acceleration for Video Diffusion
on TPUs via Certified Stabilization" -- abstract, Algorithm 1, Figure 3,
Figure 5(a).
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "_oracle.so")
_lock = threading.Lock()
_lib = None

LOG2E = 1.4426950408889634


def compile_source(src: str, dst: str) -> str:
    """gcc a copy of the oracle source into a shared library (no fast-math,
    no FMA contraction, so every operation rounds as written)."""
    tmp = dst + f".tmp{os.getpid()}"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                    "-fno-fast-math", src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, dst)
    return dst


def build(force: bool = True) -> str:
    """Compile oracle.c into _oracle.so."""
    if force or not os.path.exists(_LIB):
        compile_source(_SRC, _LIB)
    return _LIB


class CertRecord(ctypes.Structure):
    _fields_ = [("kappa", ctypes.c_double), ("qnorm_max", ctypes.c_double),
                ("bound", ctypes.c_double), ("maxabs_v", ctypes.c_double),
                ("u_exp", ctypes.c_double), ("u_acc", ctypes.c_double),
                ("G", ctypes.c_int32), ("L", ctypes.c_int32), ("A", ctypes.c_int32),
                ("C", ctypes.c_int32), ("cert", ctypes.c_int32), ("pad", ctypes.c_int32)]

    def as_dict(self) -> dict:
        return {n: getattr(self, n) for n, _ in self._fields_ if n != "pad"}


def _load(path):
    L = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int64)
    i64, ci, cd = ctypes.c_int64, ctypes.c_int, ctypes.c_double
    L.oracle_attention_rows.argtypes = [dp, dp, dp, i64, i64, ci, cd, ci, ip, i64, dp]
    L.oracle_certify_head.argtypes = [dp, dp, dp, i64, i64, ci, cd, ci, dp, dp, ctypes.POINTER(CertRecord)]
    L.oracle_fixed_mu_rows.argtypes = [dp, dp, dp, i64, i64, ci, cd, ci, dp, ip, i64, dp, dp, dp]
    L.oracle_online_rows.argtypes = [dp, dp, dp, i64, i64, ci, cd, ci, i64, cd, ip, i64, dp]
    L.oracle_lse_rows.argtypes = [dp, dp, i64, i64, ci, cd, ci, ip, i64, dp]
    L.oracle_fixed_mu_partial_rows.argtypes = [dp, dp, dp, i64, i64, ci, cd, ci, dp, i64, i64, ip, i64, dp, dp]
    for f in (L.oracle_attention_rows, L.oracle_certify_head, L.oracle_fixed_mu_rows,
              L.oracle_online_rows, L.oracle_lse_rows, L.oracle_fixed_mu_partial_rows):
        f.restype = ctypes.c_int
    return L


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build(force=False)
            _lib = _load(_LIB)
    return _lib


@contextlib.contextmanager
def using_library(path: str):
    """Run the wrapper over another build of oracle.c (the mutation tests
    build copies with planted mistakes to show the pins catch them)."""
    global _lib
    old = lib()
    with _lock:
        _lib = _load(path)
    try:
        yield
    finally:
        with _lock:
            _lib = old


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ---------------------------------------------------------------- decoding
def decode(x: np.ndarray, dtype: str) -> np.ndarray:
    """Inputs to fp64, exactly: bf16 bit patterns (uint16) or fp32 values."""
    if dtype == "bf16":
        if x.dtype != np.uint16:
            raise TypeError("bf16 inputs are passed as uint16 bit patterns")
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "fp32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "fp64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(dtype)


def _p(a, ty=ctypes.c_double):
    return a.ctypes.data_as(ctypes.POINTER(ty))


def _chunks(rows: np.ndarray, threads: int):
    n = len(rows)
    if n == 0:
        return []
    k = max(1, min(threads * 4, n))
    bounds = np.linspace(0, n, k + 1).astype(np.int64)
    return [(int(a), int(b)) for a, b in zip(bounds[:-1], bounds[1:]) if b > a]


def _fanout(fn, rows, threads):
    parts = _chunks(rows, threads)
    if threads <= 1 or len(parts) <= 1:
        for a, b in parts:
            fn(a, b)
        return
    with ThreadPoolExecutor(threads) as ex:
        for f in [ex.submit(fn, a, b) for a, b in parts]:
            f.result()


# ---------------------------------------------------------------- per head
def attention_head(q, k, v, scale: float, causal: bool = False, rows=None, threads: int | None = None):
    """Softmax attention by definition for one head. q [Nq,d], k,v [Nk,d] fp64."""
    q, k, v = (np.ascontiguousarray(a, dtype=np.float64) for a in (q, k, v))
    nq, d = q.shape
    nk = k.shape[0]
    rows = np.arange(nq, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    if causal and nq != nk:
        raise ValueError("causal attention needs Nq == Nk")
    if rows.size and (rows.min() < 0 or rows.max() >= nq):
        raise IndexError("row out of range")
    out = np.zeros((len(rows), d), dtype=np.float64)
    L = lib()

    def run(a, b):
        r = L.oracle_attention_rows(_p(q), _p(k), _p(v), nq, nk, d, float(scale), int(causal),
                                    _p(rows[a:b], ctypes.c_int64), b - a, _p(out[a:b]))
        if r != 0:
            raise MemoryError("oracle_attention_rows")

    _fanout(run, rows, threads or default_threads())
    return out


def certify_head(q, k, v, scale: float, p_bf16: bool = True):
    """Algorithm 1 statistics, flag and fixed stabilizers for one head."""
    q, k, v = (np.ascontiguousarray(a, dtype=np.float64) for a in (q, k, v))
    nq, d = q.shape
    nk = k.shape[0]
    if nk < 1 or nq < 1:
        raise ValueError("empty head")
    kbar = np.zeros(d, dtype=np.float64)
    mu = np.zeros(nq, dtype=np.float64)
    rec = CertRecord()
    lib().oracle_certify_head(_p(q), _p(k), _p(v), nq, nk, d, float(scale), int(p_bf16),
                              _p(kbar), _p(mu), ctypes.byref(rec))
    out = rec.as_dict()
    out["kbar"] = kbar
    out["mu"] = mu
    return out


def fixed_mu_head(q, k, v, scale: float, mu, causal: bool = False, rows=None, threads: int | None = None):
    """Output evaluated with fixed stabilizers mu (log2 units); also max exp2
    argument and max |accumulator| per row."""
    q, k, v = (np.ascontiguousarray(a, dtype=np.float64) for a in (q, k, v))
    mu = np.ascontiguousarray(mu, dtype=np.float64)
    nq, d = q.shape
    nk = k.shape[0]
    rows = np.arange(nq, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), d), dtype=np.float64)
    mx = np.zeros(len(rows), dtype=np.float64)
    ma = np.zeros(len(rows), dtype=np.float64)
    L = lib()

    def run(a, b):
        L.oracle_fixed_mu_rows(_p(q), _p(k), _p(v), nq, nk, d, float(scale), int(causal), _p(mu),
                               _p(rows[a:b], ctypes.c_int64), b - a, _p(out[a:b]), _p(mx[a:b]), _p(ma[a:b]))

    _fanout(run, rows, threads or default_threads())
    return out, mx, ma


def online_head(q, k, v, scale: float, causal: bool = False, block: int = 64, rows=None,
                threads: int | None = None, tau: float = 0.0):
    """Output evaluated with online softmax over key blocks of `block` keys;
    tau > 0: rescale only when a block maximum exceeds the stabilizer in use
    by more than tau (log2 units)."""
    q, k, v = (np.ascontiguousarray(a, dtype=np.float64) for a in (q, k, v))
    nq, d = q.shape
    nk = k.shape[0]
    rows = np.arange(nq, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), d), dtype=np.float64)
    L = lib()

    def run(a, b):
        L.oracle_online_rows(_p(q), _p(k), _p(v), nq, nk, d, float(scale), int(causal), int(block),
                             float(tau), _p(rows[a:b], ctypes.c_int64), b - a, _p(out[a:b]))

    _fanout(run, rows, threads or default_threads())
    return out


def lse_head(q, k, scale: float, causal: bool = False, rows=None, threads: int | None = None):
    """Per-row log-sum-exp (natural log) of the scores scale * q_i . k_j over
    the visible keys; [len(rows)] fp64."""
    q, k = (np.ascontiguousarray(a, dtype=np.float64) for a in (q, k))
    nq, d = q.shape
    nk = k.shape[0]
    rows = np.arange(nq, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    out = np.zeros(len(rows), dtype=np.float64)
    L = lib()

    def run(a, b):
        L.oracle_lse_rows(_p(q), _p(k), nq, nk, d, float(scale), int(causal),
                          _p(rows[a:b], ctypes.c_int64), b - a, _p(out[a:b]))

    _fanout(run, rows, threads or default_threads())
    return out


def fixed_mu_partial_head(q, k, v, scale: float, mu, k0: int, k1: int, causal: bool = False, rows=None,
                          threads: int | None = None):
    """Unnormalized fixed-stabilizer sums over keys [k0, k1): (acc [rows, d],
    l [rows]) with weights 2^(c q.k - mu), c = scale*log2(e)."""
    q, k, v = (np.ascontiguousarray(a, dtype=np.float64) for a in (q, k, v))
    mu = np.ascontiguousarray(mu, dtype=np.float64)
    nq, d = q.shape
    nk = k.shape[0]
    rows = np.arange(nq, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    acc = np.zeros((len(rows), d), dtype=np.float64)
    l = np.zeros(len(rows), dtype=np.float64)
    L = lib()

    def run(a, b):
        L.oracle_fixed_mu_partial_rows(_p(q), _p(k), _p(v), nq, nk, d, float(scale), int(causal), _p(mu),
                                       int(k0), int(k1), _p(rows[a:b], ctypes.c_int64), b - a,
                                       _p(acc[a:b]), _p(l[a:b]))

    _fanout(run, rows, threads or default_threads())
    return acc, l


# ---------------------------------------------------------------- batched
def certify(Q, K, V, dtype: str, scale: float):
    """Per-(b,h) certification over [B,H,N,d] inputs.

    Returns dict of arrays: cert [B,H] int32, bound, kappa, qnorm_max,
    maxabs_v [B,H] fp64, G/L/A/C [B,H] int32, kbar [B,H,d], mu [B,H,Nq] fp64.
    """
    B, H, nq, d = Q.shape
    res = {n: np.zeros((B, H), dtype=np.float64) for n in ("bound", "kappa", "qnorm_max", "maxabs_v")}
    for n in ("G", "L", "A", "C", "cert"):
        res[n] = np.zeros((B, H), dtype=np.int32)
    res["kbar"] = np.zeros((B, H, d), dtype=np.float64)
    res["mu"] = np.zeros((B, H, nq), dtype=np.float64)

    def one(flat):
        b, h = divmod(flat, H)
        r = certify_head(decode(Q[b, h], dtype), decode(K[b, h], dtype), decode(V[b, h], dtype),
                         scale, p_bf16=(dtype == "bf16"))
        for n in ("bound", "kappa", "qnorm_max", "maxabs_v", "G", "L", "A", "C", "cert"):
            res[n][b, h] = r[n]
        res["kbar"][b, h] = r["kbar"]
        res["mu"][b, h] = r["mu"]

    with ThreadPoolExecutor(default_threads()) as ex:
        list(ex.map(one, range(B * H)))
    return res


def attention(Q, K, V, dtype: str, scale: float, causal: bool = False, rows=None,
              threads: int | None = None):
    """Softmax attention by definition on [B,H,N,d] inputs.

    rows: None (all rows) or an index array applied to every head; returns
    [B,H,len(rows),d] fp64.
    """
    B, H, nq, d = Q.shape
    nr = nq if rows is None else len(rows)
    out = np.zeros((B, H, nr, d), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            out[b, h] = attention_head(decode(Q[b, h], dtype), decode(K[b, h], dtype),
                                       decode(V[b, h], dtype), scale, causal, rows, threads)
    return out
