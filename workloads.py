"""Seeded synthetic inputs for the CLiS attention workloads.

This module only draws random numbers and shapes them into the workloads'
distributions.  It holds none of the attention or certification arithmetic,
so both sides of every parity check -- the HIP library and the fp64 oracle --
read the very same bytes from it and share nothing else.

Workload shapes follow the video-diffusion setting of the pages ("CLiS:
Plug-and-Play Attention Acceleration for Video Diffusion on TPUs via Certified
Stabilization"): Wan 2.2 at 720p x 81 frames is 75,600 tokens with head dim 128
(Table 7 caption), and the 480p rows of Table 8 fix the latent grid
tokens = ((frames - 1) / 4 + 1) * 30 * 52.  Real activations are not
available; Gaussians stand in for them, with a per-head key bias so that the
key-mean centering of the certification matters.

Every tensor of every (batch, head) pair has its own PCG64 stream seeded by
SeedSequence([seed, config id, b, h, tensor id]); a single head can therefore
be regenerated without the rest.  Draws are fp32; biases and scales are applied
in fp32; bf16 workloads are rounded once (round to nearest even) at the end.
bf16 tensors are returned as uint16 arrays holding the raw bf16 bit patterns.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_KBIAS = 0, 1, 2, 3


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    B: int
    H: int
    N: int
    d: int
    dtype: str            # "bf16" or "fp32"
    causal: bool
    key_bias_std: float   # std of the per-head, per-channel key bias (0: none)
    fail_frac: float = 0.0      # fraction of heads pushed past certification
    fail_qk_scale: float = 1.0  # Q and K multiplier on those heads
    outlier_frac: float = 0.0   # fraction of key rows scaled further on those heads
    outlier_scale: float = 1.0
    note: str = ""
    Nk_: int | None = None      # key/value rows when they differ from the query rows

    @property
    def Nq(self) -> int:
        return self.N

    @property
    def Nk(self) -> int:
        return self.N if self.Nk_ is None else self.Nk_

    @property
    def scale(self) -> float:
        """1/sqrt(d) as the fp32 value the library receives (its ABI takes fp32)."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    def flops(self) -> float:
        """Attention FLOPs of one forward call: 4*d per unmasked score."""
        if self.causal:
            return 4.0 * self.B * self.H * self.d * self.N * (self.N + 1) / 2
        return 4.0 * self.B * self.H * self.Nq * self.Nk * self.d


def latent_tokens(frames: int, height: int, width: int) -> int:
    """Video latent tokens: 4x temporal and 16x spatial reduction (Table 8 rows)."""
    return ((frames - 1) // 4 + 1) * (height // 16) * (width // 16)


WORKLOADS = {
    "tiny": Workload("tiny", 0, 1, 2, 256, 64, "fp32", False, 0.0,
                     note="B1 H2 N256 d64 fp32, Q,K,V ~ N(0,1)"),
    "wan720p": Workload("wan720p", 1, 1, 20, latent_tokens(81, 720, 1280), 128, "bf16", False, 2.0,
                        note="Wan 2.2 720p x 81f, one GPU's 20-head share"),
    "wan480p": Workload("wan480p", 2, 2, 24, latent_tokens(81, 480, 832), 128, "bf16", False, 2.0,
                        note="Wan 2.2 480p x 81f shaped, B2 H24"),
    "mixed": Workload("mixed", 3, 1, 20, latent_tokens(81, 720, 1280), 128, "bf16", False, 2.0,
                      fail_frac=0.25, fail_qk_scale=40.0, outlier_frac=0.001, outlier_scale=200.0,
                      note="wan720p plus 25% heads with Q,K x40 and 0.1% key rows x200"),
    "causal": Workload("causal", 4, 4, 32, 8192, 128, "bf16", True, 1.0,
                       note="LLM-shaped causal forward, B4 H32 N8192"),
}


def custom(name: str, B: int, H: int, N: int, d: int, dtype: str = "bf16", causal: bool = False,
           key_bias_std: float = 2.0, base: str | None = None, Nk: int | None = None, **kw) -> Workload:
    """A workload of the given shape (Nk: key rows, default N) with another
    workload's distribution, or plain Gaussians plus a key bias."""
    if base is not None:
        w = WORKLOADS[base]
        params = dict(key_bias_std=w.key_bias_std, fail_frac=w.fail_frac, fail_qk_scale=w.fail_qk_scale,
                      outlier_frac=w.outlier_frac, outlier_scale=w.outlier_scale)
        params.update(kw)
        return Workload(name, 100 + w.cfg_id, B, H, N, d, dtype, causal, Nk_=Nk, **params)
    return Workload(name, 100, B, H, N, d, dtype, causal, key_bias_std, Nk_=Nk, **kw)


def _rng(seed: int, w: Workload, *ids: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, w.cfg_id, *ids])))


def failing_heads(w: Workload, seed: int = 0) -> np.ndarray:
    """Flat (b*H + h) indices of the heads scaled past certification, sorted."""
    n = w.B * w.H
    k = int(round(w.fail_frac * n))
    if k == 0:
        return np.zeros(0, dtype=np.int64)
    sel = _rng(seed, w, 1_000_001).choice(n, size=k, replace=False)
    return np.sort(sel.astype(np.int64))


def outlier_rows(w: Workload, b: int, h: int, seed: int = 0) -> np.ndarray:
    """Key rows scaled further on a failing head (a seeded 0.1% of them)."""
    k = int(round(w.outlier_frac * w.Nk))
    if k == 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(_rng(seed, w, b, h, 1_000_002).choice(w.Nk, size=k, replace=False).astype(np.int64))


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def head_f32(w: Workload, b: int, h: int, seed: int = 0, fail_set=None):
    """Q, K, V of one (b, h) head as fp32 [N, d] arrays, before any rounding."""
    d = w.d
    q = _rng(seed, w, b, h, TENSOR_Q).standard_normal((w.Nq, d), dtype=np.float32)
    k = _rng(seed, w, b, h, TENSOR_K).standard_normal((w.Nk, d), dtype=np.float32)
    v = _rng(seed, w, b, h, TENSOR_V).standard_normal((w.Nk, d), dtype=np.float32)
    if w.key_bias_std:
        bias = _rng(seed, w, b, h, TENSOR_KBIAS).standard_normal(d, dtype=np.float32)
        k += np.float32(w.key_bias_std) * bias
    if fail_set is None:
        fail_set = set(failing_heads(w, seed).tolist())
    if (b * w.H + h) in fail_set:
        q *= np.float32(w.fail_qk_scale)
        k *= np.float32(w.fail_qk_scale)
        rows = outlier_rows(w, b, h, seed)
        if rows.size:
            k[rows] *= np.float32(w.outlier_scale)
    return q, k, v


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def make_inputs(w: Workload, seed: int = 0, heads=None):
    """Q, K, V as [B, H, N, d] arrays (uint16 bf16 bits, or float32).

    `heads` optionally restricts generation to a list of flat head indices;
    the other heads are left zero (used only where a test needs a few heads).
    """
    out_dtype = np.uint16 if w.dtype == "bf16" else np.float32
    Q = np.zeros((w.B, w.H, w.Nq, w.d), dtype=out_dtype)
    K, V = (np.zeros((w.B, w.H, w.Nk, w.d), dtype=out_dtype) for _ in range(2))
    fail_set = set(failing_heads(w, seed).tolist())
    todo = range(w.B * w.H) if heads is None else heads

    def one(flat):
        b, h = divmod(int(flat), w.H)
        q, k, v = head_f32(w, b, h, seed, fail_set)
        for dst, src in ((Q, q), (K, k), (V, v)):
            dst[b, h] = round_to_bf16_bits(src) if w.dtype == "bf16" else src

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, todo))
    return Q, K, V


def sample_rows(w: Workload, n_random: int = 200, seed: int = 0, tiles=(64, 128, 256)) -> np.ndarray:
    """Query rows checked at full size: both ends, tile edges and seeded rows."""
    N = w.N
    rows = set(range(min(8, N))) | set(range(max(0, N - 8), N))
    for t in tiles:
        for e in range(t, N, t * max(1, N // (t * 16))):
            rows.update(r for r in (e - 1, e) if 0 <= r < N)
    rng = _rng(seed, w, 1_000_003)
    rows.update(rng.choice(N, size=min(n_random, N), replace=False).tolist())
    return np.array(sorted(rows), dtype=np.int64)


EDGE_HEADS = ("offset_cap", "competing_keys", "competing_keys_offset")


def edge_head(kind: str, seed: int = 0, nq: int = 300, nk: int = 1024, d: int = 128):
    """Hand-built heads whose certified bound sits just under the cap, as fp32
    [N, d] arrays (q, k, v) to be rounded to bf16 by the caller.  All the
    constants below are exact in bf16.

    offset_cap: every key is 8192 e0 +- 256 e0 (half each), so the key mean
      is 8192 e0 and the centered keys are +-256 e0; V = 0.75 everywhere;
      q0 = 3.578125 e0, q1 = 0.5 e1, other query rows 0.1 N(0,1).  A large
      shared key offset with the bound c * 3.578125 * 256 = 116.8 just under
      the cap 127 - ceil(log2 1024) - 0 = 117.
    competing_keys: keys 0.5 N(0,1) except k5 = 227 e0 and k9 = 230 e1 (the
      bf16 value nearest 2.71875 * 227 / 2.6875); v5 = +2.5, v9 = -2.5, other
      values N(0,1); q0 = 2.71875 e0 + 2.6875 e1, other rows 0.1 N(0,1).
      Row 0 weighs two keys of nearly equal score (exponents ~79) with values
      of opposite sign, so its output is sensitive to exponent errors; the
      bound c |q0| kappa = 112.0 is just under the cap 114.
    competing_keys_offset: as competing_keys, with 4096 added to channel 2 of
      every key and q0[2] = 0.5 (a shared offset the row does see).
    """
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7_000_000, EDGE_HEADS.index(kind)])))
    q = np.float32(0.1) * rng.standard_normal((nq, d), dtype=np.float32)
    if kind == "offset_cap":
        k = np.zeros((nk, d), dtype=np.float32)
        k[:, 0] = 8192.0
        k[: nk // 2, 0] += 256.0
        k[nk // 2:, 0] -= 256.0
        k = k[rng.permutation(nk)]
        v = np.full((nk, d), 0.75, dtype=np.float32)
        q[0] = 0.0
        q[0, 0] = 3.578125
        q[1] = 0.0
        q[1, 1] = 0.5
    elif kind in ("competing_keys", "competing_keys_offset"):
        k = np.float32(0.5) * rng.standard_normal((nk, d), dtype=np.float32)
        v = rng.standard_normal((nk, d), dtype=np.float32)
        k[5] = 0.0
        k[5, 0] = 227.0
        k[9] = 0.0
        k[9, 1] = 230.0
        v[5] = 2.5
        v[9] = -2.5
        q[0] = 0.0
        q[0, 0] = 2.71875
        q[0, 1] = 2.6875
        if kind == "competing_keys_offset":
            k[:, 2] += np.float32(4096.0)
            q[0, 2] = 0.5
    else:
        raise ValueError(kind)
    return q, k, v


def to_torch(a: np.ndarray, dtype: str, device: str = "cuda"):
    """Copy seeded host inputs to a torch device tensor, bytes unchanged
    (bf16 bit patterns become a bfloat16 tensor)."""
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)
