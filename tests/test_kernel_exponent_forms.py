"""The fixed-stabilizer kernel's exponent arithmetic, emulated on the CPU,
against the fp64 oracle on heads at the edge of the certificate.

The certificate (Algorithm 1 of "CLiS: Plug-and-Play Attention Acceleration
for Video Diffusion on TPUs via Certified Stabilization", steps 1-7) bounds
the exp2 argument x = c q.(k - kbar), c = scale log2(e), by B_h <= C, so that
no weight and no accumulator overflows (the abstract's per-head numerical
safety; Table 1 counts an output with NaN/Inf as invalid).  That promise holds
for the kernel only if the kernel evaluates x to within a small fraction of
the cap's one-binade margin.  These tests emulate, in numpy, the two ways a
kernel can form x from bf16 inputs:

  fma       x = fma(s, c, -mu) in fp32, s = q.k accumulated in fp32 from the
            exact bf16 products (the form every fixed kernel uses);
  prescale  the query rounded to q' = bf16(c q) before the score product,
            which starts from -mu (a shortcut that saves the fma).  It moves
            every exponent by (q' - c q).k_j: unbounded through the shared key
            offset kbar, and up to 2^-9 B_h through the centered keys.

then weights 2^x in fp32, row sums of those fp32 weights, the weights rounded
to bf16 for the P.V product, and O = sum p v / l.  The kept form must match the
oracle within the bf16 tolerances on every edge head; the shortcut fails both
ways on them (NaN from overflow on a certified head with a large key offset,
an error of ~0.4 on one with two competing keys near the bound), which is why
no kernel uses it.  CPU only.
"""
import math

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import BF16_TOL, errors

D = 128
SCALE = float(np.float32(1.0 / math.sqrt(D)))  # the fp32 value the library receives
C2 = np.float32(SCALE * oracle.LOG2E)         # c rounded to fp32, as the kernels hold it


def _bf16(x):
    """fp32 values rounded to bf16 (round to nearest even), as fp32."""
    return workloads.bf16_bits_to_f32(workloads.round_to_bf16_bits(np.asarray(x, dtype=np.float32)))


def _head(kind):
    q, k, v = workloads.edge_head(kind)
    bits = [workloads.round_to_bf16_bits(a) for a in (q, k, v)]
    return bits, [workloads.bf16_bits_to_f32(b) for b in bits]


def emulate_fixed(q, k, v, mu, form):
    """One head of the fixed-stabilizer kernel's arithmetic: q [Nq,d], k,v [Nk,d]
    fp32 (bf16 values), mu [Nq] fp32.  Returns (O fp32, max exp2 argument)."""
    q64, k64 = q.astype(np.float64), k.astype(np.float64)
    mu32 = mu.astype(np.float32)
    if form == "fma":
        s = (q64 @ k64.T).astype(np.float32)  # fp32 score accumulator
        x = (s.astype(np.float64) * np.float64(C2) - mu32.astype(np.float64)[:, None]).astype(np.float32)
    elif form == "prescale":
        qp = _bf16(q * C2)  # fp32 product, one bf16 rounding
        x = (qp.astype(np.float64) @ k64.T - mu32.astype(np.float64)[:, None]).astype(np.float32)
    else:
        raise ValueError(form)
    with np.errstate(over="ignore", invalid="ignore"):
        p32 = np.exp2(x).astype(np.float32)  # v_exp_f32
        l = p32.sum(axis=1, dtype=np.float32)  # row sums of the fp32 weights
        p = _bf16(p32)  # bf16 for the P.V operand
        acc = (p.astype(np.float64) @ v.astype(np.float64))
        acc = np.where(np.isfinite(acc) & (np.abs(acc) < np.finfo(np.float32).max), acc, np.inf * np.sign(acc))
        o = acc.astype(np.float32) / l[:, None]
    return o, float(np.max(x))


@pytest.fixture(scope="module", params=workloads.EDGE_HEADS)
def edge(request):
    bits, vals = _head(request.param)
    ref = oracle.certify(*(b[None, None] for b in bits), "bf16", SCALE)
    want = oracle.attention(*(b[None, None] for b in bits), "bf16", SCALE)[0, 0]
    return request.param, vals, ref, want


def test_edge_heads_certify_just_under_the_cap(edge):
    name, _, ref, _ = edge
    bound, cap = ref["bound"][0, 0], ref["C"][0, 0]
    assert ref["cert"][0, 0] == 1, name
    assert 0.95 * cap < bound <= cap and cap - bound > 1e-9 * cap, (name, bound, cap)


def test_fma_form_matches_the_oracle_on_edge_heads(edge):
    """The kept form: finite, the largest exponent within rounding of the
    bound, output within the bf16 tolerances."""
    name, (q, k, v), ref, want = edge
    o, xmax = emulate_fixed(q, k, v, ref["mu"][0, 0], "fma")
    assert np.all(np.isfinite(o)), name
    assert xmax <= ref["bound"][0, 0] + 1e-2, (name, xmax)
    e = errors(o.astype(np.float64), want)
    assert all(e[m] <= t for m, t in BF16_TOL.items()), (name, e)


def test_prescaled_query_form_breaks_the_certificate():
    """The shortcut on the same heads: the large shared offset pushes the
    largest exponent past the cap, the row sums overflow and O is NaN on a
    certified head; two competing keys near the bound move the output far
    outside the tolerance."""
    bits, (q, k, v) = _head("offset_cap")
    ref = oracle.certify(*(b[None, None] for b in bits), "bf16", SCALE)
    o, xmax = emulate_fixed(q, k, v, ref["mu"][0, 0], "prescale")
    assert ref["cert"][0, 0] == 1
    assert xmax > ref["C"][0, 0] + 1.0
    assert not np.all(np.isfinite(o))

    bits, (q, k, v) = _head("competing_keys")
    ref = oracle.certify(*(b[None, None] for b in bits), "bf16", SCALE)
    want = oracle.attention(*(b[None, None] for b in bits), "bf16", SCALE)[0, 0]
    o, _ = emulate_fixed(q, k, v, ref["mu"][0, 0], "prescale")
    e = errors(o.astype(np.float64), want)
    assert e["max_abs"] > 0.1, e


def test_fma_form_error_scales_with_fp32_rounding_only():
    """On the offset head the fma form's largest exponent equals the oracle's
    (c q0 . 256 e0 = B_h) to fp32 rounding of the products of size
    c |q0| |k| ~ 3.9e3, i.e. well inside the one-binade margin."""
    bits, (q, k, v) = _head("offset_cap")
    ref = oracle.certify(*(b[None, None] for b in bits), "bf16", SCALE)
    _, xmax = emulate_fixed(q, k, v, ref["mu"][0, 0], "fma")
    assert abs(xmax - ref["bound"][0, 0]) < 4e3 * 2.0 ** -20
