"""GPU parity: the HIP library, called through its C ABI, against the fp64
oracle on the same seeded inputs.

Certification: flags bit-exact, the integers G, L, A, C exact, max|V| exact,
kappa / B_h / kbar to fp64 rounding, mu to fp32 rounding.  The flag is a
decision B_h <= C taken in fp64 on both sides; each case first asserts that
the oracle's B_h is not within 1e-9 (relative) of C, where the two fp64
summation orders could disagree.
Attention: bf16 within max abs 2e-2, mean abs 1e-3 and rel L2 5e-3 of the
oracle; fp32 within max abs 1e-5; in every mode (fixed, online, online with
lazy rescaling, auto).  Routing: auto mode's output for every head equals the
forced mode of the route it took, bitwise (which query tiles the dense fixed
kernel cuts into key splits depends on the head alone, not on which other
heads are routed with it).
"""
import math

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import assert_close, assert_valid, errors, say, to_device, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def clis():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import softmax_stabilization_video_amd as m
    return m


def _inputs(w, seed=0):
    Q, K, V = workloads.make_inputs(w, seed)
    return (Q, K, V), tuple(to_device(a, w.dtype) for a in (Q, K, V))


def check_certify(clis, w, host, dev, margin=1e-9):
    """Run clis_certify on the device and compare with the oracle per head."""
    import torch
    say("certify", w.name, w.B, w.H, w.Nq, w.Nk, w.d, w.dtype)
    mu, cert, stats, kbar = clis.clis_certify(*dev, w.scale, want_stats=True)
    torch.cuda.synchronize()
    ref = oracle.certify(*host, w.dtype, w.scale)
    fin = np.isfinite(ref["bound"])
    gap = np.abs(ref["bound"] - ref["C"])
    assert np.all(~fin | (gap > margin * np.maximum(1.0, np.abs(ref["C"])))), "case too close to the cap"
    st = clis.decode_stats(stats).reshape(w.B, w.H)
    assert np.array_equal(cert.cpu().numpy(), ref["cert"]), (cert.cpu().numpy(), ref["cert"])
    assert np.array_equal(st["cert"], ref["cert"])
    for n in ("G", "L", "A", "C"):
        assert np.array_equal(st[n], ref[n]), n
    assert np.array_equal(st["maxabs_v"], ref["maxabs_v"])
    np.testing.assert_allclose(st["kappa"], ref["kappa"], rtol=1e-12)
    np.testing.assert_allclose(st["qnorm_max"], ref["qnorm_max"], rtol=1e-12)
    np.testing.assert_allclose(st["bound"], ref["bound"], rtol=1e-12)
    np.testing.assert_allclose(kbar.cpu().numpy(), ref["kbar"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(mu.cpu().numpy(), ref["mu"], rtol=2e-7, atol=1e-7)
    return mu, cert, ref


def assert_same_kernel(a, b, what: str = ""):
    """Outputs of the same kernel on the same head: bitwise equal."""
    import torch
    assert torch.equal(a, b), what


def run_attention(clis, w, host, dev, mu, cert, rows=None, modes=("fixed", "online", "online_lazy", "auto")):
    """Every mode on the device, compared with the oracle (all rows or `rows`)."""
    import torch
    want = oracle.attention(*host, w.dtype, w.scale, w.causal, rows=rows)
    outs = {}
    for m in modes:
        say("attn", m, w.name, w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, "causal" if w.causal else "dense")
        o, route = clis.clis_attn_fwd(*dev, w.scale, w.causal, mode=m, want_route=True)
        torch.cuda.synchronize()
        outs[m] = o
        r = route.cpu().numpy()
        if m == "fixed":
            assert np.all(r == 1)
        elif m in ("online", "online_lazy"):
            assert np.all(r == 0)
        else:
            assert np.array_equal(r, cert.cpu().numpy())
    c = cert.cpu().numpy().astype(bool)
    errs = {}
    ridx = None if rows is None else torch.as_tensor(rows, device=dev[0].device)
    for m, o in outs.items():
        got = to_f64(o if ridx is None else o.index_select(2, ridx))
        # forced-fixed output is only promised on certified heads
        sel = c if m == "fixed" else np.ones_like(c)
        if sel.any():
            errs[m] = assert_close(got[sel], want[sel], w.dtype, f"{w.name}/{m}")
    if "auto" in outs and "fixed" in outs and "online" in outs:
        for b in range(w.B):
            for h in range(w.H):
                ref = outs["fixed"] if c[b, h] else outs["online"]
                assert_same_kernel(outs["auto"][b, h], ref[b, h], what=f"{w.name} auto head {(b, h)}")
    return outs, errs


# ---------------------------------------------------------------- small cases
def test_tiny_fp32_workload_all_rows(clis):
    w = workloads.WORKLOADS["tiny"]
    host, dev = _inputs(w)
    mu, cert, ref = check_certify(clis, w, host, dev)
    assert ref["cert"].all()
    _, errs = run_attention(clis, w, host, dev, mu, cert)
    assert errs["fixed"]["max_abs"] <= 1e-5 and errs["online"]["max_abs"] <= 1e-5


SMALL = [
    # name, B, H, Nq, Nk, d, dtype, causal
    ("bf16_tail_d128", 1, 2, 1000, 1000, 128, "bf16", False),
    ("bf16_tail_d64", 1, 2, 1000, 1000, 64, "bf16", False),
    ("bf16_exact_tiles", 1, 1, 256, 256, 128, "bf16", False),
    ("bf16_causal_tail", 1, 3, 777, 777, 128, "bf16", True),
    ("bf16_causal_d64", 2, 1, 300, 300, 64, "bf16", True),
    # causal work order: an odd head count (a partial group of heads) and an
    # odd number of 256-row query tiles (a partial block of tiles)
    ("bf16_causal_odd_groups", 1, 5, 1200, 1200, 128, "bf16", True),
    ("bf16_cross", 2, 1, 300, 1300, 128, "bf16", False),
    ("bf16_lt_tile", 1, 1, 5, 5, 128, "bf16", False),
    ("bf16_one_key", 1, 2, 70, 1, 128, "bf16", False),
    ("bf16_one_query", 1, 2, 1, 333, 128, "bf16", False),
    ("fp32_tail_d64", 1, 2, 1000, 1000, 64, "fp32", False),
    ("fp32_tail_d128", 1, 2, 1000, 1000, 128, "fp32", False),
    ("fp32_causal", 1, 2, 700, 700, 128, "fp32", True),
    ("fp32_cross", 1, 2, 33, 517, 64, "fp32", False),
    ("fp32_causal_d64", 1, 2, 333, 333, 64, "fp32", True),
    ("fp32_one_key", 1, 2, 40, 1, 64, "fp32", False),
    ("fp32_one_query", 1, 2, 1, 77, 128, "fp32", False),
    # medium tailed fp32 shapes: 4100 = 128 tiles of 32 keys and a 4-key tail
    ("fp32_4100_d64", 1, 2, 4100, 4100, 64, "fp32", False),
    ("fp32_4100_d128_causal", 1, 1, 4100, 4100, 128, "fp32", True),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_shapes_all_rows(clis, case):
    name, B, H, Nq, Nk, d, dtype, causal = case
    w = workloads.custom(name, B, H, Nq, d, dtype, causal, key_bias_std=2.0, Nk=Nk)
    host, dev = _inputs(w, seed=11)
    mu, cert, ref = check_certify(clis, w, host, dev)
    assert ref["cert"].all()
    run_attention(clis, w, host, dev, mu, cert)


def test_mixed_routing_small(clis):
    """A quarter of 40 heads scaled past the cap: flags, routes and per-head
    outputs (auto equals the forced route bitwise, also for the heads past
    the first 32, whose last query tiles the fixed kernel does not split)."""
    w = workloads.custom("mixed_small", 2, 20, 700, 128, "bf16", False, base="mixed")
    host, dev = _inputs(w, seed=3)
    mu, cert, ref = check_certify(clis, w, host, dev)
    fails = set(workloads.failing_heads(w, 3).tolist())
    assert len(fails) == 10 and min(fails) < 32 < max(fails)
    assert {i for i, c in enumerate(ref["cert"].ravel()) if not c} == fails
    run_attention(clis, w, host, dev, mu, cert)


FP32_MIXED = [
    # name, B, H, Nq, Nk, d, causal: short fp32 heads (one-launch certification),
    # ragged and causal, and a longer one (split certification)
    ("fp32_mixed_d64", 1, 8, 256, 256, 64, False),
    ("fp32_mixed_d128_ragged", 2, 4, 77, 300, 128, False),
    ("fp32_mixed_causal", 1, 3, 500, 500, 128, True),
    ("fp32_mixed_16_heads", 1, 16, 512, 512, 64, False),
    ("fp32_mixed_split_cert", 1, 4, 1500, 1500, 64, False),
]


@pytest.mark.parametrize("case", FP32_MIXED, ids=[c[0] for c in FP32_MIXED])
def test_fp32_mixed_routing(clis, case):
    """fp32 with both routes taken.  Every third head is made to fail
    certification the way a conservative certificate does: key 0 becomes 200
    times a channel in which every query is zero, so kappa (and B_h) exceed
    the cap while every logit stays as it was (the new key's logit is exactly
    0) and fp32 keeps its 1e-5 accuracy on the online route.  Routes equal
    clis_certify's flags and the oracle's; every mode matches the oracle; auto
    mode equals the forced route of each head bitwise (the fp32 kernel fuses
    no product into an add by itself, so its online and fixed forms compute
    the same operations in every route); and certifying inside the call gives
    bitwise the outputs and log-sum-exps of a call given clis_certify's
    certificate, in auto and in forced fixed mode."""
    import torch
    name, B, H, Nq, Nk, d, causal = case
    w = workloads.custom(name, B, H, Nq, d, "fp32", causal, Nk=Nk)
    Q, K, V = (a.copy() for a in workloads.make_inputs(w, 21))
    fail = np.arange(B * H) % 3 == 1
    for i in np.flatnonzero(fail):
        b, h = divmod(int(i), H)
        Q[b, h, :, 0] = 0.0
        K[b, h, 0, :] = 0.0
        K[b, h, 0, 0] = 200.0
    host = (Q, K, V)
    dev = tuple(to_device(a, "fp32") for a in host)
    mu, cert, ref = check_certify(clis, w, host, dev)
    assert np.array_equal(ref["cert"].ravel().astype(bool), ~fail)
    run_attention(clis, w, host, dev, mu, cert)
    say("certificate inside the call vs given", name)
    o_in, route_in, lse_in = clis.clis_attn_fwd(*dev, w.scale, causal, mode="auto", want_route=True,
                                                want_lse=True)
    o_giv, route_giv, lse_giv = clis.clis_attn_fwd(*dev, w.scale, causal, mode="auto", mu=mu, cert=cert,
                                                   want_route=True, want_lse=True)
    f_in = clis.clis_attn_fwd(*dev, w.scale, causal, mode="fixed")
    f_giv = clis.clis_attn_fwd(*dev, w.scale, causal, mode="fixed", mu=mu)
    torch.cuda.synchronize()
    assert torch.equal(route_in, cert) and torch.equal(route_giv, cert)
    assert torch.equal(o_in, o_giv) and torch.equal(lse_in, lse_giv)
    # forced fixed on the failing heads is not promised finite: compare with
    # NaN and Inf mapped to numbers, so that their positions must agree too
    assert torch.equal(torch.nan_to_num(f_in), torch.nan_to_num(f_giv))


def test_caller_supplied_certificate_is_used(clis):
    """mu/cert passed in: same result as letting the call certify itself."""
    import torch
    w = workloads.custom("given_cert", 1, 4, 600, 128, "bf16", False, base="mixed")
    _, dev = _inputs(w, seed=5)
    mu, cert = clis.clis_certify(*dev, w.scale)
    a = clis.clis_attn_fwd(*dev, w.scale, mode="auto", mu=mu, cert=cert)
    b = clis.clis_attn_fwd(*dev, w.scale, mode="auto")
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    # flipping the flags the caller passes flips the routes
    flipped = 1 - cert
    c, route = clis.clis_attn_fwd(*dev, w.scale, mode="auto", mu=mu, cert=flipped, want_route=True)
    torch.cuda.synchronize()
    assert torch.equal(route, flipped)


def test_online_entry_point_equals_online_mode(clis):
    import torch
    for causal in (False, True):
        w = workloads.custom("online_eq", 1, 3, 500, 128, "bf16", causal)
        _, dev = _inputs(w, seed=7)
        a = clis.online_attn_fwd(*dev, w.scale, causal)
        b = clis.clis_attn_fwd(*dev, w.scale, causal, mode="online")
        c = clis.clis_attn_fwd(*dev, w.scale, causal, mode="online", want_route=True)[0]
        torch.cuda.synchronize()
        assert torch.equal(a, b) and torch.equal(a, c)


def test_bitwise_reproducible(clis):
    import torch
    w = workloads.custom("repro", 1, 2, 900, 128, "bf16", False)
    _, dev = _inputs(w, seed=8)
    runs = [clis.clis_attn_fwd(*dev, w.scale, mode="auto") for _ in range(3)]
    cs = [clis.clis_certify(*dev, w.scale) for _ in range(2)]
    torch.cuda.synchronize()
    assert all(torch.equal(runs[0], r) for r in runs[1:])
    assert torch.equal(cs[0][0], cs[1][0]) and torch.equal(cs[0][1], cs[1][1])


def test_non_finite_input_never_certifies(clis):
    """A NaN key makes its head uncertified; the online fallback propagates
    NaN like standard attention, and other heads are untouched."""
    import torch
    w = workloads.custom("nan", 1, 3, 200, 128, "bf16", False)
    (Q, K, V), _ = _inputs(w, seed=9)
    K = K.copy()
    K[0, 1, 17, 5] = 0x7FC0  # bf16 quiet NaN
    dev = tuple(to_device(a, w.dtype) for a in (Q, K, V))
    mu, cert = clis.clis_certify(*dev, w.scale)
    o = clis.clis_attn_fwd(*dev, w.scale, mode="auto")
    torch.cuda.synchronize()
    assert cert.cpu().numpy().tolist() == [[1, 0, 1]]
    got = to_f64(o)
    assert np.all(np.isnan(got[0, 1]))
    want = oracle.attention(Q, K, V, w.dtype, w.scale)
    assert np.all(np.isnan(want[0, 1]))
    for h in (0, 2):
        assert_close(got[0, h], want[0, h], "bf16", f"nan/head{h}")


def test_certification_inside_the_call_matches_clis_certify(clis):
    """Auto mode without a certificate certifies inside the call, taking max |V|
    from the V transpose pass instead of reading V again: its routes equal
    clis_certify's flags and the oracle's, with NaN, +Inf, the largest finite
    bf16 and a large ordinary value planted in V."""
    import torch
    w = workloads.custom("vmax", 1, 5, 300, 128, "bf16", False)
    (Q, K, V), _ = _inputs(w, seed=13)
    V = V.copy()
    V[0, 1, 7, 3] = 0x7FC0      # NaN
    V[0, 2, 250, 100] = 0x7F80  # +Inf
    V[0, 3, 0, 0] = 0xFF7F      # -3.39e38: G = 128
    V[0, 4, 299, 127] = workloads.round_to_bf16_bits(np.array([1000.0], dtype=np.float32))[0]
    dev = tuple(to_device(a, w.dtype) for a in (Q, K, V))
    mu, cert = clis.clis_certify(*dev, w.scale)
    _, route = clis.clis_attn_fwd(*dev, w.scale, mode="auto", want_route=True)
    torch.cuda.synchronize()
    ref = oracle.certify(Q, K, V, w.dtype, w.scale)["cert"]
    assert ref.tolist() == [[1, 0, 0, 0, 1]]
    assert np.array_equal(cert.cpu().numpy(), ref)
    assert np.array_equal(route.cpu().numpy(), ref)


def test_certified_head_near_the_cap_stays_finite(clis):
    """A head whose bound sits just under C, with one query aligned to one
    outlying key so the largest exp2 argument nearly reaches the bound."""
    import torch
    d, n = 128, 700
    rng = np.random.default_rng(12)
    q = rng.standard_normal((n, d)).astype(np.float32)
    k = rng.standard_normal((n, d)).astype(np.float32)
    v = rng.standard_normal((n, d)).astype(np.float32)
    k[3] = 0.0
    k[3, 0] = 40.0
    scale = float(np.float32(1 / math.sqrt(d)))  # the fp32 value the library receives
    host0 = tuple(workloads.round_to_bf16_bits(a)[None, None] for a in (q, k, v))
    base = oracle.certify(*host0, "bf16", scale)
    # put q row 0 along e1 with the largest norm, sized so B_h ~ (1 - 1e-2) C
    # (bf16 rounding of that row moves the bound by < 0.4%)
    c2 = scale * math.log2(math.e)
    target = (1 - 1e-2) * base["C"][0, 0] / (c2 * base["kappa"][0, 0])
    q[0] = 0.0
    q[0, 0] = target
    host = tuple(workloads.round_to_bf16_bits(a)[None, None] for a in (q, k, v))
    dev = tuple(to_device(a, "bf16") for a in host)
    w = workloads.custom("near_cap", 1, 1, n, d, "bf16", False)
    mu, cert, ref = check_certify(clis, w, host, dev)
    assert ref["cert"][0, 0] == 1 and ref["bound"][0, 0] > 0.98 * ref["C"][0, 0]
    qd = oracle.decode(host[0][0, 0], "bf16")
    kd = oracle.decode(host[1][0, 0], "bf16")
    _, mx, _ = oracle.fixed_mu_head(qd, kd, oracle.decode(host[2][0, 0], "bf16"), scale, ref["mu"][0, 0],
                                    rows=np.array([0]))
    assert mx[0] > 0.9 * ref["C"][0, 0]
    want = oracle.attention(*host, "bf16", scale)
    for mode in ("fixed", "auto"):
        o = clis.clis_attn_fwd(*dev, scale, mode=mode, mu=mu, cert=cert)
        o2 = clis.clis_attn_fwd(*dev, scale, mode=mode)
        torch.cuda.synchronize()
        for out in (o, o2):
            got = to_f64(out)
            assert_valid(got, f"near_cap/{mode}")
            assert_close(got, want, "bf16", f"near_cap/{mode}")


@pytest.mark.parametrize("kind", workloads.EDGE_HEADS)
def test_edge_heads_near_the_cap(clis, kind):
    """Certified heads whose bound sits just under the cap: a large shared
    key offset (the case the key-mean centering exists for) and two competing
    keys near the bound with values of opposite sign (output sensitive to any
    exponent error), with and without an offset the query row sees.  Auto
    and fixed mode, certificate computed inside the call or given, and the
    log-sum-exp form: valid and within the bf16 tolerances of the oracle."""
    import torch
    q, k, v = workloads.edge_head(kind)
    host = tuple(workloads.round_to_bf16_bits(a)[None, None] for a in (q, k, v))
    dev = tuple(to_device(a, "bf16") for a in host)
    w = workloads.custom(kind, 1, 1, q.shape[0], q.shape[1], "bf16", False, Nk=k.shape[0])
    mu, cert, ref = check_certify(clis, w, host, dev)
    assert ref["cert"][0, 0] == 1 and ref["bound"][0, 0] > 0.95 * ref["C"][0, 0]
    want = oracle.attention(*host, "bf16", w.scale)
    want_lse = oracle.lse_head(*(oracle.decode(a[0, 0], "bf16") for a in host[:2]), w.scale)
    for mode, given in (("auto", False), ("fixed", False), ("auto", True), ("fixed", True)):
        say("edge head", kind, mode, "given certificate" if given else "certified in the call")
        kw = dict(mu=mu, cert=cert) if given else {}
        o, route, lse = clis.clis_attn_fwd(*dev, w.scale, mode=mode, want_route=True, want_lse=True, **kw)
        o2 = clis.clis_attn_fwd(*dev, w.scale, mode=mode, **kw)
        torch.cuda.synchronize()
        assert route.item() == 1
        for out in (o, o2):
            got = to_f64(out)
            assert_valid(got, f"{kind}/{mode}")
            assert_close(got, want, "bf16", f"{kind}/{mode}")
        got_lse = lse.cpu().numpy().astype(np.float64)[0, 0]
        assert np.all(np.isfinite(got_lse)) and np.abs(got_lse - want_lse).max() <= 4e-3, kind


def test_forced_fixed_on_failing_head_is_invalid(clis):
    """Why certification exists: the fixed stabilizer on a head far past the
    cap overflows (NaN/Inf), while auto mode routes it online and is valid."""
    import torch
    w = workloads.custom("force_fail", 1, 1, 512, 128, "bf16", False, fail_frac=1.0, fail_qk_scale=40.0,
                         outlier_frac=0.01, outlier_scale=200.0)
    host, dev = _inputs(w, seed=4)
    mu, cert = clis.clis_certify(*dev, w.scale)
    o_fixed = clis.clis_attn_fwd(*dev, w.scale, mode="fixed", mu=mu)
    o_auto = clis.clis_attn_fwd(*dev, w.scale, mode="auto")
    torch.cuda.synchronize()
    assert cert.item() == 0
    assert not np.all(np.isfinite(to_f64(o_fixed)))
    assert_valid(to_f64(o_auto), "force_fail/auto")


def test_empty_and_errors_through_binding(clis):
    import torch
    q = torch.zeros((0, 2, 10, 128), dtype=torch.bfloat16, device="cuda")
    o = clis.clis_attn_fwd(q, q, q)
    assert o.shape == q.shape
    x = torch.zeros((1, 1, 16, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(clis.ClisError) as e:
        clis.clis_attn_fwd(x, x, x)
    assert e.value.status == 3


# ---------------------------------------------------------------- full sizes
FULL = ["wan720p", "wan480p", "mixed", "causal"]


def extreme_rows(q, k, keys, n):
    """Query rows of one head whose largest logits are largest, and rows whose
    two largest logits are closest (near ties), among the key rows `keys`
    (q, k fp64 [N, d]): two sorted arrays of n rows each."""
    s = q @ k[keys].T
    top = np.sort(s, axis=1)[:, -2:]
    big = np.argsort(-top[:, 1], kind="stable")[:n]
    tie = np.argsort(top[:, 1] - top[:, 0], kind="stable")[:n]
    return np.sort(big).astype(np.int64), np.sort(tie).astype(np.int64)


@pytest.mark.parametrize("name", FULL)
def test_full_size_workload(clis, name):
    """Full-size inputs: certification on every head, attention in every mode
    on sampled rows of every head (both ends, edges of 64-, 128- and 256-row
    tiles, 200 seeded rows), at the stated bf16 tolerances.  On the mixed
    workload also, in auto mode (the online route), the 50 rows of each
    failing head with the largest logits (stated tolerances) and the 50 rows
    whose two largest logits are closest.  Those near-tie rows have logits
    of ~3.6e6, where one fp32 ulp of a score is 0.25 (0.03 in log2 units after
    the scale): the fp32 accumulation of the score product moves the weights
    of two nearly tied keys by a few percent against the fp64 oracle, which
    no fp32-accumulating kernel avoids.  They are checked for validity and at
    the stated mean and rel-L2 tolerances; their largest element error is
    reported (printed with the case), not asserted."""
    w = workloads.WORKLOADS[name]
    say("generate", name)
    host, dev = _inputs(w, seed=0)
    mu, cert, ref = check_certify(clis, w, host, dev)
    fails = workloads.failing_heads(w, 0)
    assert {i for i, c in enumerate(ref["cert"].ravel()) if not c} == set(fails.tolist())
    rows = workloads.sample_rows(w, n_random=200, tiles=(64, 128, 256))
    outs, errs = run_attention(clis, w, host, dev, mu, cert, rows=rows)
    say("errors", name, len(rows), "rows per head", errs)
    import torch
    auto = outs["auto"]
    assert bool(torch.isfinite(auto).all()) and bool((auto != 0).any()), f"{name}: invalid output"
    for flat in fails.tolist():
        b, h = divmod(flat, w.H)
        qd, kd, vd = (oracle.decode(a[b, h], w.dtype) for a in host)
        big, tie = extreme_rows(qd, kd, workloads.outlier_rows(w, b, h, 0), 50)
        for kind, er in (("largest logits", big), ("near ties", tie)):
            want = oracle.attention_head(qd, kd, vd, w.scale, w.causal, er)
            got = to_f64(auto[b, h].index_select(0, torch.as_tensor(er, device=auto.device)))
            e = errors(got, want)
            say("extreme rows", name, (b, h), kind, len(er), e)
            assert np.all(np.isfinite(got)), f"{name} {(b, h)} {kind}: non-finite output"
            if kind == "largest logits":
                assert_close(got, want, w.dtype, f"{name} failing head {(b, h)} {kind}")
            else:
                assert e["mean_abs"] <= 1e-3 and e["rel_l2"] <= 5e-3, (name, (b, h), kind, e)


# ---------------------------------------------------------------- maximum size
def test_max_keys_uniform_weights(clis):
    """The largest key count the ABI accepts at d=128 (one head's V^T just
    under 2 GiB): with Q = 0 every score is 0, the certificate gives B_h = 0
    and mu = 0, every weight is exactly 1, and each output row is the mean of
    V over the keys (computed here in fp64 from the same bytes)."""
    import torch
    d = 128
    nk = (0x7FFFFFFF // (2 * d)) // 128 * 128  # vt_pad(Nk) * d * 2 < 2 GiB
    while nk * d * 2 >= 0x7FFFFFFF:
        nk -= 128
    nq = 300
    say("max keys", nk, "x", d, "bf16")
    rng = np.random.default_rng(77)
    v_bits = np.empty((nk, d), dtype=np.uint16)
    k_bits = np.empty((nk, d), dtype=np.uint16)
    mean = np.zeros(d, dtype=np.float64)
    step = 1 << 20
    for a in range(0, nk, step):
        b = min(nk, a + step)
        v_bits[a:b] = workloads.round_to_bf16_bits(rng.standard_normal((b - a, d), dtype=np.float32))
        k_bits[a:b] = workloads.round_to_bf16_bits(rng.standard_normal((b - a, d), dtype=np.float32))
        mean += workloads.bf16_bits_to_f32(v_bits[a:b]).astype(np.float64).sum(axis=0)
    mean /= nk
    q = torch.zeros((1, 1, nq, d), dtype=torch.bfloat16, device="cuda")
    k = workloads.to_torch(k_bits.reshape(1, 1, nk, d), "bf16")
    v = workloads.to_torch(v_bits.reshape(1, 1, nk, d), "bf16")
    del k_bits, v_bits
    mu, cert, stats, _ = clis.clis_certify(q, k, v, 1.0 / math.sqrt(d), want_stats=True)
    o = clis.clis_attn_fwd(q, k, v, 1.0 / math.sqrt(d), mode="auto", mu=mu, cert=cert)
    torch.cuda.synchronize()
    st = clis.decode_stats(stats)[0]
    assert int(cert.item()) == 1 and st["bound"] == 0.0 and st["L"] == math.ceil(math.log2(nk))
    assert not mu.any()
    got = to_f64(o)[0, 0]
    # fp32 sums of exact weights, then one bf16 rounding of |mean| < 1e-2
    np.testing.assert_allclose(got, np.broadcast_to(mean, got.shape), rtol=0, atol=2e-5)


# ---------------------------------------------------------------- many heads
@pytest.mark.parametrize("dtype,d,fail_scale", [("bf16", 64, 4.0), ("bf16", 128, 4.0), ("fp32", 128, 1.0)])
def test_many_heads_beyond_a_grid_dimension(clis, dtype, d, fail_scale):
    """66,000 (batch, head) pairs, more than a launch grid's second dimension
    holds: certification, the V transpose and attention index heads along
    one-dimensional grids.  In the bf16 case every fourth head has Q and K
    scaled x4, which multiplies its bound by 16 (bound / C >= 1.09 over all
    such heads, <= 0.14 over the others), so every head's flag is known and
    both routes run; the fp32 case keeps every head certified (its 1e-5
    bound assumes well-conditioned logits, and failing heads have large
    ones).  Flags and routes are checked on all heads, certification and
    every mode against the oracle on 400 sampled heads (the first and last
    100).  V ~ N(0, 1/16): with 4 keys a row is an average of few values, and
    at |o| ~ 1 the bf16 store alone would cost ~1e-3 mean abs error (a quarter
    ulp); at this scale outputs are as small as the long-sequence workloads',
    for which the absolute bounds are stated (rel L2 is scale-free)."""
    import torch
    B, H, N = 2, 33000, 4
    BH = B * H
    scale = 1.0 / math.sqrt(d)
    rng = np.random.default_rng(4242)
    q = rng.standard_normal((BH, N, d), dtype=np.float32)
    k = rng.standard_normal((BH, N, d), dtype=np.float32) + 2.0 * rng.standard_normal((BH, 1, d), dtype=np.float32)
    v = 0.25 * rng.standard_normal((BH, N, d), dtype=np.float32)
    fail = ((np.arange(BH) % 4) == 3) & (fail_scale != 1.0)
    q[fail] *= fail_scale
    k[fail] *= fail_scale
    host = [x.reshape(B, H, N, d) for x in (q, k, v)]
    if dtype == "bf16":
        host = [workloads.round_to_bf16_bits(x) for x in host]
    dev = [to_device(x, dtype) for x in host]
    say("many heads", dtype, B, H, N, d)
    mu, cert = clis.clis_certify(*dev, scale)
    torch.cuda.synchronize()
    expect = (~fail).astype(np.int32).reshape(B, H)
    assert np.array_equal(cert.cpu().numpy(), expect)

    pick = np.unique(np.concatenate([np.arange(100), np.arange(BH - 100, BH),
                                     np.random.default_rng(7).choice(BH, 200, replace=False)]))
    sub = [x.reshape(BH, N, d)[pick].reshape(1, len(pick), N, d) for x in host]
    ref = oracle.certify(*sub, dtype, scale)
    assert np.array_equal(ref["cert"].ravel(), expect.ravel()[pick])
    np.testing.assert_allclose(mu.reshape(BH, N).cpu().numpy()[pick], ref["mu"][0], rtol=2e-7, atol=1e-7)
    want = oracle.attention(*sub, dtype, scale)[0]
    for m in ("fixed", "online", "online_lazy", "auto"):
        say("many heads", dtype, "mode", m)
        o, route = clis.clis_attn_fwd(*dev, scale, mode=m, want_route=True)
        torch.cuda.synchronize()
        r = route.cpu().numpy()
        assert np.array_equal(r, expect if m == "auto" else np.full_like(expect, int(m == "fixed")))
        got = to_f64(o).reshape(BH, N, d)[pick]
        sel = ~fail[pick] if m == "fixed" else np.ones(len(pick), dtype=bool)  # forced fixed: certified heads only
        assert_close(got[sel], want[sel], dtype, f"many heads {dtype}/{m}")
