"""Pins for the fp64 oracle (CPU only).

Each check ties the oracle to something other than itself: hand-worked
closed forms and fixtures under tests/golden/, an independent pure-Python
brute force on tiny inputs, invariants of softmax attention, exact scaling
laws of the certification statistics, and the safety promise of the
certificate.  ``PINS`` lists them so that tests/test_oracle_mutations.py can
plant mistakes in a copy of oracle.c and show that some pin catches each one.

Pages: "CLiS: Plug-and-Play Attention Acceleration for Video Diffusion on
TPUs via Certified Stabilization" -- abstract, Algorithm 1, Figure 3,
Figure 5(a).
"""
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
LOG2E = 1.4426950408889634


def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append(line.split())
    return rows


def _rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------ brute force
def _brute_row(q, k, v, i, scale, causal):
    """Pure-Python softmax attention for one row, with no stabilizer."""
    n = i + 1 if causal else len(k)
    e = [math.exp(scale * math.fsum(q[i][c] * k[j][c] for c in range(len(q[i])))) for j in range(n)]
    z = math.fsum(e)
    return [math.fsum(e[j] * v[j][c] for j in range(n)) / z for c in range(len(v[0]))]


def pin_brute_force():
    rng = _rng(1)
    for nq in (1, 2, 3, 5, 8):
        for nk in (1, 2, 3, 5, 8):
            for d in (1, 2, 4):
                for causal in (False, True):
                    if causal and nq != nk:
                        continue
                    q, k, v = (rng.standard_normal((n, d)) for n in (nq, nk, nk))
                    scale = 0.7
                    got = oracle.attention_head(q, k, v, scale, causal, threads=1)
                    want = np.array([_brute_row(q.tolist(), k.tolist(), v.tolist(), i, scale, causal)
                                     for i in range(nq)])
                    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)


# ------------------------------------------------------------ closed forms
def pin_closed_forms():
    rng = _rng(2)
    # one key: every row returns that key's value exactly
    q, k, v = rng.standard_normal((5, 4)), rng.standard_normal((1, 4)), rng.standard_normal((1, 4))
    assert np.array_equal(oracle.attention_head(q, k, v, 0.5), np.repeat(v, 5, axis=0))
    # all-zero queries, or identical keys: uniform weights, the mean of V
    k = rng.standard_normal((7, 4))
    v = rng.standard_normal((7, 4))
    np.testing.assert_allclose(oracle.attention_head(np.zeros((3, 4)), k, v, 0.5),
                               np.repeat(v.mean(0, keepdims=True), 3, 0), atol=1e-14)
    kk = np.repeat(rng.standard_normal((1, 4)), 7, axis=0)
    np.testing.assert_allclose(oracle.attention_head(q, kk, v, 0.5),
                               np.repeat(v.mean(0, keepdims=True), 5, 0), atol=1e-14)
    # causal row 0 sees only key 0
    q, k, v = (rng.standard_normal((6, 3)) for _ in range(3))
    np.testing.assert_array_equal(oracle.attention_head(q, k, v, 0.5, causal=True)[0], v[0])
    # two keys with logits 0 and ln 3: weights 1/4, 3/4 -> 4/4 + 3*8/4 = 7
    o = oracle.attention_head(np.array([[1.0]]), np.array([[0.0], [math.log(3.0)]]),
                              np.array([[4.0], [8.0]]), 1.0)
    assert abs(o[0, 0] - 7.0) < 1e-14


# ------------------------------------------------------------ invariants
def pin_invariants():
    rng = _rng(3)
    nq, nk, d = 9, 13, 6
    q, k, v = rng.standard_normal((nq, d)), rng.standard_normal((nk, d)), rng.standard_normal((nk, d))
    scale = 0.9
    for causal in (False, True):
        kk, vv = (k[:nq], v[:nq]) if causal else (k, v)
        o = oracle.attention_head(q, kk, vv, scale, causal)
        # shifting every key by the same vector adds a per-row constant to the logits
        u = rng.standard_normal(d) * 3
        np.testing.assert_allclose(oracle.attention_head(q, kk + u, vv, scale, causal), o, atol=1e-12)
        # convex combination of the visible value rows
        for i in range(nq):
            vis = vv[: i + 1] if causal else vv
            assert np.all(o[i] >= vis.min(0) - 1e-12) and np.all(o[i] <= vis.max(0) + 1e-12)
        # affine in V: V -> aV + 1b^T gives O -> aO + 1b^T
        a, bvec = -1.7, rng.standard_normal(d)
        np.testing.assert_allclose(oracle.attention_head(q, kk, a * vv + bvec, scale, causal),
                                   a * o + bvec, atol=1e-12)
        # permuting query rows permutes output rows (dense); row order is free
        perm = rng.permutation(nq)
        if not causal:
            np.testing.assert_allclose(oracle.attention_head(q[perm], kk, vv, scale), o[perm], atol=1e-15)
    # permuting keys and values together changes nothing (dense)
    o = oracle.attention_head(q, k, v, scale)
    perm = rng.permutation(nk)
    np.testing.assert_allclose(oracle.attention_head(q, k[perm], v[perm], scale), o, atol=1e-12)


def pin_weights_sum_to_one():
    # with V = identity the output rows are the softmax weights themselves
    # (head dim = number of keys, since Q, K and V share one head dim)
    rng = _rng(4)
    nk = 11
    q, k = rng.standard_normal((5, nk)), rng.standard_normal((nk, nk))
    for causal in (False,):
        w = oracle.attention_head(q, k, np.eye(nk), 1.3, causal)
        assert np.all(w >= 0)
        np.testing.assert_allclose(w.sum(1), 1.0, atol=1e-14)
        # and each weight's log-ratio to weight 0 is the logit difference
        s = 1.3 * q @ k.T
        np.testing.assert_allclose(np.log(w / w[:, :1]), s - s[:, :1], atol=1e-12)


def pin_other_evaluations_agree():
    """The fixed-stabilizer and online (eager and lazy-rescale) evaluations
    give the definition's output."""
    rng = _rng(5)
    nq, nk, d = 17, 40, 8
    q = rng.standard_normal((nq, d))
    k = rng.standard_normal((nk, d)) + 3 * rng.standard_normal(d)
    v = rng.standard_normal((nk, d))
    scale = 1 / math.sqrt(d)
    for causal in (False, True):
        kk, vv = (k[:nq], v[:nq]) if causal else (k, v)
        o = oracle.attention_head(q, kk, vv, scale, causal)
        rec = oracle.certify_head(q, kk, vv, scale)
        of, _, _ = oracle.fixed_mu_head(q, kk, vv, scale, rec["mu"], causal)
        np.testing.assert_allclose(of, o, atol=1e-12)
        for block in (1, 3, 16, 64):
            for tau in (0.0, 1.0, 8.0):  # eager, and lazy rescaling at two thresholds
                np.testing.assert_allclose(oracle.online_head(q, kk, vv, scale, causal, block, tau=tau), o,
                                           atol=1e-12)
    # scores growing by ~72 log2 units per key: a stabilizer that stops moving
    # overflows fp64 within a few blocks
    qs, ks = np.ones((3, 1)), (50.0 * np.arange(40.0))[:, None]
    vs = rng.standard_normal((40, 2))
    want = oracle.attention_head(qs, ks, vs, 1.0)
    for tau in (0.0, 8.0):
        for block in (1, 4):
            np.testing.assert_allclose(oracle.online_head(qs, ks, vs, 1.0, False, block, tau=tau), want, atol=1e-12)


# ------------------------------------------------------------ certification
def _expected_limits():
    out = {}
    for fmt, p, emax, fl in _golden("exp2_limits.txt"):
        mx = (2.0 - 2.0 ** (1 - int(p))) * 2.0 ** int(emax)
        assert math.floor(math.log2(mx)) == int(fl)
        out[fmt] = math.log2(mx)
    return out


def pin_cert_constants():
    lim = _expected_limits()
    rng = _rng(6)
    for nk, vmax, L, G, A, C in _golden("cert_constants.txt"):
        nk, vmax = int(nk), float(vmax)
        d = 4
        v = rng.uniform(-0.2, 0.2, size=(nk, d))
        v[rng.integers(nk), rng.integers(d)] = -vmax
        k = rng.standard_normal((nk, d))
        q = rng.standard_normal((3, d))
        rec = oracle.certify_head(q, k, v, 0.5, p_bf16=True)
        assert (rec["L"], rec["G"], rec["A"], rec["C"]) == (int(L), int(G), int(A), int(C)), (nk, vmax, rec)
        assert rec["maxabs_v"] == vmax
        assert rec["u_exp"] == lim["bf16"] and rec["u_acc"] == lim["fp32"]
        rec32 = oracle.certify_head(q, k, v, 0.5, p_bf16=False)
        assert rec32["u_exp"] == lim["fp32"] and rec32["C"] == int(C)


def pin_cert_closed_forms():
    rng = _rng(7)
    d = 6
    # identical keys: kappa = 0, so the bound is 0 and the head certifies
    # (short dyadic values keep the key sum, and so the mean, exact)
    k = np.repeat(rng.integers(-100, 100, size=(1, d)) / 64.0, 10, 0)
    q, v = rng.standard_normal((4, d)) * 50, rng.standard_normal((10, d))
    rec = oracle.certify_head(q, k, v, 1.0)
    assert rec["kappa"] == 0.0 and rec["bound"] == 0.0 and rec["cert"] == 1
    np.testing.assert_allclose(rec["kbar"], k[0], rtol=1e-15)
    # two keys: kbar is their midpoint and kappa half their distance
    k2 = rng.standard_normal((2, d))
    rec = oracle.certify_head(q, k2, v[:2], 1.0)
    np.testing.assert_allclose(rec["kbar"], k2.mean(0), atol=1e-15)
    assert abs(rec["kappa"] - np.linalg.norm(k2[0] - k2[1]) / 2) < 1e-14
    # B_h = scale*log2(e) * max_r ||q_r|| * kappa
    qn = max(math.sqrt(math.fsum(x * x for x in row)) for row in q.tolist())
    assert abs(rec["qnorm_max"] - qn) < 1e-12
    assert abs(rec["bound"] - LOG2E * qn * rec["kappa"]) <= 1e-12 * rec["bound"]


def pin_cert_scaling_laws():
    rng = _rng(8)
    nk, d = 50, 8
    q = rng.standard_normal((20, d))
    k = rng.standard_normal((nk, d)) + 2 * rng.standard_normal(d)
    v = rng.standard_normal((nk, d)) * 3
    base = oracle.certify_head(q, k, v, 1 / math.sqrt(d))
    for t in (-3, 1, 5):
        # power-of-two scaling of Q is exact all the way to the bound
        r = oracle.certify_head(q * 2.0 ** t, k, v, 1 / math.sqrt(d))
        assert r["bound"] == base["bound"] * 2.0 ** t
        assert r["kappa"] == base["kappa"]
        # V -> 2^t V moves G by t (max|V| >= 1 here), and C by -t
        r = oracle.certify_head(q, k, v * 2.0 ** t, 1 / math.sqrt(d))
        if base["maxabs_v"] * 2.0 ** t >= 1:
            assert r["G"] == base["G"] + t and r["C"] == base["C"] - t
    # shifting all keys moves kbar and leaves kappa unchanged
    u = rng.standard_normal(d) * 10
    r = oracle.certify_head(q, k + u, v, 1 / math.sqrt(d))
    np.testing.assert_allclose(r["kbar"], base["kbar"] + u, atol=1e-12)
    assert abs(r["kappa"] - base["kappa"]) < 1e-12
    # mu_i is the mean over keys of row i's exp2 arguments c*q_i.k_j
    c = LOG2E / math.sqrt(d)
    x = c * (q @ k.T)
    np.testing.assert_allclose(base["mu"], x.mean(1), atol=1e-12)


def pin_flag_flips():
    """The flag flips exactly where the scaled bound crosses C."""
    rng = _rng(9)
    nk, d = 64, 8
    q = rng.standard_normal((16, d))
    k = rng.standard_normal((nk, d)) + rng.standard_normal(d)
    v = rng.standard_normal((nk, d))
    scale = 1 / math.sqrt(d)
    base = oracle.certify_head(q, k, v, scale)
    assert base["cert"] == 1
    a_star = base["C"] / base["bound"]
    assert oracle.certify_head(q * a_star * (1 - 1e-9), k, v, scale)["cert"] == 1
    assert oracle.certify_head(q * a_star * (1 + 1e-9), k, v, scale)["cert"] == 0
    # scaling Q and K together scales the bound quadratically
    r = math.sqrt(a_star)
    assert oracle.certify_head(q * r * (1 - 1e-9), k * r * (1 - 1e-9), v, scale)["cert"] == 1
    assert oracle.certify_head(q * r * (1 + 1e-9), k * r * (1 + 1e-9), v, scale)["cert"] == 0
    # larger values lower C: at 2^t V with C - t < B the head fails
    assert base["maxabs_v"] >= 1
    t = int(math.floor(base["C"] - base["bound"])) + 1
    assert oracle.certify_head(q, k, v * 2.0 ** t, scale)["cert"] == 0
    assert oracle.certify_head(q, k, v * 2.0 ** (t - 1), scale)["cert"] == 1
    # non-finite inputs never certify
    for bad in (np.nan, np.inf):
        qb = q.copy(); qb[3, 2] = bad
        assert oracle.certify_head(qb, k, v, scale)["cert"] == 0
        vb = v.copy(); vb[5, 1] = bad
        assert oracle.certify_head(q, k, vb, scale)["cert"] == 0


def pin_certificate_is_safe():
    """A certified head keeps every exp2 argument <= B_h <= C and every
    accumulator below 2^127 on the fixed-stabilizer evaluation."""
    rng = _rng(10)
    nk, d = 300, 16
    scale = 1 / math.sqrt(d)
    q = rng.standard_normal((40, d)) * 2.5
    k = rng.standard_normal((nk, d)) * 2.5 + 4 * rng.standard_normal(d)
    v = rng.standard_normal((nk, d))
    rec = oracle.certify_head(q, k, v, scale)
    assert rec["cert"] == 1
    _, mx, ma = oracle.fixed_mu_head(q, k, v, scale, rec["mu"])
    assert np.all(mx <= rec["bound"] + 1e-9) and np.all(mx >= 0.0)
    assert np.all(ma <= 2.0 ** 127)
    # Cauchy-Schwarz-tight instance: one query along e1 and one key at
    # kbar + kappa*e1 (the rest balanced) make the largest argument equal B_h
    kt = np.zeros((4, d))
    kt[0, 0], kt[1, 0], kt[2, 1], kt[3, 1] = 5.0, -5.0, 3.0, -3.0
    qt = np.zeros((1, d)); qt[0, 0] = 2.0
    rec = oracle.certify_head(qt, kt, np.ones((4, d)), 1.0)
    _, mx, _ = oracle.fixed_mu_head(qt, kt, np.ones((4, d)), 1.0, rec["mu"])
    assert abs(mx[0] - rec["bound"]) < 1e-12 and abs(rec["bound"] - LOG2E * 2 * 5) < 1e-12


# ------------------------------------------------------------ log-sum-exp
def _brute_lse(q, k, i, scale, causal):
    """Pure-Python ln sum_j exp(s_j) for one row, with no shift."""
    n = i + 1 if causal else len(k)
    return math.log(math.fsum(math.exp(scale * math.fsum(a * b for a, b in zip(q[i], k[j]))) for j in range(n)))


def pin_lse():
    rng = _rng(11)
    for nq, nk, d, causal in [(1, 1, 1, False), (3, 5, 2, False), (4, 4, 3, True), (6, 2, 4, False),
                              (5, 5, 1, True)]:
        q, k = rng.standard_normal((nq, d)), rng.standard_normal((nk, d))
        got = oracle.lse_head(q, k, 0.9, causal, threads=1)
        want = [_brute_lse(q.tolist(), k.tolist(), i, 0.9, causal) for i in range(nq)]
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)
    # identical keys: lse_i = scale q_i.k + ln(number of visible keys)
    q = rng.standard_normal((6, 3))
    kk = np.tile(rng.standard_normal((1, 3)), (6, 1))
    for causal in (False, True):
        got = oracle.lse_head(q, kk, 0.5, causal, threads=1)
        n = np.arange(1, 7) if causal else np.full(6, 6)
        np.testing.assert_allclose(got, 0.5 * q @ kk[0] + np.log(n), rtol=0, atol=1e-13)
    # scores far beyond exp's range: two keys at 1000, one at 0 -> 1000 + ln 2
    got = oracle.lse_head(np.array([[1000.0]]), np.array([[1.0], [1.0], [0.0]]), 1.0, threads=1)
    assert abs(got[0] - (1000.0 + math.log(2.0))) < 1e-12


# ------------------------------------------------ fixed-mu partial sums
def pin_partial_sums():
    rng = _rng(12)
    nq, nk, d, scale = 7, 11, 3, 0.8
    q, k, v = (rng.standard_normal((n, d)) for n in (nq, nk, nk))
    mu = rng.standard_normal(nq)
    c2 = scale * LOG2E
    # brute force: pure-Python weights 2^(c q.k - mu) over a key range
    for k0, k1 in [(0, nk), (3, 8), (5, 5), (10, 11)]:
        acc, l = oracle.fixed_mu_partial_head(q, k, v, scale, mu, k0, k1, threads=1)
        for i in range(nq):
            w = [2.0 ** (c2 * math.fsum(q[i, c] * k[j, c] for c in range(d)) - mu[i]) for j in range(k0, k1)]
            assert abs(l[i] - math.fsum(w)) <= 1e-13 * max(1.0, abs(l[i]))
            for c in range(d):
                want = math.fsum(w[t] * v[k0 + t, c] for t in range(len(w)))
                assert abs(acc[i, c] - want) <= 1e-12 * max(1.0, abs(want))
    # disjoint ranges add; the full range normalizes to softmax attention
    parts = [oracle.fixed_mu_partial_head(q, k, v, scale, mu, a, b, threads=1) for a, b in [(0, 4), (4, 9), (9, nk)]]
    full_acc, full_l = oracle.fixed_mu_partial_head(q, k, v, scale, mu, 0, nk, threads=1)
    np.testing.assert_allclose(sum(p[0] for p in parts), full_acc, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(sum(p[1] for p in parts), full_l, rtol=1e-12)
    np.testing.assert_allclose(full_acc / full_l[:, None], oracle.attention_head(q, k, v, scale, threads=1),
                               rtol=0, atol=1e-12)
    # raising mu by an integer scales both sums by 2^-delta
    acc3, l3 = oracle.fixed_mu_partial_head(q, k, v, scale, mu + 3.0, 0, nk, threads=1)
    np.testing.assert_allclose(acc3, full_acc / 8.0, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(l3, full_l / 8.0, rtol=1e-13)
    # causal: row i sees keys 0..i only
    qc, kc, vc = (rng.standard_normal((6, d)) for _ in range(3))
    mc = rng.standard_normal(6)
    for i in range(6):
        a_hi, l_hi = oracle.fixed_mu_partial_head(qc, kc, vc, scale, mc, i + 1, 6, causal=True, rows=[i], threads=1)
        assert l_hi[0] == 0.0 and not a_hi.any()
    a_c, l_c = oracle.fixed_mu_partial_head(qc, kc, vc, scale, mc, 0, 6, causal=True, threads=1)
    np.testing.assert_allclose(a_c / l_c[:, None], oracle.attention_head(qc, kc, vc, scale, True, threads=1),
                               rtol=0, atol=1e-12)
    # with the certified mu, ln 2 (mu + log2 l) is the row's log-sum-exp
    rec = oracle.certify_head(q, k, v, scale, p_bf16=False)
    _, l_mu = oracle.fixed_mu_partial_head(q, k, v, scale, rec["mu"], 0, nk, threads=1)
    np.testing.assert_allclose(math.log(2.0) * (rec["mu"] + np.log2(l_mu)), oracle.lse_head(q, k, scale, threads=1),
                               rtol=0, atol=1e-13)


PINS = [pin_brute_force, pin_closed_forms, pin_invariants, pin_weights_sum_to_one,
        pin_other_evaluations_agree, pin_cert_constants, pin_cert_closed_forms,
        pin_cert_scaling_laws, pin_flag_flips, pin_certificate_is_safe, pin_lse, pin_partial_sums]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_exp2_limits_golden():
    lim = _expected_limits()
    assert math.floor(lim["fp16"]) == 15
    assert 127.99 < lim["bf16"] < 128 and 127.99999 < lim["fp32"] < 128


def test_workload_token_counts():
    import workloads
    for frames, h, w, tokens in _golden("wan_token_counts.txt"):
        assert workloads.latent_tokens(int(frames), int(h), int(w)) == int(tokens)
    assert workloads.WORKLOADS["wan720p"].N == 75600
    assert workloads.WORKLOADS["wan480p"].N == 32760


def test_tiny_workload_full_oracle():
    """The tiny workload end to end: every head certifies, and the fixed and
    online evaluations agree with the definition on every row."""
    import workloads
    w = workloads.WORKLOADS["tiny"]
    Q, K, V = workloads.make_inputs(w, seed=0)
    cert = oracle.certify(Q, K, V, w.dtype, w.scale)
    assert cert["cert"].tolist() == [[1, 1]]
    assert cert["C"].tolist() == [[127 - 8 - cert["G"][0, 0], 127 - 8 - cert["G"][0, 1]]]
    O = oracle.attention(Q, K, V, w.dtype, w.scale)
    for h in range(w.H):
        q, k, v = (oracle.decode(a[0, h], w.dtype) for a in (Q, K, V))
        of, mx, _ = oracle.fixed_mu_head(q, k, v, w.scale, cert["mu"][0, h])
        np.testing.assert_allclose(of, O[0, h], atol=1e-12)
        assert mx.max() <= cert["bound"][0, h] + 1e-9


def test_decode_bf16_exact():
    import workloads
    x = np.array([1.0, -2.5, 3.140625, 1e-3, 65504.0, -0.0], dtype=np.float32)
    bits = workloads.round_to_bf16_bits(x)
    back = oracle.decode(bits, "bf16")
    assert back[0] == 1.0 and back[1] == -2.5 and back[2] == 3.140625
    # round to nearest even at the halfway point: 1 + 2^-8 -> 1, 1 + 3*2^-8 -> 1 + 2^-6
    h = workloads.round_to_bf16_bits(np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8], dtype=np.float32))
    assert oracle.decode(h, "bf16").tolist() == [1.0, 1 + 2 ** -6]
