"""GPU parity of the per-row log-sum-exp output and of key-sharded attention
(clis_attn_fwd_partial + clis_attn_combine), through the C ABI, against the
fp64 oracle on the same seeded inputs.

Log-sum-exp: bf16 inputs within 4e-3 absolute of the oracle (the online row
sums add weights rounded to bf16, each within a relative 2^-9, so ln l is off
by at most about 2^-9 plus the exp2 error; the fixed path adds the fp32
weights), fp32 inputs within 1e-5.  Requesting it leaves every kernel's output
bitwise unchanged.
Key shards: any partition of the keys, in any order, combines to the oracle's
attention within the usual tolerances; with shard edges on 64-key tile edges
the fp32 sums o_acc are bitwise those of a single call over all keys (the
kernel continues from the stored sums in the same order).
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import assert_close, say, to_device, to_f64

pytestmark = pytest.mark.gpu

LSE_TOL = {"bf16": 4e-3, "fp32": 1e-5}


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


def _oracle_lse(w, host, rows=None):
    Q, K, _ = host
    out = np.zeros((w.B, w.H, w.Nq if rows is None else len(rows)))
    for b in range(w.B):
        for h in range(w.H):
            out[b, h] = oracle.lse_head(oracle.decode(Q[b, h], w.dtype), oracle.decode(K[b, h], w.dtype),
                                        w.scale, w.causal, rows=rows)
    return out


LSE_CASES = [
    # name, B, H, Nq, Nk, d, dtype, causal
    ("bf16_tail_d128", 1, 2, 1000, 1000, 128, "bf16", False),
    ("bf16_causal_tail", 1, 3, 777, 777, 128, "bf16", True),
    ("bf16_cross_d64", 2, 1, 300, 1300, 64, "bf16", False),
    ("bf16_causal_d64", 2, 1, 300, 300, 64, "bf16", True),
    ("bf16_one_key", 1, 2, 70, 1, 128, "bf16", False),
    ("fp32_tail_d64", 1, 2, 1000, 1000, 64, "fp32", False),
    ("fp32_causal", 1, 2, 700, 700, 128, "fp32", True),
]


@pytest.mark.parametrize("case", LSE_CASES, ids=[c[0] for c in LSE_CASES])
def test_lse_every_mode(clis, case):
    import torch
    name, B, H, Nq, Nk, d, dtype, causal = case
    w = workloads.custom(name, B, H, Nq, d, dtype, causal, key_bias_std=2.0, Nk=Nk)
    host, dev = _inputs(w, seed=21)
    want = _oracle_lse(w, host)
    want_o = oracle.attention(*host, w.dtype, w.scale, causal)
    mu, cert = clis.clis_certify(*dev, w.scale)
    outs = {}
    for m in ("fixed", "online", "online_lazy", "auto"):
        say("lse", m, name)
        o, lse = clis.clis_attn_fwd(*dev, w.scale, causal, mode=m, mu=mu, cert=cert, want_lse=True)
        plain = clis.clis_attn_fwd(*dev, w.scale, causal, mode=m, mu=mu, cert=cert)
        torch.cuda.synchronize()
        assert torch.equal(o, plain), f"{name}/{m}: asking for lse changed the output"
        assert_close(to_f64(o), want_o, dtype, f"{name}/{m} with lse")
        got = lse.cpu().numpy().astype(np.float64)
        err = float(np.max(np.abs(got - want)))
        assert err <= LSE_TOL[dtype], f"{name}/{m}: lse max abs error {err}"
        outs[m] = lse
    o2, lse2 = clis.online_attn_fwd(*dev, w.scale, causal, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(lse2, outs["online"])
    c = cert.cpu().numpy().astype(bool)
    for b in range(B):
        for h in range(H):
            ref = outs["fixed"] if c[b, h] else outs["online"]
            assert torch.equal(outs["auto"][b, h], ref[b, h]), (b, h)


def test_lse_full_size_sampled_rows(clis):
    """wan720p, auto mode as the benchmark runs it: lse of sampled rows of
    every head against the oracle."""
    import torch
    w = workloads.WORKLOADS["wan720p"]
    say("generate", w.name)
    host, dev = _inputs(w, seed=0)
    rows = workloads.sample_rows(w, n_random=8, tiles=(256,))
    say("lse full size", w.name, len(rows), "rows per head")
    _, lse = clis.clis_attn_fwd(*dev, w.scale, mode="auto", want_lse=True)
    torch.cuda.synchronize()
    got = lse.index_select(2, torch.as_tensor(rows, device=lse.device)).cpu().numpy().astype(np.float64)
    want = _oracle_lse(w, host, rows=rows)
    err = float(np.max(np.abs(got - want)))
    assert err <= LSE_TOL["bf16"], err


# ---------------------------------------------------------------- key shards
def _shards(k, v, edges):
    return [(a, b, k[:, :, a:b].contiguous(), v[:, :, a:b].contiguous()) for a, b in zip(edges[:-1], edges[1:])]


def _run_shards(clis, q, shards, mu, scale, causal, order=None):
    import torch
    B, H, Nq, d = q.shape
    o_acc = torch.empty((B, H, Nq, d), dtype=torch.float32, device=q.device)
    l_acc = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    for i, j in enumerate(order or range(len(shards))):
        a, _, ks, vs = shards[j]
        clis.clis_attn_fwd_partial(q, ks, vs, mu, o_acc, l_acc, scale, causal, kv_offset=a, accumulate=i > 0)
    return o_acc, l_acc


SHARD_CASES = [
    # name, B, H, Nq, Nk, d, dtype, causal, shard edges
    ("bf16_dense", 1, 2, 700, 1000, 128, "bf16", False, [0, 384, 700, 1000]),
    ("bf16_causal", 1, 2, 777, 777, 128, "bf16", True, [0, 256, 300, 777]),
    ("bf16_d64_one_key_shard", 2, 1, 200, 450, 64, "bf16", False, [0, 1, 449, 450]),
    ("bf16_causal_d64", 1, 3, 520, 520, 64, "bf16", True, [0, 64, 200, 520]),
    ("fp32_dense", 1, 2, 300, 500, 64, "fp32", False, [0, 128, 500]),
    ("fp32_causal", 1, 1, 333, 333, 128, "fp32", True, [0, 100, 333]),
]


@pytest.mark.parametrize("case", SHARD_CASES, ids=[c[0] for c in SHARD_CASES])
def test_key_shards_combine_to_attention(clis, case):
    import torch
    name, B, H, Nq, Nk, d, dtype, causal, edges = case
    w = workloads.custom(name, B, H, Nq, d, dtype, causal, key_bias_std=2.0, Nk=Nk)
    host, dev = _inputs(w, seed=31)
    q, k, v = dev
    mu, cert = clis.clis_certify(q, k, v, w.scale)
    torch.cuda.synchronize()
    assert cert.cpu().numpy().all()
    shards = _shards(k, v, edges)
    say("shards", name, edges)
    o_acc, l_acc = _run_shards(clis, q, shards, mu, w.scale, causal)
    o, lse = clis.clis_attn_combine(o_acc, l_acc, dtype=q.dtype, mu=mu, want_lse=True)
    torch.cuda.synchronize()
    want = oracle.attention(*host, w.dtype, w.scale, causal)
    assert_close(to_f64(o), want, dtype, f"{name}/combined")
    err = float(np.max(np.abs(lse.cpu().numpy() - _oracle_lse(w, host))))
    assert err <= LSE_TOL[dtype], err
    # the row sums against the oracle's, with the same stabilizers
    mu64 = mu.cpu().numpy().astype(np.float64)
    for b in range(B):
        for h in range(H):
            qh, kh, vh = (oracle.decode(a[b, h], w.dtype) for a in host)
            _, l_ref = oracle.fixed_mu_partial_head(qh, kh, vh, w.scale, mu64[b, h], 0, Nk, causal)
            np.testing.assert_allclose(l_acc[b, h].cpu().numpy(), l_ref, rtol=4e-3 if dtype == "bf16" else 1e-5)
    # reversed order: the same sums up to fp32 rounding
    o_acc_r, l_acc_r = _run_shards(clis, q, shards, mu, w.scale, causal, order=list(range(len(shards)))[::-1])
    torch.cuda.synchronize()
    np.testing.assert_allclose(l_acc_r.cpu().numpy(), l_acc.cpu().numpy(), rtol=1e-5)
    np.testing.assert_allclose(o_acc_r.cpu().numpy(), o_acc.cpu().numpy(), rtol=1e-4,
                               atol=1e-5 * float(l_acc.abs().max()))
    # combine into fp32 as well
    o32 = clis.clis_attn_combine(o_acc, l_acc, dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close(o32.cpu().numpy().astype(np.float64), want, dtype, f"{name}/combined fp32")


def test_tile_aligned_shards_are_bitwise_one_call(clis):
    """Shard edges on 64-key tiles: the stored sums continue exactly."""
    import torch
    w = workloads.custom("aligned", 1, 2, 500, 128, "bf16", False, key_bias_std=2.0, Nk=640)
    host, dev = _inputs(w, seed=41)
    q, k, v = dev
    mu, _ = clis.clis_certify(q, k, v, w.scale)
    one = _run_shards(clis, q, _shards(k, v, [0, 640]), mu, w.scale, False)
    two = _run_shards(clis, q, _shards(k, v, [0, 192, 640]), mu, w.scale, False)
    torch.cuda.synchronize()
    assert torch.equal(one[0], two[0])
    np.testing.assert_allclose(two[1].cpu().numpy(), one[1].cpu().numpy(), rtol=1e-6)


def test_single_shard_matches_fixed_mode(clis):
    """One shard over all keys, combined, is bitwise clis_attn_fwd in fixed
    mode (the same kernel and the same final operations; only the division
    moves to the combine step)."""
    import torch
    w = workloads.custom("one_shard", 1, 2, 600, 128, "bf16", True, key_bias_std=2.0)
    host, dev = _inputs(w, seed=43)
    q, k, v = dev
    mu, _ = clis.clis_certify(q, k, v, w.scale)
    o_acc, l_acc = _run_shards(clis, q, _shards(k, v, [0, 600]), mu, w.scale, True)
    o, lse = clis.clis_attn_combine(o_acc, l_acc, mu=mu, want_lse=True)
    o_ref, lse_ref = clis.clis_attn_fwd(q, k, v, w.scale, True, mode="fixed", mu=mu, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    assert torch.equal(lse, lse_ref)
