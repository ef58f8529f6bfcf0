"""HIP-graph capture of whole calls.  Every call of the library only launches
kernels on the caller's stream: no host synchronization, routing read on the
device, work counters zeroed by a kernel (no memset node).  A captured auto-mode
call (certification, routing, both attention kernels, the run-time work pool and
the key-split combine; for fp32 certification and the self-routing kernel)
therefore replays to the eager result, bitwise, replay after replay, with other
work and synchronizations on the stream in between.
Key-shard calls (clis_attn_fwd_partial + clis_attn_combine) are captured too.
"""
import pytest

import workloads
from tests.gpu_util import say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def clis():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import softmax_stabilization_video_amd as m
    return m


def _capture(fn):
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the graph, as capture requires
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


GRAPH_CASES = [
    # dtype, N, d: bf16 (certification kernels, routing, both attention kernels,
    # the pools and the key-split combine); fp32 with one-launch certification
    # (N <= 1024) and with the split certification kernels, each followed by
    # the self-routing fp32 attention kernel
    ("bf16", 3000, 128),
    ("fp32", 700, 64),
    ("fp32", 1500, 128),
]


@pytest.mark.parametrize("dtype,N,d", GRAPH_CASES, ids=[f"{c[0]}_{c[1]}_d{c[2]}" for c in GRAPH_CASES])
def test_auto_mode_call_replays_bitwise(clis, dtype, N, d):
    import torch
    # a third of the heads fail certification, so both routes run; for bf16,
    # 12 query tiles per fixed head and 24 per online head give pools with
    # whole items and, in the fixed kernel, key splits
    w = workloads.custom(f"graph_auto_{dtype}", 1, 6, N, d, dtype, False, key_bias_std=2.0,
                         fail_frac=0.34, fail_qk_scale=40.0)
    Q, K, V = workloads.make_inputs(w, 61)
    q, k, v = (to_device(a, w.dtype) for a in (Q, K, V))
    ws = clis.new_workspace(w.B, w.H, w.Nq, w.Nk, w.d)
    ref, route, lse = clis.clis_attn_fwd(q, k, v, w.scale, mode="auto", want_route=True, want_lse=True, workspace=ws)
    torch.cuda.synchronize()
    n_fixed = int(route.sum())
    say("graph auto", "fixed heads", n_fixed, "of", w.B * w.H)
    assert 0 < n_fixed < w.B * w.H, "the case must route heads both ways"

    o_g = torch.empty_like(q)
    route_g = torch.empty_like(route)
    lse_g = torch.empty_like(lse)

    def call():
        clis.get_lib().clis_attn_fwd(
            clis._ptr(q), clis._ptr(k), clis._ptr(v), clis._ptr(o_g), w.B, w.H, w.Nq, w.Nk, w.d, w.scale, 0,
            clis._dtype_code(q), clis.MODES["auto"], None, None, clis._ptr(route_g), clis._ptr(lse_g),
            clis._ptr(ws), ws.numel(), clis._stream())

    g = _capture(call)
    for rep in range(4):
        o_g.fill_(float("nan"))
        lse_g.fill_(float("nan"))
        route_g.fill_(-1)
        # eager work on the same stream and workspace between replays
        other = clis.clis_attn_fwd(q, k, v, w.scale, mode="online", workspace=ws)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say("replay", rep)
        assert torch.equal(o_g, ref), f"replay {rep}: output differs from the eager call"
        assert torch.equal(lse_g, lse), f"replay {rep}: lse differs"
        assert torch.equal(route_g, route), f"replay {rep}: routes differ"
        assert not torch.isnan(other).any()


def test_key_shard_calls_replay_bitwise(clis):
    import torch
    w = workloads.custom("graph_shards", 1, 2, 700, 128, "bf16", True, key_bias_std=2.0)
    Q, K, V = workloads.make_inputs(w, 62)
    q, k, v = (to_device(a, w.dtype) for a in (Q, K, V))
    mu, _ = clis.clis_certify(q, k, v, w.scale)
    edges = [0, 256, 700]
    shards = [(a, k[:, :, a:b].contiguous(), v[:, :, a:b].contiguous()) for a, b in zip(edges[:-1], edges[1:])]
    o_acc = torch.empty((1, 2, 700, 128), dtype=torch.float32, device=q.device)
    l_acc = torch.empty((1, 2, 700), dtype=torch.float32, device=q.device)
    o = torch.empty_like(q)
    wss = [clis.new_workspace(1, 2, 700, ks.shape[2], 128) for _, ks, _ in shards]

    def call():
        for i, (a, ks, vs) in enumerate(shards):
            clis.clis_attn_fwd_partial(q, ks, vs, mu, o_acc, l_acc, w.scale, True, kv_offset=a, accumulate=i > 0,
                                       workspace=wss[i])
        clis.clis_attn_combine(o_acc, l_acc, out=o)

    call()
    torch.cuda.synchronize()
    ref = o.clone()
    g = _capture(call)
    for rep in range(3):
        o.fill_(float("nan"))
        o_acc.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref), f"replay {rep}: combined output differs"
