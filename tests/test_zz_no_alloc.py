"""clis_attn_fwd_noalloc (the entry point for callers that cannot allocate:
its scratch is the library's static per-GPU array) against clis_attn_fwd with
a workspace: bitwise equal outputs, routes and log-sum-exps, on two calls in a
row, the second with smaller inputs, so that nothing the second call reads is
left over from the first.  Mixed routing (some heads fail certification)
exercises certification, both kernels and the key-split pool."""
import numpy as np
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


CASES = [
    # name, B, H, N, d, causal, seed, dtype
    ("larger", 2, 5, 2000, 128, False, 21, "bf16"),
    ("smaller", 1, 3, 700, 64, False, 22, "bf16"),
    ("smaller_causal", 1, 2, 500, 128, True, 23, "bf16"),
    ("fp32", 1, 4, 600, 64, False, 24, "fp32"),
    # short fp32 heads: one-launch certification
    ("fp32_short", 1, 4, 256, 64, False, 25, "fp32"),
]


def _run_case(clis, name, B, H, N, d, causal, seed, dtype, mode):
    import torch
    w = workloads.custom(f"noalloc_{name}", B, H, N, d, dtype, causal, base="mixed", fail_frac=0.4)
    assert clis.workspace_bytes(B, H, N, N, d) <= clis.NOALLOC_SCRATCH_BYTES
    Q, K, V = workloads.make_inputs(w, seed)
    q, k, v = (to_device(a, dtype) for a in (Q, K, V))
    say("noalloc", name, mode, B, H, N, d, dtype, "causal" if causal else "dense")
    ref, ref_route, ref_lse = clis.clis_attn_fwd(q, k, v, w.scale, causal, mode=mode, want_route=True,
                                                 want_lse=True)
    o = torch.full_like(q, float("nan"))
    route = torch.full((B, H), -1, dtype=torch.int32, device=q.device)
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=q.device)
    clis.clis_attn_fwd_noalloc(q, k, v, w.scale, causal, mode=mode, out=o, route=route, lse=lse)
    o2 = torch.empty_like(q)
    clis.clis_attn_fwd_noalloc(q, k, v, w.scale, causal, mode=mode, out=o2)
    torch.cuda.synchronize()
    # bit patterns (forced fixed mode gives NaN on the heads that fail certification)
    bits = lambda t: t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)
    assert torch.equal(bits(o), bits(ref)) and torch.equal(bits(o2), bits(ref)), name
    assert torch.equal(route, ref_route) and torch.equal(bits(lse), bits(ref_lse)), name
    return ref_route


@pytest.mark.parametrize("mode", ["auto", "fixed", "online"])
def test_noalloc_equals_workspace_entry_point(clis, mode):
    routes = [_run_case(clis, *c, mode) for c in CASES]
    if mode == "auto":  # both routes taken
        r = routes[0].cpu().numpy()
        assert 0 < r.sum() < r.size


def test_noalloc_rejects_shapes_beyond_its_scratch(clis):
    """A shape whose workspace would exceed the static scratch: an error,
    nothing enqueued (the output keeps its contents)."""
    import torch
    B, H, N, d = 1, 12, 40000, 128
    assert clis.workspace_bytes(B, H, N, N, d) > clis.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, 3.0)
    with pytest.raises(clis.ClisError) as e:
        clis.clis_attn_fwd_noalloc(q, q, q, out=o)
    torch.cuda.synchronize()
    assert e.value.status == 5
    assert bool((o == 3.0).all())
