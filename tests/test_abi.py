"""The C-ABI library loads and exports every symbol include/clis.h declares,
and its argument checks reject bad calls before touching the GPU (CPU only:
no compute call is made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "clis.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


@pytest.fixture(scope="module")
def clis():
    import softmax_stabilization_video_amd as m
    return m


def test_header_declares_the_three_entry_points():
    names = _declared_functions()
    for n in ("clis_certify", "clis_attn_fwd", "online_attn_fwd"):
        assert n in names


def test_library_exports_every_declared_symbol(clis):
    raw = ctypes.CDLL(clis.LIB_PATH)
    names = _declared_functions()
    assert names, "no declarations parsed"
    for n in names:
        assert hasattr(raw, n), f"libclis.so does not export {n}"
    assert sorted(names) == sorted(clis.EXPORTS)


def test_abi_version_and_strings(clis):
    assert clis.lib.clis_abi_version() == 2
    assert clis.lib.clis_status_string(0) == b"ok"
    assert clis.lib.clis_status_string(5).startswith(b"workspace")
    assert clis.lib.clis_status_string(99) == b"unknown status"


def test_stats_struct_size_matches_header(clis):
    assert clis.STATS_BYTES == 56


def test_workspace_size_is_monotone(clis):
    a = clis.workspace_bytes(1, 20, 75600, 75600, 128)
    b = clis.workspace_bytes(1, 20, 1000, 1000, 128)
    assert a > b > 0 and a % 256 == 0
    assert clis.workspace_bytes(0, 1, 1, 1, 64) == 256


def _fake(addr=0x10000):
    return ctypes.c_void_p(addr)


@pytest.mark.parametrize("case,expected", [
    (dict(d=96), 3),                     # unsupported head dim
    (dict(dtype=7), 3),                  # unknown dtype
    (dict(mode=9), 3),                   # unknown mode
    (dict(Nq=10, Nk=12, causal=1), 2),   # causal needs Nq == Nk
    (dict(scale=0.0), 2),
    (dict(scale=float("inf")), 2),
    (dict(B=-1), 2),
    (dict(Nk=0), 2),                     # query rows but no keys
    (dict(q=None), 1),
    (dict(o=None), 1),
    (dict(q=0x10008), 4),                # not 16-byte aligned
    (dict(ws=None, mode=0), 5),          # auto mode needs a workspace
    (dict(ws_bytes=10, mode=0), 5),
    (dict(lse=0x60002), 4),              # lse_out not 4-byte aligned
    (dict(mu=0x70002), 4),               # fp32 / int32 arrays need 4-byte alignment
    (dict(cert=0x70001), 4),
    (dict(route=0x70003), 4),
])
def test_argument_checks_reject_before_launch(clis, case, expected):
    a = dict(q=0x10000, k=0x20000, v=0x30000, o=0x40000, B=1, H=2, Nq=10, Nk=10, d=64, scale=0.125,
             causal=0, dtype=0, mode=1, ws=0x50000, ws_bytes=1 << 30, lse=None, mu=None, cert=None, route=None)
    a.update(case)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    st = clis.lib.clis_attn_fwd(vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["o"]), a["B"], a["H"], a["Nq"],
                                a["Nk"], a["d"], a["scale"], a["causal"], a["dtype"], a["mode"], vp(a["mu"]),
                                vp(a["cert"]), vp(a["route"]), vp(a["lse"]), vp(a["ws"]), a["ws_bytes"], None)
    assert st == expected, clis.lib.clis_last_error()
    assert clis.lib.clis_last_error() != b""


@pytest.mark.parametrize("case,expected", [
    (dict(d=96), 3),
    (dict(mode=7), 3),
    (dict(o=None), 1),
    (dict(q=0x10004), 4),
    (dict(lse=0x60002), 4),
    (dict(Nq=10, Nk=12, causal=1), 2),
    (dict(H=12, Nq=40000, Nk=40000, d=128), 5),   # workspace beyond the static scratch
])
def test_noalloc_argument_checks(clis, case, expected):
    """clis_attn_fwd_noalloc rejects bad calls, and shapes whose workspace
    exceeds its static scratch, before any HIP call (CPU only)."""
    a = dict(q=0x10000, k=0x20000, v=0x30000, o=0x40000, B=1, H=2, Nq=10, Nk=10, d=64, causal=0, mode=0,
             lse=None)
    a.update(case)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    st = clis.lib.clis_attn_fwd_noalloc(vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["o"]), a["B"], a["H"], a["Nq"],
                                        a["Nk"], a["d"], 0.125, a["causal"], 0, a["mode"], None, None, None,
                                        vp(a["lse"]), None)
    assert st == expected, clis.lib.clis_last_error()
    if expected == 5:
        assert b"scratch" in clis.lib.clis_last_error()


def test_noalloc_scratch_constant_matches_header(clis):
    text = open(HEADER).read()
    m = re.search(r"#define CLIS_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == clis.NOALLOC_SCRATCH_BYTES


def test_empty_batch_is_a_no_op(clis):
    # nothing to compute: CLIS_OK without touching any pointer
    for B, H, Nq in ((0, 4, 10), (2, 0, 10), (2, 4, 0)):
        assert clis.lib.clis_attn_fwd(None, None, None, None, B, H, Nq, 10, 128, 0.1, 0, 0, 0, None, None,
                                      None, None, None, 0, None) == 0
        assert clis.lib.online_attn_fwd(None, None, None, None, B, H, Nq, 10, 128, 0.1, 0, 0, None, None, 0,
                                        None) == 0
        assert clis.lib.clis_attn_fwd_partial(None, None, None, B, H, Nq, 10, 128, 0.1, 0, 0, None, 0, 0, None,
                                              None, None, 0, None) == 0
        assert clis.lib.clis_attn_combine(None, None, None, B, H, Nq, 128, 0, None, None, None) == 0
        assert clis.lib.clis_attn_fwd_noalloc(None, None, None, None, B, H, Nq, 10, 128, 0.1, 0, 0, 0, None, None,
                                              None, None, None) == 0
        assert clis.lib.clis_certify(None, None, None, B, H, Nq, 10, 128, 0.1, 0, None, None, None, None,
                                     None, 0, None) == 0


@pytest.mark.parametrize("case,expected", [
    (dict(mu=None), 1),
    (dict(o_acc=None), 1),
    (dict(o_acc=0x60008), 4),            # fp32 accumulators need 16-byte alignment
    (dict(kv_offset=-1), 2),
    (dict(accumulate=2), 2),
    (dict(d=80), 3),
    (dict(ws=None), 5),                  # bf16 shards need a workspace for V^T
    (dict(Nk=0), 2),
])
def test_partial_argument_checks(clis, case, expected):
    a = dict(q=0x10000, k=0x20000, v=0x30000, B=1, H=2, Nq=10, Nk=6, d=64, mu=0x40000, kv_offset=4,
             accumulate=1, o_acc=0x60000, l_acc=0x70000, ws=0x50000)
    a.update(case)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    st = clis.lib.clis_attn_fwd_partial(vp(a["q"]), vp(a["k"]), vp(a["v"]), a["B"], a["H"], a["Nq"], a["Nk"],
                                        a["d"], 0.125, 1, 0, vp(a["mu"]), a["kv_offset"], a["accumulate"],
                                        vp(a["o_acc"]), vp(a["l_acc"]), vp(a["ws"]), 1 << 30, None)
    assert st == expected, clis.lib.clis_last_error()


@pytest.mark.parametrize("case,expected", [
    (dict(o=None), 1),
    (dict(lse=0x40000, mu=None), 1),     # the log-sum-exp needs the stabilizers
    (dict(d=96), 3),
    (dict(dtype=5), 3),
    (dict(o=0x30004), 4),
    (dict(B=-2), 2),
])
def test_combine_argument_checks(clis, case, expected):
    a = dict(o_acc=0x10000, l_acc=0x20000, o=0x30000, B=1, H=2, Nq=10, d=128, dtype=0, mu=None, lse=None)
    a.update(case)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    st = clis.lib.clis_attn_combine(vp(a["o_acc"]), vp(a["l_acc"]), vp(a["o"]), a["B"], a["H"], a["Nq"], a["d"],
                                    a["dtype"], vp(a["mu"]), vp(a["lse"]), None)
    assert st == expected, clis.lib.clis_last_error()


def test_certify_requires_outputs(clis):
    st = clis.lib.clis_certify(_fake(), _fake(), _fake(), 1, 1, 8, 8, 64, 0.1, 0, None, None, None, None,
                               _fake(0x1000000), 1 << 30, None)
    assert st == 1


@pytest.mark.parametrize("mu,cert,stats,kbar", [
    (0x40002, 0x50000, None, None),
    (0x40000, 0x50002, None, None),
    (0x40000, 0x50000, 0x60004, None),   # clis_head_stats_t and fp64 outputs need 8 bytes
    (0x40000, 0x50000, None, 0x60004),
])
def test_certify_rejects_misaligned_outputs(clis, mu, cert, stats, kbar):
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    st = clis.lib.clis_certify(_fake(), _fake(), _fake(), 1, 1, 8, 8, 64, 0.1, 0, vp(mu), vp(cert), vp(stats),
                               vp(kbar), _fake(0x1000000), 1 << 30, None)
    assert st == 4, clis.lib.clis_last_error()


def test_product_path_never_touches_the_oracle():
    """The HIP library's sources and binding name nothing under oracle/."""
    pkg = os.path.join(ROOT, "softmax_stabilization_video_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, flags=re.M), f
                assert "oracle.c" not in text and "_oracle.so" not in text, f
