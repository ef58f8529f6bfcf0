"""Host checks of the generated two-half tile code (csrc/gen_tile_h2.py):
the committed tile_h2.inc is what the generator writes, and the window
schedule it encodes runs every part of every tile exactly once, in chain
order, reading only LDS stages that hold the tile it wants (three stages, the
next tile loading into the third)."""
import importlib.util
import os
import re

import pytest

CSRC = os.path.join(os.path.dirname(__file__), "..", "softmax_stabilization_video_amd", "csrc")


def _gen():
    spec = importlib.util.spec_from_file_location("gen_tile_h2", os.path.join(CSRC, "gen_tile_h2.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_committed_include_is_generated(tmp_path, monkeypatch):
    g = _gen()
    want = open(os.path.join(CSRC, "tile_h2.inc")).read()
    # write into a scratch copy of the folder layout
    monkeypatch.setattr(g.os.path, "abspath", lambda p: str(tmp_path / "gen_tile_h2.py"))
    g.main()
    got = (tmp_path / "tile_h2.inc").read_text()
    assert got == want, "tile_h2.inc is stale: run gen_tile_h2.py"


CHAIN = ["qk0", "sm0", "pv0", "qk1", "sm1", "pv1"]


def _window_kind(w, ntiles, nt_wave, pair):
    # the kernel's choice (attn_bf16.hip, the two-half loop)
    if w > nt_wave or nt_wave == 0:
        return 6
    return (2 if w == 0 else 0 if w < nt_wave else 4) + pair


@pytest.mark.parametrize("ntiles", range(0, 8))
def test_window_schedule_covers_the_chain(ntiles):
    g = _gen()
    names = [v[0] for v in g.VARIANTS]
    assert names[6] == "loads" and not g.VARIANTS[6][1]
    for nt_wave in range(0, ntiles + 1):
        for pair in (0, 1):
            done, live, st = [], {0: 0}, 0  # stage -> tile it holds; tile 0 loads first
            for w in range(ntiles + 1):
                if w + 1 < ntiles:  # issued after window w's barrier
                    live[(st + 1) % 3] = w + 1
                parts = g.VARIANTS[_window_kind(w, ntiles, nt_wave, pair)][1]
                for p in parts:
                    t = w - 1 if p.endswith("p") else w
                    if p[:2] in ("qk", "pv"):
                        stage = st if t == w else (st - 1) % 3
                        assert live.get(stage) == t, (ntiles, nt_wave, pair, w, p)
                    done.append((t, p[:3]))
                st = (st + 1) % 3
            assert done == [(t, p) for t in range(nt_wave) for p in CHAIN], (ntiles, nt_wave, pair)


def test_pair_phases_alternate():
    """In a whole window the first wave starts with products and the second
    with weights, and their phases alternate (products vs weights)."""
    g = _gen()
    kinds = lambda parts: ["V" if p.startswith("sm") else "M" for p in parts]
    squash = lambda ks: [k for i, k in enumerate(ks) if i == 0 or ks[i - 1] != k]
    a, b = squash(kinds(g.VARIANTS[0][1])), squash(kinds(g.VARIANTS[1][1]))
    assert a == ["M", "V", "M", "V"] and b == ["V", "M", "V", "M"]


def test_generated_code_uses_only_listed_instructions():
    """Every instruction of the generated code is one of a short list (vector
    ALU, LDS reads, LDS-direct buffer loads, and scalar control: waits, nops,
    priority, compares and branches, M0 / scalar-offset setup); no packed fp32
    op is hand-written; every MFMA is the bf16 32x32x16 one."""
    text = open(os.path.join(CSRC, "tile_h2.inc")).read()
    ops = set(re.findall(r'^\s*"([a-z_0-9]+)[^"]*\\n"', text, re.M))  # the asm lines
    allowed_scalar = {"s_waitcnt", "s_nop", "s_setprio", "s_cmp_eq_u32", "s_cmp_lt_u32", "s_cbranch_scc0",
                      "s_cbranch_scc1", "s_branch", "s_add_u32", "s_mov_b32"}
    for o in ops:
        assert (o.startswith("v_") or o == "ds_read_b128" or o in ("buffer_load_dword", "buffer_load_dwordx4")
                or o in allowed_scalar), o
    assert not any(o.startswith("v_pk_") for o in ops)
    assert {o for o in ops if "mfma" in o} == {"v_mfma_f32_32x32x16_bf16"}


def test_block_placement():
    """The block starts with a jump over padding to a 256-byte boundary (plus
    the chosen no-ops) and ends on a 64-byte boundary, so the code around it
    does not move it (its speed depends on its placement)."""
    text = open(os.path.join(CSRC, "tile_h2.inc")).read()
    lines = re.findall(r'^\s*"([^"]*)\\n"', text, re.M)
    g = _gen()
    assert lines[:3] == ["s_branch .Lanchor_%=", ".p2align 8", ".Lanchor_%=:"]
    assert lines[3:3 + g.ANCHOR_NOPS] == ["s_nop 0"] * g.ANCHOR_NOPS
    assert not lines[3 + g.ANCHOR_NOPS].startswith("s_nop")
    assert lines[-2:] == [".p2align 6", ".Lend_%=:"]
    # every variant is left by a jump to the end except the last, which falls
    # into the padding and the end label
    assert sum(1 for l in lines if l == "s_branch .Lend_%=") == len(g.VARIANTS) - 1
