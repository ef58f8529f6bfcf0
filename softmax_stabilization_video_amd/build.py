"""Build libclis.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m softmax_stabilization_video_amd.build

Each .hip source is compiled to an object in parallel, then linked into a
shared library next to this file.  A second, separate library,
libclis_probe.so, holds the MFMA-rate probe that the benchmark reports
beside the published peak.  Flags: gfx950 only; -O3; packed-fp32 VALU
forms disabled (they are not used by this code and stay off by policy).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libclis.so")
BUILD = os.path.join(HERE, "_build")
SOURCES = ["api.hip", "certify.hip", "transpose.hip", "attn_bf16.hip", "attn_fp32.hip", "combine.hip"]
PROBE_SOURCES = ["probe_mfma.hip"]
PROBE_LIB = os.path.join(HERE, "libclis_probe.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", INCLUDE, "-I", CSRC]


def _compile(src: str, extra=(), tag: str = "") -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + tag + ".o")
    cmd = [HIPCC, *CFLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(sources, extra, out: str) -> str:
    os.makedirs(BUILD, exist_ok=True)
    tag = "" if out in (LIB, PROBE_LIB) else "." + os.path.basename(out).replace(".so", "")
    with ThreadPoolExecutor(len(sources)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, tag), sources))
    tmp = out + f".tmp{os.getpid()}"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    # every kernel launched from host code must have its host stub defined;
    # a silently dropped kernel instantiation shows up as an undefined symbol
    nm = subprocess.run(["nm", "-C", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [l.strip() for l in nm.stdout.splitlines() if "clis::" in l]
    if missing:
        os.remove(tmp)
        raise RuntimeError(f"{os.path.basename(out)} has undefined library symbols:\n" + "\n".join(missing))
    os.replace(tmp, out)
    return out


def build(verbose: bool = False, extra=(), out: str = LIB) -> str:
    """Compile every source and link `out` (default: the package's libclis.so,
    plus libclis_probe.so; `extra` adds compiler flags, e.g. -D tuning knobs
    for a variant library, which skips the probe)."""
    _link(SOURCES, extra, out)
    if verbose:
        print(f"built {out}")
    if out == LIB:
        _link(PROBE_SOURCES, (), PROBE_LIB)
        if verbose:
            print(f"built {PROBE_LIB}")
    return out


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
