"""Build libjagged_attn.so (gfx950) in-tree with hipcc.

    python -m recsys_jagged_attention_gdpa_amd.build [--jobs N]

Every HIP translation unit is compiled for gfx950 only, with packed-fp32
instructions disabled, then linked into one shared library next to this file.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libjagged_attn.so")
OBJDIR = os.path.join(HERE, "_build")

SOURCES = ["ja_api.cpp", "ja_plan.hip", "ja_fwd.hip", "ja_fwd_gdpa.hip", "ja_fwd_mx.hip", "ja_bwd.hip", "ja_bwd_kv.hip",
           "ja_dbias.hip", "ja_f32.hip", "ja_rope.hip"]
# Per-unit compiler options (instruction schedulers), each measured against the
# default on the kernels of its unit:
#   * bf16 forward: latency-hiding "max-ilp", JFA forward 3.5 % faster (the
#     MXFP8 forward, 2 % slower with it, is its own unit for that reason);
#   * the bf16 GDPA long-sequence forward: iterative latency-hiding, GELU-erf
#     long-tail forward 2 % faster (the short-K/V forward, 3 % slower with it,
#     stays in the max-ilp unit);
#   * dK/dV: iterative latency-hiding, 6 % faster with the GELU-erf
#     activation, 0.5 % with the softmax;
#   * delta, fused short-K/V and dQ units: iterative occupancy-first, dQ 1-2 %
#     faster (the iterative latency-hiding one made dQ 2.8x slower).
_SCHED = "-amdgpu-sched-strategy="
EXTRA = {"ja_fwd.hip": ["-mllvm", _SCHED + "max-ilp"],
         "ja_fwd_gdpa.hip": ["-mllvm", _SCHED + "iterative-ilp"],
         "ja_bwd_kv.hip": ["-mllvm", _SCHED + "iterative-ilp"],
         "ja_bwd.hip": ["-mllvm", _SCHED + "iterative-maxocc"]}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument"]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def sources_digest() -> str:
    """sha256 over the C/HIP sources, the public headers and the compiler options."""
    h = hashlib.sha256()
    files = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC)) if f.endswith((".hip", ".cpp", ".h"))]
    files += [os.path.join(INCLUDE, f) for f in sorted(os.listdir(INCLUDE)) if f.endswith(".h")]
    for f in files:
        h.update(os.path.basename(f).encode() + b"\0")
        with open(f, "rb") as fh:
            h.update(fh.read())
    h.update(repr(compile_config()).encode())
    return h.hexdigest()


def compile_config():
    """What decides the compiled code besides the sources: units, options, target
    (directory paths left out, so the value does not depend on where the tree sits)."""
    return (SOURCES, [a for a in COMMON if not os.path.isabs(a)], sorted(EXTRA.items()), ARCH)


STAMP = LIB + ".sources"  # digest of the sources the library was built from


def build(jobs: int = 0, verbose: bool = True) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Wl,--no-undefined", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    with open(STAMP, "w") as fh:
        fh.write(sources_digest() + "\n")
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=0)
    a = ap.parse_args()
    try:
        build(a.jobs)
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
