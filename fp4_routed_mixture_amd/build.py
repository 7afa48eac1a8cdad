"""Build the gfx950 HIP libraries in-tree with hipcc.

  libfp4moe.so        the routed-MoE layer (csrc/*.hip except synth.hip)
  libfp4moe_synth.so  test and benchmark support: the device side of the seeded
                      input generator, the streaming-read and FP4 MFMA probes,
                      and a hook evaluating the kernels' exp and sigmoid

Every kernel is compiled for gfx950 only, without fast-math, with fp
contraction off (fused multiply-adds are written explicitly where the
numerics call for them) and without packed-fp32 instruction selection.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfp4moe.so")
SYNTH_LIB = os.path.join(HERE, "libfp4moe_synth.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]
LIB_SOURCES = ["api.hip", "prepack.hip", "route.hip", "sort.hip", "quant.hip",
               "gemm_decode.hip", "gemm_prefill.hip", "gemm_dense.hip", "combine.hip"]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (p.stdout + p.stderr).splitlines()
                    if "is not a recognized feature for this target" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def _link(objs, target):
    tmp = target + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed for {target}:\n{p.stdout}{p.stderr}")
    os.replace(tmp, target)


def build(verbose: bool = True) -> None:
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError("hipcc not found: the HIP libraries cannot be built")
    os.makedirs(OBJ, exist_ok=True)
    srcs = LIB_SOURCES + ["synth.hip"]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in LIB_SOURCES], LIB)
    _link([objs["synth.hip"]], SYNTH_LIB)
    if verbose:
        print(f"built {LIB} and {SYNTH_LIB}")


if __name__ == "__main__":
    build()
