"""Build libpoetx.so (the HIP/gfx950 library behind include/poetx.h) in-tree.

Every source is compiled with hipcc for gfx950 only, objects in parallel,
then linked into ``orthogonal_reparameterized_poetx_amd/libpoetx.so``.
"""

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpoetx.so")
SOURCES = ["api.hip", "build.hip", "chain.hip", "transform.hip", "blockdiag.hip", "gemm.hip", "gram.hip", "merge.hip", "quant.hip", "cnp.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function", "-Wno-unused-variable",
    # packed fp32 (v_pk_*_f32) is kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    return p.returncode, out


def build(verbose=False, jobs=None):
    """Compile every HIP source for gfx950 and link libpoetx.so.  Raises on error."""
    os.makedirs(BUILD, exist_ok=True)
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    jobs = jobs or min(len(cmds), os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_run, cmds))
    for cmd, (rc, out) in zip(cmds, results):
        if verbose and out.strip():
            print(out)
        if rc != 0:
            raise RuntimeError("hipcc failed for %s:\n%s" % (cmd[-3], out))
    tmp = LIB + ".tmp"
    rc, out = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    if rc != 0:
        raise RuntimeError("link failed:\n%s" % out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
