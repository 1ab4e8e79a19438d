"""Build libmi355norm.so (gfx950) in-tree with hipcc.

Each .hip translation unit under csrc/ is compiled in parallel, then linked
into rmsnorm_forward_amd/libmi355norm.so; csrc/pycalls.c (host C) becomes
the package's CPython module of the per-call entry points.  Run as
`python rmsnorm_forward_amd/build.py` or through `__graft_entry__.build()`
(the package itself refuses to import until the library exists).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmi355norm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-fp32 VALU ops are disabled for all device code (-packed-fp32-ops);
# hipcc's host pass warns that it does not know the feature, harmlessly.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src).replace(".hip", ".o"))
    cmd = [HIPCC, *HIP_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    if verbose and r.stderr.strip():
        noise = "is not a recognized feature for this target"
        lines = [l for l in r.stderr.splitlines() if noise not in l]
        if lines:
            print("\n".join(lines), file=sys.stderr)
    return obj


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = jobs or min(len(srcs), max(1, min(os.cpu_count() or 1, 8)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    build_calls()
    return LIB


def build_calls() -> str:
    """The CPython module of the per-call entry points (host C, gcc): it
    links nothing and is bound to the loaded library at import."""
    import sysconfig
    out = os.path.join(HERE, "_calls" + sysconfig.get_config_var("EXT_SUFFIX"))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [os.environ.get("CC", "gcc"), "-O2", "-shared", "-fPIC", "-Wall", "-Werror",
           "-I" + sysconfig.get_paths()["include"], os.path.join(CSRC, "pycalls.c"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building the CPython module failed:\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
