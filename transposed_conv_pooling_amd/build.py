"""Build libct.so (the HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libct.so")
OBJ = os.path.join(PKG, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in device code (the host pass
# warns that it does not know the feature; that is harmless).
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Wall", "-Wno-unused-result",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-fvisibility=hidden"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln]
    return r.returncode, msgs


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every csrc/*.hip to an object in parallel, then link libct.so."""
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(OBJ, os.path.basename(s)[:-4] + ".o") for s in srcs]
    cflags = [f for f in FLAGS if f != "-shared"]
    cmds = [[HIPCC, *cflags, "-I", INCLUDE, "-I", CSRC, "-c", "-o", o, s]
            for s, o in zip(srcs, objs)]
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        results = list(ex.map(lambda c: _run(c, verbose), cmds))
    msgs = [m for _, ms in results for m in ms]
    if verbose and msgs:
        print("\n".join(msgs))
    if any(rc != 0 for rc, _ in results):
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    tmp = LIB + ".tmp"
    rc, msgs = _run([HIPCC, *FLAGS, "-o", tmp, *objs], verbose)
    if verbose and msgs:
        print("\n".join(msgs))
    if rc != 0:
        raise RuntimeError("hipcc link failed:\n" + "\n".join(msgs))
    os.replace(tmp, LIB)
    build_call(verbose)
    return LIB


def build_call(verbose: bool = False) -> str:
    """The CPython module _ctcall (argument forwarding into libct.so), with gcc
    against this interpreter's headers; libct.so is found next to it."""
    import sysconfig
    src = os.path.join(PKG, "_ctcall.c")
    dst = os.path.join(PKG, "_ctcall" + sysconfig.get_config_var("EXT_SUFFIX"))
    tmp = dst + ".tmp"
    cmd = ["gcc", "-O2", "-shared", "-fPIC", "-Wall", "-I", sysconfig.get_paths()["include"],
           "-I", INCLUDE, "-o", tmp, src, "-L", PKG, "-l:libct.so", "-Wl,-rpath,$ORIGIN"]
    rc, msgs = _run(cmd, verbose)
    if verbose and msgs:
        print("\n".join(msgs))
    if rc != 0:
        raise RuntimeError("gcc (_ctcall) failed:\n" + "\n".join(msgs))
    os.replace(tmp, dst)
    return dst


if __name__ == "__main__":
    print(build(verbose=True))
