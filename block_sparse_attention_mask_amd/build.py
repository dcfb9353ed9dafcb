"""Compile the HIP sources into libbsattn.so for gfx950 (in-tree)."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libbsattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    # packed fp32 VALU forms stay off: ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# Per-source compiler flags beyond FLAGS (none at present).
EXTRA: dict = {}


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    import tempfile
    from concurrent.futures import ThreadPoolExecutor
    tmp = LIB + ".tmp%d" % os.getpid()
    with tempfile.TemporaryDirectory(prefix="bsattn_build_") as od:
        objs, cmds = [], []
        for src in sources():
            obj = os.path.join(od, os.path.basename(src) + ".o")
            flags = [f for f in FLAGS if f != "-shared"]
            cmds.append([HIPCC] + flags + EXTRA.get(os.path.basename(src), []) + ["-c", src, "-o", obj])
            objs.append(obj)
        with ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds))
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp], verbose)
    # every symbol must resolve (a kernel whose host launch stub was not
    # emitted shows up here, not on the first GPU call)
    import ctypes
    ctypes.CDLL(tmp, mode=os.RTLD_NOW | os.RTLD_LOCAL)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
