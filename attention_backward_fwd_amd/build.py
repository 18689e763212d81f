"""Compile libmi355_attn.so for gfx950 in-tree with hipcc.

Usage: ``python -m attention_backward_fwd_amd.build`` (or ``build()``).
Each csrc/*.hip file is compiled to an object in parallel, then linked into
``attention_backward_fwd_amd/libmi355_attn.so``.  hipcc cross-compiles, so
this needs no GPU.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmi355_attn.so")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed fp32 VALU instructions stay off in every kernel of this library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(hipcc, src, extra):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc, *FLAGS, *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def _check_stubs(lib):
    """Fail if a kernel's host launch stub is left unresolved.

    The host pass can drop a kernel's stub without any diagnostic (the kernel
    body is only checked, not compiled, there), and the library then fails
    only when the GPU loader resolves it.
    """
    nm = shutil.which("nm") or "/usr/bin/nm"
    res = subprocess.run([nm, "-u", lib], capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"nm failed on {lib}:\n{res.stderr}")
    missing = [ln.split()[-1] for ln in res.stdout.splitlines() if "__device_stub__" in ln]
    if missing:
        raise RuntimeError("kernel launch stubs left undefined: " + ", ".join(missing))


def build(verbose: bool = False, extra=()) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(hipcc, s, list(extra)), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    _check_stubs(tmp)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
