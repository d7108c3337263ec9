"""Build libcsa.so (the gfx950 HIP kernels and their C ABI) in-tree.

    python compressed_sparse_kv_compress_amd/build.py

Compiles every csrc/*.hip and csrc/*.cpp with hipcc for gfx950 only and links
them into compressed_sparse_kv_compress_amd/libcsa.so.  Always rebuilds.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libcsa.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU ops stay off (the compiler would otherwise form them)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-function",
]
# Per-source flags: MFMA accumulators in ordinary VGPRs.  attn.hip: the (rare)
# re-scaling of the output accumulators then does not make the compiler copy
# all of them between AGPRs and VGPRs on every loop iteration.  index.hip: the
# scan's epilogue reads each tile's accumulators with VALU ops, which the AGPR
# form turns into sixteen v_accvgpr_read per tile (fp8 scan 4% faster).
FILE_FLAGS = {
    "attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "index.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str, obj_dir: str = OBJ, extra=()) -> str:
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, *FILE_FLAGS.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-xhip")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose: bool = False, out: str = LIB, extra=()) -> str:
    """Compile and link; `extra` adds compiler flags (e.g. -D tuning constants)."""
    obj_dir = OBJ if out == LIB else os.path.join(os.path.dirname(os.path.abspath(out)), "_obj")
    os.makedirs(obj_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    workers = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(lambda f: _compile(f, obj_dir, tuple(extra)), srcs))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
