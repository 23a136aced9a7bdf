"""Build libdg.so (HIP kernels + C ABI runtime) for gfx950 with hipcc, in-tree.

    python -m block_diffusion_decoding_dg_amd.build
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdg.so")

SOURCES = ["k_dense.hip", "k_attn.hip", "k_moe.hip", "k_ws.hip", "k_wsd.hip", "k_sample.hip", "k_selfcond.hip", "dg_runtime.hip"]
ARCH = os.environ.get("DG_OFFLOAD_ARCH", "gfx950")

# Packed-fp32 instructions are kept out of the generated code on purpose.
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-I", INCLUDE, "-I", CSRC]


def hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src, build_dir=BUILD, defines=()):
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + HIP_FLAGS + ["-D" + d for d in defines] + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr[-6000:]))
    return obj


def build(verbose=False, out=LIB, defines=()):
    """Compile and link the library.  `defines` (NAME=VALUE strings) and `out`
    give variant builds, e.g. other tile parameters, without touching the
    in-tree library."""
    build_dir = BUILD if out == LIB else out + ".objs"
    os.makedirs(build_dir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda f: _compile(f, build_dir, defines), SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr[-6000:]))
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
