"""Build libpkv.so in-tree with hipcc for gfx950.

    python paged_kv_cache_217_amd/build.py        (or __graft_entry__.build())

This file is run or loaded by path, never imported through the package (the
package loads libpkv.so when imported).

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled (the plain float code still vectorises to scalar
v_fma_f32); objects are linked into paged_kv_cache_217_amd/libpkv.so.
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libpkv.so")
BUILD_DIR = os.path.join(PKG, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          f"-I{INCLUDE}", f"-I{CSRC}"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


def sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src):
    obj = os.path.join(BUILD_DIR, src + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [HIPCC, "-x", "hip", *DEVICE, *COMMON, "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, *COMMON, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(line for line in r.stderr.splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    return obj, err


def build(verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(_compile, srcs))
    for _, err in results:
        if err.strip() and verbose:
            print(err, file=sys.stderr)
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
           *[o for o, _ in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, OUT)
    shutil.rmtree(BUILD_DIR, ignore_errors=True)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
