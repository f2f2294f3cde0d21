"""Build libflux.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

    python block_sparse_attention_flux_amd/build.py      # or build() from Python

(Run it as a file: importing the package itself loads the built library.)

The library lands at ``block_sparse_attention_flux_amd/lib/libflux.so``, with
``libflux.stamp`` beside it: the sha256 of every source, header and build
flag it was built from.  ensure_built() rebuilds whenever that stamp does not
match the tree, so nothing runs against a library built from other sources.
"""

import concurrent.futures
import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(PKG, "lib")
OBJ_DIR = os.path.join(ROOT, "_build", "flux")
LIB_NAME = "libflux.so"
ARCH = "gfx950"

# Packed FP32 ops are switched off: every float op is issued unpacked.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


# Extra flags per source.  prefill.hip: LLVM's iterative scheduler in its ILP
# mode (each region scheduled for instruction-level parallelism, kept only
# where the kernel's occupancy still holds); measured on the 32K layers at the
# same occupancy: ~1 % faster FA, ~0.5 % SA, bit-identical results.
EXTRA_FLAGS = {"prefill.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]}


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libflux")
    return exe


def sources():
    names = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    return [os.path.join(CSRC, f) for f in names]


def _compile(src):
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    extra = EXTRA_FLAGS.get(os.path.basename(src), [])
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, f"-I{INCLUDE}", f"-I{CSRC}", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{r.stderr}")
    return obj


STAMP = os.path.join(OUT_DIR, "libflux.stamp")


def source_digest():
    """sha256 over the sources, the public headers and the build flags."""
    h = hashlib.sha256()
    files = sources() + sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h"))
    files += sorted(os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h"))
    for path in files:
        h.update(os.path.relpath(path, ROOT).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    h.update(repr((HIPCC_FLAGS, sorted(EXTRA_FLAGS.items()))).encode())
    return h.hexdigest()


def is_current():
    out = os.path.join(OUT_DIR, LIB_NAME)
    try:
        with open(STAMP) as f:
            return os.path.exists(out) and f.read().strip() == source_digest()
    except OSError:
        return False


def ensure_built():
    """Build unless libflux.so exists and its stamp matches the current tree."""
    out = os.path.join(OUT_DIR, LIB_NAME)
    if is_current():
        return out
    why = "not built" if not os.path.exists(out) else "built from other sources"
    print(f"[flux build] libflux.so {why}: building", file=sys.stderr, flush=True)
    return build()


def build(verbose=False):
    """Compile every source and link libflux.so; always rebuilds."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    os.makedirs(OUT_DIR, exist_ok=True)
    digest = source_digest()  # of the tree the objects are compiled from
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    out = os.path.join(OUT_DIR, LIB_NAME)
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    with open(STAMP, "w") as f:
        f.write(digest + "\n")
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
