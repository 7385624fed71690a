"""Build the two C-ABI libraries.

* libpagedkv.so -- the GPU path, from the HIP sources, for gfx950: every
  source is compiled by hipcc into an object under csrc/_build/, then
  linked.  Packed-FP32 VALU instructions are disabled for device code.
* libpkvhost.so -- the host block manager and decode-loop simulator, plain
  C++ built with g++ (no GPU code).

Usable as a script:
    python -m paged_kv_cache_311_amd.build_lib
"""

import glob
import hashlib
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(CSRC, "_build")
LIB_PATH = os.path.join(HERE, "libpagedkv.so")
SOURCES = ["paged_attention.hip", "cache_ops.hip", "prefill.hip", "vpool.hip",
           "shared_prefix.hip"]
HOST_LIB_PATH = os.path.join(HERE, "libpkvhost.so")
HOST_SOURCES = ["block_manager.cpp"]
CXX = os.environ.get("CXX", "g++")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(HERE, "..", "include"),
]


# Per-source extra flags.  The decode kernel picks each tile's cache policy
# with a uniform branch; structurizing that branch adds a path that issues
# neither load, and the compiler's wait counts then assume it, waiting for
# the next tile's loads before computing the current one.  Leaving uniform
# regions unstructurized (they are lowered as scalar branches) keeps them.
SOURCE_FLAGS = {
    "paged_attention.hip": ["-mllvm", "-structurizecfg-skip-uniform-regions"],
}


def source_digest():
    """sha256 of every source and header the library is built from, and of
    the compile flags.  Built into the library (pkv_build_id) and checked by
    the binding at load time, so a library older than its sources never
    runs."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(CSRC, "*.hip")) +
                   glob.glob(os.path.join(CSRC, "*.h")) +
                   [os.path.join(HERE, "..", "include", "pagedkv.h"),
                    os.path.join(HERE, "..", "include", "pkv_vpool.h")])
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    h.update(" ".join(FLAGS[:-1]).encode())  # flags other than the include path
    for src in sorted(SOURCE_FLAGS):
        h.update((src + " " + " ".join(SOURCE_FLAGS[src])).encode())
    return h.hexdigest()


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device-only target feature: harmless
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l and
                    "ignoring feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed: {' '.join(cmd)}\n{err}")
    return err


def build_host(verbose=False):
    """Compile the host library (always rebuilds)."""
    tmp = HOST_LIB_PATH + ".tmp"
    warn = _run([CXX, "-O2", "-std=c++17", "-Wall", "-Wextra", "-fPIC", "-shared",
                 *[os.path.join(CSRC, f) for f in HOST_SOURCES], "-o", tmp])
    if verbose and warn.strip():
        print(warn, file=sys.stderr)
    os.replace(tmp, HOST_LIB_PATH)
    return HOST_LIB_PATH


def build(verbose=False):
    """Compile every HIP source and link the GPU library, then the host
    library (always rebuilds both)."""
    os.makedirs(BUILD_DIR, exist_ok=True)

    stamp = f'-DPKV_BUILD_ID="{source_digest()}"'

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, src.rsplit(".", 1)[0] + ".o")
        warn = _run([HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), stamp, "-c",
                     os.path.join(CSRC, src), "-o", obj])
        if verbose and warn.strip():
            print(warn, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB_PATH)
    build_host(verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
