"""Build the in-tree HIP library libpagedkv.so for gfx950.

Run as a script (``python -m paged_kv_cache_293_amd.build``) or call
``build()``.  It always recompiles.  The library lands in
``paged_kv_cache_293_amd/lib/libpagedkv.so`` and is what the Python binding
loads.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_DIR = os.path.join(HERE, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libpagedkv.so")
# Standalone probes (not part of the library): the HBM read ceiling
# (bench.py --ceiling) and the paged-read floor at the decode kernel's shape
# (bench.py --floor).
PROBES = [("read_ceiling.hip", "read_ceiling"), ("paged_read_floor.hip", "paged_read_floor")]
SOURCES = ["api.cpp", "block_manager.cpp", "attention.hip", "cache.hip", "prefill.hip", "speculative.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # packed-FP32 VALU instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose=False, probes=True):
    """Compile the library (errors raise), then the standalone probes, whose
    failure is reported but does not fail the library build."""
    os.makedirs(LIB_DIR, exist_ok=True)
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC] + FLAGS + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    if probes:
        for src, ok, msg in build_probes():
            if not ok:
                print(f"warning: the probe {src} did not build (the library did):\n{msg}", file=sys.stderr)
    return LIB_PATH


def build_probes():
    """Compile the standalone probes; returns (source, ok, compiler messages) per probe."""
    noise = "is not a recognized feature for this target"
    results = []
    for src, exe in PROBES:
        out = os.path.join(LIB_DIR, exe)
        cmd = [HIPCC] + [f for f in FLAGS if f not in ("-shared", "-fPIC")] + [os.path.join(HERE, "probe", src),
                                                                             "-o", out + ".tmp"]
        res = subprocess.run(cmd, capture_output=True, text=True)
        msg = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
        if res.returncode == 0:
            os.replace(out + ".tmp", out)
        results.append((src, res.returncode == 0, msg))
    return results


if __name__ == "__main__":
    print(build(verbose=True))
