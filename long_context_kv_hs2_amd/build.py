"""Build libhs2.so in-tree with hipcc for gfx950.

    python -m long_context_kv_hs2_amd.build          # or build() from Python

Each HIP source compiles to an object under ``long_context_kv_hs2_amd/_build``
(in parallel), then one link makes ``long_context_kv_hs2_amd/libhs2.so``.
Packed-fp32 VALU forms are switched off for the device code.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libhs2.so")
SOURCES = ["hs2_api.hip", "full_decode.hip", "merge.hip", "topk_select.hip", "sparse_decode.hip", "bridge_kv.hip", "block_select.hip", "bridge_append.hip", "multi_decode.hip", "full_multi.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-variable",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(HERE, "..", "include"),
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the device-only feature flag; drop that line
    lines = [ln for ln in r.stdout.splitlines() if "packed-fp32-ops" not in ln]
    return r.returncode, "\n".join(lines)


def build(verbose: bool = False, extra_flags=None) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    flags = FLAGS + list(extra_flags or [])
    objs = [os.path.join(OUT_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]

    def compile_one(i):
        return _run([HIPCC, *flags, "-c", os.path.join(CSRC, SOURCES[i]), "-o", objs[i]])

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        results = list(ex.map(compile_one, range(len(SOURCES))))
    for src, (rc, out) in zip(SOURCES, results):
        if out.strip() and (verbose or rc):
            print(f"[{src}]\n{out}", file=sys.stderr)
        if rc:
            raise RuntimeError(f"hipcc failed on {src}")
    tmp = LIB + ".tmp"
    rc, out = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    if rc:
        print(out, file=sys.stderr)
        raise RuntimeError("link of libhs2.so failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
