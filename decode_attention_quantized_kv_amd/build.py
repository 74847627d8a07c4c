"""Build the gfx950 shared library ``libq8k4v.so`` in-tree with hipcc.

Every HIP source is compiled for gfx950 only.  Packed fp32 VALU
instructions are disabled for device code (``-packed-fp32-ops``).

    python -m decode_attention_quantized_kv_amd.build          # build
    python -m decode_attention_quantized_kv_amd.build --check  # build, list exported symbols
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(PKG, "_lib")
LIB = os.path.join(OUT_DIR, "libq8k4v.so")
OBJ_DIR = os.path.join(ROOT, "_build", "q8k4v")

SOURCES = ["abi.cpp", "append.hip", "attn_paged.hip", "combine.hip", "noalloc.cpp", "probe.hip", "tuner.cpp"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMMON = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-inline-asm", "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def _source_hash() -> str:
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)) + ["../../include/q8k4v.h"]:
        path = os.path.join(CSRC, name)
        if os.path.isfile(path):
            h.update(name.encode())
            h.update(open(path, "rb").read())
    return h.hexdigest()[:12]


# MFMA accumulators in ordinary VGPRs (gfx950's unified register file): the
# online-softmax rescale then multiplies them in place instead of copying
# them out of and back into accumulation registers.
PER_SOURCE = {
    "attn_paged.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def _compile(src: str, build_id: str) -> str:
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *PER_SOURCE.get(src, []), f'-DQ8K4V_BUILD_ID="{build_id}"', "-c",
           os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True, jobs: int = 0) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    os.makedirs(OBJ_DIR, exist_ok=True)
    build_id = _source_hash()
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_id), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} ({build_id})")
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--check", action="store_true")
    args = ap.parse_args(argv)
    lib = build()
    if args.check:
        r = subprocess.run(["nm", "-D", "--defined-only", lib], capture_output=True, text=True)
        print("\n".join(l for l in r.stdout.splitlines() if " T " in l))
    return 0


if __name__ == "__main__":
    sys.exit(main())
