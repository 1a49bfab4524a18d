"""Build libbsattn.so in-tree with hipcc for gfx950.

    python -m block_sparse_attention_flash_amd.build [--debug]

The shared library lands in ``block_sparse_attention_flash_amd/lib/``.
Every translation unit is compiled on each call (the build is the check).
Device code is built with packed-FP32 instructions disabled.
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIBDIR, "libbsattn.so")
ARCH = os.environ.get("BSATTN_ARCH", "gfx950")

HOST_SOURCES = ["api.cpp", "block_index.cpp", "calibrate.cpp"]
DEVICE_SOURCES = ["prefill_bf16.hip", "prefill_f32.hip", "prefill_bwd.hip", "decode.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libbsattn)")


def _compile(args):
    cmd, src = args
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return src


def build(debug: bool = False, verbose: bool = False) -> str:
    cc = hipcc()
    os.makedirs(LIBDIR, exist_ok=True)
    opt = ["-O0", "-g"] if debug else ["-O3"]
    common = ["-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result", *opt, f"--offload-arch={ARCH}",
              "-I", os.path.join(HERE, "..", "include")]
    # device passes: never emit packed-FP32 VALU ops
    device_only = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    with tempfile.TemporaryDirectory(prefix="bsattn_build_") as tmp:
        jobs = []
        objs = []
        for s in HOST_SOURCES:
            o = os.path.join(tmp, s + ".o")
            jobs.append(([cc, *common, "-x", "hip", "-c", os.path.join(CSRC, s), "-o", o], s))
            objs.append(o)
        for s in DEVICE_SOURCES:
            o = os.path.join(tmp, s + ".o")
            jobs.append(([cc, *common, *device_only, "-x", "hip", "-c", os.path.join(CSRC, s), "-o", o], s))
            objs.append(o)
        with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
            for s in ex.map(_compile, jobs):
                if verbose:
                    print("compiled", s, flush=True)
        tmp_lib = LIB + ".tmp"
        link = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp_lib]
        r = subprocess.run(link, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{' '.join(link)}\n{r.stdout}\n{r.stderr}")
        os.replace(tmp_lib, LIB)
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--debug", action="store_true")
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(debug=a.debug, verbose=a.verbose))
    return 0


if __name__ == "__main__":
    sys.exit(main())
