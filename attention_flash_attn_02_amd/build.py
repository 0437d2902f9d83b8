"""Build the gfx950 attention library (libattn.so) in-tree with hipcc.

Usage: python -m attention_flash_attn_02_amd.build  (or build() from Python).
Every HIP source under csrc/ is compiled for gfx950 to an object file in
_build/, in parallel, and linked into attention_flash_attn_02_amd/libattn.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
COMMON_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


# per-source flags.  prefill_sp.hip: select the VGPR form of the MFMAs, so
# the score tiles the softmax reads stay in VGPRs (with accumulation
# registers the compiler keeps copying them back and forth).
SOURCE_FLAGS = {"prefill_sp.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
                "prefill_sp8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "is not a recognized feature for this target" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every csrc/*.hip for gfx950 and link libattn.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD_DIR, os.path.basename(s)[:-4] + ".o") for s in sources]
    jobs = jobs or min(8, len(sources), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_run, [HIPCC, *COMMON_FLAGS, *SOURCE_FLAGS.get(os.path.basename(s), []), "-c", s, "-o", o])
                for s, o in zip(sources, objs)]
        for f in futs:
            out = f.result()
            if verbose and out.strip():
                print(out)
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
