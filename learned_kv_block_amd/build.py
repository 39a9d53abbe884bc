"""Build libmsa.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(HERE, "libmsa.so")
OUT_TIMED = os.path.join(HERE, "libmsa_timed.so")
BUILD = os.path.join(HERE, "_build")

# kernels and the C ABI, linked into both libraries
SOURCES = ["msa_api.cpp", "msa_select.hip", "msa_attn.hip", "msa_decode.hip", "msa_kl.hip",
           "msa_bwd.hip", "msa_dense.hip", "msa_fp8.hip"]
# the launch hooks: no-ops in the product library, HIP-event timing in the measurement build
HOOK_PRODUCT = "msa_prof_off.cpp"
HOOK_TIMED = "msa_timing.cpp"

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def hipcc() -> str:
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src),
           "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 target feature; that warning is expected
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _link(out: str, objs) -> None:
    tmp = out + ".tmp"
    subprocess.check_call([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, out)


def build(jobs: int = 8) -> str:
    """Compile every source and link libmsa.so (the product) and libmsa_timed.so (the same
    objects with the kernel-timing hook, for measurement tools); always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES + [HOOK_PRODUCT, HOOK_TIMED]))
    common, hook_off, hook_timed = objs[:-2], objs[-2], objs[-1]
    _link(OUT, common + [hook_off])
    _link(OUT_TIMED, common + [hook_timed])
    return OUT


if __name__ == "__main__":
    print(build())
