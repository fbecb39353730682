"""Build libdgmi.so (gfx950) in-tree with hipcc.

    python -m moe_grouped_gemm_x128_amd.build [--jobs N]

Every HIP source under csrc/ is compiled for gfx950 only, then linked with
the host-side ABI into moe_grouped_gemm_x128_amd/libdgmi.so.  Packed FP32
instructions are disabled on the device (-packed-fp32-ops) and FP32 division
is correctly rounded (the quantizers divide by the block scale).
"""

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdgmi.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["abi.cpp", "quant.hip", "gemm.hip", "moe.hip"]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-ffp-contract=fast",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device-only packed-fp32 feature; that warning is expected
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    return obj, r.returncode, err, cmd


def build(jobs=None, verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1, 8)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_compile, SOURCES))
    failed = False
    for obj, rc, err, cmd in results:
        if err.strip() and (verbose or rc != 0):
            sys.stderr.write(err + "\n")
        if rc != 0:
            sys.stderr.write("FAILED: " + " ".join(cmd) + "\n")
            failed = True
    if failed:
        raise RuntimeError("libdgmi build failed")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + [o for o, *_ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stderr)
        raise RuntimeError("libdgmi link failed")
    os.replace(tmp, LIB)
    return LIB


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args()
    print(build(args.jobs, args.verbose))


if __name__ == "__main__":
    main()
