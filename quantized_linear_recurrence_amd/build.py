"""Build liblores.so (HIP kernels for gfx950 + host C ABI) in-tree.

    python -m quantized_linear_recurrence_amd.build [--jobs N] [--save-temps]

Each translation unit is compiled by hipcc in parallel into _build/, then
linked into quantized_linear_recurrence_amd/liblores.so.
"""
import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(os.path.dirname(PKG), "_build")
LIB = os.path.join(PKG, "liblores.so")
ARCH = "gfx950"

SOURCES = ["lores_api.cpp", "lores_aux.hip", "lores_step_int8.hip", "lores_step_int4.hip",
           "lores_step_int6.hip", "lores_step_fp8.hip", "lores_step_bf16.hip", "lores_step_fp32.hip",
           "lores_step_int8_int4.hip", "lores_step_int4_int6.hip", "lores_step_bf16_int8.hip",
           "lores_step_bf16_int4.hip", "lores_step_key_int8.hip", "lores_step_key_int4.hip",
           "lores_step_key_int6.hip", "lores_step_key_fp8.hip", "lores_window.hip",
           "lores_window_int8.hip", "lores_window_int4.hip", "lores_window_int6.hip",
           "lores_window_fp8.hip"]

COMMON = [
    "-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
    # no implicit contraction: every fused multiply-add is an explicit fmaf
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # fully unroll the per-element loops (register-resident rows) even where
    # the unrolled body is large
    "-mllvm", "-pragma-unroll-threshold=1000000",
    # no packed fp32 instructions in any GPU code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build liblores.so")
    return path


def _compile(src, save_temps):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    if save_temps:
        cmd.insert(1, "-save-temps=obj")
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=BUILD)
    errs = "\n".join(l for l in (r.stderr or "").splitlines()
                     if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    return obj, errs


def build(jobs=None, save_temps=False, verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, save_temps), SOURCES))
    for _, errs in results:
        if errs.strip() and verbose:
            print(errs, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *[o for o, _ in results], "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--save-temps", action="store_true")
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.save_temps, a.verbose))


if __name__ == "__main__":
    main()
