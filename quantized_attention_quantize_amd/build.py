"""Build libqattn.so (the HIP kernels and the C ABI) and libqaprobe.so (the
measurement probes of qa_probe.h) in-tree for gfx950.

Usage: python quantized_attention_quantize_amd/build.py [--verbose]
(run by path: importing the package needs the library this builds)
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libqattn.so")
SOURCES = ["api.hip", "quantize.hip", "decode.hip", "flash.hip", "prefill_fp8.hip"]
PROBE_LIB = os.path.join(PKG, "libqaprobe.so")
PROBE_SOURCES = ["probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
    # no packed fp32 instructions anywhere (they are not trusted on this part)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-rdc", "-Wall", "-Wno-unused-result",
    f"-I{os.path.join(ROOT, 'include')}",
]


# The probes measure instruction rates: their accumulators live in ordinary
# VGPRs (with AGPR accumulators the compiler rotates the 16x16 accumulators
# through copies inside the loops, which then measure the copies).
EXTRA = {"probe.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         # the softmax maxima: IEEE mode off lets v_max_f32 take its inputs as
         # they are, instead of quieting possible signaling NaNs first (one
         # extra instruction per score); the kernels never see a NaN score
         "prefill_fp8.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans"],
         "flash.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans"]}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr)
    # the host pass does not know the gfx950-only feature flag; that note is harmless
    lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines))
    return obj


def _link(lib: str, objs: list) -> None:
    tmp = lib + ".tmp"
    r = subprocess.run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every kernel source for gfx950 and link libqattn.so and
    libqaprobe.so (always rebuilds). Returns the attention library's path."""
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(OBJ, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1)) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
    _link(LIB, [objs[s] for s in SOURCES])
    _link(PROBE_LIB, [objs[s] for s in PROBE_SOURCES])
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
