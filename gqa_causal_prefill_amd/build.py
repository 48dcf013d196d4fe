"""Compile the HIP sources of this package for gfx950 with hipcc.

Produces, next to this file:
  libgqa_prefill.so       the C-ABI library declared in include/gqa_prefill.h
  libgqa_layout_probe.so  a test-only library with one MFMA per entry point, used
                          to check the CPU model of the gfx950 MFMA register layouts
"""

from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")

LIB = os.path.join(PKG, "libgqa_prefill.so")
PROBE_LIB = os.path.join(PKG, "libgqa_layout_probe.so")
# the same library with 32 query columns per wave (64 tokens x 2 heads per workgroup)
# instead of 48: tests compare the two for bitwise-identical output
QB2_LIB = os.path.join(PKG, "libgqa_prefill_qb2.so")

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in any generated code.
# -amdgpu-mfma-vgpr-form: MFMA accumulators in architectural VGPRs where they fit. The
#   attention kernel's softmax reads every score accumulator with vector ALU
#   instructions, which cannot address AGPRs; in the AGPR form the compiler moves
#   each one (and, short of AGPRs, part of the output accumulator) between the two
#   files on every tile.
# -amdgpu-sched-strategy=max-ilp: the machine scheduler favours instruction-level
#   parallelism over register pressure (the kernel runs one wave per SIMD at any
#   register count). Measured 1.5% faster on the bf16 prefill loop, neutral with INT8
#   keys.
HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-mllvm", "-amdgpu-sched-strategy=max-ilp",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _start(sources, output, defines=()):
    cmd = [hipcc(), *HIPCC_FLAGS, *defines, f"-I{INCLUDE}", "-o", output + ".tmp", *sources]
    proc = subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    return cmd, proc, output


def _finish(job, verbose=False):
    cmd, proc, output = job
    text, _ = proc.communicate()
    msgs = [ln for ln in text.splitlines() if "not a recognized feature" not in ln]
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(output + ".tmp", output)


def build(verbose: bool = False) -> None:
    """Compile the libraries (always, even if they exist), the three in parallel."""
    src = os.path.join(CSRC, "gqa_prefill.hip")
    jobs = [_start([src], LIB),
            _start([src], QB2_LIB, ("-DGQA_DEFAULT_QB=2",)),
            _start([os.path.join(CSRC, "layout_probe.hip")], PROBE_LIB)]
    errors = []
    for job in jobs:
        try:
            _finish(job, verbose)
        except RuntimeError as e:
            errors.append(str(e))
    if errors:
        raise RuntimeError("\n\n".join(errors))


VARIANT_DIR = os.path.join(PKG, "variants")


def build_variant(name: str, defines) -> str:
    """Build the library with extra preprocessor definitions (tuning constants such as
    -DGQA_VT_DEPTH=4) as variants/libgqa_prefill_<name>.so, for comparing a tuning
    choice with bench.py --library; returns its path. Not used by the library itself."""
    os.makedirs(VARIANT_DIR, exist_ok=True)
    out = os.path.join(VARIANT_DIR, f"libgqa_prefill_{name}.so")
    _finish(_start([os.path.join(CSRC, "gqa_prefill.hip")], out, tuple(defines)))
    return out


if __name__ == "__main__":
    build(verbose=True)
    print("built", LIB, "and", PROBE_LIB)
