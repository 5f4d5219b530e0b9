"""Build libqsa.so for gfx950 with hipcc (objects in _build/, library in-tree).

    python -m sparse_attention_block_scores_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIBRARY = os.path.join(PKG, "libqsa.so")
SOURCES = ["qsa_api.hip", "topk_kernels.hip", "topk_filter.hip", "scores_kernel.hip", "attn_kernels.hip"]
HEADERS = ["qsa_internal.h", "topk_device.h", "topk_select.h", "scores_device.h"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # Packed FP32 ALU instructions are kept out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]
# The top-k kernels issue their few workgroup atomics from one lane; the
# compiler's atomic optimizer would wrap each in a wave-wide reduction loop
# (scalar instructions the tail pays for in every wave).
SOURCE_FLAGS = {
    "topk_kernels.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"],
    "topk_filter.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"],
}


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    procs = []
    objects = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objects.append(obj)
        cmd = [hipcc(), *HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the GPU-only feature flag; that note is expected.
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]
        if lines and (verbose or p.returncode != 0):
            print("\n".join(lines), file=sys.stderr)
        if p.returncode != 0:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIBRARY + ".tmp"
    subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objects, "-o", tmp], check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
