"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only, no GPU touched): the library's sources are compiled for gfx950
with the sanitizers on the host side only, linked with
tests/host/qsa_host_checks.cpp, and run. The driver sweeps the plan and
workspace-size entry points over valid and far-out-of-range arguments and
calls every entry point with arguments it must reject before any launch; any
sanitizer report or failed expectation makes it exit non-zero."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "sparse_attention_block_scores_amd", "csrc")
UNITS = ["qsa_api", "topk_kernels", "topk_filter", "scores_kernel", "attn_kernels"]
CLANG = "/opt/rocm/llvm/bin/clang++"


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ... failed:\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.mark.skipif(shutil.which("hipcc") is None or not os.path.exists(CLANG), reason="needs hipcc and clang++")
def test_host_code_under_sanitizers(tmp_path):
    inc = os.path.join(ROOT, "include")
    objs = [str(tmp_path / f"{u}.o") for u in UNITS]

    def compile_unit(u, o):
        _run(["hipcc", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", f"-I{inc}",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
              "-Xarch_host", "-fno-sanitize-recover=all", "-c", os.path.join(SRC, f"{u}.hip"), "-o", o])

    with ThreadPoolExecutor(max_workers=len(UNITS)) as ex:
        list(ex.map(compile_unit, UNITS, objs))
    drv = str(tmp_path / "drv.o")
    _run([CLANG, "-O1", "-g", "-std=c++17", f"-I{inc}", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-c",
          os.path.join(ROOT, "tests", "host", "qsa_host_checks.cpp"), "-o", drv])
    exe = str(tmp_path / "host_checks")
    _run([CLANG, "-fsanitize=address,undefined", drv, *objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1",
               HIP_VISIBLE_DEVICES="")
    r = _run([exe], env=env, timeout=600)
    assert "failures 0" in r.stdout, r.stdout
