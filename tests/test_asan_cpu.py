"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

The HIP library's host side (argument checks, workspace sizing, dispatch
decisions up to the first launch) is compiled host-only with the sanitizers,
the CPU oracle with the same, and both are linked into tests/asan_driver.c,
which exercises every check that returns before a launch and runs the oracle
over small random cases.  No GPU, no device code."""
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
CLANGXX = "/opt/rocm/llvm/bin/clang++"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain not found")
def test_host_code_and_oracle_clean_under_sanitizers(tmp_path):
    inc = os.path.join(ROOT, "include")
    srcs = sorted(glob.glob(os.path.join(ROOT, "segmented_gather_rank_amd", "csrc", "*.hip")))
    from concurrent.futures import ThreadPoolExecutor

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        # the device code is built as usual (the objects carry it); each
        # sanitizer flag is scoped to the host pass
        subprocess.run([HIPCC, "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-fPIC", f"-I{inc}",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                        "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                        "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all",
                        "-c", src, "-o", obj], check=True, capture_output=True)
        return obj

    with ThreadPoolExecutor(max(1, min(len(srcs), os.cpu_count() or 1))) as pool:
        objs = list(pool.map(compile_one, srcs))
    san = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all", "-g", "-O1"]
    for name, src in (("oracle.o", os.path.join(ROOT, "oracle", "lora_oracle.c")),
                      ("driver.o", os.path.join(ROOT, "tests", "asan_driver.c"))):
        subprocess.run([CLANG, "-std=c99", *san, f"-I{inc}", "-c", src, "-o", str(tmp_path / name)],
                       check=True, capture_output=True)
        objs.append(str(tmp_path / name))
    exe = str(tmp_path / "asan_driver")
    subprocess.run([CLANGXX, *san, "-o", exe, *objs, "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,/opt/rocm/lib"], check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-8000:]
    assert "all checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-8000:]
