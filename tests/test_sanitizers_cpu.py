"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The oracle (anchor_oracle.c) is rebuilt with gcc's -fsanitize=address,undefined (UB
  fatal) and its pin tests run against that build in a child process.
* The C ABI's host code (anchor_attn_api.cpp) is rebuilt with the sanitizers on its host
  side only and linked with the library's other objects; the CPU ABI tests (argument
  checks, NULL handling, the missing-device path) run against that build.

The child processes preload the sanitizer runtime (Python itself is not instrumented);
leak checking is off because the interpreter keeps its allocations until exit.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "efficient_vision_transformer_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run_tests(env_extra, files):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider", *files],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    print(r.stdout[-3000:], r.stderr[-3000:])
    assert r.returncode == 0, "tests failed under the sanitizers"
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr


def test_oracle_under_asan_and_ubsan(tmp_path):
    lib = str(tmp_path / "libanchor_oracle_asan.so")
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
                    "-ffp-contract=off", "-fPIC", "-shared", "-Wall",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-o", lib, os.path.join(ROOT, "oracle", "anchor_oracle.c"),
                    "-lm", "-lpthread"], check=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True, check=True).stdout.strip()
    _run_tests({"ANCHOR_ORACLE_LIB": lib, "LD_PRELOAD": asan},
               ["tests/test_oracle_pins.py", "tests/test_oracle_backward_pins.py",
                "tests/test_oracle_block_pins.py"])


def test_host_library_under_asan_and_ubsan(tmp_path):
    objs = [os.path.join(CSRC, "_build", f) for f in sorted(os.listdir(os.path.join(CSRC, "_build")))
            if f.endswith(".o") and f != "anchor_attn_api.o"] if os.path.isdir(
                os.path.join(CSRC, "_build")) else []
    if len(objs) < 8:
        from efficient_vision_transformer_amd import build
        build.build()
        objs = [os.path.join(CSRC, "_build", f) for f in sorted(os.listdir(os.path.join(CSRC, "_build")))
                if f.endswith(".o") and f != "anchor_attn_api.o"]
    api = str(tmp_path / "anchor_attn_api_asan.o")
    # host-side instrumentation only: every sanitizer flag follows -Xarch_host
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *san,
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-x", "hip", "-c",
                    os.path.join(CSRC, "anchor_attn_api.cpp"), "-o", api], check=True)
    lib = str(tmp_path / "libanchor_attn_asan.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib, api, *objs,
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-shared-libsan", "-L/opt/rocm/lib", "-lhipblaslt",
                    "-Wl,-rpath,/opt/rocm/lib"], check=True)
    rt = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"],
                        capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(rt) or not os.path.exists(rt):
        import glob
        cands = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        if not cands:
            pytest.fail("clang's ASan runtime was not found")
        rt = cands[0]
    _run_tests({"ANCHOR_ATTN_LIBRARY": lib, "LD_PRELOAD": rt}, ["tests/test_abi_cpu.py"])
