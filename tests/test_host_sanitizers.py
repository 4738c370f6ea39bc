"""The host entry points of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

sdv2.cpp is compiled with the sanitizers on its host code only (the device code of the file is
built as usual and never run) and linked with tests/host_sanitize_driver.cpp, which calls
validation, layout, sizes, the schedule, the noise schedule, the latency fit and SLO choice,
and the error paths that return before any HIP call.  CPU only; any report aborts the driver.
"""
import os
import pathlib
import subprocess

import pytest

ROOT = pathlib.Path(__file__).resolve().parents[1]
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all"]


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang++ is not installed")
def test_host_entry_points_are_clean_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "host_sanitize"
    compile_cmd = [CLANG, "-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-O1", "-g",
                   "-fno-omit-frame-pointer", *SAN,
                   "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                   "-I", str(ROOT / "include"), "-I", str(ROOT / "rolling_kv_causal_amd" / "csrc"), "-c"]
    objs = []
    for src in (ROOT / "rolling_kv_causal_amd" / "csrc" / "sdv2.cpp", ROOT / "tests" / "host_sanitize_driver.cpp"):
        obj = tmp_path / (src.stem + ".o")
        r = subprocess.run(compile_cmd + [str(src), "-o", str(obj)], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        objs.append(str(obj))
    # host link of the two objects with the sanitizer runtimes
    link = [CLANG, "--hip-link", "-fsanitize=address,undefined", *objs, "-o", str(exe),
            "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(link, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-6000:]
    assert "clean under ASan + UBSan" in r.stdout
