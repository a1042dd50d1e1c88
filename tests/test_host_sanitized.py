"""The library's host code and the scalar C oracle under AddressSanitizer,
UndefinedBehaviorSanitizer and LeakSanitizer, on the CPU.

layout.cpp and capi.cpp (the C ABI's host side: layout, segment tables,
arena plan, argument checks, loss-scale control) and oracle/zero_oracle.c are
compiled with g++/gcc and -fsanitize=address,undefined, linked with
tests/host_sanitize_driver.cpp (stubs for the kernel launches, which a
host-only build leaves out and nothing here reaches) and run without a
device.  Any sanitizer report fails the run.  Leaks inside the HIP runtime's
own libraries are suppressed; the library's are not."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sharded_zero_partition_amd", "csrc")
ROCM = "/opt/rocm"
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(f"{ROCM}/include/hip"),
                    reason="needs g++ and the HIP headers")
def test_host_code_and_oracle_are_sanitizer_clean(tmp_path):
    inc = ["-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{ROOT}/include", f"-I{CSRC}"]
    objs = []
    for src in ("layout.cpp", "capi.cpp"):
        obj = str(tmp_path / (src + ".o"))
        subprocess.check_call(["g++", "-std=c++17", *SAN, *inc, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    obj = str(tmp_path / "zero_oracle.o")
    subprocess.check_call(["gcc", "-std=c11", *SAN, "-ffp-contract=off", "-c",
                           os.path.join(ROOT, "oracle", "zero_oracle.c"), "-o", obj])
    objs.append(obj)
    exe = str(tmp_path / "driver")
    subprocess.check_call(["g++", "-std=c++17", *SAN, *inc,
                           os.path.join(ROOT, "tests", "host_sanitize_driver.cpp"), *objs,
                           f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-lm", "-o", exe])
    supp = tmp_path / "lsan.supp"
    supp.write_text("leak:libamdhip64\nleak:libhsa-runtime64\nleak:libamd_comgr\n")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               LSAN_OPTIONS=f"suppressions={supp}", UBSAN_OPTIONS="print_stacktrace=1")
    out = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stdout[-2000:] + out.stderr[-4000:]
    assert out.stdout.strip().endswith("OK")
    assert "runtime error" not in out.stderr and "ERROR: AddressSanitizer" not in out.stderr
