"""Host code under sanitizers (CPU only, no GPU needed).

* The fp64 oracle (oracle/ssd_oracle.c, with its worker threads) is built with
  AddressSanitizer + UndefinedBehaviorSanitizer and, separately, with
  ThreadSanitizer, together with tests/sanitize/oracle_driver.c, which runs
  every oracle entry point on small random inputs, edge cases and argument
  errors.
* The HIP library's host code (argument checks, plans, workspace layout) is
  built with AddressSanitizer + UndefinedBehaviorSanitizer on the host side
  only (device code is compiled as usual and never launched here), and
  tests/sanitize/abi_driver.c calls every entry point on the paths that need no
  GPU: plans and workspace sizes over a sweep of shapes up to sizes where the
  size arithmetic could overflow, status texts, and argument checks.
A sanitizer report fails the test.
"""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ORACLE_C = os.path.join(ROOT, "oracle", "ssd_oracle.c")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", TSAN_OPTIONS="halt_on_error=1")


def _gcc_can(flag, tmp):
    src = os.path.join(tmp, "probe.c")
    with open(src, "w") as f:
        f.write("int main(void) { return 0; }\n")
    r = subprocess.run(["gcc", flag, src, "-o", os.path.join(tmp, "probe")], capture_output=True)
    return r.returncode == 0


def _run(exe, env):
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    for bad in ("ERROR: AddressSanitizer", "runtime error:", "WARNING: ThreadSanitizer",
                "ERROR: LeakSanitizer"):
        assert bad not in out, out[-4000:]
    return out


@pytest.mark.parametrize("flags", [["-fsanitize=address,undefined", "-fno-omit-frame-pointer"],
                                   ["-fsanitize=thread"]], ids=["asan_ubsan", "tsan"])
def test_oracle_under_sanitizers(tmp_path, flags):
    if not _gcc_can(flags[0], str(tmp_path)):
        pytest.skip(f"gcc has no {flags[0]} runtime here")
    exe = str(tmp_path / "oracle_driver")
    subprocess.run(["gcc", "-g", "-O1", *flags, ORACLE_C, os.path.join(SAN, "oracle_driver.c"),
                    "-lm", "-lpthread", "-o", exe], check=True)
    assert "every check passed" in _run(exe, ENV)


def test_library_host_code_under_asan_ubsan(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    clang = "/opt/rocm/llvm/bin/clang"
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("no hipcc / ROCm clang here")
    csrc = os.path.join(ROOT, "structured_state_space_ssd_amd", "csrc")
    inc = os.path.join(ROOT, "include")
    san = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Wno-unused-command-line-argument", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", *san, f"-I{inc}", f"-I{csrc}"]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([hipcc, *flags, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    srcs = sorted(glob.glob(os.path.join(csrc, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 2)) as ex:
        objs = list(ex.map(compile_one, srcs))
    lib = str(tmp_path / "libssd_san.so")
    subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host",
                    "-fsanitize=address,undefined", *objs, "-o", lib], check=True,
                   capture_output=True)
    exe = str(tmp_path / "abi_driver")
    subprocess.run([clang, "-g", "-O1", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                    f"-I{inc}", os.path.join(SAN, "abi_driver.c"), lib,
                    f"-Wl,-rpath,{tmp_path}", "-o", exe], check=True)
    # the HIP runtime's own allocations are not this library's: leaks are not checked here
    env = dict(ENV, ASAN_OPTIONS="detect_leaks=0")
    assert "every check passed" in _run(exe, env)
