"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the host code.

- The CPU oracle (oracle/oracle.c), driven through every entry point and mode
  by tests/sanitize/oracle_driver.c (gcc, with the leak checker).
- The C ABI's host side (csrc/sv_api.hip: argument checks, capacity checks,
  the choice of passes, grid sizing, post_update, draft-side, LM-head and
  debug entry points, the allocation-free entry point's checks), with the
  sanitizers on the host pass only and the kernel launchers stubbed, driven by
  tests/sanitize/host_driver.cpp.  No GPU is involved: the stubs record what
  would have been launched.

CPU only; each build takes a few seconds."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r.stdout


def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    sanitizers = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off", *sanitizers,
         f"-I{ROOT}/oracle", f"{ROOT}/oracle/oracle.c", f"{SAN}/oracle_driver.c", "-lm", "-o", exe])
    out = run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1"))
    assert out.strip().endswith("ok")


@pytest.mark.skipif(not os.path.exists(os.path.join(ROCM, "bin", "hipcc")), reason="needs hipcc")
def test_host_api_under_asan_and_ubsan(tmp_path):
    obj = str(tmp_path / "host_driver.o")
    exe = str(tmp_path / "host_driver")
    # every sanitizer flag applies to the host pass only (the device pass
    # compiles the library's device-side data and nothing of the driver)
    compile_cmd = [os.path.join(ROCM, "bin", "hipcc"), "-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-O1",
                   "-g", "-fno-omit-frame-pointer"]
    for flag in ("address", "undefined"):
        compile_cmd += ["-Xarch_host", "-fsanitize=" + flag]
    compile_cmd += ["-Xarch_host", "-fno-sanitize-recover=all", f"-I{ROOT}/include",
                    f"-I{ROOT}/rejection_sampling_verify_05_amd/csrc", "-c", f"{SAN}/host_driver.cpp", "-o", obj]
    run(compile_cmd)
    clang = os.path.join(ROCM, "llvm", "bin", "clang++")
    link_flags = ["-fsanitize=address,undefined"]
    run([clang, *link_flags, obj, f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", exe])
    out = run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1"))
    assert out.strip().endswith("ok")
