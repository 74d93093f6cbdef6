"""The C ABI's argument handling under the address and undefined-behaviour sanitizers (CPU only).

tests/abi_driver.cpp is compiled with the boundary's source (rsq_api.hip,
host code only) and replaces the kernel launchers by recorders; the test
builds it with the sanitizers on the host code and runs it. It covers every
entry point's checks, that nothing is launched after a failed check, that
arguments reach the launcher, and that a launch failure maps to RSQ_ERR_HIP.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang++")


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not found")
def test_abi_argument_checks_under_sanitizers(tmp_path):
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    common = ["-std=c++17", "-O1", "-g", "--cuda-host-only", "-x", "hip", f"-I{os.path.join(ROOT, 'include')}"]
    objs = []
    for src in (os.path.join(ROOT, "rotation_bit_post_amd", "csrc", "rsq_api.hip"),
                os.path.join(ROOT, "tests", "abi_driver.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        res = subprocess.run([HIPCC, *common, *host_san, "-c", src, "-o", obj], capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-4000:]
        objs.append(obj)
    exe = str(tmp_path / "abi_driver")
    link = [CLANG, "-fsanitize=address,undefined", *objs, f"-L{os.path.join(ROCM, 'lib')}", "-lamdhip64",
            f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe]
    res = subprocess.run(link, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-4000:]
    assert res.stdout.strip().startswith("ok:"), res.stdout
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr[-4000:]
