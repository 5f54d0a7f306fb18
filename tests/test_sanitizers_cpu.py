"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code:
the oracle (plain C, gcc) driven over its paths, and the library's host-side
argument validation (api.cpp and the no-allocation entry point, built with
hipcc's clang, sanitizers on the host side only) driven through every entry
point with malformed arguments. CPU only: no call reaches the GPU."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "bidirectional_mamba_ssm_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                    os.path.join(ROOT, "oracle", "ssd_oracle.c"), os.path.join(HERE, "oracle_main.c"),
                    "-o", exe, "-lm"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, env=dict(ENV, ASAN_OPTIONS="detect_leaks=1"),
                       timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr, r.stderr
    assert "oracle sanitized runs: ok" in r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_host_validation_under_asan_ubsan(tmp_path):
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include")]
    objs = []
    # the host-side entry points with the sanitizers; the kernel files as built
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp"))):
        base = os.path.basename(src)
        obj = str(tmp_path / (base + ".o"))
        if base in ("api.cpp", "noalloc.hip"):
            subprocess.run([HIPCC] + flags + SAN + ["-c", src, "-o", obj], check=True,
                           capture_output=True)
        else:
            built = os.path.join(ROOT, "_build", base + ".o")
            if os.path.exists(built):
                shutil.copy(built, obj)
            else:
                subprocess.run([HIPCC] + flags + ["-O3", "-c", src, "-o", obj], check=True,
                               capture_output=True)
        objs.append(obj)
    lib = str(tmp_path / "libbimamba_asan.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib] + objs,
                   check=True, capture_output=True)
    exe = str(tmp_path / "abi_asan")
    subprocess.run(["/opt/rocm/llvm/bin/clang", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
                    os.path.join(HERE, "abi_main.c"), lib, "-Wl,-rpath," + str(tmp_path),
                    "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe],
                   check=True)
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr, r.stderr
    assert "abi sanitized checks: ok" in r.stdout, r.stdout
