"""Compiles libbimamba.so (HIP for gfx950) in-tree.

Every translation unit under csrc/ is compiled with hipcc for gfx950 only,
in parallel, into ``_build/``, then linked into
``bidirectional_mamba_ssm_amd/libbimamba.so``. Packed-fp32 VALU ops are
disabled for the device code (the compiler must not form v_pk_*_f32).
"""
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libbimamba.so")
ARCH = "gfx950"


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def compile_flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    hipcc = _hipcc()
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) +
                  glob.glob(os.path.join(CSRC, "*.cpp")))
    objs, procs = [], []
    for src in srcs:
        obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
        cmd = [hipcc] + compile_flags() + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                            stderr=subprocess.STDOUT)))
        objs.append(obj)
        while len([p for _, p in procs if p.poll() is None]) >= jobs:
            procs[0][1].wait()
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # the host pass does not know the packed-fp32 feature; that note is noise
        lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l]
        if p.returncode != 0:
            failed.append(src)
            sys.stderr.write("\n".join(lines) + "\n")
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        raise RuntimeError("compilation failed: " + ", ".join(failed))
    tmp = LIB + ".tmp"
    cmd = [hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
