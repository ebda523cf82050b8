"""Build libmxfp4.so for gfx950 with hipcc (in-tree, next to this file).

    python -m precision_mxfp4_producers_amd.build

Every HIP source is compiled with
  -O3 --offload-arch=gfx950 -ffp-contract=off
  -Xclang -target-feature -Xclang -packed-fp32-ops
no fused multiply-add contraction (the producers' rounding decisions are
defined by single fp32 roundings) and no packed-fp32 instruction selection.
"""

import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_NAME = "libmxfp4.so"
SOURCES = ["quantize.hip", "gemm.hip", "swiglu_bwd.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def lib_path():
    return os.path.join(HERE, LIB_NAME)


def build(verbose=False, jobs=4):
    """Compile every source and link the shared library; raises on failure."""
    objs = []
    with tempfile.TemporaryDirectory(prefix="mxfp4_build_") as tmp:
        procs = []
        for src in SOURCES:
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
            if len(procs) >= jobs:
                _wait(procs.pop(0))
        for p in procs:
            _wait(p)
        tmp_lib = lib_path() + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp_lib] + objs
        out = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        if out.returncode != 0:
            raise RuntimeError("link failed:\n" + out.stdout.decode())
        os.replace(tmp_lib, lib_path())
    return lib_path()


def _wait(item):
    src, p = item
    out, _ = p.communicate()
    text = out.decode()
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{text}")
    noise = [ln for ln in text.splitlines() if ln.strip() and "packed-fp32-ops" not in ln]
    if noise:
        sys.stderr.write(f"[{src}]\n" + "\n".join(noise) + "\n")


if __name__ == "__main__":
    print(build(verbose=True))
