"""Build libsinkattn.so in-tree for gfx950 with hipcc.

Usage: python -m softmax_sink_amd.build  (or softmax_sink_amd.build.build()).
Every call recompiles every source. The library lands next to this file.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsinkattn.so")
OBJDIR = os.path.join(ROOT, "_build")
SOURCES = ["schedule.cpp", "metadata.cpp", "api.cpp", "fwd_bf16.hip", "bwd_bf16.hip", "f32_path.hip",
           "merge.hip"]
ARCH = os.environ.get("SINK_ATTN_ARCH", "gfx950")
# Per-source compiler flags. The backward kernels are scheduled with the
# max-ILP machine scheduler: same instructions and results bit for bit, and
# the dK/dV kernel 2.4% faster on the long causal training workload (3.238 ->
# 3.160 ms, median of six alternating passes); the forward gained nothing
# from it and keeps the default scheduler.
SOURCE_FLAGS = {
    "bwd_bf16.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
}


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-I", os.path.join(ROOT, "include"),
            # packed fp32 VALU ops are kept out of the device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument"]


def _compile(src):
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [hipcc()] + flags()
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += SOURCE_FLAGS.get(src, [])
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose=False):
    os.makedirs(OBJDIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
