"""Build libsms.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m attention_softmax_amd.build

Compiles each translation unit with hipcc in parallel and links the shared
library next to this file. Every call rebuilds.
"""

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsms.so")

SOURCES = ["api.hip", "inst_f32.hip", "inst_f16.hip", "inst_bf16.hip", "inst_f64.hip",
           "attention.hip", "attention_bwd.hip", "attention_api.hip", "copy_ref.hip"]
ARCH = "gfx950"

# Per-source flags. The attention backward's MFMAs keep their accumulators in
# ordinary VGPRs: with the compiler's default (AGPR accumulators) the D = 64
# dK/dV kernel copied an accumulator out of AGPRs at its loop head three wait
# states after the MFMA that wrote it (an 8-pass MFMA needs 11), and the copy
# read a stale value (isa_check.py finds such reads).
EXTRA_FLAGS = {"attention_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def common_flags():
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Wall",
        "-Wno-unused-function",
        # Keep the compiler from forming packed fp32 instructions.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        f"-I{INCLUDE}",
        f"-I{CSRC}",
    ]


def source_flags(src):
    """Every hipcc flag the build uses for one source file."""
    return common_flags() + EXTRA_FLAGS.get(src, [])


def device_asm(src, out):
    """Compile one source's gfx950 device code to assembly at ``out``, with the
    build's flags (for inspection; the build itself does not need it)."""
    cmd = [hipcc()] + source_flags(src) + ["--cuda-device-only", "-S", os.path.join(CSRC, src),
                                           "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stderr}")
    return out


def _compile(src):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + source_flags(src) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that line.
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = min(len(SOURCES), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
