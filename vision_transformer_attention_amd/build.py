"""Build librpe_attn.so (and the roof microbenchmarks, librpe_roofs.so) for
gfx950 in-tree with hipcc.

Run ``python -m vision_transformer_attention_amd.build`` (or call ``build()``).
The libraries land next to this file and are loaded by the ctypes bindings.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "librpe_attn.so")
ROOFS_LIB = os.path.join(HERE, "librpe_roofs.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed-FP32 instructions are kept out of the device code on purpose; MFMA
# operands and accumulators stay in ordinary VGPRs (no AGPR round trips
# between the matrix products and the softmax arithmetic).
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans"]
SOURCES = ["plan.cpp", "api.cpp", "kernels.hip", "bwd.hip", "fwd_dispatch.cpp",
           "fwd_bf16_d16.hip", "fwd_bf16_d32.hip", "fwd_bf16_d64.hip",
           "fwd_f32_d16.hip", "fwd_f32_d32.hip", "fwd_f32_d64.hip",
           "fwd_cross_bf16_d16.hip", "fwd_cross_bf16_d32.hip", "fwd_cross_bf16_d64.hip",
           "fwd_cross_f32_d16.hip", "fwd_cross_f32_d32.hip", "fwd_cross_f32_d64.hip",
           "fwd_und_bf16_d16.hip", "fwd_und_bf16_d32.hip", "fwd_und_bf16_d64.hip",
           "fwd_und_f32_d16.hip", "fwd_und_f32_d32.hip", "fwd_und_f32_d64.hip"]
ROOFS_SOURCES = ["roofs.hip"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose=True):
    os.makedirs(OBJ, exist_ok=True)
    jobs = []
    for src in SOURCES + ROOFS_SOURCES:
        obj = os.path.join(OBJ, src + ".o")
        jobs.append(([HIPCC] + HIP_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj], obj))
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 4)) as ex:
        list(ex.map(lambda j: _run(j[0], verbose), jobs))
    for lib, srcs in ((LIB, SOURCES), (ROOFS_LIB, ROOFS_SOURCES)):
        tmp = lib + ".tmp"
        objs = [os.path.join(OBJ, s + ".o") for s in srcs]
        _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs, verbose)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
