"""Build libdust.so (the HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m activation_perturbation_es_amd.build [--force]

Objects go to activation_perturbation_es_amd/_build/; the shared library is written next to this
file, where the Python binding loads it from.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdust.so")
INCLUDE = os.path.join(ROOT, "include")

SOURCES = ["dust_api.cpp", "noise.hip", "delta_scan.hip", "error_estimate.hip",
           "weight_grad.hip", "head_ce.hip", "optim.hip", "attn_scores.hip",
           "perturbed_linear.hip"]
HEADERS = [os.path.join(CSRC, h) for h in ("dust_noise.hpp", "dust_internal.hpp")] + \
          [os.path.join(INCLUDE, "dust.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 instructions (v_pk_add/mul/fma_f32), which the compiler would otherwise form from
# scalar or float2 code, are disabled for all device code; the host pass warns that it does not
# know the feature, which is harmless.
FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-I", INCLUDE, "-I", CSRC,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


# Per-source additions. attn_scores.hip reads its matrix-core results with plain vector
# instructions, so its MFMAs accumulate in VGPRs (no v_accvgpr_read per result element).
SOURCE_FLAGS = {"attn_scores.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


PROBES_SRC = "probes.hip"
PROBES_LIB = os.path.join(PKG, "libdust_probes.so")


def build_probes() -> str:
    """Compile the ceiling probes (bench.py --ceilings) into libdust_probes.so."""
    os.makedirs(BUILD, exist_ok=True)
    tmp = PROBES_LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-shared", os.path.join(CSRC, PROBES_SRC), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (PROBES_SRC, " ".join(cmd), r.stderr))
    os.replace(tmp, PROBES_LIB)
    return PROBES_LIB


def build(force: bool = True) -> str:
    """Compile every source and link libdust.so. Always recompiles when force is True."""
    os.makedirs(BUILD, exist_ok=True)
    if not force and os.path.exists(LIB):
        newest = max(os.path.getmtime(p) for p in
                     [os.path.join(CSRC, s) for s in SOURCES] + HEADERS)
        if os.path.getmtime(LIB) >= newest:
            return LIB
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force="--force" in sys.argv or True))
