"""Builds libvarattn.so in-tree with hipcc for gfx950.

Usage: ``python -m scale_wise_attention_amd.build`` (or ``build()``).  Every
source is compiled to an object under ``_build/`` in parallel, then linked
into ``scale_wise_attention_amd/libvarattn.so`` (replaced atomically).
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libvarattn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

SOURCES = ["attn_bf16.hip", "attn_fp8.hip", "attn_f32.hip", "quant_e4m3.hip", "tile_mask.hip", "scatter.hip", "saliency.hip", "dynamic_sparse.hip", "var_attn_api.cpp"]
# The attention kernels (bf16 and e4m3 q / k) run with the IEEE mode bit off and without NaN
# semantics (infinities stay honoured: masked logits are -inf): max/min then
# need no NaN-quieting instructions in the softmax.  Their MFMAs write VGPRs
# (S and O are read by VALU code); the kernel itself places the MFMA operands
# that stay resident (Q) or come from LDS (K, V^T) in AGPRs.
_ATTN_FLAGS = ["-mno-amdgpu-ieee", "-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"]
# (the quantiser shares the e4m3 conversion with the attention kernel that
# quantises its queries, so it is built in the same floating-point mode)
PER_FILE_FLAGS = {"attn_bf16.hip": _ATTN_FLAGS, "attn_fp8.hip": _ATTN_FLAGS, "quant_e4m3.hip": _ATTN_FLAGS}

ARCH = "gfx950"
COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    # packed fp32 VALU ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-Wall",
    "-Wno-unused-function",
]


def hipcc_path():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libvarattn.so)")


def _compile(hipcc, src, extra):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + COMMON_FLAGS + PER_FILE_FLAGS.get(src, []) + extra
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj, r.stderr


def build(verbose=False, extra_flags=()):
    hipcc = hipcc_path()
    os.makedirs(BUILD_DIR, exist_ok=True)
    extra = list(extra_flags)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(lambda s: _compile(hipcc, s, extra), SOURCES))
    objs = [o for o, _ in results]
    if verbose:
        for (_, err), s in zip(results, SOURCES):
            text = "\n".join(ln for ln in err.splitlines() if "packed-fp32-ops" not in ln)
            if text.strip():
                print(f"[{s}]\n{text}", file=sys.stderr)
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking {LIB_NAME} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    flags = sys.argv[1:]
    print(build(verbose=True, extra_flags=flags))
