"""Compile the HIP sources under csrc/ into libattn.so (gfx950 only), in-tree.

Run as ``python -m causal_softmax_attention_amd._build``.  Every source is
compiled with hipcc for --offload-arch=gfx950 with packed-FP32 instruction
selection switched off (the host pass warns that it does not know the feature;
that warning is harmless), then linked into one shared library next to this
file.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["attn_api.hip", "attn_rowwise.hip", "attn_fwd_bf16.hip", "attn_bwd_bf16.hip",
           "attn_bwd_dq_bf16.hip", "attn_fwd_f32.hip", "attn_loss.hip", "nw.hip", "attn_table.hip",
           "attn_project.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics", "-fvisibility=hidden",
]

# Per-source additions.  The dQ pass is built with MFMA results in VGPRs
# (-amdgpu-mfma-vgpr-form), where its softmax reads them with plain VALU
# instructions; at two waves per SIMD (256 registers each) no accumulator then
# moves between AGPRs and VGPRs.  The other kernels get that placement from the
# compiler's defaults.
EXTRA = {
    "attn_bwd_dq_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
