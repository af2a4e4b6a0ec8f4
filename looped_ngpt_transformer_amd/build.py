"""Build the HIP library libdory.so in-tree for gfx950 (hipcc, one object per source).
The compiler's per-kernel resource report (registers, spills, scratch, occupancy, LDS)
is kept in _build/kernel_resources.json."""
from __future__ import annotations

import json
import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdory.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["runtime.cpp", "k_update.hip", "k_rope.hip", "k_attn.hip", "k_attn_prefill.hip", "k_mlp.hip", "k_gemm.hip", "k_vocab.hip", "k_nvfp4.hip"]

FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         # packed fp32 VALU ops are kept off for every device pass
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-result", "-Rpass-analysis=kernel-resource-usage"]
RESOURCES = os.path.join(OBJ, "kernel_resources.json")
_FIELDS = {"VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch",
           "VGPRs Spill": "vgpr_spill", "SGPRs Spill": "sgpr_spill",
           "Occupancy [waves/SIMD]": "occupancy", "LDS Size [bytes/block]": "lds"}


def _resources(stderr: str) -> dict:
    """Per-kernel fields from the kernel-resource-usage remarks of one compile."""
    out, cur = {}, None
    for line in stderr.splitlines():
        m = re.search(r"remark: +Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark: +([A-Za-z ]+(?:\[[^\]]*\])?): (\d+)", line)
        if cur is not None and m and m.group(1).strip() in _FIELDS:
            cur[_FIELDS[m.group(1).strip()]] = int(m.group(2))
    return out


def _compile(src: str):
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj, _resources(r.stderr)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        done = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in done]
    res = {}
    for _, r in done:
        res.update(r)
    with open(RESOURCES, "w") as f:
        json.dump(res, f, indent=1, sort_keys=True)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
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
