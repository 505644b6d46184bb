"""Build libmoe.so in-tree with hipcc for gfx950 (no JIT, no site-packages)."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "_lib", "libmoe.so")
# (source, object, extra flags): the grouped GEMM is built twice, for large
# chunks and for mid-size batches
SOURCES = [("route.hip", "route.o", []), ("dispatch.hip", "dispatch.o", []),
           ("ffn_small.hip", "ffn_small.o", []), ("ffn_prefill.hip", "ffn_prefill.o", []),
           ("ffn_prefill.hip", "ffn_prefill_mid.o", ["-DMOE_PF_MID"]),
           ("combine.hip", "combine.o", []), ("abi.hip", "abi.o", [])]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# packed fp32 VALU forms are disabled for all device code
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


# small-batch expert kernels read every matrix-core result right away: keep
# the results in VGPRs instead of accumulation registers
# the grouped GEMM takes its work tickets with one lane's atomic add, whose
# result is used only later: without the compiler's atomic optimizer the add
# is not widened into a wave reduction that waits for it (and for every
# load and store in flight) on the spot
EXTRA = {"ffn_small.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
         "ffn_prefill.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def _compile(entry) -> str:
    src, obj_name, extra = entry
    obj = os.path.join(OBJ, obj_name)
    r = subprocess.run([HIPCC, *FLAGS, *EXTRA.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj],
                       capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if msg.strip():
        print(msg)
    return obj


def build(jobs: int = 8) -> str:
    os.makedirs(OBJ, exist_ok=True)
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
