"""Build libtq.so (the HIP library behind include/tq.h) for gfx950, in-tree.

    python -m kv_cache_vector_amd.build

Every .hip file under csrc/ is compiled by hipcc for gfx950 with packed-FP32
instruction selection disabled; the host dispatcher (.cpp) is compiled by
hipcc as host C++.  Objects go to _build/, the library next to this file.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libtq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-function"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics", "-ffp-contract=fast"]
# Per-file code generation options.  The codec, scores and attention kernels
# feed MFMA results straight into VALU work; keeping them in arch VGPRs instead
# of AGPRs saves the v_accvgpr moves in between.
PER_FILE = {name: ["-mllvm", "-amdgpu-mfma-vgpr-form"] for name in ("tq_codec.hip", "tq_scores.hip", "tq_attn.hip")}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON
    if src.endswith(".hip"):
        cmd += DEVICE + PER_FILE.get(os.path.basename(src), []) + ["-x", "hip"]
    else:
        cmd += [f"--offload-arch={ARCH}"]
    cmd += ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    noisy = [ln for ln in r.stderr.splitlines() if ln.strip() and "not a recognized feature" not in ln]
    if noisy:
        sys.stderr.write("\n".join(noisy) + "\n")
    return obj


def build(jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    jobs = jobs or min(8, len(srcs))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
