"""Builds libmoe_int4.so (the HIP/C-ABI library) in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe_int4.so")

# the streaming-read probe the benchmark measures the HBM ceiling with: a
# library of its own, not part of the MoE path
PROBE_SRC = "hbm_probe.hip"
PROBE_LIB = os.path.join(HERE, "libhbm_probe.so")

SOURCES = ["moe_api.hip", "moe_stage.hip", "k_pack.hip", "k_small.hip", "k_large.hip", "k_gemv.hip", "k_gemm.hip", "k_tok1.hip", "k_midt.hip"]

# -packed-fp32-ops: keep hipcc from forming v_pk_{add,mul,fma}_f32 out of
# ordinary float code (the host pass warns that it does not know the
# feature; that warning is harmless).
HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-munsafe-fp-atomics",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = ["hipcc", *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed for {src}")
    return obj


def build() -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + 1)) as ex:
        objs = list(ex.map(_compile, SOURCES + [PROBE_SRC]))
    tmp = LIB + ".tmp"
    subprocess.check_call(["hipcc", "-shared", "-fPIC", "--offload-arch=gfx950", *objs[:-1], "-o",
                           tmp])
    os.replace(tmp, LIB)
    subprocess.check_call(["hipcc", "-shared", "-fPIC", "--offload-arch=gfx950", objs[-1], "-o",
                           PROBE_LIB + ".tmp"])
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build())
