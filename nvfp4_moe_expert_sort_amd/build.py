"""Build libnvfp4moe.so (all HIP sources, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "lib", "libnvfp4moe.so")
SOURCES = ["quant.hip", "route.hip", "gemm.hip", "gemm_w4a16.hip", "producer.hip", "backward.hip", "combine.hip",
           "router.hip", "api.hip", "selftest.hip"]

# -ffp-contract=off and no fast-math: the quantizer's binary32 divisions and
# products must be the IEEE operations the numeric contract names.  Packed
# FP32 instructions are disabled for all device code.
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fno-fast-math",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-result", "-fvisibility=hidden"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.sep not in c or os.path.exists(c)):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


# Stand-alone measurement programs (not part of the library): the GEMM path
# comparison behind the choice of exact f16 dequantization, and the L2 -> CU
# read bandwidth of the GEMMs' operand-fetch patterns.
PROBES = {"mfma_path_probe": os.path.join(HERE, "probes", "mfma_path.hip"),
          "l2_patterns_probe": os.path.join(HERE, "probes", "l2_patterns.hip")}


def _build_probe(item) -> str:
    name, src = item
    exe = os.path.join(os.path.dirname(LIB), name)
    r = subprocess.run([hipcc(), *[f for f in HIPCC_FLAGS if f not in ("-fPIC", "-fvisibility=hidden")], src, "-o", exe],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return exe


def build(jobs: int = 6, probes: bool = False) -> str:
    """Compile every library source and link lib/libnvfp4moe.so; with
    probes=True also the stand-alone measurement programs (not needed by the
    library, its tests or bench.py)."""
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    with ThreadPoolExecutor(max(1, jobs)) as ex:
        built = ex.map(_build_probe, PROBES.items()) if probes else iter(())
        objs = list(ex.map(_compile, SOURCES))
        list(built)
    tmp = LIB + ".tmp"
    r = subprocess.run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    import sys
    print(build(probes="--probes" in sys.argv[1:]))
