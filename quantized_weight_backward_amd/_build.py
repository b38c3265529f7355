"""Build the HIP library libretro_out_prod.so in-tree for gfx950.

The kernels of each weight type are compiled into an object of their own
(retro_unit.hip with -DRETRO_UNIT_TYPE=<type id>) and the C ABI into another
(retro_api.hip), the measured-ceiling probes into a third (retro_probe.hip);
the objects are built in parallel and linked into one shared library.
"""

from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(REPO_DIR, "include")
OBJ_DIR = os.path.join(PKG_DIR, "_obj")
LIB_NAME = "libretro_out_prod.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
API_SOURCE = os.path.join(CSRC, "retro_api.hip")
UNIT_SOURCE = os.path.join(CSRC, "retro_unit.hip")
PROBE_SOURCE = os.path.join(CSRC, "retro_probe.hip")
# GGUF ids of the weight types, one kernel object each
UNIT_TYPES = {"f32": 0, "f16": 1, "q4_0": 2, "q4_1": 3, "q5_0": 6, "q5_1": 7, "q8_0": 8, "q2_k": 10, "q3_k": 11,
              "q4_k": 12, "q5_k": 13, "q6_k": 14, "bf16": 30, "mxfp4": 39,
              "nvfp4": 40}

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # keep the compiler from emitting packed-FP32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]
# the host pass warns that it does not know the packed-fp32 feature
_NOISE = "is not a recognized feature for this target"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def _jobs() -> int:
    limit = int(os.environ.get("MAX_JOBS", "16") or 16)
    return max(1, min(limit, os.cpu_count() or 1, len(UNIT_TYPES) + 2))


def _run(cmd: list[str]) -> str:
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if _NOISE not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False) -> str:
    """Compile every HIP source into LIB_PATH (always recompiles)."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    base = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c"]
    jobs = [(os.path.join(OBJ_DIR, "retro_api.o"), [API_SOURCE]),
            (os.path.join(OBJ_DIR, "retro_probe.o"), [PROBE_SOURCE])]
    for name, tid in UNIT_TYPES.items():
        jobs.append((os.path.join(OBJ_DIR, f"retro_unit_{name}.o"), [f"-DRETRO_UNIT_TYPE={tid}", UNIT_SOURCE]))
    with ThreadPoolExecutor(max_workers=_jobs()) as pool:
        logs = list(pool.map(lambda j: _run([*base, *j[1], "-o", j[0]]), jobs))
    tmp = LIB_PATH + ".tmp"
    logs.append(_run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *[j[0] for j in jobs], "-o", tmp]))
    if verbose:
        for log in logs:
            if log.strip():
                print(log)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
