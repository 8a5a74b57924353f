"""Build the HIP library libssm_mi355x.so in-tree for gfx950 (hipcc cross-compiles; no GPU
needed).  Used by ``__graft_entry__.build()`` and runnable as ``python
ssm_sequence_models_amd/build.py``; it imports nothing from the package, whose import loads
the library this file builds."""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libssm_mi355x.so")
SOURCES = ["abi.hip", "bwd.hip", "conv.hip", "init_state.hip", "pool.hip", "recurrent.hip", "ssd.hip", "vchunk.hip", "vdecay.hip"]
ARCH = "gfx950"

# -packed-fp32-ops off: no v_pk_{add,mul,fma}_f32 in the device code (hipcc's host pass
# warns that it does not know the feature; that warning is harmless)
HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-ffp-contract=fast", "-munsafe-fp-atomics"]


def hipcc() -> str:
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
