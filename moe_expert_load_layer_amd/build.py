"""Build the HIP library (gfx950) in-tree: moe_expert_load_layer_amd/libepbalance.so."""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "libepbalance.so")
OBJ_DIR = os.path.join(HERE, "_build")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(HERE, '..', 'include')}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


PHASES_LIB_PATH = os.path.join(HERE, "libepbalance_phases.so")


def build(verbose: bool = False, jobs: int = 6, defines=(), out: str = LIB_PATH, obj_dir: str = OBJ_DIR) -> str:
    """Compile every csrc/*.hip for gfx950 and link libepbalance.so (always rebuilds).

    defines/out/obj_dir serve the planner's profiling build (plan_phases.py),
    a separate library with the phase marks compiled in."""
    hipcc = _hipcc()
    os.makedirs(obj_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))

    def compile_one(src: str) -> str:
        obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
        cmd = [hipcc, *HIPCC_FLAGS, *defines, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = out + f".tmp{os.getpid()}"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build_plan_phases(verbose: bool = False) -> str:
    """The profiling build: libepbalance_phases.so with the planner's phase marks."""
    return build(verbose, defines=("-DEP_PLAN_PHASES",), out=PHASES_LIB_PATH, obj_dir=os.path.join(OBJ_DIR, "phases"))


if __name__ == "__main__":
    import sys
    print(build_plan_phases(verbose=True) if "--plan-phases" in sys.argv[1:] else build(verbose=True))
