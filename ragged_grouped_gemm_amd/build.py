"""Build the gfx950 shared library ``libmoe_mi355x.so`` in-tree with hipcc.

Each ``csrc/*.hip`` file is compiled to an object in parallel, then linked.
Packed-fp32 instruction forms are disabled for all device code.

    python -m ragged_grouped_gemm_amd.build [--jobs N] [--debug] [--tuning]

--tuning builds ``libmoe_mi355x_tuning.so`` instead, with -DMOE_GEMM_TUNING:
that library reads the grouped GEMM's tuning variables (MOE_GEMM_TILE,
MOE_GEMM_GM, MOE_GEMM_GM_K, MOE_GEMM_SNAKE, MOE_GEMM_WGRAD, MOE_GEMM_GLU_DIRECT) from the environment, for sweeps; the product
library never does.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe_mi355x.so")
LIB_TUNING = os.path.join(HERE, "libmoe_mi355x_tuning.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-munsafe-fp-atomics",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src, extra, build_dir):
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 8, debug: bool = False, verbose: bool = False,
          tuning: bool = False) -> str:
    build_dir = BUILD + ("_tuning" if tuning else "")
    lib = LIB_TUNING if tuning else LIB
    os.makedirs(build_dir, exist_ok=True)
    extra = (["-g"] if debug else []) + (["-DMOE_GEMM_TUNING"] if tuning else [])
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, build_dir), srcs))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    # A kernel whose host-side stub the compiler failed to emit shows up only as
    # an undefined symbol; refuse such a library instead of failing at load time.
    nm = subprocess.run(["nm", "-C", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [l.strip() for l in nm.stdout.splitlines() if "moe::" in l]
    if missing:
        os.remove(tmp)
        raise RuntimeError("library has undefined internal symbols:\n" + "\n".join(missing[:20]))
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib} from {len(srcs)} sources")
    return lib


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=8)
    ap.add_argument("--debug", action="store_true")
    ap.add_argument("--tuning", action="store_true")
    args = ap.parse_args(argv)
    build(args.jobs, args.debug, verbose=True, tuning=args.tuning)


if __name__ == "__main__":
    sys.exit(main())
