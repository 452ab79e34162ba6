"""Build the HIP library libmoe_amd.so in-tree for gfx950 (hipcc, no GPU needed)."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe_amd.so")
SOURCES = ["router.hip", "router_opts.hip", "router_proj.hip", "permute.hip", "gemm.hip", "mx.hip", "aux_loss.hip", "noalloc.hip", "moe_api.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-mcode-object-version=5",
    # packed fp32 VALU ops stay off: ordinary float code must not become v_pk_*_f32
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # atomics stay as written: the wave-level atomic rewrite would read a tile ticket back
    # (and wait for every load in flight) right where it is issued
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # hipcc's host pass warns about the device-only target feature; keep other warnings
    warn = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    return "\n".join(warn)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = [os.path.join(BUILD, s.replace(".hip", ".o")) for s in SOURCES]

    def compile_one(i):
        return _run([HIPCC, *FLAGS, "-c", os.path.join(CSRC, SOURCES[i]), "-o", objs[i]])

    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        logs = list(ex.map(compile_one, range(len(SOURCES))))
    tmp = LIB + ".tmp"
    # -z defs: a symbol missing from the objects fails the link instead of the first load
    logs.append(_run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,-z,defs", *objs, "-o", tmp]))
    os.replace(tmp, LIB)
    log = "\n".join(l for l in logs if l)
    if verbose and log:
        print(log, file=sys.stderr)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
