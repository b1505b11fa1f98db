"""Build libmoe.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m routed_expert_ffn_route_amd.build   (always recompiles)
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe.so")
# (source, object, extra defines): decode_inst.hip is compiled once per dtype combination and
# token tile so that the decode kernels build in parallel
SOURCES = [("api.hip", "api.o", []), ("route.hip", "route.o", []), ("decode.hip", "decode.o", []),
           ("prefill.hip", "prefill.o", []), ("measure.hip", "measure.o", [])] + [
    ("decode_inst.hip", f"decode_{n}_t{tm}.o", [f"-DMOE_DEC_NAME={n}", f"-DMOE_DEC_TM={tm}"])
    for n in ("fp4", "i4", "bf16", "f32") for tm in (1, 4, 8, 16)]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Wno-unused-function", "-Wno-unused-variable",
         # packed fp32 VALU ops stay off: plain fp32 code only
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(HERE, "..", "include")]


def _compile(unit) -> str:
    src, objname, defs = unit
    obj = os.path.join(OBJ, objname)
    cmd = [HIPCC, *FLAGS, *defs, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {objname}:\n{r.stdout}\n{r.stderr}")
    warn = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if warn:
        sys.stderr.write("\n".join(warn) + "\n")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    for f in os.listdir(OBJ):  # objects of units that no longer exist must not be linked
        if f.endswith(".o"):
            os.remove(os.path.join(OBJ, f))
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, LIB)
    return LIB


# Host-side sanitizer build (ASan + UBSan) of the C-ABI unit for the CPU tests: api.hip is
# recompiled with the host pass instrumented (the device code is unchanged) and linked with the
# other objects of the last build().  Loading it needs the clang ASan runtime preloaded.
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def build_sanitized(outdir: str) -> str:
    objs = [os.path.join(OBJ, u[1]) for u in SOURCES if u[0] != "api.hip"]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"run build() first: {missing[0]} is missing")
    os.makedirs(outdir, exist_ok=True)
    api = os.path.join(outdir, "api_san.o")
    flags = [f for f in FLAGS if f != "-O3"] + ["-O1", "-g"]
    subprocess.run([HIPCC, *flags, *SAN_HOST, "-c", os.path.join(CSRC, "api.hip"), "-o", api],
                   check=True, capture_output=True)
    lib = os.path.join(outdir, "libmoe_san.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *SAN_HOST, "-Xarch_host", "-shared-libsan",
                    "-o", lib, api, *objs], check=True, capture_output=True)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
