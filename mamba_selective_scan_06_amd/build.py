"""Build libssm_scan.so in-tree with hipcc for gfx950.

    python -m mamba_selective_scan_06_amd.build [--jobs N]

Every HIP source is compiled with packed FP32 instructions disabled
(-target-feature -packed-fp32-ops): the compiler would otherwise fuse pairs of
fp32 operations into v_pk_*_f32, whose results are not trusted on this
hardware generation's toolchain.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libssm_scan.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# (source, extra defines, object name)
NSPLIT_INST = [(s, k, w) for s in ("float", "uint16_t") for k in (1, 2, 4, 8, 16) for w in (0, 1)]
UNITS = [("api.cpp", [], "api"), ("nsplit_dispatch.cpp", [], "nsplit_dispatch"),
         ("scan_lane.hip", [], "scan_lane"), ("scan_decode.hip", [], "scan_decode"),
         ("scan_bwd.hip", [], "scan_bwd"), ("conv_prologue.hip", [], "conv_prologue"),
         ("ssd_fwd.hip", [], "ssd_fwd"), ("noalloc_scratch.hip", [], "noalloc_scratch"), ("carry_scan.hip", [], "carry_scan"),
         ("scan_bwd_inst.hip", ["-DBWD_S=float"], "bwd_f32"), ("scan_bwd_inst.hip", ["-DBWD_S=uint16_t"], "bwd_bf16")] + [
    ("nsplit_inst.hip", [f"-DNSPLIT_S={s}", f"-DNSPLIT_K={k}", f"-DNSPLIT_WIN={w}"],
     f"nsplit_{'f32' if s == 'float' else 'bf16'}_k{k}{'_win' if w else ''}")
    for s, k, w in NSPLIT_INST]
SOURCES = sorted({u[0] for u in UNITS})
HEADERS = ["buffer_io.hpp", "device_common.hpp", "scan_bwd_impl.hpp", "scan_internal.hpp", "scan_nsplit_impl.hpp"]

COMMON = ["-O3", "-std=c++20", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-command-line-argument", f"-I{os.path.join(ROOT, 'include')}"]


def _compile(unit) -> str:
    src, defs, name = unit
    out = os.path.join(OBJ, name + ".o")
    cmd = [HIPCC, *COMMON, *defs, "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {name}:\n{r.stdout}\n{r.stderr}")
    return out


def _device_asm(unit) -> str:
    """gfx950 assembly of one NSPLIT unit, for the DPP hazard check."""
    src, defs, name = unit
    out = os.path.join(OBJ, name + ".s")
    cmd = [HIPCC, *COMMON, *defs, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {name}:\n{r.stdout}\n{r.stderr}")
    return out


def build(jobs: int | None = None, verbose: bool = False) -> str:
    """Compile every source, check the NSPLIT device code for the DPP hazard
    that inline asm hides from the compiler, and link the shared library;
    returns its path."""
    from . import dpp_hazard_check

    os.makedirs(OBJ, exist_ok=True)
    jobs = jobs or min(len(UNITS), os.cpu_count() or 1, 16)
    asm_units = [u for u in UNITS if u[0] == "nsplit_inst.hip"]
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, UNITS))
        listings = list(ex.map(_device_asm, asm_units))
    problems = []
    for path in listings:
        problems += dpp_hazard_check.check_file(path)
    if problems:
        raise RuntimeError("VALU -> DPP hazard in generated code:\n" + "\n".join(problems[:20]))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def sources_newer_than_lib() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    files = [os.path.join(CSRC, f) for f in SOURCES + HEADERS] + [os.path.join(ROOT, "include", "ssm_scan.h")]
    return any(os.path.getmtime(f) > t for f in files)


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    a = ap.parse_args()
    build(a.jobs, verbose=True)
    sys.exit(0)
