"""Build libkda.so in-tree for gfx950.

    python -m gated_delta_rule_82_amd.build

The host argument checker is plain C++ (g++); the kernel files (decode and
chunked prefill) go through hipcc for gfx950 with packed-fp32 instructions
disabled; hipcc links them into ``gated_delta_rule_82_amd/lib/libkda.so``.
The benchmark's streaming-copy kernels (its HBM ceiling) build into a
separate ``lib/libkda_bench.so`` that the library itself never loads.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libkda.so")
BENCH_LIB = os.path.join(LIBDIR, "libkda_bench.so")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep hipcc from emitting packed fp32 arithmetic (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


# Per-file additions.  The prefill kernel keeps its MFMA accumulators (the
# state slab and the chunk products) in the architectural VGPRs: its
# elementwise work reads and scales them every chunk, and with accumulators
# in AGPRs every such access costs a copy (measured 5-8% faster this way).
EXTRA_FLAGS = {"kda_prefill": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libkda")


def _run(cmd, verbose):
    if verbose:
        print("+", " ".join(cmd), flush=True)
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in proc.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def _run_all(cmds, verbose):
    if verbose:
        for cmd in cmds:
            print("+", " ".join(cmd), flush=True)
    procs = [subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
             for cmd in cmds]
    failed = []
    for cmd, proc in zip(cmds, procs):
        out, _ = proc.communicate()
        out = "\n".join(line for line in out.splitlines()
                        if "packed-fp32-ops' is not a recognized feature" not in line)
        if proc.returncode != 0:
            failed.append(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{out}")
        elif verbose and out.strip():
            print(out, flush=True)
    if failed:
        raise RuntimeError("\n".join(failed))


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    hipcc = _hipcc()
    api_o = os.path.join(BUILD, "kda_api.o")
    # (source, object, extra defines): the prefill file once per dk, each
    # object holding that dk's kernels
    units = [("kda_decode", "kda_decode", [])]
    units += [("kda_prefill", f"kda_prefill_dk{dk}", [f"-DKDA_PREFILL_DK={dk}"]) for dk in (32, 64, 128)]
    lib_objs = [os.path.join(BUILD, f"{obj}.o") for _, obj, _ in units]
    bench_o = os.path.join(BUILD, "bench_copy.o")
    units.append(("bench_copy", "bench_copy", []))
    _run(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", f"-I{INCLUDE}", f"-I{CSRC}",
          "-c", os.path.join(CSRC, "kda_api.cpp"), "-o", api_o], verbose)
    # the kernel objects compile in parallel (each takes tens of seconds)
    cmds = [[hipcc, *HIP_FLAGS, *EXTRA_FLAGS.get(src, []), *defs, f"-I{INCLUDE}", f"-I{CSRC}", "-c",
             os.path.join(CSRC, f"{src}.hip"), "-o", os.path.join(BUILD, f"{obj}.o")]
            for src, obj, defs in units]
    _run_all(cmds, verbose)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", api_o, *lib_objs, "-o", tmp,
          "-Wl,-z,defs", "-Wl,--no-undefined",
          f"-Wl,--version-script={os.path.join(CSRC, 'libkda.map')}"], verbose)
    os.replace(tmp, LIB)
    tmp = BENCH_LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", bench_o, "-o", tmp,
          "-Wl,-z,defs", "-Wl,--no-undefined"], verbose)
    os.replace(tmp, BENCH_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
