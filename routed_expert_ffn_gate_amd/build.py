"""Build libmoelb.so (HIP, gfx950) in-tree.

    python -m routed_expert_ffn_gate_amd.build

Compiles every ``csrc/*.hip`` with hipcc for gfx950 and links them into
``routed_expert_ffn_gate_amd/libmoelb.so``.  No GPU is needed.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoelb.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # no packed-fp32 instructions (v_pk_*_f32) in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # atomics on one address from many lanes: combine the lanes with DPP
    # (a few cross-lane steps) rather than a loop over the active lanes
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=DPP",
    "-I", os.path.join(ROOT, "include"),
]
COMPILE_TIMEOUT = 900


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=COMPILE_TIMEOUT)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _check_kernel_stubs(lib_path: str) -> None:
    """A kernel whose host launch stub was not emitted only shows up as an
    undefined symbol when the library is loaded: fail the build instead."""
    p = subprocess.run(["nm", "-u", lib_path], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    missing = [l.split()[-1] for l in p.stdout.splitlines() if "_kernel" in l or "__device_stub__" in l]
    if missing:
        raise RuntimeError(f"{lib_path}: kernels without a host stub: {missing[:4]}")


_M0_WRITE = re.compile(r"^\s*s_mov_b32\s+m0,\s*s\d+\s*$")


def m0_violations(asm_lines) -> list:
    """Lines of device assembly that use M0 other than as the LDS DMA helpers
    do (s_mov_b32 m0, sN; s_nop 0; global_load_lds_dwordx4)."""
    lines = [l.split(";")[0].strip() for l in asm_lines]
    lines = [l for l in lines if l]
    bad = []
    for i, l in enumerate(lines):
        if not re.search(r"\bm0\b", l):
            continue
        ok = (_M0_WRITE.match(l) and i + 2 < len(lines) and lines[i + 1] == "s_nop 0"
              and lines[i + 2].startswith("global_load_lds_dwordx4"))
        if not ok:
            bad.append(l)
    return bad


def _check_m0(src: str) -> None:
    """The LDS DMA helpers set M0 in inline asm and list it as clobbered; the
    compiler does not preserve a reserved register across such asm, so the
    build requires that no compiler code relies on M0."""
    asm = os.path.join(BUILD, os.path.basename(src)[:-4] + ".device.s")
    _run([HIPCC, *FLAGS, "--cuda-device-only", "-S", src, "-o", asm])
    with open(asm) as fh:
        bad = m0_violations(fh)
    if bad:
        raise RuntimeError(f"{src}: M0 used outside the LDS DMA helpers: {bad[:4]}")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o") for s in srcs]

    def one(pair):
        src, obj = pair
        return _run([HIPCC, *FLAGS, "-c", src, "-o", obj])

    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        for out in ex.map(one, zip(srcs, objs)):
            if verbose and out.strip():
                print(out)
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        list(ex.map(_check_m0, [src for src in srcs if "m0" in open(src).read()]))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    _check_kernel_stubs(tmp)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
