"""Build libattn_jvp.so (C ABI + gfx950 kernels) in-tree with hipcc.

Usage: python attention_jvp_causal_attn_amd/csrc/build.py [--verbose]
Writes attention_jvp_causal_attn_amd/libattn_jvp.so next to the package.
"""

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libattn_jvp.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["attn_jvp_mask.cpp", "attn_jvp_api.cpp", "attn_jvp_bf16_wide.hip",
           "attn_jvp_f32.hip", "attn_jvp_merge.hip", "attn_jvp_bwd_wide.hip",
           "attn_jvp_bwd_f32.hip", "attn_jvp_noalloc.hip"]
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-I", INCLUDE, "-I", HERE,
    "-Wall", "-Wno-unused-function",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build")
    return path


def compile_one(src, verbose):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + COMMON + ["-c", os.path.join(HERE, src), "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


# Kernels that set M0 in inline assembly for their direct-to-LDS copies.  The
# asm lists M0 as clobbered, but the compiler does not save a reserved
# register around an asm block, so the invariant these kernels rely on is that
# compiled code never writes or reads M0 itself.  check_m0 enforces it on the
# device assembly of every build.
M0_ASM_SOURCES = ["attn_jvp_bf16_wide.hip", "attn_jvp_bwd_wide.hip"]
# mnemonic fragments of instructions that read M0 implicitly on gfx9
M0_IMPLICIT = ("_lds_", "_gws", "sendmsg", "movrel", "interp", "addtid", "ds_append",
               "ds_consume", "ds_ordered", "s_ttracedata")


def check_m0(asm_path):
    """Fail when compiled code (outside inline-asm blocks) names M0 or uses an
    instruction that reads it implicitly.  Returns the number of asm-block
    lines that set M0 (the copies)."""
    in_asm = False
    asm_writes = 0
    bad = []
    with open(asm_path) as f:
        for n, raw in enumerate(f, 1):
            line = raw.split(";")[0].strip()
            if ";;#ASMSTART" in raw:
                in_asm = True
                continue
            if ";;#ASMEND" in raw:
                in_asm = False
                continue
            if not line or line.startswith(".") or line.endswith(":"):
                continue
            mnem = line.split()[0]
            names_m0 = any(tok.strip(",") == "m0" for tok in line.split()[1:])
            if in_asm:
                asm_writes += names_m0
                continue
            if names_m0 or any(frag in mnem for frag in M0_IMPLICIT):
                bad.append(f"{os.path.basename(asm_path)}:{n}: {line}")
    if bad:
        raise RuntimeError("compiled code touches M0, which the kernels' inline-asm copies "
                           "overwrite without a save:\n" + "\n".join(bad[:20]))
    return asm_writes


def device_asm(src, verbose):
    out = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".gfx950.s")
    cmd = [hipcc(), "-x", "hip"] + COMMON + ["-S", "--offload-device-only",
                                             os.path.join(HERE, src), "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"device assembly of {src} failed:\n{r.stdout}\n{r.stderr}")
    return out


def build(verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES) + len(M0_ASM_SOURCES)) as ex:
        objs_f = [ex.submit(compile_one, s, verbose) for s in SOURCES]
        asm_f = [ex.submit(device_asm, s, verbose) for s in M0_ASM_SOURCES]
        objs = [f.result() for f in objs_f]
        for f in asm_f:
            check_m0(f.result())
    tmp = OUT + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    print(build(ap.parse_args().verbose))
