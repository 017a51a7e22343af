"""Build libmaple_moe.so in-tree with hipcc for gfx950.

Usage: python -m ternary_weight_moe_amd.build [--force] [-j N]
Objects go to ternary_weight_moe_amd/_build/ (not committed); the library to
ternary_weight_moe_amd/libmaple_moe.so, where the binding loads it.  The
two measurement probes (csrc/read_probe.hip and csrc/mfma_probe.hip, run by
bench.py --read-probe / --mfma-probe) build to ternary_weight_moe_amd/read_probe
and ternary_weight_moe_amd/mfma_probe.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmaple_moe.so")
PROBES = ("read_probe", "mfma_probe")
SOURCES = ["api.cpp", "route.hip", "gemv.hip", "decode1.hip", "grouped.hip", "misc.hip", "head.hip",
           "attn.hip", "convert.hip"]
HEADERS = [os.path.join(CSRC, "internal.h"), os.path.join(CSRC, "wave.h"),
           os.path.join(CSRC, "limbs.h"), os.path.join(CSRC, "quant.h"),
           os.path.join(CSRC, "digits.h"),
           os.path.join(ROOT, "include", "maple_moe.h"),
           os.path.join(ROOT, "include", "maple_head.h"),
           os.path.join(ROOT, "include", "maple_attn.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall",
         "-Wno-unused-function", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
         # packed-fp32 VALU instructions stay off (device pass only; the host
         # pass ignores the feature with a warning)
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str, force: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    deps = [src] + HEADERS
    if not force and os.path.exists(obj) and all(
            os.path.getmtime(obj) >= os.path.getmtime(d) for d in deps):
        return obj
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build(force: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, force), srcs))
    if force or not os.path.exists(LIB) or any(
            os.path.getmtime(o) > os.path.getmtime(LIB) for o in objs):
        tmp = LIB + f".tmp{os.getpid()}"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("link of libmaple_moe.so failed")
        os.replace(tmp, LIB)
    return LIB


def build_probes(force: bool = False) -> list:
    outs = []
    for name in PROBES:
        src, exe = os.path.join(CSRC, name + ".hip"), os.path.join(PKG, name)
        outs.append(exe)
        if not force and os.path.exists(exe) and os.path.getmtime(exe) >= os.path.getmtime(src):
            continue
        tmp = exe + f".tmp{os.getpid()}"
        r = subprocess.run([HIPCC, *[f for f in FLAGS if f != "-fPIC"], src, "-o", tmp],
                           capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError(f"hipcc failed on {name}.hip")
        os.replace(tmp, exe)
    return outs


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--force", action="store_true")
    ap.add_argument("-j", type=int, default=8)
    a = ap.parse_args()
    print(build(a.force, a.j))
    print(*build_probes(a.force), sep="\n")
