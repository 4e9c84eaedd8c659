"""Build libtq.so (the HIP library) and libtqsynth.so (the input generator) for gfx950.

Each .hip source is compiled separately (in parallel) with hipcc and linked
into a shared library next to its sources' package.  Run as
``python -m ternary_weight_amd.build``; ``__graft_entry__.build()`` calls
``build_all()``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBTQ = os.path.join(PKG, "libtq.so")
SYNTH_SRC = os.path.join(ROOT, "synth", "synth_kernels.hip")
LIBSYNTH = os.path.join(ROOT, "synth", "libtqsynth.so")
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = os.environ.get("TQ_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-fvisibility=hidden",
    "-ffp-contract=off", "-Wall", "-Wno-unused-function",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]

TQ_SOURCES = ["tq_api.hip", "tq_pack.hip", "tq_act.hip", "tq_gemv.hip", "tq_entry.hip", "tq_gemm.hip",
               "tq_gemm_i8.hip", "tq_gemm_bf16.hip", "tq_gemm_bf16_skinny.hip",
               "tq_gemm_i8_skinny.hip", "tq_chain.hip", "tq_ternarize.hip"] + [
    "tq_gemv_%s_m%d.hip" % (x, m) for x in ("f32", "bf16", "i8", "f32q8") for m in (1, 4)]


def _deps_mtime() -> float:
    heads = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
    heads.append(os.path.join(ROOT, "include", "tq.h"))
    return max(os.path.getmtime(h) for h in heads)


INCREMENTAL = False
# --sanitize: the host code of every translation unit built with AddressSanitizer
# and UndefinedBehaviorSanitizer (device code unchanged) into _build/asan/libtq.so,
# for running the CPU tests of the ABI's validation paths under the sanitizers.
SANITIZE = False
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src: str, obj: str, extra=()) -> str:
    os.makedirs(os.path.dirname(obj), exist_ok=True)
    if INCREMENTAL and os.path.exists(obj) and \
            os.path.getmtime(obj) > max(os.path.getmtime(src), _deps_mtime()):
        return obj
    cmd = [HIPCC, *COMMON, *(SAN_FLAGS if SANITIZE else []), *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr[-6000:]))
    return obj


def _link(objs, out):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *(SAN_FLAGS if SANITIZE else []), *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed for %s:\n%s" % (out, r.stderr[-4000:]))
    os.replace(tmp, out)


def build_libtq(jobs: int = 0) -> str:
    jobs = jobs or min(8, os.cpu_count() or 4)
    objs = []
    sub = "asan" if SANITIZE else "tq"
    out = os.path.join(BUILD_DIR, "asan", "libtq.so") if SANITIZE else LIBTQ
    with cf.ThreadPoolExecutor(jobs) as ex:
        futs = [ex.submit(_compile, os.path.join(CSRC, s), os.path.join(BUILD_DIR, sub, s + ".o"))
                for s in TQ_SOURCES]
        for f in futs:
            objs.append(f.result())
    _link(objs, out)
    return out


def build_synth() -> str:
    obj = _compile(SYNTH_SRC, os.path.join(BUILD_DIR, "synth", "synth_kernels.o"))
    _link([obj], LIBSYNTH)
    return LIBSYNTH


def build_all() -> None:
    build_libtq()
    if os.path.exists(SYNTH_SRC):
        build_synth()


if __name__ == "__main__":
    INCREMENTAL = "--incremental" in sys.argv
    SANITIZE = "--sanitize" in sys.argv
    if SANITIZE:
        print("built", build_libtq(), file=sys.stderr)
    else:
        build_all()
        print("built", LIBTQ, file=sys.stderr)
