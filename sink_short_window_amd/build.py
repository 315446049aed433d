"""Build the native libraries in-tree.

* ``lib/libll.so``        -- the product: HIP kernels for gfx950 + the C ABI.
* ``lib/libll_hoststub.so`` -- CPU test library: the same C ABI layer and
  bookkeeping linked against a launch stub that records instead of launching
  (g++ only, no HIP), so the ABI's host logic is testable without a GPU.
* ``lib/libll_hoststub_san.so`` -- the same, built with AddressSanitizer and
  UndefinedBehaviorSanitizer (host code only; loaded with the ASan runtime
  preloaded, see tests/test_host_sanitizers.py).

Run ``python -m sink_short_window_amd.build``.
"""

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "lib")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 VALU ops are switched off for all device code.
DEVICE_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-munsafe-fp-atomics"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]

DEVICE_SOURCES = ("kernels.hip", "attn_bwd.hip", "linear_attn.hip")
LIB_LL = os.path.join(LIB, "libll.so")
LIB_HOSTSTUB = os.path.join(LIB, "libll_hoststub.so")
LIB_HOSTSTUB_SAN = os.path.join(LIB, "libll_hoststub_san.so")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer", "-g"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


def build_hoststub(verbose=False, sanitize=False):
    os.makedirs(LIB, exist_ok=True)
    cxx = shutil.which("g++") or "g++"
    srcs = [os.path.join(CSRC, f) for f in ("cache_state.cpp", "ll_api.cpp", "launch_stub.cpp")]
    dst = LIB_HOSTSTUB_SAN if sanitize else LIB_HOSTSTUB
    tmp = dst + ".tmp"
    flags = HOST_FLAGS + (SAN_FLAGS if sanitize else [])
    out = _run([cxx] + flags + ["-shared", "-I", INCLUDE, "-I", CSRC] + srcs + ["-o", tmp])
    os.replace(tmp, dst)
    if verbose and out:
        print(out)
    return dst


def build_ll(verbose=False):
    os.makedirs(LIB, exist_ok=True)
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    out = ""
    for src in DEVICE_SOURCES:
        o = os.path.join(BUILD, src.replace(".hip", ".o"))
        out += _run([HIPCC] + DEVICE_FLAGS + ["-I", INCLUDE, "-I", CSRC, "-c",
                                              os.path.join(CSRC, src), "-o", o])
        objs.append(o)
    for f in ("cache_state.cpp", "ll_api.cpp"):
        o = os.path.join(BUILD, f.replace(".cpp", ".o"))
        _run(["g++"] + HOST_FLAGS + ["-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, f), "-o", o])
        objs.append(o)
    tmp = LIB_LL + ".tmp"
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + ["-o", tmp])
    os.replace(tmp, LIB_LL)
    if verbose and out:
        print(out)
    return LIB_LL


def build_all(verbose=False):
    return build_ll(verbose), build_hoststub(verbose), build_hoststub(verbose, sanitize=True)


if __name__ == "__main__":
    for p in build_all(verbose="-v" in sys.argv):
        print("built", p)
