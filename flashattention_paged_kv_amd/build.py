"""Build libpagedattn.so (all HIP sources, gfx950) in place, with hipcc.

    python -m flashattention_paged_kv_amd.build [--debug | --sanitize]

Compiles each csrc/*.hip to an object (in parallel) and links the shared
library next to this file.  Packed fp32 instructions are disabled for the
device code.

--debug builds libpagedattn_debug.so beside it: the same kernels with the
device-side range checks of block-table entries, lengths and prefix sums
compiled in (PA_DEVICE_CHECKS=1; each call then waits for its kernels and
reports PA_ERR_DEVICE_ASSERT).

--sanitize builds libpagedattn_hostsan.so beside it: the host-side sources
(argument checks, dispatch, the page pool) compiled with AddressSanitizer
and UndefinedBehaviorSanitizer on the host pass only (device code is built
as usual), linked against the shared ASan runtime, which the process must
preload (tests/test_host_sanitizers.py does).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libpagedattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Host-pass-only sanitizers (each flag applies to the host compilation alone).
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
HOST_SANITIZED_SOURCES = ("api.hip", "page_pool.hip", "noalloc.hip")
SAN_OUT = os.path.join(HERE, "libpagedattn_hostsan.so")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


# Per-source device code generation options.  backward.hip: MFMA results in
# ordinary vector registers (the dK/dV kernel's score and dP blocks then need
# no copies out of the accumulation registers before the softmax arithmetic:
# 134 against 148 us at L=2048); its long-lived dK / dV sums are pinned to
# the accumulation registers in the source instead.
SOURCE_FLAGS = {"backward.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str, obj: str, opt: str, extra=()) -> None:
    cmd = [HIPCC, *DEVICE_FLAGS, opt, "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", *extra,
           "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)


DEBUG_OUT = os.path.join(HERE, "libpagedattn_debug.so")


def build(debug: bool = False, verbose: bool = True) -> str:
    objdir = os.path.join(HERE, "_build_debug" if debug else "_build")
    os.makedirs(objdir, exist_ok=True)
    extra = ["-DPA_DEVICE_CHECKS=1"] if debug else []
    out = DEBUG_OUT if debug else OUT
    srcs = sources()
    objs = [os.path.join(objdir, os.path.basename(s)[:-4] + ".o") for s in srcs]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        list(ex.map(lambda so: _compile(so[0], so[1], "-O3", extra + SOURCE_FLAGS.get(os.path.basename(so[0]), [])),
                    zip(srcs, objs)))
    tmp = out + ".tmp"
    # -z defs: an unresolved symbol fails the link here, not the first load
    # (a kernel whose host-side launch stub the compiler dropped shows up so).
    cmd = [HIPCC, *DEVICE_FLAGS, "-shared", "-fPIC", "-Wl,-z,defs", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


def asan_runtime() -> str:
    """Path of clang's shared ASan runtime next to hipcc's compiler, or ''."""
    llvm = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "lib", "clang")
    for root, _, files in os.walk(os.path.normpath(llvm)):
        if "libclang_rt.asan-x86_64.so" in files:
            return os.path.join(root, "libclang_rt.asan-x86_64.so")
    return ""


def build_sanitized(verbose: bool = True) -> str:
    """libpagedattn_hostsan.so: the host-side sources with ASan + UBSan (host
    pass), the kernels' sources as in the release build."""
    objdir = os.path.join(HERE, "_build_hostsan")
    os.makedirs(objdir, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(objdir, os.path.basename(s)[:-4] + ".o") for s in srcs]

    def one(so):
        src, obj = so
        san = os.path.basename(src) in HOST_SANITIZED_SOURCES
        _compile(src, obj, "-O1" if san else "-O3",
                 HOST_SANITIZE if san else SOURCE_FLAGS.get(os.path.basename(src), []))

    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        list(ex.map(one, zip(srcs, objs)))
    tmp = SAN_OUT + ".tmp"
    cmd = [HIPCC, *DEVICE_FLAGS, "-shared", "-fPIC", "-Xarch_host", "-shared-libasan", *HOST_SANITIZE, *objs,
           "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, SAN_OUT)
    if verbose:
        print(f"built {SAN_OUT}")
    return SAN_OUT


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--debug", action="store_true")
    ap.add_argument("--sanitize", action="store_true")
    a = ap.parse_args()
    if a.sanitize:
        build_sanitized()
    else:
        build(debug=a.debug)
