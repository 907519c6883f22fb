"""Build libpka.so (HIP kernels for gfx950 + the C ABI) in the package dir.

    python -m paged_kv_attention_24_amd._build [-v] [--only a.hip,b.cpp]

``--only`` recompiles just the named sources and relinks with the objects
already in _build/ (a quick rebuild after editing one file; ``build()``
always compiles everything).

Every HIP translation unit is compiled with packed FP32 instructions
disabled (``-Xclang -target-feature -Xclang -packed-fp32-ops``); the host
pass prints a harmless warning about that feature.
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
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libpka.so")

ARCH = "gfx950"
SOURCES = ["paged_decode.hip", "paged_prefill.hip", "kv_cache_write.hip", "block_ops.hip",
           "paged_int8.hip", "abi.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
VARIANTS = {}

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fhip-fp32-correctly-rounded-divide-sqrt",
          "-I", INCLUDE, "-I", CSRC, "-Wall"]


def _compile_cmd(src: str, obj: str, extra=()):
    lang = ["-x", "hip"]  # the ABI file includes the HIP runtime headers too
    return [HIPCC, *lang, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]


def build(verbose: bool = False, extra_flags=(), variant: str | None = None,
          only=None) -> str:
    build_dir, lib_path = BUILD_DIR, LIB_PATH
    if variant is not None:
        extra_flags = [*extra_flags, *VARIANTS[variant]]
        build_dir = os.path.join(BUILD_DIR, variant)
        lib_path = os.path.join(PKG, f"libpka_{variant}.so")
    os.makedirs(build_dir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        if only is not None and src not in only and os.path.exists(obj):
            continue
        cmd = _compile_cmd(src, obj, extra_flags)
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                            text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = "\n".join(l for l in out.splitlines()
                         if "packed-fp32-ops' is not a recognized feature" not in l)
        if text.strip() and (verbose or p.returncode):
            print(text, file=sys.stderr)
        if p.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = lib_path + ".tmp"
    link = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(tmp, lib_path)
    if variant is None and (only is None or CALIB_SOURCE in only or not os.path.exists(CALIB_LIB)):
        build_calibration(verbose)
    return lib_path


# The HBM read-ceiling kernels the benchmark measures against: a library of
# their own, not linked into libpka.so.
CALIB_SOURCE = "calibrate.hip"
CALIB_LIB = os.path.join(PKG, "libpka_calib.so")


def build_calibration(verbose: bool = False) -> str:
    tmp = CALIB_LIB + ".tmp"
    cmd = [HIPCC, "-x", "hip", *COMMON, "-shared", os.path.join(CSRC, CALIB_SOURCE), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, capture_output=True, text=True)
    text = "\n".join(l for l in (p.stdout + p.stderr).splitlines()
                     if "packed-fp32-ops' is not a recognized feature" not in l)
    if p.returncode:
        print(text, file=sys.stderr)
        raise RuntimeError(f"hipcc failed for {CALIB_SOURCE}")
    os.replace(tmp, CALIB_LIB)
    return CALIB_LIB


# Host-side sanitizers for the C ABI layer: AddressSanitizer and
# UndefinedBehaviorSanitizer on the host pass only (the device code is built
# as usual), every finding fatal.
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host",
                 "-fno-omit-frame-pointer"]
SANITIZED_LIB = os.path.join(PKG, "libpka_sanitized.so")


def build_sanitized(verbose: bool = False) -> str:
    """libpka_sanitized.so: abi.cpp (argument checks, sizing, dispatch) with
    host sanitizers, linked with the kernel objects of the regular build
    (built first if missing).  Load it with PKA_LIBRARY=libpka_sanitized.so
    and clang's ASan runtime preloaded."""
    objs = [os.path.join(BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    if not all(os.path.exists(o) for o in objs):
        build(verbose)
    san_dir = os.path.join(BUILD_DIR, "sanitized")
    os.makedirs(san_dir, exist_ok=True)
    abi_obj = os.path.join(san_dir, "abi.o")
    cmd = [HIPCC, "-x", "hip", *[f for f in COMMON if f != "-O3"], "-O1", "-g", *SANITIZE_HOST,
           "-c", os.path.join(CSRC, "abi.cpp"), "-o", abi_obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, capture_output=not verbose)
    link = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Xarch_host",
            "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", abi_obj,
            *[o for o in objs if not o.endswith("abi.o")], "-o", SANITIZED_LIB + ".tmp"]
    subprocess.run(link, check=True, capture_output=not verbose)
    os.replace(SANITIZED_LIB + ".tmp", SANITIZED_LIB)
    return SANITIZED_LIB


def asan_runtime() -> str:
    """clang's ASan runtime that a process loading the sanitized library
    must preload (empty when absent)."""
    import glob

    root = os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "lib", "clang")
    hits = sorted(glob.glob(os.path.join(root, "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else ""


def clean():
    shutil.rmtree(BUILD_DIR, ignore_errors=True)


if __name__ == "__main__":
    var = sys.argv[sys.argv.index("--variant") + 1] if "--variant" in sys.argv else None
    only = sys.argv[sys.argv.index("--only") + 1].split(",") if "--only" in sys.argv else None
    print(build(verbose="-v" in sys.argv, variant=var, only=only))
