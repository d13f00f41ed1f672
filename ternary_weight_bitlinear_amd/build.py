"""Ahead-of-time build of libbitnet_hip.so for gfx950 (MI355X).

Each source is compiled by hipcc into an object under ``_build/`` (in
parallel), then linked into ``libbitnet_hip.so`` next to this file.  Device
code is built for gfx950 only, with contraction off and correctly rounded
fp32 division, so the device arithmetic is the IEEE operation order that the
header documents; packed-fp32 instructions are disabled.

Usage: ``python -m ternary_weight_bitlinear_amd.build`` (or ``build()``).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
BUILD = PKG / "_build"
LIBRARY = PKG / "libbitnet_hip.so"
ARCH = "gfx950"

SOURCES = ["bitnet_api.cpp", "act_quant.hip", "gemv.hip", "gemm.hip", "pack.hip", "i2s.hip", "gemv_a16.hip"]

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    f"-I{ROOT / 'include'}", f"-I{CSRC}",
]


def hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _compile(src: str) -> Path:
    obj = BUILD / (Path(src).stem + ".o")
    cmd = [hipcc(), *FLAGS, "-c", str(CSRC / src), "-o", str(obj)]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> Path:
    """Compile every source for gfx950 and link the shared library."""
    BUILD.mkdir(exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as pool:
        objs = list(pool.map(_compile, SOURCES))
    tmp = LIBRARY.with_suffix(f".so.tmp{os.getpid()}")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIBRARY)
    if verbose:
        print(f"built {LIBRARY}")
    return LIBRARY


SANITIZED = BUILD / "sanitize" / "libbitnet_hip_san.so"
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def build_sanitized(verbose: bool = False) -> Path:
    """A copy of the library whose host code (argument checks, host packer, host
    I2_S paths, packed-weight files, plans) is built with AddressSanitizer and
    UndefinedBehaviorSanitizer; device code as in build().  For CPU tests only:
    load it with the compiler's ASan runtime preloaded."""
    build(verbose=verbose)
    out_dir = SANITIZED.parent
    out_dir.mkdir(parents=True, exist_ok=True)
    obj = out_dir / "bitnet_api.o"
    flags = [f for f in FLAGS if f != "-O3"] + ["-O1", "-g"] + SANITIZE_FLAGS
    res = subprocess.run([hipcc(), "-x", "hip", *flags, "-c", str(CSRC / "bitnet_api.cpp"), "-o", str(obj)],
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on bitnet_api.cpp (sanitized):\n{res.stderr}")
    objs = [obj] + [BUILD / (Path(src).stem + ".o") for src in SOURCES if src != "bitnet_api.cpp"]
    tmp = SANITIZED.with_suffix(f".so.tmp{os.getpid()}")
    res = subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)],
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed (sanitized):\n{res.stderr}")
    os.replace(tmp, SANITIZED)
    if verbose:
        print(f"built {SANITIZED}")
    return SANITIZED


def asan_runtime() -> Path:
    """The ASan runtime of the compiler that built the sanitized library."""
    root = Path(hipcc()).resolve().parent.parent
    for base in (root / "llvm" / "lib" / "clang", root / "lib" / "llvm" / "lib" / "clang", Path("/opt/rocm/llvm/lib/clang")):
        found = sorted(base.glob("*/lib/linux/libclang_rt.asan-x86_64.so"))
        if found:
            return found[-1]
    raise FileNotFoundError("libclang_rt.asan-x86_64.so not found")


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "sanitized":
        build_sanitized(verbose=True)
    else:
        build(verbose=True)
    sys.exit(0)
