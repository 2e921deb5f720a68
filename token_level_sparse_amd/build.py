"""Build libjssa.so (HIP, gfx950) in-tree.

    python -m token_level_sparse_amd.build

Compiles every source under csrc/ with hipcc for gfx950 and links the shared
library next to this file. Objects are cached under _build/ and rebuilt when a
source or header is newer.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libjssa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # packed fp32 ops (v_pk_*_f32) stay off: plain fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics", "-Wall", "-Wno-unused-result",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def headers():
    hs = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hpp")]
    return hs + [os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h")]


# Host-sanitizer build (tests only): the host C++ sources (the C-ABI layer and
# the host spectral step) compiled with AddressSanitizer and UBSan on their
# host side; the GPU kernels are the ordinary objects. Loaded with the ASan
# runtime preloaded (see sanitizer_runtime()).
SAN_BUILD = os.path.join(BUILD, "san")
SAN_LIB = os.path.join(SAN_BUILD, "libjssa.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _compile(src: str, force: bool, san: bool = False) -> str:
    obj = os.path.join(SAN_BUILD if san else BUILD, os.path.basename(src) + ".o")
    newest = max(os.path.getmtime(p) for p in [src] + headers())
    if force or not os.path.exists(obj) or os.path.getmtime(obj) < newest:
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        extra = [f for f in FLAGS if f != "-O3"] + ["-O1"] + SAN_FLAGS if san else FLAGS
        cmd = [HIPCC, *extra, *lang, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        noise = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
        if noise:
            sys.stderr.write("\n".join(noise) + "\n")
    return obj


def build(force: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, force), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def sanitizer_runtime() -> str:
    """Path of the AddressSanitizer runtime the sanitized library needs
    preloaded (LD_PRELOAD) into an unsanitized Python."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return r.stdout.strip()


def build_sanitized(force: bool = False) -> str:
    """_build/san/libjssa.so: the library with its host C++ sources (.cpp)
    built under ASan + UBSan; kernels (.hip) as in the ordinary build."""
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(SAN_BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, force, san=s.endswith(".cpp")), srcs))
    tmp = SAN_LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs,
           "-fsanitize=address", "-fsanitize=undefined", "-shared-libsan"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitized(force="--force" in sys.argv))
    else:
        print(build(force="--force" in sys.argv))
