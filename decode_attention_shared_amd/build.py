"""Build libhp_attn.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Each translation unit is compiled by hipcc in parallel into ``_build/`` and
linked next to this file.  Every HIP compile carries
``-Xclang -target-feature -Xclang -packed-fp32-ops`` (no packed fp32 ALU
instructions are generated); hipcc's host pass warns that it does not know
the feature, which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libhp_attn.so")
SOURCES = ["api.cpp", "tree.cpp", "pakv.cpp", "prefix_kernel.hip", "suffix_kernel.hip",
           "merge_kernel.hip", "append_kernel.hip", "stream_kernel.hip", "noalloc.hip",
           "probe_kernel.hip"]
SOURCE_FLAGS = {}  # per-source extra flags
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    return "hipcc"


def _compile(src: str, extra, out_dir: str = BUILD_DIR) -> str:
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), "-x", "hip", *COMMON_FLAGS, *SOURCE_FLAGS.get(src, []), *extra, "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass always warns about the packed-fp32 feature; show anything else
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


# Host-side sanitizer build (AddressSanitizer + UndefinedBehaviorSanitizer on the
# host code of the C ABI: validation, planning, the prefix-tree manager).  Each
# -fsanitize applies to the host pass only (-Xarch_host); the kernels are built
# as usual.  The result is a separate library, loaded by setting HP_ATTN_LIB;
# Python itself is not instrumented, so the runtime has to be preloaded:
#   python -m decode_attention_shared_amd.build --sanitize
#   HP_ATTN_LIB=$PWD/_build_san/libhp_attn_san.so \
#   LD_PRELOAD=$(/opt/rocm/llvm/bin/clang -print-file-name=libclang_rt.asan-x86_64.so) \
#   ASAN_OPTIONS=detect_leaks=0:halt_on_error=1 UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1 \
#   python -m pytest tests -m "not gpu"
SAN_BUILD_DIR = os.path.join(ROOT, "_build_san")
SAN_LIB_PATH = os.path.join(SAN_BUILD_DIR, "libhp_attn_san.so")
SAN_SOURCES = ("api.cpp", "tree.cpp", "pakv.cpp", "noalloc.hip")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all",
             "-g"]


def build(extra_flags=(), jobs: int = 4, sanitize: bool = False) -> str:
    """Compile every source and link libhp_attn.so (with sanitize=True, the host-side
    sanitizer build instead).  Always recompiles."""
    out_dir = SAN_BUILD_DIR if sanitize else BUILD_DIR
    out_lib = SAN_LIB_PATH if sanitize else LIB_PATH
    os.makedirs(out_dir, exist_ok=True)

    def one(src):
        flags = list(extra_flags) + (SAN_FLAGS if sanitize and src in SAN_SOURCES else [])
        return _compile(src, flags, out_dir)

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = out_lib + f".tmp{os.getpid()}"
    # the sanitizer runtime is not linked in: it is preloaded into the process
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out_lib)
    return out_lib


if __name__ == "__main__":
    print(build(sanitize="--sanitize" in sys.argv[1:]))
