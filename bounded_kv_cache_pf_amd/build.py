"""Compile libpf.so (HIP for gfx950) in place, next to this file.

`python -m bounded_kv_cache_pf_amd.build --sanitize` builds libpf_asan.so
instead: the same sources with AddressSanitizer and UndefinedBehaviorSanitizer
on the host code only (argument validation, planning, error reporting); the
device code is compiled as usual. It is for running the host-side tests under
the sanitizers; nothing loads it by default."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpf.so")
ASAN_LIB = os.path.join(HERE, "libpf_asan.so")
SOURCES = ["pf_status.hip", "pf_rope.hip", "pf_select.hip", "pf_attn.hip", "pf_rollin.hip", "pf_hr.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    # packed fp32 VALU forms stay off: plain float code is scheduled as scalar ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


# host-side sanitizers: each -fsanitize= applies to the host compilation only
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined", "-g"]


def asan_runtime() -> str:
    """Path of the compiler's AddressSanitizer runtime (preloaded into the
    process that loads libpf_asan.so), or '' if it is not installed."""
    res = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        import glob
        found = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        path = found[0] if found else ""
    return path


def build(verbose: bool = False, sanitize: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    out = ASAN_LIB if sanitize else LIB
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *(SANITIZE_FLAGS if sanitize else []), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
