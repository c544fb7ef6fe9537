"""Build libgemma3_attn.so (gfx950) in-tree with hipcc.

    python -m global_layers_amd.build        # or: python global_layers_amd/build.py

Each source is compiled to an object under ``_build/`` (in parallel), then
linked into ``global_layers_amd/libgemma3_attn.so``. Always recompiles.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgemma3_attn.so")
SOURCES = ["api.cpp", "gemm_bf16.hip", "qk_norm_rope.hip", "flash_attn.hip",
           "decode_attn.hip", "fp32_path.hip", "cache_write.hip",
           "block.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-I", os.path.join(ROOT, "include"),
            # packed fp32 VALU forms off (see the design notes)
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-result"]


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer instrumentation
# (device code is built as usual); the sanitizer runtime is not linked in, the
# process that loads such a library preloads it (see tests/test_abi_sanitized.py).
SANITIZE_FLAGS = ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                  "-fsanitize=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src: str, build_dir: str = BUILD, sanitize: bool = False) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    flags = common_flags() + (SANITIZE_FLAGS if sanitize else [])
    cmd = [hipcc(), *flags, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    noise = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if noise:
        sys.stderr.write(f"[{src}]\n" + "\n".join(noise) + "\n")
    return obj


def build(verbose: bool = True, out_dir: str = None, sanitize: bool = False) -> str:
    """Compile every source and link the library (into the package, or into
    out_dir with its objects, e.g. for the host-sanitizer build)."""
    build_dir = BUILD if out_dir is None else os.path.join(out_dir, "_build")
    lib_path = LIB if out_dir is None else os.path.join(out_dir, os.path.basename(LIB))
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, sanitize), SOURCES))
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path}")
    return lib_path


if __name__ == "__main__":
    build()
