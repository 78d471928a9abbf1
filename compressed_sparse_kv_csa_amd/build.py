"""Build libdsv4.so (the gfx950 HIP kernels + the C ABI) in-tree with hipcc.

    python -m compressed_sparse_kv_csa_amd.build      # or build() from Python
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libdsv4.so")
SOURCES = ["dsv4_api.cpp", "dsv4_compress.hip", "dsv4_indexer.hip", "dsv4_attn.hip", "dsv4_quant.hip", "dsv4_cache.hip", "dsv4_linear.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 (v_pk_*_f32) instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the attention kernels touch their accumulators
    # only through MFMAs, and VGPR-form avoids AGPR<->VGPR copies every tile
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source to an object (in parallel) and link the shared library."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [HIPCC] + FLAGS + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _wait(procs.pop(0), verbose)
    for p in procs:
        _wait(p, verbose)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


def _wait(item, verbose):
    src, p = item
    out, _ = p.communicate()
    text = out.decode(errors="replace")
    # hipcc's host pass does not know the packed-fp32 feature name: harmless
    lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]
    if p.returncode != 0:
        sys.stderr.write("\n".join(lines) + "\n")
        raise RuntimeError(f"hipcc failed on {src}")
    if verbose and lines:
        print("\n".join(lines))


def sanitizer_runtime() -> str:
    """Path of the clang AddressSanitizer runtime (ASan and UBSan handlers) that a
    host process must preload to load a sanitizer build, or '' if absent."""
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "lib", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/lib/llvm/bin/clang"
    try:
        out = subprocess.check_output([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], text=True).strip()
    except (OSError, subprocess.CalledProcessError):
        return ""
    return out if os.path.isabs(out) and os.path.exists(out) else ""


def build_sanitized(outdir: str) -> str:
    """A copy of libdsv4.so whose host C-ABI layer (argument validation, workspace
    sizing, dispatch: dsv4_api.cpp) is built with AddressSanitizer and
    UndefinedBehaviorSanitizer, linked with the device objects of build().  The
    sanitizers apply to host code only (-Xarch_host); the GPU code is the same.
    Load it by setting DSV4_LIB, with sanitizer_runtime() preloaded."""
    objdir = os.path.join(HERE, "_build")
    dev = [os.path.join(objdir, s + ".o") for s in SOURCES if s.endswith(".hip")]
    if not all(os.path.exists(o) for o in dev):
        build()
    os.makedirs(outdir, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    api = os.path.join(outdir, "dsv4_api_san.o")
    subprocess.check_call([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "-fno-omit-frame-pointer"] + san +
                          [f"-I{INCLUDE}", f"-I{CSRC}", "-c", os.path.join(CSRC, "dsv4_api.cpp"), "-o", api])
    lib = os.path.join(outdir, "libdsv4_san.so")
    subprocess.check_call([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC"] + san + ["-shared-libsan", "-o", lib, api] + dev)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
