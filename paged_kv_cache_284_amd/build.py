"""Build libpagedkv.so in-tree with hipcc for gfx950.

    python -m paged_kv_cache_284_amd.build        # or __graft_entry__.build()
    python -m paged_kv_cache_284_amd.build --host-sanitized OUT.so   # allocator, ASan + UBSan

Every source under csrc/ is compiled (in parallel) into csrc/../_build and linked into
paged_kv_cache_284_amd/libpagedkv.so.  The build always recompiles.
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
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpagedkv.so")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]


# Per-source flags.  The prefill kernel keeps its score tiles in VGPRs: with the default
# heuristics at one wave per SIMD the compiler places them in accumulator registers that
# overlap the P.V accumulators and copies both sides through VGPRs every key pair.
EXTRA = {
    "prefill_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc() -> str:
    env = os.environ.get("HIPCC")
    if env:
        return env
    for cand in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc(), *COMMON, *EXTRA.get(os.path.basename(src), []), *lang, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device-only feature flag; that warning is expected
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


# The host allocator alone (csrc/alloc.cpp: plain C++17, no HIP) built with AddressSanitizer and
# UndefinedBehaviorSanitizer by the host compiler.  The result exports the allocator's C ABI and
# nothing else; a process loads it with the ASan runtime preloaded (see
# tests/test_host_sanitizers.py) and binds it with paged_kv_cache_284_amd.use_host_library().
SANITIZE_FLAGS = [
    "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
]


def build_host_sanitized(out: str) -> str:
    cxx = os.environ.get("CXX", "g++")
    cmd = [cxx, *SANITIZE_FLAGS, "-shared", "-fPIC", f"-I{os.path.join(ROOT, 'include')}",
           os.path.join(CSRC, "alloc.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized host build failed:\n{' '.join(cmd)}\n{r.stderr}")
    return out


if __name__ == "__main__":
    if len(sys.argv) > 2 and sys.argv[1] == "--host-sanitized":
        print("built", build_host_sanitized(os.path.abspath(sys.argv[2])))
    else:
        build(verbose=True)
