"""Build libkvq.so (HIP, gfx950) in-tree.

Every HIP source is compiled separately with hipcc and linked into
``evicted_kv_cache_amd/libkvq.so``.  Compile flags:
  --offload-arch=gfx950      MI355X only
  -ffp-contract=off          no implicit FMA: the quantization arithmetic is a
                             bit-exact specification; kernels that want FMA
                             call fmaf explicitly
  -target-feature -packed-fp32-ops
                             no compiler-generated packed fp32 instructions

Sources that hold inline asm are also compiled to device assembly, which
``asm_check.scan`` reads for asm statements placed where the hardware needs
wait states the compiler does not insert for them; a hit fails the build.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkvq.so")
BUILD_DIR = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.hip", "quantize.hip", "decode.hip", "decode_mfma.hip", "prefill_attn.hip", "evict.hip",
           "snapkv.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = [l for l in (r.stderr or "").splitlines()
             if l.strip() and "packed-fp32-ops" not in l and "not a recognized feature" not in l]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    if noise and verbose:
        print("\n".join(noise), flush=True)
    return obj


def _check_asm(src: str, verbose: bool) -> None:
    from .asm_check import scan
    out = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".device.s")
    cmd = [HIPCC, *FLAGS, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{r.stderr}")
    with open(out) as f:
        hits = scan(f.read())
    if hits:
        raise RuntimeError(f"{src}: inline asm right after a transcendental instruction it depends on "
                           f"(needs a wait state the compiler does not add):\n" + "\n".join(hits[:20]))


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    asm_srcs = [s for s in srcs if "asm(" in open(os.path.join(CSRC, s)).read()]
    with ThreadPoolExecutor(min(8, len(srcs) + len(asm_srcs))) as ex:
        checks = [ex.submit(_check_asm, s, verbose) for s in asm_srcs]
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
        for c in checks:
            c.result()
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
