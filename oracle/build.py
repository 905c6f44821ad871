"""Compile the C oracle into oracle/libkvq_oracle.so (test infrastructure only)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.environ.get("KVQ_ORACLE_LIB") or os.path.join(HERE, "libkvq_oracle.so")


def build(verbose: bool = False, src: str | None = None, out: str | None = None,
          extra_flags: list[str] | None = None) -> str:
    """Compile `src` (default: the oracle) into `out`; `extra_flags` go to gcc
    before the sources (e.g. a sanitizer build for the CPU checks)."""
    src = src or os.path.join(HERE, "kvq_oracle.c")
    out = out or LIB
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-Wextra", "-fPIC", "-shared", *(extra_flags or []), "-I", HERE, src,
           "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
