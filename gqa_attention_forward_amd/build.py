"""Build libgqa.so in-tree with hipcc for gfx950.

    python -m gqa_attention_forward_amd.build [--verbose]

Always recompiles.  The library is written next to this file, where the
ctypes loader looks for it.  The C ABI and the kernels of each head dim are
separate translation units, compiled in parallel, then linked.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", name) for name in
           ("dispatch_d128.hip", "dispatch_d256.hip", "dispatch_d512.hip", "dispatch_d64.hip",
            "dispatch_d32.hip", "gqa_api.hip")]
OUT = os.path.join(HERE, "libgqa.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
NOISE = ("packed-fp32-ops", "not a recognized feature")


def hipcc() -> str:
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(ln for ln in res.stderr.splitlines() if not any(n in ln for n in NOISE))
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]
    tmpdir = tempfile.mkdtemp(prefix="gqa_build_")
    try:
        objs = [os.path.join(tmpdir, os.path.basename(src) + ".o") for src in SOURCES]
        jobs = [[hipcc(), *HIPCC_FLAGS, *inc, "-c", src, "-o", obj]
                for src, obj in zip(SOURCES, objs)]
        workers = max(1, min(len(jobs), os.cpu_count() or 1))
        with ThreadPoolExecutor(max_workers=workers) as pool:
            for f in [pool.submit(_run, cmd, verbose) for cmd in jobs]:
                f.result()
        tmp = OUT + ".tmp"
        _run([hipcc(), *HIPCC_FLAGS, "-shared", *objs, "-o", tmp], verbose)
        os.replace(tmp, OUT)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return OUT


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
