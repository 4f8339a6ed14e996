"""Build libdit_attn.so (gfx950) in-tree with hipcc.

    python -m attention_qk_norm_rope_amd.build

Compiles every csrc/*.hip for gfx950 only and links them into
attention_qk_norm_rope_amd/libdit_attn.so.  hipcc cross-compiles, so this runs
on a machine without a GPU.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdit_attn.so")
BUILD_DIR = os.path.join(PKG, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 VALU ops are disabled on purpose (-packed-fp32-ops).
DEVICE_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics",
]


def sources() -> list:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *DEVICE_FLAGS, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    # hipcc's host pass does not know the packed-fp32 feature; that warning is expected.
    noise = [l for l in res.stderr.splitlines() if l.strip() and "packed-fp32-ops" not in l
             and "unknown target feature" not in l and "warning generated" not in l]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def build(verbose: bool = False) -> str:
    """Compile and link; always rebuilds.  Returns the library path."""
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    # A kernel whose host-side launch stub the compiler dropped would leave
    # an undefined __device_stub__ symbol that only fails at load time.
    nm = shutil.which("nm")
    if nm:
        syms = subprocess.run([nm, "-u", tmp], capture_output=True, text=True).stdout
        missing = [l.split()[-1] for l in syms.splitlines() if "__device_stub__" in l]
        if missing:
            raise RuntimeError(f"undefined kernel launch stubs in {tmp}: {missing}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
