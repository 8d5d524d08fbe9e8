"""Build libattn_sinks.so (gfx950) in-tree with hipcc.

    python -m gqa_paged_attention_amd.build        # or build() from Python

Every HIP/C++ source under csrc/ is compiled for gfx950 only and linked into
one shared library next to this file.  Packed fp32 VALU instructions are
disabled on the device pass (the host pass warns that it does not know the
feature; that warning is harmless).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libattn_sinks.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
BUILD_DIR = os.path.join(PKG_DIR, "_build")

SOURCES = ["api.cpp", "append.hip", "decode.hip", "prefill.hip", "rows_f32.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


COMMON_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-Wall",
    "-Wno-unused-command-line-argument",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


# Kernels whose waits for their direct global-to-LDS tile loads are counted
# by hand (s_waitcnt vmcnt(N) leaves the next tile's loads in flight): that
# count is right only while those loads are the wave's only vector-memory
# operations in the loop, so a register spill (scratch traffic) there would
# let a wave read an LDS stage before it lands.  The build refuses them with
# any scratch.
NO_SCRATCH_KERNELS = ("prefill_bf16I", "mixed_bf16I")


def check_no_scratch(remarks: str, src: str) -> None:
    """Parse -Rpass-analysis=kernel-resource-usage remarks; raise if a kernel
    of NO_SCRATCH_KERNELS uses scratch."""
    name = None
    for line in remarks.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name and any(k in name for k in NO_SCRATCH_KERNELS) and int(m.group(1)):
            raise RuntimeError(
                f"{src}: kernel {name} uses {m.group(1)} bytes/lane of scratch; its hand-counted "
                "waits for the direct tile loads assume no other vector-memory operation in its "
                "loop (reduce its register use)")


# A vector instruction that writes a scalar register (v_readlane,
# v_readfirstlane: spill restores among them) needs five wait states before a
# vector-memory instruction reads that register.  The compiler inserts them
# for its own instructions but does not look inside inline assembly, so the
# direct tile loads carry them in their assembly; check_dma_hazards checks
# the compiled assembly for any load that lacks them.
_DMA = re.compile(r"global_load_lds_dwordx4\s+v\d+,\s+s\[(\d+):(\d+)\]")
_VALU_SGPR_WRITE = re.compile(r"^(v_readlane_b32|v_readfirstlane_b32)\s+s(\d+)\b")
_NOP = re.compile(r"^s_nop\s+(\d+)")


def check_dma_hazards(asm: str) -> int:
    """Raise if some global_load_lds reads a scalar base register that a
    vector instruction wrote fewer than five wait states earlier (walking back
    through the listing; s_nop N counts N + 1).  Returns the loads checked."""
    lines = [l.strip() for l in asm.splitlines()]
    checked = 0
    for i, line in enumerate(lines):
        m = _DMA.search(line)
        if not m:
            continue
        checked += 1
        regs = {int(m.group(1)), int(m.group(2))}
        waits, k = 0, i - 1
        while k >= 0 and waits < 5:
            t = lines[k]
            k -= 1
            if not t or t[0] in ";." or t.endswith(":"):
                continue
            w = _VALU_SGPR_WRITE.match(t)
            if w and int(w.group(2)) in regs:
                raise RuntimeError(f"line {i + 1}: {line!r} reads s{w.group(2)}, written by "
                                   f"{t!r} only {waits} wait states before")
            n = _NOP.match(t)
            waits += int(n.group(1)) + 1 if n else 1
    return checked


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, "-Rpass-analysis=kernel-resource-usage", "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    check_no_scratch(res.stderr, src)
    return obj


def build(verbose: bool = False) -> str:
    """Compile and link the library; returns its path.  Always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
