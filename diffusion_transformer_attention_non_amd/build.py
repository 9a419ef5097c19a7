"""Build libditattn.so in place with hipcc for gfx950.

Usage: python -m diffusion_transformer_attention_non_amd.build [--verbose]
"""
from __future__ import annotations

import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libditattn.so")
SOURCES = ["dit_attn.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 VALU instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in VGPRs: avoids AGPR<->VGPR copies around VALU rescaling
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-command-line-argument",
    # per-kernel register and scratch report, checked below
    "-Rpass-analysis=kernel-resource-usage",
]


def check_no_spills(report: str) -> None:
    """The attention kernels run one wave per SIMD with every register in
    use; a spill to scratch adds vector-memory waits that stall the LDS-DMA
    pipeline (several times slower). Refuse such a build."""
    name = None
    bad = []
    for ln in report.splitlines():
        m = re.search(r"Function Name: (\S+)", ln)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", ln)
        if m and name and re.search(r"attn_(fwd|split)", name) and int(m.group(1)) > 0:
            bad.append(f"{name}: {m.group(1)} bytes/lane")
    if bad:
        raise RuntimeError("attention kernels spill registers to scratch:\n" + "\n".join(bad))


def build(verbose: bool = False, extra=None) -> str:
    cmd = [HIPCC, *FLAGS, *(extra or []), f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = res.stdout + res.stderr
    lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln and "remark:" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(lines))
    check_no_spills(out)
    if verbose and lines:
        print("\n".join(lines))
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
