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


_SREG = re.compile(r"\bs(?:\[(\d+):(\d+)\]|(\d+)\b)")


def _sgprs(operand: str) -> set:
    out = set()
    for m in _SREG.finditer(operand):
        lo, hi = (int(m.group(1)), int(m.group(2))) if m.group(1) else (int(m.group(3)), int(m.group(3)))
        out.update(range(lo, hi + 1))
    return out


def check_vmem_sgpr_hazards(asm: str, wait_states: int = 5) -> None:
    """A VALU instruction that writes an SGPR (v_readfirstlane, v_readlane, a
    VOP3 compare with an SGPR destination, ...) needs 5 wait states before a
    vector-memory instruction reads that SGPR (its buffer resource or soffset).
    The compiler inserts them for the loads it emits itself, not for the LDS
    DMA, which is inline asm, and a DMA that reads a stale descriptor fills a
    tile with the wrong rows. Walk every buffer instruction back in program
    order (each instruction one wait state, s_nop n counts n + 1) and refuse
    the build if such a write is closer than that."""
    lines = [ln.split(";")[0].strip() for ln in asm.splitlines()]
    bad = []
    func = None
    for k, ln in enumerate(lines):
        m = re.match(r"(_Z\S+):$", ln)
        if m:
            func = m.group(1)
            continue
        if not ln.startswith("buffer_"):
            continue
        # the SGPR operands of a buffer instruction are its resource descriptor
        # and soffset, both read
        reads = _sgprs(ln.split(None, 1)[1] if " " in ln else "")
        ws = 0
        for kk in range(k - 1, -1, -1):
            prev = lines[kk]
            if not prev or prev.startswith(".") or prev.endswith(":"):
                if re.match(r"_Z\S+:$", prev):
                    break
                continue
            op = prev.split()[0]
            if op.startswith("v_") and " " in prev:
                dst = prev.split(None, 1)[1].split(",")[0]
                if _sgprs(dst) & reads:
                    bad.append(f"{func}: '{ln}' reads an SGPR that '{prev}' wrote {ws} wait states earlier")
                    break
            ws += int(prev.split()[1], 0) + 1 if op == "s_nop" else 1
            if ws >= wait_states:
                break
    if bad:
        raise RuntimeError("VALU-written SGPR read by a vector-memory instruction too soon:\n" + "\n".join(bad[:20]))


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
    # the device assembly of the same sources, for the hazard check
    asm_path = LIB + ".s"
    acmd = [HIPCC, *[f for f in FLAGS if f not in ("-fPIC", "-shared") and "kernel-resource-usage" not in f],
            *(extra or []), f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", "--cuda-device-only", "-S",
            *[os.path.join(CSRC, s_) for s_ in SOURCES], "-o", asm_path]
    ares = subprocess.run(acmd, capture_output=True, text=True)
    if ares.returncode != 0:
        raise RuntimeError("hipcc -S failed:\n" + ares.stderr[-2000:])
    with open(asm_path) as fh:
        check_vmem_sgpr_hazards(fh.read())
    os.remove(asm_path)
    if verbose and lines:
        print("\n".join(lines))
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
