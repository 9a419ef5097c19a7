"""The C-ABI library loads, exports what include/dit_attn.h declares, and rejects
bad arguments on the host before any launch. No compute call is made here."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dit_attn.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"DIT_ATTN_API\s+[\w\s\*]+?\b(dit_attn_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import diffusion_transformer_attention_non_amd as pkg
    return pkg


def test_header_declares_the_entry_points():
    assert _declared() == sorted(["dit_attn_fwd", "dit_attn_fwd_blocksparse", "dit_attn_fwd_ex", "dit_attn_fwd_mx",
                                  "dit_attn_fwd_noalloc", "dit_attn_fwd_strided", "dit_attn_mfma_ceiling", "dit_attn_plan",
                                  "dit_attn_quantize_e4m3",
                                  "dit_attn_quantize_mx", "dit_attn_strerror", "dit_attn_version"])


def test_library_exports_every_declared_symbol(lib):
    so = ctypes.CDLL(lib._lib.LIB_PATH)
    for name in _declared():
        assert hasattr(so, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", lib._lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(_declared()) <= exported
    assert set(lib._lib.EXPORTED) == set(_declared())


def test_strerror_and_version(lib):
    assert lib.dit_attn_version() >> 16 == 2
    for st in (0, -1, -2, -3, -4, -5, 7):
        assert isinstance(lib.dit_attn_strerror(st), str) and lib.dit_attn_strerror(st)
    assert lib.dit_attn_strerror(-2) != lib.dit_attn_strerror(-1)
    assert "workspace" in lib.dit_attn_strerror(-5)


A, B_, C, O = 0x10000, 0x20000, 0x30000, 0x40000   # fake, aligned, disjoint addresses (never dereferenced)


@pytest.mark.parametrize("args,expect", [
    ((0, B_, C, O, 1, 1, 8, 64, 0.125, 0), -1),           # NULL q
    ((A, B_, C, 0, 1, 1, 8, 64, 0.125, 0), -1),           # NULL o
    ((A + 2, B_, C, O, 1, 1, 8, 64, 0.125, 0), -1),       # misaligned q
    ((A, B_, C, O + 8, 1, 1, 8, 64, 0.125, 0), -1),       # misaligned o
    ((A, B_, C, O, 0, 1, 8, 64, 0.125, 0), -1),           # B < 1
    ((A, B_, C, O, 1, 0, 8, 64, 0.125, 0), -1),           # H < 1
    ((A, B_, C, O, 1, 1, 0, 64, 0.125, 0), -1),           # N < 1
    ((A, B_, C, O, 1, 1, 8, 64, 0.0, 0), -1),             # scale 0
    ((A, B_, C, O, 1, 1, 8, 64, -1.0, 0), -1),            # negative scale
    ((A, B_, C, O, 1, 1, 8, 64, float("nan"), 0), -1),    # NaN scale
    ((A, B_, C, O, 1, 1, 8, 64, float("inf"), 0), -1),    # inf scale
    ((A, B_, C, O, 1, 1, 8, 96, 0.125, 0), -2),           # d = 96 not implemented
    ((A, B_, C, O, 1, 1, 8, 64, 0.125, 1), -2),           # fp8 needs d = 128
    ((A, B_, C, O, 1, 1, 8, 64, 0.125, 5), -2),           # unknown dtype
    ((A, B_, C, A, 1, 1, 8, 64, 0.125, 0), -1),           # o aliases q
    ((A, B_, C, C + 256, 1, 1, 8, 64, 0.125, 0), -1),     # o overlaps v (v spans 1 KiB)
    ((A, B_, C, O, 2**30, 2**30, 2**30, 128, 0.125, 0), -1),  # size overflow
])
def test_fwd_rejects_bad_arguments_before_launch(lib, args, expect):
    assert lib.dit_attn_fwd(*args, None) == expect
    assert lib.dit_attn_fwd_ex(*args, None, None, None) == expect


def test_fwd_rejects_bad_arguments_strided_too(lib):
    for args, expect in [((0, B_, C, O, 1, 1, 8, 64, 0.125, 0), -1), ((A, B_, C, O, 1, 1, 8, 96, 0.125, 0), -2)]:
        assert lib.dit_attn_fwd_strided(*args, None, None, None, None, None, 0, None) == expect
        assert lib.dit_attn_fwd_noalloc(*args, None, None, None, None, None) == expect


def test_noalloc_scratch_size_is_the_stated_bound():
    """The static scratch holds the largest workspace any plan asks for (2^17
    partial rows of 129 floats plus 2^17 floats)."""
    assert lib_scratch() == (1 << 17) * 129 * 4 + (1 << 17) * 4
    text = open(HEADER).read()
    assert f"#define DIT_ATTN_NOALLOC_SCRATCH_BYTES {lib_scratch()}" in text


def lib_scratch():
    import diffusion_transformer_attention_non_amd as pkg
    return pkg.DIT_ATTN_NOALLOC_SCRATCH_BYTES


# (B, H, N, d) = (2, 3, 8, 64) bf16 at disjoint fake addresses 16 MiB apart
SA, SB, SC, SO = 0x1000000, 0x2000000, 0x3000000, 0x4000000
BNHD = (8 * 3 * 64, 64, 3 * 64)              # [B][N][H][d]


@pytest.mark.parametrize("qkv,o,expect,why", [
    (BNHD, None, -3, "[B][N][H][d] inputs are valid (no GPU here: device error)"),
    (BNHD, BNHD, -3, "[B][N][H][d] output too"),
    ((8 * 9 * 64, 64, 9 * 64), None, -3, "token stride past H d (fused QKV buffer)"),
    ((0, 0, 64), None, -3, "inputs may share rows across batch and heads"),
    ((8 * 3 * 64, 64, 32), None, -1, "token stride below d"),
    ((8 * 3 * 64, 64, 3 * 64 + 4), None, -1, "row start not 16-byte aligned (bf16: stride % 8)"),
    ((-64, 64, 3 * 64), None, -1, "negative stride"),
    (None, (0, 64, 3 * 64), -1, "output rows repeat across the batch"),
    (None, (8 * 3 * 64, 64, 64), -1, "output heads overlap tokens"),
    (None, (8 * 64, 2 * 8 * 64, 64), -3, "output: any one-to-one order of the dimensions ([H][B][N][d])"),
    (None, (3 * 64, 8 * 3 * 64 * 2, 64), -1, "output batch stride inside the token range"),
    ((2 ** 41, 64, 192), None, -1, "stride above 2^40"),
    ((8 * 3 * 2 ** 24, 2 ** 24, 2 ** 24), None, -1, "a 128-token tile would pass 2^31 bytes"),
])
def test_strided_layout_checks(lib, qkv, o, expect, why):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; layouts are run by the GPU tests")
    st = lib.dit_attn_fwd_strided(SA, SB, SC, SO, 2, 3, 8, 64, 0.125, 0, qkv, o, None, None, None, 0, None)
    assert st == expect, why


def test_strided_output_overlap_uses_the_span(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    # o starts inside the span of a [B][N][H][d] v (v covers 2*8*3*64*2 bytes)
    assert lib.dit_attn_fwd_strided(SA, SB, SC, SC + 4096, 2, 3, 8, 64, 0.125, 0, BNHD, None, None, None, None, 0,
                                    None) == -1


# block-sparse: (B, H, N, d) = (1, 2, 1000, 128) bf16, 4 query blocks, 16 key blocks
LB, LC = 0x5000000, 0x6000000


@pytest.mark.parametrize("args,lists,expect,why", [
    ((SA, SB, SC, SO, 1, 2, 1000, 128, 0.1, 0), (LB, LC, 16), -3, "valid (no GPU here: device error)"),
    ((SA, SB, SC, SO, 1, 2, 1000, 128, 0.1, 0), (LB, LC, 1), -3, "max_blocks 1"),
    ((SA, SB, SC, SO, 1, 2, 1000, 128, 0.1, 0), (0, LC, 16), -1, "NULL block list"),
    ((SA, SB, SC, SO, 1, 2, 1000, 128, 0.1, 0), (LB, 0, 16), -1, "NULL counts"),
    ((SA, SB, SC, SO, 1, 2, 1000, 128, 0.1, 0), (LB + 2, LC, 16), -1, "misaligned block list"),
    ((SA, SB, SC, SO, 1, 2, 1000, 128, 0.1, 0), (LB, LC + 1, 16), -1, "misaligned counts"),
    ((SA, SB, SC, SO, 1, 2, 1000, 128, 0.1, 0), (LB, LC, 0), -1, "max_blocks 0"),
    ((SA, SB, SC, SO, 1, 2, 1000, 128, 0.1, 0), (LB, LC, 17), -1, "max_blocks above the key-block count"),
    ((SA, SB, SC, SO, 1, 2, 1000, 128, 0.1, 0), (SO + 64, LC, 16), -1, "block list overlaps o"),
    ((SA, SB, SC, SO, 1, 2, 1000, 128, 0.1, 0), (LB, SO, 16), -1, "counts alias o"),
    ((SA, SB, SC, SO, 1, 2, 1000, 128, 0.1, 0), (SA, SB, 16), -3, "lists may share memory with inputs"),
    ((SA, SB, SC, SO, 1, 2, 1000, 64, 0.1, 0), (LB, LC, 16), -2, "d = 64 not implemented"),
    ((SA, SB, SC, SO, 1, 2, 1000, 128, 0.1, 1), (LB, LC, 16), -2, "fp8 not implemented"),
    ((0, SB, SC, SO, 1, 2, 1000, 128, 0.1, 0), (LB, LC, 16), -1, "NULL q (shared checks)"),
    ((SA, SB, SC, SO, 1, 2, 1000, 128, 0.0, 0), (LB, LC, 16), -1, "scale 0 (shared checks)"),
])
def test_blocksparse_checks(lib, args, lists, expect, why):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; the block-sparse path is run by the GPU tests")
    assert lib.dit_attn_fwd_blocksparse(*args, *lists, None, None, None, None, 0, None) == expect, why


def test_blocksparse_list_overlapping_lse(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    lse = 0x7000000
    args = (SA, SB, SC, SO, 1, 2, 1000, 128, 0.1, 0)
    assert lib.dit_attn_fwd_blocksparse(*args, LB, LC, 16, None, None, lse, None, 0, None) == -3
    assert lib.dit_attn_fwd_blocksparse(*args, lse + 4000, LC, 16, None, None, lse, None, 0, None) == -1
    assert lib.dit_attn_fwd_blocksparse(*args, LB, lse + 8, 16, None, None, lse, None, 0, None) == -1


# MX: (B, H, N, d) = (1, 2, 100, 128); codes 25600 bytes, row scales 800, V scales 4 * 128 * 2 = 1024
QS, KS, VS = 0x8000000, 0x9000000, 0xA000000


@pytest.mark.parametrize("args,expect,why", [
    ((SA, SB, SC, QS, KS, VS, SO, 1, 2, 100, 128, 0.1, None), -3, "valid (no GPU here: device error)"),
    ((SA, SB, SC, 0, KS, VS, SO, 1, 2, 100, 128, 0.1, None), -1, "NULL q scales"),
    ((SA, SB, SC, QS, KS + 4, VS, SO, 1, 2, 100, 128, 0.1, None), -1, "k scales not 16-byte aligned"),
    ((SA, SB, SC, QS, KS, SO + 64, SO, 1, 2, 100, 128, 0.1, None), -1, "v scales overlap o"),
    ((SA, SB, SC, QS, KS, VS, SO, 1, 2, 100, 64, 0.1, None), -2, "d = 64"),
    ((SA, SB, SC, QS, KS, VS, SO, 1, 2, 100, 128, -1.0, None), -1, "negative scale"),
    ((SA, SB, SC, QS, KS, VS, SA + 16, 1, 2, 100, 128, 0.1, None), -1, "o overlaps q8"),
    ((SA, SB, SC, QS, KS, VS, SO, 1, 2, 100, 128, 0.1, QS + 400), -1, "lse overlaps q scales"),
])
def test_mx_attention_checks(lib, args, expect, why):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert lib.dit_attn_fwd_mx(*args, None, 0, None) == expect, why


@pytest.mark.parametrize("args,expect,why", [
    ((SA, 1, 2, 100, 128, 0, SB, SC), -3, "along d (no GPU here: device error)"),
    ((SA, 1, 2, 100, 128, 1, SB, SC), -3, "along tokens"),
    ((SA, 1, 2, 100, 128, 2, SB, SC), -1, "unknown axis"),
    ((SA, 1, 2, 100, 48, 0, SB, SC), -1, "d not a multiple of 32"),
    ((SA, 1, 2, 100, 2048, 0, SB, SC), -1, "d above 1024"),
    ((SA, 1, 2, 0, 128, 0, SB, SC), -1, "N = 0"),
    ((SA, 1, 2, 100, 128, 0, SA + 64, SC), -1, "codes overlap x"),
    ((SA, 1, 2, 100, 128, 0, SB, SB + 100), -1, "scales overlap codes"),
    ((SA, 300, 300, 100, 128, 1, SB, SC), -1, "B H above the token kernel's grid"),
])
def test_mx_quantize_checks(lib, args, expect, why):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert lib.dit_attn_quantize_mx(*args, None) == expect, why


WS = 0xB000000     # a fake workspace address, 16 MiB from the others


@pytest.mark.parametrize("ws,nbytes,expect,why", [
    (WS, 1 << 20, -3, "valid workspace (no GPU here: device error)"),
    (None, 0, -3, "no workspace"),
    (WS + 8, 0, -3, "a pointer without bytes is not used, so not checked"),
    (None, 1 << 20, -1, "bytes without a pointer"),
    (WS + 8, 1 << 20, -1, "workspace not 16-byte aligned"),
    (WS, -16, -1, "negative size"),
    (SA - 256, 1024, -1, "workspace runs into q"),
    (SO + 512, 1 << 20, -1, "workspace inside o"),
    (0x7000000 - 64, 128, -1, "workspace runs into lse"),
])
def test_workspace_checks(lib, ws, nbytes, expect, why):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st = lib.dit_attn_fwd_strided(SA, SB, SC, SO, 2, 3, 8, 128, 0.125, 0, None, None, None, 0x7000000, ws, nbytes,
                                  None)
    assert st == expect, why


def test_workspace_checks_of_the_list_and_scale_forms(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    sparse = (SA, SB, SC, SO, 1, 2, 1000, 128, 0.1, 0, LB, LC, 16, None, None, None)
    assert lib.dit_attn_fwd_blocksparse(*sparse, WS, 1 << 20, None) == -3
    assert lib.dit_attn_fwd_blocksparse(*sparse, LB - 64, 1 << 20, None) == -1      # over the block lists
    assert lib.dit_attn_fwd_blocksparse(*sparse, LC, 16, None) == -1                # over the counts
    mx = (SA, SB, SC, QS, KS, VS, SO, 1, 2, 100, 128, 0.1, None)
    assert lib.dit_attn_fwd_mx(*mx, WS, 1 << 20, None) == -3
    assert lib.dit_attn_fwd_mx(*mx, VS - 16, 64, None) == -1                        # over the V scales
    assert lib.dit_attn_fwd_mx(*mx, WS + 4, 64, None) == -1


def test_fwd_ex_rejects_bad_lse(lib):
    args = (A, B_, C, O, 1, 1, 8, 64, 0.125, 0)
    assert lib.dit_attn_fwd_ex(*args, None, 0x50002, None) == -1      # misaligned lse
    assert lib.dit_attn_fwd_ex(*args, None, O + 4, None) == -1        # lse overlaps o
    assert lib.dit_attn_fwd_ex(*args, 0x50002, None, None) == -1      # misaligned descale


def test_quantize_rejects_bad_arguments(lib):
    assert lib.dit_attn_quantize_e4m3(0, 64, B_, C, O, None) == -1
    assert lib.dit_attn_quantize_e4m3(A, 60, B_, C, O, None) == -1    # n not a multiple of 8
    assert lib.dit_attn_quantize_e4m3(A, 0, B_, C, O, None) == -1
    assert lib.dit_attn_quantize_e4m3(A, 64, A + 64, C, O, None) == -1  # x8 overlaps x
    assert lib.dit_attn_quantize_e4m3(A, 64, B_, O, O, None) == -1      # descale aliases ws


def test_mfma_ceiling_rejects_bad_arguments(lib):
    f = lib.dit_attn_mfma_ceiling
    assert f(0, 0, 1, A, 64)[0] == -1             # rounds < 1
    assert f(0, 10, -1, A, 64)[0] == -1           # workgroups < 0
    assert f(0, 10, (1 << 20) + 1, A, 1 << 30)[0] == -1
    assert f(0, 10, 1, 0, 64)[0] == -1            # NULL record
    assert f(0, 10, 1, A + 4, 64)[0] == -1        # misaligned record
    assert f(0, 10, 1, A, -1)[0] == -1
    assert f(7, 10, 1, A, 64)[0] == -2            # dtype


def test_valid_call_without_gpu_reports_device_error(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; covered by the GPU tests")
    assert lib.dit_attn_fwd(A, B_, C, O, 1, 1, 8, 64, 0.125, 0, None) == -3
    assert lib.dit_attn_mfma_ceiling(0, 10, 1, A, 64)[0] == -3


def test_build_refuses_spilling_attention_kernels():
    """The build reads hipcc's per-kernel resource report and refuses an
    attention kernel with scratch (spill) bytes; other kernels may spill."""
    from diffusion_transformer_attention_non_amd.build import check_no_spills
    ok = ("a.h:1:1: remark: Function Name: _ZN7ditattn24attn_fwd_fp8_pipe_kernelX [-Rpass-analysis=kernel-resource-usage]\n"
          "a.h:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]\n"
          "b.h:1:1: remark: Function Name: _ZN7ditattn17quant_e4m3_kernelX [-Rpass-analysis=kernel-resource-usage]\n"
          "b.h:1:1: remark:     ScratchSize [bytes/lane]: 64 [-Rpass-analysis=kernel-resource-usage]\n")
    check_no_spills(ok)
    bad = ok.replace("ScratchSize [bytes/lane]: 0", "ScratchSize [bytes/lane]: 384")
    with pytest.raises(RuntimeError, match="attn_fwd_fp8_pipe_kernelX: 384"):
        check_no_spills(bad)


def test_build_refuses_a_dma_reading_a_fresh_valu_written_sgpr():
    """A VALU write of an SGPR needs 5 wait states before a buffer
    instruction reads it (resource descriptor or soffset); the inline-asm LDS
    DMA gets none from the compiler, so the build checks the ISA."""
    from diffusion_transformer_attention_non_amd.build import check_vmem_sgpr_hazards
    head = "_ZN7ditattn1kE:\n"
    bad = head + ("\tv_readfirstlane_b32 s66, v1\n\t;;#ASMSTART\n"
                  "\tbuffer_load_dwordx4 v233, s[64:67], 0 offen lds\n\t;;#ASMEND\n")
    with pytest.raises(RuntimeError, match="s66"):
        check_vmem_sgpr_hazards(bad)
    # five wait states (instructions, or an s_nop 4) in between are enough
    check_vmem_sgpr_hazards(head + "\tv_readfirstlane_b32 s66, v1\n\ts_nop 4\n"
                            "\tbuffer_load_dwordx4 v233, s[64:67], 0 offen lds\n")
    check_vmem_sgpr_hazards(head + "\tv_readfirstlane_b32 s66, v1\n" + "\ts_add_i32 s1, s1, 1\n" * 5 +
                            "\tbuffer_load_dwordx4 v233, s[64:67], 0 offen lds\n")
    with pytest.raises(RuntimeError):
        check_vmem_sgpr_hazards(head + "\tv_readfirstlane_b32 s70, v1\n\ts_nop 2\n"
                                "\tbuffer_load_dwordx4 v2, s[68:71], 0 offen lds\n")
    # scalar writes and unrelated VALU-written SGPRs are fine
    check_vmem_sgpr_hazards(head + "\ts_min_i32 s66, s66, 64\n\tv_readfirstlane_b32 s5, v1\n"
                            "\tbuffer_load_dwordx4 v233, s[64:67], 0 offen lds\n")


def test_inline_asm_that_writes_scc_declares_it():
    """Scalar ALU instructions (compares, min/max, add/sub, shifts, logic) set
    SCC. An inline-asm statement that contains one without declaring "scc"
    clobbered lets the compiler keep a carry or compare result in SCC across
    it: a 64-bit address add split by such an asm gets a wrong high word (a
    GPU memory fault). Every asm statement of the kernels is checked."""
    csrc = os.path.join(ROOT, "diffusion_transformer_attention_non_amd", "csrc")
    writes_scc = re.compile(r"\bs_(cmp|min|max|add|sub|and|or|xor|lsh|ashr|bfe|bitcmp|absdiff|mul_hi)\w*")
    checked = 0
    for fn in sorted(os.listdir(csrc)):
        text = open(os.path.join(csrc, fn)).read()
        for m in re.finditer(r"\basm\s*(volatile\s*)?\(", text):
            depth, k = 1, m.end()
            while depth:
                depth += {"(": 1, ")": -1}.get(text[k], 0)
                k += 1
            stmt = text[m.start():k]
            checked += 1
            if writes_scc.search(stmt):
                assert '"scc"' in stmt, (fn, stmt[:200])
    assert checked > 10
