"""dit_attn_fwd_noalloc, the entry point for callers that cannot allocate,
through the C ABI: its output against dit_attn_fwd_strided's with a
caller-owned workspace (the same plan and kernels, so the same bytes), and
against the fp64 oracle to the bf16 bound, on calls in a row that reuse the
library's scratch array with shrinking inputs."""
import math

import numpy as np
import pytest
import torch

import oracle
from parity import check_full, oracle_ref, say
from workloads import one_growing_row, random_qkv, sample_rows

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _dit():
    import diffusion_transformer_attention_non_amd as dit
    return dit


def _both(q, k, v, scale, dtype=None, descale=None, want_lse=True):
    """(O, lse) from dit_attn_fwd_noalloc and from dit_attn_fwd_strided with a workspace."""
    dit = _dit()
    dtype = dit.DIT_ATTN_BF16 if dtype is None else dtype
    B, H, N, d = q.shape
    handle = torch.cuda.current_stream().cuda_stream
    outs = []
    for noalloc in (True, False):
        o = torch.full((B, H, N, d), float("nan"), dtype=torch.bfloat16, device=DEV)
        lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=DEV) if want_lse else None
        if noalloc:
            st = dit.dit_attn_fwd_noalloc(q, k, v, o, B, H, N, d, scale, dtype, None, None, descale, lse, handle)
        else:
            nbytes = dit.workspace_bytes(B, H, N, d, dtype, lse=want_lse)
            ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=DEV)
            st = dit.dit_attn_fwd_strided(q, k, v, o, B, H, N, d, scale, dtype, None, None, descale, lse, ws,
                                          nbytes, handle)
        assert st == dit.DIT_ATTN_OK, dit.dit_attn_strerror(st)
        torch.cuda.synchronize()
        outs.append((o, lse))
    return outs


@pytest.mark.parametrize("shapes", [[(1, 24, 16896), (1, 3, 4608)], [(1, 6, 16896), (2, 3, 1000)]])
def test_noalloc_matches_the_workspace_entry_point_on_consecutive_calls(shapes):
    """Two calls in a row, the second smaller (stale scratch contents from the
    first must not leak into it): bit for bit the workspace form's result, and
    sampled rows within the bf16 bound of the oracle."""
    dit = _dit()
    for i, (B, H, N) in enumerate(shapes):
        d = 128
        q, k, v = random_qkv(B, H, N, d, seed=2000 + 10 * i + H)
        scale = 1 / math.sqrt(d)
        _, plan = dit.dit_attn_plan(B, H, N, d, dit.DIT_ATTN_BF16, 0, True, 0, dit.DIT_ATTN_NOALLOC_SCRATCH_BYTES)
        say(f"[gpu] noalloc call {i}: B={B} H={H} N={N}, schedule {plan.schedule}, scratch used "
            f"{plan.workspace_bytes} bytes")
        (o_na, l_na), (o_ws, l_ws) = _both(q.to(DEV), k.to(DEV), v.to(DEV), scale)
        assert torch.equal(o_na, o_ws) and torch.equal(l_na, l_ws), (B, H, N)
        rows = sample_rows(N, seed=i, n_edge=128, stride=32)
        o = o_na.float().cpu().double().numpy()[:, :, rows]
        l = l_na.cpu().double().numpy()[:, :, rows]
        check_full(o, l, q, k, scale, oracle_ref(q, k, v, scale, rows=rows),
                   f"noalloc B={B} H={H} N={N}", rows=rows)


def test_noalloc_fp8_then_smaller_bf16():
    dit = _dit()
    q, k, v = random_qkv(1, 24, 16896, 128, seed=2100)
    quant = [dit.quantize_e4m3(t.to(DEV)) for t in (q, k, v)]
    descale = torch.cat([s for _, s in quant]).contiguous()
    say("[gpu] noalloc fp8 B=1 H=24 N=16896 with lse")
    (o_na, l_na), (o_ws, l_ws) = _both(*(c for c, _ in quant), 1 / math.sqrt(128), dit.DIT_ATTN_FP8_E4M3, descale)
    assert torch.equal(o_na, o_ws) and torch.equal(l_na, l_ws)
    q, k, v = random_qkv(1, 2, 3000, 128, seed=2101)
    say("[gpu] noalloc bf16 B=1 H=2 N=3000 after it")
    (o_na, l_na), (o_ws, l_ws) = _both(q.to(DEV), k.to(DEV), v.to(DEV), 1 / math.sqrt(128))
    assert torch.equal(o_na, o_ws) and torch.equal(l_na, l_ws)
    check_full(o_na.float().cpu().double().numpy(), l_na.cpu().double().numpy(), q, k, 1 / math.sqrt(128),
               oracle_ref(q, k, v, 1 / math.sqrt(128)), "noalloc B=1 H=2 N=3000")


def test_noalloc_one_growing_row_reruns_like_the_workspace_form():
    """One row whose logits outgrow the unchecked first pass (row 700, not a
    lane-0 row): the workgroup's checked rerun under the static scratch, at
    a stream-K shape and then a smaller split shape, bit for bit the
    workspace form's result and every row within the bound of the oracle."""
    for B, H, N in [(1, 3, 4096), (1, 2, 1000)]:
        d = 128
        q, k, v = one_growing_row(B, H, N, d)
        scale = 1 / math.sqrt(d)
        say(f"[gpu] noalloc one growing row: B={B} H={H} N={N}")
        (o_na, l_na), (o_ws, l_ws) = _both(q.to(DEV), k.to(DEV), v.to(DEV), scale)
        assert torch.equal(o_na, o_ws) and torch.equal(l_na, l_ws), (B, H, N)
        check_full(o_na.float().cpu().double().numpy(), l_na.cpu().double().numpy(), q, k, scale,
                   oracle_ref(q, k, v, scale), f"noalloc one growing row B={B} H={H} N={N}")


def test_noalloc_rejects_bad_arguments_before_launch():
    dit = _dit()
    x = torch.zeros((1, 1, 64, 96), dtype=torch.bfloat16, device=DEV)
    o = torch.empty_like(x)
    handle = torch.cuda.current_stream().cuda_stream
    assert dit.dit_attn_fwd_noalloc(x, x, x, o, 1, 1, 64, 96, 0.1, dit.DIT_ATTN_BF16, None, None, None, None,
                                    handle) == dit.DIT_ATTN_EUNSUPPORTED
    assert dit.dit_attn_fwd_noalloc(x, x, x, x, 1, 1, 64, 64, 0.1, dit.DIT_ATTN_BF16, None, None, None, None,
                                    handle) == dit.DIT_ATTN_EINVAL
