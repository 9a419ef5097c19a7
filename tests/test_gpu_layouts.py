"""GPU tests of strided layouts (dit_attn_fwd_strided): rows of q, k, v and o
taken from [B][N][H][d] buffers and from a fused [B][N][3][H][d] QKV buffer.
The kernels only change how they address rows, so every result must equal,
bit for bit, the same attention on contiguous copies; one case per kernel is
also held to the oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
from parity import check_full, oracle_ref, say
from workloads import WORKLOADS, make_qkv, random_qkv

pytestmark = pytest.mark.gpu


def _dit():
    import diffusion_transformer_attention_non_amd as dit
    return dit


def _bnhd_views(t, dev):
    """t: (B, H, N, d) CPU tensor -> a (B, H, N, d) view of a contiguous
    (B, N, H, d) device buffer holding the same values."""
    return t.permute(0, 2, 1, 3).contiguous().to(dev).permute(0, 2, 1, 3)


def _fused_views(q, k, v, dev):
    """One contiguous (B, N, 3, H, d) buffer; q, k, v are strided views of it."""
    buf = torch.stack([t.permute(0, 2, 1, 3) for t in (q, k, v)], dim=2).contiguous().to(dev)
    return [buf[:, :, i].permute(0, 2, 1, 3) for i in range(3)]


def _run(q, k, v, scale, out=None, lse=True, descale=None):
    dit = _dit()
    B, H, N, d = q.shape
    l = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse else None
    o = dit.attention(q, k, v, scale, out=out, lse=l, descale=descale)
    torch.cuda.synchronize()
    return o, l


@pytest.mark.parametrize("d,N", [(128, 1000), (128, 300), (64, 1000), (64, 65)])
def test_bnhd_inputs_and_output_bitwise(d, N):
    dev = torch.device("cuda:0")
    q, k, v = random_qkv(2, 3, N, d, seed=40 + d + N)
    scale = 1 / math.sqrt(d)
    say(f"[gpu] layouts bf16 B=2 H=3 N={N} d={d}")
    o_ref, l_ref = _run(q.to(dev), k.to(dev), v.to(dev), scale)
    qs, ks, vs = (_bnhd_views(t, dev) for t in (q, k, v))
    assert qs.stride() == (N * 3 * d, d, 3 * d, 1)
    out_buf = torch.full((2, N, 3, d), float("nan"), dtype=torch.bfloat16, device=dev)
    o, l = _run(qs, ks, vs, scale, out=out_buf.permute(0, 2, 1, 3))
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)
    assert not torch.isnan(out_buf).any()          # every output row written
    qf, kf, vf = _fused_views(q, k, v, dev)
    assert qf.stride()[2] == 3 * 3 * d
    o2, l2 = _run(qf, kf, vf, scale)
    assert torch.equal(o2, o_ref) and torch.equal(l2, l_ref)


def test_fused_qkv_against_oracle():
    dev = torch.device("cuda:0")
    q, k, v = random_qkv(1, 4, 777, 128, seed=47)
    scale = 1 / math.sqrt(128)
    qf, kf, vf = _fused_views(q, k, v, dev)
    o, l = _run(qf, kf, vf, scale)
    check_full(o.float().cpu().double().numpy(), l.cpu().double().numpy(), q, k, scale,
               oracle_ref(q, k, v, scale), "fused QKV (B=1 H=4 N=777)")


def test_fp8_bnhd_bitwise():
    dev = torch.device("cuda:0")
    dit = _dit()
    q, k, v = random_qkv(1, 3, 1000, 128, seed=48)
    codes, desc = [], []
    for t in (q, k, v):
        c, dsc = dit.quantize_e4m3(t.permute(0, 2, 1, 3).contiguous().to(dev))   # (B, N, H, d) codes
        codes.append(c)
        desc.append(dsc)
    descale = torch.cat(desc).contiguous()
    strided = [c.permute(0, 2, 1, 3) for c in codes]
    packed = [c.permute(0, 2, 1, 3).contiguous() for c in codes]
    for lse in (False, True):
        o1, l1 = _run(*packed, 1 / math.sqrt(128), lse=lse, descale=descale)
        o2, l2 = _run(*strided, 1 / math.sqrt(128), lse=lse, descale=descale)
        assert torch.equal(o1, o2)
        if lse:
            assert torch.equal(l1, l2)


def test_bnhd_full_workload_bitwise():
    """The 16896-token workload in [B][N][H][d]: same launch configuration as
    the benchmark (tail split included), bitwise equal to the packed layout."""
    dev = torch.device("cuda:0")
    w = WORKLOADS["t2i_2048"]
    q, k, v = make_qkv(w)
    scale = 1 / math.sqrt(w.d)
    say("[gpu] layouts t2i_2048 [B][N][H][d]")
    o_ref, _ = _run(q.to(dev), k.to(dev), v.to(dev), scale, lse=False)
    o, _ = _run(*(_bnhd_views(t, dev) for t in (q, k, v)), scale, lse=False)
    assert torch.equal(o, o_ref)


def test_strided_rejects_mismatched_views():
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in random_qkv(1, 2, 64, 64, seed=49))
    with pytest.raises(ValueError):
        _dit().attention(q.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3), k, v)   # q strides differ
