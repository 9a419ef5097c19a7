"""GPU tests of the boundary itself: calls without a workspace (the short entry
points) against the oracle and against the workspace form, an undersized
workspace refused before any launch, HIP-graph capture of a whole call
replayed bit for bit, and the binding refusing host or mis-shaped buffers
before any launch."""
import math

import numpy as np
import pytest
import torch

import oracle
from parity import check_bf16, check_lse, logit_scale, oracle_ref, say
from workloads import WORKLOADS, make_qkv, random_qkv, sample_rows

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _dit():
    import diffusion_transformer_attention_non_amd as dit
    return dit


def _workspace(dit, B, H, N, d, dtype, lse=False):
    nbytes = dit.workspace_bytes(B, H, N, d, dtype, lse=lse)
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=DEV), nbytes


def _call(dit, q, k, v, o, scale, dtype=None, descale=None, lse=None, ws=None, ws_bytes=0, stream=None):
    B, H, N, d = q.shape
    dtype = dit.DIT_ATTN_BF16 if dtype is None else dtype
    s = torch.cuda.current_stream() if stream is None else stream
    st = dit.dit_attn_fwd_strided(q, k, v, o, B, H, N, d, scale, dtype, None, None, descale, lse, ws, ws_bytes,
                                  s.cuda_stream)
    assert st == dit.DIT_ATTN_OK, dit.dit_attn_strerror(st)


@pytest.mark.parametrize("name", ["t2i_2048", "t2i_2048_h3"])
def test_short_form_without_workspace(name):
    """dit_attn_fwd runs one workgroup per query tile (no workspace): sampled
    rows against the oracle, and the workspace form's result within the
    bf16 bound of it (the two differ only in how a tile's keys are summed)."""
    dit = _dit()
    w = WORKLOADS[name]
    q, k, v = make_qkv(w)
    scale = 1 / math.sqrt(w.d)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    B, H, N, d = q.shape
    o_short = torch.empty_like(qd)
    say(f"[gpu] dit_attn_fwd (no workspace) {name}")
    st = dit.dit_attn_fwd(qd, kd, vd, o_short, B, H, N, d, scale, dit.DIT_ATTN_BF16,
                          torch.cuda.current_stream().cuda_stream)
    assert st == dit.DIT_ATTN_OK
    ws, nbytes = _workspace(dit, B, H, N, d, dit.DIT_ATTN_BF16)
    assert nbytes > 0
    o_ws = torch.empty_like(qd)
    _call(dit, qd, kd, vd, o_ws, scale, ws=ws, ws_bytes=nbytes)
    torch.cuda.synchronize()
    rows = sample_rows(N, seed=7, n_edge=128, stride=64)
    o_ref, _, a_ref, m2_ref = oracle_ref(q, k, v, scale, rows=rows)
    kw = dict(n_keys=N, m2_ref=m2_ref, logit_mag=logit_scale(q, k, scale, rows))
    a = o_short.float().cpu().double().numpy()
    b = o_ws.float().cpu().double().numpy()
    check_bf16(a[:, :, rows], o_ref, a_ref, f"{name} no workspace", **kw)
    check_bf16(b[:, :, rows], o_ref, a_ref, f"{name} workspace", **kw)


def test_undersized_workspace_is_refused_and_nothing_runs():
    dit = _dit()
    q, k, v = random_qkv(1, 24, 4608, 128, seed=61)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    B, H, N, d = q.shape
    need = dit.workspace_bytes(B, H, N, d)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    o = torch.full_like(qd, float("nan"))
    st = dit.dit_attn_fwd_strided(qd, kd, vd, o, B, H, N, d, 0.1, dit.DIT_ATTN_BF16, None, None, None, None, ws,
                                  need - 16, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == dit.DIT_ATTN_EWORKSPACE
    assert torch.isnan(o).all()
    with pytest.raises(dit.DitAttnError) as e:
        dit.attention(qd, kd, vd, workspace=ws[:need - 16])
    assert e.value.status == dit.DIT_ATTN_EWORKSPACE


@pytest.mark.parametrize("B,H,N,kind", [(1, 24, 16896, "bf16 split"), (1, 3, 16896, "bf16 stream-K"),
                                        (1, 24, 16896, "fp8 split + lse"), (2, 3, 1000, "bf16 tile + lse")])
def test_graph_capture_replays_bit_for_bit(B, H, N, kind):
    """A whole call (attention kernel and merge) captured in a HIP graph with
    its workspace: every replay, with other work and synchronisations between
    replays, returns the eager call's bytes."""
    dit = _dit()
    d = 128
    q, k, v = random_qkv(B, H, N, d, seed=70 + H)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    scale = 1 / math.sqrt(d)
    want_lse = "lse" in kind
    descale = None
    dtype = dit.DIT_ATTN_BF16
    if kind.startswith("fp8"):
        quant = [dit.quantize_e4m3(t) for t in (qd, kd, vd)]
        qd, kd, vd = (c for c, _ in quant)
        descale = torch.cat([s for _, s in quant]).contiguous()
        dtype = dit.DIT_ATTN_FP8_E4M3
    ws, nbytes = _workspace(dit, B, H, N, d, dtype, lse=want_lse)
    _, plan = dit.dit_attn_plan(B, H, N, d, dtype, 0, want_lse, 0, nbytes)
    say(f"[gpu] graph capture {kind} B={B} H={H} N={N}: schedule {plan.schedule}")
    o_eager = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=DEV)
    l_eager = torch.empty((B, H, N), dtype=torch.float32, device=DEV) if want_lse else None
    _call(dit, qd, kd, vd, o_eager, scale, dtype, descale, l_eager, ws, nbytes)
    torch.cuda.synchronize()

    o_g = torch.full_like(o_eager, float("nan"))
    l_g = torch.full_like(l_eager, float("nan")) if want_lse else None
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                 # warm the capture stream once
        _call(dit, qd, kd, vd, o_g, scale, dtype, descale, l_g, ws, nbytes, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _call(dit, qd, kd, vd, o_g, scale, dtype, descale, l_g, ws, nbytes)
    other = torch.empty_like(o_eager)
    for rep in range(4):
        o_g.fill_(float("nan"))
        if want_lse:
            l_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_eager), rep
        if want_lse:
            assert torch.equal(l_g, l_eager), rep
        # eager work between replays, on the same workspace
        _call(dit, qd, kd, vd, other, scale * 0.5, dtype, descale, None, ws, nbytes)
        torch.cuda.synchronize()


def test_binding_refuses_bad_buffers_before_any_launch():
    dit = _dit()
    q = torch.zeros((1, 2, 64, 128), dtype=torch.bfloat16, device=DEV)
    cases = [
        dict(lse=torch.empty((1, 2, 64), dtype=torch.float32)),                       # host lse
        dict(lse=torch.empty((1, 2, 64), dtype=torch.float16, device=DEV)),           # wrong dtype
        dict(lse=torch.empty((1, 2, 63), dtype=torch.float32, device=DEV)),           # wrong shape
        dict(lse=torch.empty((1, 64, 2), dtype=torch.float32, device=DEV).transpose(1, 2)),   # not contiguous
        dict(out=torch.empty((1, 2, 64, 128), dtype=torch.bfloat16)),                 # host out
        dict(out=torch.empty((1, 2, 64, 128), dtype=torch.float32, device=DEV)),      # wrong dtype
        dict(workspace=torch.empty(1 << 20, dtype=torch.uint8)),                      # host workspace
        dict(workspace=torch.empty(1 << 18, dtype=torch.float32, device=DEV)),        # not bytes
    ]
    for kw in cases:
        with pytest.raises(ValueError):
            dit.attention(q, q, q, **kw)
    q8 = torch.zeros((1, 2, 64, 128), dtype=torch.float8_e4m3fn, device=DEV)
    with pytest.raises(ValueError):
        dit.attention(q8, q8, q8, descale=torch.ones(3))                                # host descale
    with pytest.raises(ValueError):
        dit.quantize_e4m3(q, out=torch.empty((1, 2, 64, 128), dtype=torch.uint8, device=DEV))
    with pytest.raises(ValueError):
        dit.quantize_e4m3(q, descale=torch.empty(1, dtype=torch.float32))
    with pytest.raises(ValueError):
        dit.quantize_e4m3(q, workspace=torch.empty(1, dtype=torch.int32))
    with pytest.raises(ValueError):
        dit.quantize_mx(q, "d", scales=torch.empty((1, 2, 64, 3), dtype=torch.uint8, device=DEV))
    with pytest.raises(ValueError):
        dit.quantize_mx(q, "tokens", out=torch.empty((1, 2, 64, 128), dtype=torch.float8_e4m3fn))
    codes, sc = dit.quantize_mx(q, "d")
    vcodes, vsc = dit.quantize_mx(q, "tokens")
    with pytest.raises(ValueError):
        dit.attention_mx(codes, sc, codes, sc, vcodes, vsc, lse=torch.empty((1, 2, 64), dtype=torch.float32))
    counts = torch.ones((1, 2, 1), dtype=torch.int32, device=DEV)
    blocks = torch.zeros((1, 2, 1, 1), dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        dit.attention_blocksparse(q, q, q, blocks, counts, lse=torch.empty((1, 2, 64), dtype=torch.float32))
    with pytest.raises(ValueError):
        dit.attention_blocksparse(q, q, q, blocks.cpu(), counts)
    torch.cuda.synchronize()
