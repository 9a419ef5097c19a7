"""GPU parity of the stream-K schedule (bf16, d = 128), which the library picks
when the query tiles leave the last round of workgroups badly filled and a
key-range split of that round cannot fix it, e.g. one GPU's share of the
16896-token call (H = 3 or 6), or (B, H, N) = (1, 4, 12800) and (1, 2, 16896).
Every workgroup then takes an equal contiguous range of (query tile, key
tile) pairs; tiles cut by range boundaries are merged through their
log-sum-exps. Checked against the oracle (sampled rows, LSE), exact
structure (every 64-key block counted once), strided rows (bitwise equal to
packed), and run-to-run determinism."""
import math

import numpy as np
import pytest
import torch

import oracle
from parity import check_bf16, check_full, gpu_attention, oracle_ref, say
from workloads import coverage_pattern, random_qkv, sample_rows

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("B,H,N", [(1, 4, 12800), (1, 1, 16896), (1, 5, 16896), (1, 3, 16896)])
def test_streamk_every_row(B, H, N):
    q, k, v = random_qkv(B, H, N, 128, seed=900 + H)
    say(f"[gpu] stream-K B={B} H={H} N={N}, every row")
    o, l = gpu_attention(q, k, v, 1 / math.sqrt(128), want_lse=True)
    check_full(o, l, q, k, 1 / math.sqrt(128), oracle_ref(q, k, v, 1 / math.sqrt(128)),
               f"stream-K H={H} N={N}")


@pytest.mark.parametrize("H,N", [(3, 16896), (4, 12800), (1, 16896)])
def test_streamk_tile_coverage_exact(H, N):
    """All logits equal, V one-hot by 64-key block: each channel is the exact
    fraction of keys in its blocks; a key block lost or counted twice at a
    range boundary moves a channel by 64/N."""
    q, k, v = coverage_pattern(1, H, N, 128, block=64)
    say(f"[gpu] stream-K coverage H={H} N={N}")
    o, l = gpu_attention(q, k, v, 1 / math.sqrt(128), want_lse=True)
    j = np.arange(N)
    counts = np.bincount((j // 64) % 128, minlength=128).astype(np.float64)
    exact = np.broadcast_to(counts / N, o.shape)
    assert (np.abs(o - exact) <= 2.0**-8 * exact).all(), np.abs(o - exact).max()
    # equal logits (0): lse = log N
    assert np.abs(l - math.log(N)).max() <= 1e-5 * math.log(N) + 2e-6


def test_streamk_strided_rows_bitwise_and_deterministic():
    import diffusion_transformer_attention_non_amd as dit
    B, H, N, d = 1, 3, 16896, 128
    q, k, v = random_qkv(B, H, N, d, seed=950)
    say(f"[gpu] stream-K strided rows H={H} N={N}")
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    l1 = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    o1 = dit.attention(qd, kd, vd, 1 / math.sqrt(d), lse=l1)
    l2 = torch.empty_like(l1)
    o2 = dit.attention(qd, kd, vd, 1 / math.sqrt(d), lse=l2)
    views = [t.permute(0, 2, 1, 3).contiguous().to(DEV).permute(0, 2, 1, 3) for t in (q, k, v)]
    out = torch.full((B, N, H, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    l3 = torch.empty_like(l1)
    o3 = dit.attention(*views, 1 / math.sqrt(d), out=out.permute(0, 2, 1, 3), lse=l3)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o3, o1) and torch.equal(l3, l1)
    assert not torch.isnan(out).any()


def test_plan_for_the_current_device():
    import diffusion_transformer_attention_non_amd as dit
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    st, p = dit.dit_attn_plan(1, 3, 16896, 128, dit.DIT_ATTN_BF16, 0, 0, 0, 1 << 40)
    assert st == dit.DIT_ATTN_OK
    st2, p2 = dit.dit_attn_plan(1, 3, 16896, 128, dit.DIT_ATTN_BF16, 0, 0, n_cu, 1 << 40)
    assert st2 == dit.DIT_ATTN_OK
    assert (p.schedule, p.workgroups, p.workspace_bytes) == (p2.schedule, p2.workgroups, p2.workspace_bytes)
    say(f"[gpu] plan H=3 N=16896 on {n_cu} CUs: schedule {p.schedule}, {p.workgroups} workgroups")
