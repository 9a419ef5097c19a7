"""GPU parity of the bf16 path against the fp64 oracle, through the C ABI."""
import math

import numpy as np
import pytest
import torch

import oracle
from parity import check_bf16, check_full, gpu_attention, logit_scale, oracle_ref, oracle_workload, say
from workloads import (WORKLOADS, coverage_pattern, constant_values, dominating_key, identical_keys,
                       make_qkv, one_growing_row, random_qkv)

pytestmark = pytest.mark.gpu


def _full_check(q, k, v, scale, label, lse=True, workspace=None):
    say(f"[gpu] {label}: shape {tuple(q.shape)}")
    o, l = gpu_attention(q, k, v, scale, want_lse=lse, workspace=workspace)
    check_full(o, l, q, k, scale, oracle_ref(q, k, v, scale), label)
    return o


def test_tiny_workload_full():
    w = WORKLOADS["tiny"]
    q, k, v = make_qkv(w)
    _full_check(q, k, v, 1 / math.sqrt(w.d), "tiny B=1 H=2 N=256 d=64")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 2, 31, 63, 64, 65, 127, 129, 300, 1000])
def test_odd_lengths(N, d):
    q, k, v = random_qkv(1, 2, N, d, seed=N + d)
    _full_check(q, k, v, 1 / math.sqrt(d), f"N={N} d={d}")


def test_batch_heads_and_peaked_small():
    q, k, v = random_qkv(2, 3, 777, 128, seed=5)
    _full_check(q * 4, k, v, 1 / math.sqrt(128), "B=2 H=3 N=777 peaked")


@pytest.mark.timeout(900)
# t2i_2048 last: its oracle result stays cached for the fp8 spec gate on the same tensors
@pytest.mark.parametrize("name", ["t2i_1024", "t2i_2048_peaked", "i2i_2048", "t2i_2048_h6", "t2i_2048_h3",
                                  "t2i_2048"])
def test_workload_every_row(name):
    """Every element of every workload at its full size, in the launch
    configuration the benchmark times (the binding passes the workspace the
    fastest schedule needs): split last round at 24 heads, stream-K at 3 and
    6 heads, against the fp64 oracle on the same inputs."""
    w = WORKLOADS[name]
    q, k, v = make_qkv(w)
    scale = 1 / math.sqrt(w.d)
    say(f"[gpu] {name}: B={w.B} H={w.H} N={w.N} d={w.d}, every row")
    o, l = gpu_attention(q, k, v, scale, want_lse=True)
    check_full(o, l, q, k, scale, oracle_workload(name), f"{name} (all {w.N} rows/head)")


# ------------------------------------------------------------ exact structure
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [300, 4608, 16896])
def test_tile_coverage_exact(N, d):
    """All logits equal and V one-hot by 64-key block: O[c] = (#tokens j with
    (j // 64) % d == c) / N, exact in fp32 then one bf16 rounding. A dropped or
    repeated key block moves some channel by 64/N."""
    q, k, v = coverage_pattern(1, 2, N, d, block=64)
    say(f"[gpu] coverage N={N} d={d}")
    o, _ = gpu_attention(q, k, v, 1 / math.sqrt(d))
    j = np.arange(N)
    counts = np.bincount((j // 64) % d, minlength=d).astype(np.float64)
    exact = np.broadcast_to(counts / N, o.shape)
    # one bf16 rounding (half an ulp) plus fp32 noise; a dropped block moves a channel by ~50%
    assert (np.abs(o - exact) <= 2.0**-8 * exact).all(), np.abs(o - exact).max()


@pytest.mark.parametrize("d", [64, 128])
def test_dominating_key_every_position(d):
    N = 300
    for j_star in range(N):
        q, k, v = dominating_key(1, 1, N, d, j_star, seed=j_star)
        o, _ = gpu_attention(q, k, v, 1 / math.sqrt(d))
        ref = v[:, :, j_star:j_star + 1].double().numpy()
        assert np.array_equal(o, np.broadcast_to(ref, o.shape)), j_star


def test_dominating_key_tile_edges_long():
    N, d = 16896, 128
    for j_star in [0, 1, 31, 32, 63, 64, 127, 128, 8191, 8192, N - 65, N - 64, N - 1]:
        say(f"[gpu] dominating key N={N} j*={j_star}")
        q, k, v = dominating_key(1, 1, N, d, j_star, seed=j_star)
        o, _ = gpu_attention(q, k, v, 1 / math.sqrt(d))
        ref = v[:, :, j_star:j_star + 1].double().numpy()
        assert np.array_equal(o, np.broadcast_to(ref, o.shape)), j_star


@pytest.mark.parametrize("d", [64, 128])
def test_constant_values_and_identical_keys(d):
    q, k, v = constant_values(1, 2, 1000, d, seed=1, c=0.75)
    o, _ = gpu_attention(q, k, v, 1 / math.sqrt(d))
    # rows of p sum to one: only the bf16 rounding of p (<= 2^-8 relative) separates O from c
    assert np.abs(o - 0.75).max() <= 2.0**-8 * 0.75
    q, k, v = identical_keys(1, 2, 1000, d, seed=2)
    o, _ = gpu_attention(q, k, v, 1 / math.sqrt(d))
    mean = oracle.bf16_round(v.double().numpy().mean(axis=2, keepdims=True))
    assert np.abs(o - mean).max() <= 2.0**-8 * np.abs(mean).max() + 1e-6


def test_single_token_is_exact():
    q, k, v = random_qkv(2, 3, 1, 128, seed=9)
    o, _ = gpu_attention(q, k, v, 0.1)
    assert np.array_equal(o, v.double().numpy())


def test_joint_key_value_permutation_and_query_permutation():
    q, k, v = random_qkv(1, 2, 2000, 128, seed=11)
    scale = 1 / math.sqrt(128)
    g = torch.Generator().manual_seed(3)
    pk = torch.randperm(2000, generator=g)
    pq = torch.randperm(2000, generator=g)
    o, _ = gpu_attention(q, k, v, scale)
    o_k, _ = gpu_attention(q, k[:, :, pk].contiguous(), v[:, :, pk].contiguous(), scale)
    o_q, _ = gpu_attention(q[:, :, pq].contiguous(), k, v, scale)
    o_ref, _, a_ref, m2_ref = oracle_ref(q, k, v, scale)
    lm = logit_scale(q, k, scale)
    check_bf16(o_k, o_ref, a_ref, "K/V permuted", n_keys=2000, m2_ref=m2_ref, logit_mag=lm)
    pi = pq.numpy()
    check_bf16(o_q, o_ref[:, :, pi], a_ref[:, :, pi], "Q permuted", n_keys=2000, m2_ref=m2_ref[:, :, pi],
               logit_mag=lm[:, :, pi])
    assert np.abs(o_k - o).max() <= 2 * (2.0**-8) * (np.abs(o_ref).max() + a_ref.max())


def test_deterministic_and_heads_independent():
    """Bitwise run-to-run determinism. A head computed alone matches the same
    head inside a batch: bitwise here (both shapes take the same key split), and
    in general within the rounding of a different key-range split."""
    q, k, v = random_qkv(2, 3, 1500, 128, seed=12)
    scale = 1 / math.sqrt(128)
    o1, l1 = gpu_attention(q, k, v, scale, want_lse=True)
    o2, l2 = gpu_attention(q, k, v, scale, want_lse=True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    o_one, _ = gpu_attention(q[1:2, 2:3].contiguous(), k[1:2, 2:3].contiguous(), v[1:2, 2:3].contiguous(), scale)
    assert np.array_equal(o_one[0, 0], o1[1, 2])
    # a different batch shape: other key ranges, same values to within rounding
    o_pair, _ = gpu_attention(q[1:2].contiguous(), k[1:2].contiguous(), v[1:2].contiguous(), scale)
    o_ref, _, a_ref, m2_ref = oracle_ref(q[1:2], k[1:2], v[1:2], scale)
    check_bf16(o_pair, o_ref, a_ref, "B=1 H=3 slice", n_keys=1500, m2_ref=m2_ref,
               logit_mag=logit_scale(q[1:2], k[1:2], scale))
    assert (np.abs(o_pair - o1[1:2]) <= 2 * (2.0**-8) * (np.abs(o_ref) + a_ref) + 1e-6).all()


def test_unsupported_head_dim_on_device():
    import diffusion_transformer_attention_non_amd as dit
    x = torch.zeros((1, 1, 64, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dit.DitAttnError) as e:
        dit.attention(x, x, x)
    assert e.value.status == dit.DIT_ATTN_EUNSUPPORTED


def _ramp_qkv(N, d, slope, seed):
    """Logits that grow along the keys: q = e_0, k_j = slope * j * e_0 (plus
    small noise in the other coordinates), V random. The running maximum taken
    from the first keys goes stale by slope * scale * N nats over the row."""
    g = torch.Generator().manual_seed(seed)
    q = torch.zeros((1, 2, N, d))
    q[..., 0] = 1.0
    k = 0.01 * torch.randn((1, 2, N, d), generator=g)
    k[..., 0] = slope * torch.arange(N, dtype=torch.float32)
    v = torch.randn((1, 2, N, d), generator=g)
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


@pytest.mark.parametrize("slope,label", [(17.5, "rare path every sub-tile"), (0.4, "large P, no rare path")])
def test_growing_logits(slope, label):
    """17.5: each 32-key sub-tile raises the maximum by more than 64 bits, so
    every sub-tile takes the recompute path. 0.4: the maximum grows by about
    50 bits over the row, below the 2^64 guard, so probabilities relative to
    the first sub-tile's maximum reach about 2^50 and are used as they are."""
    q, k, v = _ramp_qkv(1000, 128, slope, seed=31)
    _full_check(q, k, v, 1 / math.sqrt(128), f"ramp slope {slope} ({label})")


@pytest.mark.parametrize("schedule,H,N,q_700,lse", [("split", 2, 1000, 100.0, True), ("split", 2, 1000, 100.0, False),
                                                     ("tile", 2, 1000, 45.0, True), ("tile", 2, 1000, 100.0, False),
                                                     ("streamk", 3, 4096, 100.0, True)])
def test_one_row_overflow_reruns_its_workgroup(schedule, H, N, q_700, lse):
    """One query row (row 700: lane 12 of the third wave of the third 256-row
    tile, a row that lane 0 does not hold) has logits that grow by 0.0044 q_700
    nats per key; the other rows grow about 50 times more slowly. The unchecked
    first pass of a range of keys in which that row's growth passes 64 bits
    overflows (a p past 2^128 also makes the row sums of its 16-row group
    NaN), and only in that wave, so the whole workgroup must run the range
    again checked. The split schedule of B=1 H=2 N=1000 gives a workgroup 4 key
    tiles (about 163 bits of growth at q_700 = 100); without workspace a
    workgroup takes all 1000 keys (287 bits at q_700 = 45); stream-K at B=1
    H=3 N=4096 gives each workgroup 12 key tiles, cut across tile boundaries,
    so a workgroup may run two ranges back to back. Every row must match the
    oracle."""
    import diffusion_transformer_attention_non_amd as dit
    d = 128
    want = {"tile": dit.DIT_ATTN_SCHED_TILE, "split": dit.DIT_ATTN_SCHED_SPLIT,
            "streamk": dit.DIT_ATTN_SCHED_STREAMK}[schedule]
    ws_bytes = dit.workspace_bytes(1, H, N, d, lse=lse) if schedule != "tile" else 0
    st, plan = dit.dit_attn_plan(1, H, N, d, dit.DIT_ATTN_BF16, 0, lse, 0, ws_bytes)
    assert st == 0 and plan.schedule == want, (plan.schedule, want)
    q, k, v = one_growing_row(1, H, N, d, q_row=q_700)
    _full_check(q, k, v, 1 / math.sqrt(d), f"one overflowing row (row 700, q {q_700}, {schedule}, H={H} N={N})",
                lse=lse, workspace=ws_bytes if schedule != "tile" else 0)


def test_one_row_overflow_d64():
    """The d = 64 kernel with one row whose logits grow about 0.64 bits per
    key (row 700, not a lane-0 row) while the others stay near the first
    sub-tile's maximum."""
    N, d = 1000, 64
    q, k, v = one_growing_row(1, 2, N, d, q_row=100.0 * math.sqrt(64 / 128))
    _full_check(q, k, v, 1 / math.sqrt(d), "d=64 one overflowing row (row 700)")
