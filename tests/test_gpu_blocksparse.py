"""GPU parity of block-sparse attention (dit_attn_fwd_blocksparse, bf16, d = 128)
against the fp64 block-sparse oracle on the same seeded inputs and lists.

Cases: lists with the text blocks plus a random fraction of the rest, the
ragged last key block, empty lists, counts above max_blocks and below 0,
every block listed (which must equal the dense kernel bit for bit where the
dense call takes the same schedule), [B][N][H][d] rows, and the full 2048x2048-equivalent
shape on sampled rows."""
import math

import numpy as np
import pytest
import torch

import oracle
from parity import check_bf16, lse_tolerance, logit_scale, say
from workloads import make_qkv, one_growing_row, random_kv_blocks, random_qkv, sample_rows

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _dit():
    import diffusion_transformer_attention_non_amd as dit
    return dit


def _sparse(q, k, v, blocks, counts, scale, lse=True):
    """q, k, v device tensors; blocks, counts CPU int32 tensors."""
    dit = _dit()
    B, H, N, d = q.shape
    l = torch.empty((B, H, N), dtype=torch.float32, device=DEV) if lse else None
    o = dit.attention_blocksparse(q, k, v, blocks.to(DEV), counts.to(DEV), scale, lse=l)
    torch.cuda.synchronize()
    return o, l


def _check_lse(l_gpu, l_ref, tol, label):
    """As for dense rows; rows of empty lists must be -inf on both sides."""
    empty = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(l_gpu), empty), label
    err = np.abs(l_gpu[~empty] - l_ref[~empty])
    say(f"  {label} lse: max {float(err.max()) if err.size else 0.0:.3e}")
    assert (err <= tol[~empty]).all(), label


def _compare(q, k, v, blocks, counts, scale, label, rows=None):
    o, l = _sparse(q.to(DEV), k.to(DEV), v.to(DEV), blocks, counts, scale)
    o_ref, l_ref, a_ref = oracle.attention_blocksparse(q, k, v, scale, blocks, counts, rows=rows, want_abs=True)
    og = o.float().cpu().double().numpy()
    lg = l.cpu().double().numpy()
    if rows is not None:
        og, lg = og[:, :, rows], lg[:, :, rows]
    empty = np.isneginf(l_ref)
    assert np.all(og[empty] == 0.0), label
    check_bf16(og, o_ref, a_ref, label, n_keys=q.shape[2], logit_mag=logit_scale(q, k, scale, rows))
    tol = lse_tolerance(q.shape[2], np.where(empty, 0.0, l_ref), logit_scale(q, k, scale, rows))
    _check_lse(lg, l_ref, tol, label)
    return o, l


@pytest.mark.parametrize("B,H,N,density,empty_every,seed", [
    (1, 2, 1000, 0.5, 3, 1),     # 4 query tiles, 16 key tiles, 40-key tail
    (2, 3, 300, 0.6, 4, 2),      # 2 query tiles, 5 key tiles, 44-key tail
    (1, 2, 65, 1.0, 0, 3),       # one query tile, a one-key tail block
    (1, 1, 64, 1.0, 0, 4),       # one full key tile
    (1, 4, 4608, 0.3, 7, 5),     # 1024x1024-equivalent length, long lists
    (1, 2, 2000, 0.05, 5, 6),    # very sparse: text blocks plus a few
])
def test_blocksparse_matches_oracle(B, H, N, density, empty_every, seed):
    d = 128
    q, k, v = random_qkv(B, H, N, d, seed=300 + seed)
    blocks, counts = random_kv_blocks(B, H, N, density, seed=seed, empty_every=empty_every)
    say(f"[gpu] blocksparse B={B} H={H} N={N} density={density} empty_every={empty_every} "
        f"max_blocks={blocks.shape[-1]}")
    _compare(q, k, v, blocks, counts, 1 / math.sqrt(d), f"sparse N={N}")


@pytest.mark.parametrize("density", [0.6, 1.0])
def test_blocksparse_one_row_overflow(density):
    """One row (row 700, lane 12 of its wave) whose logits grow far faster
    along the keys than the others': its unchecked first pass over a tile's
    listed key blocks overflows in one wave, and the workgroup must run the
    tile again checked."""
    d = 128
    q, k, v = one_growing_row(1, 2, 1000, d)
    blocks, counts = random_kv_blocks(1, 2, 1000, density, seed=7)
    say(f"[gpu] blocksparse one growing row, density {density}")
    _compare(q, k, v, blocks, counts, 1 / math.sqrt(d), f"sparse one growing row density={density}")


def test_blocksparse_hand_lists():
    """Lists without the text blocks, with only the tail block, and with one block each."""
    B, H, N, d = 1, 2, 777, 128
    q, k, v = random_qkv(B, H, N, d, seed=310)
    nq, nk = 4, 13
    blocks = torch.full((B, H, nq, 3), -1, dtype=torch.int32)
    counts = torch.zeros((B, H, nq), dtype=torch.int32)
    pats = [[12], [0, 12], [5], [3, 7, 12], [1, 2], [11], [0], [6, 9]]
    for i, p in enumerate(pats):
        h, t = divmod(i, nq)
        blocks[0, h, t, :len(p)] = torch.tensor(p, dtype=torch.int32)
        counts[0, h, t] = len(p)
    say(f"[gpu] blocksparse hand lists N={N}")
    _compare(q, k, v, blocks, counts, 1 / math.sqrt(d), "hand lists")


def test_blocksparse_count_clamps():
    """Counts above max_blocks read max_blocks entries; negative counts are empty lists."""
    B, H, N, d = 1, 2, 600, 128
    q, k, v = (t.to(DEV) for t in random_qkv(B, H, N, d, seed=320))
    # lists are valid rows of max_blocks ascending entries: a shuffled block
    # subset of length 6 out of 10, sorted
    rng = np.random.default_rng(21)
    nq, nk, mb = 3, 10, 6
    rows = [np.sort(rng.choice(nk, mb, replace=False)) for _ in range(B * H * nq)]
    blocks = torch.from_numpy(np.stack(rows).astype(np.int32).reshape(B, H, nq, mb))
    counts = torch.full((B, H, nq), mb, dtype=torch.int32)
    big = torch.full_like(counts, mb + 1000)
    say(f"[gpu] blocksparse count clamps N={N} max_blocks={mb}")
    o1, l1 = _sparse(q, k, v, blocks, counts, 0.09)
    o2, l2 = _sparse(q, k, v, blocks, big, 0.09)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    neg = counts.clone()
    neg[0, 1, 1] = -5
    zero = counts.clone()
    zero[0, 1, 1] = 0
    o3, l3 = _sparse(q, k, v, blocks, neg, 0.09)
    o4, l4 = _sparse(q, k, v, blocks, zero, 0.09)
    assert torch.equal(o3, o4) and torch.equal(l3, l4)
    assert torch.all(o3[0, 1, 256:512] == 0) and torch.all(torch.isneginf(l3[0, 1, 256:512]))


@pytest.mark.parametrize("B,H,N", [(2, 3, 448), (1, 2, 200), (1, 1, 100)])
def test_full_lists_equal_dense(B, H, N):
    """Every block listed: with the dense call on the same schedule (one
    workgroup per tile, or the same split; dit_attn_plan says which), the
    same tiles in the same order, so identical bytes. Where the dense call
    takes stream-K instead (small calls of few tiles), the sums run in
    another order: then within the bf16 bound of each other."""
    d = 128
    dit = _dit()
    q, k, v = (t.to(DEV) for t in random_qkv(B, H, N, d, seed=330 + N))
    nq, nk = -(-N // 256), -(-N // 64)
    blocks = torch.arange(nk, dtype=torch.int32).expand(B, H, nq, nk).contiguous()
    counts = torch.full((B, H, nq), nk, dtype=torch.int32)
    # attention() passes the workspace the fastest schedule needs
    _, dense_plan = dit.dit_attn_plan(B, H, N, d, dit.DIT_ATTN_BF16, 0, 1, 0, 1 << 40)
    _, sparse_plan = dit.dit_attn_plan(B, H, N, d, dit.DIT_ATTN_BF16, nk, 1, 0, 1 << 40)
    say(f"[gpu] blocksparse full lists vs dense B={B} H={H} N={N} (schedules {dense_plan.schedule}, "
        f"{sparse_plan.schedule})")
    o, l = _sparse(q, k, v, blocks, counts, 1 / math.sqrt(d))
    ld = torch.empty_like(l)
    od = dit.attention(q, k, v, 1 / math.sqrt(d), lse=ld)
    torch.cuda.synchronize()
    if (dense_plan.schedule, dense_plan.parts) == (sparse_plan.schedule, sparse_plan.parts):
        assert torch.equal(o, od) and torch.equal(l, ld)
    else:
        assert dense_plan.schedule == dit.DIT_ATTN_SCHED_STREAMK
        of, odf = o.float(), od.float()
        assert ((of - odf).abs() <= 2.0**-7 * (of.abs() + odf.abs()) + 1e-3).all()
        assert (l - ld).abs().max().item() <= 1e-5 * l.abs().max().item() + 1e-5


def test_full_lists_equal_dense_bitwise_with_split():
    """B 2, H 24, N 4608: 864 query tiles, so the last round is split into key
    ranges; with every block listed the sparse call splits the same way."""
    B, H, N, d = 2, 24, 4608, 128
    dit = _dit()
    q, k, v = (t.to(DEV) for t in random_qkv(B, H, N, d, seed=335))
    nq, nk = N // 256, N // 64
    blocks = torch.arange(nk, dtype=torch.int32).expand(B, H, nq, nk).contiguous()
    counts = torch.full((B, H, nq), nk, dtype=torch.int32)
    say(f"[gpu] blocksparse full lists vs dense (split) B={B} H={H} N={N}")
    o, l = _sparse(q, k, v, blocks, counts, 1 / math.sqrt(d))
    ld = torch.empty_like(l)
    od = dit.attention(q, k, v, 1 / math.sqrt(d), lse=ld)
    torch.cuda.synchronize()
    assert torch.equal(o, od) and torch.equal(l, ld)


def test_blocksparse_split_parts_with_short_lists():
    """H 3, N 4608: 54 query tiles, each split into key ranges (list
    positions). Lists of 0 to 8 blocks against max_blocks 72 leave many parts
    empty, and a tile with every part empty."""
    B, H, N, d = 1, 3, 4608, 128
    q, k, v = random_qkv(B, H, N, d, seed=350)
    nq, nk = N // 256, N // 64
    rng = np.random.default_rng(35)
    blocks = np.full((B, H, nq, nk), -1, dtype=np.int32)
    counts = np.zeros((B, H, nq), dtype=np.int32)
    for h in range(H):
        for t in range(nq):
            c = int(rng.integers(0, 9))
            blocks[0, h, t, :c] = np.sort(rng.choice(nk, c, replace=False))
            counts[0, h, t] = c
    counts[0, 0, 0] = 0
    say(f"[gpu] blocksparse split parts, short lists H={H} N={N}")
    _compare(q, k, v, torch.from_numpy(blocks), torch.from_numpy(counts), 1 / math.sqrt(d), "short lists")


def test_blocksparse_bnhd_rows_and_lse_optional():
    B, H, N, d = 2, 3, 700, 128
    q, k, v = random_qkv(B, H, N, d, seed=340)
    blocks, counts = random_kv_blocks(B, H, N, 0.5, seed=34, empty_every=4)
    say(f"[gpu] blocksparse [B][N][H][d] rows N={N}")
    o_ref, l_ref = _sparse(q.to(DEV), k.to(DEV), v.to(DEV), blocks, counts, 0.1)
    views = [t.permute(0, 2, 1, 3).contiguous().to(DEV).permute(0, 2, 1, 3) for t in (q, k, v)]
    out_buf = torch.full((B, N, H, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    dit = _dit()
    l = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    o = dit.attention_blocksparse(*views, blocks.to(DEV), counts.to(DEV), 0.1, out=out_buf.permute(0, 2, 1, 3),
                                  lse=l)
    o_nolse, _ = _sparse(q.to(DEV), k.to(DEV), v.to(DEV), blocks, counts, 0.1, lse=False)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref) and torch.equal(o_nolse, o_ref)
    assert not torch.isnan(out_buf).any()


def test_blocksparse_t2i_2048_sampled_rows():
    """The 2048x2048-equivalent shape (H 24, N 16896) with 30% of the image blocks
    plus the text blocks, every 9th list empty; sampled rows against the oracle."""
    q, k, v = make_qkv("t2i_2048")
    B, H, N, d = q.shape
    blocks, counts = random_kv_blocks(B, H, N, 0.3, seed=7, empty_every=9)
    rows = sample_rows(N, seed=7, n_edge=256, stride=64)
    say(f"[gpu] blocksparse t2i_2048 H={H} N={N} max_blocks={blocks.shape[-1]} rows={rows.size}")
    _compare(q, k, v, blocks, counts, 1 / math.sqrt(d), "sparse t2i_2048", rows=rows)


def test_blocksparse_rejects_fp8_and_d64():
    dit = _dit()
    q8 = torch.zeros((1, 1, 64, 128), dtype=torch.float8_e4m3fn, device=DEV)
    b = torch.zeros((1, 1, 1, 1), dtype=torch.int32, device=DEV)
    c = torch.ones((1, 1, 1), dtype=torch.int32, device=DEV)
    o = torch.empty((1, 1, 64, 128), dtype=torch.bfloat16, device=DEV)
    st = dit.dit_attn_fwd_blocksparse(q8, q8, q8, o, 1, 1, 64, 128, 0.1, dit.DIT_ATTN_FP8_E4M3, b, c, 1)
    assert st == dit.DIT_ATTN_EUNSUPPORTED
    q = torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16, device=DEV)
    st = dit.dit_attn_fwd_blocksparse(q, q, q, o, 1, 1, 64, 64, 0.1, dit.DIT_ATTN_BF16, b, c, 1)
    assert st == dit.DIT_ATTN_EUNSUPPORTED
