"""Pins of the block-sparse attention oracle against things other than itself.

Each pin takes a block-sparse attention function, so the same pins also run
against copies with a planted mistake (an off-by-one block end, a dense
normaliser, the wrong query-block size, ...): every mutant must fail one.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import random_kv_blocks


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _lists(B, H, nq, nk, seed, density=0.4, empty=()):
    """Random ascending lists (numpy) with the flat query-block indices in ``empty`` left empty."""
    rng = np.random.default_rng(seed)
    rows, counts = [], []
    for t in range(B * H * nq):
        sel = np.nonzero(rng.random(nk) < density)[0]
        if sel.size == 0:
            sel = np.array([rng.integers(nk)])
        if t in empty:
            sel = sel[:0]
        rows.append(sel)
        counts.append(sel.size)
    mb = max(1, max(counts))
    blocks = np.full((B * H * nq, mb), -1, dtype=np.int64)
    for t, sel in enumerate(rows):
        blocks[t, :sel.size] = sel
    return blocks.reshape(B, H, nq, mb), np.array(counts).reshape(B, H, nq)


def _allowed(blocks, counts, N, qb, kb):
    """(B, H, N, N) boolean: query i may attend to key j (built here, independently of the oracle)."""
    B, H, nq, _ = blocks.shape
    allow = np.zeros((B, H, N, N), dtype=bool)
    for b in range(B):
        for h in range(H):
            for t in range(nq):
                keys = np.zeros(N, dtype=bool)
                for u in blocks[b, h, t, :max(0, counts[b, h, t])]:
                    lo = u * kb
                    keys[lo:lo + kb] = True                # numpy clips at N
                allow[b, h, t * qb:(t + 1) * qb, :] = keys
    return allow


CASES = [((1, 2, 37, 8), 8, 4, 0), ((2, 1, 300, 16), 256, 64, 1), ((1, 2, 700, 8), 256, 64, 2),
         ((1, 1, 129, 4), 16, 8, 3)]


# ------------------------------------------------------------------ pins
def pin_masked_sdpa(bs):
    """Against torch's float64 CPU SDPA with a boolean mask and torch.logsumexp."""
    for (B, H, N, d), qb, kb, seed in CASES:
        q, k, v = (_rand((B, H, N, d), seed * 10 + i) for i in range(3))
        nq, nk = -(-N // qb), -(-N // kb)
        blocks, counts = _lists(B, H, nq, nk, seed, empty={1})
        scale = 1.0 / math.sqrt(d)
        allow = _allowed(blocks, counts, N, qb, kb)
        o, lse = bs(q, k, v, scale, blocks, counts, q_block=qb, kv_block=kb)
        live = allow.any(-1)                               # rows with at least one key
        tq, tk, tv, tm = (torch.from_numpy(x) for x in (q, k, v, allow))
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=tm, scale=scale).numpy()
        logits = torch.matmul(tq, tk.transpose(-1, -2)) * scale
        ref_lse = torch.logsumexp(logits.masked_fill(~tm, -math.inf), dim=-1).numpy()
        if not np.allclose(o[live], ref[live], rtol=0, atol=1e-12):
            return False
        if not np.allclose(lse[live], ref_lse[live], rtol=0, atol=1e-12):
            return False
        if not (np.all(o[~live] == 0.0) and np.all(np.isneginf(lse[~live]))):
            return False
    return True


def pin_full_lists_are_dense(bs):
    """Listing every key block gives the dense attention (pinned on its own)."""
    for (B, H, N, d), qb, kb, seed in CASES:
        q, k, v = (_rand((B, H, N, d), 50 + seed * 10 + i) for i in range(3))
        nq, nk = -(-N // qb), -(-N // kb)
        blocks = np.broadcast_to(np.arange(nk), (B, H, nq, nk)).copy()
        counts = np.full((B, H, nq), nk)
        o, lse = bs(q, k, v, 0.3, blocks, counts, q_block=qb, kv_block=kb)
        od, ld = oracle.attention(q, k, v, 0.3)
        if not (np.allclose(o, od, rtol=0, atol=1e-12) and np.allclose(lse, ld, rtol=0, atol=1e-12)):
            return False
    return True


def pin_single_tail_key(bs):
    """A list of only the last, one-key block: O is that key's V row, lse its logit."""
    B, H, N, d = 1, 2, 3 * 64 + 1, 8
    q, k, v = (_rand((B, H, N, d), 70 + i) for i in range(3))
    blocks = np.full((B, H, 1, 2), 3)
    counts = np.ones((B, H, 1), dtype=np.int64)
    o, lse = bs(q, k, v, 0.5, blocks, counts, q_block=256, kv_block=64)
    want_o = np.broadcast_to(v[:, :, N - 1:N, :], o.shape)
    want_l = 0.5 * (q * k[:, :, N - 1:N, :]).sum(-1)
    return np.array_equal(o, want_o) and np.allclose(lse, want_l, rtol=0, atol=1e-13)


def pin_merge_of_disjoint_lists(bs):
    """S = S1 u S2 disjoint: lse = log(e^lse1 + e^lse2), O = sum_i O_i e^(lse_i - lse)."""
    B, H, N, d = 1, 2, 600, 8
    q, k, v = (_rand((B, H, N, d), 80 + i) for i in range(3))
    nq, nk = 3, 10
    rng = np.random.default_rng(81)
    b1 = np.full((B, H, nq, nk), -1)
    b2 = np.full((B, H, nq, nk), -1)
    bu = np.full((B, H, nq, nk), -1)
    c1 = np.zeros((B, H, nq), dtype=np.int64)
    c2 = np.zeros_like(c1)
    cu = np.zeros_like(c1)
    for h in range(H):
        for t in range(nq):
            side = rng.integers(0, 3, nk)                  # 0: S1, 1: S2, 2: neither
            side[rng.integers(nk)] = 0
            side[rng.integers(nk)] = 1
            for arr, cnt, sel in ((b1, c1, side == 0), (b2, c2, side == 1), (bu, cu, side < 2)):
                idx = np.nonzero(sel)[0]
                arr[0, h, t, :idx.size] = idx
                cnt[0, h, t] = idx.size
    o1, l1 = bs(q, k, v, 0.4, b1, c1)
    o2, l2 = bs(q, k, v, 0.4, b2, c2)
    ou, lu = bs(q, k, v, 0.4, bu, cu)
    lm = np.logaddexp(l1, l2)
    om = o1 * np.exp(l1 - lm)[..., None] + o2 * np.exp(l2 - lm)[..., None]
    return np.allclose(lu, lm, rtol=0, atol=1e-12) and np.allclose(ou, om, rtol=0, atol=1e-12)


def pin_lists_are_sets(bs):
    """Order and repeats of list entries do not change the result; entries past the count are not read."""
    B, H, N, d = 1, 1, 300, 8
    q, k, v = (_rand((B, H, N, d), 90 + i) for i in range(3))
    base = np.array([[[[0, 2, 4, -1, -1, -1], [1, 3, -1, -1, -1, -1]]]])
    shuffled = np.array([[[[4, 0, 2, 2, 0, 77], [3, 1, 3, 99, 99, 99]]]])
    o1, l1 = bs(q, k, v, 0.3, base, np.array([[[3, 2]]]))
    o2, l2 = bs(q, k, v, 0.3, shuffled, np.array([[[5, 3]]]))
    return np.allclose(o1, o2, rtol=0, atol=1e-13) and np.allclose(l1, l2, rtol=0, atol=1e-13)


def pin_empty_lists(bs):
    """Count 0 (or negative): zero output rows and lse = -inf, other blocks unaffected."""
    B, H, N, d = 1, 1, 512, 4
    q, k, v = (_rand((B, H, N, d), 100 + i) for i in range(3))
    blocks = np.array([[[[0, 1], [5, 6]]]])
    o, lse = bs(q, k, v, 0.3, blocks, np.array([[[0, 2]]]))
    o_neg, lse_neg = bs(q, k, v, 0.3, blocks, np.array([[[-3, 2]]]))
    if not (np.all(o[:, :, :256] == 0) and np.all(np.isneginf(lse[:, :, :256]))):
        return False
    if not (np.array_equal(o, o_neg) and np.array_equal(lse, lse_neg)):
        return False
    return bool(np.isfinite(lse[:, :, 256:]).all())


PINS = [pin_masked_sdpa, pin_full_lists_are_dense, pin_single_tail_key, pin_merge_of_disjoint_lists,
        pin_lists_are_sets, pin_empty_lists]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_blocksparse_oracle_passes_pin(pin):
    assert pin(oracle.attention_blocksparse)


def test_blocksparse_oracle_row_subset_exact():
    q, k, v = (_rand((1, 2, 700, 8), 110 + i) for i in range(3))
    blocks, counts = _lists(1, 2, 3, 11, 111, empty={2})
    o, lse = oracle.attention_blocksparse(q, k, v, 0.3, blocks, counts)
    rows = np.array([0, 1, 255, 256, 511, 512, 699])
    orow, lrow = oracle.attention_blocksparse(q, k, v, 0.3, blocks, counts, rows=rows)
    # the matrix product over fewer rows may round differently in the last bit
    assert np.allclose(orow, o[:, :, rows], rtol=0, atol=1e-13)
    assert np.allclose(lrow, lse[:, :, rows], rtol=0, atol=1e-13)
    assert np.isneginf(lse[:, 0, 512:]).all() and np.isneginf(lrow[:, 0, -2:]).all()   # list (h 0, t 2) is empty


def test_blocksparse_weighted_abs():
    """A is O of |V|; with every block listed it is the dense oracle's A."""
    q, k, v = (_rand((1, 2, 300, 8), 120 + i) for i in range(3))
    blocks, counts = _lists(1, 2, 2, 5, 121, empty={3})
    o, lse, a = oracle.attention_blocksparse(q, k, v, 0.3, blocks, counts, want_abs=True)
    oa, _ = oracle.attention_blocksparse(q, k, np.abs(v), 0.3, blocks, counts)
    assert np.allclose(a, oa, rtol=0, atol=1e-14)
    assert np.all(a[:, 1, 256:] == 0)
    full = np.broadcast_to(np.arange(5), (1, 2, 2, 5)).copy()
    _, _, af = oracle.attention_blocksparse(q, k, v, 0.3, full, np.full((1, 2, 2), 5), want_abs=True)
    _, _, ad = oracle.attention(q, k, v, 0.3, want_abs=True)
    assert np.allclose(af, ad, rtol=0, atol=1e-13)


def test_random_kv_blocks_shape_and_order():
    blocks, counts = random_kv_blocks(2, 3, 1000, 0.3, seed=4, empty_every=5)
    assert blocks.dtype == torch.int32 and counts.dtype == torch.int32
    assert blocks.shape[:3] == (2, 3, 4) and counts.shape == (2, 3, 4)
    nk = -(-1000 // 64)
    flat_b, flat_c = blocks.reshape(-1, blocks.shape[-1]).numpy(), counts.reshape(-1).numpy()
    for t, (row, c) in enumerate(zip(flat_b, flat_c)):
        live = row[:c]
        assert (np.diff(live) > 0).all() and ((live >= 0) & (live < nk)).all()
        assert (row[c:] == -1).all()
        if t % 5 == 4:
            assert c == 0
        else:
            assert list(live[:8]) == list(range(8))       # the text blocks


# ------------------------------------------------------------------ planted mistakes
def _mutant(kind):
    def bs(q, k, v, scale, kv_blocks, kv_counts, q_block=256, kv_block=64, rows=None):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        B, H, N, d = q.shape
        qsz = kv_block if kind == "query_block_is_kv_block" else q_block
        nq = -(-N // q_block)
        out = np.zeros_like(q)
        lse = np.full((B, H, N), -np.inf)
        for b in range(B):
            for h in range(H):
                hb = (h + 1) % H if kind == "lists_of_next_head" else h
                for t in range(nq):
                    cnt = int(kv_counts[b, hb, t])
                    if kind == "count_minus_one":
                        cnt -= 1
                    mask = np.zeros(N, dtype=bool)
                    for u in np.asarray(kv_blocks[b, hb, t])[:max(0, cnt)]:
                        end = (u + 1) * kv_block + (1 if kind == "block_end_plus_one" else 0)
                        mask[u * kv_block:min(N, end)] = True
                    rs = slice(t * qsz, min(N, (t + 1) * qsz))
                    if not mask.any():
                        if kind == "empty_is_dense":
                            mask[:] = True
                        else:
                            continue
                    s = (q[b, h, rs] @ k[b, h].T) * scale
                    dense = s.copy()
                    if kind == "masked_logit_zero":
                        s[:, ~mask] = 0.0
                    else:
                        s[:, ~mask] = -np.inf
                    m = s.max(axis=1, keepdims=True)
                    e = np.exp(s - m)
                    den = e.sum(axis=1, keepdims=True)
                    if kind == "dense_normaliser":
                        den = np.exp(dense - m).sum(axis=1, keepdims=True)
                    out[b, h, rs] = (e @ v[b, h]) / den
                    lse[b, h, rs] = m[:, 0] + np.log(den[:, 0])
        return out, lse
    return bs


MUTANTS = ["query_block_is_kv_block", "lists_of_next_head", "count_minus_one", "block_end_plus_one",
           "empty_is_dense", "masked_logit_zero", "dense_normaliser"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistake_is_caught(kind):
    bs = _mutant(kind)
    with np.errstate(all="ignore"):
        failed = [p.__name__ for p in PINS if not p(bs)]
    assert failed, f"mutant {kind} passed every pin"


def test_unmutated_copy_passes():
    bs = _mutant("none")
    assert all(p(bs) for p in PINS)
