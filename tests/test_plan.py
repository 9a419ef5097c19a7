"""Host logic of the launch schedule, through dit_attn_plan (no GPU: an
explicit CU count). The launch itself calls the same planner, so these pin
what the kernels are given: one workgroup per 256-row query tile, the last
round's tiles split along the keys when that shortens the last round, or
stream-K for calls of at most two rounds when it is cheaper."""
import itertools

import pytest

import diffusion_transformer_attention_non_amd as dit

BF16, FP8 = dit.DIT_ATTN_BF16, dit.DIT_ATTN_FP8_E4M3
TILE, SPLIT, STREAMK = dit.DIT_ATTN_SCHED_TILE, dit.DIT_ATTN_SCHED_SPLIT, dit.DIT_ATTN_SCHED_STREAMK
ROW_BYTES = 129 * 4        # a partial row: 128 fp32 values and its log-sum-exp


BIG = 1 << 40              # a workspace larger than any plan needs: the fastest schedule
MAX_WS = (1 << 17) * ROW_BYTES + (1 << 17) * 4    # the bound include/dit_attn.h states


def plan(B, H, N, d=128, dtype=BF16, max_blocks=0, lse=False, n_cu=256, ws=BIG):
    st, p = dit.dit_attn_plan(B, H, N, d, dtype, max_blocks, lse, n_cu, ws)
    assert st == dit.DIT_ATTN_OK, st
    assert p.best_schedule == p.schedule or ws < p.workspace_wanted
    if ws >= p.workspace_wanted:
        assert p.workspace_bytes == p.workspace_wanted
    return p


def test_headline_shape_splits_its_last_round():
    # 24 heads x 66 tiles = 1584 = 6 rounds of 256 + 48: those 48 split into 5 key ranges
    p = plan(1, 24, 16896)
    assert (p.schedule, p.parts, p.split_tiles) == (SPLIT, 5, 48)
    assert p.workgroups == 1584 - 48 + 48 * 5
    assert p.workspace_bytes == 48 * 5 * 256 * ROW_BYTES


@pytest.mark.parametrize("H", [1, 3, 5, 6])
def test_per_gpu_shares_use_streamk(H):
    """At most two rounds of tiles (H <= 7 at 66 tiles a head): every CU takes an
    equal share; two workspace slots of 256 partial rows per CU. (H = 4, 264
    tiles, is the near tie where splitting the 8 tiles past one round costs
    the same.)"""
    p = plan(1, H, 16896)
    assert p.schedule == STREAMK and p.workgroups == 256 and p.parts == 1 and p.split_tiles == 0
    assert p.workspace_bytes == 2 * 256 * 256 * ROW_BYTES


def test_many_rounds_never_streamk():
    for H in range(8, 49):
        p = plan(1, H, 16896)
        assert p.schedule in (TILE, SPLIT), H


def test_tiny_and_d64_calls_run_one_workgroup_per_tile():
    p = plan(1, 1, 256)
    assert (p.schedule, p.workgroups, p.workspace_bytes) == (TILE, 1, 0)
    p = plan(1, 2, 256, d=64)
    assert p.schedule == TILE and p.workspace_bytes == 0


def test_fp8_plans_over_128_key_tiles_and_lse_adds_exact_sums():
    p = plan(1, 24, 16896, dtype=FP8)
    q = plan(1, 24, 16896, dtype=FP8, lse=True)
    assert p.schedule == SPLIT and p.split_tiles == 48
    units = p.split_tiles * p.parts * 256
    assert p.workspace_bytes == units * ROW_BYTES
    assert q.workspace_bytes == units * ROW_BYTES + units * 4
    # the fp8 path never takes stream-K
    assert plan(1, 3, 16896, dtype=FP8).schedule != STREAMK


def test_blocksparse_plans_with_the_list_length():
    full = plan(1, 24, 16896)
    short = plan(1, 24, 16896, max_blocks=20)       # 20 key tiles: at most 5 parts of 4
    assert short.schedule in (TILE, SPLIT) and short.parts <= 5
    assert plan(1, 3, 16896, max_blocks=264).schedule != STREAMK
    assert full.parts >= short.parts


@pytest.mark.parametrize("n_cu", [80, 104, 228, 256, 304])
def test_plan_invariants_over_shapes(n_cu):
    for B, H, N in itertools.product([1, 2], [1, 2, 3, 6, 12, 24], [64, 300, 4608, 16896, 25088]):
        tiles = B * H * -(-N // 256)
        n_t = -(-N // 64)
        p = plan(B, H, N, n_cu=n_cu)
        if p.schedule == TILE:
            assert p.workgroups == tiles and p.workspace_bytes == 0
        elif p.schedule == SPLIT:
            assert p.split_tiles == tiles % n_cu and p.parts >= 2
            assert n_t // p.parts >= 4                                   # at least 4 key tiles a range
            assert p.workgroups == tiles - p.split_tiles + p.split_tiles * p.parts
            assert p.workspace_bytes == p.split_tiles * p.parts * 256 * ROW_BYTES
            # a split last round must not take more waves than it saves
            assert -(-p.split_tiles * p.parts // n_cu) < p.parts
        else:
            assert tiles <= 2 * n_cu
            min_range = max(4, -(-n_t // 13))
            # one group per CU, at most 256 (2 x 256 slots of 256 partial rows: the workspace bound)
            assert p.workgroups == min(n_cu, 256, tiles * n_t // min_range) and p.workgroups >= 2
            # the merge takes at most 16 parts of a cut tile: ranges are at least
            # ceil(n_t / 13) key tiles, so at most 14 boundaries fall inside a tile
            assert (tiles * n_t) // p.workgroups >= -(-n_t // 13)
            assert p.workspace_bytes == 2 * p.workgroups * 256 * ROW_BYTES


def test_plan_rejects_bad_arguments():
    bad = [((0, 1, 64, 128, BF16, 0, 0, 256), dit.DIT_ATTN_EINVAL),
           ((1, 1, 64, 96, BF16, 0, 0, 256), dit.DIT_ATTN_EUNSUPPORTED),
           ((1, 1, 64, 64, FP8, 0, 0, 256), dit.DIT_ATTN_EUNSUPPORTED),
           ((1, 1, 64, 128, 7, 0, 0, 256), dit.DIT_ATTN_EUNSUPPORTED),
           ((1, 1, 64, 128, BF16, 2, 0, 256), dit.DIT_ATTN_EINVAL),          # max_blocks past ceil(N/64)
           ((1, 1, 64, 64, BF16, 1, 0, 256), dit.DIT_ATTN_EUNSUPPORTED),     # sparse needs d = 128
           ((1, 1, 64, 128, BF16, 0, 0, -1), dit.DIT_ATTN_EINVAL),
           ((1, 1, 64, 128, BF16, 0, 0, 256, -1), dit.DIT_ATTN_EINVAL)]
    for args, want in bad:
        assert dit.dit_attn_plan(*args)[0] == want, args


def test_plan_for_the_current_device_needs_one():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert dit.dit_attn_plan(1, 1, 64, 128, BF16, 0, 0, 0)[0] == dit.DIT_ATTN_EDEVICE


@pytest.mark.parametrize("n_cu", [80, 256, 304])
def test_streamk_ranges_cover_each_pair_once_and_cut_tiles_into_at_most_16_parts(n_cu):
    """The stream-K kernel gives group g the pairs [work*g/G, work*(g+1)/G)
    (integer division) and its merge handles at most 16 parts of one tile;
    for every stream-K plan over the shapes below, the ranges tile the
    (tile, key tile) pairs exactly and no tile meets more than 16 ranges."""
    seen = 0
    for B, H in itertools.product([1, 2], [1, 2, 3, 4, 5, 6, 8]):
        for N in [64, 300, 2048, 4608, 12800, 16896, 25088, 40001]:
            p = plan(B, H, N, n_cu=n_cu)
            if p.schedule != STREAMK:
                continue
            seen += 1
            tiles, n_t, G = B * H * -(-N // 256), -(-N // 64), p.workgroups
            work = tiles * n_t
            bounds = [work * g // G for g in range(G + 1)]
            assert bounds[0] == 0 and bounds[-1] == work
            assert all(b1 > b0 for b0, b1 in zip(bounds, bounds[1:]))       # no empty range
            parts = [0] * tiles
            for g in range(G):
                first, last = bounds[g] // n_t, (bounds[g + 1] - 1) // n_t
                for t in range(first, last + 1):
                    parts[t] += 1
            assert max(parts) <= 16, (B, H, N, n_cu, max(parts))
    assert seen >= 5


def test_without_workspace_one_workgroup_per_tile_and_the_plan_says_what_one_buys():
    """No workspace (dit_attn_fwd, dit_attn_fwd_ex, or a 0-byte one): one
    workgroup per query tile, and the plan still reports the fastest schedule
    and its workspace, so the fallback is never silent."""
    for H, best in [(24, SPLIT), (3, STREAMK)]:
        fast = plan(1, H, 16896)
        p = plan(1, H, 16896, ws=0)
        assert (p.schedule, p.workgroups, p.workspace_bytes) == (TILE, H * 66, 0)
        assert p.best_schedule == best == fast.schedule
        assert p.workspace_wanted == fast.workspace_bytes > 0
        p = plan(1, H, 16896, ws=fast.workspace_bytes)      # exactly enough
        assert p.schedule == best


def test_a_workspace_too_small_is_an_error_not_a_fallback():
    need = plan(1, 24, 16896).workspace_bytes
    for ws in (16, need - 16):
        st, _ = dit.dit_attn_plan(1, 24, 16896, 128, BF16, 0, 0, 256, ws)
        assert st == dit.DIT_ATTN_EWORKSPACE
    # a shape whose fastest schedule needs none takes any workspace
    assert plan(1, 1, 256, ws=16).schedule == TILE


@pytest.mark.parametrize("n_cu", [80, 256])
def test_workspace_never_exceeds_the_stated_bound(n_cu):
    worst = 0
    for B, H, N in itertools.product([1, 2, 3], [1, 3, 6, 24, 48, 100], [300, 4608, 16896, 25088, 65536]):
        for dtype, lse in [(BF16, False), (FP8, True)]:
            worst = max(worst, plan(B, H, N, dtype=dtype, lse=lse, n_cu=n_cu).workspace_bytes)
    assert 0 < worst <= MAX_WS
