"""The seeded input generator: reproducible, the stated shapes, exact peaked scaling."""
import numpy as np
import torch

from workloads import WORKLOADS, coverage_pattern, make_qkv, sample_rows


def test_reproducible_bytes():
    a = make_qkv("tiny")
    b = make_qkv("tiny")
    for x, y in zip(a, b):
        assert x.dtype == torch.bfloat16 and x.shape == (1, 2, 256, 64) and x.is_contiguous()
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    c = make_qkv("tiny", seed=1)
    assert not torch.equal(a[0], c[0])


def test_token_counts_add_up():
    for w in WORKLOADS.values():
        assert w.N == w.n_text + w.n_image + w.n_ref, w.name
    assert WORKLOADS["t2i_2048"].flops == 4 * 24 * 16896**2 * 128


def test_peaked_is_exactly_four_times_seed1_draw():
    base = make_qkv("tiny", seed=1)
    w = WORKLOADS["t2i_2048_peaked"]
    q, k, v = make_qkv(w, B=1, H=2, N=256, d=64)
    assert torch.equal(q, base[0] * 4) and torch.equal(k, base[1]) and torch.equal(v, base[2])
    assert torch.equal((q.float() / 4).to(torch.bfloat16), base[0])


def test_sample_rows_cover_edges():
    r = sample_rows(16896, seed=0)
    assert r[0] == 0 and r[-1] == 16895 and np.all(np.diff(r) > 0)
    assert set(range(256)) <= set(r.tolist()) and set(range(16896 - 256, 16896)) <= set(r.tolist())
    assert np.array_equal(sample_rows(100, 3), np.arange(100))


def test_coverage_pattern_one_hot():
    _, _, v = coverage_pattern(1, 1, 300, 8, block=64)
    assert torch.equal(v.float().sum(-1), torch.ones(1, 1, 300))
    assert v[0, 0, 64 * 4 + 3, 4] == 1 and v[0, 0, 63, 0] == 1
