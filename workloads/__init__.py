"""Seeded synthetic inputs for DiT joint text+image attention.

This module only draws and shapes inputs. It holds none of the attention
arithmetic, so both the CPU oracle and the GPU path may take their inputs
from it.

Where the shapes come from
--------------------------
The pages describe FLUX 3 Image Klein on Blackwell: a DiT whose denoising
loop dominates latency at 2048x2048 and whose dense BF16 attention takes
about 60% of the DiT kernel time ("Speed Up Image Generation with FLUX 3
Image Klein on NVIDIA Blackwell GPUs", "Key takeaways"; the Italian
commentary, section "NVFP4, attention e caching"). They print no head count,
head dimension or token count. The shapes below are the stated workload of
this library: 24 heads of dimension 128, 512 text tokens, a 16-pixel
effective patch (so 64x64 image tokens at 1024x1024 and 128x128 at
2048x2048) and, for image-to-image, two 64x64-token reference images. The
pages mention up to ten reference images (Japanese summary, first
paragraph); two is the workload chosen here. No claim is made that these
are the model's real dimensions.

Values are iid N(0,1) drawn in float32 from a CPU ``torch.Generator`` seeded
with ``seed``, drawn in the order q, k, v, each of shape (B, H, N, d), then
rounded to bfloat16 (round-to-nearest-even, torch's cast). The "peaked"
variant multiplies Q by 4 after the draw (exact in bf16: a power of two).
The pages used seed 0 for their requests (Japanese summary, paragraph on
limitations); seed 0 is the default here too.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    n_text: int
    n_image: int
    n_ref: int = 0
    q_mult: float = 1.0
    seed: int = 0
    dtype: str = "bf16"
    note: str = ""

    @property
    def flops(self) -> float:
        """Two dense contractions of N x N x d per head, 2 flop per MAC."""
        return 4.0 * self.B * self.H * self.N * self.N * self.d


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 256, 64, 64, 192,
                     note="64 text + 192 image tokens, d=64"),
    "t2i_1024": Workload("t2i_1024", 2, 24, 4608, 128, 512, 4096,
                         note="1024x1024-equivalent, CFG cond/uncond pair as B=2, 64x64 image grid"),
    "t2i_2048": Workload("t2i_2048", 1, 24, 16896, 128, 512, 16384,
                         note="2048x2048-equivalent, 128x128 image grid"),
    "t2i_2048_peaked": Workload("t2i_2048_peaked", 1, 24, 16896, 128, 512, 16384,
                                q_mult=4.0, seed=1,
                                note="2048x2048-equivalent, seed 1, Q scaled by 4 (peaked rows)"),
    "t2i_2048_fp8": Workload("t2i_2048_fp8", 1, 24, 16896, 128, 512, 16384, dtype="fp8",
                             note="2048x2048-equivalent, inputs quantised to e4m3 per tensor, output bf16"),
    "i2i_2048": Workload("i2i_2048", 1, 24, 25088, 128, 512, 16384, n_ref=8192,
                         note="image-to-image-equivalent: 512 text + 128x128 target + 2x64x64 reference tokens"),
    # One GPU's share of the 2048x2048-equivalent call under sequence
    # parallelism over the heads: 24 heads over 4 (cfg 2 x ulysses 4 on 8 GPUs)
    # or 8 sequence-parallel ranks.
    "t2i_2048_h6": Workload("t2i_2048_h6", 1, 6, 16896, 128, 512, 16384,
                            note="per-GPU share of t2i_2048 with 4-way head sharding"),
    "t2i_2048_h3": Workload("t2i_2048_h3", 1, 3, 16896, 128, 512, 16384,
                            note="per-GPU share of t2i_2048 with 8-way head sharding"),
    # The head dimension of the tiny case at a full sequence: measures the
    # d = 64 kernel (the workloads above are all d = 128).
    "t2i_2048_d64": Workload("t2i_2048_d64", 1, 24, 16896, 64, 512, 16384,
                             note="2048x2048-equivalent sequence at head dimension 64"),
}


def make_qkv(w: Workload | str, seed: int | None = None, *, B=None, H=None, N=None, d=None):
    """Return (q, k, v) as contiguous CPU bfloat16 tensors of shape (B, H, N, d).

    Shape fields may be overridden (used for odd-N and small cases)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    B = w.B if B is None else B
    H = w.H if H is None else H
    N = w.N if N is None else N
    d = w.d if d is None else d
    seed = w.seed if seed is None else seed
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    shape = (B, H, N, d)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    q = q.to(torch.bfloat16)
    if w.q_mult != 1.0:
        q = q * w.q_mult
    return q.contiguous(), k.to(torch.bfloat16).contiguous(), v.to(torch.bfloat16).contiguous()


def random_qkv(B, H, N, d, seed=0, std=1.0):
    """iid N(0, std^2) bf16 tensors of an arbitrary shape (odd N, edge cases)."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    shape = (B, H, N, d)
    out = [(torch.randn(shape, generator=g, dtype=torch.float32) * std).to(torch.bfloat16).contiguous()
           for _ in range(3)]
    return tuple(out)


def one_growing_row(B, H, N, d, row=700, q_row=100.0, slope=0.05, seed=41):
    """iid N(0, 1) bf16 tensors in which one query row's logits grow along
    the keys: K's first feature is slope * j for key j and Q's first feature
    is q_row in that row, so its logits rise by slope * q_row / sqrt(d) per
    key (the other rows, whose first feature is N(0, 1), about 50 times
    more slowly at q_row = 100)."""
    q, k, v = random_qkv(B, H, N, d, seed=seed)
    q, k = q.float(), k.float()
    k[..., 0] = slope * torch.arange(N, dtype=torch.float32)
    q[:, :, row, 0] = q_row
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v


def sample_rows(N: int, seed: int, n_edge: int = 256, stride: int = 16) -> np.ndarray:
    """Sorted query-row indices: every row of the first and last ``n_edge``
    rows plus a seeded 1/``stride`` sample of the rest. Used to compare large
    cases row by row (each output row depends on one query row only)."""
    rng = np.random.default_rng(seed)
    edge = np.concatenate([np.arange(min(n_edge, N)), np.arange(max(0, N - n_edge), N)])
    mid = np.arange(min(n_edge, N), max(min(n_edge, N), N - n_edge))
    pick = mid[rng.random(mid.size) < 1.0 / stride] if mid.size else mid
    return np.unique(np.concatenate([edge, pick])).astype(np.int64)


# ---------------------------------------------------------------- structured inputs
# Inputs whose exact attention output has a closed form. They are input
# constructions only; the expected values are computed by the oracle.

def identical_keys(B, H, N, d, seed=0):
    """All keys of a head equal one random vector: every logit of a row is equal."""
    q, k, v = random_qkv(B, H, N, d, seed)
    k = k[:, :, :1, :].expand(B, H, N, d).contiguous()
    return q, k, v


def constant_values(B, H, N, d, seed=0, c=1.0):
    """V has the same row c*1 at every token."""
    q, k, _ = random_qkv(B, H, N, d, seed)
    v = torch.full((B, H, N, d), c, dtype=torch.bfloat16)
    return q, k, v


def coverage_pattern(B, H, N, d, block=64):
    """Identical (zero) keys and a one-hot V: V[j, c] = 1 iff (j // block) % d == c.

    With all logits equal, output channel c equals the fraction of tokens
    whose block index is congruent to c mod d. Dropping or repeating any
    key block shifts at least one channel by block/N."""
    q = torch.zeros((B, H, N, d), dtype=torch.bfloat16)
    k = torch.zeros((B, H, N, d), dtype=torch.bfloat16)
    j = torch.arange(N)
    v = torch.zeros((N, d), dtype=torch.bfloat16)
    v[j, (j // block) % d] = 1.0
    v = v.expand(B, H, N, d).contiguous()
    return q.contiguous(), k, v


def dominating_key(B, H, N, d, j_star, seed=0, a=4.0, b=4.0):
    """Queries a*u, keys small noise except K[j_star] = b*u (u a unit-RMS bf16 vector)."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    u = torch.sign(torch.randn((d,), generator=g)).to(torch.float32)  # +-1 entries: |u|^2 = d
    q = (a * u).expand(B, H, N, d).to(torch.bfloat16).contiguous()
    k = (0.05 * torch.randn((B, H, N, d), generator=g)).to(torch.bfloat16)
    k[:, :, j_star, :] = (b * u).to(torch.bfloat16)
    v = torch.randn((B, H, N, d), generator=g).to(torch.bfloat16).contiguous()
    return q, k.contiguous(), v


# ---------------------------------------------------------------- block lists
def random_kv_blocks(B, H, N, density, seed=0, *, q_block=256, kv_block=64, n_text=512, max_blocks=None,
                     empty_every=0):
    """Seeded key-block lists for block-sparse attention.

    For each (b, h, query block) the list holds every block of the first
    ``n_text`` tokens (the text prompt, which each image token attends to)
    and each remaining key block with probability ``density``, ascending.
    The pages report a sparse attention mode without its selection rule, so
    this pattern is only a stand-in with a plausible structure. With
    ``empty_every`` = m > 0 every m-th query block (flat index) gets an empty
    list. Returns (blocks int32 (B, H, nq, max_blocks) padded with -1,
    counts int32 (B, H, nq)); max_blocks defaults to the longest list (>= 1).
    """
    nq = -(-N // q_block)
    nk = -(-N // kv_block)
    n_text_blocks = min(nk, -(-n_text // kv_block)) if n_text > 0 else 0
    rng = np.random.default_rng(seed)
    lists = []
    for t in range(B * H * nq):
        keep = np.zeros(nk, dtype=bool)
        keep[:n_text_blocks] = True
        keep[n_text_blocks:] = rng.random(nk - n_text_blocks) < density
        if empty_every and t % empty_every == empty_every - 1:
            keep[:] = False
        lists.append(np.nonzero(keep)[0].astype(np.int32))
    longest = max([1] + [x.size for x in lists])
    mb = longest if max_blocks is None else max_blocks
    assert mb >= longest
    blocks = np.full((B * H * nq, mb), -1, dtype=np.int32)
    counts = np.zeros(B * H * nq, dtype=np.int32)
    for t, x in enumerate(lists):
        blocks[t, :x.size] = x
        counts[t] = x.size
    return (torch.from_numpy(blocks.reshape(B, H, nq, mb)).contiguous(),
            torch.from_numpy(counts.reshape(B, H, nq)).contiguous())


def block_varied_qkv(B, H, N, d, seed=0, qk_range=2, v_range=6):
    """Q, K, V whose 32-value blocks carry different powers of two: iid N(0,1)
    values times 2^k, k uniform in [-qk_range, qk_range] per (row, 32 d values)
    of Q and K and in [-v_range, v_range] per (32 tokens, column) of V. The
    block-scaled formats give each such block its own scale, so inputs like
    these tell apart the blocks that iid values (whose blocks all have about
    the same maximum) would not."""
    q, k, v = random_qkv(B, H, N, d, seed=seed)
    rng = np.random.default_rng(seed + 1000)
    def along_d(t, r):
        ex = rng.integers(-r, r + 1, size=(B, H, N, d // 32))
        f = torch.from_numpy(np.repeat(np.ldexp(1.0, ex), 32, axis=-1)).float()
        return (t.float() * f).to(torch.bfloat16).contiguous()
    nt = -(-N // 32)
    ex = rng.integers(-v_range, v_range + 1, size=(B, H, nt, d))
    fv = torch.from_numpy(np.repeat(np.ldexp(1.0, ex), 32, axis=2)[:, :, :N]).float()
    return along_d(q, qk_range), along_d(k, qk_range), (v.float() * fv).to(torch.bfloat16).contiguous()
