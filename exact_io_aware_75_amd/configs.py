"""Workload shapes and throughput accounting.

The shapes restate the measured grid the pages describe: sequence lengths
512..16k with an attention layer of hidden size 2048 and head dimension 64 or
128, causal and not (FlashAttention-2 announcement, "实验评估" section;
FlashAttention-2 review, "Результаты" section -- both say "64 or 128 heads",
which with hidden size 2048 can only mean head dimension 64 or 128); head
dimension up to 256 and MQA/GQA ("具体实现" section); long sequences up to 64k
(FlashAttention-1 news page, results on block-sparse attention at 64k).

FLOP accounting: forward 4*B*Hq*N^2*d (two N x N x d products), halved under a
causal mask; backward 2.5 x forward (five products instead of two).
Block-sparse: the same count over the computed blocks only (128 x 128 pairs
each; under a causal mask a diagonal block counts half).

Block-sparse workload (the pages benchmark block-sparse attention next to the
dense method without giving its pattern): the hidden-2048, d = 128 layer at
N = 16384, one mask for all heads, every diagonal block plus a seeded 25% of
the other blocks.
"""

from __future__ import annotations

from dataclasses import dataclass, asdict

SWEEP_N = (512, 1024, 2048, 4096, 8192, 16384)
TOKENS = 16384  # B * N for the hidden-size-2048 sweep


@dataclass(frozen=True)
class Shape:
    name: str
    cfg_id: int
    b: int
    n: int
    hq: int
    hkv: int
    d: int
    dtype: str
    causal: bool

    def fwd_flops(self) -> float:
        f = 4.0 * self.b * self.hq * self.n * self.n * self.d
        return f / 2 if self.causal else f

    def bwd_flops(self) -> float:
        return 2.5 * self.fwd_flops()

    def as_dict(self):
        return asdict(self)


def small_fp16() -> Shape:
    """Forward-only parity case: B=1, H=2, N=128, d=64, fp16, non-causal."""
    return Shape("fwd_small_fp16", 1, 1, 128, 2, 2, 64, "fp16", False)


def hidden2048(d: int, n: int, causal: bool) -> Shape:
    """Hidden size 2048 (H = 2048/d), B*N = 16384 tokens, bf16."""
    return Shape(f"h2048_d{d}", 2 if d == 64 else 3, TOKENS // n, n, 2048 // d, 2048 // d,
                 d, "bf16", causal)


def long_seq(n: int) -> Shape:
    """B=1, H=8, d=128, causal, N in {32768, 65536}."""
    return Shape("long_seq", 4, 1, n, 8, 8, 128, "bf16", True)


def gqa(hkv: int) -> Shape:
    """B=4, N=4096, Hq=32, Hkv in {8, 1}, d=128, causal."""
    return Shape(f"gqa_hkv{hkv}", 5, 4, 4096, 32, hkv, 128, "bf16", True)


def wide_head() -> Shape:
    """B=4, N=4096, H=8, d=256, causal (MHA)."""
    return Shape("mha_d256", 5, 4, 4096, 8, 8, 256, "bf16", True)


BLOCKSPARSE_DENSITY = 0.25


def blocksparse(causal: bool, n: int = 16384) -> Shape:
    """Hidden size 2048, d = 128 (H = 16), B = 16384 / N, block mask of
    BLOCKSPARSE_DENSITY plus the diagonal."""
    return Shape("blocksparse_h2048_d128", 6, TOKENS // n, n, 16, 16, 128, "bf16", causal)


def masked_fwd_flops(s: Shape, mask, block: int = 128) -> float:
    """Forward FLOPs over the computed blocks of ``mask`` ([1 or Hkv, nb, nb]):
    4 * d * block^2 per (head, batch, computed block), a causal diagonal block
    counting half and blocks past the diagonal not at all.  N must be a
    multiple of ``block``."""
    import numpy as np

    if s.n % block:
        raise ValueError("N must be a multiple of the block size")
    m = np.asarray(mask) != 0
    nb = m.shape[1]
    if s.causal:
        w = np.tril(np.ones((nb, nb))) - 0.5 * np.eye(nb)
    else:
        w = np.ones((nb, nb))
    per_mask = (m * w).sum(axis=(1, 2))  # weighted block count per mask
    heads_per_mask = s.hq if m.shape[0] == 1 else s.hq // s.hkv
    return 4.0 * s.d * block * block * s.b * heads_per_mask * float(per_mask.sum())


def all_shapes():
    out = [small_fp16()]
    for d in (64, 128):
        for n in SWEEP_N:
            for c in (False, True):
                out.append(hidden2048(d, n, c))
    out += [long_seq(32768), long_seq(65536), gqa(8), gqa(1), wide_head()]
    return out
