"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle runs.

This module holds no attention arithmetic: it only draws iid N(0, 1) samples
and rounds them once to the storage dtype, so that the HIP path and the CPU
oracle see bit-identical values (the oracle upcasts them exactly to float64).

Recipe: every tensor is drawn in float32 from
``numpy.random.default_rng(SeedSequence([cfg_id, N, tensor_id, seed]))`` with
tensor ids Q=0, K=1, V=2, dO=3, then rounded to nearest-even to bf16 or fp16.
Causal and non-causal runs reuse the same tensors.  Block masks for
block-sparse attention are drawn the same way (tensor id 4): each (query
block, key block) entry is 1 with a given probability, optionally with every
diagonal block set.
"""

from __future__ import annotations

import numpy as np

TENSOR_ID = {"q": 0, "k": 1, "v": 2, "do": 3, "mask": 4}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 values that are exactly representable in bfloat16.  Inputs
    must be finite (normal samples always are).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 ``x`` once to ``dtype`` ('bf16' or 'fp16'); return float32."""
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "fp16":
        return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)
    raise ValueError(f"unsupported dtype {dtype!r}")


def draw(shape, dtype: str, cfg_id: int, n: int, tensor: str, seed: int = 0) -> np.ndarray:
    """iid N(0,1) float32 tensor of ``shape``, rounded once to ``dtype``."""
    ss = np.random.SeedSequence([int(cfg_id), int(n), TENSOR_ID[tensor], int(seed)])
    rng = np.random.default_rng(ss)
    x = rng.standard_normal(size=tuple(shape), dtype=np.float32)
    return round_to_dtype(x, dtype)


def make_inputs(b: int, n: int, hq: int, hkv: int, d: int, dtype: str = "bf16",
                cfg_id: int = 0, seed: int = 0, with_do: bool = True):
    """Q [B,N,Hq,d], K/V [B,N,Hkv,d] and optionally dO [B,N,Hq,d] (float32 arrays
    holding values exactly representable in ``dtype``)."""
    out = {
        "q": draw((b, n, hq, d), dtype, cfg_id, n, "q", seed),
        "k": draw((b, n, hkv, d), dtype, cfg_id, n, "k", seed),
        "v": draw((b, n, hkv, d), dtype, cfg_id, n, "v", seed),
    }
    if with_do:
        out["do"] = draw((b, n, hq, d), dtype, cfg_id, n, "do", seed)
    return out


def make_block_mask(mask_heads: int, n: int, density: float, cfg_id: int = 0, seed: int = 0,
                    block: int = 128, diagonal: bool = True) -> np.ndarray:
    """Seeded block mask, uint8 [mask_heads, nb, nb] with nb = ceil(n / block):
    each entry is 1 with probability ``density``; ``diagonal`` also sets every
    diagonal block (each query block then sees its own keys)."""
    nb = -(-n // block)
    rng = np.random.default_rng(np.random.SeedSequence([int(cfg_id), int(n), TENSOR_ID["mask"], int(seed)]))
    m = (rng.random((mask_heads, nb, nb)) < density).astype(np.uint8)
    if diagonal:
        m[:, np.arange(nb), np.arange(nb)] = 1
    return m


def to_torch(x: np.ndarray, dtype: str, device="cpu"):
    """Upload a float32 array of ``dtype``-exact values as a torch tensor of that dtype.

    The conversion is exact because the values are already representable.
    """
    import torch

    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device=device).to(tdt)
