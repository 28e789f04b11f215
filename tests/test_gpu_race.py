"""Race checks on the GPU: every kernel's result must be independent of the
order and the concurrency in which its workgroups run.

Each case runs the forward and backward passes three times through the C ABI
on the same inputs -- in the normal launch order, with every kernel's
workgroups taking their work items in reversed order, and with every CU held
to one workgroup at a time (LDS padding) -- and requires bitwise equal
outputs.  No kernel uses atomics, so any difference would be a race (a read
of LDS or of another workgroup's output before it is complete) or a
dependence on scheduling.  The modes are the library's ATTN_LAUNCH_TEST
settings, read on every call.
"""

import os

import numpy as np
import pytest

from exact_io_aware_75_amd import inputs as gen
from gpu_util import log, make_rect_inputs, run_fwd_bwd

pytestmark = pytest.mark.gpu

MODES = ("reverse", "one_wg_per_cu")

CASES = [
    # b, n, hq, hkv, d, dtype, causal
    (2, 1000, 4, 2, 128, "bf16", True),
    (2, 1000, 4, 2, 128, "bf16", False),
    (1, 2100, 2, 1, 128, "bf16", False),   # eight-wavefront forward, ragged end
    (1, 8250, 1, 1, 64, "fp16", False),    # three wavefronts per SIMD (d = 64, short keys)
    (1, 16500, 1, 1, 64, "fp16", False),   # eight-wavefront forward at d = 64
    (1, 8250, 2, 1, 128, "bf16", True),    # eight-wavefront causal forward and dQ at d = 128
    (1, 512, 8, 1, 64, "bf16", True),      # MQA: dK/dV head split + reduce
    (1, 777, 8, 2, 128, "bf16", False),    # GQA head split, non-causal
    (1, 600, 4, 4, 256, "bf16", True),
    (3, 333, 2, 2, 64, "bf16", True),
    (1, 600, 4, 2, 128, "bf16", True),    # paired short causal passes, odd block count
    (1, 640, 8, 1, 128, "bf16", True),    # the same with the MQA dK/dV head split
]


def _run_modes(fn):
    base = fn()
    outs = {}
    try:
        for m in MODES:
            os.environ["ATTN_LAUNCH_TEST"] = m
            outs[m] = fn()
    finally:
        os.environ.pop("ATTN_LAUNCH_TEST", None)
    return base, outs


def _same(tag, base, outs):
    names = ("o", "lse", "dq", "dk", "dv")
    for m, out in outs.items():
        for nm, a, b in zip(names, base, out):
            assert np.array_equal(a, b, equal_nan=True), (tag, m, nm, float(np.nanmax(np.abs(a - b))))
    log(f"{tag}: identical in modes {', '.join(outs)}")


@pytest.mark.parametrize("b,n,hq,hkv,d,dtype,causal", CASES)
def test_dense_independent_of_launch_order(gpu_device, b, n, hq, hkv, d, dtype, causal):
    x = gen.make_inputs(b, n, hq, hkv, d, dtype, cfg_id=51, seed=n)
    scale = 1.0 / np.sqrt(d)
    tag = f"race b{b} n{n} hq{hq} hkv{hkv} d{d} {dtype} causal={causal}"
    log(tag)
    base, outs = _run_modes(lambda: run_fwd_bwd(x, dtype, causal, scale, gpu_device))
    _same(tag, base, outs)


def test_rect_independent_of_launch_order(gpu_device):
    x = make_rect_inputs(1, 450, 1000, 2, 2, 128, "bf16", cfg_id=52)
    tag = "race rect nq450 nk1000 offset 211"
    log(tag)
    base, outs = _run_modes(lambda: run_fwd_bwd(x, "bf16", True, 1.0 / np.sqrt(128), gpu_device,
                                                causal_offset=211))
    _same(tag, base, outs)


@pytest.mark.parametrize("causal", [False, True])
def test_blocksparse_independent_of_launch_order(gpu_device, causal):
    n, hkv = 1000, 2
    x = gen.make_inputs(1, n, 4, hkv, 128, "bf16", cfg_id=53)
    mask = gen.make_block_mask(hkv, n, 0.4, cfg_id=53, diagonal=True)
    tag = f"race block-sparse n{n} causal={causal}"
    log(tag)
    base, outs = _run_modes(lambda: run_fwd_bwd(x, "bf16", causal, 1.0 / np.sqrt(128), gpu_device,
                                                block_mask=mask))
    _same(tag, base, outs)


def test_splitkv_independent_of_launch_order(gpu_device):
    import torch
    import exact_io_aware_75_amd as ea

    x = make_rect_inputs(1, 128, 5000, 4, 2, 128, "bf16", cfg_id=54)
    q, k, v = (gen.to_torch(x[t], "bf16", gpu_device) for t in ("q", "k", "v"))

    def fn():
        o, lse = ea.forward(q, k, v, causal=False, num_splits=8)
        torch.cuda.synchronize()
        return o.float().cpu().numpy(), lse.cpu().numpy()

    base, outs = _run_modes(fn)
    for m, out in outs.items():
        for a, b_ in zip(base, out):
            assert np.array_equal(a, b_), m
    log("race split-KV nq128 nk5000: identical")
