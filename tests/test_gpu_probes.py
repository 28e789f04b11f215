"""The throughput probes of libattn_probe.so (include/attn_probe.h) run on the
GPU and leave results that show the work was done: MFMA outputs equal to the
product their operands define, exponential chains inside their fixed-point
range, LDS reads of the values written, and a plausible shader clock."""

import ctypes
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    lib = ctypes.CDLL(os.path.join(ROOT, "exact_io_aware_75_amd", "libattn_probe.so"))
    vp, i = ctypes.c_void_p, ctypes.c_int
    lib.attn_probe_mfma.argtypes = [vp, vp, i, i, vp]
    lib.attn_probe_exp.argtypes = [vp, vp, i, i, vp]
    lib.attn_probe_lds.argtypes = [vp, vp, i, i, vp]
    return lib


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def test_mfma_probe_computes_its_products(gpu_device, lib):
    import torch

    # constant operands 0.5: each 32x32x16 product adds 16 * 0.25 = 4 to every
    # accumulator element; 4 accumulators x 4 products per iteration, summed
    wgs, iters = 2, 3
    ops = torch.full((wgs * 256 * 64,), 0.5, dtype=torch.bfloat16, device=gpu_device)
    out = torch.empty(wgs * 256 * 16, dtype=torch.float32, device=gpu_device)
    assert lib.attn_probe_mfma(_p(ops), _p(out), wgs, iters, None) == 0
    torch.cuda.synchronize()
    assert torch.all(out == 4.0 * 16 * iters).item()


def test_exp_probe_stays_in_range(gpu_device, lib):
    import torch

    wgs = 4
    seed = torch.rand(wgs * 256 * 8, device=gpu_device)
    out = torch.empty(wgs * 256, device=gpu_device)
    assert lib.attn_probe_exp(_p(seed), _p(out), wgs, 50, None) == 0
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    # eight chains x <- 2^-x, each in (0.5, 1): their sum lies in (4, 8)
    assert np.all((o > 4.0) & (o < 8.0))


def test_lds_probe_reads_what_it_wrote(gpu_device, lib):
    import torch

    wgs, iters = 4, 8
    out = torch.empty(wgs * 256, device=gpu_device)
    clk = torch.zeros(2, dtype=torch.int64, device=gpu_device)
    assert lib.attn_probe_lds(_p(out), _p(clk), wgs, iters, None) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    buf = (np.arange(8192, dtype=np.uint64) * 2654435761 % (1 << 32)).astype(np.uint32)
    for tid in (0, 1, 77, 255):
        acc = np.uint32(0)
        for it in range(iters):
            for blk in range(8):
                word = (it + blk) & 3
                acc ^= buf[(tid * 16 + blk * 4096) // 4 + word]
        assert got[tid] == acc, tid
        assert got[256 + tid] == acc  # every workgroup reads the same data
    # a loop long enough (about a millisecond) for the 100 MHz counter's
    # granularity not to matter: shader cycles per 10 ns tick give the clock
    assert lib.attn_probe_lds(_p(out), _p(clk), wgs, 4000, None) == 0
    torch.cuda.synchronize()
    c = clk.cpu().numpy().astype(np.float64)
    assert c[1] > 0
    ghz = c[0] / c[1] * 0.1
    assert 0.5 < ghz < 3.5, ghz
