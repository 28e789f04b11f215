"""attn_bwd_noalloc (the backward pass with the library's static device
scratch instead of a caller workspace) against attn_bwd, through the C ABI.

Two calls in a row, the second on a smaller input, so that the second reads
nothing the first left in the shared scratch; each must equal attn_bwd on the
same inputs bitwise (both take the same kernels and the same GQA head split
whenever its partials fit the scratch, as they do here), and agree with the
CPU fp64 oracle within the stated tolerances.  A size whose D does not fit
the scratch is rejected before anything is launched.
"""

import numpy as np
import pytest

import oracle
from exact_io_aware_75_amd import inputs as gen
from gpu_util import TOL_GRAD, excess, log, tol_kv

pytestmark = pytest.mark.gpu

# (b, n, hq, hkv, d, dtype, causal): first call, then a smaller second call
PAIRS = [
    ((2, 1000, 4, 2, 128, "bf16", True), (1, 300, 2, 1, 64, "bf16", False)),
    # MQA with a small grid: the dK/dV pass splits the 8 query heads of the
    # group over 8 workgroups per key block, fp32 partials in the scratch
    ((1, 1024, 8, 1, 128, "bf16", True), (1, 512, 4, 1, 128, "fp16", True)),
]


def _grads(x, dtype, causal, scale, device, noalloc):
    import torch
    import exact_io_aware_75_amd as ea

    q, k, v, do = (gen.to_torch(x[t], dtype, device) for t in ("q", "k", "v", "do"))
    o, lse = ea.forward(q, k, v, causal=causal, scale=scale)
    if noalloc:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ea.attn_bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv, causal, scale)
    else:
        dq, dk, dv = ea.backward(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return [t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv)]


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_matches_attn_bwd(gpu_device, first, second):
    for i, (b, n, hq, hkv, d, dtype, causal) in enumerate((first, second)):
        x = gen.make_inputs(b, n, hq, hkv, d, dtype, cfg_id=61, seed=n)
        scale = 1.0 / np.sqrt(d)
        tag = f"noalloc call {i + 1}: b{b} n{n} hq{hq} hkv{hkv} d{d} {dtype} causal={causal}"
        log(tag)
        got = _grads(x, dtype, causal, scale, gpu_device, noalloc=True)
        ref = _grads(x, dtype, causal, scale, gpu_device, noalloc=False)
        for nm, a, r in zip(("dq", "dk", "dv"), got, ref):
            assert np.array_equal(a, r), (tag, nm, float(np.abs(a - r).max()))
        rdq, rdk, rdv = oracle.attention_bwd(x["q"], x["k"], x["v"], x["do"], causal, scale)
        for nm, a, r in zip(("dq", "dk", "dv"), got, (rdq, rdk, rdv)):
            tol = TOL_GRAD if nm == "dq" else tol_kv(hq, hkv)
            assert excess(a, r, tol, dtype) <= 0, (tag, nm, float(np.abs(a - r).max()))
        log(f"  equal to attn_bwd; max|err| vs oracle dq {np.abs(got[0] - rdq).max():.2e} "
            f"dk {np.abs(got[1] - rdk).max():.2e} dv {np.abs(got[2] - rdv).max():.2e}")


def test_noalloc_rejects_sizes_beyond_its_scratch(gpu_device):
    """D of B * Hq * N floats above the 64 MiB scratch: ATTN_ERR_SCRATCH, and
    the output buffers are left untouched."""
    import torch
    from exact_io_aware_75_amd import _lib

    lib = _lib.load_library()
    b, n, hq, hkv, d = 64, 65536, 8, 8, 64  # D alone is 128 MiB
    dq = torch.full((16,), 7.0, device=gpu_device)
    ptr = dq.data_ptr()
    st = lib.attn_bwd_noalloc(ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, b, n, hq, hkv, d, 1, 0, 0.125, None)
    assert st == 11, st
    assert "scratch" in _lib.strerror(st)
    torch.cuda.synchronize()
    assert (dq == 7.0).all()
