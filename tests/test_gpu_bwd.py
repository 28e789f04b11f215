"""GPU parity of the backward pass (attn_bwd through the C ABI) against the
CPU fp64 oracle, on seeded inputs.

Small shapes: every element of dQ, dK, dV.  Full-size workloads (the launch
configuration the benchmark times): dQ on sampled rows (computable row by
row); dK/dV on a whole sampled K/V head up to N = 16384 and for the MQA group,
and on 64 sampled keys of one head (each summed over every query row) at
N = 32768 and 65536; and at every size the gradient identities that hold
exactly:
sum_j dV_j = sum over the group's heads of sum_i dO_i, sum_j dK_j = 0 and,
under a causal mask, dQ of row 0 = 0.
"""

import numpy as np
import pytest

import oracle
from exact_io_aware_75_amd import inputs as gen
from gpu_util import TOL_GRAD, TOL_LSE, TOL_O, excess, full_size_shapes, log, max_err, record, run_fwd_bwd, tol_kv

pytestmark = pytest.mark.gpu


def _check_all(x, out, causal, scale, tag, dtype):
    o, lse, dq, dk, dv = out
    tkv = tol_kv(x["q"].shape[2], x["k"].shape[2])
    ro, rlse = oracle.attention_fwd(x["q"], x["k"], x["v"], causal, scale)
    rdq, rdk, rdv = oracle.attention_bwd(x["q"], x["k"], x["v"], x["do"], causal, scale)
    tols = {"o": TOL_O, "lse": TOL_LSE, "dq": TOL_GRAD, "dk": tkv, "dv": tkv}
    errs = {n: record(tag, n, a, r, tols[n], None if n == "lse" else dtype)
            for n, a, r in (("o", o, ro), ("lse", lse, rlse), ("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv))}
    log(f"{tag}: " + "  ".join(f"{n}={e:.2e}(|ref| {m:.2f})" for n, (e, m) in errs.items()))
    for t in (o, lse, dq, dk, dv):
        assert np.isfinite(t).all()
    assert excess(o, ro, TOL_O, dtype) <= 0, (tag, "o", errs["o"])
    assert errs["lse"][0] <= TOL_LSE
    for n, a_, r_ in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        assert excess(a_, r_, tols[n], dtype) <= 0, (tag, n, errs[n])


SMALL = [
    # b, n, hq, hkv, d, dtype
    (1, 1, 1, 1, 64, "bf16"),
    (2, 17, 2, 2, 64, "bf16"),
    (1, 100, 4, 2, 128, "bf16"),
    (1, 129, 2, 1, 128, "fp16"),
    (1, 300, 2, 2, 256, "bf16"),
    (1, 520, 4, 4, 64, "fp16"),
    (1, 700, 2, 2, 128, "bf16"),
    (1, 333, 8, 2, 256, "fp16"),
    (2, 256, 4, 1, 128, "bf16"),
    (1, 640, 2, 2, 64, "bf16"),
    (1, 600, 2, 2, 128, "bf16"),   # five blocks of 128: the middle one unpaired, ragged end
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("b,n,hq,hkv,d,dtype", SMALL)
def test_small_shapes(gpu_device, b, n, hq, hkv, d, dtype, causal):
    x = gen.make_inputs(b, n, hq, hkv, d, dtype, cfg_id=17, seed=n)
    scale = 1.0 / np.sqrt(d)
    out = run_fwd_bwd(x, dtype, causal, scale, gpu_device)
    _check_all(x, out, causal, scale, f"b{b} n{n} hq{hq} hkv{hkv} d{d} {dtype} causal={causal}", dtype)


def test_deterministic(gpu_device):
    """No atomics anywhere: two runs give bitwise identical gradients."""
    import torch

    x = gen.make_inputs(2, 1000, 4, 2, 128, "bf16", cfg_id=19)
    a = run_fwd_bwd(x, "bf16", True, 1.0 / np.sqrt(128), gpu_device)
    b = run_fwd_bwd(x, "bf16", True, 1.0 / np.sqrt(128), gpu_device)
    for u, w in zip(a, b):
        assert np.array_equal(u, w)
    del torch


@pytest.mark.parametrize("scale", [0.0, -0.1])
def test_unusual_scales(gpu_device, scale):
    x = gen.make_inputs(1, 150, 2, 1, 64, "bf16", cfg_id=18)
    out = run_fwd_bwd(x, "bf16", True, scale, gpu_device)
    _check_all(x, out, True, scale, f"scale={scale}", "bf16")


def test_workspace_contents_are_ignored(gpu_device):
    """A workspace full of garbage (NaNs) from a previous user gives the same result."""
    import torch
    import exact_io_aware_75_amd as ea

    b, n, hq, hkv, d = 1, 200, 2, 2, 128
    x = gen.make_inputs(b, n, hq, hkv, d, "bf16", cfg_id=19)
    q, k, v, do = (gen.to_torch(x[t], "bf16", gpu_device) for t in ("q", "k", "v", "do"))
    o, lse = ea.forward(q, k, v, causal=True)
    ws = torch.full((ea.attn_bwd_workspace_bytes(b, n, hq, hkv, d),), 0xFF, dtype=torch.uint8,
                    device=gpu_device)
    dq, dk, dv = ea.backward(q, k, v, o, lse, do, causal=True, workspace=ws)
    dq2, dk2, dv2 = ea.backward(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    for a_, b_ in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.isfinite(a_.float()).all()
        assert (a_.float() - b_.float()).abs().max().item() <= 2 * 2 ** -7 * b_.float().abs().max().item()


def _identities(s, x, dq, dk, dv):
    rep = s.hq // s.hkv
    dsum = x["do"].astype(np.float64).reshape(s.b, s.n, s.hkv, rep, s.d).sum(axis=(1, 3))
    e_dv = np.abs(dv.sum(axis=1) - dsum).max()
    e_dk = np.abs(dk.sum(axis=1)).max()
    # sums of N rounded terms: allow the rounding of each dV/dK element (half ulp of
    # the element's magnitude, <= 2^-8 relative in bf16) to accumulate like a random walk
    tol_dv = 4 * np.sqrt(s.n) * 2 ** -8 * max(1.0, np.abs(dv).max())
    tol_dk = 4 * np.sqrt(s.n) * 2 ** -8 * max(1.0, np.abs(dk).max())
    log(f"  identities: |sum dV - sum dO|={e_dv:.3e} (tol {tol_dv:.2e})  |sum dK|={e_dk:.3e} (tol {tol_dk:.2e})")
    assert e_dv <= tol_dv and e_dk <= tol_dk
    if s.causal:
        # row 0 attends only key 0, so P = 1 and dS = dP - D = 0 up to the fp32
        # summation order of dP (MFMA) versus D (row sum): |dQ_0| ~ 1e-7
        assert np.abs(dq[:, 0]).max() <= 1e-4


@pytest.mark.parametrize("s", full_size_shapes(), ids=lambda s: f"{s.name}_n{s.n}_c{int(s.causal)}")
def test_full_size(gpu_device, s):
    x = gen.make_inputs(s.b, s.n, s.hq, s.hkv, s.d, s.dtype, cfg_id=s.cfg_id)
    scale = 1.0 / np.sqrt(s.d)
    log(f"full-size fwd+bwd {s}")
    o, lse, dq, dk, dv = run_fwd_bwd(x, s.dtype, s.causal, scale, gpu_device)
    for t in (o, lse, dq, dk, dv):
        assert np.isfinite(t).all()
    _identities(s, x, dq, dk, dv)
    rng = np.random.default_rng(3 * s.n + s.d)
    # dQ on sampled rows
    got, ref = [], []
    for _ in range(24):
        bi, h, i = int(rng.integers(s.b)), int(rng.integers(s.hq)), int(rng.integers(s.n))
        g = oracle.kv_head_of(h, s.hq, s.hkv)
        rdq, _, _ = oracle.attention_head_bwd(x["q"][bi, :, h], x["k"][bi, :, g], x["v"][bi, :, g],
                                              x["do"][bi, :, h], s.causal, scale, rows=[i])
        got.append(dq[bi, i, h])
        ref.append(rdq[0])
    got, ref = np.array(got), np.array(ref)
    worst, _ = record(f"{s.name} n{s.n} causal={int(s.causal)} rows=24", "dq", got, ref, TOL_GRAD, s.dtype)
    log(f"  sampled dQ rows: max err {worst:.3e}")
    assert excess(got, ref, TOL_GRAD, s.dtype) <= 0
    # dK / dV of one whole K/V head (all query heads of its group summed)
    # wherever the oracle does that in seconds -- every workload up to
    # N = 16384, and the MQA group of 32 heads at N = 4096 -- else of 64 keys
    # of it (first and last keys, tile and block edges, random keys), each
    # summed over every query row
    rep = s.hq // s.hkv
    bi, g = int(rng.integers(s.b)), int(rng.integers(s.hkv))
    if s.n * s.n * rep <= 16384 * 16384 * 2:
        cols = np.arange(s.n)
        kw = {}
    else:
        fixed = [0, 1, 31, 32, 127, 128, s.n // 2, s.n - 129, s.n - 128, s.n - 2, s.n - 1]
        cols = np.unique(np.concatenate([fixed, rng.choice(s.n, 64 - len(fixed), replace=False)]))
        kw = {"cols": cols}
    rdk = np.zeros((len(cols), s.d))
    rdv = np.zeros((len(cols), s.d))
    for h in range(g * rep, (g + 1) * rep):
        _, a_, b_ = oracle.attention_head_bwd(x["q"][bi, :, h], x["k"][bi, :, g], x["v"][bi, :, g],
                                              x["do"][bi, :, h], s.causal, scale, **kw)
        rdk += a_
        rdv += b_
    tag = f"{s.name} n{s.n} causal={int(s.causal)}"
    tkv = tol_kv(s.hq, s.hkv)
    ek, _ = record(tag + f" keys={len(cols)}", "dk", dk[bi, cols, g], rdk, tkv, s.dtype)
    ev, _ = record(tag + f" keys={len(cols)}", "dv", dv[bi, cols, g], rdv, tkv, s.dtype)
    log(f"  K/V head (b={bi}, g={g}, {len(cols)} keys): max|ddK|={ek:.3e} max|ddV|={ev:.3e} (bound {tkv:.3f})")
    assert excess(dk[bi, cols, g], rdk, tkv, s.dtype) <= 0
    assert excess(dv[bi, cols, g], rdv, tkv, s.dtype) <= 0


# The stage entry points, enqueued in order (the last two either way round),
# are exactly attn_bwd.
@pytest.mark.parametrize("causal", [False, True])
def test_stages_match_whole_pass(gpu_device, causal):
    import torch
    import exact_io_aware_75_amd as ea

    b, n, hq, hkv, d = 2, 700, 4, 2, 128
    x = gen.make_inputs(b, n, hq, hkv, d, "bf16", cfg_id=61, seed=n)
    q, k, v, do = (gen.to_torch(x[t], "bf16", gpu_device) for t in ("q", "k", "v", "do"))
    scale = 1.0 / np.sqrt(d)
    o, lse = ea.forward(q, k, v, causal=causal, scale=scale)
    ws = torch.empty(ea.attn_bwd_workspace_bytes(b, n, hq, hkv, d), dtype=torch.uint8, device=gpu_device)

    def run(stages):
        g = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
        for st in stages:
            ea.attn_bwd(q, k, v, o, do, lse, *g, ws, causal, scale, stage=st)
        torch.cuda.synchronize()
        return [t.float().cpu().numpy() for t in g]

    whole = run(["attn_bwd"])
    for order in (["attn_bwd_preprocess", "attn_bwd_dkdv", "attn_bwd_dq"],
                  ["attn_bwd_preprocess", "attn_bwd_dq", "attn_bwd_dkdv"]):
        staged = run(order)
        for nm, a_, b_ in zip(("dq", "dk", "dv"), whole, staged):
            assert np.array_equal(a_, b_), (order, nm)
    log(f"stages causal={causal}: bitwise equal to attn_bwd in both orders")
