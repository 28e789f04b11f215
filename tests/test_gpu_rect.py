"""GPU parity of rectangular attention (attn_fwd_rect / attn_bwd_rect through
the C ABI) against the CPU fp64 oracle: Nq queries against Nk keys with a
causal offset (query i sees key j iff j <= i + offset; default Nk - Nq).

This is the shape one device computes when the sequence is split across
devices (the pages parallelise over the sequence): small shapes element by
element (more keys than queries, more queries than keys, negative offsets
that leave rows without keys, offsets past either end), an exact LSE merge of
key shards computed separately on the GPU back into whole causal attention,
and a full-size shard (8192 queries against 65536 keys) on sampled rows and
one whole head.
"""

import numpy as np
import pytest

import oracle
from exact_io_aware_75_amd import inputs as gen
from gpu_util import TOL_GRAD, TOL_LSE, TOL_O, excess, log, make_rect_inputs, max_err, run_fwd_bwd

pytestmark = pytest.mark.gpu


def _check(x, out, causal, offset, scale, tag, dtype):
    o, lse, dq, dk, dv = out
    ro, rlse = oracle.attention_fwd(x["q"], x["k"], x["v"], causal, scale, causal_offset=offset)
    rdq, rdk, rdv = oracle.attention_bwd(x["q"], x["k"], x["v"], x["do"], causal, scale, causal_offset=offset)
    fin = np.isfinite(rlse)
    errs = {n: max_err(a, r) for n, a, r in (("o", o, ro), ("lse", lse[fin], rlse[fin]), ("dq", dq, rdq),
                                             ("dk", dk, rdk), ("dv", dv, rdv))}
    log(f"{tag}: " + "  ".join(f"{n}={e:.2e}(|ref| {m:.2f})" for n, (e, m) in errs.items())
        + f"  empty rows {int((~fin).sum())}")
    for t in (o, dq, dk, dv):
        assert np.isfinite(t).all()
    assert np.array_equal(np.isfinite(lse), fin) and (lse[~fin] == -np.inf).all()
    assert excess(o, ro, TOL_O, dtype) <= 0, (tag, "o", errs["o"])
    assert errs["lse"][0] <= TOL_LSE
    for n, a_, r_ in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        assert excess(a_, r_, TOL_GRAD, dtype) <= 0, (tag, n, errs[n])
    for bi, h, i in np.transpose(np.nonzero(~fin)):
        assert (o[bi, i, h] == 0).all() and (dq[bi, i, h] == 0).all()


SMALL = [
    # b, nq, nk, hq, hkv, d, dtype, causal, offset
    (1, 100, 300, 2, 2, 128, "bf16", True, None),    # bottom-right aligned
    (1, 300, 100, 2, 1, 64, "bf16", True, None),     # offset -200: rows 0..199 see no key
    (2, 129, 257, 4, 2, 128, "fp16", True, -50),
    (1, 200, 640, 2, 2, 256, "bf16", True, 77),
    (1, 64, 1000, 4, 4, 64, "bf16", False, None),
    (1, 1000, 64, 2, 2, 128, "bf16", False, None),
    (1, 33, 33, 2, 2, 128, "bf16", True, 5),         # square, shifted diagonal
    (1, 500, 200, 4, 1, 128, "bf16", True, 1000),    # past the last key: every key visible
    (1, 300, 300, 2, 2, 64, "bf16", True, -10000),   # before the first key: no row sees a key
    (1, 520, 1300, 8, 2, 256, "fp16", True, None),
    # diagonals at unaligned offsets over many key tiles: a wavefront's rows
    # can cross two masked tiles, with 0, 1 or 2 unmasked tiles between the
    # paired steady-state steps and its last tile
    (1, 400, 1100, 2, 2, 64, "bf16", True, 333),
    (2, 700, 900, 4, 2, 64, "fp16", True, 40),
    (1, 450, 1000, 2, 2, 128, "bf16", True, 211),
    (1, 260, 2000, 2, 1, 128, "fp16", True, 1650),
]


@pytest.mark.parametrize("b,nq,nk,hq,hkv,d,dtype,causal,offset", SMALL)
def test_small_shapes(gpu_device, b, nq, nk, hq, hkv, d, dtype, causal, offset):
    x = make_rect_inputs(b, nq, nk, hq, hkv, d, dtype, cfg_id=41, seed=nq + nk)
    scale = 1.0 / np.sqrt(d)
    tag = f"rect b{b} nq{nq} nk{nk} hq{hq} hkv{hkv} d{d} {dtype} causal={causal} offset={offset}"
    log(tag)
    out = run_fwd_bwd(x, dtype, causal, scale, gpu_device, causal_offset=offset)
    _check(x, out, causal, offset, scale, tag, dtype)



# scale = 0 with a causal offset that is not a multiple of 32: rows with no
# key sit in the same wavefronts as rows with keys, and diagonal tiles are
# fully masked for some rows, where the scaled row max would be -inf * 0.
# With scale 0 every visible key has probability 1 / (number visible).
@pytest.mark.parametrize("b,nq,nk,hq,hkv,d,dtype,offset", [
    (1, 300, 400, 2, 1, 128, "bf16", -45),
    (1, 257, 700, 2, 2, 64, "fp16", -77),
    (1, 200, 500, 2, 2, 256, "bf16", -13),
])
def test_scale_zero_with_empty_rows(gpu_device, b, nq, nk, hq, hkv, d, dtype, offset):
    x = make_rect_inputs(b, nq, nk, hq, hkv, d, dtype, cfg_id=43, seed=nq)
    tag = f"rect scale=0 b{b} nq{nq} nk{nk} hq{hq} hkv{hkv} d{d} {dtype} offset={offset}"
    log(tag)
    out = run_fwd_bwd(x, dtype, True, 0.0, gpu_device, causal_offset=offset)
    _check(x, out, True, offset, 0.0, tag, dtype)
    o, lse = out[0], out[1]
    v = x["v"].astype(np.float64)
    for i in (0, -offset - 1, -offset, -offset + 1, nq - 1):  # closed form: prefix means of V
        if 0 <= i < nq:
            nvis = min(max(i + offset + 1, 0), nk)
            if nvis == 0:
                assert (o[:, i] == 0).all() and (lse[:, :, i] == -np.inf).all()
            else:
                rep = hq // hkv
                mean = np.repeat(v[:, :nvis].mean(axis=1), rep, axis=1)
                assert np.abs(o[:, i] - mean).max() <= TOL_O
                assert np.abs(lse[:, :, i] - np.log(nvis)).max() <= TOL_LSE

def test_square_offset_zero_is_attn_fwd_bitwise(gpu_device):
    import torch
    import exact_io_aware_75_amd as ea

    x = gen.make_inputs(1, 700, 4, 2, 128, "bf16", cfg_id=42)
    q, k, v = (gen.to_torch(x[t], "bf16", gpu_device) for t in ("q", "k", "v"))
    o1, l1 = torch.empty_like(q), torch.empty((1, 4, 700), dtype=torch.float32, device=gpu_device)
    o2, l2 = torch.empty_like(q), torch.empty_like(l1)
    ea.attn_fwd(q, k, v, o1, l1, True, 0.1)
    st = ea.load_library().attn_fwd_rect(q.data_ptr(), k.data_ptr(), v.data_ptr(), o2.data_ptr(), l2.data_ptr(),
                                         1, 700, 700, 4, 2, 128, 1, 1, 0, 0.1, None)
    torch.cuda.synchronize()
    assert st == 0
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shards_merge_to_whole_attention(gpu_device, causal):
    """Context-parallel use: the keys of one sequence in 4 shards, each shard
    a separate rectangular call with offset -start; the partial (O, LSE) merge
    exactly (LSE = ln sum exp LSE_s, O = sum exp(LSE_s - LSE) O_s) into the
    oracle's attention over all keys."""
    n, hq, hkv, d = 2048, 4, 2, 128
    x = gen.make_inputs(1, n, hq, hkv, d, "bf16", cfg_id=43)
    cuts = [0, 300, 1024, 1500, n]
    parts = []
    for a_, b_ in zip(cuts[:-1], cuts[1:]):
        xs = {"q": x["q"], "k": x["k"][:, a_:b_], "v": x["v"][:, a_:b_], "do": x["do"]}
        o, lse, _, _, _ = run_fwd_bwd(xs, "bf16", causal, 1.0 / np.sqrt(d), gpu_device, causal_offset=-a_)
        parts.append((o, lse))
    lses = np.stack([p[1] for p in parts])
    m = lses.max(axis=0)
    lse = m + np.log(np.exp(lses - m).sum(axis=0))
    o = sum(np.exp(p[1] - lse).transpose(0, 2, 1)[..., None] * p[0] for p in parts)
    ro, rlse = oracle.attention_fwd(x["q"], x["k"], x["v"], causal, 1.0 / np.sqrt(d))
    log(f"shard merge causal={causal}: o err {max_err(o, ro)[0]:.2e}, lse err {np.abs(lse - rlse).max():.2e}")
    assert excess(o, ro, TOL_O, "bf16") <= 0
    assert np.abs(lse - rlse).max() <= TOL_LSE


def test_full_size_shard(gpu_device):
    """One device's share of a 65536-token causal sequence split 8 ways: its
    8192 queries (the last shard) against all 65536 keys, B = 1, H = 8, d = 128."""
    b, nq, nk, h, d = 1, 8192, 65536, 8, 128
    x = make_rect_inputs(b, nq, nk, h, h, d, "bf16", cfg_id=44)
    scale = 1.0 / np.sqrt(d)
    log(f"full-size shard fwd+bwd: Nq={nq} Nk={nk} H={h} d={d} causal, offset Nk - Nq")
    o, lse, dq, dk, dv = run_fwd_bwd(x, "bf16", True, scale, gpu_device)
    for t in (o, lse, dq, dk, dv):
        assert np.isfinite(t).all()
    rng = np.random.default_rng(11)
    worst = {"o": -1.0, "lse": 0.0, "dq": -1.0}
    for _ in range(12):
        hh, i = int(rng.integers(h)), int(rng.integers(nq))
        ro, rlse = oracle.attention_head_fwd(x["q"][0, :, hh], x["k"][0, :, hh], x["v"][0, :, hh], True, scale,
                                             rows=[i])
        rdq, _, _ = oracle.attention_head_bwd(x["q"][0, :, hh], x["k"][0, :, hh], x["v"][0, :, hh],
                                              x["do"][0, :, hh], True, scale, rows=[i])
        worst["o"] = max(worst["o"], excess(o[0, i, hh], ro[0], TOL_O, "bf16"))
        worst["lse"] = max(worst["lse"], abs(lse[0, hh, i] - rlse[0]))
        worst["dq"] = max(worst["dq"], excess(dq[0, i, hh], rdq[0], TOL_GRAD, "bf16"))
    log(f"  sampled rows: excess o {worst['o']:.2e}, lse err {worst['lse']:.2e}, excess dq {worst['dq']:.2e}")
    assert worst["o"] <= 0 and worst["lse"] <= TOL_LSE and worst["dq"] <= 0
    # dK / dV of one head on a sample of keys: every query row contributes, so
    # the oracle runs the head's whole backward pass once
    hh = int(rng.integers(h))
    _, rdk, rdv = oracle.attention_head_bwd(x["q"][0, :, hh], x["k"][0, :, hh], x["v"][0, :, hh],
                                            x["do"][0, :, hh], True, scale)
    log(f"  head {hh}: max|ddK|={max_err(dk[0, :, hh], rdk)[0]:.3e} max|ddV|={max_err(dv[0, :, hh], rdv)[0]:.3e}")
    assert excess(dk[0, :, hh], rdk, TOL_GRAD, "bf16") <= 0
    assert excess(dv[0, :, hh], rdv, TOL_GRAD, "bf16") <= 0


SPLIT = [
    # b, nq, nk, hq, hkv, d, dtype, causal, offset, splits
    (1, 1, 5000, 4, 1, 128, "bf16", False, None, 8),
    (2, 17, 3000, 2, 2, 64, "bf16", True, None, 5),
    (1, 128, 8192, 8, 2, 128, "fp16", True, None, 16),
    (1, 300, 1000, 2, 2, 256, "bf16", True, -100, 3),
    (1, 64, 700, 2, 1, 128, "bf16", False, None, 40),   # more splits than 128-key runs: empty splits
    (1, 100, 100, 2, 2, 64, "bf16", True, None, 1),
]


@pytest.mark.parametrize("b,nq,nk,hq,hkv,d,dtype,causal,offset,splits", SPLIT)
def test_splitkv_matches_oracle(gpu_device, b, nq, nk, hq, hkv, d, dtype, causal, offset, splits):
    import torch
    import exact_io_aware_75_amd as ea

    x = make_rect_inputs(b, nq, nk, hq, hkv, d, dtype, cfg_id=45, seed=nq + splits)
    scale = 1.0 / np.sqrt(d)
    tag = f"split-KV b{b} nq{nq} nk{nk} hq{hq} hkv{hkv} d{d} {dtype} causal={causal} offset={offset} splits={splits}"
    log(tag)
    q, k, v = (gen.to_torch(x[t], dtype, gpu_device) for t in ("q", "k", "v"))
    o, lse = ea.forward(q, k, v, causal=causal, scale=scale, causal_offset=offset, num_splits=splits)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    ro, rlse = oracle.attention_fwd(x["q"], x["k"], x["v"], causal, scale, causal_offset=offset)
    fin = np.isfinite(rlse)
    log(f"  o err {max_err(o, ro)[0]:.2e}  lse err {np.abs(lse[fin] - rlse[fin]).max() if fin.any() else 0:.2e}"
        f"  empty rows {int((~fin).sum())}")
    assert np.isfinite(o).all()
    assert excess(o, ro, TOL_O, dtype) <= 0
    assert np.array_equal(np.isfinite(lse), fin)
    if fin.any():
        assert np.abs(lse[fin] - rlse[fin]).max() <= TOL_LSE
