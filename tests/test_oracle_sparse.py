"""Pins for the block-sparse part of the CPU fp64 oracle.

Block-sparse attention is the variant the FlashAttention-1 news page
benchmarks beside the dense method (its paragraph on runtime and memory
against the A100 baselines).  The pages print no definition, so the oracle
reads it as attention restricted to the (query block, key block) pairs a block
mask allows, combined with the causal mask by AND; a row with no allowed key
has O = 0, LSE = -inf and no gradient.  Each test ties that to something other
than the oracle's own dense path alone: PyTorch's fp64 masked
scaled_dot_product_attention and autograd, central finite differences,
closed forms and the tiled online-softmax model with block skipping.  Planted
mistakes at the end check that the pins catch the usual slips.
"""

import numpy as np
import pytest

import oracle
from oracle import attention as oa
from exact_io_aware_75_amd.inputs import make_inputs


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _random_mask(hm, nb, seed, density=0.5, empty_row=None):
    m = (np.random.default_rng(seed).random((hm, nb, nb)) < density).astype(np.uint8)
    if empty_row is not None:
        m[:, empty_row, :] = 0
    return m


def _element_mask(head_mask, n, block, causal):
    idx = np.arange(n) // block
    ok = np.asarray(head_mask)[idx[:, None], idx[None, :]] != 0
    if causal:
        ok &= np.arange(n)[None, :] <= np.arange(n)[:, None]
    return ok


def _torch_masked_ref(q, k, v, do, block_mask, block, causal, scale):
    """PyTorch CPU fp64 scaled_dot_product_attention with an explicit boolean
    mask, plus autograd, head by head.  Rows with no allowed key are left out
    of the library call (it returns NaN for them) and set to the reading:
    O = 0, LSE = -inf, dQ = 0; rows are independent, so leaving them out does
    not change the other rows or dK / dV."""
    import torch

    b, n, hq, d = q.shape
    hkv = k.shape[2]
    o = np.zeros((b, n, hq, d)); lse = np.full((b, hq, n), -np.inf)
    dq = np.zeros((b, n, hq, d)); dk = np.zeros((b, n, hkv, d)); dv = np.zeros((b, n, hkv, d))
    for bi in range(b):
        for h in range(hq):
            g = h // (hq // hkv)
            hm = block_mask[0] if block_mask.shape[0] == 1 else block_mask[g]
            ok = _element_mask(hm, n, block, causal)
            rows = np.nonzero(ok.any(axis=1))[0]
            if len(rows) == 0:
                continue
            tq = torch.tensor(q[bi, rows, h]).requires_grad_()
            tk = torch.tensor(k[bi, :, g]).requires_grad_()
            tv = torch.tensor(v[bi, :, g]).requires_grad_()
            am = torch.tensor(ok[rows])
            out = torch.nn.functional.scaled_dot_product_attention(
                tq[None], tk[None], tv[None], attn_mask=am[None], scale=scale)[0]
            out.backward(torch.tensor(do[bi, rows, h]))
            s = (scale * (tq.detach() @ tk.detach().T)).masked_fill(~am, float("-inf"))
            o[bi, rows, h] = out.detach().numpy()
            lse[bi, h, rows] = torch.logsumexp(s, dim=-1).numpy()
            dq[bi, rows, h] = tq.grad.numpy()
            dk[bi, :, g] += tk.grad.numpy()
            dv[bi, :, g] += tv.grad.numpy()
    return o, lse, dq, dk, dv


@pytest.mark.parametrize("b,n,hq,hkv,d,block,hm,causal", [
    (1, 40, 2, 2, 8, 8, 1, False),     # ragged last block, shared mask
    (2, 37, 4, 2, 16, 8, 2, True),     # per-K/V-head masks, causal, ragged
    (1, 64, 4, 1, 8, 16, 1, True),     # MQA
    (1, 50, 3, 3, 8, 16, 3, False),
])
def test_matches_torch_masked_sdpa_fp64(b, n, hq, hkv, d, block, hm, causal):
    x = make_inputs(b, n, hq, hkv, d, "bf16", cfg_id=88, seed=n)
    q, k, v, do = (x[t].astype(np.float64) for t in ("q", "k", "v", "do"))
    nb = -(-n // block)
    mask = _random_mask(hm, nb, seed=n + hm, empty_row=1)  # row block 1 has no allowed key
    scale = 1.0 / np.sqrt(d)
    o, lse = oracle.attention_fwd(q, k, v, causal, scale, block_mask=mask, block=block)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, causal, scale, block_mask=mask, block=block)
    ro, rlse, rdq, rdk, rdv = _torch_masked_ref(q, k, v, do, mask, block, causal, scale)
    for a, r in ((o, ro), (dq, rdq), (dk, rdk), (dv, rdv)):
        assert np.abs(a - r).max() < 1e-12
    fin = np.isfinite(rlse)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.abs(lse[fin] - rlse[fin]).max() < 1e-12
    # the empty row block: O = 0, LSE = -inf, dQ = 0
    er = slice(block, 2 * block)
    assert (o[:, er] == 0).all() and (lse[:, :, er] == -np.inf).all() and (dq[:, er] == 0).all()


def _loss(q, k, v, do, causal, scale, mask, block):
    o, _ = oracle.attention_fwd(q, k, v, causal, scale, block_mask=mask, block=block)
    return float((o * do).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_sparse_gradients_match_finite_differences(causal):
    """Brute force at N = 8, d = 4, blocks of 2, with one empty row block."""
    q, k, v, do = _rand((1, 8, 2, 4), 21), _rand((1, 8, 1, 4), 22), _rand((1, 8, 1, 4), 23), _rand((1, 8, 2, 4), 24)
    mask = np.array([[[1, 0, 0, 1], [0, 0, 0, 0], [1, 1, 0, 0], [0, 1, 1, 1]]], dtype=np.uint8)
    scale, block, hstep = 0.7, 2, 1e-6
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, causal, scale, block_mask=mask, block=block)
    for which, an in enumerate((dq, dk, dv)):
        base = [q, k, v]
        x = base[which]
        g = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += hstep
            xm[idx] -= hstep
            ap, am = list(base), list(base)
            ap[which], am[which] = xp, xm
            g[idx] = (_loss(*ap, do, causal, scale, mask, block) - _loss(*am, do, causal, scale, mask, block)) / (2 * hstep)
        assert np.abs(an - g).max() / np.abs(g).max() < 1e-6


@pytest.mark.parametrize("causal", [False, True])
def test_full_mask_is_dense(causal):
    x = make_inputs(1, 45, 2, 1, 8, "bf16", cfg_id=87)
    ones = np.ones((1, 6, 6), dtype=np.uint8)
    o, lse = oracle.attention_fwd(x["q"], x["k"], x["v"], causal, 0.3, block_mask=ones, block=8)
    od, lsed = oracle.attention_fwd(x["q"], x["k"], x["v"], causal, 0.3)
    assert np.array_equal(o, od) and np.array_equal(lse, lsed)


def test_lower_block_triangle_with_causal_is_causal():
    x = make_inputs(1, 45, 2, 2, 8, "bf16", cfg_id=86)
    tril = np.tril(np.ones((6, 6), dtype=np.uint8))[None]
    o, lse = oracle.attention_fwd(x["q"], x["k"], x["v"], True, 0.3, block_mask=tril, block=8)
    od, lsed = oracle.attention_fwd(x["q"], x["k"], x["v"], True, 0.3)
    assert np.array_equal(o, od) and np.array_equal(lse, lsed)


def test_block_diagonal_mask_is_independent_segments():
    """Closed form: a block-diagonal mask makes each block its own sequence,
    whose attention is then softmax(scale Q_b K_b^T) V_b written out with no
    masking at all."""
    n, d, block = 30, 8, 8
    x = make_inputs(1, n, 1, 1, d, "bf16", cfg_id=85)
    q, k, v = (x[t][0, :, 0].astype(np.float64) for t in ("q", "k", "v"))
    eye = np.eye(4, dtype=np.uint8)[None]
    o, lse = oracle.attention_fwd(x["q"], x["k"], x["v"], False, 0.5, block_mask=eye, block=block)
    for s0 in range(0, n, block):
        sl = slice(s0, min(s0 + block, n))
        s = 0.5 * (q[sl] @ k[sl].T)
        e = np.exp(s - s.max(axis=1, keepdims=True))
        np.testing.assert_allclose(o[0, sl, 0], (e / e.sum(axis=1, keepdims=True)) @ v[sl], atol=1e-13)
        np.testing.assert_allclose(lse[0, 0, sl], np.log(np.exp(s).sum(axis=1)), atol=1e-12)


def test_zero_scale_sparse_is_mean_over_allowed_keys():
    """Closed form: at scale 0, O_i is the mean of V over row i's allowed keys
    and LSE_i = ln(count)."""
    n, d, block = 33, 4, 8
    x = make_inputs(1, n, 1, 1, d, "bf16", cfg_id=84)
    mask = _random_mask(1, 5, seed=3)
    mask[0, :, 0] = 1  # every row block sees block 0
    for causal in (False, True):
        o, lse = oracle.attention_fwd(x["q"], x["k"], x["v"], causal, 0.0, block_mask=mask, block=block)
        ok = _element_mask(mask[0], n, block, causal)
        v = x["v"][0, :, 0].astype(np.float64)
        np.testing.assert_allclose(o[0, :, 0], (ok @ v) / ok.sum(axis=1)[:, None], atol=1e-13)
        np.testing.assert_allclose(lse[0, 0], np.log(ok.sum(axis=1)), atol=1e-13)


@pytest.mark.parametrize("n,bm,bn,block,causal", [
    (64, 16, 16, 16, False), (64, 16, 16, 32, True), (100, 16, 32, 32, True), (129, 32, 16, 32, False),
])
def test_tiled_block_skipping_equals_standard(n, bm, bn, block, causal):
    """The tiled model that never visits zero blocks equals the plain sparse
    definition, and visits exactly the allowed tiles."""
    x = make_inputs(1, n, 1, 1, 16, "bf16", cfg_id=83, seed=n)
    q, k, v = x["q"][0, :, 0], x["k"][0, :, 0], x["v"][0, :, 0]
    nb = -(-n // block)
    mask = _random_mask(1, nb, seed=n, empty_row=min(1, nb - 1))[0]
    mask[0, 0] = 1  # at least one row block with allowed keys
    o, lse, visited = oracle.tiled_attention_fwd(q, k, v, causal, 0.2, bm=bm, bn=bn, head_mask=mask, block=block)
    o_ref, lse_ref = oracle.attention_head_fwd(q, k, v, causal, 0.2, head_mask=mask, block=block)
    assert np.abs(o - o_ref).max() < 1e-12
    assert np.array_equal(np.isfinite(lse), np.isfinite(lse_ref))
    f = np.isfinite(lse_ref)
    assert np.abs(lse[f] - lse_ref[f]).max() < 1e-12
    expect = 0
    for i0 in range(0, n, bm):
        for j0 in range(0, n, bn):
            if mask[i0 // block, j0 // block] and not (causal and j0 > min(i0 + bm, n) - 1):
                expect += 1
    assert visited == expect


def test_mask_shape_is_checked():
    x = make_inputs(1, 20, 2, 2, 4, "bf16", cfg_id=82)
    with pytest.raises(ValueError):
        oracle.attention_fwd(x["q"], x["k"], x["v"], False, 0.5, block_mask=np.ones((1, 2, 3)), block=8)
    with pytest.raises(ValueError):  # neither 1 nor Hkv = 2 masks
        oracle.attention_fwd(x["q"], x["k"], x["v"], False, 0.5, block_mask=np.ones((3, 3, 3)), block=8)


# ---- planted mistakes: each mutated oracle must fail at least one pin ----

def test_planted_transposed_mask_is_caught(monkeypatch):
    real = oa._allowed

    def transposed(rows, n, causal, head_mask=None, block=128, offset=0):
        hm = None if head_mask is None else np.asarray(head_mask).T
        return real(rows, n, causal, hm, block, offset)

    monkeypatch.setattr(oa, "_allowed", transposed)
    with pytest.raises(AssertionError):
        test_matches_torch_masked_sdpa_fp64(1, 40, 2, 2, 8, 8, 1, False)


def test_planted_mask_ignored_in_backward_is_caught(monkeypatch):
    real = oa.attention_head_bwd
    monkeypatch.setattr(oa, "attention_head_bwd",
                        lambda *a, head_mask=None, block=128, **kw: real(*a, block=block, **kw))
    with pytest.raises(AssertionError):
        test_sparse_gradients_match_finite_differences(False)
