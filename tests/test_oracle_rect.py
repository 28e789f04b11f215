"""Pins for rectangular attention in the CPU fp64 oracle: Nq queries against
Nk keys, with a causal offset (query i sees key j iff j <= i + offset; by
default offset = Nk - Nq).

That is the shape one device computes when a sequence is split across
devices, whose partial results combine exactly through their LSEs.  The pins:
PyTorch's fp64 scaled_dot_product_attention with the explicit mask plus
autograd, central finite differences, the exact LSE merge of key shards back
into the whole, and the tail rows of square causal attention.
"""

import numpy as np
import pytest

import oracle
from oracle import attention as oa
from exact_io_aware_75_amd.inputs import make_inputs


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _torch_ref(q, k, v, do, causal, offset, scale):
    """Masked SDPA + autograd per head; rows with no allowed key are left out
    of the library call and set to O = 0, LSE = -inf, dQ = 0."""
    import torch

    b, nq, hq, d = q.shape
    nk, hkv = k.shape[1], k.shape[2]
    ok = np.ones((nq, nk), dtype=bool)
    if causal:
        ok = np.arange(nk)[None, :] <= np.arange(nq)[:, None] + offset
    rows = np.nonzero(ok.any(axis=1))[0]
    o = np.zeros((b, nq, hq, d)); lse = np.full((b, hq, nq), -np.inf)
    dq = np.zeros((b, nq, hq, d)); dk = np.zeros((b, nk, hkv, d)); dv = np.zeros((b, nk, hkv, d))
    am = torch.tensor(ok[rows])
    for bi in range(b):
        for h in range(hq):
            g = h // (hq // hkv)
            tq = torch.tensor(q[bi, rows, h]).requires_grad_()
            tk = torch.tensor(k[bi, :, g]).requires_grad_()
            tv = torch.tensor(v[bi, :, g]).requires_grad_()
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


@pytest.mark.parametrize("nq,nk,causal,offset", [
    (20, 50, True, None),     # bottom-right aligned
    (50, 20, True, None),     # more queries than keys: the first 30 rows see nothing
    (33, 33, True, -7),       # negative offset
    (17, 40, True, 5),
    (25, 60, False, None),
])
def test_matches_torch_masked_sdpa_fp64(nq, nk, causal, offset):
    b, hq, hkv, d = 2, 4, 2, 8
    q, do = _rand((b, nq, hq, d), nq), _rand((b, nq, hq, d), nq + 1)
    k, v = _rand((b, nk, hkv, d), nk + 2), _rand((b, nk, hkv, d), nk + 3)
    scale = 0.4
    o, lse = oracle.attention_fwd(q, k, v, causal, scale, causal_offset=offset)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, causal, scale, causal_offset=offset)
    off = nk - nq if offset is None else offset
    ro, rlse, rdq, rdk, rdv = _torch_ref(q, k, v, do, causal, off, scale)
    for a, r in ((o, ro), (dq, rdq), (dk, rdk), (dv, rdv)):
        assert np.abs(a - r).max() < 1e-12
    fin = np.isfinite(rlse)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.abs(lse[fin] - rlse[fin]).max() < 1e-12


@pytest.mark.parametrize("offset", [-2, 3])
def test_gradients_match_finite_differences(offset):
    """Brute force at Nq = 5, Nk = 7, d = 3 (offset -2 leaves rows 0-1 empty)."""
    q, do = _rand((1, 5, 2, 3), 41), _rand((1, 5, 2, 3), 42)
    k, v = _rand((1, 7, 1, 3), 43), _rand((1, 7, 1, 3), 44)
    scale, hstep = 0.8, 1e-6

    def loss(q_, k_, v_):
        o, _ = oracle.attention_fwd(q_, k_, v_, True, scale, causal_offset=offset)
        return float((o * do).sum())

    grads = oracle.attention_bwd(q, k, v, do, True, scale, causal_offset=offset)
    for which in range(3):
        base = [q, k, v]
        x = base[which]
        g = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += hstep
            xm[idx] -= hstep
            ap, am = list(base), list(base)
            ap[which], am[which] = xp, xm
            g[idx] = (loss(*ap) - loss(*am)) / (2 * hstep)
        assert np.abs(grads[which] - g).max() / np.abs(g).max() < 1e-6


@pytest.mark.parametrize("causal", [False, True])
def test_key_shards_merge_to_the_whole(causal):
    """Split the keys into shards at positions p_s: each shard's attention
    (offset shifted by -p_s) merged through LSE = ln sum exp(LSE_s) and
    O = sum exp(LSE_s - LSE) O_s gives attention over all keys."""
    n = 70
    x = make_inputs(1, n, 2, 1, 8, "bf16", cfg_id=81)
    q, k, v = (x[t].astype(np.float64) for t in ("q", "k", "v"))
    o, lse = oracle.attention_fwd(q, k, v, causal, 0.3)
    cuts = [0, 23, 45, n]
    parts = []
    for a_, b_ in zip(cuts[:-1], cuts[1:]):
        parts.append(oracle.attention_fwd(q, k[:, a_:b_], v[:, a_:b_], causal, 0.3, causal_offset=-a_))
    lses = np.stack([p[1] for p in parts])                  # [S, B, H, N]
    m = np.max(lses, axis=0)
    w = np.exp(lses - m)                                      # exp(-inf) = 0 for empty shards
    merged_lse = m + np.log(w.sum(axis=0))
    merged_o = sum(np.exp(p[1] - merged_lse).transpose(0, 2, 1)[..., None] * p[0] for p in parts)
    np.testing.assert_allclose(merged_lse, lse, atol=1e-12)
    np.testing.assert_allclose(merged_o, o, atol=1e-12)


def test_query_tail_of_square_causal():
    """The last Nq queries of square causal attention over Nk keys are the
    rectangular case with the default offset Nk - Nq."""
    nk, nq = 60, 19
    x = make_inputs(1, nk, 2, 2, 8, "bf16", cfg_id=80)
    q, k, v, do = (x[t].astype(np.float64) for t in ("q", "k", "v", "do"))
    o, lse = oracle.attention_fwd(q, k, v, True, 0.3)
    dq, _, _ = oracle.attention_bwd(q, k, v, do, True, 0.3)
    ot, lset = oracle.attention_fwd(q[:, nk - nq:], k, v, True, 0.3)
    dqt, _, _ = oracle.attention_bwd(q[:, nk - nq:], k, v, do[:, nk - nq:], True, 0.3)
    np.testing.assert_allclose(ot, o[:, nk - nq:], atol=1e-14)
    np.testing.assert_allclose(lset, lse[:, :, nk - nq:], atol=1e-14)
    np.testing.assert_allclose(dqt, dq[:, nk - nq:], atol=1e-14)


def test_planted_offset_sign_is_caught(monkeypatch):
    real = oa._allowed
    monkeypatch.setattr(oa, "_allowed", lambda rows, n, causal, hm=None, block=128, offset=0:
                        real(rows, n, causal, hm, block, -offset))
    with pytest.raises(AssertionError):
        test_matches_torch_masked_sdpa_fp64(20, 50, True, None)
