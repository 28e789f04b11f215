"""Plain fp64 attention: the definition the tiled method must reproduce.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

Sources.  The pages state that the IO-aware method is exact -- mathematically
equivalent, up to numerical precision, to standard attention (FlashAttention-2
review, "Введение" section; FlashAttention-1 news page, "FlashAttention"
section, which calls it an "exact attention algorithm") -- and that standard
attention materialises the N x N score matrix (FlashAttention-1 news page,
"FlashAttention" section; FlashAttention-2 announcement, "具体实现" section).
The backward pass recomputes that matrix block by block (same sections); here
it is recomputed whole, row chunk by row chunk, and differentiated
analytically.  The pages print no formulas, so the formulas below are the
textbook definition of softmax attention and its gradient:

forward, for one query head h with key/value head g:
    S[i, j]   = scale * <Q[i], K[j]>
    allowed   = (not causal) or (j <= i)          rows are queries, columns keys
    m_i       = max_{allowed j} S[i, j]
    e[i, j]   = exp(S[i, j] - m_i) if allowed else 0
    l_i       = sum_j e[i, j]
    P[i, j]   = e[i, j] / l_i
    O[i]      = sum_j P[i, j] V[j]
    LSE[i]    = m_i + ln l_i                      natural logarithm

backward, with upstream gradient dO (loss L = sum O * dO):
    dP[i, j]  = <dO[i], V[j]>
    D_i       = sum_j P[i, j] dP[i, j]            by this definition, not dO . O
    dS[i, j]  = P[i, j] (dP[i, j] - D_i)
    dQ[i]     = scale * sum_j dS[i, j] K[j]
    dK[j]     = scale * sum_{h in group} sum_i dS[i, j] Q[i]
    dV[j]     = sum_{h in group} sum_i P[i, j] dO[i]

Block-sparse attention (the variant the FlashAttention-1 news page benchmarks
as "block-sparse FlashAttention", in the paragraph on runtime and memory
against the A100 baselines; no definition is printed) restricts `allowed`
further by a block mask over (query block, key block) pairs:
    allowed   = allowed and mask[i // block, j // block]
with block = 128 rows by 128 keys on the GPU; every other formula is
unchanged.  A row whose allowed set is empty gets O = 0, LSE = -inf and
dQ = 0, and adds nothing to dK or dV.

Rectangular attention (Nq queries, Nk keys; the shard shape of a sequence
split across devices) with a causal offset: query i may attend key j iff
    j <= i + offset,
by default offset = Nk - Nq, which aligns the last query with the last key
(for Nq = Nk the usual causal mask).  Rows whose i + offset is negative have
no allowed key.  Each device's partial results for one query shard combine
exactly through their LSEs: LSE = ln sum_p exp(LSE_p) and
O = sum_p exp(LSE_p - LSE) O_p.

Readings where the pages are silent:
  * causal orientation: query i may attend key j iff j <= i (the pages only
    say the masked triangle is skipped rather than computed and zeroed;
    FlashAttention-2 review, "Алгоритм вычисления" subsection);
  * GQA/MQA (named, not defined, in the FlashAttention-2 announcement,
    "具体实现" section): query head h reads K/V head h // (Hq / Hkv), i.e.
    consecutive query heads share a K/V head;
  * a row with no allowed key (impossible when Nq = Nk) has O = 0 and
    LSE = -inf;
  * LSE is the natural-log log-sum-exp of the scaled scores.

Layouts: Q, O, dO, dQ are [B, N, Hq, d]; K, V, dK, dV are [B, N, Hkv, d];
LSE is [B, Hq, N].  Every input is upcast to float64; nothing is rounded on
the way out.
"""

from __future__ import annotations

import numpy as np

_F = np.float64


def kv_head_of(h: int, hq: int, hkv: int) -> int:
    """K/V head read by query head ``h`` (consecutive groups of Hq/Hkv heads)."""
    if hkv <= 0 or hq % hkv != 0:
        raise ValueError(f"Hq={hq} must be a positive multiple of Hkv={hkv}")
    return h // (hq // hkv)


def _allowed(rows: np.ndarray, n_keys: int, causal: bool, head_mask=None, block: int = 128,
             offset: int = 0) -> np.ndarray:
    """Boolean [len(rows), n_keys] mask: key j visible to query row i.

    Causal: j <= i + offset.  ``head_mask`` (optional, [ceil(Nq / block),
    ceil(Nk / block)]) is the block mask of the head: key j is visible only if
    its (row block, key block) entry is nonzero.
    """
    cols = np.arange(n_keys)
    if not causal:
        ok = np.ones((len(rows), n_keys), dtype=bool)
    else:
        ok = cols[None, :] <= rows[:, None] + offset
    if head_mask is not None:
        hm = np.asarray(head_mask) != 0
        ok = ok & hm[rows[:, None] // block, cols[None, :] // block]
    return ok


def _row_softmax(s: np.ndarray, allowed: np.ndarray):
    """Max-subtracted softmax of each row over its allowed entries.

    Returns (P, lse).  Rows with no allowed entry give P = 0 and lse = -inf.
    """
    masked = np.where(allowed, s, -np.inf)
    m = masked.max(axis=1)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.where(allowed, np.exp(masked - m_safe[:, None]), 0.0)
    l = e.sum(axis=1)
    l_safe = np.where(empty, 1.0, l)
    p = e / l_safe[:, None]
    lse = np.where(empty, -np.inf, m_safe + np.log(l_safe))
    return p, lse


def _offset(causal_offset, n_q: int, n_k: int) -> int:
    """Causal offset: default Nk - Nq (last query aligned with last key)."""
    return n_k - n_q if causal_offset is None else int(causal_offset)


def attention_head_probs(q, k, causal: bool, scale: float, head_mask=None, block: int = 128,
                         causal_offset=None) -> np.ndarray:
    """Full probability matrix P [Nq, Nk] of one head (small inputs only)."""
    q = np.asarray(q, dtype=_F)
    k = np.asarray(k, dtype=_F)
    s = scale * (q @ k.T)
    off = _offset(causal_offset, q.shape[0], k.shape[0])
    p, _ = _row_softmax(s, _allowed(np.arange(q.shape[0]), k.shape[0], causal, head_mask, block, off))
    return p


def attention_head_fwd(q, k, v, causal: bool, scale: float, rows=None, chunk: int = 512,
                       head_mask=None, block: int = 128, causal_offset=None):
    """O and LSE of one head for the query ``rows`` (default: all rows).

    q: [Nq, d] all query rows of the head; k, v: [Nk, d] of its K/V head;
    head_mask: optional block mask of the head (see ``_allowed``);
    causal_offset: see ``_allowed`` (default Nk - Nq).
    Rows are independent, so they are processed in chunks of whole rows.
    """
    q = np.asarray(q, dtype=_F)
    k = np.asarray(k, dtype=_F)
    v = np.asarray(v, dtype=_F)
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    off = _offset(causal_offset, q.shape[0], k.shape[0])
    o = np.empty((len(rows), v.shape[1]), dtype=_F)
    lse = np.empty(len(rows), dtype=_F)
    for c0 in range(0, len(rows), chunk):
        r = rows[c0:c0 + chunk]
        s = scale * (q[r] @ k.T)
        p, lse[c0:c0 + chunk] = _row_softmax(s, _allowed(r, k.shape[0], causal, head_mask, block, off))
        o[c0:c0 + chunk] = p @ v
    return o, lse


def attention_head_bwd(q, k, v, do, causal: bool, scale: float, rows=None, chunk: int = 512,
                       head_mask=None, block: int = 128, causal_offset=None, cols=None):
    """Gradients of L = sum(O * dO) for one query head.

    Returns (dq_rows, dk, dv): dq for the query ``rows`` (default: all) and this
    head's whole contribution to dK and dV of its K/V head.  dK/dV need every
    query row, so they are only returned when ``rows`` is None.  ``cols``
    (optional key indices) restricts dK/dV to those keys: the same sums over
    every query row, kept only for the listed columns ([len(cols), d] each),
    so that long sequences can be checked key by key; dq is then not formed
    (returned as None).
    """
    q = np.asarray(q, dtype=_F)
    k = np.asarray(k, dtype=_F)
    v = np.asarray(v, dtype=_F)
    do = np.asarray(do, dtype=_F)
    full = rows is None
    rows = np.arange(q.shape[0]) if full else np.asarray(rows, dtype=np.int64)
    cols = None if cols is None else np.asarray(cols, dtype=np.int64)
    off = _offset(causal_offset, q.shape[0], k.shape[0])
    dq = np.empty((len(rows), q.shape[1]), dtype=_F) if cols is None else None
    kc = k if cols is None else k[cols]
    dk = np.zeros_like(kc) if full else None
    dv = np.zeros((kc.shape[0], v.shape[1]), dtype=_F) if full else None
    for c0 in range(0, len(rows), chunk):
        r = rows[c0:c0 + chunk]
        s = scale * (q[r] @ k.T)
        p, _ = _row_softmax(s, _allowed(r, k.shape[0], causal, head_mask, block, off))
        dp = do[r] @ v.T
        dsum = (p * dp).sum(axis=1)
        ds = p * (dp - dsum[:, None])
        if dq is not None:
            dq[c0:c0 + chunk] = scale * (ds @ k)
        if full:
            pc, dsc = (p, ds) if cols is None else (p[:, cols], ds[:, cols])
            dk += scale * (dsc.T @ q[r])
            dv += pc.T @ do[r]
    return dq, dk, dv


def _check_shapes(q, k, v):
    """(B, Nq, Nk, Hq, Hkv, d) of q [B,Nq,Hq,d] and k, v [B,Nk,Hkv,d]."""
    if q.ndim != 4 or k.shape != v.shape or k.ndim != 4:
        raise ValueError("expected q [B,Nq,Hq,d] and k, v [B,Nk,Hkv,d]")
    b, nq, hq, d = q.shape
    if k.shape[0] != b or k.shape[3] != d:
        raise ValueError("q and k/v disagree in B or d")
    return b, nq, k.shape[1], hq, k.shape[2], d


def _head_masks(block_mask, n: int, hkv: int, block: int):
    """Per-K/V-head block masks: ``block_mask`` is [Hm, nb, nb] with
    nb = ceil(N / block) and Hm = 1 (shared by every head) or Hkv (query head
    h uses the mask of its K/V head).  Returns a function g -> mask or None."""
    if block_mask is None:
        return lambda g: None
    m = np.asarray(block_mask)
    nb = -(-n // block)
    if m.ndim != 3 or m.shape[1:] != (nb, nb) or m.shape[0] not in (1, hkv):
        raise ValueError(f"block mask must be [1 or Hkv, {nb}, {nb}], got {m.shape}")
    return lambda g: m[0] if m.shape[0] == 1 else m[g]


def attention_fwd(q, k, v, causal: bool, scale: float, block_mask=None, block: int = 128,
                  causal_offset=None):
    """O [B,Nq,Hq,d] and LSE [B,Hq,Nq] in float64 (optionally block-sparse,
    which needs Nq = Nk; optionally rectangular with a causal offset)."""
    b, n, nk, hq, hkv, d = _check_shapes(q, k, v)
    if block_mask is not None and nk != n:
        raise ValueError("a block mask needs Nq = Nk")
    mask_of = _head_masks(block_mask, n, hkv, block)
    o = np.empty((b, n, hq, d), dtype=_F)
    lse = np.empty((b, hq, n), dtype=_F)
    for bi in range(b):
        for h in range(hq):
            g = kv_head_of(h, hq, hkv)
            o[bi, :, h], lse[bi, h] = attention_head_fwd(
                q[bi, :, h], k[bi, :, g], v[bi, :, g], causal, scale,
                head_mask=mask_of(g), block=block, causal_offset=causal_offset)
    return o, lse


def attention_bwd(q, k, v, do, causal: bool, scale: float, block_mask=None, block: int = 128,
                  causal_offset=None):
    """(dQ, dK, dV) in float64; dK/dV sum the contributions of each group."""
    b, n, nk, hq, hkv, d = _check_shapes(q, k, v)
    if block_mask is not None and nk != n:
        raise ValueError("a block mask needs Nq = Nk")
    mask_of = _head_masks(block_mask, n, hkv, block)
    dq = np.empty((b, n, hq, d), dtype=_F)
    dk = np.zeros((b, nk, hkv, d), dtype=_F)
    dv = np.zeros((b, nk, hkv, d), dtype=_F)
    for bi in range(b):
        for h in range(hq):
            g = kv_head_of(h, hq, hkv)
            dqh, dkh, dvh = attention_head_bwd(
                q[bi, :, h], k[bi, :, g], v[bi, :, g], do[bi, :, h], causal, scale,
                head_mask=mask_of(g), block=block, causal_offset=causal_offset)
            dq[bi, :, h] = dqh
            dk[bi, :, g] += dkh
            dv[bi, :, g] += dvh
    return dq, dk, dv
