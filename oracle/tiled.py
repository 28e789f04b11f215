"""fp64 model of the block-wise (online-softmax) forward, used only as a pin.

TEST INFRASTRUCTURE ONLY: never imported by the product path.

The pages say attention need not be materialised whole: it can be computed
block by block and the blocks aggregated afterwards, with a result equal to
standard attention up to numerical precision (FlashAttention-2 review,
"Введение" section).  The aggregation rule itself is not printed; this module
writes out the standard one.  For a row block (rows i) visiting key blocks j in
order, with running max m, running sum l and unnormalised accumulator acc:

    m_new = max(m, rowmax S_ij)
    alpha = exp(m - m_new)
    P~    = exp(S_ij - m_new)
    l     = alpha * l + rowsum P~
    acc   = alpha * acc + P~ V_j
    m     = m_new

and only at the end O = acc / l, LSE = m + ln l -- the single deferred division
the FlashAttention-2 announcement describes as rewriting the softmax trick to
cut rescaling work without changing the output ("具体实现" section).  Under a
causal mask, key blocks lying wholly above the diagonal are never visited
(FlashAttention-2 review, "Алгоритм вычисления" subsection), and only blocks
that straddle the diagonal apply an element mask.

With a block mask (block-sparse attention, which the FlashAttention-1 news
page benchmarks next to the dense method), key tiles whose (row block, key
block) entry is zero are skipped the same way; a row that visits no tile gets
O = 0 and LSE = -inf.

The test compares this model with ``attention.attention_head_fwd`` to 1e-12,
which pins the pages' equivalence claim in exact (fp64) arithmetic.
"""

from __future__ import annotations

import numpy as np


def tiled_attention_fwd(q, k, v, causal: bool, scale: float, bm: int = 16, bn: int = 16,
                        head_mask=None, block: int = 128):
    """Online-softmax forward of one head: returns (O [N,d], LSE [N], visited).

    ``visited`` counts the (row block, key block) pairs actually computed, so a
    test can check that fully masked causal blocks were skipped.  ``head_mask``
    ([ceil(N / block)]^2, optional) is a block mask; ``block`` must then be a
    multiple of both tile sizes, so that each tile lies in one mask block.
    """
    if head_mask is not None and (block % bm or block % bn):
        raise ValueError("the mask block must be a multiple of the tile sizes")
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n_q, n_k = q.shape[0], k.shape[0]
    o = np.empty((n_q, v.shape[1]))
    lse = np.empty(n_q)
    visited = 0
    for i0 in range(0, n_q, bm):
        rows = np.arange(i0, min(i0 + bm, n_q))
        m = np.full(len(rows), -np.inf)
        l = np.zeros(len(rows))
        acc = np.zeros((len(rows), v.shape[1]))
        for j0 in range(0, n_k, bn):
            if causal and j0 > rows[-1]:
                break  # this key block and every later one is fully masked
            if head_mask is not None and not head_mask[i0 // block][j0 // block]:
                continue  # a zero block of the mask: never loaded or computed
            visited += 1
            cols = np.arange(j0, min(j0 + bn, n_k))
            s = scale * (q[rows] @ k[cols].T)
            if causal and cols[-1] > rows[0]:  # block straddles the diagonal
                s = np.where(cols[None, :] <= rows[:, None], s, -np.inf)
            m_new = np.maximum(m, s.max(axis=1))
            alpha = np.exp(m - m_new)  # m = -inf on the first visit gives 0
            p = np.exp(s - m_new[:, None])
            l = alpha * l + p.sum(axis=1)
            acc = alpha[:, None] * acc + p @ v[cols]
            m = m_new
        if not np.isfinite(m).any():  # no tile visited: no allowed key
            o[rows], lse[rows] = 0.0, -np.inf
            continue
        o[rows] = acc / l[:, None]
        lse[rows] = m + np.log(l)
    return o, lse, visited
