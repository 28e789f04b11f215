"""Helpers for the GPU parity tests: run the HIP path through the C ABI on
seeded inputs and compare element by element with the CPU oracle."""

import sys

import numpy as np

from exact_io_aware_75_amd import configs
from exact_io_aware_75_amd import inputs as gen

# Tolerances stated for this path: max-abs error vs the fp64 oracle for
# unit-variance inputs with fp32 accumulation.
TOL_O = 1e-2
TOL_LSE = 1e-3
TOL_GRAD = 2e-2


def tol_kv(hq, hkv):
    """Bound on dK / dV of a K/V head.  They sum the contributions of the
    Hq / Hkv query heads of its group, each computed from its own rounded
    probabilities (P and dS enter the matrix products in the 16-bit input
    type); the stated 2e-2 bounds one head's contribution, and independent
    rounding errors of Hq / Hkv contributions add in quadrature, so the group
    sum is held to 2e-2 * sqrt(Hq / Hkv) (2e-2 itself without grouping)."""
    return TOL_GRAD * float(np.sqrt(hq // hkv))


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def upload(x, dtype, device):
    return gen.to_torch(x, dtype, device)


def run_fwd(x, dtype, causal, scale, device):
    import torch
    import exact_io_aware_75_amd as ea

    q, k, v = (upload(x[t], dtype, device) for t in ("q", "k", "v"))
    o, lse = ea.forward(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def run_fwd_bwd(x, dtype, causal, scale, device, block_mask=None, causal_offset=None):
    """Forward then backward through the C ABI; ``block_mask`` (numpy uint8
    [1 or Hkv, nb, nb]) selects the block-sparse entry points, K/V longer or
    shorter than Q or a ``causal_offset`` the rectangular ones."""
    import torch
    import exact_io_aware_75_amd as ea

    q, k, v, do = (upload(x[t], dtype, device) for t in ("q", "k", "v", "do"))
    bm = None if block_mask is None else torch.from_numpy(np.ascontiguousarray(block_mask, dtype=np.uint8)).to(device)
    o, lse = ea.forward(q, k, v, causal=causal, scale=scale, block_mask=bm, causal_offset=causal_offset)
    dq, dk, dv = ea.backward(q, k, v, o, lse, do, causal=causal, scale=scale, block_mask=bm,
                             causal_offset=causal_offset)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    return f(o), lse.cpu().numpy().astype(np.float64), f(dq), f(dk), f(dv)


def make_rect_inputs(b, nq, nk, hq, hkv, d, dtype, cfg_id, seed=0):
    """Q, dO [B,Nq,Hq,d] and K, V [B,Nk,Hkv,d] from the seeded generator."""
    return {"q": gen.draw((b, nq, hq, d), dtype, cfg_id, nq, "q", seed),
            "k": gen.draw((b, nk, hkv, d), dtype, cfg_id, nk, "k", seed),
            "v": gen.draw((b, nk, hkv, d), dtype, cfg_id, nk, "v", seed),
            "do": gen.draw((b, nq, hq, d), dtype, cfg_id, nq, "do", seed)}


def half_ulp(ref, dtype):
    """Half a unit in the last place of |ref| in the 16-bit output type: the
    error of merely storing the exact result in that type (normal range)."""
    mant = {"bf16": 7, "fp16": 10}[dtype]
    mag = np.maximum(np.abs(ref), 2.0 ** -14)
    return 0.5 * np.exp2(np.floor(np.log2(mag)) - mant)


def excess(a, ref, tol, dtype):
    """Largest (|a - ref| - allowed) over all elements, where allowed = tol +
    half an output ulp of |ref|.  <= 0 means every element is within bounds.

    The stated tolerances bound the computed value; the oracle is fp64 and
    unrounded, so the comparison also allows the rounding of the result into
    the 16-bit output type (which alone exceeds 1e-2 once |x| >= 4 in bf16).
    """
    if a.size == 0:
        return 0.0
    return float((np.abs(a - ref) - (tol + half_ulp(ref, dtype))).max())


def max_err(a, ref):
    """(max abs error, |ref| at that element)."""
    diff = np.abs(a - ref)
    i = np.unravel_index(np.argmax(diff), diff.shape) if diff.size else ()
    return (float(diff[i]), float(np.abs(ref[i]))) if diff.size else (0.0, 0.0)


def record(tag, name, a, ref, tol, dtype=None):
    """Flat max-abs error of ``a`` against ``ref`` (and |ref| there), appended
    as one JSON line to the file named by ATTN_PARITY_LOG, if set, with
    whether it exceeds the flat bound ``tol`` (i.e. whether the test needed
    the half-ulp output-rounding allowance of ``excess``).  Returns
    (error, |ref|)."""
    import json
    import os

    err, mag = max_err(a, ref)
    path = os.environ.get("ATTN_PARITY_LOG")
    if path:
        rec = {"case": tag, "tensor": name, "max_abs": err, "ref_at_max": mag, "max_ref": float(np.abs(ref).max()) if ref.size else 0.0,
               "flat_tol": tol, "within_flat": err <= tol, "checked": int(a.size)}
        if dtype is not None and ref.size:
            rec["within_checked_bound"] = excess(a, ref, tol, dtype) <= 0
        with open(path, "a") as f:
            f.write(json.dumps(rec) + "\n")
    return err, mag


def full_size_shapes():
    """Every full-size workload: the hidden-size-2048 sweep (d = 64 and 128,
    N = 512 .. 16384, causal and not), long sequences, GQA/MQA and d = 256."""
    out = []
    for d in (64, 128):
        for n in configs.SWEEP_N:
            for c in (False, True):
                out.append(configs.hidden2048(d, n, c))
    out += [configs.long_seq(32768), configs.long_seq(65536), configs.gqa(8), configs.gqa(1),
            configs.wide_head()]
    return out
