"""ATTN_DEBUG=1 (include/attn.h, "Errors"): every call waits for its stream and
reports kernel failures itself.  The results must be those of the normal,
asynchronous calls.  The library reads the variable once per process, so the
check runs in a child process."""

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
import numpy as np
import torch
import exact_io_aware_75_amd as ea
import oracle
from exact_io_aware_75_amd import inputs as gen

dev = torch.device("cuda:0")
b, n, hq, hkv, d = 1, 300, 4, 2, 128
scale = d ** -0.5
x = gen.make_inputs(b, n, hq, hkv, d, "bf16", cfg_id=41)
q, k, v, do = (gen.to_torch(x[t], "bf16", dev) for t in ("q", "k", "v", "do"))
f = lambda t: t.float().cpu().numpy().astype(np.float64)
ro, rlse = oracle.attention_fwd(x["q"], x["k"], x["v"], True, scale)
rdq, rdk, rdv = oracle.attention_bwd(x["q"], x["k"], x["v"], x["do"], True, scale)
# tiled path
o, lse = ea.forward(q, k, v, causal=True, scale=scale)
dq, dk, dv = ea.backward(q, k, v, o, lse, do, causal=True, scale=scale)
# standard path
ws = torch.empty(ea.attn_standard_workspace_bytes(b, n, hq, hkv, d), dtype=torch.uint8, device=dev)
so, slse = torch.empty_like(q), torch.empty_like(lse)
ea.attn_fwd_standard(q, k, v, so, slse, ws, True, scale)
sdq, sdk, sdv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
ea.attn_bwd_standard(q, k, v, do, sdq, sdk, sdv, ws, True, scale)
torch.cuda.synchronize()
for name, a_, r_, tol in (("o", o, ro, 2e-2), ("dq", dq, rdq, 3e-2), ("dk", dk, rdk, 3e-2), ("dv", dv, rdv, 3e-2),
                          ("std o", so, ro, 2e-2), ("std dq", sdq, rdq, 3e-2), ("std dk", sdk, rdk, 3e-2),
                          ("std dv", sdv, rdv, 3e-2)):
    err = float(np.abs(f(a_) - r_).max())
    print(name, err, flush=True)
    assert err <= tol, (name, err)
assert float(np.abs(lse.cpu().numpy() - rlse).max()) <= 1e-3
assert float(np.abs(slse.cpu().numpy() - rlse).max()) <= 1e-3
print("OK", flush=True)
"""


def test_debug_mode_gives_the_same_results(gpu_device):
    # tolerances: the stated ones (1e-2 on O, 2e-2 on gradients) plus one bf16
    # rounding of |values| < 4 (0.0078), since this check has no per-element allowance
    env = dict(os.environ, ATTN_DEBUG="1")
    r = subprocess.run([sys.executable, "-u", "-c", CHILD.format(root=ROOT)], env=env, capture_output=True,
                       text=True, timeout=300)
    print(r.stdout[-2000:], flush=True)
    assert r.returncode == 0, r.stderr[-4000:]
    assert r.stdout.strip().endswith("OK")
