"""CPU checks of the parity harness itself (no GPU)."""

import numpy as np

from gpu_util import excess, half_ulp


def test_half_ulp_matches_the_16_bit_formats():
    import torch

    for dtype, tdt in (("bf16", torch.bfloat16), ("fp16", torch.float16)):
        for x in (0.7, 1.0, 1.5, 3.99, 5.26, 100.0, -6.0):
            # the gap to the next representable value above |x|, halved
            t = torch.tensor(abs(x), dtype=tdt)
            nxt = torch.nextafter(t, torch.tensor(np.inf, dtype=tdt)).double().item()
            assert half_ulp(np.array([x]), dtype)[0] == (nxt - t.double().item()) / 2


def test_excess_accepts_rounding_and_rejects_more():
    ref = np.array([5.26, 0.3])
    rounded = np.array([5.25, 0.30078125])  # nearest bf16 values
    assert excess(rounded, ref, 0.0, "bf16") <= 0
    assert excess(rounded + 0.03, ref, 0.0, "bf16") > 0
    assert excess(ref + 0.019, ref, 0.02, "bf16") <= 0


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus N > 1 exits with a message saying so
    (before anything touches a GPU)."""
    import os
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr
