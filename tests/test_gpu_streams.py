"""Streams and graph capture: every entry point enqueues on the caller's
stream and allocates nothing, so calls work on a side stream and inside a
captured HIP graph.  The kernels are deterministic, so both must reproduce the
default-stream results bitwise."""

import numpy as np
import pytest

from exact_io_aware_75_amd import inputs as gen
from gpu_util import log

pytestmark = pytest.mark.gpu


def _setup(device, b=2, n=700, hq=4, hkv=2, d=128):
    import torch
    import exact_io_aware_75_amd as ea

    x = gen.make_inputs(b, n, hq, hkv, d, "bf16", cfg_id=43)
    q, k, v, do = (gen.to_torch(x[t], "bf16", device) for t in ("q", "k", "v", "do"))
    bufs = {"o": torch.empty_like(q), "lse": torch.empty((b, hq, n), dtype=torch.float32, device=device),
            "dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
            "ws": torch.empty(ea.attn_bwd_workspace_bytes(b, n, hq, hkv, d), dtype=torch.uint8, device=device)}
    return (q, k, v, do), bufs, d ** -0.5


def _run(ea, inp, bufs, causal, scale, stream=None):
    q, k, v, do = inp
    ea.attn_fwd(q, k, v, bufs["o"], bufs["lse"], causal, scale, stream)
    ea.attn_bwd(q, k, v, bufs["o"], do, bufs["lse"], bufs["dq"], bufs["dk"], bufs["dv"], bufs["ws"], causal, scale,
                stream)


def _snapshot(bufs):
    return {k_: t.clone() for k_, t in bufs.items() if k_ != "ws"}


@pytest.mark.parametrize("causal", [False, True])
def test_side_stream_matches_default_stream(gpu_device, causal):
    import torch
    import exact_io_aware_75_amd as ea

    inp, bufs, scale = _setup(gpu_device)
    _run(ea, inp, bufs, causal, scale)
    torch.cuda.synchronize()
    ref = _snapshot(bufs)
    for t in bufs.values():
        t.zero_()
    side = torch.cuda.Stream(device=gpu_device)  # default priority
    side.wait_stream(torch.cuda.current_stream(gpu_device))
    _run(ea, inp, bufs, causal, scale, stream=side)  # explicit stream argument
    side.synchronize()
    for k_, t in ref.items():
        assert torch.equal(bufs[k_], t), k_
    for t in bufs.values():
        t.zero_()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):  # the binding's default: the current stream
        _run(ea, inp, bufs, causal, scale)
    side.synchronize()
    for k_, t in ref.items():
        assert torch.equal(bufs[k_], t), k_


@pytest.mark.parametrize("causal", [False, True])
def test_captured_graph_replays_match_eager(gpu_device, causal):
    import torch
    import exact_io_aware_75_amd as ea

    inp, bufs, scale = _setup(gpu_device)
    _run(ea, inp, bufs, causal, scale)
    torch.cuda.synchronize()
    ref = _snapshot(bufs)
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream(device=gpu_device)
    cap.wait_stream(torch.cuda.current_stream(gpu_device))
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            _run(ea, inp, bufs, causal, scale)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in bufs.values():
            t.fill_(0x7F if t.dtype == torch.uint8 else 3.0)  # garbage the replay must overwrite
        _run(ea, inp, _snapshot(bufs) | {"ws": bufs["ws"]}, causal, scale)  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k_, t in ref.items():
            assert torch.equal(bufs[k_], t), (rep, k_)
        log(f"replay {rep}: bitwise equal to eager")
    del graph
    assert np.isfinite(ref["dq"].float().cpu().numpy()).all()
