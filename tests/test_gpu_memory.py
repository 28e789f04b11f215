"""Device memory of the tiled path on the GPU: nothing N x N is ever
allocated (FlashAttention-2 announcement, "具体实现": memory linear instead of
quadratic in the sequence length; FlashAttention-1 news page,
"FlashAttention": the attention matrix is never stored in HBM).

The library allocates nothing itself: a forward + backward pass changes
neither torch's allocation counters nor the driver's free-memory figure, and
the memory beyond the inputs and outputs is the LSE and the backward
workspace (D), B * Hq * N floats each, linear in N.
"""

import pytest

from gpu_util import log

pytestmark = pytest.mark.gpu


def test_fwd_bwd_allocates_only_linear_extra_memory(gpu_device):
    import torch
    import exact_io_aware_75_amd as ea

    b, n, h, d = 1, 16384, 8, 128
    g = torch.Generator(device=gpu_device)
    g.manual_seed(0)
    q, k, v, do = (torch.randn(b, n, h, d, device=gpu_device, generator=g).to(torch.bfloat16) for _ in range(4))
    o = torch.empty_like(q)
    lse = torch.empty((b, h, n), dtype=torch.float32, device=gpu_device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = ea.attn_bwd_workspace_bytes(b, n, h, h, d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=gpu_device)
    # the extra memory: LSE and D, one float per (batch, head, query row) each
    assert ws_bytes == b * h * n * 4
    extra = lse.numel() * 4 + ws_bytes
    tensors = q.numel() * 2 * 8  # q, k, v, do, o, dq, dk, dv
    log(f"inputs+outputs {tensors / 2**20:.0f} MiB, extra {extra / 2**20:.2f} MiB; "
        f"an N x N fp32 score matrix per head would be {b * h * n * n * 4 / 2**30:.1f} GiB")
    assert extra <= tensors / 100

    def run(causal):
        ea.attn_fwd(q, k, v, o, lse, causal, d ** -0.5)
        ea.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, causal, d ** -0.5)

    for causal in (False, True):
        run(causal)  # first launches load the code objects
    torch.cuda.synchronize()
    alloc0 = torch.cuda.memory_allocated(gpu_device)
    torch.cuda.reset_peak_memory_stats(gpu_device)
    free0, _ = torch.cuda.mem_get_info(gpu_device)
    for causal in (False, True):
        run(causal)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info(gpu_device)
    assert torch.cuda.max_memory_allocated(gpu_device) == alloc0
    assert torch.cuda.memory_allocated(gpu_device) == alloc0
    log(f"driver free memory before {free0 / 2**30:.3f} GiB, after {free1 / 2**30:.3f} GiB")
    assert free1 == free0
    assert torch.isfinite(dq.float()).all() and torch.isfinite(dk.float()).all()
