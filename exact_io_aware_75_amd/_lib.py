"""ctypes binding of libattn.so (declared in include/attn.h).

Argument marshalling only: shape/dtype/contiguity checks on torch tensors,
then raw device pointers, sizes and the current HIP stream go through the C
ABI.  Every step of the computation runs in the library's HIP kernels.  There
is no fallback: if the library cannot be loaded, calls raise.
"""

from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libattn.so"
_lib = None

ATTN_DTYPE_FP16 = 0
ATTN_DTYPE_BF16 = 1

# Entry points declared in include/attn.h (checked by the ABI test).
EXPORTS = ("attn_fwd", "attn_bwd", "attn_bwd_preprocess", "attn_bwd_dkdv", "attn_bwd_dq",
           "attn_bwd_workspace_bytes", "attn_fwd_blocksparse", "attn_bwd_blocksparse",
           "attn_fwd_rect", "attn_bwd_rect", "attn_fwd_splitkv", "attn_fwd_splitkv_workspace_bytes",
           "attn_fwd_standard", "attn_bwd_standard", "attn_standard_workspace_bytes",
           "attn_bwd_noalloc", "attn_strerror", "attn_last_hip_error", "attn_version")
NOALLOC_SCRATCH_BYTES = 64 << 20  # ATTN_NOALLOC_SCRATCH_BYTES
SPARSE_BLOCK = 128  # ATTN_SPARSE_BLOCK: rows / keys per block of the block mask
BWD_STAGES = ("attn_bwd_preprocess", "attn_bwd_dkdv", "attn_bwd_dq")


class AttnError(RuntimeError):
    """A libattn call returned a non-zero attn_status_t."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {strerror(status)} (status {status}, "
                         f"hip error {last_hip_error()})")


def library_path() -> str:
    return os.environ.get("ATTN_LIBRARY", os.path.join(_HERE, _LIB_NAME))


def load_library():
    """Load libattn.so once and declare its prototypes."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp]
    lib.attn_fwd.restype = i
    for name in ("attn_bwd",) + BWD_STAGES:
        fn = getattr(lib, name)
        fn.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, i, f, vp]
        fn.restype = i
    lib.attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp]
    lib.attn_bwd_noalloc.restype = i
    lib.attn_fwd_blocksparse.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, vp]
    lib.attn_fwd_blocksparse.restype = i
    lib.attn_bwd_blocksparse.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, vp, vp, vp, vp, sz,
                                         i, i, i, i, i, i, i, f, vp]
    lib.attn_bwd_blocksparse.restype = i
    ll = ctypes.c_longlong
    lib.attn_fwd_rect.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, ll, f, vp]
    lib.attn_fwd_rect.restype = i
    lib.attn_bwd_rect.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, i, i, ll, f, vp]
    lib.attn_bwd_rect.restype = i
    lib.attn_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, i, i, ll, f, i, vp]
    lib.attn_fwd_splitkv.restype = i
    lib.attn_fwd_splitkv_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.attn_fwd_splitkv_workspace_bytes.restype = sz
    lib.attn_bwd_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.attn_bwd_workspace_bytes.restype = sz
    lib.attn_fwd_standard.argtypes = [vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, i, f, vp]
    lib.attn_fwd_standard.restype = i
    lib.attn_bwd_standard.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, i, f, vp]
    lib.attn_bwd_standard.restype = i
    lib.attn_standard_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.attn_standard_workspace_bytes.restype = sz
    lib.attn_strerror.argtypes = [i]
    lib.attn_strerror.restype = ctypes.c_char_p
    lib.attn_last_hip_error.argtypes = []
    lib.attn_last_hip_error.restype = i
    lib.attn_version.argtypes = []
    lib.attn_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def strerror(status: int) -> str:
    return load_library().attn_strerror(int(status)).decode()


def last_hip_error() -> int:
    return int(load_library().attn_last_hip_error())


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return ATTN_DTYPE_BF16
    if t.dtype == torch.float16:
        return ATTN_DTYPE_FP16
    raise TypeError(f"unsupported dtype {t.dtype}; expected bfloat16 or float16")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(t, shape, dtype, device, name):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _dims(q, k):
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B,Nq,Hq,d] and k/v [B,Nk,Hkv,d]")
    b, n, hq, d = q.shape
    return b, n, hq, k.shape[2], d


def _rect(n, nk, causal_offset, block_mask):
    """Whether a call needs the rectangular entry point, and its causal offset."""
    if nk == n and causal_offset in (None, 0):
        return False, 0
    if block_mask is not None:
        raise ValueError("block-sparse attention needs Nq = Nk and no causal offset")
    return True, (nk - n) if causal_offset is None else int(causal_offset)


def _check_mask(block_mask, n, hkv, device):
    """Shape/dtype of a block mask: uint8 [1 or Hkv, nb, nb], nb = ceil(N / 128)."""
    import torch

    nb = -(-n // SPARSE_BLOCK)
    if block_mask.dim() != 3 or tuple(block_mask.shape[1:]) != (nb, nb) or block_mask.shape[0] not in (1, hkv):
        raise ValueError(f"block_mask: shape {tuple(block_mask.shape)}, expected (1 or {hkv}, {nb}, {nb})")
    _check(block_mask, tuple(block_mask.shape), torch.uint8, device, "block_mask")
    return int(block_mask.shape[0])


def attn_fwd(q, k, v, o, lse, causal: bool, scale: float, stream=None, block_mask=None,
             causal_offset=None) -> None:
    """Enqueue the forward pass into preallocated ``o`` and ``lse``.

    ``block_mask`` (optional, uint8 [1 or Hkv, nb, nb] on q's device) selects
    the block-sparse entry point ``attn_fwd_blocksparse``.  K/V with a
    different sequence length than q, or an explicit ``causal_offset``
    (default Nk - Nq), select the rectangular entry point ``attn_fwd_rect``.
    """
    import torch

    lib = load_library()
    b, n, hq, hkv, d = _dims(q, k)
    nk = k.shape[1]
    for t, shp, nm in ((q, (b, n, hq, d), "q"), (k, (b, nk, hkv, d), "k"),
                       (v, (b, nk, hkv, d), "v"), (o, (b, n, hq, d), "o")):
        _check(t, shp, q.dtype, q.device, nm)
    _check(lse, (b, hq, n), torch.float32, q.device, "lse")
    rect, off = _rect(n, nk, causal_offset, block_mask)
    if rect:
        st = lib.attn_fwd_rect(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), b, n, nk, hq, hkv, d,
                               _dtype_code(q), int(bool(causal)), off, float(scale), _stream(stream, q.device))
        if st != 0:
            raise AttnError(st, "attn_fwd_rect")
        return
    tail = (b, n, hq, hkv, d, _dtype_code(q), int(bool(causal)), float(scale), _stream(stream, q.device))
    if block_mask is None:
        st, name = lib.attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), *tail), "attn_fwd"
    else:
        mh = _check_mask(block_mask, n, hkv, q.device)
        st = lib.attn_fwd_blocksparse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(block_mask), mh, *tail)
        name = "attn_fwd_blocksparse"
    if st != 0:
        raise AttnError(st, name)


def attn_fwd_splitkv_workspace_bytes(b: int, nq: int, hq: int, d: int, num_splits: int) -> int:
    return int(load_library().attn_fwd_splitkv_workspace_bytes(b, nq, hq, d, num_splits))


def attn_fwd_splitkv(q, k, v, o, lse, workspace, causal: bool, scale: float, num_splits: int,
                     stream=None, causal_offset=None) -> None:
    """Enqueue the split-KV forward pass (keys cut into ``num_splits`` runs
    processed in parallel, then merged); ``workspace`` is a uint8 device
    tensor of at least ``attn_fwd_splitkv_workspace_bytes`` bytes."""
    import torch

    lib = load_library()
    b, n, hq, hkv, d = _dims(q, k)
    nk = k.shape[1]
    for t, shp, nm in ((q, (b, n, hq, d), "q"), (k, (b, nk, hkv, d), "k"),
                       (v, (b, nk, hkv, d), "v"), (o, (b, n, hq, d), "o")):
        _check(t, shp, q.dtype, q.device, nm)
    _check(lse, (b, hq, n), torch.float32, q.device, "lse")
    if workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    off = (nk - n) if causal_offset is None else int(causal_offset)
    st = lib.attn_fwd_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), b, n, nk, hq, hkv, d,
                              _dtype_code(q), int(bool(causal)), off, float(scale), int(num_splits),
                              _stream(stream, q.device))
    if st != 0:
        raise AttnError(st, "attn_fwd_splitkv")


def attn_bwd_workspace_bytes(b: int, n: int, hq: int, hkv: int, d: int) -> int:
    return int(load_library().attn_bwd_workspace_bytes(b, n, hq, hkv, d))


def attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, causal: bool, scale: float,
             stream=None, stage: str = "attn_bwd", block_mask=None, causal_offset=None) -> None:
    """Enqueue the backward pass into preallocated ``dq``, ``dk``, ``dv``.

    ``workspace`` is a uint8 device tensor of at least
    ``attn_bwd_workspace_bytes(B, N, Hq, Hkv, d)`` bytes.  ``stage`` selects
    the whole pass ("attn_bwd") or one of its stages (``BWD_STAGES``), which
    must then be enqueued in order.  ``block_mask`` (as for ``attn_fwd``)
    selects ``attn_bwd_blocksparse`` (whole pass only); K/V of another
    length than q or a ``causal_offset`` select ``attn_bwd_rect`` (whole pass
    only, workspace sized for the Nq queries).
    """
    import torch

    if stage != "attn_bwd" and stage not in BWD_STAGES:
        raise ValueError(f"unknown backward stage {stage!r}")
    if block_mask is not None and stage != "attn_bwd":
        raise ValueError("the block-sparse backward pass has no separate stages")
    lib = load_library()
    b, n, hq, hkv, d = _dims(q, k)
    nk = k.shape[1]
    for t, shp, nm in ((q, (b, n, hq, d), "q"), (k, (b, nk, hkv, d), "k"),
                       (v, (b, nk, hkv, d), "v"), (o, (b, n, hq, d), "o"),
                       (dout, (b, n, hq, d), "dout"), (dq, (b, n, hq, d), "dq"),
                       (dk, (b, nk, hkv, d), "dk"), (dv, (b, nk, hkv, d), "dv")):
        _check(t, shp, q.dtype, q.device, nm)
    rect, off = _rect(n, nk, causal_offset, block_mask)
    if rect and stage != "attn_bwd":
        raise ValueError("the rectangular backward pass has no separate stages")
    _check(lse, (b, hq, n), torch.float32, q.device, "lse")
    if workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    ws_bytes = workspace.numel() * workspace.element_size()
    tail = (_ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes, b, n, hq, hkv, d,
            _dtype_code(q), int(bool(causal)), float(scale), _stream(stream, q.device))
    if rect:
        stage = "attn_bwd_rect"
        st = lib.attn_bwd_rect(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                               _ptr(dv), _ptr(workspace), ws_bytes, b, n, nk, hq, hkv, d, _dtype_code(q),
                               int(bool(causal)), off, float(scale), _stream(stream, q.device))
    elif block_mask is None:
        st = getattr(lib, stage)(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), *tail)
    else:
        mh = _check_mask(block_mask, n, hkv, q.device)
        stage = "attn_bwd_blocksparse"
        st = lib.attn_bwd_blocksparse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                      _ptr(block_mask), mh, *tail)
    if st != 0:
        raise AttnError(st, stage)


def attn_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, causal: bool, scale: float, stream=None) -> None:
    """Enqueue ``attn_bwd_noalloc``: the backward pass into preallocated
    ``dq``, ``dk``, ``dv`` with the library's static device scratch instead of
    a workspace (calls on one device must not overlap)."""
    import torch

    lib = load_library()
    b, n, hq, hkv, d = _dims(q, k)
    for t, shp, nm in ((q, (b, n, hq, d), "q"), (k, (b, n, hkv, d), "k"),
                       (v, (b, n, hkv, d), "v"), (o, (b, n, hq, d), "o"),
                       (dout, (b, n, hq, d), "dout"), (dq, (b, n, hq, d), "dq"),
                       (dk, (b, n, hkv, d), "dk"), (dv, (b, n, hkv, d), "dv")):
        _check(t, shp, q.dtype, q.device, nm)
    _check(lse, (b, hq, n), torch.float32, q.device, "lse")
    st = lib.attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                              _ptr(dv), b, n, hq, hkv, d, _dtype_code(q), int(bool(causal)), float(scale),
                              _stream(stream, q.device))
    if st != 0:
        raise AttnError(st, "attn_bwd_noalloc")


def attn_standard_workspace_bytes(b: int, n: int, hq: int, hkv: int, d: int) -> int:
    return int(load_library().attn_standard_workspace_bytes(b, n, hq, hkv, d))


def _check_ws(workspace, device):
    if workspace.device != device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    return workspace.numel() * workspace.element_size()


def attn_fwd_standard(q, k, v, o, lse, workspace, causal: bool, scale: float, stream=None) -> None:
    """Enqueue standard (materialising) attention's forward pass: S, then P,
    in full in ``workspace`` (a uint8 device tensor of at least
    ``attn_standard_workspace_bytes`` bytes), then ``o`` and ``lse``."""
    import torch

    lib = load_library()
    b, n, hq, hkv, d = _dims(q, k)
    for t, shp, nm in ((q, (b, n, hq, d), "q"), (k, (b, n, hkv, d), "k"), (v, (b, n, hkv, d), "v"),
                       (o, (b, n, hq, d), "o")):
        _check(t, shp, q.dtype, q.device, nm)
    _check(lse, (b, hq, n), torch.float32, q.device, "lse")
    st = lib.attn_fwd_standard(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(workspace),
                               _check_ws(workspace, q.device), b, n, hq, hkv, d, _dtype_code(q),
                               int(bool(causal)), float(scale), _stream(stream, q.device))
    if st != 0:
        raise AttnError(st, "attn_fwd_standard")


def attn_bwd_standard(q, k, v, dout, dq, dk, dv, workspace, causal: bool, scale: float, stream=None) -> None:
    """Enqueue standard attention's backward pass, which reads the P that
    ``attn_fwd_standard`` left in the same ``workspace``."""
    lib = load_library()
    b, n, hq, hkv, d = _dims(q, k)
    for t, shp, nm in ((q, (b, n, hq, d), "q"), (k, (b, n, hkv, d), "k"), (v, (b, n, hkv, d), "v"),
                       (dout, (b, n, hq, d), "dout"), (dq, (b, n, hq, d), "dq"),
                       (dk, (b, n, hkv, d), "dk"), (dv, (b, n, hkv, d), "dv")):
        _check(t, shp, q.dtype, q.device, nm)
    st = lib.attn_bwd_standard(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                               _ptr(workspace), _check_ws(workspace, q.device), b, n, hq, hkv, d,
                               _dtype_code(q), int(bool(causal)), float(scale), _stream(stream, q.device))
    if st != 0:
        raise AttnError(st, "attn_bwd_standard")


def standard_probs(workspace, b: int, n: int, hq: int, dtype):
    """The materialised P [B, Hq, N, N] inside a standard-attention workspace
    (a view; layout as include/attn.h states it: row pitch N rounded up to 64,
    after the fp32 score matrix rounded up to 256 bytes)."""
    ldn = -(-n // 64) * 64
    elems = b * hq * n * ldn
    p_off = -(-(4 * elems) // 256) * 256
    return workspace[p_off:p_off + 2 * elems].view(dtype).view(b, hq, n, ldn)[..., :n]


def _default_scale(d: int, scale):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def forward(q, k, v, causal: bool = False, scale=None, stream=None, block_mask=None, causal_offset=None,
            num_splits=None):
    """Allocate ``o`` and ``lse`` and run ``attn_fwd`` (with a block mask
    ``attn_fwd_blocksparse``; with Nk != Nq or a causal offset
    ``attn_fwd_rect``; with ``num_splits`` ``attn_fwd_splitkv``, allocating
    its workspace); returns (o, lse)."""
    import torch

    b, n, hq, _, d = _dims(q, k)
    o = torch.empty_like(q)
    lse = torch.empty((b, hq, n), dtype=torch.float32, device=q.device)
    if num_splits is not None:
        if block_mask is not None:
            raise ValueError("split-KV and block-sparse attention do not combine")
        ws = torch.empty(attn_fwd_splitkv_workspace_bytes(b, n, hq, d, num_splits), dtype=torch.uint8,
                         device=q.device)
        attn_fwd_splitkv(q, k, v, o, lse, ws, causal, _default_scale(d, scale), num_splits, stream,
                         causal_offset=causal_offset)
        return o, lse
    attn_fwd(q, k, v, o, lse, causal, _default_scale(d, scale), stream, block_mask=block_mask,
             causal_offset=causal_offset)
    return o, lse


def backward(q, k, v, o, lse, dout, causal: bool = False, scale=None, stream=None, workspace=None,
             block_mask=None, causal_offset=None):
    """Allocate gradients (and the workspace if not given) and run ``attn_bwd``
    (or the block-sparse / rectangular entry point, as in ``forward``)."""
    import torch

    b, n, hq, hkv, d = _dims(q, k)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if workspace is None:
        workspace = torch.empty(attn_bwd_workspace_bytes(b, n, hq, hkv, d), dtype=torch.uint8,
                                device=q.device)
    attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, causal, _default_scale(d, scale), stream,
             block_mask=block_mask, causal_offset=causal_offset)
    return dq, dk, dv
