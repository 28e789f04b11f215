"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/attn.h, and rejects invalid arguments with the documented
status codes before launching anything."""

import ctypes
import math
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


@pytest.fixture(scope="module")
def lib():
    from exact_io_aware_75_amd import _lib

    if not os.path.exists(_lib.library_path()):
        from exact_io_aware_75_amd.build import build

        build()
    return _lib.load_library()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def _status_codes():
    text = open(HEADER).read()
    return {k: int(v) for k, v in re.findall(r"\b(ATTN_(?:OK|ERR_[A-Z_]+))\s*=\s*(\d+)", text)}


def test_header_declares_the_binding_exports():
    from exact_io_aware_75_amd._lib import EXPORTS

    assert _declared() == sorted(EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", lib._name], capture_output=True, text=True).stdout
    for name in _declared():
        assert re.search(rf"\bT {name}\b", out), name


def test_strerror_and_version(lib):
    codes = _status_codes()
    assert codes["ATTN_OK"] == 0 and len(set(codes.values())) == len(codes)
    for v in codes.values():
        s = lib.attn_strerror(v).decode()
        assert s and s != "unknown status"
    assert lib.attn_strerror(12345).decode() == "unknown status"
    assert b"gfx950" in lib.attn_version()
    assert lib.attn_last_hip_error() == 0


A = 0x10000  # fake, 16-byte aligned device addresses: never dereferenced on these paths


def _fwd(lib, q=A, k=A, v=A, o=A, lse=A, B=1, N=128, Hq=2, Hkv=2, d=64, dtype=1, causal=0, scale=0.125):
    return lib.attn_fwd(q, k, v, o, lse, B, N, Hq, Hkv, d, dtype, causal, scale, None)


def _bwd(lib, ws_bytes=None, ws=A, B=1, N=128, Hq=2, Hkv=2, d=64, dtype=1, scale=0.125, **ptrs):
    p = dict(q=A, k=A, v=A, o=A, do=A, lse=A, dq=A, dk=A, dv=A)
    p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = lib.attn_bwd_workspace_bytes(B, N, Hq, Hkv, d)
    return lib.attn_bwd(p["q"], p["k"], p["v"], p["o"], p["do"], p["lse"], p["dq"], p["dk"], p["dv"],
                        ws, ws_bytes, B, N, Hq, Hkv, d, dtype, 0, scale, None)


def test_fwd_rejects_invalid_arguments(lib):
    c = _status_codes()
    assert _fwd(lib, q=None) == c["ATTN_ERR_NULLPTR"]
    assert _fwd(lib, lse=None) == c["ATTN_ERR_NULLPTR"]
    assert _fwd(lib, B=0) == c["ATTN_ERR_SHAPE"]
    assert _fwd(lib, N=0) == c["ATTN_ERR_SHAPE"]
    assert _fwd(lib, Hq=4, Hkv=3) == c["ATTN_ERR_SHAPE"]
    assert _fwd(lib, Hkv=0) == c["ATTN_ERR_SHAPE"]
    for d in (0, 32, 96, 512):
        assert _fwd(lib, d=d) == c["ATTN_ERR_HEADDIM"]
    assert _fwd(lib, dtype=2) == c["ATTN_ERR_DTYPE"]
    assert _fwd(lib, v=A + 8) == c["ATTN_ERR_ALIGN"]
    assert _fwd(lib, scale=math.nan) == c["ATTN_ERR_SCALE"]
    assert _fwd(lib, scale=math.inf) == c["ATTN_ERR_SCALE"]
    assert _fwd(lib, N=1 << 24, Hq=1, Hkv=1, d=128) == c["ATTN_ERR_TOO_LARGE"]


def test_bwd_rejects_invalid_arguments(lib):
    c = _status_codes()
    for name in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv"):
        assert _bwd(lib, **{name: None}) == c["ATTN_ERR_NULLPTR"], name
    assert _bwd(lib, Hq=6, Hkv=4) == c["ATTN_ERR_SHAPE"]
    assert _bwd(lib, d=80) == c["ATTN_ERR_HEADDIM"]
    assert _bwd(lib, dtype=-1) == c["ATTN_ERR_DTYPE"]
    assert _bwd(lib, dk=A + 4) == c["ATTN_ERR_ALIGN"]
    assert _bwd(lib, scale=-math.inf) == c["ATTN_ERR_SCALE"]
    need = lib.attn_bwd_workspace_bytes(1, 128, 2, 2, 64)
    assert _bwd(lib, ws_bytes=need - 1) == c["ATTN_ERR_WORKSPACE"]
    assert _bwd(lib, ws=None) == c["ATTN_ERR_WORKSPACE"]
    assert _bwd(lib, ws=A + 2) == c["ATTN_ERR_ALIGN"]


def test_workspace_is_linear_in_sequence_length(lib):
    """Memory linear in N (FlashAttention-2 announcement, "具体实现": the tiled
    method cuts memory from quadratic to linear in sequence length)."""
    f = lambda n: lib.attn_bwd_workspace_bytes(2, n, 8, 2, 128)  # noqa: E731
    sizes = [f(n) for n in (1024, 2048, 4096, 8192)]
    assert all(s > 0 for s in sizes)
    # exact affine form up to 256-byte alignment padding
    assert abs((sizes[3] - sizes[2]) - 2 * (sizes[2] - sizes[1])) <= 512
    assert sizes[3] <= 4.01 * sizes[1]
    # one fp32 per query row (D = rowsum(dO * O)), plus, for this small grid
    # (2 * 2 * 32 = 128 dK/dV workgroups at N = 4096), fp32 partial dK/dV of the
    # whole group of 4 query heads split 4 ways (128 * 2 < 1024), plus alignment
    assert f(4096) == 2 * 8 * 4096 * 4 + 4 * 2 * 2 * 4096 * 2 * 128 * 4
    # MHA, d = 256, or a grid of >= 512 dK/dV workgroups: D only
    assert lib.attn_bwd_workspace_bytes(2, 4096, 8, 8, 128) == 2 * 8 * 4096 * 4
    assert lib.attn_bwd_workspace_bytes(2, 4096, 8, 2, 256) == 2 * 8 * 4096 * 4
    assert lib.attn_bwd_workspace_bytes(4, 16384, 8, 2, 128) == 4 * 8 * 16384 * 4
    # MQA, B = 4, N = 4096, Hq = 32: 128 workgroups, split 8 ways (the smallest divisor reaching 1024)
    assert lib.attn_bwd_workspace_bytes(4, 4096, 32, 1, 128) == 4 * 32 * 4096 * 4 + 8 * 2 * 4 * 4096 * 128 * 4
    assert lib.attn_bwd_workspace_bytes(0, 16, 1, 1, 64) == 0
    assert lib.attn_bwd_workspace_bytes(1, 16, 3, 2, 64) == 0


def test_valid_call_without_gpu_reports_device_error():
    """On a machine with no GPU a valid call must fail cleanly with
    ATTN_ERR_DEVICE (run in a child process so the HIP runtime's probe of a
    missing device cannot disturb this one)."""
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    code = (
        "import ctypes,sys; sys.path.insert(0, %r)\n"
        "from exact_io_aware_75_amd import _lib\n"
        "lib=_lib.load_library()\n"
        "print(lib.attn_fwd(%d,%d,%d,%d,%d,1,128,2,2,64,1,0,0.125,None))\n" % (ROOT, A, A, A, A, A)
    )
    r = subprocess.run(["python", "-c", code], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert int(r.stdout.strip().splitlines()[-1]) == _status_codes()["ATTN_ERR_DEVICE"]


def test_blocksparse_rejects_invalid_arguments(lib):
    c = _status_codes()
    fwd = lambda mask=A, mh=1, N=128, Hkv=2: lib.attn_fwd_blocksparse(  # noqa: E731
        A, A, A, A, A, mask, mh, 1, N, 2, Hkv, 64, 1, 0, 0.125, None)
    assert fwd(mask=None) == c["ATTN_ERR_NULLPTR"]
    assert fwd(mh=0) == c["ATTN_ERR_SHAPE"]
    assert fwd(mh=3) == c["ATTN_ERR_SHAPE"]
    assert fwd(mh=2, Hkv=1) == c["ATTN_ERR_SHAPE"]
    assert fwd(N=(1 << 18) + 1) == c["ATTN_ERR_TOO_LARGE"]
    ws = lib.attn_bwd_workspace_bytes(1, 128, 2, 2, 64)
    bwd = lambda mask=A, mh=2, ws_bytes=ws: lib.attn_bwd_blocksparse(  # noqa: E731
        A, A, A, A, A, A, mask, mh, A, A, A, A, ws_bytes, 1, 128, 2, 2, 64, 1, 1, 0.125, None)
    assert bwd(mask=None) == c["ATTN_ERR_NULLPTR"]
    assert bwd(mh=4) == c["ATTN_ERR_SHAPE"]
    assert bwd(ws_bytes=ws - 1) == c["ATTN_ERR_WORKSPACE"]


def test_rect_rejects_invalid_arguments(lib):
    c = _status_codes()
    fwd = lambda Nq=128, Nk=256, off=0, q=A: lib.attn_fwd_rect(  # noqa: E731
        q, A, A, A, A, 1, Nq, Nk, 2, 2, 64, 1, 1, off, 0.125, None)
    assert fwd(q=None) == c["ATTN_ERR_NULLPTR"]
    assert fwd(Nq=0) == c["ATTN_ERR_SHAPE"]
    assert fwd(Nk=0) == c["ATTN_ERR_SHAPE"]
    assert fwd(Nk=1 << 24) == c["ATTN_ERR_TOO_LARGE"]
    ws = lib.attn_bwd_workspace_bytes(1, 128, 2, 2, 64)
    bwd = lambda ws_bytes=ws, Nk=256: lib.attn_bwd_rect(  # noqa: E731
        A, A, A, A, A, A, A, A, A, A, ws_bytes, 1, 128, Nk, 2, 2, 64, 1, 1, -(1 << 40), 0.125, None)
    assert bwd(ws_bytes=ws - 1) == c["ATTN_ERR_WORKSPACE"]
    assert bwd(Nk=-1) == c["ATTN_ERR_SHAPE"]


def test_splitkv_rejects_invalid_arguments(lib):
    c = _status_codes()
    need = lib.attn_fwd_splitkv_workspace_bytes(1, 128, 2, 64, 4)
    assert need >= 4 * 128 * 2 * 64 * 4
    assert lib.attn_fwd_splitkv_workspace_bytes(1, 128, 2, 64, 0) == 0
    assert lib.attn_fwd_splitkv_workspace_bytes(1, 128, 2, 64, 257) == 0
    f = lambda splits=4, ws=A, ws_bytes=need, q=A: lib.attn_fwd_splitkv(  # noqa: E731
        q, A, A, A, A, ws, ws_bytes, 1, 128, 1000, 2, 2, 64, 1, 0, 0, 0.125, splits, None)
    assert f(splits=0) == c["ATTN_ERR_SHAPE"]
    assert f(splits=1000) == c["ATTN_ERR_SHAPE"]
    assert f(ws=None) == c["ATTN_ERR_WORKSPACE"]
    assert f(ws_bytes=need - 1) == c["ATTN_ERR_WORKSPACE"]
    assert f(ws=A + 4) == c["ATTN_ERR_ALIGN"]
    assert f(q=None) == c["ATTN_ERR_NULLPTR"]


def test_standard_rejects_invalid_arguments(lib):
    c = _status_codes()
    need = lib.attn_standard_workspace_bytes(1, 100, 2, 1, 64)
    # S (fp32), P and dS (16-bit), each [B, Hq, N, ldn] with ldn = 128, 256-byte aligned
    assert need == 4 * 2 * 100 * 128 + 2 * (2 * 2 * 100 * 128)
    assert lib.attn_standard_workspace_bytes(1, 100, 3, 2, 64) == 0
    assert lib.attn_standard_workspace_bytes(1, 1 << 20, 32, 32, 64) == 0  # B * Hq * N >= 2^24
    fwd = lambda ws=A, ws_bytes=need, o=A, N=100, d=64, scale=0.125: lib.attn_fwd_standard(  # noqa: E731
        A, A, A, o, A, ws, ws_bytes, 1, N, 2, 1, d, 1, 1, scale, None)
    assert fwd(o=None) == c["ATTN_ERR_NULLPTR"]
    assert fwd(ws=None) == c["ATTN_ERR_WORKSPACE"]
    assert fwd(ws_bytes=need - 1) == c["ATTN_ERR_WORKSPACE"]
    assert fwd(ws=A + 8) == c["ATTN_ERR_ALIGN"]
    assert fwd(o=A + 2) == c["ATTN_ERR_ALIGN"]
    assert fwd(d=32) == c["ATTN_ERR_HEADDIM"]
    assert fwd(N=0) == c["ATTN_ERR_SHAPE"]
    assert fwd(N=1 << 23) == c["ATTN_ERR_TOO_LARGE"]
    assert fwd(scale=math.nan) == c["ATTN_ERR_SCALE"]
    bwd = lambda dq=A, ws_bytes=need: lib.attn_bwd_standard(  # noqa: E731
        A, A, A, A, dq, A, A, A, ws_bytes, 1, 100, 2, 1, 64, 0, 0, 0.125, None)
    assert bwd(dq=None) == c["ATTN_ERR_NULLPTR"]
    assert bwd(ws_bytes=need - 1) == c["ATTN_ERR_WORKSPACE"]


def test_standard_workspace_is_quadratic_in_sequence_length(lib):
    """The materialising baseline needs O(N^2) memory (FlashAttention-1 news
    page, "FlashAttention": standard attention keeps the N x N matrix in HBM),
    against the tiled path's O(N)."""
    f = lambda n: lib.attn_standard_workspace_bytes(1, n, 4, 4, 64)  # noqa: E731
    for n in (1024, 2048, 4096):
        assert f(n) == 4 * n * n * (4 + 2 + 2)
        assert f(n) / lib.attn_bwd_workspace_bytes(1, n, 4, 4, 64) == 2 * n


def test_probe_library_exports_its_header():
    """libattn_probe.so (the benchmark's MFMA throughput probe) exports every
    entry point include/attn_probe.h declares, and rejects bad arguments."""
    path = os.path.join(ROOT, "exact_io_aware_75_amd", "libattn_probe.so")
    if not os.path.exists(path):
        from exact_io_aware_75_amd.build import build

        build()
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "attn_probe.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))
    assert names == ["attn_probe_exp", "attn_probe_lds", "attn_probe_mfma", "attn_probe_mfma_flops"]
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True).stdout
    for name in names:
        assert re.search(rf"\bT {name}\b", out), name
    lib = ctypes.CDLL(path)
    lib.attn_probe_mfma_flops.restype = ctypes.c_double
    assert lib.attn_probe_mfma_flops(2, 3) == 2 * 4 * 3 * 16 * 2 * 32 * 32 * 16
    assert lib.attn_probe_mfma(None, ctypes.c_void_p(A), 1, 1, None) == 1
    assert lib.attn_probe_mfma(ctypes.c_void_p(A), ctypes.c_void_p(A), 0, 1, None) == 2


def test_probe_library_rejects_bad_arguments_of_every_probe():
    path = os.path.join(ROOT, "exact_io_aware_75_amd", "libattn_probe.so")
    lib = ctypes.CDLL(path)
    assert lib.attn_probe_exp(None, ctypes.c_void_p(A), 1, 1, None) == 1
    assert lib.attn_probe_exp(ctypes.c_void_p(A), ctypes.c_void_p(A), 1, 0, None) == 2
    assert lib.attn_probe_lds(ctypes.c_void_p(A), None, 1, 1, None) == 1
    assert lib.attn_probe_lds(ctypes.c_void_p(A), ctypes.c_void_p(A), (1 << 20) + 1, 1, None) == 2
