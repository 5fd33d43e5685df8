"""The C-ABI library: it loads, exports every symbol include/fa.h declares,
and rejects bad arguments before touching the GPU.  No compute call is made,
so these run without a GPU."""

import ctypes
import os
import re

import pytest

from exact_attention_51_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_expected_entry_points():
    names = _declared_functions()
    assert names == sorted(
        [
            "fa_fwd",
            "fa_fwd_f32",
            "fa_fwd_kv",
            "fa_fwd_kv_noalloc",
            "fa_fwd_kv_splits",
            "fa_fwd_kv_workspace_bytes",
            "fa_fwd_sparse",
            "fa_bwd_dq",
            "fa_bwd_dkdv",
            "fa_strerror",
            "fa_version",
        ]
    )


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert set(_declared_functions()) == set(_lib.SIGNATURES)


def test_header_signatures_match_binding():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    for name, (_, args) in _lib.SIGNATURES.items():
        m = re.search(rf"\b{name}\s*\(([^)]*)\)", text)
        assert m, name
        params = [p.strip() for p in m.group(1).split(",") if p.strip() and p.strip() != "void"]
        assert len(params) == len(args), (name, params)
        for p, a in zip(params, args):
            if "*" in p:
                assert a is ctypes.c_void_p, (name, p)
            elif p.startswith("float"):
                assert a is ctypes.c_float, (name, p)
            elif p.startswith("size_t"):
                assert a is ctypes.c_size_t, (name, p)
            else:
                assert p.startswith("int") and a is ctypes.c_int, (name, p)


def test_version_and_strerror():
    lib = _lib.load()
    assert lib.fa_version() >> 16 == 1
    for code in (0, -1, -2, -3, 12345):
        s = lib.fa_strerror(code)
        assert isinstance(s, bytes) and len(s) > 0


FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every case below fails validation first


def _fwd(lib, fn="fa_fwd", ptrs=None, B=1, H=1, N=128, D=64, scale=0.125, causal=0):
    ptrs = ptrs or [FAKE] * 5
    return getattr(lib, fn)(*ptrs, B, H, N, D, scale, causal, None)


@pytest.mark.parametrize("fn", ["fa_fwd", "fa_fwd_f32"])
def test_forward_argument_validation(fn):
    lib = _lib.load()
    inv, uns = _lib.FA_ERR_INVALID_ARG, _lib.FA_ERR_UNSUPPORTED
    for i in range(5):
        ptrs = [FAKE] * 5
        ptrs[i] = None
        assert _fwd(lib, fn, ptrs=ptrs) == inv
    assert _fwd(lib, fn, B=0) == inv
    assert _fwd(lib, fn, H=-1) == inv
    assert _fwd(lib, fn, N=0) == inv
    assert _fwd(lib, fn, D=0) == inv
    assert _fwd(lib, fn, scale=0.0) == inv
    assert _fwd(lib, fn, scale=-1.0) == inv
    assert _fwd(lib, fn, scale=float("nan")) == inv
    assert _fwd(lib, fn, scale=float("inf")) == inv
    assert _fwd(lib, fn, causal=2) == inv
    assert _fwd(lib, fn, B=1024, H=1024, N=4096, D=64) == inv  # 2^38 elements
    # head dims no kernel serves (the float32 forward also rejects 96 and 160
    # in its launcher, before any launch)
    for d in (1, 48, 100, 512) + ((32, 96, 160) if fn == "fa_fwd_f32" else ()):
        assert _fwd(lib, fn, D=d) == uns


@pytest.mark.parametrize("fn,nptr", [("fa_bwd_dq", 8), ("fa_bwd_dkdv", 8)])
def test_backward_argument_validation(fn, nptr):
    lib = _lib.load()
    f = getattr(lib, fn)
    inv, uns = _lib.FA_ERR_INVALID_ARG, _lib.FA_ERR_UNSUPPORTED
    for i in range(nptr):
        ptrs = [FAKE] * nptr
        ptrs[i] = None
        assert f(*ptrs, 1, 1, 128, 64, 0.125, 0, None) == inv
    ptrs = [FAKE] * nptr
    assert f(*ptrs, 1, 1, 0, 64, 0.125, 0, None) == inv
    assert f(*ptrs, 1, 1, 128, 64, float("nan"), 0, None) == inv
    assert f(*ptrs, 1, 1, 128, 64, 0.125, 7, None) == inv
    for d in (48, 80, 192, 512):  # head dims no backward kernel serves: rejected before any launch
        assert f(*ptrs, 1, 1, 128, d, 0.125, 0, None) == uns


def _fwd_kv(lib, ptrs=None, B=1, H=1, Nq=16, Nk=300, D=128, scale=0.125, causal=0, splits=4, ws=None, ws_bytes=0):
    ptrs = ptrs or [FAKE] * 5
    return lib.fa_fwd_kv(*ptrs, B, H, Nq, Nk, D, scale, causal, splits, ws, ws_bytes, None)


def test_forward_kv_argument_validation():
    lib = _lib.load()
    inv, uns = _lib.FA_ERR_INVALID_ARG, _lib.FA_ERR_UNSUPPORTED
    need = lib.fa_fwd_kv_workspace_bytes(1, 1, 16, 128, 4)
    assert need == 4 * 16 * 129 * 4
    for i in range(5):
        ptrs = [FAKE] * 5
        ptrs[i] = None
        assert _fwd_kv(lib, ptrs=ptrs, ws=FAKE, ws_bytes=need) == inv
    ok = dict(ws=FAKE, ws_bytes=need)
    assert _fwd_kv(lib, Nq=0, **ok) == inv
    assert _fwd_kv(lib, Nk=0, **ok) == inv
    assert _fwd_kv(lib, scale=float("nan"), **ok) == inv
    assert _fwd_kv(lib, causal=1, Nq=301, Nk=300, **ok) == inv  # causal needs Nq <= Nk
    assert _fwd_kv(lib, splits=-1, **ok) == inv
    assert _fwd_kv(lib, splits=257, **ok) == inv
    assert _fwd_kv(lib, splits=4) == inv  # no workspace
    assert _fwd_kv(lib, splits=4, ws=FAKE, ws_bytes=need - 1) == inv  # short workspace
    assert _fwd_kv(lib, splits=4, ws=ctypes.c_void_p(0x10008), ws_bytes=need) == inv  # misaligned
    assert _fwd_kv(lib, B=1024, H=1024, Nq=16, Nk=4096, D=64, **ok) == inv  # K holds 2^38 elements
    # 2^23 heads x 256 key ranges: more workgroups than a 1-D grid holds
    huge = lib.fa_fwd_kv_workspace_bytes(4096, 2048, 1, 64, 256)
    assert _fwd_kv(lib, B=4096, H=2048, Nq=1, Nk=2, D=64, splits=256, ws=FAKE, ws_bytes=huge) == inv
    for d in (48, 80):
        assert _fwd_kv(lib, D=d, **ok) == uns
    # sizes of the workspace
    assert lib.fa_fwd_kv_workspace_bytes(2, 3, 5, 64, 1) == 0
    assert lib.fa_fwd_kv_workspace_bytes(2, 3, 5, 64, 7) == 7 * 2 * 3 * 5 * 65 * 4
    assert lib.fa_fwd_kv_workspace_bytes(0, 3, 5, 64, 7) == 0
    assert lib.fa_fwd_kv_splits(1, 1, 0, 10, 64, 0) == inv
    assert lib.fa_fwd_kv_splits(1, 1, 10, 5, 64, 1) == inv


def _no_gpu_visible():
    """The two tests below pass sizes that only a host-side check stops; on a
    machine with a GPU a missing check would launch on fake pointers, so they
    run only where no GPU is visible (device_count does not initialise one)."""
    import torch

    if torch.cuda.device_count() > 0:
        pytest.skip("host-side size checks are exercised on machines without a GPU")


def test_forward_kv_work_items_checked_before_launch():
    """HIP's grid limit is on work-items (workgroups x threads < 2^32): 2^24
    query rows merged from 16 ranges need one 256-thread merge workgroup per
    row, 2^32 work-items, which fa_fwd_kv rejects before the range kernel
    runs."""
    _no_gpu_visible()
    lib = _lib.load()
    nq = 1 << 24
    need = lib.fa_fwd_kv_workspace_bytes(1, 1, nq, 32, 16)
    assert _fwd_kv(lib, Nq=nq, Nk=nq, D=32, splits=16, ws=FAKE, ws_bytes=need) == _lib.FA_ERR_INVALID_ARG
    # 8 ranges take the narrow merge (D/4 threads per row): it fits
    need8 = lib.fa_fwd_kv_workspace_bytes(1, 1, nq, 32, 8)
    assert need8 > 0


def test_forward_kv_noalloc_validation():
    """The no-allocation variant rejects what fa_fwd_kv rejects and any range
    count whose partials exceed its scratch array, before any HIP call."""
    _no_gpu_visible()
    lib = _lib.load()
    inv = _lib.FA_ERR_INVALID_ARG

    def call(ptrs=None, B=1, H=64, Nq=4096, Nk=8192, D=128, scale=0.125, causal=0, splits=8):
        ptrs = ptrs or [FAKE] * 5
        return lib.fa_fwd_kv_noalloc(*ptrs, B, H, Nq, Nk, D, scale, causal, splits, None)

    assert lib.fa_fwd_kv_workspace_bytes(1, 64, 4096, 128, 8) > _lib.FA_FWD_KV_NOALLOC_MAX_BYTES
    assert call() == inv  # partials of 8 ranges: 1.08 GB
    for i in range(5):
        ptrs = [FAKE] * 5
        ptrs[i] = None
        assert call(ptrs=ptrs, H=1, Nq=16, splits=4) == inv
    assert call(H=1, Nq=16, splits=257) == inv
    assert call(H=1, Nq=16, splits=-1) == inv
    assert call(H=1, Nq=8193, causal=1) == inv


def test_forward_sparse_argument_validation():
    lib = _lib.load()
    inv, uns = _lib.FA_ERR_INVALID_ARG, _lib.FA_ERR_UNSUPPORTED

    def call(ptrs=None, mask=FAKE, heads=1, B=1, H=2, N=300, D=128, scale=0.125, causal=0):
        ptrs = ptrs or [FAKE] * 5
        return lib.fa_fwd_sparse(*ptrs, B, H, N, D, scale, causal, mask, heads, None)

    for i in range(5):
        ptrs = [FAKE] * 5
        ptrs[i] = None
        assert call(ptrs=ptrs) == inv
    assert call(mask=None) == inv
    assert call(heads=0) == inv
    assert call(heads=3) == inv  # neither 1 nor B*H
    assert call(N=0) == inv
    assert call(scale=float("nan")) == inv
    assert call(D=48) == uns
    assert call(B=1, H=1, N=4096 * 64 + 1, D=64) == uns  # more key tiles than the tile list holds


def test_python_binding_rejects_cpu_tensors():
    import torch

    import exact_attention_51_amd as fa

    x = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fwd(x, x, x)
