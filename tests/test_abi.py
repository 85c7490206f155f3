"""The C ABI: the library loads, exports every declared symbol, sizes its
workspace on the host, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

from rank_lm_head_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lrhead.h")

A = ctypes.c_void_p(0x10000)        # aligned stand-ins: never dereferenced
MIS = ctypes.c_void_p(0x10008)      # 8-byte aligned only


def declared_functions() -> list:
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)
    return [n for n in names if n not in ("defined",)]


def test_library_loads_and_exports_every_declared_function():
    lib = _lib.load()
    names = declared_functions()
    assert set(names) == set(_lib.SIGNATURES), names
    for n in names:
        assert hasattr(lib, n), n


def test_workspace_bytes_host_only():
    lib = _lib.load()
    ws = lib.lrhead_workspace_bytes
    assert ws(_lib.BF16, 151936, 5120, 128, 1, 32) > 0
    assert ws(_lib.BF16, 151936, 5120, 128, 2048, 64) >= ws(_lib.BF16, 151936, 5120, 128, 64, 64)
    assert ws(_lib.BF16, 151936, 5120, 128, 64, 64) >= ws(_lib.BF16, 151936, 5120, 128, 64, 32)
    # z (B_max x r) alone bounds it from below
    assert ws(_lib.BF16, 151936, 5120, 256, 2048, 64) >= 2048 * 256 * 2
    for bad in [(7, 100, 64, 16, 1, 4),          # dtype
                (_lib.BF16, 0, 64, 16, 1, 1),    # V
                (_lib.BF16, 100, 60, 16, 1, 4),  # d % 8
                (_lib.BF16, 100, 64, 12, 1, 4),  # r % 8
                (_lib.BF16, 100, 64, 520, 1, 4),  # r > 512
                (_lib.BF16, 100, 64, 16, 0, 4),  # B_max
                (_lib.BF16, 100, 64, 16, 1, 65),  # k_max > 64
                (_lib.BF16, 10, 64, 16, 1, 11)]:  # k_max > V
        assert ws(*bad) == 0, bad


def _create(dtype=_lib.BF16, V=1000, d=64, r=16, Q=A, P=A, W=A, B_max=4, k_max=8, wsp=A, wsb=1 << 30):
    lib = _lib.load()
    h = ctypes.c_void_p()
    return lib.lrhead_create(ctypes.byref(h), dtype, V, d, r, Q, P, W, B_max, k_max, wsp, wsb)


@pytest.mark.parametrize("kwargs,code", [
    (dict(dtype=3), _lib.EDTYPE),
    (dict(V=0), _lib.ERANGE),
    (dict(d=12), _lib.ERANGE),
    (dict(r=520), _lib.ERANGE),
    (dict(B_max=0), _lib.ERANGE),
    (dict(k_max=0), _lib.ERANGE),
    (dict(k_max=65), _lib.ERANGE),
    (dict(V=5, k_max=6), _lib.ERANGE),
    (dict(Q=None), _lib.EINVAL),
    (dict(W=None), _lib.EINVAL),
    (dict(wsp=None), _lib.EINVAL),
    (dict(P=MIS), _lib.EALIGN),
    (dict(wsp=MIS), _lib.EALIGN),
    (dict(wsb=16), _lib.EWORKSPACE),
])
def test_create_rejects_bad_arguments_before_hip(kwargs, code):
    assert _create(**kwargs) == code
    assert _lib.load().lrhead_last_error()


def test_calls_reject_null_handle():
    lib = _lib.load()
    out = ctypes.c_void_p(0x20000)
    assert lib.lrhead_candidates(None, A, 1, 4, out, None, None) == _lib.EINVAL
    assert lib.fullhead_logits(None, A, 1, out, 4, out, None) == _lib.EINVAL
    assert lib.fullhead_topk(None, A, 1, 4, out, out, None) == _lib.EINVAL
    assert lib.lrhead_draft(None, A, 1, 4, out, None, out, None) == _lib.EINVAL
    lib.lrhead_destroy(None)        # a no-op


def test_branch_rejects_bad_arguments_before_hip():
    lib = _lib.load()
    p = ctypes.c_void_p(0x20000)
    args = lambda B, k, nb, ptr=p: (ptr, ptr, None, B, k, nb, ptr, ptr, ptr, ptr, None)
    assert lib.lrhead_branch(*args(1, 0, 1)) == _lib.ERANGE       # k < 1
    assert lib.lrhead_branch(*args(1, 65, 1)) == _lib.ERANGE      # k > 64
    assert lib.lrhead_branch(*args(1, 8, 9)) == _lib.ERANGE       # nb > k
    assert lib.lrhead_branch(*args(1, 8, 0)) == _lib.ERANGE
    assert lib.lrhead_branch(*args(-1, 8, 2)) == _lib.ERANGE
    assert lib.lrhead_branch(*args(1, 8, 2, None)) == _lib.EINVAL
    assert lib.lrhead_branch(*args(0, 8, 2, None)) == _lib.OK      # B == 0 enqueues nothing


def test_strerror_covers_every_code():
    lib = _lib.load()
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        assert lib.lrhead_strerror(code) != b"unknown error code"
    assert lib.lrhead_strerror(-99) == b"unknown error code"


def test_python_binding_refuses_cpu_tensors():
    import torch
    import rank_lm_head_amd as lr
    Q = torch.zeros(16, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        lr.Head(Q, torch.zeros(100, 16, dtype=torch.bfloat16), torch.zeros(100, 64, dtype=torch.bfloat16),
                B_max=1, k_max=4)


def test_factor_validates_on_the_host():
    lib = _lib.load()
    assert lib.lrhead_factor_workspace_bytes(151936, 5120, 128) > 0
    assert lib.lrhead_factor_workspace_bytes(100, 64, 65) == 0        # r > d
    assert lib.lrhead_factor_workspace_bytes(100, 64, 0) == 0
    p = ctypes.c_void_p(0x20000)
    n = lib.lrhead_factor_workspace_bytes(1000, 64, 8)
    assert lib.lrhead_factor(p, 1000, 64, 513, 1, p, p, p, p, n, None) == _lib.ERANGE
    assert lib.lrhead_factor(p, 1000, 64, 8, 9, p, p, p, p, n, None) == _lib.ERANGE
    assert lib.lrhead_factor(p, 1000, 64, 8, 1, None, p, p, p, n, None) == _lib.EINVAL
    assert lib.lrhead_factor(p, 1000, 64, 8, 1, ctypes.c_void_p(0x20004), p, p, p, n, None) == _lib.EALIGN
    assert lib.lrhead_factor(p, 1000, 64, 8, 1, p, p, p, p, n - 1, None) == _lib.EWORKSPACE
