"""The C ABI without a GPU: the library loads, exports every function that
include/fluxattn.h declares, and rejects bad arguments with the documented
status before touching the device.  No compute call is made here."""
import ctypes
import os
import re

import pytest

import joint_attention_head_amd as fa

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "fluxattn.h")

OK, NULLP, SHAPE, ALIGN, ALIAS, NODEV, HIPERR = range(7)


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fluxattn_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return fa.lib()


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(fa.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_status_strings_and_version(lib):
    for s in range(7):
        assert lib.fluxattn_status_string(s).decode()
    assert lib.fluxattn_status_string(99) == b"unknown status"
    assert lib.fluxattn_version() >= 100
    assert lib.fluxattn_last_hip_error() == 0


# Fake, 16-byte aligned, non-overlapping "device" addresses: validation
# rejects every call below before any of them is dereferenced.
B, H, N, D = 1, 2, 320, 128
SZ = B * H * N * D * 2
Q, K, V, O, QO, KO = (0x10000000 * (i + 1) for i in range(6))
WQ, WK, POS = 0x90000000, 0x90001000, 0x90002000
SQ, SK, SV, SQO, SKO = (0xA0000000 + 0x1000 * i for i in range(5))


def prologue(lib, q=Q, k=K, qo=QO, ko=KO, wq=WQ, wk=WK, pos=POS, b=B, h=H, n=N, d=D,
             axes=(16, 56, 56), theta=1e4, eps=1e-6):
    return lib.fluxattn_qk_norm_rope_bf16(q, k, qo, ko, wq, wk, pos, b, h, n, d, *axes, theta, eps, None)


def prologue8(lib, q=Q, k=K, sq=SQ, sk=SK, qo=QO, ko=KO, sqo=SQO, sko=SKO, b=B, h=H, n=N, d=D):
    return lib.fluxattn_qk_norm_rope_fp8(q, k, sq, sk, qo, ko, sqo, sko, WQ, WK, POS, b, h, n, d,
                                         16, 56, 56, 1e4, 1e-6, None)


def forward(lib, q=Q, k=K, v=V, o=O, b=B, h=H, n=N, d=D, scale=0.0):
    return lib.fluxattn_forward_bf16(q, k, v, o, b, h, n, d, scale, None)


def forward8(lib, q=Q, k=K, v=V, sq=SQ, sk=SK, sv=SV, o=O, b=B, h=H, n=N, d=D):
    return lib.fluxattn_forward_fp8(q, k, v, sq, sk, sv, o, b, h, n, d, 0.0, None)


def test_null_pointers(lib):
    for kw in ("q", "k", "qo", "ko", "wq", "wk", "pos"):
        assert prologue(lib, **{kw: None}) == NULLP, kw
    for kw in ("q", "k", "sq", "sk", "qo", "ko", "sqo", "sko"):
        assert prologue8(lib, **{kw: None}) == NULLP, kw
    for kw in ("q", "k", "v", "o"):
        assert forward(lib, **{kw: None}) == NULLP, kw
    for kw in ("q", "k", "v", "sq", "sk", "sv", "o"):
        assert forward8(lib, **{kw: None}) == NULLP, kw


def test_invalid_shapes(lib):
    for kw in ({"b": 0}, {"h": 0}, {"n": 0}, {"d": 64}, {"d": 256}, {"n": (1 << 22) + 1}, {"b": -1}):
        assert prologue(lib, **kw) == SHAPE, kw
        assert forward(lib, **kw) == SHAPE, kw
        assert prologue8(lib, **kw) == SHAPE, kw
        assert forward8(lib, **kw) == SHAPE, kw
    assert prologue(lib, axes=(16, 56, 54)) == SHAPE     # does not sum to D
    assert prologue(lib, axes=(15, 57, 56)) == SHAPE     # odd axis
    assert prologue(lib, axes=(-16, 88, 56)) == SHAPE
    assert prologue(lib, theta=0.0) == SHAPE
    assert prologue(lib, theta=float("nan")) == SHAPE
    assert prologue(lib, eps=-1.0) == SHAPE
    assert prologue(lib, eps=float("inf")) == SHAPE
    assert forward(lib, scale=float("nan")) == SHAPE
    assert forward(lib, scale=float("inf")) == SHAPE


def test_misaligned(lib):
    assert prologue(lib, q=Q + 8) == ALIGN
    assert prologue(lib, ko=KO + 2) == ALIGN
    assert prologue(lib, wq=WQ + 2) == ALIGN
    assert prologue(lib, pos=POS + 1) == ALIGN
    assert forward(lib, o=O + 4) == ALIGN
    assert forward(lib, v=V + 8) == ALIGN
    assert forward8(lib, sv=SV + 2) == ALIGN
    assert prologue8(lib, sqo=SQO + 1) == ALIGN


def test_aliasing(lib):
    # forward output may not overlap any input
    assert forward(lib, o=Q) == ALIAS
    assert forward(lib, o=K + SZ - 16) == ALIAS
    assert forward(lib, o=V - SZ + 16) == ALIAS
    assert forward8(lib, o=SQ - 16) == ALIAS
    # prologue outputs: exact in-place is fine, partial or cross overlap is not
    assert prologue(lib, qo=Q + 16) == ALIAS
    assert prologue(lib, qo=K) == ALIAS
    assert prologue(lib, ko=QO) == ALIAS
    assert prologue(lib, ko=POS - 16) == ALIAS
    assert prologue8(lib, sqo=SQ) == ALIAS
    assert prologue8(lib, sko=SQO) == ALIAS


def test_valid_calls_need_a_gfx950_device(lib):
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:
        has_gpu = False
    if has_gpu:
        pytest.skip("a GPU is present: fake pointers must not reach a launch")
    assert prologue(lib) == NODEV
    assert prologue(lib, qo=Q, ko=K) == NODEV   # exact in-place passes aliasing
    assert prologue8(lib) == NODEV
    assert forward(lib) == NODEV
    assert forward8(lib) == NODEV


def test_python_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 4, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fluxattn_forward_bf16(q, q, q)
