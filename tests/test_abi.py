"""The C ABI without a GPU: the library loads, exports every function that
include/fluxattn.h declares, and rejects bad arguments with the documented
status before touching the device.  No compute call is made here."""
import ctypes
import os
import re

import pytest

import joint_attention_head_amd as fa

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
HEADERS = sorted(os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h"))

OK, NULLP, SHAPE, ALIGN, ALIAS, NODEV, HIPERR, WORKSPACE = range(8)


def declared_functions():
    """Every function the headers under include/ declare."""
    names = set()
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(fluxattn_\w+)\s*\(", src))
    return sorted(names)


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
    for s in range(8):
        assert lib.fluxattn_status_string(s).decode() != "unknown status"
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


KW = 0x70000000
SKW = 0xA0008000


def joint(lib, q=Q, k=K, v=V, kw=KW, o=O, wq=WQ, wk=WK, pos=POS, b=B, h=H, n=N, d=D,
          axes=(16, 56, 56), theta=1e4, eps=1e-6, scale=0.0):
    return lib.fluxattn_joint_attention_bf16(q, k, v, kw, o, wq, wk, pos, b, h, n, d, *axes, theta, eps,
                                             scale, None)


def joint8(lib, q=Q, k=K, v=V, sq=SQ, sk=SK, sv=SV, kw=KW, skw=SKW, o=O, wq=WQ, wk=WK, pos=POS,
           b=B, h=H, n=N, d=D):
    return lib.fluxattn_joint_attention_fp8(q, k, v, sq, sk, sv, kw, skw, o, wq, wk, pos, b, h, n, d,
                                            16, 56, 56, 1e4, 1e-6, 0.0, None)


def fused(lib, q=Q, k=K, v=V, o=O, wq=WQ, pos=POS, b=B, h=H, n=N, d=D, scale=0.0):
    return lib.fluxattn_forward_fused_bf16(q, k, v, o, wq, pos, b, h, n, d, 16, 56, 56, 1e4, 1e-6, scale, None)


def fused8(lib, q=Q, k=K, v=V, sq=SQ, sk=SK, sv=SV, o=O, wq=WQ, pos=POS, b=B, h=H, n=N, d=D):
    return lib.fluxattn_forward_fused_fp8(q, k, v, sq, sk, sv, o, wq, pos, b, h, n, d, 16, 56, 56, 1e4, 1e-6,
                                          0.0, None)


# Split workspace layout: 2 * 16384 int32 arrival counts, then two partial
# slots per workgroup of 512 threads x (64 fp32 accumulators + shifts and
# normalisers of the thread's one or two query rows, a float4).
COUNT_BYTES = 2 * 16384 * 4
SLOT_BYTES = 512 * (64 + 4) * 4


def ws_bytes(lib, b, h, n, groups, d=D):
    out = ctypes.c_uint64(12345)
    st = lib.fluxattn_split_workspace_bytes(b, h, n, d, groups, ctypes.byref(out))
    return st, out.value


def test_split_workspace_bytes_is_host_only(lib):
    """The workspace a split launch needs, computed without a device for an
    explicit workgroup count: N = 1000 gives 4 query blocks of 256 per head
    and 16 key tiles, so B*H = 2 heads are 8 blocks."""
    assert ws_bytes(lib, 1, 2, 1000, 3) == (OK, COUNT_BYTES + 3 * 2 * SLOT_BYTES)
    assert ws_bytes(lib, 1, 2, 1000, 7) == (OK, COUNT_BYTES + 7 * 2 * SLOT_BYTES)
    # more workgroups than blocks: at most one per key tile of the 8 blocks
    assert ws_bytes(lib, 1, 2, 1000, 100) == (OK, COUNT_BYTES + 100 * 2 * SLOT_BYTES)
    assert ws_bytes(lib, 1, 2, 1000, 200) == (OK, COUNT_BYTES + 128 * 2 * SLOT_BYTES)
    assert ws_bytes(lib, 1, 2, 1000, 1) == (OK, 0)        # one workgroup: never cut
    assert ws_bytes(lib, 1, 2, 1000, -1) == (OK, 0)
    assert ws_bytes(lib, 1, 2, 1000, 16384)[0] == OK
    assert ws_bytes(lib, 1, 2, 1000, 16385)[0] == SHAPE
    assert ws_bytes(lib, 1, 2, 1000, 3, d=64)[0] == SHAPE
    assert lib.fluxattn_split_workspace_bytes(1, 2, 1000, D, 3, None) == NULLP
    # the default setting depends on the device's compute units
    assert ws_bytes(lib, 2, 24, 16896, 0)[0] == NODEV


def test_library_imports_no_allocation_or_synchronisation():
    """Every entry point enqueues work and returns: the library does not
    even import an allocation, free, memset or synchronisation call of the
    HIP runtime (the split workspace comes from the caller)."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("binutils nm is not installed")
    out = subprocess.run([nm, "-D", "--undefined-only", fa.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    imported = {line.split()[-1].split("@")[0] for line in out.splitlines() if line.strip()}
    hip = sorted(n for n in imported if n.lower().startswith("hip"))
    assert hip, "no HIP imports found: wrong file?"
    banned = re.compile(r"(Malloc|Free|Memset|Memcpy|Synchronize|StreamCreate|Alloc|HostRegister)", re.I)
    assert [n for n in hip if banned.search(n)] == [], hip


def test_null_pointers(lib):
    for kw in ("q", "k", "qo", "ko", "wq", "wk", "pos"):
        assert prologue(lib, **{kw: None}) == NULLP, kw
    for kw in ("q", "k", "sq", "sk", "qo", "ko", "sqo", "sko"):
        assert prologue8(lib, **{kw: None}) == NULLP, kw
    for kw in ("q", "k", "v", "o"):
        assert forward(lib, **{kw: None}) == NULLP, kw
    for kw in ("q", "k", "v", "sq", "sk", "sv", "o"):
        assert forward8(lib, **{kw: None}) == NULLP, kw
    for kw in ("q", "k", "v", "kw", "o", "wq", "wk", "pos"):
        assert joint(lib, **{kw: None}) == NULLP, kw
    for kw in ("q", "k", "v", "o", "wq", "pos"):
        assert fused(lib, **{kw: None}) == NULLP, kw
    for kw in ("q", "k", "v", "sq", "sk", "sv", "o", "wq", "pos"):
        assert fused8(lib, **{kw: None}) == NULLP, kw
    # keys-only prologue: q, q_out, q_norm_w all NULL; any one of them alone is an error
    assert prologue(lib, q=None, qo=None, wq=None) != NULLP
    assert prologue(lib, q=None, qo=None) == NULLP
    assert prologue(lib, q=None, wq=None) == NULLP
    assert prologue8(lib, q=None, qo=None, sq=None, sqo=None) == NULLP       # q_norm_w still set
    assert lib.fluxattn_qk_norm_rope_fp8(None, K, None, SK, None, KO, None, SKO, None, WK, POS, B, H, N, D,
                                         16, 56, 56, 1e4, 1e-6, None) != NULLP
    for kw in ("q", "k", "v", "sq", "sk", "sv", "kw", "skw", "o", "wq", "wk", "pos"):
        assert joint8(lib, **{kw: None}) == NULLP, kw


def test_invalid_shapes(lib):
    for kw in ({"b": 0}, {"h": 0}, {"n": 0}, {"d": 64}, {"d": 256}, {"n": (1 << 22) + 1}, {"b": -1}):
        assert prologue(lib, **kw) == SHAPE, kw
        assert forward(lib, **kw) == SHAPE, kw
        assert prologue8(lib, **kw) == SHAPE, kw
        assert forward8(lib, **kw) == SHAPE, kw
        assert joint(lib, **kw) == SHAPE, kw
        assert fused(lib, **kw) == SHAPE, kw
        assert fused8(lib, **kw) == SHAPE, kw
        assert joint8(lib, **kw) == SHAPE, kw
    assert joint(lib, axes=(16, 56, 54)) == SHAPE
    assert joint(lib, theta=-1.0) == SHAPE
    assert joint(lib, scale=float("nan")) == SHAPE
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
    assert joint(lib, wq=WQ + 4) == ALIGN        # the fused query load reads 16-byte weight vectors
    assert fused(lib, wq=WQ + 4) == ALIGN
    assert fused8(lib, sq=SQ + 2) == ALIGN
    assert joint(lib, kw=KW + 8) == ALIGN
    assert joint8(lib, skw=SKW + 2) == ALIGN


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
    # fused path: k_work may be k itself, nothing else may overlap
    assert joint(lib, kw=K + 16) == ALIAS
    assert joint(lib, kw=V) == ALIAS
    assert joint(lib, o=KW) == ALIAS
    assert joint(lib, o=Q + 32) == ALIAS
    assert joint8(lib, skw=SK) == ALIAS          # scales read while the new ones are written
    assert joint8(lib, skw=SQ) == ALIAS
    assert fused(lib, o=K) == ALIAS
    assert fused(lib, o=WQ - 64) == ALIAS
    assert fused8(lib, o=SV) == ALIAS


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
    assert joint(lib) == NODEV
    assert joint(lib, kw=K) == NODEV             # in place passes aliasing
    assert joint8(lib) == NODEV
    assert fused(lib) == NODEV
    assert fused8(lib) == NODEV
    assert prologue(lib, q=None, qo=None, wq=None) == NODEV
    assert lib.fluxattn_qk_norm_rope_fp8(None, K, None, SK, None, KO, None, SKO, None, WK, POS, B, H, N, D,
                                         16, 56, 56, 1e4, 1e-6, None) == NODEV


def test_python_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 4, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fluxattn_forward_bf16(q, q, q)
