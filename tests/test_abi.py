"""C-ABI contract tests that need no GPU.

The library must load, export every entry point include/fa.h declares, and
reject every invalid argument with its documented status before any HIP call.
Pointers passed here are never dereferenced: each call carries exactly one
invalid argument, so validation returns before a launch could happen.
"""
import ctypes
import math
import os
import re

import pytest

import exact_io_aware_44_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

OK, NULL, SHAPE, UNSUP, ALIGN, WS, LAUNCH, ARG, TOO_LARGE, SCRATCH = range(10)
P = 0x10000          # a 16-byte-aligned stand-in address, never dereferenced
PM = 0x10008         # misaligned by 8 bytes


@pytest.fixture(scope="module")
def lib():
    return fa.load()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert names == ["fa_bwd", "fa_bwd_dropout", "fa_bwd_dropout_f16", "fa_bwd_f16",
                     "fa_bwd_noalloc",
                     "fa_bwd_varlen", "fa_bwd_varlen_dropout", "fa_bwd_varlen_dropout_f16",
                     "fa_bwd_varlen_f16",
                     "fa_bwd_workspace_size", "fa_fwd", "fa_fwd_dropout",
                     "fa_fwd_dropout_f16", "fa_fwd_f16", "fa_fwd_qk", "fa_fwd_qk_f16",
                     "fa_fwd_splitkv",
                     "fa_fwd_splitkv_f16", "fa_fwd_splitkv_workspace_size",
                     "fa_fwd_varlen", "fa_fwd_varlen_dropout", "fa_fwd_varlen_dropout_f16",
                     "fa_fwd_varlen_f16", "fa_status_string"]
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in range(10):
        s = fa.fa_status_string(code)
        assert s.startswith("FA_"), s
    assert "unknown" in fa.fa_status_string(99)
    assert "unknown" in fa.fa_status_string(-1)
    err = fa.FaError(UNSUP, "fa_fwd")
    assert err.status == UNSUP and "FA_ERR_UNSUPPORTED" in str(err)


def fwd(lib, q=P, k=P, v=P, o=P, lse=P, B=1, H=1, N=16, D=64, scale=0.125,
        causal=0):
    return lib.fa_fwd(q, k, v, o, lse, B, H, N, D, scale, causal, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(v=None), NULL),
    (dict(o=None), NULL),
    (dict(B=0), SHAPE), (dict(H=0), SHAPE), (dict(N=0), SHAPE),
    (dict(N=-5), SHAPE), (dict(B=70000), SHAPE), (dict(H=70000), SHAPE),
    (dict(D=96), UNSUP), (dict(D=256), UNSUP), (dict(D=0), UNSUP),
    (dict(causal=2), UNSUP), (dict(causal=-1), UNSUP),
    (dict(scale=0.0), ARG), (dict(scale=-0.1), ARG),
    (dict(scale=float("nan")), ARG), (dict(scale=float("inf")), ARG),
    (dict(q=PM), ALIGN), (dict(k=PM), ALIGN), (dict(v=PM), ALIGN),
    (dict(o=PM), ALIGN), (dict(lse=P + 4), ALIGN),
    (dict(N=1 << 23, D=128), TOO_LARGE), (dict(N=1 << 24, D=64), TOO_LARGE),
    # one row past the largest accepted slice: (N + 256) * D * 2 reaches 2 GiB
    (dict(N=8388352, D=128), TOO_LARGE), (dict(N=16776960, D=64), TOO_LARGE),
])
def test_fwd_rejects(lib, kw, code):
    assert fwd(lib, **kw) == code


def fwd_qk(lib, q=P, k=P, v=P, o=P, lse=P, B=1, H=1, Nq=16, Nk=40, D=64, scale=0.125,
           causal=1):
    return lib.fa_fwd_qk(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(o=None), NULL),
    (dict(B=0), SHAPE), (dict(Nq=0), SHAPE), (dict(Nk=0), SHAPE), (dict(Nk=-3), SHAPE),
    (dict(H=70000), SHAPE), (dict(D=80), UNSUP), (dict(causal=3), UNSUP),
    (dict(scale=float("nan")), ARG), (dict(v=PM), ALIGN), (dict(lse=P + 8), ALIGN),
    (dict(Nk=1 << 23, D=128), TOO_LARGE), (dict(Nq=1 << 24, D=64), TOO_LARGE),
    (dict(Nk=8388352, D=128), TOO_LARGE), (dict(Nk=16776960, D=64), TOO_LARGE),
])
def test_fwd_qk_rejects(lib, kw, code):
    assert fwd_qk(lib, **kw) == code


def splitkv(lib, q=P, k=P, v=P, o=P, lse=P, ws=P, ws_bytes=1 << 30, B=2, H=4, Nq=1,
            Nk=4096, D=128, scale=0.1, causal=1, splits=0):
    return lib.fa_fwd_splitkv(q, k, v, o, lse, ws, ws_bytes, B, H, Nq, Nk, D, scale,
                              causal, splits, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(v=None), NULL), (dict(B=0), SHAPE), (dict(Nk=0), SHAPE),
    (dict(Nq=-1), SHAPE), (dict(D=48), UNSUP), (dict(causal=7), UNSUP),
    (dict(scale=0.0), ARG), (dict(splits=-2), ARG), (dict(o=PM), ALIGN),
    (dict(ws=None), WS), (dict(ws_bytes=1000), WS), (dict(ws=PM), ALIGN),
    (dict(Nk=1 << 23), TOO_LARGE), (dict(Nq=1 << 22), TOO_LARGE),
])
def test_splitkv_rejects(lib, kw, code):
    assert splitkv(lib, **kw) == code


def test_splitkv_workspace_size():
    ws = fa.fa_fwd_splitkv_workspace_size
    # B2 H4 Nq1 Nk4096 (decoding kernel): automatic count min(128, 256/8,
    # 4096/512) = 8 ranges of 512 keys; partial O (8*8 rows * 128 fp32) then
    # partial L (padded to 64 floats)
    assert ws(2, 4, 1, 4096, 128) == 4 * (8 * 8 * 128 + 64)
    # B2 H4 Nq64 Nk4096 (forward tiles): min(128, 512/8, 4096/256) = 16 ranges
    # of 256 keys; partial O (16*8*64 rows * 128 fp32) then partial L
    assert ws(2, 4, 64, 4096, 128) == 4 * (16 * 8 * 64 * 128 + 16 * 8 * 64)
    assert ws(2, 4, 1, 4096, 128, 4) == 4 * (4 * 8 * 128 + 64)
    assert ws(2, 4, 1, 4096, 128, 1) == 0       # one range: plain forward
    assert ws(64, 32, 1, 200, 128) == 0         # enough heads and a short cache
    assert ws(1, 1, 1, 100, 64, 50) == 4 * (2 * 64 + 64)  # at most one range per 64 keys
    assert ws(0, 4, 1, 4096, 128) == 0 and ws(2, 4, 1, 4096, 96) == 0
    assert ws(2, 4, 1, 4096, 128, -1) == 0


@pytest.mark.parametrize("f16", [False, True])
@pytest.mark.parametrize("pdrop,code", [(-0.1, ARG), (1.0, ARG), (1.5, ARG),
                                        (float("nan"), ARG), (float("inf"), ARG)])
def test_dropout_rejects(lib, pdrop, code, f16):
    sfx = "_f16" if f16 else ""
    fwd_d = getattr(lib, "fa_fwd_dropout" + sfx)
    bwd_d = getattr(lib, "fa_bwd_dropout" + sfx)
    assert fwd_d(P, P, P, P, P, 1, 2, 64, 128, 0.1, 1, pdrop, 1, 0, None) == code
    assert bwd_d(P, P, P, P, P, P, P, P, P, P, 1 << 30, 1, 2, 64, 128, 0.1, 1, pdrop, 1, 0,
                 None) == code
    # a valid probability with one other invalid argument reports that one
    assert fwd_d(P, P, P, P, P, 1, 2, 64, 96, 0.1, 1, 0.2, 1, 0, None) == UNSUP
    assert bwd_d(P, P, P, P, P, P, P, P, P, None, 1 << 30, 1, 2, 64, 128, 0.1, 1, 0.2, 1, 0,
                 None) == WS


def varlen(lib, q=P, k=P, v=P, o=P, lse=P, cu=P, nseq=2, total=32, maxlen=16,
           H=2, D=128, scale=0.1, causal=1):
    return lib.fa_fwd_varlen(q, k, v, o, lse, cu, nseq, total, maxlen, H, D,
                             scale, causal, None)


@pytest.mark.parametrize("kw,code", [
    (dict(cu=None), NULL), (dict(q=None), NULL), (dict(o=None), NULL),
    (dict(nseq=0), SHAPE), (dict(total=0), SHAPE), (dict(maxlen=0), SHAPE),
    (dict(H=0), SHAPE), (dict(nseq=70000), SHAPE),
    (dict(D=32), UNSUP), (dict(causal=5), UNSUP), (dict(scale=-1.0), ARG),
    (dict(cu=P + 2), ALIGN), (dict(v=PM), ALIGN),
    (dict(total=1 << 23, D=128), TOO_LARGE),
])
def test_varlen_rejects(lib, kw, code):
    assert varlen(lib, **kw) == code


def test_workspace_size(lib):
    # two fp32 values per row, as two regions each padded to 256 bytes
    assert fa.fa_bwd_workspace_size(2, 32, 4096, 128) == 2 * (2 * 32 * 4096 * 4)
    assert fa.fa_bwd_workspace_size(1, 1, 3, 64) == 2 * 256
    assert fa.fa_bwd_workspace_size(0, 1, 3, 64) == 0
    assert fa.fa_bwd_workspace_size(1, 1, 3, 80) == 0


def bwd(lib, q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, ws=P,
        ws_bytes=1 << 20, B=1, H=2, N=64, D=128, scale=0.1, causal=1):
    return lib.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, ws_bytes, B, H, N, D,
                      scale, causal, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(lse=None), NULL), (dict(do=None), NULL),
    (dict(dq=None), NULL), (dict(dk=None), NULL), (dict(dv=None), NULL),
    (dict(B=0), SHAPE), (dict(N=0), SHAPE), (dict(H=-1), SHAPE),
    (dict(D=100), UNSUP), (dict(causal=7), UNSUP), (dict(scale=0.0), ARG),
    (dict(dk=PM), ALIGN), (dict(lse=P + 4), ALIGN), (dict(ws=PM), ALIGN),
    (dict(ws=None), WS), (dict(ws_bytes=100), WS),
    (dict(N=1 << 24), TOO_LARGE),
])
def test_bwd_rejects(lib, kw, code):
    assert bwd(lib, **kw) == code


def bwd_noalloc(lib, q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=1, H=2, N=64,
                D=128, scale=0.1, causal=1):
    return lib.fa_bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, B, H, N, D, scale, causal,
                              None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(lse=None), NULL), (dict(do=None), NULL),
    (dict(dq=None), NULL), (dict(dk=None), NULL), (dict(dv=None), NULL),
    (dict(B=0), SHAPE), (dict(N=0), SHAPE), (dict(H=-1), SHAPE), (dict(B=70000), SHAPE),
    (dict(D=100), UNSUP), (dict(causal=7), UNSUP), (dict(scale=float("inf")), ARG),
    (dict(dk=PM), ALIGN), (dict(lse=P + 4), ALIGN),
    (dict(N=1 << 24), TOO_LARGE),
    # the static scratch serves 2^21 query rows (B * H * N)
    (dict(B=1, H=32, N=65537), SCRATCH), (dict(B=2, H=32, N=32769), SCRATCH),
    (dict(B=512, H=4097, N=1), SCRATCH),
])
def test_bwd_noalloc_rejects(lib, kw, code):
    """Every invalid argument is rejected before any HIP call; sizes above the
    static scratch return FA_ERR_SCRATCH."""
    assert bwd_noalloc(lib, **kw) == code


def bwd_varlen(lib, q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, cu=P, nseq=2,
               total=32, maxlen=16, ws=P, ws_bytes=1 << 20, H=2, D=128, scale=0.1,
               causal=1):
    return lib.fa_bwd_varlen(q, k, v, o, lse, do, dq, dk, dv, cu, nseq, total, maxlen, ws,
                             ws_bytes, H, D, scale, causal, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(lse=None), NULL), (dict(do=None), NULL),
    (dict(dv=None), NULL), (dict(cu=None), NULL),
    (dict(nseq=0), SHAPE), (dict(total=0), SHAPE), (dict(maxlen=0), SHAPE),
    (dict(H=0), SHAPE), (dict(nseq=70000), SHAPE),
    (dict(D=32), UNSUP), (dict(causal=2), UNSUP), (dict(scale=float("nan")), ARG),
    (dict(cu=P + 2), ALIGN), (dict(dq=PM), ALIGN), (dict(ws=PM), ALIGN),
    (dict(ws=None), WS),
    # one row per packed token and head: H * total fp32 values, twice
    (dict(ws_bytes=2 * 2 * 32 * 4 - 1), WS),
    (dict(total=1 << 23, D=128), TOO_LARGE),
])
def test_bwd_varlen_rejects(lib, kw, code):
    assert bwd_varlen(lib, **kw) == code


@pytest.mark.parametrize("p,code", [(-0.1, ARG), (1.0, ARG), (float("nan"), ARG)])
def test_varlen_dropout_rejects_probability(lib, p, code):
    assert lib.fa_fwd_varlen_dropout(P, P, P, P, P, P, 2, 32, 16, 2, 128, 0.1, 1, p, 1, 0,
                                     None) == code
    assert lib.fa_bwd_varlen_dropout(P, P, P, P, P, P, P, P, P, P, 2, 32, 16, P, 1 << 20, 2,
                                     128, 0.1, 1, p, 1, 0, None) == code


def test_varlen_dropout_validates_like_varlen(lib):
    # one invalid argument each: the packed checks run after the dropout ones
    assert lib.fa_fwd_varlen_dropout(P, P, P, P, P, None, 2, 32, 16, 2, 128, 0.1, 1, 0.1, 1, 0,
                                     None) == NULL
    assert lib.fa_bwd_varlen_dropout(P, P, P, P, P, P, P, P, P, P, 2, 32, 16, P, 100, 2, 128,
                                     0.1, 1, 0.1, 1, 0, None) == WS


def test_bwd_varlen_workspace_is_dense_size_of_packed_rows(lib):
    # fa_bwd_varlen takes fa_bwd_workspace_size(1, H, total, D) bytes
    assert fa.fa_bwd_workspace_size(1, 2, 32, 128) == 2 * 2 * 32 * 4


def test_python_binding_checks_dtypes():
    import torch
    x = torch.zeros(1, 1, 4, 64)
    with pytest.raises(TypeError):
        fa.fa_fwd(x, x, x)
    y = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fa_fwd(y, y, y)  # CPU tensors are refused: no CPU fallback
    z = torch.zeros(1, 1, 4, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        fa.fa_fwd(z, z, z)  # fp16 is accepted as a type, CPU still refused


@pytest.mark.parametrize("name", ["fa_fwd", "fa_fwd_qk", "fa_fwd_splitkv",
                                  "fa_fwd_varlen", "fa_bwd"])
def test_f16_twins_validate_like_bf16(lib, name):
    """The fp16 entry points share the validation of their bf16 twins: the
    same argument list with one invalid value gets the same status."""
    calls = {
        "fa_fwd": lambda f, **kw: f(*[kw.get(n, d) for n, d in (
            ("q", P), ("k", P), ("v", P), ("o", P), ("lse", P), ("B", 1), ("H", 1),
            ("N", 16), ("D", 64), ("s", 0.125), ("c", 0))], None),
        "fa_fwd_qk": lambda f, **kw: f(P, P, P, P, P, 1, 1, 16, kw.get("Nk", 40),
                                       kw.get("D", 64), 0.125, 1, None),
        "fa_fwd_splitkv": lambda f, **kw: f(P, P, P, P, P, kw.get("ws", P), 1 << 30, 2, 4, 1,
                                            4096, kw.get("D", 128), 0.1, 1, 0, None),
        "fa_fwd_varlen": lambda f, **kw: f(P, P, P, P, P, kw.get("cu", P), 2, 32, 16, 2,
                                           kw.get("D", 128), 0.1, 1, None),
        "fa_bwd": lambda f, **kw: f(P, P, P, P, P, P, P, P, P, kw.get("ws", P), 1 << 30, 1, 2,
                                    64, kw.get("D", 128), 0.1, 1, None),
    }
    call = calls[name]
    bf, hf = getattr(lib, name), getattr(lib, name + "_f16")
    for kw, code in ((dict(D=96), UNSUP), (dict(q=None) if name == "fa_fwd" else dict(D=0), None)):
        a, b = call(bf, **kw), call(hf, **kw)
        assert a == b and a != OK and (code is None or a == code)
