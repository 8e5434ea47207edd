"""The C-ABI library loads without a GPU, exports every entry point that
include/fa.h declares, and rejects bad arguments before touching the GPU."""

import ctypes
import os
import re

import pytest

import exact_attention_101_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.lib_path):
        from exact_attention_101_amd import build
        build.build()
    return fa.library()


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("fa_fwd", "fa_fwd_fp8", "fa_bwd", "fa_fwd_splitkv",
              "fa_fwd_varlen", "fa_fwd_masked",
              "fa_splitkv_num_splits", "fa_fp8_quantize",
              "fa_fwd_splitkv_noalloc",
              "fa_status_string",
              "fa_last_hip_error", "fa_version"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for n in _declared():
        assert hasattr(lib, n), n


def test_probe_library_exports_its_header():
    """libfa_probe.so (issue-rate probes, measurement support) exports what
    include/fa_probe.h declares, and rejects bad arguments without a GPU."""
    from exact_attention_101_amd import build
    if not os.path.exists(build.PROBE_LIB):
        build.build()
    text = open(os.path.join(ROOT, "include", "fa_probe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))
    assert names == ["fa_probe_rates", "fa_probe_read"]
    plib = ctypes.CDLL(build.PROBE_LIB)
    for n in names:
        assert hasattr(plib, n), n
    r = plib.fa_probe_read
    r.argtypes = [ctypes.c_void_p, ctypes.c_ulonglong, ctypes.c_int,
                  ctypes.c_void_p, ctypes.c_void_p]
    r.restype = ctypes.c_int
    S = ctypes.c_void_p(0x2000)                          # never dereferenced
    assert r(None, 1 << 20, 8, S, None) == 1             # null source
    assert r(S, 1 << 20, 8, None, None) == 1             # null sink
    assert r(S, 0, 8, S, None) == 1                      # nothing to read
    assert r(S, (1 << 20) + 8, 8, S, None) == 1          # not 16-byte units
    assert r(ctypes.c_void_p(0x2008), 1 << 20, 8, S, None) == 1  # misaligned
    assert r(S, 1 << 20, 0, S, None) == 1                # empty grid
    f = plib.fa_probe_rates
    f.argtypes = [ctypes.c_int] * 6 + [ctypes.c_void_p] * 3
    f.restype = ctypes.c_int
    assert f(1, 0, 4, 1, 8, 1, None, None, None) == 1    # null output
    assert f(1, 0, 6, 1, 8, 1, A, None, None) == 1       # waves not 4k
    assert f(1, 0, 4, 2, 8, 1, A, None, None) == 1       # na > waves / 4
    assert f(99, 0, 4, 1, 8, 1, A, None, None) == 1      # unknown body
    assert f(0, 0, 4, 1, 8, 1, A, None, None) == 1       # body a idle
    assert f(12, 0, 4, 1, 8, 1, A, None, None) == 1      # data body, no data
    assert f(12, 0, 4, 1, 8, 1, A, M, None) == 1         # data misaligned
    assert f(13, 1, 8, 1, 8, 1, A, A, None) == 1         # data body mixed
    assert f(18, 1, 8, 1, 8, 1, A, None, None) == 1      # same-wave mix mixed
    assert f(21, 1, 8, 1, 8, 1, A, None, None) == 1      # slot body mixed
    assert f(23, 2, 8, 1, 8, 1, A, None, None) == 1      # LDS body mixed
    assert f(30, 0, 4, 1, 8, 1, A, None, None) == 1      # past the last body
    assert f(27, 0, 4, 1, 8, 1, A, None, None) == 1      # copy body, no data
    assert f(26, 1, 8, 1, 8, 1, A, None, None) == 1      # slot body mixed


def test_version_and_status_strings(lib):
    assert lib.fa_version() == 100
    for s in range(0, 6):
        assert lib.fa_status_string(s)
    assert lib.fa_last_hip_error() == 0


# Fake, never-dereferenced device addresses: validation must fail before any
# HIP call.
A = 0x10000          # 16-byte aligned
M = 0x10008          # misaligned


def _fwd(lib, q=A, k=A, v=A, o=A, lse=A, B=1, H=2, Hkv=2, N=8, d=128,
         causal=0, scale=0.1, dtype=0):
    return lib.fa_fwd(q, k, v, o, lse, B, H, Hkv, N, d, causal, scale, dtype,
                      None)


@pytest.mark.parametrize("kw", [dict(q=None), dict(k=None), dict(v=None),
                                dict(o=None), dict(lse=None), dict(B=0),
                                dict(H=0), dict(Hkv=0), dict(N=0), dict(d=0),
                                dict(N=-3), dict(H=6, Hkv=4),
                                dict(scale=float("nan")),
                                dict(scale=float("inf")),
                                dict(B=1 << 20, H=1 << 20, N=1 << 10)])
def test_invalid_arguments(lib, kw):
    assert _fwd(lib, **kw) == fa.FA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("kw", [dict(d=96), dict(d=256), dict(d=32),
                                dict(dtype=7)])
def test_unsupported(lib, kw):
    assert _fwd(lib, **kw) == fa.FA_ERR_UNSUPPORTED


def test_fp8_only_d128(lib):
    assert _fwd(lib, d=64, dtype=1) == fa.FA_ERR_UNSUPPORTED
    assert lib.fa_fwd_fp8(A, A, A, A, A, 1, 1, 1, 8, 64, 0, 0.1, None,
                          None) == fa.FA_ERR_UNSUPPORTED


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "lse"])
def test_misaligned(lib, which):
    assert _fwd(lib, **{which: M}) == fa.FA_ERR_MISALIGNED


def test_invalid_before_unsupported_before_misaligned(lib):
    assert _fwd(lib, q=M, d=96, N=0) == fa.FA_ERR_INVALID_ARGUMENT
    assert _fwd(lib, q=M, d=96) == fa.FA_ERR_UNSUPPORTED


def test_noalloc_splitkv_validation(lib):
    """The entry point without a workspace checks its arguments like
    fa_fwd_splitkv, then whether the sizes fit its fixed scratch (4 Mi
    floats), before touching the GPU."""
    f = lib.fa_fwd_splitkv_noalloc
    f.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 7 + \
        [ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
    f.restype = ctypes.c_int
    ok = (1, 8, 2, 1, 4096, 128, 1, 0.1, 8)
    assert f(None, A, A, A, A, *ok, None) == fa.FA_ERR_INVALID_ARGUMENT
    assert f(A, A, A, A, A, 1, 8, 2, 1, 4096, 128, 1, 0.1, 0,
             None) == fa.FA_ERR_INVALID_ARGUMENT
    assert f(A, A, A, A, A, 1, 8, 2, 1, 4096, 64, 1, 0.1, 8,
             None) == fa.FA_ERR_UNSUPPORTED
    assert f(M, A, A, A, A, *ok, None) == fa.FA_ERR_MISALIGNED
    # 256 splits x 16384 rows x 129 floats > 4 Mi floats
    assert f(A, A, A, A, A, 2, 16, 4, 512, 4096, 128, 1, 0.1, 256,
             None) == fa.FA_ERR_WORKSPACE
    # the scratch check comes last: a misaligned pointer is reported first
    assert f(M, A, A, A, A, 2, 16, 4, 512, 4096, 128, 1, 0.1, 256,
             None) == fa.FA_ERR_MISALIGNED
    assert b"scratch" in lib.fa_status_string(fa.FA_ERR_WORKSPACE)


def test_quantize_validation(lib):
    signs = (ctypes.c_int8 * 128)(*([1] * 128))
    bad = (ctypes.c_int8 * 128)(*([1] * 127 + [0]))
    q = lib.fa_fp8_quantize
    assert q(None, A, A, 4, 128, None, None) == fa.FA_ERR_INVALID_ARGUMENT
    assert q(A, A, A, 0, 128, None, None) == fa.FA_ERR_INVALID_ARGUMENT
    assert q(A, A, A, 4, 128, bad, None) == fa.FA_ERR_INVALID_ARGUMENT
    assert q(A, A, A, 4, 64, None, None) == fa.FA_ERR_UNSUPPORTED
    assert q(M, A, A, 4, 128, signs, None) == fa.FA_ERR_MISALIGNED


def test_python_wrapper_raises_without_gpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.forward(x, x, x)


def _bwd(lib, q=A, k=A, v=A, o=A, lse=A, do=A, dq=A, dk=A, dv=A, ws=A, B=1,
         H=2, Hkv=2, N=8, d=128, causal=0, scale=0.1):
    return lib.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, B, H, Hkv, N, d,
                      causal, scale, None)


@pytest.mark.parametrize("kw", [dict(q=None), dict(o=None), dict(lse=None),
                                dict(do=None), dict(dq=None), dict(dk=None),
                                dict(dv=None), dict(ws=None), dict(N=0),
                                dict(H=6, Hkv=4), dict(scale=float("nan"))])
def test_bwd_invalid_arguments(lib, kw):
    assert _bwd(lib, **kw) == fa.FA_ERR_INVALID_ARGUMENT


def test_bwd_only_d128(lib):
    assert _bwd(lib, d=64) == fa.FA_ERR_UNSUPPORTED


@pytest.mark.parametrize("name", ["q", "do", "dq", "dk", "dv", "ws"])
def test_bwd_misaligned(lib, name):
    assert _bwd(lib, **{name: M}) == fa.FA_ERR_MISALIGNED


def _skv(lib, q=A, k=A, v=A, o=A, lse=A, B=1, H=4, Hkv=2, Nq=1, Nk=100,
         d=128, causal=0, scale=0.1, splits=4, ws=A):
    return lib.fa_fwd_splitkv(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, causal,
                              scale, splits, ws, None)


@pytest.mark.parametrize("kw", [dict(q=None), dict(lse=None), dict(ws=None),
                                dict(Nq=0), dict(Nk=0), dict(H=6, Hkv=4),
                                dict(splits=0), dict(splits=257),
                                dict(scale=float("inf"))])
def test_splitkv_invalid_arguments(lib, kw):
    assert _skv(lib, **kw) == fa.FA_ERR_INVALID_ARGUMENT


def test_splitkv_only_d128_and_alignment(lib):
    assert _skv(lib, d=64) == fa.FA_ERR_UNSUPPORTED
    assert _skv(lib, ws=M) == fa.FA_ERR_MISALIGNED
    assert _skv(lib, k=M) == fa.FA_ERR_MISALIGNED


def test_splitkv_num_splits(lib):
    assert lib.fa_splitkv_num_splits(0, 4, 2, 1, 100) == 0
    for args in ((1, 32, 8, 1, 32768), (8, 32, 8, 4, 4096), (1, 4, 4, 1, 1),
                 (64, 64, 64, 16, 1 << 20)):
        s = lib.fa_splitkv_num_splits(*args)
        assert 1 <= s <= 256
        assert s <= max(1, -(-args[4] // 32) // 4)


def _vl(lib, q=A, k=A, v=A, o=A, lse=A, cq=A, ck=A, B=2, H=4, Hkv=2,
        tq=100, tk=120, mq=60, d=128, causal=0, wl=-1, wr=-1, scale=0.1):
    return lib.fa_fwd_varlen(q, k, v, o, lse, cq, ck, B, H, Hkv, tq, tk, mq, d,
                             causal, wl, wr, scale, None)


@pytest.mark.parametrize("kw", [dict(q=None), dict(cq=None), dict(ck=None),
                                dict(B=0), dict(tq=0), dict(tk=0), dict(mq=0),
                                dict(H=6, Hkv=4), dict(wl=-2), dict(wr=-5),
                                dict(scale=float("nan"))])
def test_varlen_invalid_arguments(lib, kw):
    assert _vl(lib, **kw) == fa.FA_ERR_INVALID_ARGUMENT


def test_varlen_only_d128_and_alignment(lib):
    assert _vl(lib, d=64) == fa.FA_ERR_UNSUPPORTED
    assert _vl(lib, q=M) == fa.FA_ERR_MISALIGNED
    assert _vl(lib, cq=A + 2) == fa.FA_ERR_MISALIGNED


def _mk(lib, q=A, k=A, v=A, o=A, lse=A, mask=A, mbs=0, mhs=0, B=2, H=4,
        Hkv=2, Nq=100, Nk=120, d=128, scale=0.1):
    return lib.fa_fwd_masked(q, k, v, o, lse, mask, mbs, mhs, B, H, Hkv, Nq,
                             Nk, d, scale, None)


@pytest.mark.parametrize("kw", [dict(q=None), dict(mask=None), dict(B=0),
                                dict(Nq=0), dict(Nk=0), dict(H=6, Hkv=4),
                                dict(mbs=-1), dict(mhs=-3),
                                dict(scale=float("inf"))])
def test_masked_invalid_arguments(lib, kw):
    assert _mk(lib, **kw) == fa.FA_ERR_INVALID_ARGUMENT


def test_masked_unsupported_and_alignment(lib):
    assert _mk(lib, d=64) == fa.FA_ERR_UNSUPPORTED
    assert _mk(lib, Nk=262145) == fa.FA_ERR_UNSUPPORTED
    assert _mk(lib, Nk=262144, q=M) == fa.FA_ERR_MISALIGNED
    assert _mk(lib, mask=A + 2) == fa.FA_ERR_MISALIGNED
    assert _mk(lib, lse=A + 1) == fa.FA_ERR_MISALIGNED



def test_fp8_exp2_fma_validation(lib):
    """The fp8 forward with FMA-pipe exponentials checks its arguments like
    fa_fwd_fp8; fma_pairs other than 0, 4, 8, 16 is unsupported, reported
    in the same place as an unsupported d."""
    g = lib.fa_fwd_fp8_exp2_fma

    def call(q=A, N=8, d=128, pairs=8, desc=None):
        return g(q, A, A, A, A, 1, 2, 2, N, d, 0, 0.1, desc, pairs, None)

    for pairs in (1, 2, 3, 5, 12, 32, -4):
        assert call(pairs=pairs) == fa.FA_ERR_UNSUPPORTED
    assert call(d=64) == fa.FA_ERR_UNSUPPORTED
    assert call(N=0, pairs=3) == fa.FA_ERR_INVALID_ARGUMENT
    assert call(q=None) == fa.FA_ERR_INVALID_ARGUMENT
    assert call(q=M) == fa.FA_ERR_MISALIGNED
    assert call(desc=A + 2) == fa.FA_ERR_MISALIGNED
    assert call(q=M, pairs=5) == fa.FA_ERR_UNSUPPORTED


def test_exp2_fma_validation(lib):
    f = lib.fa_exp2_fma
    assert f(None, A, 4, None) == fa.FA_ERR_INVALID_ARGUMENT
    assert f(A, None, 4, None) == fa.FA_ERR_INVALID_ARGUMENT
    assert f(A, A, -1, None) == fa.FA_ERR_INVALID_ARGUMENT
    assert f(A + 2, A, 4, None) == fa.FA_ERR_MISALIGNED
    assert f(A, A + 1, 4, None) == fa.FA_ERR_MISALIGNED
    assert f(A + 4, A + 4, 0, None) == fa.FA_OK        # nothing enqueued
