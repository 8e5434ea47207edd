"""Race check of the forward kernels' LDS pipelines: the race-check build
(libfa_serial.so, built from the same sources with FA_SERIAL_COPIES=1, in
which every batch of tile copies sits between workgroup barriers and is
waited for at once) must give the same bits as the pipelined library, which
reads one LDS stage while the copies into the other are in flight.  A stage
read before its copies land, or overwritten while a wave still reads it,
would make the two differ."""

import ctypes
import os

import numpy as np
import pytest

import workloads
from gpu_helpers import dev

pytestmark = pytest.mark.gpu


def _serial_lib():
    from exact_attention_101_amd import build
    if not os.path.exists(build.SERIAL_LIB):
        pytest.fail(f"{build.SERIAL_LIB} is not built (run the build first)")
    lib = ctypes.CDLL(build.SERIAL_LIB)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.fa_fwd.argtypes = [vp] * 5 + [i32] * 6 + [f32, i32, vp]
    lib.fa_fwd.restype = i32
    lib.fa_fwd_fp8.argtypes = [vp] * 5 + [i32] * 6 + [f32, vp, vp]
    lib.fa_fwd_fp8.restype = i32
    lib.fa_fwd_varlen.argtypes = [vp] * 7 + [i32] * 10 + [f32, vp]
    lib.fa_fwd_varlen.restype = i32
    i64 = ctypes.c_longlong
    lib.fa_fwd_masked.argtypes = [vp] * 6 + [i64, i64] + [i32] * 6 + [f32, vp]
    lib.fa_fwd_masked.restype = i32
    return lib


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,Hkv,N", [(2, 4, 2, 2000), (1, 8, 8, 4096),
                                       (1, 2, 1, 333)])
def test_bf16_forward_serial_equals_pipelined(B, H, Hkv, N, d, causal):
    import torch
    import exact_attention_101_amd as fa
    q, k, v = workloads.qkv(B, H, Hkv, N, d, 8000 + N + d)
    qb, kb, vb = (workloads.to_bf16(x).to(dev()) for x in (q, k, v))
    o1, l1 = fa.forward(qb, kb, vb, causal=causal)
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    lib = _serial_lib()
    assert lib.fa_fwd(qb.data_ptr(), kb.data_ptr(), vb.data_ptr(),
                      o2.data_ptr(), l2.data_ptr(), B, H, Hkv, N, d,
                      int(causal), d ** -0.5, 0, _stream()) == 0
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_forward_serial_equals_pipelined(causal):
    import torch
    import exact_attention_101_amd as fa
    B, H, N = 2, 4, 3000
    q, k, v = workloads.qkv(B, H, H, N, 128, 8100, outliers=True)
    c8 = []
    for x in (q, k, v):
        codes, ad = fa.quantize_fp8(torch.from_numpy(x).to(dev()))
        c8.append((codes, ad[1]))
    desc = torch.stack([c[1] for c in c8]).contiguous()
    q8, k8, v8 = (c[0] for c in c8)
    o1, l1 = fa.forward_fp8(q8, k8, v8, desc, causal=causal)
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    lib = _serial_lib()
    assert lib.fa_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(),
                          o2.data_ptr(), l2.data_ptr(), B, H, H, N, 128,
                          int(causal), 128 ** -0.5, desc.data_ptr(),
                          _stream()) == 0
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_varlen_forward_serial_equals_pipelined():
    """The variable-length configuration of the pipelined kernel (causal,
    wide window): 8 waves of 32 rows and per-sequence key ranges."""
    import torch
    import exact_attention_101_amd as fa
    lens = [1500, 300, 2500, 77]
    H, Hkv, tot = 4, 2, sum(lens)
    q = workloads.draw((H, tot, 128), 8200)
    k = workloads.draw((Hkv, tot, 128), 8201)
    v = workloads.draw((Hkv, tot, 128), 8202)
    qb, kb, vb = (workloads.to_bf16(x).to(dev()) for x in (q, k, v))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]),
                      dtype=torch.int32, device=dev())
    o1, l1 = fa.forward_varlen(qb, kb, vb, cu, cu, max(lens), causal=True,
                               window=(1000, -1))
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    lib = _serial_lib()
    assert lib.fa_fwd_varlen(qb.data_ptr(), kb.data_ptr(), vb.data_ptr(),
                             o2.data_ptr(), l2.data_ptr(), cu.data_ptr(),
                             cu.data_ptr(), len(lens), H, Hkv, tot, tot,
                             max(lens), 128, 1, 1000, -1, 128 ** -0.5,
                             _stream()) == 0
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("kind", ["block_sparse", "random", "causal"])
def test_masked_forward_serial_equals_pipelined(kind):
    """The masked configuration (128-row workgroups over the listed key
    tiles, mask words fetched with the K copies): block-sparse (whole
    tiles), random (every tile partial) and causal-shaped masks, a ragged
    key count and a shared mask."""
    import torch
    import exact_attention_101_amd as fa
    B, H, Hkv, Nq, Nk = 2, 4, 2, 700, 1000
    q = workloads.draw((B, H, Nq, 128), 8300)
    k = workloads.draw((B, Hkv, Nk, 128), 8301)
    v = workloads.draw((B, Hkv, Nk, 128), 8302)
    qb, kb, vb = (workloads.to_bf16(x).to(dev()) for x in (q, k, v))
    if kind == "block_sparse":
        m = workloads.block_sparse_mask(Nq, Nk, 128, 2, 8303)
    elif kind == "random":
        m = workloads.random_mask((Nq, Nk), 0.3, 8304)
    else:
        m = np.tril(np.ones((Nq, Nk), dtype=bool), k=Nk - Nq)
    mw = torch.from_numpy(workloads.pack_mask(m).view(np.int32)).to(dev())
    o1, l1 = fa.forward_masked(qb, kb, vb, mw[None, None])
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    lib = _serial_lib()
    assert lib.fa_fwd_masked(qb.data_ptr(), kb.data_ptr(), vb.data_ptr(),
                             o2.data_ptr(), l2.data_ptr(), mw.data_ptr(), 0,
                             0, B, H, Hkv, Nq, Nk, 128, 128 ** -0.5,
                             _stream()) == 0
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
