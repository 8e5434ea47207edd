"""Robustness of the boundary on the GPU: caller-supplied outputs are checked
before any launch, the library allocates no device memory, windows wider
than any sequence behave as unbounded ones, and an undersized
max_seqlen_q leaves the rows past it unwritten (as fa.h states)."""

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import BF16_O_TOL, LSE_TOL, dev, nan_filled

pytestmark = pytest.mark.gpu

INT_MAX = 2 ** 31 - 1


def _bf16(B, H, Hkv, N, d, seed):
    q, k, v = workloads.qkv(B, H, Hkv, N, d, seed)
    return tuple(workloads.to_bf16(x).to(dev()) for x in (q, k, v))


def _sentinel(shape, dtype):
    import torch
    return torch.full(tuple(shape), 7.0, dtype=dtype, device=dev())


def test_forward_rejects_bad_output_buffers():
    """Wrong dtype, shape, layout or device for out / lse raises ValueError
    and launches nothing (the buffers passed keep their contents)."""
    import torch
    import exact_attention_101_amd as fa
    q, k, v = _bf16(1, 2, 2, 100, 128, 31)
    good_o = torch.empty_like(q)
    good_l = torch.empty((1, 2, 100), dtype=torch.float32, device=dev())
    bad_outs = [
        _sentinel(q.shape, torch.float32),                 # dtype
        _sentinel((1, 2, 99, 128), torch.bfloat16),        # shape
        _sentinel((1, 2, 128, 100), torch.bfloat16).transpose(2, 3),  # layout
        _sentinel(q.shape, torch.bfloat16).cpu(),          # device
    ]
    for bad in bad_outs:
        before = bad.clone()
        with pytest.raises(ValueError):
            fa.forward(q, k, v, out=bad, lse=good_l)
        torch.cuda.synchronize()
        assert torch.equal(bad, before)
    bad_lses = [
        _sentinel((1, 2, 100), torch.bfloat16),
        _sentinel((1, 2, 101), torch.float32),
        _sentinel((2, 1, 100), torch.float32),
    ]
    for bad in bad_lses:
        before = bad.clone()
        with pytest.raises(ValueError):
            fa.forward(q, k, v, out=good_o, lse=bad)
        torch.cuda.synchronize()
        assert torch.equal(bad, before)


def test_other_entry_points_reject_bad_output_buffers():
    import torch
    import exact_attention_101_amd as fa
    q, k, v = _bf16(1, 2, 2, 64, 128, 32)
    # fp8 forward
    q8, k8, v8 = (x.float().to(torch.float8_e4m3fn) for x in (q, k, v))
    with pytest.raises(ValueError):
        fa.forward_fp8(q8, k8, v8, out=_sentinel((1, 2, 64, 64),
                                                 torch.bfloat16))
    with pytest.raises(ValueError):
        fa.forward_fp8(q8, k8, v8, lse=_sentinel((1, 2, 64), torch.float64))
    # backward
    o, lse = fa.forward(q, k, v)
    with pytest.raises(ValueError):
        fa.backward(q, k, v, o, lse, o, dk=_sentinel((1, 2, 63, 128),
                                                     torch.bfloat16))
    with pytest.raises(ValueError):
        fa.backward(q, k, v, o, lse, o, dq=_sentinel(q.shape, torch.float16))
    # split-KV
    with pytest.raises(ValueError):
        fa.forward_kv(q[:, :, :1].contiguous(), k, v,
                      out=_sentinel((1, 2, 2, 128), torch.bfloat16))
    # masked
    mask = torch.from_numpy(workloads.pack_mask(
        np.ones((64, 64), dtype=bool))[None, None].view(np.int32)).to(dev())
    with pytest.raises(ValueError):
        fa.forward_masked(q, k, v, mask, lse=_sentinel((1, 1, 64),
                                                       torch.float32))
    # quantisation
    x = torch.zeros((8, 128), dtype=torch.float32, device=dev())
    with pytest.raises(ValueError):
        fa.quantize_fp8(x, out=_sentinel((8, 127), torch.uint8))
    with pytest.raises(ValueError):
        fa.quantize_fp8(x, amax_descale=_sentinel((3,), torch.float32))
    torch.cuda.synchronize()


def test_entry_points_allocate_no_device_memory():
    """With every output and workspace preallocated, a call changes neither
    torch's allocator statistics nor the device's free memory: the library
    itself never allocates (linear memory in N is the caller's O and LSE,
    FlashAttention v1 post, section «Итог»)."""
    import torch
    import exact_attention_101_amd as fa
    q, k, v = _bf16(2, 4, 2, 1000, 128, 33)
    o = torch.empty_like(q)
    lse = torch.empty((2, 4, 1000), dtype=torch.float32, device=dev())
    dq, dk, dv = (torch.empty_like(t) for t in (q, k, v))
    ws_b = torch.empty(2 * 2 * 4 * 1000, dtype=torch.float32, device=dev())
    qd = q[:, :, :3].contiguous()
    od = torch.empty_like(qd)
    ld = torch.empty((2, 4, 3), dtype=torch.float32, device=dev())
    ns = 8
    ws_s = torch.empty(ns * 2 * 4 * 3 * 129, dtype=torch.float32,
                       device=dev())
    q8, k8, v8 = (t.float().to(torch.float8_e4m3fn) for t in (q, k, v))

    def calls():
        fa.forward(q, k, v, causal=True, out=o, lse=lse)
        fa.forward_fp8(q8, k8, v8, out=o, lse=lse)
        fa.backward(q, k, v, o, lse, q, causal=True, dq=dq, dk=dk, dv=dv,
                    workspace=ws_b)
        fa.forward_kv(qd, k, v, causal=True, num_splits=ns, out=od, lse=ld,
                      workspace=ws_s)

    calls()                                     # first launches load code
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    used = torch.cuda.memory_allocated()
    free = torch.cuda.mem_get_info()[0]
    for _ in range(3):
        calls()
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated() == used
    assert torch.cuda.mem_get_info()[0] == free


def _varlen_inputs(lens, H, Hkv, seed):
    qs, ks, vs = [], [], []
    for i, (nq, nk) in enumerate(lens):
        qs.append(workloads.draw((H, nq, 128), seed + 3 * i))
        ks.append(workloads.draw((Hkv, nk, 128), seed + 3 * i + 1))
        vs.append(workloads.draw((Hkv, nk, 128), seed + 3 * i + 2))
    t = [workloads.to_bf16(np.concatenate(x, axis=1)) for x in (qs, ks, vs)]
    cq = np.concatenate([[0], np.cumsum([a for a, _ in lens])]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum([b for _, b in lens])]).astype(np.int32)
    return t, cq, ck


@pytest.mark.parametrize("causal,wide,ref", [
    (False, (INT_MAX, INT_MAX), (-1, -1)),
    (False, (INT_MAX, 0), (-1, 0)),
    (True, (INT_MAX, INT_MAX), (-1, -1)),
    (False, (5, INT_MAX), (5, -1)),
])
def test_varlen_window_wider_than_any_sequence(causal, wide, ref):
    """Window widths up to INT_MAX (the header allows any value >= -1) are
    the unbounded window: same bits as -1 (no int overflow in the kernels'
    row + offset + window sums)."""
    import torch
    import exact_attention_101_amd as fa
    lens = [(300, 300), (37, 90), (129, 64)]
    (tq, tk, tv), cq, ck = _varlen_inputs(lens, 4, 2, 6500)
    q, k, v = (t.to(dev()) for t in (tq, tk, tv))
    cuq, cuk = (torch.from_numpy(c).to(dev()) for c in (cq, ck))
    a = fa.forward_varlen(q, k, v, cuq, cuk, causal=causal, window=wide)
    b = fa.forward_varlen(q, k, v, cuq, cuk, causal=causal, window=ref)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_varlen_max_seqlen():
    """max_seqlen_q = None reads the longest sequence from cu_seqlens_q;
    a value below it computes the rows before it and leaves the rows from
    the next 256-row boundary on unwritten (fa.h)."""
    import torch
    import exact_attention_101_amd as fa
    lens = [(300, 300), (1000, 1000)]
    (tq, tk, tv), cq, ck = _varlen_inputs(lens, 2, 2, 6600)
    q, k, v = (t.to(dev()) for t in (tq, tk, tv))
    cuq, cuk = (torch.from_numpy(c).to(dev()) for c in (cq, ck))
    a = fa.forward_varlen(q, k, v, cuq, cuk, None, causal=True)
    b = fa.forward_varlen(q, k, v, cuq, cuk, 1000, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    o = nan_filled(q.shape, torch.bfloat16)
    lse = nan_filled((2, q.shape[1]), torch.float32)
    fa.forward_varlen(q, k, v, cuq, cuk, 600, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    s1 = int(cq[1])                       # second sequence's first row
    # rows before max_seqlen_q: computed, and equal to the full launch
    full_o = b[0].float().cpu().numpy()
    np.testing.assert_array_equal(o[:, :s1 + 600], full_o[:, :s1 + 600])
    # rows from the next 256-row boundary on: untouched
    assert np.all(np.isnan(o[:, s1 + 768:])) and np.all(np.isnan(lse[:, s1 + 768:]))
    # and the short sequence is complete
    vals = [workloads.bf16_values(t) for t in (tq, tk, tv)]
    ro, rl = oracle.attention_varlen([vals[0][:, :s1]], [vals[1][:, :int(ck[1])]],
                                     [vals[2][:, :int(ck[1])]], causal=True)
    assert np.abs(o[:, :s1] - ro[0]).max() <= BF16_O_TOL
    assert np.abs(lse[:, :s1] - rl[0]).max() <= LSE_TOL
