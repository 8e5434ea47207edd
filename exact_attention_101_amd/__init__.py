"""MI355X (gfx950) FlashAttention forward: thin Python binding of libfa.so.

Every step of the computation runs in the HIP kernels of libfa.so; this
module only checks tensor metadata, allocates outputs with torch (device
memory) and passes pointers plus torch's current HIP stream through ctypes.
There is no fallback: if libfa.so is missing or cannot be loaded, every call
raises.

    o, lse = forward(q, k, v, causal=False, scale=None)
    q8, amax_descale = quantize_fp8(x, signs=None)
    o, lse = forward_fp8(q8, k8, v8, descale_qkv, causal=False, scale=None)

Shapes: q [B, H, N, d], k/v [B, Hkv, N, d] (contiguous), o like q (bf16),
lse [B, H, N] (fp32, natural log).
"""

from __future__ import annotations

import ctypes
import math
import os

__all__ = ["forward", "forward_kv", "forward_kv_noalloc", "forward_varlen", "forward_masked", "backward", "forward_fp8", "exp2_fma", "quantize_fp8", "library", "lib_path",
           "FaError", "FA_DTYPE_BF16", "FA_DTYPE_FP8_E4M3"]

FA_DTYPE_BF16 = 0
FA_DTYPE_FP8_E4M3 = 1

FA_OK = 0
FA_ERR_INVALID_ARGUMENT = 1
FA_ERR_UNSUPPORTED = 2
FA_ERR_MISALIGNED = 3
FA_ERR_HIP = 4
FA_ERR_WORKSPACE = 5

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libfa.so")
_lib = None


class FaError(RuntimeError):
    """A non-OK status from libfa.so."""


def library() -> ctypes.CDLL:
    """Load libfa.so (once).  Raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise ImportError(
                f"{lib_path} is not built; run "
                "`python -m exact_attention_101_amd.build` first")
        lib = ctypes.CDLL(lib_path)
        vp, i32, f32, i64 = (ctypes.c_void_p, ctypes.c_int, ctypes.c_float,
                             ctypes.c_longlong)
        lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                               i32, f32, i32, vp]
        lib.fa_fwd.restype = i32
        lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                   i32, i32, f32, vp, vp]
        lib.fa_fwd_fp8.restype = i32
        lib.fa_fwd_fp8_exp2_fma.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32,
                                            i32, i32, i32, f32, vp, i32, vp]
        lib.fa_fwd_fp8_exp2_fma.restype = i32
        lib.fa_exp2_fma.argtypes = [vp, vp, i64, vp]
        lib.fa_exp2_fma.restype = i32
        lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32,
                               i32, i32, i32, i32, i32, f32, vp]
        lib.fa_bwd.restype = i32
        lib.fa_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32,
                                       i32, i32, i32, i32, f32, i32, vp, vp]
        lib.fa_fwd_splitkv.restype = i32
        lib.fa_fwd_splitkv_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i32,
                                               i32, i32, i32, i32, i32, f32,
                                               i32, vp]
        lib.fa_fwd_splitkv_noalloc.restype = i32
        lib.fa_splitkv_num_splits.argtypes = [i32, i32, i32, i32, i32]
        lib.fa_splitkv_num_splits.restype = i32
        lib.fa_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32,
                                      i32, i32, i32, i32, i32, i32, i32, i32,
                                      f32, vp]
        lib.fa_fwd_varlen.restype = i32
        lib.fa_fwd_masked.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i32,
                                      i32, i32, i32, i32, i32, f32, vp]
        lib.fa_fwd_masked.restype = i32
        lib.fa_fp8_quantize.argtypes = [vp, vp, vp, i64, i32, vp, vp]
        lib.fa_fp8_quantize.restype = i32
        lib.fa_status_string.argtypes = [i32]
        lib.fa_status_string.restype = ctypes.c_char_p
        lib.fa_last_hip_error.argtypes = []
        lib.fa_last_hip_error.restype = i32
        lib.fa_version.argtypes = []
        lib.fa_version.restype = i32
        _lib = lib
    return _lib


def _check(status: int) -> None:
    if status == FA_OK:
        return
    lib = library()
    msg = lib.fa_status_string(status).decode()
    if status == FA_ERR_HIP:
        raise FaError(f"{msg} (hipError {lib.fa_last_hip_error()})")
    raise ValueError(msg)


def _stream_handle(device) -> int:
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def _out_check(t, name, shape, dtypes, device, align=16):
    """A caller-supplied output buffer must be exactly what the kernels
    write: the expected dtype and shape, contiguous, on the inputs' device
    and aligned as the C ABI requires.  Anything else raises ValueError
    before any launch (a smaller buffer would be written past its end)."""
    if not isinstance(dtypes, tuple):
        dtypes = (dtypes,)
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must be {' or '.join(map(str, dtypes))}, "
                         f"got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got "
                         f"{tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if t.data_ptr() % align:
        raise ValueError(f"{name} must be {align}-byte aligned")
    return t


def _shape_check(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H(kv), N, d]")
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    B, H, N, d = q.shape
    if k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError("k/v shape does not match q")
    for t in (q, k, v):
        if not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous")
        if not t.is_cuda or t.device != q.device:
            raise ValueError("q, k, v must be on the same GPU")
    return B, H, k.shape[1], N, d


def forward(q, k, v, *, causal: bool = False, scale=None, out=None,
            lse=None):
    """bf16 attention forward.  Returns (o bf16 [B,H,N,d], lse fp32 [B,H,N])."""
    import torch
    B, H, Hkv, N, d = _shape_check(q, k, v)
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or \
            v.dtype != torch.bfloat16:
        raise ValueError("forward expects bfloat16 q, k, v")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _out_check(out, "out", q.shape, torch.bfloat16, q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _out_check(lse, "lse", (B, H, N), torch.float32, q.device)
    _check(library().fa_fwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
        lse.data_ptr(), B, H, Hkv, N, d, int(bool(causal)), float(scale),
        FA_DTYPE_BF16, _stream_handle(q.device)))
    return out, lse


def forward_kv(q, k, v, *, causal: bool = False, scale=None, num_splits=None,
               out=None, lse=None, workspace=None):
    """bf16 forward of Nq queries against Nk keys with the key range split
    across workgroups (decode).  q: [B,H,Nq,128]; k, v: [B,Hkv,Nk,128];
    causal uses bottom-right alignment.  Returns (o bf16 [B,H,Nq,128], lse
    fp32 [B,H,Nq])."""
    import torch
    for t in (q, k, v):
        if t.dim() != 4 or not t.is_contiguous() or not t.is_cuda or \
                t.dtype != torch.bfloat16 or t.device != q.device:
            raise ValueError("forward_kv expects contiguous 4-D bfloat16 "
                             "tensors on one GPU")
    B, H, Nq, d = q.shape
    _, Hkv, Nk, dk = k.shape
    if k.shape != v.shape or k.shape[0] != B or dk != d:
        raise ValueError("k/v shape does not match q")
    lib = library()
    if num_splits is None:
        num_splits = lib.fa_splitkv_num_splits(B, H, Hkv, Nq, Nk) or 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _out_check(out, "out", q.shape, torch.bfloat16, q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _out_check(lse, "lse", (B, H, Nq), torch.float32, q.device)
    need = num_splits * B * H * Nq * (d + 1)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.float32, device=q.device)
    elif workspace.dtype != torch.float32 or workspace.numel() < need or \
            not workspace.is_contiguous() or workspace.device != q.device or \
            workspace.data_ptr() % 16:
        raise ValueError(f"workspace must be a contiguous, 16-byte aligned "
                         f"float32 tensor of at least {need} elements on "
                         f"{q.device}")
    _check(lib.fa_fwd_splitkv(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
        lse.data_ptr(), B, H, Hkv, Nq, Nk, d, int(bool(causal)), float(scale),
        int(num_splits), workspace.data_ptr(), _stream_handle(q.device)))
    return out, lse


def forward_kv_noalloc(q, k, v, out, lse, *, causal: bool = False,
                       scale=None, num_splits=None):
    """forward_kv for callers that cannot allocate (graph capture, serving
    loops): the caller passes out and lse, and the splits' partial results
    go to the library's fixed per-device scratch (fa_fwd_splitkv_noalloc), so
    nothing is allocated.  Sizes whose num_splits * B * H * Nq * (d + 1)
    exceed that scratch raise ValueError; calls that overlap on one GPU
    race."""
    import torch
    for t in (q, k, v):
        if t.dim() != 4 or not t.is_contiguous() or not t.is_cuda or \
                t.dtype != torch.bfloat16 or t.device != q.device:
            raise ValueError("forward_kv_noalloc expects contiguous 4-D "
                             "bfloat16 tensors on one GPU")
    B, H, Nq, d = q.shape
    _, Hkv, Nk, dk = k.shape
    if k.shape != v.shape or k.shape[0] != B or dk != d:
        raise ValueError("k/v shape does not match q")
    _out_check(out, "out", q.shape, torch.bfloat16, q.device)
    _out_check(lse, "lse", (B, H, Nq), torch.float32, q.device)
    lib = library()
    if num_splits is None:
        num_splits = lib.fa_splitkv_num_splits(B, H, Hkv, Nq, Nk) or 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check(lib.fa_fwd_splitkv_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
        lse.data_ptr(), B, H, Hkv, Nq, Nk, d, int(bool(causal)), float(scale),
        int(num_splits), _stream_handle(q.device)))
    return out, lse


def forward_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q=None, *,
                   causal: bool = False, window=(-1, -1), scale=None, out=None,
                   lse=None):
    """bf16 forward over a packed batch of sequences of different lengths,
    with an optional sliding window (left, right; -1 = unbounded).
    q: [H, total_q, 128]; k, v: [Hkv, total_k, 128]; cu_seqlens_q/k: int32
    CUDA tensors of B + 1 row offsets.  max_seqlen_q: the longest query
    sequence; None reads it from cu_seqlens_q (one device-to-host copy).  A
    value below the longest sequence leaves that sequence's rows past it
    unwritten.  Returns (o bf16 [H, total_q, 128], lse fp32 [H, total_q])."""
    import torch
    for t in (q, k, v):
        if t.dim() != 3 or not t.is_contiguous() or not t.is_cuda or \
                t.dtype != torch.bfloat16 or t.device != q.device:
            raise ValueError("forward_varlen expects contiguous 3-D bfloat16 "
                             "tensors on one GPU")
    for t in (cu_seqlens_q, cu_seqlens_k):
        if t.dtype != torch.int32 or t.dim() != 1 or not t.is_cuda or \
                not t.is_contiguous() or t.device != q.device:
            raise ValueError("cu_seqlens must be contiguous int32 CUDA "
                             "tensors")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or \
            cu_seqlens_q.numel() < 2:
        raise ValueError("cu_seqlens_q and cu_seqlens_k need B + 1 entries")
    H, total_q, d = q.shape
    Hkv, total_k, dk = k.shape
    if k.shape != v.shape or dk != d:
        raise ValueError("k/v shape does not match q")
    if max_seqlen_q is None:
        max_seqlen_q = max(int((cu_seqlens_q[1:] - cu_seqlens_q[:-1]).max()),
                           1)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _out_check(out, "out", q.shape, torch.bfloat16, q.device)
    if lse is None:
        lse = torch.empty((H, total_q), dtype=torch.float32, device=q.device)
    _out_check(lse, "lse", (H, total_q), torch.float32, q.device, align=4)
    wl, wr = window
    _check(library().fa_fwd_varlen(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
        lse.data_ptr(), cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(),
        cu_seqlens_q.numel() - 1, H, Hkv, total_q, total_k, int(max_seqlen_q),
        d, int(bool(causal)), int(wl), int(wr), float(scale),
        _stream_handle(q.device)))
    return out, lse


def forward_masked(q, k, v, mask, *, scale=None, out=None, lse=None):
    """bf16 forward under an arbitrary visibility mask.  q: [B, H, Nq, 128];
    k, v: [B, Hkv, Nk, 128]; mask: int32 (or uint32) CUDA tensor of packed
    bits [Bm, Hm, Nq, ceil(Nk / 32)] with Bm in (1, B) and Hm in (1, H) (a
    size-1 axis is shared): bit j % 32 of word j // 32 of row i set means
    query i sees key j.  Returns (o bf16 [B, H, Nq, 128], lse fp32
    [B, H, Nq]); rows that see no key get o = 0, lse = -inf."""
    import torch
    for t in (q, k, v):
        if t.dim() != 4 or not t.is_contiguous() or not t.is_cuda or \
                t.dtype != torch.bfloat16 or t.device != q.device:
            raise ValueError("forward_masked expects contiguous 4-D bfloat16 "
                             "tensors on one GPU")
    B, H, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if k.shape != v.shape or Bk != B or dk != d:
        raise ValueError("k/v shape does not match q")
    W = (Nk + 31) // 32
    if mask.dtype not in (torch.int32, getattr(torch, "uint32", torch.int32)) \
            or mask.dim() != 4 or not mask.is_contiguous() or \
            not mask.is_cuda or mask.device != q.device:
        raise ValueError("mask must be a contiguous 4-D int32 CUDA tensor")
    Bm, Hm, Nqm, Wm = mask.shape
    if Bm not in (1, B) or Hm not in (1, H) or Nqm != Nq or Wm != W:
        raise ValueError(f"mask must be [1|{B}, 1|{H}, {Nq}, {W}]")
    bstride = Hm * Nq * W if (Bm == B and B > 1) else 0
    hstride = Nq * W if (Hm == H and H > 1) else 0
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _out_check(out, "out", q.shape, torch.bfloat16, q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _out_check(lse, "lse", (B, H, Nq), torch.float32, q.device, align=4)
    _check(library().fa_fwd_masked(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
        lse.data_ptr(), mask.data_ptr(), bstride, hstride, B, H, Hkv, Nq, Nk,
        d, float(scale), _stream_handle(q.device)))
    return out, lse


def backward(q, k, v, o, lse, dout, *, causal: bool = False, scale=None,
             dq=None, dk=None, dv=None, workspace=None):
    """bf16 attention backward (d = 128): gradients of the forward that
    produced o and lse, for the output gradient dout.  Returns (dq, dk, dv),
    bfloat16, shaped like q, k, v.  workspace: optional float32 tensor of
    2 * B * H * N elements (allocated if None)."""
    import torch
    B, H, Hkv, N, d = _shape_check(q, k, v)
    for t in (q, k, v, o, dout):
        if t.dtype != torch.bfloat16:
            raise ValueError("backward expects bfloat16 q, k, v, o, dout")
    for t in (o, dout):
        if t.shape != q.shape or not t.is_contiguous() or t.device != q.device:
            raise ValueError("o and dout must be contiguous and shaped like q")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N) or \
            not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if dq is None:
        dq = torch.empty_like(q)
    if dk is None:
        dk = torch.empty_like(k)
    if dv is None:
        dv = torch.empty_like(v)
    for t, name, ref in ((dq, "dq", q), (dk, "dk", k), (dv, "dv", v)):
        _out_check(t, name, ref.shape, torch.bfloat16, q.device)
    if workspace is None:
        workspace = torch.empty(2 * B * H * N, dtype=torch.float32,
                                device=q.device)
    elif workspace.dtype != torch.float32 or workspace.numel() < 2 * B * H * N \
            or not workspace.is_contiguous() or workspace.device != q.device \
            or workspace.data_ptr() % 16:
        raise ValueError("workspace must be a contiguous, 16-byte aligned "
                         "float32 tensor of at least 2 * B * H * N elements")
    _check(library().fa_bwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
        lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
        dv.data_ptr(), workspace.data_ptr(), B, H, Hkv, N, d,
        int(bool(causal)), float(scale), _stream_handle(q.device)))
    return dq, dk, dv


def forward_fp8(q8, k8, v8, descale_qkv=None, *, causal: bool = False,
                scale=None, out=None, lse=None, exp2_fma_pairs: int = 0):
    """e4m3 attention forward.  q8/k8/v8: torch.float8_e4m3fn or uint8 codes;
    descale_qkv: device float32 tensor of 3 descales (or None for 1).
    exp2_fma_pairs (0, 4, 8 or 16): how many of the 16 weight pairs a lane
    forms per 64-key tile take the FMA-pipe exponential
    (fa_fwd_fp8_exp2_fma); 0 is fa_fwd_fp8.
    Returns (o bf16, lse fp32)."""
    import torch
    B, H, Hkv, N, d = _shape_check(q8, k8, v8)
    for t in (q8, k8, v8):
        if t.dtype not in (torch.float8_e4m3fn, torch.uint8):
            raise ValueError("forward_fp8 expects float8_e4m3fn/uint8 codes")
    if descale_qkv is not None:
        if descale_qkv.dtype != torch.float32 or descale_qkv.numel() != 3 or \
                not descale_qkv.is_cuda or not descale_qkv.is_contiguous():
            raise ValueError("descale_qkv must be a contiguous float32 CUDA "
                             "tensor of 3 elements")
        if descale_qkv.device != q8.device:
            raise ValueError(f"descale_qkv must be on {q8.device}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device)
    _out_check(out, "out", (B, H, N, d), torch.bfloat16, q8.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    _out_check(lse, "lse", (B, H, N), torch.float32, q8.device)
    desc = descale_qkv.data_ptr() if descale_qkv is not None else None
    if exp2_fma_pairs:
        _check(library().fa_fwd_fp8_exp2_fma(
            q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), out.data_ptr(),
            lse.data_ptr(), B, H, Hkv, N, d, int(bool(causal)), float(scale),
            desc, int(exp2_fma_pairs), _stream_handle(q8.device)))
    else:
        _check(library().fa_fwd_fp8(
            q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), out.data_ptr(),
            lse.data_ptr(), B, H, Hkv, N, d, int(bool(causal)), float(scale),
            desc, _stream_handle(q8.device)))
    return out, lse


def exp2_fma(x, *, out=None):
    """2^x elementwise by the FMA-pipe exponential of the fp8 forward's
    exp2_fma_pairs option (fa_exp2_fma).  x: contiguous float32 CUDA tensor.
    Returns a float32 tensor like x."""
    import torch
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("exp2_fma expects a contiguous float32 CUDA tensor")
    if out is None:
        out = torch.empty_like(x)
    _out_check(out, "out", x.shape, torch.float32, x.device, align=4)
    _check(library().fa_exp2_fma(x.data_ptr(), out.data_ptr(), x.numel(),
                                 _stream_handle(x.device)))
    return out


def quantize_fp8(x, signs=None, *, out=None, amax_descale=None):
    """Per-tensor e4m3 quantisation of a contiguous float32 CUDA tensor whose
    last dimension is 128, with an optional +-1 sign vector for the Hadamard
    rotation.  Returns (codes as torch.float8_e4m3fn, amax_descale float32
    [2] = {amax, descale})."""
    import torch
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("quantize_fp8 expects a contiguous float32 CUDA tensor")
    d = x.shape[-1]
    rows = x.numel() // d if d else 0
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _out_check(out, "out", x.shape, (torch.uint8, torch.float8_e4m3fn),
               x.device)
    if amax_descale is None:
        amax_descale = torch.empty(2, dtype=torch.float32, device=x.device)
    _out_check(amax_descale, "amax_descale", (2,), torch.float32, x.device,
               align=4)
    sign_buf = None
    if signs is not None:
        import numpy as np
        s = np.ascontiguousarray(np.asarray(signs, dtype=np.int8).reshape(-1))
        if s.shape[0] != d:
            raise ValueError("signs must have length d")
        sign_buf = s
    _check(library().fa_fp8_quantize(
        x.data_ptr(), out.data_ptr(), amax_descale.data_ptr(), rows, d,
        sign_buf.ctypes.data if sign_buf is not None else None,
        _stream_handle(x.device)))
    return out.view(torch.float8_e4m3fn), amax_descale
