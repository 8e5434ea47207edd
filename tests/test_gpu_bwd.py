"""GPU parity of the bf16 backward (fa_bwd through the C ABI) against the
float64 gradient oracle, on the same seeded inputs.

The kernel is fed the library's own forward outputs (O in bf16, LSE), as a
training step would; the oracle recomputes everything from Q, K, V, dO.
Tolerances (per gradient tensor): max |G_gpu - G_ref| <= 2e-2 * max |G_ref|
and ||G_gpu - G_ref|| / ||G_ref|| <= 1e-2.  P and dS enter the matrix cores
in bf16 (relative rounding 2^-9), D comes from the bf16 O, and the outputs
are rounded to bf16 (2^-9 again), so a few units of 2^-9 relative to the
tensor's scale is the expected error.
"""

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import block_rows, dev, nan_filled

pytestmark = pytest.mark.gpu

MAX_TOL = 2e-2
L2_TOL = 1e-2


def _inputs(B, H, Hkv, N, d, seed):
    q, k, v = workloads.qkv(B, H, Hkv, N, d, seed)
    do = workloads.draw((B, H, N, d), seed + 7)
    tb = [workloads.to_bf16(x) for x in (q, k, v, do)]
    return tb, [workloads.bf16_values(t) for t in tb]


def _gpu_backward(tb, causal, scale=None):
    import torch
    import exact_attention_101_amd as fa
    q, k, v, do = (t.to(dev()) for t in tb)
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return [t.float().cpu().numpy() for t in (dq, dk, dv)]


def _compare(got, want, label):
    for name, g, w in zip(("dq", "dk", "dv"), got, want):
        assert np.all(np.isfinite(g)), name
        err = np.abs(g - w)
        scale = np.abs(w).max()
        if scale < 1e-6:
            # An exactly zero gradient: dQ = dK = 0 when scale is 0, or when
            # a row sees a single key (its softmax weight is 1 whatever the
            # score; the kernel's D_i = dO_i . O_i and dP_ii then differ only
            # by fp32 rounding).
            print(f"{label} {name}: zero reference, max|got| {err.max():.3e}")
            assert err.max() <= 1e-3, name
            continue
        rel = np.linalg.norm(g - w) / np.linalg.norm(w)
        print(f"{label} {name}: max|err|/max|ref| {err.max() / scale:.3e} "
              f"rel-L2 {rel:.3e}")
        assert err.max() <= MAX_TOL * scale, name
        assert rel <= L2_TOL, name


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 2, 64), (2, 4, 2, 100),
                                   (1, 2, 1, 257), (1, 1, 1, 1),
                                   (1, 2, 2, 300)],
                         ids=lambda s: "x".join(map(str, s)))
def test_bwd_small_full(shape, causal):
    B, H, Hkv, N = shape
    tb, vals = _inputs(B, H, Hkv, N, 128, 9000 + N)
    got = _gpu_backward(tb, causal)
    want = oracle.attention_backward(*vals, causal=causal)
    _compare(got, want, f"{shape} causal={causal}")


@pytest.mark.parametrize("scale", [-0.05, 0.0])
def test_bwd_scale_sign_and_zero(scale):
    tb, vals = _inputs(1, 2, 2, 130, 128, 9400)
    got = _gpu_backward(tb, False, scale=scale)
    want = oracle.attention_backward(*vals, causal=False, scale=scale)
    _compare(got, want, f"scale={scale}")


def test_bwd_causal_gqa_medium():
    tb, vals = _inputs(1, 8, 2, 1000, 128, 9500)
    got = _gpu_backward(tb, True)
    want = oracle.attention_backward(*vals, causal=True)
    _compare(got, want, "causal gqa 1000")


def test_bwd_full_size_every_head():
    """The headline shape (B4 H16 N8192 d128, non-causal): every KV head, at
    one random row of every 128-row block plus the boundary rows, for dQ
    (every query head of the group) and for dK, dV.  The gradients start as
    NaN, so a block the launches never write fails."""
    import torch
    import exact_attention_101_amd as fa
    w = workloads.WORKLOADS[workloads.HEADLINE]
    tb, vals = _inputs(w.B, w.H, w.Hkv, w.N, w.d, 9700)
    q, k, v, do = (t.to(dev()) for t in tb)
    o, lse = fa.forward(q, k, v, causal=w.causal)
    dq, dk, dv = (nan_filled(t.shape, torch.bfloat16) for t in (q, k, v))
    fa.backward(q, k, v, o, lse, do, causal=w.causal, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    got = [t.float().cpu().numpy() for t in (dq, dk, dv)]
    for g in got:
        assert np.all(np.isfinite(g))
    rows = block_rows(w.N, 128, np.random.default_rng(9701))
    kv_heads = [(b, kvh) for b in range(w.B) for kvh in range(w.Hkv)]
    sq, sk, sv = oracle.attention_backward_sampled(*vals, rows, rows, kv_heads,
                                                   causal=w.causal)
    g = w.H // w.Hkv
    gq = np.stack([[got[0][b, kvh * g + j][rows] for j in range(g)]
                   for b, kvh in kv_heads])
    gk = np.stack([got[1][b, kvh][rows] for b, kvh in kv_heads])
    gv = np.stack([got[2][b, kvh][rows] for b, kvh in kv_heads])
    _compare((gq, gk, gv), (sq, sk, sv), "headline, every KV head")


def test_bwd_deterministic():
    tb, _ = _inputs(1, 4, 2, 600, 128, 9800)
    a = _gpu_backward(tb, True)
    b = _gpu_backward(tb, True)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
