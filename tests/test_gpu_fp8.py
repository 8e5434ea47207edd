"""Parity of the fp8 path (GPU quantisation + e4m3 forward) against the CPU
oracle, through the C ABI (fa_fp8_quantize, fa_fwd_fp8)."""

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import (FP8_LSE_TOL, FP8_REL_L2_TOL, block_rows, dev,
                         nan_filled)

pytestmark = pytest.mark.gpu


def _quant(x, signs=None):
    import torch
    import exact_attention_101_amd as fa
    codes, ad = fa.quantize_fp8(torch.from_numpy(x).to(dev()), signs)
    torch.cuda.synchronize()
    return codes, ad


@pytest.mark.parametrize("rotate", [False, True])
@pytest.mark.parametrize("rows", [1, 7, 1000, 33000, 70001])
def test_quantize_matches_oracle(rotate, rows):
    x = workloads.draw((rows, 128), 1234 + rows, outliers=True)
    signs = workloads.hadamard_signs(128, 9) if rotate else None
    codes, ad = _quant(x, signs)
    g = codes.view(__import__("torch").uint8).cpu().numpy()
    rc, rdesc, ramax = oracle.quantize_per_tensor(x, signs)
    ad = ad.cpu().numpy()
    if not rotate:
        # same fp32 decision on both sides: bit-exact
        assert ad[0] == ramax and ad[1] == rdesc
        np.testing.assert_array_equal(g, rc)
    else:
        # the GPU rotation rounds in fp32 in its own order; codes may differ
        # only where x' * inv lies within a few ulps of a rounding boundary
        assert abs(ad[0] - ramax) <= 4e-6 * ramax
        diff = g != rc
        assert diff.mean() <= 1e-3
        dv = np.abs(oracle.e4m3_decode(g[diff]) - oracle.e4m3_decode(rc[diff]))
        step = np.maximum(np.abs(oracle.e4m3_decode(rc[diff])) * 2.0 ** -3,
                          2.0 ** -9)
        assert np.all(dv <= step * 1.0001)


def test_quantize_zero_tensor():
    codes, ad = _quant(np.zeros((64, 128), np.float32))
    assert np.all(codes.view(__import__("torch").uint8).cpu().numpy() == 0)
    np.testing.assert_array_equal(ad.cpu().numpy(), [0.0, 1.0])


def _fp8_forward(q, k, v, signs, causal, Hkv=None, scale=None):
    import torch
    import exact_attention_101_amd as fa
    q8, sq = _quant(q, signs)
    k8, sk = _quant(k, signs)
    v8, sv = _quant(v, None)
    desc = torch.stack([sq[1], sk[1], sv[1]]).contiguous()
    o, lse = fa.forward_fp8(q8, k8, v8, desc, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def _oracle_deq(x, signs):
    codes, ds, _ = oracle.quantize_per_tensor(x, signs)
    return oracle.e4m3_decode(codes) * float(ds)


@pytest.mark.parametrize("rotate", [False, True])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 2, 256), (2, 4, 2, 300), (1, 2, 2, 1),
                                   (1, 2, 1, 1000)],
                         ids=lambda s: "x".join(map(str, s)))
def test_fp8_small_full(shape, causal, rotate):
    B, H, Hkv, N = shape
    q, k, v = workloads.qkv(B, H, Hkv, N, 128, 5000 + N, outliers=True)
    signs = workloads.hadamard_signs(128, 5009) if rotate else None
    o, lse = _fp8_forward(q, k, v, signs, causal)
    qd, kd, vd = _oracle_deq(q, signs), _oracle_deq(k, signs), _oracle_deq(v, None)
    ro, rl = oracle.attention(qd, kd, vd, causal=causal)
    rel = np.linalg.norm(o - ro) / np.linalg.norm(ro)
    print(f"fp8 rel-L2={rel:.3e} max|dLSE|={np.abs(lse - rl).max():.3e}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert rel <= FP8_REL_L2_TOL


def _fp8_full_size(w, signs):
    """The fp8 workload through the benchmark's launch, O and LSE starting
    as NaN; returns the outputs and the oracle's dequantised inputs."""
    import torch
    import exact_attention_101_amd as fa
    q, k, v = workloads.workload_qkv(w)
    q8, sq = _quant(q, signs)
    k8, sk = _quant(k, signs)
    v8, sv = _quant(v, None)
    desc = torch.stack([sq[1], sk[1], sv[1]]).contiguous()
    o_t = nan_filled((w.B, w.H, w.N, w.d), torch.bfloat16)
    l_t = nan_filled((w.B, w.H, w.N), torch.float32)
    fa.forward_fp8(q8, k8, v8, desc, causal=w.causal, out=o_t, lse=l_t)
    torch.cuda.synchronize()
    deq = (_oracle_deq(q, signs), _oracle_deq(k, signs), _oracle_deq(v, None))
    return o_t.float().cpu().numpy(), l_t.cpu().numpy(), (q, k, v), deq


def test_fp8_full_size_every_block():
    """The fp8 workload at full size, both variants (with and without the
    Hadamard rotation of Q and K).  Every (batch, head) is compared with the
    oracle on its own dequantised inputs on one random row of every 128-row
    query block plus the boundary rows (O: rel-L2 over all of them; LSE:
    FP8_LSE_TOL).  Also measured against the oracle on the unquantised
    inputs: the rotation must lower that error (the direction of the
    FlashAttention-3 summary's claim, section «Baixa precisão»; the size of
    the gain depends on the input distribution, which the pages do not
    give)."""
    w = workloads.WORKLOADS["fp8_n8192"]
    exact_err = {}
    for rotate in (False, True):
        signs = workloads.hadamard_signs(w.d, w.seed(9)) if rotate else None
        o, lse, (q, k, v), (qd, kd, vd) = _fp8_full_size(w, signs)
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
        rng = np.random.default_rng(w.index)
        num = den = num_x = den_x = 0.0
        el = 0.0
        for b in range(w.B):
            for h in range(w.H):
                rows = block_rows(w.N, 128, rng)
                sl = (slice(b, b + 1), slice(h, h + 1))
                ro, rl = oracle.attention_rows(qd[sl], kd[sl], vd[sl], rows)
                go = o[b, h][rows]
                num += float(np.sum((go - ro[0]) ** 2))
                den += float(np.sum(ro[0] ** 2))
                el = max(el, float(np.abs(lse[b, h][rows] - rl[0]).max()))
                rx, _ = oracle.attention_rows(q[sl], k[sl], v[sl], rows)
                num_x += float(np.sum((go - rx[0]) ** 2))
                den_x += float(np.sum(rx[0] ** 2))
        rel = (num / den) ** 0.5
        exact_err[rotate] = (num_x / den_x) ** 0.5
        print(f"fp8 rotate={rotate}: rel-L2 vs dequantised oracle {rel:.3e}, "
              f"max|dLSE| {el:.3e}; vs unquantised inputs "
              f"{exact_err[rotate]:.3e}")
        assert rel <= FP8_REL_L2_TOL, rel
        assert el <= FP8_LSE_TOL, el
    print(f"fp8 error against the unquantised inputs, unrotated / rotated: "
          f"{exact_err[False] / exact_err[True]:.2f}x")
    assert exact_err[True] < exact_err[False]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", ["zero_q", "large_scale", "rising_keys",
                                  "rising_large"])
def test_fp8_reference_moves(case, causal):
    """Inputs that drive the kernel's per-tile reference (block 0's row
    maximum plus a whole power of two that only grows): uniform weights
    (all-zero Q: the reference never moves and every p is 1), a large scale
    (peaky rows, jumps of many powers of two), keys whose norm rises along
    the sequence (the reference keeps moving mid-row) and both together
    (scores rise well over 64 log2 units above block 0, so O and l are
    renormalised mid-row, several times).  Against the oracle on the
    dequantised inputs, same scale."""
    B, H, Hkv, N, d = 1, 2, 2, 1000, 128
    q, k, v = workloads.qkv(B, H, Hkv, N, d, 7100, outliers=False)
    scale = d ** -0.5
    if case == "zero_q":
        q = np.zeros_like(q)
    elif case == "large_scale":
        scale = 12.0 * d ** -0.5
    else:
        if case == "rising_large":
            scale = 12.0 * d ** -0.5
        ramp = np.linspace(0.25, 4.0, N, dtype=np.float32)[None, None, :, None]
        k = (k * ramp).astype(np.float32)
    o, lse = _fp8_forward(q, k, v, None, causal, scale=scale)
    qd, kd, vd = _oracle_deq(q, None), _oracle_deq(k, None), _oracle_deq(v, None)
    ro, rl = oracle.attention(qd, kd, vd, causal=causal, scale=scale)
    rel = np.linalg.norm(o - ro) / np.linalg.norm(ro)
    el = np.abs(lse - rl).max()
    print(f"fp8 {case}: rel-L2={rel:.3e} max|dLSE|={el:.3e}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert rel <= FP8_REL_L2_TOL
    assert el <= FP8_LSE_TOL
