"""The FMA-pipe exponential (fa_exp2_fma) against exact 2^x, and the fp8
forward with part of its exponentials on it (fa_fwd_fp8_exp2_fma) against
the CPU oracle, through the C ABI.  The technique is the FlashAttention-4
article's («Оптимизируйте производительность с FlashAttention-4»,
paragraph 3)."""

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import FP8_LSE_TOL, FP8_REL_L2_TOL, block_rows, dev, nan_filled

pytestmark = pytest.mark.gpu

# Relative error bound of the software 2^x on [-125, 127] (fa.h).
EXP2_FMA_REL = 7.5e-5


def _exp2_gpu(x):
    import torch
    import exact_attention_101_amd as fa
    y = fa.exp2_fma(torch.from_numpy(x).to(dev()))
    torch.cuda.synchronize()
    return y.cpu().numpy()


def test_exp2_fma_error_bound():
    rng = np.random.default_rng(5)
    dense = np.linspace(-125.0, 127.0, 3_000_001, dtype=np.float32)
    special = np.concatenate([
        np.arange(-125, 128, dtype=np.float32),                # 2^n
        np.arange(-125, 127, dtype=np.float32) + 0.5,          # rint ties
        np.nextafter(np.arange(-124, 128, dtype=np.float32) - 0.5,
                     np.float32(-np.inf)),
        rng.uniform(-30.0, 9.0, 1_000_000).astype(np.float32),  # softmax range
        np.array([0.0, -0.0, 1e-30, -1e-30, 126.99, -124.99], np.float32),
    ])
    x = np.concatenate([dense, special])
    y = _exp2_gpu(x).astype(np.float64)
    ref = np.exp2(x.astype(np.float64))
    rel = np.abs(y / ref - 1.0)
    print(f"max relative error {rel.max():.3e} over {x.size} points")
    assert np.all(np.isfinite(y))
    assert rel.max() <= EXP2_FMA_REL


def test_exp2_fma_below_range():
    """x < -125 (and -inf) give 2^-125 * p(0) ~ 2.35e-38, a positive normal
    number; above it the result is 2^x to the bound."""
    x = np.array([-np.inf, -1e30, -300.0, -126.0, -125.4], np.float32)
    y = _exp2_gpu(x)
    assert np.all(y > 0) and np.all(y <= 2.36e-38)
    assert np.all(y >= 2.0 ** -125 * 0.9999)


def _quant(x, signs=None):
    import torch
    import exact_attention_101_amd as fa
    codes, ad = fa.quantize_fp8(torch.from_numpy(x).to(dev()), signs)
    return codes, ad


def _oracle_deq(x, signs):
    codes, ds, _ = oracle.quantize_per_tensor(x, signs)
    return oracle.e4m3_decode(codes) * float(ds)


@pytest.mark.parametrize("pairs", [4, 8, 16])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 2, 256), (2, 4, 2, 300),
                                   (1, 2, 1, 1000)],
                         ids=lambda s: "x".join(map(str, s)))
def test_fp8_exp2_fma_small(shape, causal, pairs):
    import torch
    import exact_attention_101_amd as fa
    B, H, Hkv, N = shape
    q, k, v = workloads.qkv(B, H, Hkv, N, 128, 5300 + N, outliers=True)
    q8, sq = _quant(q)
    k8, sk = _quant(k)
    v8, sv = _quant(v)
    desc = torch.stack([sq[1], sk[1], sv[1]]).contiguous()
    o, lse = fa.forward_fp8(q8, k8, v8, desc, causal=causal,
                            exp2_fma_pairs=pairs)
    o0, lse0 = fa.forward_fp8(q8, k8, v8, desc, causal=causal)
    torch.cuda.synchronize()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    o0 = o0.float().cpu().numpy()
    ro, rl = oracle.attention(_oracle_deq(q, None), _oracle_deq(k, None),
                              _oracle_deq(v, None), causal=causal)
    rel = np.linalg.norm(o - ro) / np.linalg.norm(ro)
    rel0 = np.linalg.norm(o0 - ro) / np.linalg.norm(ro)
    el = np.abs(lse - rl).max()
    print(f"pairs={pairs}: rel-L2 {rel:.3e} (v_exp_f32: {rel0:.3e}), "
          f"max|dLSE| {el:.3e}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert rel <= FP8_REL_L2_TOL
    assert el <= FP8_LSE_TOL


def test_fp8_exp2_fma_full_size_every_block():
    """The fp8 workload at full size with half of the exponentials on the
    FMA pipe (the launch the benchmark times): every (batch, head), one
    random row of every 128-row query block plus the boundary rows, against
    the oracle on the dequantised inputs; O and LSE start as NaN."""
    import torch
    import exact_attention_101_amd as fa
    w = workloads.WORKLOADS["fp8_n8192"]
    q, k, v = workloads.workload_qkv(w)
    q8, sq = _quant(q)
    k8, sk = _quant(k)
    v8, sv = _quant(v)
    desc = torch.stack([sq[1], sk[1], sv[1]]).contiguous()
    o_t = nan_filled((w.B, w.H, w.N, w.d), torch.bfloat16)
    l_t = nan_filled((w.B, w.H, w.N), torch.float32)
    fa.forward_fp8(q8, k8, v8, desc, causal=w.causal, out=o_t, lse=l_t,
                   exp2_fma_pairs=8)
    torch.cuda.synchronize()
    o, lse = o_t.float().cpu().numpy(), l_t.cpu().numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    qd, kd, vd = (_oracle_deq(x, None) for x in (q, k, v))
    rng = np.random.default_rng(w.index + 77)
    num = den = el = 0.0
    for b in range(w.B):
        for h in range(w.H):
            rows = block_rows(w.N, 128, rng)
            sl = (slice(b, b + 1), slice(h, h + 1))
            ro, rl = oracle.attention_rows(qd[sl], kd[sl], vd[sl], rows)
            num += float(np.sum((o[b, h][rows] - ro[0]) ** 2))
            den += float(np.sum(ro[0] ** 2))
            el = max(el, float(np.abs(lse[b, h][rows] - rl[0]).max()))
    rel = (num / den) ** 0.5
    print(f"fp8 with 8 FMA-pipe pairs: rel-L2 {rel:.3e}, max|dLSE| {el:.3e}")
    assert rel <= FP8_REL_L2_TOL
    assert el <= FP8_LSE_TOL
