"""GPU parity of the variable-length / sliding-window forward
(fa_fwd_varlen through the C ABI) against the oracle's attention_varlen,
on the same seeded bf16 inputs.  Same bars as the square forward:
max |O_gpu - O_oracle| <= 2e-2 and max |LSE_gpu - LSE_oracle| <= 1e-3; a
query that sees no key must give O = 0 and LSE = -inf exactly."""

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import BF16_O_TOL, LSE_TOL, dev

pytestmark = pytest.mark.gpu


def _packed(lens, H, Hkv, seed):
    """Seeded per-sequence inputs, packed per head as the kernel wants."""
    qs, ks, vs = [], [], []
    for i, (nq, nk) in enumerate(lens):
        qs.append(workloads.draw((H, nq, 128), seed + 3 * i))
        ks.append(workloads.draw((Hkv, nk, 128), seed + 3 * i + 1))
        vs.append(workloads.draw((Hkv, nk, 128), seed + 3 * i + 2))
    tq = workloads.to_bf16(np.concatenate(qs, axis=1))
    tk = workloads.to_bf16(np.concatenate(ks, axis=1))
    tv = workloads.to_bf16(np.concatenate(vs, axis=1))
    cq = np.concatenate([[0], np.cumsum([a for a, _ in lens])]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum([b for _, b in lens])]).astype(np.int32)
    # The oracle takes the same bf16 values, split back per sequence.
    qv, kv, vv = (workloads.bf16_values(t) for t in (tq, tk, tv))
    split = lambda x, c: [x[:, c[i]:c[i + 1]] for i in range(len(lens))]
    return (tq, tk, tv, cq, ck), (split(qv, cq), split(kv, ck), split(vv, ck))


def _run(packed, lens, causal, window, scale=None):
    import torch
    import exact_attention_101_amd as fa
    tq, tk, tv, cq, ck = packed
    q, k, v = (t.to(dev()) for t in (tq, tk, tv))
    cuq = torch.from_numpy(cq).to(dev())
    cuk = torch.from_numpy(ck).to(dev())
    o, lse = fa.forward_varlen(q, k, v, cuq, cuk, max(a for a, _ in lens),
                               causal=causal, window=window, scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def _check(o, lse, ro, rl, cq, label):
    ro = np.concatenate(ro, axis=1)
    rl = np.concatenate(rl, axis=1)
    dead = np.isneginf(rl)
    de = np.abs(lse[~dead] - rl[~dead]).max() if (~dead).any() else 0.0
    print(f"{label}: max|dO| {np.abs(o - ro).max():.3e} max|dLSE| {de:.3e} "
          f"rows without keys {int(dead.sum())}")
    assert np.all(np.isfinite(o))
    np.testing.assert_array_equal(np.isneginf(lse), dead)
    assert np.all(o[dead] == 0)
    assert np.abs(o - ro).max() <= BF16_O_TOL
    assert de <= LSE_TOL


LENS = [(200, 200), (1, 1), (37, 90), (129, 64), (300, 301)]


@pytest.mark.parametrize("causal,window", [
    (False, (-1, -1)), (True, (-1, -1)), (False, (40, 7)), (True, (64, -1)),
    (False, (0, 0)), (False, (-1, 33)), (True, (1, -1))])
def test_varlen_windows(causal, window):
    packed, vals = _packed(LENS, 4, 2, 6000)
    o, lse = _run(packed, LENS, causal, window)
    ro, rl = oracle.attention_varlen(*vals, causal=causal,
                                     window_left=window[0],
                                     window_right=window[1])
    _check(o, lse, ro, rl, packed[3], f"causal={causal} window={window}")


def test_varlen_signed_scale_mha():
    lens = [(70, 150), (150, 70)]
    packed, vals = _packed(lens, 2, 2, 6100)
    o, lse = _run(packed, lens, True, (20, -1), scale=-0.06)
    ro, rl = oracle.attention_varlen(*vals, causal=True, window_left=20,
                                     scale=-0.06)
    _check(o, lse, ro, rl, packed[3], "scale -0.06")


def test_varlen_long_sliding_window_sampled():
    """4096-token sequences with a 256-key causal sliding window: rows
    sampled per sequence, against the oracle on the same rows' keys."""
    lens = [(4096, 4096), (3000, 3000)]
    packed, (qs, ks, vs) = _packed(lens, 8, 2, 6200)
    o, lse = _run(packed, lens, True, (256, -1))
    cq = packed[3]
    rows = np.array([0, 1, 255, 256, 257, 1000, 2999])
    for b in range(2):
        # Row i of a sequence with Nq = Nk sees keys [i - 256, i]: the same
        # set as a single query against keys 0 .. i (bottom-right alignment).
        for i in rows:
            (o1,), (l1,) = oracle.attention_varlen(
                [qs[b][:, i:i + 1]], [ks[b][:, :i + 1]], [vs[b][:, :i + 1]],
                causal=True, window_left=256)
            got_o = o[:, cq[b] + i]
            got_l = lse[:, cq[b] + i]
            assert np.abs(got_o - o1[:, 0]).max() <= BF16_O_TOL
            assert np.abs(got_l - l1[:, 0]).max() <= LSE_TOL
    print("long sliding window sampled rows ok")


def test_varlen_deterministic():
    packed, _ = _packed(LENS, 4, 2, 6300)
    a = _run(packed, LENS, True, (50, -1))
    b = _run(packed, LENS, True, (50, -1))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_varlen_long_sequence_narrow_window_sampled():
    """One 131072-token sequence beside a short one, a 512-key causal
    window: sampled rows, each against the oracle on its own window."""
    lens = [(131072, 131072), (100, 100)]
    packed, (qs, ks, vs) = _packed(lens, 2, 1, 6400)
    o, lse = _run(packed, lens, True, (512, -1))
    cq = packed[3]
    for i in (0, 511, 512, 513, 70000, 131071):
        lo = max(0, i - 512)
        (o1,), (l1,) = oracle.attention_varlen(
            [qs[0][:, i:i + 1]], [ks[0][:, lo:i + 1]], [vs[0][:, lo:i + 1]],
            causal=True)
        assert np.abs(o[:, cq[0] + i] - o1[:, 0]).max() <= BF16_O_TOL
        assert np.abs(lse[:, cq[0] + i] - l1[:, 0]).max() <= LSE_TOL
    (o2,), (l2,) = oracle.attention_varlen([qs[1]], [ks[1]], [vs[1]],
                                           causal=True, window_left=512)
    assert np.abs(o[:, cq[1]:cq[2]] - o2).max() <= BF16_O_TOL
    assert np.abs(lse[:, cq[1]:cq[2]] - l2).max() <= LSE_TOL
    print("131072-token sequence, window 512: sampled rows ok")


@pytest.mark.parametrize("causal,window", [(True, (300, -1)),
                                           (False, (100, 50)),
                                           (True, (700, -1)),
                                           (False, (400, 200))])
def test_varlen_window_large_scores(causal, window):
    """Windows whose rows first see a key several blocks into their
    workgroup's key range, with scores large enough that blocks often pass
    the pipelined kernel's sum test: every row against the oracle.  Widths
    below 512 run on the 128-row kernel, the others on the pipelined one."""
    lens = [(1500, 1500), (700, 900)]
    packed, vals = _packed(lens, 4, 2, 6500)
    o, lse = _run(packed, lens, causal, window, scale=0.35)
    ro, rl = oracle.attention_varlen(*vals, causal=causal,
                                     window_left=window[0],
                                     window_right=window[1], scale=0.35)
    _check(o, lse, ro, rl, packed[3], f"scale 0.35 window={window}")


@pytest.mark.parametrize("causal,window", [(True, (-1, -1)), (True, (64, -1)),
                                           (False, (40, 7)), (True, (600, -1)),
                                           (False, (300, 300))])
def test_varlen_kv_heads_multiple_of_8(causal, window):
    """16 query heads on 8 KV heads: the launch then spreads each KV head's
    work over the XCDs by head, not by sequence."""
    packed, vals = _packed(LENS, 16, 8, 6600)
    o, lse = _run(packed, LENS, causal, window)
    ro, rl = oracle.attention_varlen(*vals, causal=causal,
                                     window_left=window[0],
                                     window_right=window[1])
    _check(o, lse, ro, rl, packed[3], f"Hkv 8 causal={causal} window={window}")
