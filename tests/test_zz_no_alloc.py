"""The entry point that allocates nothing, fa_fwd_splitkv_noalloc (for
callers that cannot allocate: graph capture, serving loops), against the
split-KV entry point with a caller workspace, through the C ABI: two calls
in a row on the same GPU, the second with a smaller input, each bitwise
equal to the workspace entry point's output and within the bf16 bars of
the oracle."""

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import BF16_O_TOL, LSE_TOL, dev

pytestmark = pytest.mark.gpu

# B, H, Hkv, Nq, Nk, causal, splits: the second call is the smaller one.
CASES = [(4, 32, 8, 2, 9000, True, 16), (1, 8, 2, 1, 3000, False, 4)]


def test_noalloc_equals_workspace_entry_point_twice():
    import torch
    import exact_attention_101_amd as fa
    lib = fa.library()
    stream = torch.cuda.current_stream().cuda_stream
    for B, H, Hkv, Nq, Nk, causal, ns in CASES:
        q = workloads.draw((B, H, Nq, 128), 9100 + Nk)
        k = workloads.draw((B, Hkv, Nk, 128), 9101 + Nk)
        v = workloads.draw((B, Hkv, Nk, 128), 9102 + Nk)
        tb = [workloads.to_bf16(x) for x in (q, k, v)]
        qd, kd, vd = (t.to(dev()) for t in tb)
        o1, l1 = fa.forward_kv(qd, kd, vd, causal=causal, num_splits=ns)
        o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
        rc = lib.fa_fwd_splitkv_noalloc(
            qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o2.data_ptr(),
            l2.data_ptr(), B, H, Hkv, Nq, Nk, 128, int(causal), 128 ** -0.5,
            ns, stream)
        assert rc == fa.FA_OK
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        ro, rl = oracle.attention_kv(*(workloads.bf16_values(t) for t in tb),
                                     causal=causal)
        go, gl = o2.float().cpu().numpy(), l2.cpu().numpy()
        print(f"B{B} H{H} Nq{Nq} Nk{Nk}: max|dO| {np.abs(go - ro).max():.3e} "
              f"max|dLSE| {np.abs(gl - rl).max():.3e}")
        assert np.abs(go - ro).max() <= BF16_O_TOL
        assert np.abs(gl - rl).max() <= LSE_TOL


def test_noalloc_rejects_sizes_beyond_its_scratch():
    import torch
    import exact_attention_101_amd as fa
    lib = fa.library()
    B, H, Hkv, Nq, Nk = 2, 16, 4, 64, 4096        # 256 * 2048 * 129 > 4 Mi
    q = torch.zeros((B, H, Nq, 128), dtype=torch.bfloat16, device=dev())
    k = torch.zeros((B, Hkv, Nk, 128), dtype=torch.bfloat16, device=dev())
    o = torch.full_like(q, 3.0)
    lse = torch.full((B, H, Nq), 3.0, device=dev())
    rc = lib.fa_fwd_splitkv_noalloc(
        q.data_ptr(), k.data_ptr(), k.data_ptr(), o.data_ptr(),
        lse.data_ptr(), B, H, Hkv, Nq, Nk, 128, 1, 0.1, 256,
        torch.cuda.current_stream().cuda_stream)
    assert rc == fa.FA_ERR_WORKSPACE
    with pytest.raises(ValueError, match="scratch"):
        fa.forward_kv_noalloc(q, k, k, o, lse, num_splits=256)
    torch.cuda.synchronize()
    assert torch.all(o == 3.0) and torch.all(lse == 3.0)   # nothing ran
