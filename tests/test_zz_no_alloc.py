"""The allocation-free decode (entmax_attn_decode_noalloc: static per-device
scratch instead of a workspace) against the decode with a caller workspace,
through the C ABI, on two calls in a row with the second input smaller.

Bar (as for every forward result): tau within 1e-4 * max(1, |tau|), o within
2e-3 for bf16 inputs and 1e-5 for fp32 inputs.  Both calls run the same
kernels on the same inputs, so they are expected to agree exactly; the test
reports whether they do."""
import math

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

CASES = [
    # (B, H, L, cache_len, d, dtype, mask, window, seed): the first large, the second smaller
    (4, 8, 5000, 5200, 128, "bf16", 1, 0, 101),
    (2, 3, 700, 700, 64, "bf16", 2, 32, 102),
    (1, 2, 300, 320, 64, "f32", 0, 0, 103),
]
O_TOL = {"bf16": 2e-3, "f32": 1e-5}


def test_noalloc_decode_matches_workspace_decode():
    import torch
    from adaptive_sparse_attention_row_amd import api
    assert torch.cuda.is_available()
    api.lib()
    for (B, H, L, Lc, d, dtype, mask, W, seed) in CASES:
        print(f"noalloc decode B={B} H={H} L={L} cache={Lc} d={d} {dtype} mask={mask} W={W}", flush=True)
        g = torch.Generator("cpu").manual_seed(seed)
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        K = torch.randn(B, H, Lc, d, generator=g).to(tdt).cuda()
        V = torch.randn(B, H, Lc, d, generator=g).to(tdt).cuda()
        q = torch.randn(B, H, d, generator=g).to(tdt).cuda()
        scale = 1.0 / math.sqrt(d)
        o_ref, t_ref = api.attn_decode(q, K, V, L=L, scale=scale, mask=mask, window=W)
        o = torch.full((B, H, d), float("nan"), device="cuda")
        tau = torch.full((B, H), float("nan"), device="cuda")
        api.attn_decode_noalloc(q, K, V, L=L, scale=scale, mask=mask, window=W, out=o, tau=tau)
        torch.cuda.synchronize()
        o, tau, o_ref, t_ref = (x.cpu().numpy() for x in (o, tau, o_ref, t_ref))
        assert np.all(np.abs(tau - t_ref) <= 1e-4 * np.maximum(1.0, np.abs(t_ref))), "tau differs"
        err = float(np.abs(o - o_ref).max())
        assert err <= O_TOL[dtype], f"o differs by {err}"
        same = np.array_equal(o.view(np.uint32), o_ref.view(np.uint32)) and \
            np.array_equal(tau.view(np.uint32), t_ref.view(np.uint32))
        print(f"  max |do| {err:.3e}, bit-identical: {same}")
