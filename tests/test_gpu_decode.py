"""GPU parity of entmax_attn_decode (one decode step over a KV cache) against
the fp64 oracle's forward, evaluated at the last query position L - 1.

Same acceptance as the forward: |dtau| <= 1e-4 max(1, |tau|); max |dO| <=
2e-3 for bf16 inputs and 1e-5 for fp32 inputs.
"""
import math

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

TAU_TOL = 1e-4
O_TOL = {"bf16": 2e-3, "f32": 1e-5}


@pytest.fixture(scope="module")
def env():
    import torch
    from adaptive_sparse_attention_row_amd import api
    assert torch.cuda.is_available()
    api.lib()
    return api, torch


def make(B, H, L, cap, d, dtype, seed, q_std=1.0):
    import torch
    from adaptive_sparse_attention_row_amd.workloads import gen_attn
    inp = gen_attn(B, H, cap, d, dtype, seed, q_std=q_std)
    q = inp["q"][:, :, L - 1].contiguous()   # the newest query
    return q, inp["k"], inp["v"]


def oracle_last_row(orc, q, K, V, L, scale, mode, W, alpha):
    B, H, d = q.shape
    Kf = K[:, :, :L].float().numpy()
    Vf = V[:, :, :L].float().numpy()
    Qf = np.zeros((B, H, L, d), dtype=np.float32)
    Qf[:, :, L - 1] = q.float().numpy()
    rows = np.array([bh * L + L - 1 for bh in range(B * H)])
    O, tau, _, _ = orc.attn_fwd(Qf, Kf, Vf, scale, mode, W, rows=rows, alpha=alpha)
    return O.reshape(B, H, d), tau.reshape(B, H)


def check(api, torch, orc, q, K, V, L, mode, W, alpha, dtype, label):
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d)
    o, tau = api.attn_decode(q.cuda(), K.cuda(), V.cuda(), L=L, scale=scale, mask=mode, window=W, alpha=alpha)
    torch.cuda.synchronize()
    o, tau = o.cpu().numpy(), tau.cpu().numpy()
    O_ref, tau_ref = oracle_last_row(orc, q, K, V, L, scale, mode, W, alpha)
    dt = np.abs(tau - tau_ref)
    assert np.all(dt <= TAU_TOL * np.maximum(1.0, np.abs(tau_ref))), f"{label}: tau max err {dt.max()}"
    err = np.abs(o - O_ref).max()
    assert err <= O_TOL[dtype], f"{label}: O max err {err}"
    return err


SHAPES = [
    # (B, H, L, cache_len, d, dtype)
    (1, 1, 1, 1, 64, "bf16"),
    (1, 2, 2, 8, 128, "bf16"),
    (2, 3, 65, 80, 64, "bf16"),
    (1, 2, 1000, 1000, 128, "bf16"),
    (2, 2, 300, 512, 128, "f32"),
    (1, 2, 4999, 5003, 64, "f32"),
    (1, 2, 20000, 20000, 128, "bf16"),
    # quarters of 4096 scores (all held in registers) and of 4096 / 4097
    # (the last wave streams its quarter twice)
    (1, 1, 16384, 16384, 128, "bf16"),
    (1, 2, 16385, 16400, 64, "bf16"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%dH%dL%dcap%dd%d%s" % s)
@pytest.mark.parametrize("mode,W", [(0, 0), (1, 0), (2, 32), (2, 0)], ids=["none", "causal", "win32", "win0"])
@pytest.mark.parametrize("alpha", [1.5, 2.0, 1.25])
def test_decode_shapes(env, orc, shape, mode, W, alpha):
    api, torch = env
    B, H, L, cap, d, dtype = shape
    a = float(np.float32(alpha))
    q, K, V = make(B, H, L, cap, d, dtype, seed=L + d + mode)
    print(f"decode shape={shape} mode={mode} W={W} alpha={alpha}", flush=True)
    check(api, torch, orc, q, K, V, L, mode, W, a, dtype, f"{shape} mode={mode} alpha={alpha}")


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_decode_candidate_overflow(env, orc, alpha):
    """All keys equal: every score is a candidate (more than the LDS list
    holds), so tau and o come from the streamed score row."""
    api, torch = env
    import torch as T
    B, H, L, d = 1, 2, 6000, 64
    q, K, V = make(B, H, L, L, d, "bf16", seed=3)
    K[0, 0] = K[0, 0, 7]                       # head 0: identical keys
    K[0, 1, :, :] = (0.01 * T.randn(L, d)).to(T.bfloat16)  # head 1: near-ties
    check(api, torch, orc, q, K, V, L, 1, 0, float(np.float32(alpha)), "bf16", f"overflow alpha={alpha}")


def test_decode_one_hot_and_scaled_queries(env, orc):
    api, torch = env
    import torch as T
    B, H, L, d = 1, 2, 700, 128
    q, K, V = make(B, H, L, L, d, "bf16", seed=4)
    q[0, 0] = (20 * K[0, 0, 123].float()).to(T.bfloat16)  # one key far above the rest
    for q_std in (0.05, 4.0):
        q2 = (q.float() * q_std).to(T.bfloat16)
        check(api, torch, orc, q2, K, V, L, 1, 0, 1.5, "bf16", f"q_std={q_std}")


def test_decode_matches_forward_last_row(env, orc):
    """The decode step and the forward kernels agree on the last row (both
    against the oracle, and with each other to the forward's bound)."""
    api, torch = env
    from adaptive_sparse_attention_row_amd.workloads import gen_attn
    B, H, L, d = 1, 3, 777, 64
    inp = gen_attn(B, H, L, d, "bf16", seed=5)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    for mode, W in ((1, 0), (2, 32)):
        O, tau, _ = api.attn_fwd(q, k, v, scale=0.125, mask=mode, window=W)
        o, t = api.attn_decode(q[:, :, L - 1].contiguous(), k, v, scale=0.125, mask=mode, window=W)
        torch.cuda.synchronize()
        assert np.abs(t.cpu().numpy() - tau[:, :, L - 1].cpu().numpy()).max() <= 1e-4 * 4
        assert np.abs(o.cpu().numpy() - O[:, :, L - 1].cpu().numpy()).max() <= 2e-3
