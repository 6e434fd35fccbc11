"""GPU parity of entmax_tau_rows against the fp64 oracle.

Tolerances (from the acceptance bar on tau and the support): |dtau| <=
1e-4 * max(1, |tau|); the support {P > 0} equals {S > tau_ref} except where
|S - tau_ref| < 1e-4; |dP| <= 1e-4 (|dp/dtau| = sqrt(p) <= 1, so the tau bound
carries over) and every row of P sums to 1 within 1e-4.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

TAU_TOL = 1e-4
P_TOL = 1e-4
BAND = 1e-4


def _check(S_np, tau_gpu, P_gpu, orc, label="", alpha=1.5):
    tau_ref, P_ref = orc.tau_rows(S_np, want_p=True, alpha=alpha)
    S64 = S_np.astype(np.float64)
    finite_rows = np.isfinite(tau_ref)
    assert np.array_equal(np.isfinite(tau_gpu), finite_rows), label
    dt = np.abs(tau_gpu[finite_rows] - tau_ref[finite_rows])
    assert np.all(dt <= TAU_TOL * np.maximum(1.0, np.abs(tau_ref[finite_rows]))), \
        f"{label} max dtau {dt.max()}"
    if P_gpu is None:
        return
    assert np.max(np.abs(P_gpu - P_ref)) <= P_TOL, f"{label} max dP {np.max(np.abs(P_gpu - P_ref))}"
    sup_ref = S64 > tau_ref[:, None]
    sup_gpu = P_gpu > 0
    # weights below ~1e-30 are not kept in fp32 (denormal results flush to
    # zero): for alpha near 1 that widens the band above tau to
    # (1e-30)^(alpha-1)/(alpha-1) (1e-2 at alpha = 1.1, far below 1e-4 at 1.5)
    band = max(BAND, 1e-30 ** (alpha - 1.0) / (alpha - 1.0))
    with np.errstate(invalid="ignore"):
        d = S64 - tau_ref[:, None]
    far = (d >= band) | (d <= -BAND)
    assert np.array_equal(sup_ref & far, sup_gpu & far), label
    sums = P_gpu.astype(np.float64).sum(1)
    # a shift of tau by one fp32 rounding step of the scores moves the sum by
    # that step times sum_j dp_j/ds_j = sum_j p_j^(2 - alpha) (sqrt(p) at 1.5,
    # the support size at 2)
    slope = np.where(P_ref > 0, np.power(np.maximum(P_ref, 1e-300), 2.0 - alpha), 0.0).sum(1)
    tol = 1e-4 + 2.4e-7 * np.maximum(1.0, np.abs(np.nan_to_num(tau_ref, neginf=0.0))) * slope
    assert np.all(np.abs(sums[finite_rows] - 1.0) <= tol[finite_rows]), label
    assert np.all(P_gpu[~finite_rows] == 0), label


def _run(api, torch, S_np, want_p=True, ld=None, alpha=1.5, row_plain_bracket=False):
    rows, cols = S_np.shape
    if ld is None or ld == cols:
        S = torch.from_numpy(S_np).cuda()
    else:
        big = torch.zeros(rows, ld, dtype=torch.float32)
        big[:, :cols] = torch.from_numpy(S_np)
        S = big.cuda()[:, :cols]
    tau, P = api.tau_rows(S, want_p=want_p, alpha=alpha, row_plain_bracket=row_plain_bracket)
    torch.cuda.synchronize()
    return tau.cpu().numpy(), (P.cpu().numpy() if P is not None else None)


@pytest.fixture(scope="module")
def env():
    import torch
    from adaptive_sparse_attention_row_amd import api
    assert torch.cuda.is_available()
    api.lib()
    return api, torch


@pytest.mark.parametrize("cols", [1, 2, 3, 63, 64, 65, 257, 1000, 1024, 1025, 4096, 8191,
                                  8192, 8193, 16384, 20000, 32768, 40000])
def test_widths(env, orc, cols):
    api, torch = env
    rng = np.random.default_rng(cols)
    S = rng.normal(size=(37, cols)).astype(np.float32) * rng.uniform(0.2, 3.0)
    tau, P = _run(api, torch, S)
    print(f"cols={cols}", flush=True)
    _check(S, tau, P, orc, f"cols={cols}")


@pytest.mark.parametrize("cols,ld", [(100, 104), (100, 101), (5000, 5003), (9000, 9001)])
def test_row_stride_and_alignment(env, orc, cols, ld):
    api, torch = env
    rng = np.random.default_rng(ld)
    S = rng.normal(size=(19, cols)).astype(np.float32)
    tau, P = _run(api, torch, S, ld=ld)
    _check(S, tau, P, orc, f"cols={cols} ld={ld}")


def test_tau_only(env, orc):
    api, torch = env
    S = np.random.default_rng(5).normal(size=(50, 700)).astype(np.float32)
    tau, P = _run(api, torch, S, want_p=False)
    assert P is None
    _check(S, tau, None, orc, "tau only")


def test_degenerate_rows(env, orc):
    api, torch = env
    cols = 3000
    rng = np.random.default_rng(6)
    S = rng.normal(size=(8, cols)).astype(np.float32)
    S[0] = 1.25                                  # all equal: p = 1/n
    S[1] = -np.inf; S[1, 17] = 4.0               # single active entry
    S[2] = rng.normal(size=cols) - 10; S[2, 5] = 3.0  # one-hot (gap > 2)
    S[3] = -np.inf                               # no active entry
    S[4, ::2] = -np.inf                          # half masked
    S[5] = np.linspace(-1, 1, cols)              # every score a candidate
    S[6] = 0.0; S[6, :7] = 1e-3                  # near-ties
    S[7] = rng.normal(size=cols) * 1e-3          # all within 2 of the max
    tau, P = _run(api, torch, S)
    _check(S, tau, P, orc, "degenerate")
    np.testing.assert_allclose(P[0], 1.0 / cols, rtol=1e-4)
    assert P[1, 17] == 1.0 and np.sum(P[1] > 0) == 1
    assert P[2, 5] == 1.0 and np.sum(P[2] > 0) == 1
    assert tau[3] == -np.inf and np.all(P[3] == 0)


def test_overflowing_candidates(env, orc):
    # more than the LDS candidate capacity within 2 of the max, register and
    # streamed rows both
    api, torch = env
    rng = np.random.default_rng(7)
    for cols in (8192, 12000):
        S = (rng.normal(size=(6, cols)) * 0.05).astype(np.float32)
        tau, P = _run(api, torch, S)
        _check(S, tau, P, orc, f"overflow cols={cols}")


def test_resident_waves_mixed_rows(env, orc):
    """More rows than stay resident, so every wave solves several rows in
    turn: kinds that take different paths (ordinary, one-hot, all masked,
    all equal, more candidates than LDS holds) interleaved so that each
    wave meets them one after another."""
    api, torch = env
    rows, cols = 4001, 8192
    rng = np.random.default_rng(11)
    S = rng.normal(size=(rows, cols)).astype(np.float32)
    kind = np.arange(rows) % 5
    S[kind == 0] *= 3.0
    S[kind == 1] -= 10.0
    S[kind == 1, 123] = 4.0                       # one-hot (gap > 2)
    S[kind == 2] = -np.inf                        # no active entry
    S[kind == 3] = 0.5                            # all equal: p = 1/n
    S[kind == 4] *= 0.05                          # every score a candidate
    print("mixed rows generated", flush=True)
    tau, P = _run(api, torch, S)
    _check(S, tau, P, orc, "mixed")
    assert np.all(P[kind == 1, 123] == 1.0)
    assert np.all(tau[kind == 2] == -np.inf)
    np.testing.assert_allclose(P[kind == 3], 1.0 / cols, rtol=1e-4)


def test_zero_rows(env):
    api, torch = env
    S = torch.empty(0, 10, device="cuda")
    tau, P = api.tau_rows(S)
    assert tau.numel() == 0


def test_full_size_c2(env, orc):
    """The 8192 x 8192 N(0, 1) workload, every row and every element."""
    api, torch = env
    from adaptive_sparse_attention_row_amd.workloads import C2, gen_rows
    S = gen_rows(C2.rows, C2.cols, C2.seed)
    print("c2 generated", flush=True)
    tau, P = api.tau_rows(S.cuda())
    torch.cuda.synchronize()
    _check(S.numpy(), tau.cpu().numpy(), P.cpu().numpy(), orc, "c2")


# ------------------------------------------------------------- general alpha
# alpha-entmax for alpha in (1, 2] ("AdaSplash-2: Faster Differentiable Sparse
# Attention" sec. 2.3).  Same tolerances: |dp/dtau| = u^(1/(alpha-1) - 1) <= 1
# on the support (u <= 1 there), so the tau bound carries over to P.  The
# oracle gets alpha as the fp32 value the library sees.

ALPHAS = [1.1, 1.25, 1.75, 2.0]


@pytest.mark.parametrize("alpha", ALPHAS)
@pytest.mark.parametrize("cols", [1, 65, 1000, 8192, 8193, 20000, 32768])
def test_alpha_widths(env, orc, cols, alpha):
    api, torch = env
    a = float(np.float32(alpha))
    rng = np.random.default_rng(cols + int(alpha * 100))
    S = rng.normal(size=(23, cols)).astype(np.float32) * rng.uniform(0.5, 3.0)
    print(f"alpha={alpha} cols={cols}", flush=True)
    tau, P = _run(api, torch, S, alpha=a)
    _check(S, tau, P, orc, f"alpha={alpha} cols={cols}", alpha=a)


@pytest.mark.parametrize("alpha", [1.25, 2.0])
def test_alpha_degenerate_rows(env, orc, alpha):
    api, torch = env
    a = float(np.float32(alpha))
    e = 1.0 / (a - 1.0)
    cols = 3000
    rng = np.random.default_rng(8)
    S = rng.normal(size=(7, cols)).astype(np.float32)
    S[0] = 1.25                                      # all equal: p = 1/n
    S[1] = -np.inf; S[1, 17] = 4.0                   # single active entry
    S[2] = rng.normal(size=cols) - 3 * e; S[2, 5] = 3.0  # one-hot (gap > 1/(alpha-1))
    S[3] = -np.inf                                   # no active entry
    S[4, ::2] = -np.inf                              # half masked
    S[5] = np.linspace(-1, 1, cols)                  # dense support
    S[6] = rng.normal(size=cols) * 1e-3              # near-ties
    tau, P = _run(api, torch, S, alpha=a)
    _check(S, tau, P, orc, f"degenerate alpha={alpha}", alpha=a)
    np.testing.assert_allclose(P[0], 1.0 / cols, rtol=1e-3)
    assert np.sum(P[1] > 0) == 1 and abs(P[1, 17] - 1.0) <= 1e-6
    assert np.sum(P[2] > 0) == 1 and abs(P[2, 5] - 1.0) <= 1e-6
    assert tau[3] == -np.inf and np.all(P[3] == 0)


@pytest.mark.parametrize("alpha", [1.25, 2.0])
def test_alpha_full_size_sampled(env, orc, alpha):
    """The 8192 x 8192 N(0, 1) matrix at another alpha: sampled rows."""
    api, torch = env
    a = float(np.float32(alpha))
    from adaptive_sparse_attention_row_amd.workloads import C2, gen_rows
    S = gen_rows(C2.rows, C2.cols, C2.seed)
    tau, P = api.tau_rows(S.cuda(), alpha=a)
    torch.cuda.synchronize()
    rows = np.random.default_rng(9).choice(C2.rows, 96, replace=False)
    _check(S.numpy()[rows], tau.cpu().numpy()[rows], P.cpu().numpy()[rows], orc, f"c2 alpha={alpha}", alpha=a)


def test_alpha_out_of_range_rejected(env):
    api, torch = env
    S = torch.zeros(2, 8, device="cuda")
    for bad in (1.0, 0.5, 2.5, float("nan")):
        with pytest.raises(api.EntmaxError) as ei:
            api.tau_rows(S, alpha=bad)
        assert ei.value.status == api.ERR_ALPHA


@pytest.mark.parametrize("alpha", [1.5, 1.25, 2.0])
@pytest.mark.parametrize("hist", [1, 0], ids=["hist", "nohist"])
@pytest.mark.parametrize("cols", [20000, 32768, 40000])
def test_wide_rows_histogram_bracket(env, orc, alpha, hist, cols):
    """Rows wider than 8192 (held in a workgroup's registers up to 32768,
    streamed beyond), with and without the histogram-initialised bracket:
    sparse rows, dense rows that overflow any LDS list, near-constant and
    one-hot rows; same results either way."""
    api, torch = env
    a = float(np.float32(alpha))
    rng = np.random.default_rng(70 + hist)
    S = rng.normal(size=(8, cols)).astype(np.float32)
    S[1] *= 0.02                       # dense: every score near the max
    S[2] = 3.0; S[2, ::7] = 2.9        # near-constant
    S[3] = -5.0; S[3, 1234] = 5.0      # one-hot
    S[4] *= 4.0
    S[5, :cols // 2] = -np.inf         # half masked
    S[6] = np.linspace(-0.5, 0.5, cols)
    S[7] *= 0.3
    tau, P = _run(api, torch, S, alpha=a, row_plain_bracket=not hist)
    _check(S, tau, P, orc, f"wide alpha={alpha} hist={hist}", alpha=a)
