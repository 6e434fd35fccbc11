"""Pins of the oracle's general-alpha entmax (alpha in (1, 2]).

"AdaSplash-2: Faster Differentiable Sparse Attention" sec. 2.3 defines
alpha-entmax as the maximiser of p.s + H_alpha(p) over the simplex, with the
Tsallis entropy H_alpha(p) = sum_j (p_j - p_j^alpha) / (alpha (alpha - 1)),
and gives its solution p_j = [(alpha - 1) s_j - tau']_+^(1/(alpha - 1)).  The
oracle works in score units (tau' = (alpha - 1) tau).  Each check below is
independent of the oracle's solvers (sorting at alpha = 2, bisection
otherwise): hand-solved closed forms, brute force over every support
(sparsemax), the objective and its first-order conditions, continuity with
the independently pinned alpha = 1.5 solver, the softmax limit, and finite
differences for the backward.
"""
import itertools
import math

import numpy as np
import pytest

ALPHAS = [1.1, 1.25, 1.5, 1.75, 2.0]


def tsallis_obj(p, s, alpha):
    return float(p @ s + np.sum(p - p ** alpha) / (alpha * (alpha - 1.0)))


@pytest.mark.parametrize("alpha", ALPHAS)
def test_constant_rows_give_uniform_weights(orc, alpha):
    """s = c * 1_n: p = 1/n, so (alpha-1)(c - tau) = n^(1-alpha) and tau is the
    upper bracket end c - n^(1-alpha)/(alpha-1) (AdaSplash-2 sec. 2.4)."""
    for n, c in ((1, 0.0), (2, 0.0), (7, -3.25), (64, 11.5)):
        p, tau, k = orc.entmax(np.full(n, c), alpha)
        expect = c - n ** (1.0 - alpha) / (alpha - 1.0)
        assert abs(tau - expect) <= 1e-12 * max(1.0, abs(expect)), (n, c, tau, expect)
        np.testing.assert_allclose(p, 1.0 / n, rtol=1e-12)
        assert k == n


@pytest.mark.parametrize("alpha", ALPHAS)
def test_two_equal_scores_closed_form(orc, alpha):
    """s = [0, 0]: p = [1/2, 1/2], tau = -(1/2)^(alpha-1)/(alpha-1); at
    alpha = 1.5 this is the -sqrt(2) of the GPT-2 model card's example."""
    p, tau, _ = orc.entmax(np.zeros(2), alpha)
    assert abs(tau + 0.5 ** (alpha - 1.0) / (alpha - 1.0)) <= 1e-12
    if alpha == 1.5:
        assert abs(tau + math.sqrt(2.0)) <= 1e-12
    np.testing.assert_allclose(p, [0.5, 0.5], rtol=1e-12)


@pytest.mark.parametrize("alpha", ALPHAS)
def test_one_hot_at_the_lower_bracket_end(orc, alpha):
    """When the maximum leads every other score by at least 1/(alpha-1), p is
    one-hot and tau = max - 1/(alpha-1) (p_max = 1)."""
    e = 1.0 / (alpha - 1.0)
    s = np.array([5.0 - e - 0.3, 5.0, 5.0 - e - 0.01, 5.0 - e - 2.0, 5.0 - 3 * e])
    p, tau, k = orc.entmax(s, alpha)
    assert abs(tau - (5.0 - e)) <= 1e-12 * 5
    np.testing.assert_allclose(p, [0.0, 1.0, 0.0, 0.0, 0.0], atol=1e-12)
    assert np.count_nonzero(p) == 1 and k == 1


def _sparsemax_brute(s):
    """Every non-empty support S gives tau_S = (sum_S s - 1)/|S|; keep the
    self-consistent ones (s > tau on S, s <= tau off S)."""
    n = s.size
    found = []
    for r in range(1, n + 1):
        for sup in itertools.combinations(range(n), r):
            x = s[list(sup)]
            t = (x.sum() - 1.0) / len(x)
            rest = np.delete(s, list(sup))
            if np.all(x > t - 1e-12) and np.all(rest <= t + 1e-12):
                found.append(t)
    return found


def test_sparsemax_against_brute_force_supports(orc):
    rng = np.random.default_rng(31)
    for _ in range(60):
        n = int(rng.integers(1, 11))
        s = np.round(rng.normal(size=n) * 1.2, 3)
        p, tau, k = orc.entmax(s, 2.0)
        cands = _sparsemax_brute(s)
        assert cands
        assert min(abs(tau - t) for t in cands) <= 1e-12 * max(1.0, abs(tau))
        np.testing.assert_allclose(p, np.maximum(s - tau, 0.0), atol=1e-15)
        assert k == int(np.sum(s > tau))


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_bisection_agrees_with_the_sorting_solvers(orc, alpha):
    """The generic bisection reproduces the exact sorting solvers of alpha =
    1.5 (quadratic per support, pinned in test_oracle.py) and alpha = 2."""
    rng = np.random.default_rng(32)
    worst = 0.0
    for _ in range(200):
        n = int(rng.integers(1, 300))
        s = rng.normal(size=n) * rng.uniform(0.1, 4.0) + rng.normal() * 5
        _, tau, _ = orc.entmax(s, alpha)
        tb = orc.tau_bisect(s, alpha)
        worst = max(worst, abs(tau - tb) / max(1.0, abs(tb)))
    assert worst <= 1e-12


@pytest.mark.parametrize("alpha", [1.25, 1.5 + 1e-9])
def test_continuity_in_alpha(orc, alpha):
    """tau and p move continuously with alpha: alpha = 1.5 + 1e-9 by bisection
    matches the exact alpha = 1.5 solver to ~1e-8."""
    rng = np.random.default_rng(33)
    for _ in range(30):
        s = rng.normal(size=int(rng.integers(2, 80))) * 1.5
        p, tau, _ = orc.entmax(s, alpha)
        p2, tau2, _ = orc.entmax(s, alpha + 1e-7)
        assert abs(tau - tau2) <= 1e-4 * max(1.0, abs(tau))
        np.testing.assert_allclose(p, p2, atol=1e-4)
        if abs(alpha - 1.5) < 1e-6:
            p15, tau15, _ = orc.entmax(s, 1.5)
            assert abs(tau - tau15) <= 1e-6 * max(1.0, abs(tau15))


@pytest.mark.parametrize("alpha", [1.1, 1.25, 1.75, 2.0])
def test_tsallis_objective_optimality(orc, alpha):
    """p maximises p.s + H_alpha(p) over the simplex; on the support the
    first-order condition reads s_j - p_j^(alpha-1)/(alpha-1) = tau, and off
    it s_j <= tau."""
    rng = np.random.default_rng(34)
    for _ in range(40):
        n = int(rng.integers(2, 25))
        s = rng.normal(size=n) * 2
        p, tau, _ = orc.entmax(s, alpha)
        assert abs(p.sum() - 1.0) <= 1e-12 and np.all(p >= 0)
        best = tsallis_obj(p, s, alpha)
        for _ in range(150):
            q = rng.dirichlet(np.ones(n) * 0.3)
            for eps in (1e-3, 1e-1, 1.0):
                assert tsallis_obj((1 - eps) * p + eps * q, s, alpha) <= best + 1e-12
        sup = p > 0
        np.testing.assert_allclose(s[sup] - p[sup] ** (alpha - 1.0) / (alpha - 1.0), tau, atol=1e-9)
        assert np.all(s[~sup] <= tau + 1e-12)


def test_softmax_limit(orc):
    """alpha-entmax tends to softmax as alpha -> 1 (AdaSplash-2 sec. 2.3):
    the gap shrinks roughly in proportion to alpha - 1."""
    rng = np.random.default_rng(35)
    s = rng.normal(size=20)
    sm = np.exp(s - s.max())
    sm /= sm.sum()
    gaps = []
    for alpha in (1.01, 1.001):
        p, _, _ = orc.entmax(s, alpha)
        gaps.append(np.abs(p - sm).max())
    assert gaps[1] < 2e-3
    assert gaps[1] < gaps[0] / 5


@pytest.mark.parametrize("alpha", [1.25, 1.75, 2.0])
def test_masked_and_shifted_rows(orc, alpha):
    rng = np.random.default_rng(36)
    s = rng.normal(size=40)
    keep = rng.random(40) < 0.5
    keep[0] = True
    p, tau, _ = orc.entmax(np.where(keep, s, -np.inf), alpha)
    p2, tau2, _ = orc.entmax(s[keep], alpha)
    assert tau == tau2 and np.all(p[~keep] == 0)
    np.testing.assert_array_equal(p[keep], p2)
    p3, tau3, _ = orc.entmax(s + 17.5, alpha)
    assert abs(tau3 - 17.5 - orc.entmax(s, alpha)[1]) <= 1e-9
    np.testing.assert_allclose(p3, orc.entmax(s, alpha)[0], atol=1e-9)


@pytest.mark.parametrize("alpha", [1.25, 2.0])
def test_tau_rows_and_attention_plumbing(orc, alpha):
    """Row-wise and attention forms use the same per-row map: O = A V with
    numpy matmuls over the oracle's own rows."""
    rng = np.random.default_rng(37)
    S = rng.normal(size=(16, 75)).astype(np.float32)
    tau, P = orc.tau_rows(S, alpha=alpha)
    for r in range(16):
        p, t, _ = orc.entmax(S[r].astype(np.float64), alpha)
        assert t == tau[r]
        np.testing.assert_array_equal(P[r], p)
    B, H, L, d = 1, 2, 29, 8
    Q = rng.normal(size=(B, H, L, d)).astype(np.float32)
    K = rng.normal(size=(B, H, L, d)).astype(np.float32)
    V = rng.normal(size=(B, H, L, d)).astype(np.float32)
    O, tau, _, _ = orc.attn_fwd(Q, K, V, 0.7, 1, 0, alpha=alpha)
    O = O.reshape(B, H, L, d)
    for h in range(H):
        s = 0.7 * (Q[0, h].astype(np.float64) @ K[0, h].astype(np.float64).T)
        s = np.where(np.arange(L)[None, :] <= np.arange(L)[:, None], s, -np.inf)
        A = np.stack([orc.entmax(s[i], alpha)[0] for i in range(L)])
        np.testing.assert_allclose(O[0, h], A @ V[0, h].astype(np.float64), atol=1e-12)


def _loss(orc, Q, K, V, dO, scale, mask, W, alpha):
    O, _, _, _ = orc.attn_fwd(Q[None, None], K[None, None], V[None, None], scale, mask, W, alpha=alpha)
    return float(np.sum(O * dO))


@pytest.mark.parametrize("alpha", [1.25, 1.75, 2.0])
def test_backward_against_finite_differences(orc, alpha):
    """Central differences of sum(O * dO) (fp64) against the oracle's
    backward with g = [(alpha-1)(s - tau)]_+^(1/(alpha-1) - 1).  At alpha = 2
    the map is piecewise linear: steps that cross a support change would
    disagree, so those entries are skipped (one-sided differences differ)."""
    rng = np.random.default_rng(40 + int(alpha * 4))
    L, d, scale = 9, 4, 0.9
    Q = rng.normal(size=(L, d)).astype(np.float32)
    K = rng.normal(size=(L, d)).astype(np.float32)
    V = rng.normal(size=(L, d)).astype(np.float32)
    dO = rng.normal(size=(L, d)).astype(np.float32)
    dQ, dK, dV, _, _ = orc.attn_bwd_head(Q, K, V, dO, scale, 1, 0, alpha=alpha)
    h = 2.0 ** -12
    checked = 0
    for name, X, G in (("Q", Q, dQ), ("K", K, dK), ("V", V, dV)):
        for idx in itertools.product(range(L), range(d)):
            args = {"Q": Q, "K": K, "V": V}
            vals = []
            for sgn in (1, 0, -1):
                Xs = X.copy()
                Xs[idx] += sgn * h
                args[name] = Xs
                vals.append(_loss(orc, args["Q"], args["K"], args["V"], dO, scale, 1, 0, alpha))
            fwd, bwd = (vals[0] - vals[1]) / h, (vals[1] - vals[2]) / h
            if abs(fwd - bwd) > 1e-3 * max(1.0, abs(fwd)):
                continue  # a kink of the piecewise map lies inside the step
            fd = (vals[0] - vals[2]) / (2 * h)
            assert abs(fd - G[idx]) <= 5e-5 * max(1.0, abs(G[idx])), (alpha, name, idx, fd, G[idx])
            checked += 1
    assert checked >= 0.9 * 3 * L * d


@pytest.mark.parametrize("alpha", [1.25, 2.0])
def test_backward_invariants(orc, alpha):
    rng = np.random.default_rng(45)
    L, d = 30, 6
    Q = rng.normal(size=(L, d)).astype(np.float32)
    K = rng.normal(size=(L, d)).astype(np.float32)
    V = rng.normal(size=(L, d)).astype(np.float32)
    dO = rng.normal(size=(L, d)).astype(np.float32)
    dQ, dK, dV, tau, delta = orc.attn_bwd_head(Q, K, V, dO, 0.6, 0, 0, alpha=alpha)
    np.testing.assert_allclose(dK.sum(0), 0.0, atol=1e-12)
    np.testing.assert_allclose(dV.sum(0), dO.astype(np.float64).sum(0), atol=1e-12)
    rows = np.array([0, 11, L - 1])
    dQr, deltar, taur = orc.attn_bwd_rows(Q[None, None], K[None, None], V[None, None], dO[None, None],
                                          0.6, 0, 0, rows, alpha=alpha)
    np.testing.assert_array_equal(dQr, dQ[rows])
    np.testing.assert_array_equal(taur, tau[rows])


# ------------------------------------------------ histogram initialisation
# AdaSplash-2 sec. 3.1 / appendix C.3: left-edge bins give a threshold tau_h
# with tau* - h < tau_h <= tau* (Proposition 3.1), h = 1/(B (alpha - 1)) in
# score units.

@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0])
@pytest.mark.parametrize("bins", [8, 64])
def test_histogram_threshold_brackets_tau(orc, alpha, bins):
    rng = np.random.default_rng(50 + bins)
    a = float(np.float32(alpha))
    h = 1.0 / (bins * (a - 1.0))
    worst = 0.0
    for _ in range(150):
        n = int(rng.integers(1, 3000))
        s = (rng.normal(size=n) * rng.uniform(0.05, 3.0)).astype(np.float32)
        if rng.random() < 0.2:
            s[rng.random(n) < 0.5] = -np.inf
            s[0] = 0.5
        _, tau, _ = orc.entmax(s.astype(np.float64), a)
        th = orc.tau_histogram(s, a, bins)
        assert th <= tau + 1e-9 * max(1.0, abs(tau)), (n, th, tau)
        assert tau - th <= h + 1e-9, (n, th, tau, h)
        worst = max(worst, tau - th)
    print(f"alpha={alpha} B={bins}: worst tau - tau_h = {worst:.4f} (bin width {h:.4f})")


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0])
def test_histogram_threshold_of_constant_rows(orc, alpha):
    """A constant row has z = 1 everywhere, and the top bin's left edge is
    (B-1)/B: every entry moves down by exactly one bin width, so tau_h =
    tau* - 1/(B (alpha-1)) = c - n^(1-alpha)/(alpha-1) - 1/(B (alpha-1)).
    (The bound of Proposition 3.1 is attained here, so the bracket the
    kernels use is closed: [tau_h, tau_h + h].)"""
    a = float(np.float32(alpha))
    for B in (8, 64):
        for n, c in ((1, 0.0), (5, 2.5), (300, -1.0)):
            th = orc.tau_histogram(np.full(n, c, dtype=np.float32), a, B)
            expect = c - n ** (1.0 - a) / (a - 1.0) - 1.0 / (B * (a - 1.0))
            assert abs(th - expect) <= 1e-9 * max(1.0, abs(expect)), (B, n, c, th, expect)
