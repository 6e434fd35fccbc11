"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Every check here is independent of the oracle's own algorithm (sorting plus a
quadratic per support size): closed forms solved by hand, the bracket of
AdaSplash-2 sec. 2.4 attained at both ends, plain bisection on the normaliser,
brute-force enumeration of every support, the Tsallis-objective optimality of
the DistilBERT model card's sec. 1, finite differences for the backward, and
numpy matmuls for the attention plumbing.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def load_golden(name):
    with open(os.path.join(HERE, "golden", name)) as f:
        return json.load(f)


def normaliser(s, tau):
    """f(tau) + 1 = sum_j [(s_j - tau)/2]_+^2 over finite entries."""
    s = np.asarray(s, dtype=np.float64)
    s = s[np.isfinite(s)]
    g = np.maximum(0.5 * (s - tau), 0.0)
    return float(np.sum(g * g))


def bisect_tau(s, iters=200):
    """Plain bisection on the bracket [max - 2, max - 2/sqrt(n)] (AdaSplash-2
    sec. 2.4, m - 1 <= tau' <= m - n^(1 - alpha) with tau = 2 tau' for
    alpha = 1.5)."""
    s = np.asarray(s, dtype=np.float64)
    s = s[np.isfinite(s)]
    m, n = s.max(), s.size
    lo, hi = m - 2.0, m - 2.0 / math.sqrt(n)
    assert normaliser(s, lo) >= 1.0 - 1e-15
    assert normaliser(s, hi) <= 1.0 + 1e-15
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if normaliser(s, mid) > 1.0:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def brute_force_tau(s):
    """Try every non-empty support; keep the one that is self-consistent."""
    s = np.asarray(s, dtype=np.float64)
    n = s.size
    found = []
    for r in range(1, n + 1):
        for sup in itertools.combinations(range(n), r):
            x = s[list(sup)]
            k = len(x)
            # k t^2 - 2 sum(x) t + sum(x^2) - 4 = 0, smaller root
            a, b = x.sum(), (x * x).sum()
            disc = a * a - k * (b - 4.0)
            if disc < 0:
                continue
            t = (a - math.sqrt(disc)) / k
            rest = np.delete(s, list(sup))
            if np.all(x > t - 1e-12) and np.all(rest <= t + 1e-12):
                found.append(t)
    assert found, "no consistent support"
    return found


# ---------------------------------------------------------------- closed forms

def test_golden_closed_forms(orc):
    for case in load_golden("entmax15_closed_forms.json")["cases"]:
        p, tau, _ = orc.entmax15(case["s"])
        assert abs(tau - case["tau"]) <= 1e-15 * max(1.0, abs(case["tau"])), case["name"]
        np.testing.assert_allclose(p, case["p"], rtol=0, atol=1e-15, err_msg=case["name"])


def test_worked_example_sqrt2(orc):
    p, tau, k = orc.entmax15([0.0, 0.0])
    assert tau == -math.sqrt(2.0)
    assert k == 2
    np.testing.assert_allclose(p, [0.5, 0.5], rtol=0, atol=2e-16)


@pytest.mark.parametrize("n", [1, 2, 3, 7, 64, 1000])
@pytest.mark.parametrize("c", [0.0, -3.25, 17.5])
def test_upper_bracket_attained_by_constant_rows(orc, n, c):
    # all scores equal: p = 1/n and tau = c - 2/sqrt(n), the upper bracket end
    p, tau, k = orc.entmax15(np.full(n, c))
    assert k == n
    assert abs(tau - (c - 2.0 / math.sqrt(n))) <= 1e-13 * max(1.0, abs(c))
    np.testing.assert_allclose(p, 1.0 / n, rtol=1e-12)


def test_lower_bracket_attained_one_hot(orc):
    rng = np.random.default_rng(11)
    for _ in range(200):
        n = int(rng.integers(1, 40))
        s = rng.normal(size=n) * 3
        top = int(rng.integers(0, n))
        s[top] = np.delete(s, top).max(initial=-np.inf) + 2.0 + rng.uniform(0.0, 3.0) if n > 1 else s[top]
        p, tau, k = orc.entmax15(s)
        assert k == 1
        assert abs(tau - (s[top] - 2.0)) <= 1e-13 * max(1.0, abs(s[top]))
        expect = np.zeros(n)
        expect[top] = 1.0
        assert p.tolist() == expect.tolist()


# ------------------------------------------------------- solver exactness pins

def test_agrees_with_bisection(orc):
    rng = np.random.default_rng(12)
    worst = 0.0
    for _ in range(300):
        n = int(rng.integers(1, 200))
        s = rng.normal(size=n) * rng.uniform(0.1, 5.0) + rng.normal() * 10
        _, tau, _ = orc.entmax15(s)
        tb = bisect_tau(s)
        worst = max(worst, abs(tau - tb) / max(1.0, abs(tb)))
    assert worst <= 1e-12


def test_agrees_with_brute_force_supports(orc):
    rng = np.random.default_rng(13)
    for trial in range(60):
        n = int(rng.integers(1, 11))
        s = np.round(rng.normal(size=n) * 1.5, 3)
        _, tau, k = orc.entmax15(s)
        cands = brute_force_tau(s)
        assert min(abs(tau - t) for t in cands) <= 1e-12 * max(1.0, abs(tau))
        # uniqueness of the root: all consistent supports give the same tau
        assert max(cands) - min(cands) <= 1e-12 * max(1.0, abs(tau))
        assert k == int(np.sum(s > tau))


def test_masked_entries_are_absent(orc):
    rng = np.random.default_rng(14)
    s = rng.normal(size=50)
    keep = rng.random(50) < 0.4
    keep[3] = True
    sm = np.where(keep, s, -np.inf)
    p, tau, _ = orc.entmax15(sm)
    p2, tau2, _ = orc.entmax15(s[keep])
    assert tau == tau2
    assert np.all(p[~keep] == 0.0)
    np.testing.assert_array_equal(p[keep], p2)
    # all masked: tau = -inf, no weights
    p3, tau3, k3 = orc.entmax15(np.full(4, -np.inf))
    assert tau3 == -np.inf and k3 == 0 and np.all(p3 == 0)


# ---------------------------------------------------------------- invariants

def test_simplex_and_support_invariants(orc):
    rng = np.random.default_rng(15)
    for _ in range(200):
        n = int(rng.integers(1, 300))
        s = rng.normal(size=n) * rng.uniform(0.1, 4.0)
        p, tau, k = orc.entmax15(s)
        assert np.all(p >= 0)
        assert abs(p.sum() - 1.0) <= 1e-12
        assert np.array_equal(p > 0, s > tau)
        assert k == int(np.sum(s > tau))
        m = s.max()
        assert m - 2.0 - 1e-12 <= tau <= m - 2.0 / math.sqrt(n) + 1e-12


def test_translation_invariance(orc):
    rng = np.random.default_rng(16)
    for _ in range(50):
        s = rng.normal(size=int(rng.integers(2, 100)))
        c = float(rng.normal() * 100)
        p, tau, _ = orc.entmax15(s)
        p2, tau2, _ = orc.entmax15(s + c)
        assert abs((tau2 - c) - tau) <= 1e-12 * max(1.0, abs(c))
        np.testing.assert_allclose(p2, p, atol=1e-11)


def test_tsallis_objective_optimality(orc):
    """p maximises p.s + (4/3) sum(p - p^1.5) over the simplex (DistilBERT MNLI
    with AdaSplash Attention via NeuralOps, Mathematical Formulation item 1)."""
    rng = np.random.default_rng(17)

    def obj(p, s):
        return float(p @ s + (4.0 / 3.0) * np.sum(p - p ** 1.5))

    for _ in range(50):
        n = int(rng.integers(2, 30))
        s = rng.normal(size=n) * 2
        p, tau, _ = orc.entmax15(s)
        best = obj(p, s)
        for _ in range(200):
            q = rng.dirichlet(np.ones(n) * 0.3)
            for eps in (1e-3, 1e-1, 1.0):
                cand = (1 - eps) * p + eps * q
                assert obj(cand, s) <= best + 1e-12
        # first-order (KKT) conditions: s - 2 sqrt(p) = tau on the support,
        # s <= tau off it
        sup = p > 0
        np.testing.assert_allclose(s[sup] - 2 * np.sqrt(p[sup]), tau, atol=1e-12)
        assert np.all(s[~sup] <= tau + 1e-12)


def test_tau_rows_matches_row_solver(orc):
    rng = np.random.default_rng(18)
    S = rng.normal(size=(64, 333)).astype(np.float32)
    tau, P = orc.tau_rows(S)
    for r in range(S.shape[0]):
        tb = bisect_tau(S[r].astype(np.float64))
        assert abs(tau[r] - tb) <= 1e-12 * max(1.0, abs(tb))
    np.testing.assert_allclose(P.sum(1), 1.0, atol=1e-12)
    assert np.array_equal(P > 0, S.astype(np.float64) > tau[:, None])


# ------------------------------------------------------------------- masks

def test_mask_predicate_table(orc):
    g = load_golden("mask_tables.json")
    L, W = g["L"], g["window"]
    for mode, table in g["modes"].items():
        for i in range(L):
            active = [j for j in range(L) if orc.key_active(int(mode), W, i, j)]
            assert active == table[i], (mode, i)


def test_window_mask_matches_model_card_formula(orc):
    # {0} U [max(1, i - W), i] for every i, W
    for W in (0, 1, 2, 5, 32):
        for i in range(80):
            want = sorted({0} | set(range(max(1, i - W), i + 1)))
            got = [j for j in range(80) if orc.key_active(2, W, i, j)]
            assert got == want


# -------------------------------------------------------- attention forward

def _np_scores(q, k, scale, mask, W):
    L = q.shape[0]
    s = scale * (q.astype(np.float64) @ k.astype(np.float64).T)
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    if mask == 1:
        s = np.where(j <= i, s, -np.inf)
    elif mask == 2:
        s = np.where((j <= i) & ((j == 0) | (i - j <= W)), s, -np.inf)
    return s


@pytest.mark.parametrize("mask,W", [(0, 0), (1, 0), (2, 3)])
def test_attn_fwd_plumbing_against_numpy(orc, mask, W):
    """S = scale Q K^T and O = A V checked with numpy matmuls; A's rows are
    pinned above."""
    rng = np.random.default_rng(19)
    B, H, L, d = 2, 3, 37, 16
    Q = rng.normal(size=(B, H, L, d)).astype(np.float32)
    K = rng.normal(size=(B, H, L, d)).astype(np.float32)
    V = rng.normal(size=(B, H, L, d)).astype(np.float32)
    scale = 0.3
    O, tau, nsup, gsum = orc.attn_fwd(Q, K, V, scale, mask, W)
    O = O.reshape(B, H, L, d)
    tau = tau.reshape(B, H, L)
    for b in range(B):
        for h in range(H):
            s = _np_scores(Q[b, h], K[b, h], scale, mask, W)
            A = np.zeros_like(s)
            for i in range(L):
                tb = bisect_tau(s[i])
                assert abs(tau[b, h, i] - tb) <= 1e-12 * max(1, abs(tb))
                A[i] = np.where(s[i] > tau[b, h, i], (0.5 * (s[i] - tau[b, h, i])) ** 2, 0.0)
            np.testing.assert_allclose(O[b, h], A @ V[b, h].astype(np.float64), atol=1e-12)
    # row subset gives the same rows
    rows = np.array([0, 5, L + 3, 3 * L - 1, B * H * L - 1])
    O2, tau2, _, _ = orc.attn_fwd(Q, K, V, scale, mask, W, rows=rows)
    np.testing.assert_array_equal(O2, O.reshape(-1, d)[rows])
    np.testing.assert_array_equal(tau2, tau.reshape(-1)[rows])


def test_attn_fwd_identity_values_return_weights(orc):
    # V = identity (d = L): O_i = A_i exactly
    rng = np.random.default_rng(20)
    L = 24
    Q = rng.normal(size=(1, 1, L, L)).astype(np.float32)
    K = rng.normal(size=(1, 1, L, L)).astype(np.float32)
    V = np.eye(L, dtype=np.float32)[None, None]
    O, tau, _, _ = orc.attn_fwd(Q, K, V, 0.5, 1, 0)
    s = _np_scores(Q[0, 0], K[0, 0], 0.5, 1, 0)
    for i in range(L):
        p, t, _ = orc.entmax15(s[i])
        np.testing.assert_array_equal(O[i], p)
        assert t == tau[i]
        assert abs(O[i].sum() - 1.0) < 1e-12


# ---------------------------------------------------------------- block mask

def test_block_mask_against_dense_weights(orc):
    rng = np.random.default_rng(21)
    L, d, br, bc = 150, 8, 16, 4
    for mask, W in ((0, 0), (1, 0), (2, 5)):
        Q = rng.normal(size=(L, d)).astype(np.float32)
        K = rng.normal(size=(L, d)).astype(np.float32)
        ex, lo, hi, tau = orc.block_mask_head(Q, K, 0.7, mask, W, br, bc, tol=1e-4)
        s = _np_scores(Q, K, 0.7, mask, W)
        A = np.zeros_like(s)
        for i in range(L):
            A[i], _, _ = orc.entmax15(s[i])
        Tr, Tc = -(-L // br), -(-L // bc)
        dense = np.zeros((Tr, Tc), dtype=bool)
        for I in range(Tr):
            for J in range(Tc):
                dense[I, J] = np.any(A[I * br:(I + 1) * br, J * bc:(J + 1) * bc] > 0)
        # unpack: bit J % 32 of word J // 32
        unpacked = np.zeros((Tr, Tc), dtype=bool)
        for I in range(Tr):
            for J in range(Tc):
                unpacked[I, J] = (int(ex[I, J // 32]) >> (J % 32)) & 1
        assert np.array_equal(unpacked, dense)
        # traversal by popcount / find-next-set: j = 32 m + bit position
        for I in range(Tr):
            js = []
            for m in range(ex.shape[1]):
                w = int(ex[I, m])
                while w:
                    b = (w & -w).bit_length() - 1
                    js.append(32 * m + b)
                    w &= w - 1
            assert js == list(np.nonzero(dense[I])[0])
        # the tolerance-band masks bracket the exact one
        assert np.all((lo & ~ex) == 0) and np.all((ex & ~hi) == 0)


# ------------------------------------------------------------------ backward

def _loss_fwd(orc, Q, K, V, dO, scale, mask, W):
    O, _, _, _ = orc.attn_fwd(Q[None, None], K[None, None], V[None, None], scale, mask, W)
    return float(np.sum(O * dO))


@pytest.mark.parametrize("mask,W", [(0, 0), (1, 0), (2, 3)])
def test_backward_against_finite_differences(orc, mask, W):
    """Central differences of sum(O * dO) in fp64.  The oracle's inputs are
    fp32 arrays, so the step is applied to values that fp32 holds exactly."""
    rng = np.random.default_rng(22 + mask)
    L, d, scale = 10, 5, 0.9
    Q = rng.normal(size=(L, d)).astype(np.float32)
    K = rng.normal(size=(L, d)).astype(np.float32)
    V = rng.normal(size=(L, d)).astype(np.float32)
    dO = rng.normal(size=(L, d)).astype(np.float32)
    dQ, dK, dV, tau, delta = orc.attn_bwd_head(Q, K, V, dO, scale, mask, W)
    h = 2.0 ** -12
    for name, X, G in (("Q", Q, dQ), ("K", K, dK), ("V", V, dV)):
        for idx in itertools.product(range(L), range(d)):
            Xp = X.copy(); Xm = X.copy()
            Xp[idx] += h; Xm[idx] -= h
            args = {"Q": Q, "K": K, "V": V}
            args[name] = Xp
            fp = _loss_fwd(orc, args["Q"], args["K"], args["V"], dO, scale, mask, W)
            args[name] = Xm
            fm = _loss_fwd(orc, args["Q"], args["K"], args["V"], dO, scale, mask, W)
            fd = (fp - fm) / (float(Xp[idx]) - float(Xm[idx]))
            assert abs(fd - G[idx]) <= 2e-5 * max(1.0, abs(G[idx])), (name, idx, fd, G[idx])


def test_backward_invariants(orc):
    rng = np.random.default_rng(25)
    L, d, scale = 40, 8, 0.6
    for mask, W in ((0, 0), (1, 0), (2, 4)):
        Q = rng.normal(size=(L, d)).astype(np.float32)
        K = rng.normal(size=(L, d)).astype(np.float32)
        V = rng.normal(size=(L, d)).astype(np.float32)
        dO = rng.normal(size=(L, d)).astype(np.float32)
        dQ, dK, dV, tau, delta = orc.attn_bwd_head(Q, K, V, dO, scale, mask, W)
        # a common shift of all keys moves each row's scores by a constant,
        # which leaves entmax unchanged: sum_j dK_j = 0
        np.testing.assert_allclose(dK.sum(0), 0.0, atol=1e-12)
        # rows of A sum to one: sum_j dV_j = sum_i dO_i
        np.testing.assert_allclose(dV.sum(0), dO.astype(np.float64).sum(0), atol=1e-12)
        # scaling V by c scales dA and delta by c: dQ, dK scale, dV does not
        dQ2, dK2, dV2, _, delta2 = orc.attn_bwd_head(Q, K, 2 * V, dO, scale, mask, W)
        np.testing.assert_allclose(dQ2, 2 * dQ, atol=1e-12)
        np.testing.assert_allclose(dV2, dV, atol=1e-12)
        np.testing.assert_allclose(delta2, 2 * delta, atol=1e-12)
        # the row-sampled variant agrees with the full head
        rows = np.array([0, 7, L - 1])
        dQr, deltar, taur = orc.attn_bwd_rows(Q[None, None], K[None, None], V[None, None],
                                              dO[None, None], scale, mask, W, rows)
        np.testing.assert_array_equal(dQr, dQ[rows])
        np.testing.assert_array_equal(deltar, delta[rows])
        np.testing.assert_array_equal(taur, tau[rows])


def test_backward_zero_off_support(orc):
    """A key outside every row's support gets dK = dV = 0 (gradients live on
    the support only, AdaSplash-2 sec. 3.3)."""
    rng = np.random.default_rng(26)
    L, d = 12, 4
    Q = np.abs(rng.normal(size=(L, d))).astype(np.float32) + 1
    K = rng.normal(size=(L, d)).astype(np.float32)
    K[5] = -10.0  # scores of key 5 far below every row's maximum
    V = rng.normal(size=(L, d)).astype(np.float32)
    dO = rng.normal(size=(L, d)).astype(np.float32)
    dQ, dK, dV, tau, delta = orc.attn_bwd_head(Q, K, V, dO, 1.0, 0, 0)
    assert np.all(dK[5] == 0) and np.all(dV[5] == 0)
