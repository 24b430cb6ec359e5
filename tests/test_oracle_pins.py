"""Pins of the float64 oracle against facts fixed by the pages or by mathematics.

Each test reaches the expected value by a route other than the oracle's own code: a library
routine (scipy softmax, Python sorting), a closed form, exact enumeration over rational cases
whose decision boundaries sit on a uniform grid, brute force, or a value printed on the pages
(tests/golden). A plausible slip in the oracle (a dropped term, a swapped p/q, a wrong index or
an off-by-one in the first-rejection scan) fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _logits(weights):
    """Logits whose softmax is exactly proportional to the given non-negative weights."""
    w = np.asarray(weights, dtype=np.float64)
    with np.errstate(divide="ignore"):
        return np.log(w)


def _grid(G):
    return (np.arange(G) + 0.5) / G


# ------------------------------------------------------------------------------------------
# softmax
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("T", [0.3, 0.7, 1.0, 2.5])
def test_softmax_is_scipy_softmax_of_scaled_logits(T):
    rng = np.random.default_rng(1)
    z = rng.normal(0, 3, size=257)
    np.testing.assert_allclose(O.softmax_t(z, T), sp_softmax(z / T), rtol=1e-13, atol=0)


def test_softmax_two_token_logistic_and_masked_entries():
    for d in [-7.0, -0.5, 0.0, 1.3, 9.0]:
        p = O.softmax_t(np.array([0.0, d]), 1.0)
        assert abs(p[1] - 1.0 / (1.0 + math.exp(-d))) < 1e-15
    p = O.softmax_t(np.array([-np.inf, 0.0, -np.inf, 0.0]), 0.5)
    assert list(p) == [0.0, 0.5, 0.0, 0.5]
    with pytest.raises(ValueError):
        O.softmax_t(np.zeros(3), 0.0)


# ------------------------------------------------------------------------------------------
# Saguaro
# ------------------------------------------------------------------------------------------
def test_saguaro_is_softmax_with_log_c_added_on_the_set():
    rng = np.random.default_rng(2)
    z = rng.normal(0, 2, size=300)
    S = [5, 17, 123]
    for C in [0.0, 0.1, 0.5, 0.9, 1.0]:
        q = O.softmax_t(z, 0.8)
        qp, sigma, N = O.saguaro(q, S, C)
        with np.errstate(divide="ignore"):
            shifted = z / 0.8 + np.where(np.isin(np.arange(300), S), np.log(C), 0.0)
        np.testing.assert_allclose(qp, sp_softmax(shifted), rtol=1e-12, atol=1e-300)
        assert abs(qp.sum() - 1.0) < 1e-12
        assert abs(sigma - sp_softmax(z / 0.8)[S].sum()) < 1e-14
        assert abs(N - (1 - (1 - C) * sigma)) < 1e-15


def test_saguaro_identity_conditional_and_set_hygiene():
    rng = np.random.default_rng(3)
    q = O.softmax_t(rng.normal(0, 1, size=50), 1.0)
    qp, sigma, N = O.saguaro(q, [3, 4], 1.0)
    assert np.array_equal(qp, q) and N == 1.0
    # C = 0 conditions on the complement of S
    qp0, _, _ = O.saguaro(q, [3, 4], 0.0)
    cond = q.copy()
    cond[[3, 4]] = 0
    cond /= cond.sum()
    np.testing.assert_allclose(qp0, cond, rtol=1e-13)
    # -1, out-of-range and repeated entries are ignored
    a = O.saguaro(q, [4, -1, 3, 4, 999, 3], 0.3)[0]
    b = O.saguaro(q, [4, 3], 0.3)[0]
    assert np.array_equal(a, b)
    with pytest.raises(ValueError):
        O.saguaro(np.array([0.5, 0.5]), [0, 1], 0.0)  # normaliser 0
    with pytest.raises(ValueError):
        O.saguaro(q, [1], 1.5)


def test_saguaro_raises_residual_mass_on_cached_tokens():
    """Lowering C lowers q on the cached tokens, so max(p - q', 0) gains mass there."""
    rng = np.random.default_rng(4)
    zq = rng.normal(0, 2, size=400)
    zp = zq + rng.normal(0, 0.5, size=400)
    p, q = O.softmax_t(zp, 1.0), O.softmax_t(zq, 1.0)
    S = list(np.argsort(-zq)[:3])
    prev = -1.0
    for C in [1.0, 0.7, 0.4, 0.1, 0.0]:
        qp, _, _ = O.saguaro(q, S, C)
        r = np.maximum(p - qp, 0.0)
        share = r[S].sum() / r.sum()
        assert share >= prev
        prev = share


# ------------------------------------------------------------------------------------------
# acceptance, first rejection, residual, lossless property
# Rational rows: softmax(log w) = w / sum(w); every decision boundary (p/q ratios, cumulative
# residual fractions) is a multiple of 1/G, so the midpoint-grid average is the exact probability.
# ------------------------------------------------------------------------------------------
P1, Q1 = [1, 2, 3, 2], [3, 1, 2, 2]          # a = [1/3, 1, 1, 1]; residual [0, 1, 1, 0]/8
P2, Q2 = [2, 2, 2, 2], [4, 2, 1, 1]          # a = [1/2, 1, 1, 1]; residual [0, 0, 1, 1]/8
P3 = [1, 3, 1, 1]                             # target row after the last draft position


def _norm(w):
    w = np.asarray(w, dtype=np.float64)
    return w / w.sum()


def test_acceptance_rate_is_sum_of_min_p_q():
    zq, zp = _logits([Q1]), _logits([P1, P3])
    q, p = _norm(Q1), _norm(P1)
    G = 24
    acc = 0.0
    for x in range(4):
        n = sum(O.verify_sequence(zq, zp, [x], [u, 0.5], 1.0).k == 1 for u in _grid(G))
        acc += q[x] * n / G
    assert abs(acc - np.minimum(p, q).sum()) < 1e-12
    assert abs(acc - 0.75) < 1e-12


def test_accept_rule_cases_from_the_blog():
    """p(x) >= q(x): always accepted; p(x) < q(x): accepted with probability p/q."""
    zq, zp = _logits([Q1]), _logits([P1, P3])
    for x in [1, 2, 3]:  # p >= q
        assert O.verify_sequence(zq, zp, [x], [np.float32(1 - 2 ** -24), 0.5], 1.0).k == 1
    r = O.verify_sequence(zq, zp, [0], [0.2, 0.5], 1.0)
    assert abs(r.a[0] - 1.0 / 3.0) < 1e-15 and r.k == 1
    assert O.verify_sequence(zq, zp, [0], [0.34, 0.5], 1.0).k == 0


@pytest.mark.parametrize("temperature", [1.0, 0.5])
def test_lossless_first_token_exact_enumeration(temperature):
    """Output token marginal equals p ([SD7.3] 7.3.3; [HW] section three; [SSD] 接受-拒绝机制)."""
    T = temperature
    zq, zp = _logits([Q1]) * T, _logits([P1, P3]) * T   # softmax(z/T) stays the rational rows
    q, p = _norm(Q1), _norm(P1)
    G = 24
    out = np.zeros(4)
    for x in range(4):
        for u1 in _grid(G):
            for u2 in _grid(G):
                r = O.verify_sequence(zq, zp, [x], [u1, u2], T)
                first = x if r.k >= 1 else r.bonus
                out[first] += q[x] / (G * G)
    np.testing.assert_allclose(out, p, atol=1e-12)


def test_lossless_with_saguaro_draft_distribution():
    """Drafting from q' (C on the set) and verifying against q' keeps the marginal equal to p."""
    zq = _logits([[1, 1, 1, 1]])
    zp = _logits([[3, 2, 1, 1], P3])
    S, C = [[0]], 0.5
    qp = np.array([1, 2, 2, 2]) / 7.0               # q' = q w / N with N = 7/8
    p = _norm([3, 2, 1, 1])
    G = 24
    out = np.zeros(4)
    for x in range(4):
        for u1 in _grid(G):
            for u2 in _grid(G):
                r = O.verify_sequence(zq, zp, [x], [u1, u2], 1.0, S, C)
                out[x if r.k >= 1 else r.bonus] += qp[x] / (G * G)
    np.testing.assert_allclose(out, p, atol=1e-12)


def test_lossless_two_positions_and_bonus_after_full_acceptance():
    zq = _logits([Q1, Q2])
    zp = _logits([P1, P2, P3])
    q1, q2 = _norm(Q1), _norm(Q2)
    G = 12
    first = np.zeros(4)
    second = np.zeros(4)       # second emitted token, given the first draft was accepted
    third = np.zeros(4)        # bonus after both drafts were accepted
    p_k1 = p_k2 = 0.0
    g = _grid(G)
    for x1, x2 in itertools.product(range(4), range(4)):
        w = q1[x1] * q2[x2] / G ** 3
        for u1, u2, u3 in itertools.product(g, g, g):
            r = O.verify_sequence(zq, zp, [x1, x2], [u1, u2, u3], 1.0)
            first[x1 if r.k >= 1 else r.bonus] += w
            if r.k >= 1:
                p_k1 += w
                second[x2 if r.k == 2 else r.bonus] += w
            if r.k == 2:
                p_k2 += w
                third[r.bonus] += w
    np.testing.assert_allclose(first, _norm(P1), atol=1e-12)
    np.testing.assert_allclose(second / p_k1, _norm(P2), atol=1e-12)
    np.testing.assert_allclose(third / p_k2, _norm(P3), atol=1e-12)


def test_lossless_two_positions_with_per_position_saguaro():
    """Drafts from per-position q'_i (C_1 = 1/3 and C_2 = 1/2 on token 0), verified against them:
    every emitted token keeps the target marginal. q'_1 = [1,1,2,2]/6 and q'_2 = [2,2,1,1]/6 are
    worked by hand; every decision boundary falls on the 1/12 grid, so the integral is exact."""
    zq = _logits([Q1, Q2])
    zp = _logits([P1, P2, P3])
    q1, q2 = np.array([1, 1, 2, 2]) / 6.0, np.array([2, 2, 1, 1]) / 6.0
    G = 12
    first, second, third = np.zeros(4), np.zeros(4), np.zeros(4)
    p_k1 = p_k2 = 0.0
    g = _grid(G)
    for x1, x2 in itertools.product(range(4), range(4)):
        w = q1[x1] * q2[x2] / G ** 3
        for u1, u2, u3 in itertools.product(g, g, g):
            r = O.verify_sequence(zq, zp, [x1, x2], [u1, u2, u3], 1.0, [[0], [0]], [1.0 / 3.0, 0.5])
            first[x1 if r.k >= 1 else r.bonus] += w
            if r.k >= 1:
                p_k1 += w
                second[x2 if r.k == 2 else r.bonus] += w
            if r.k == 2:
                p_k2 += w
                third[r.bonus] += w
    np.testing.assert_allclose(first, _norm(P1), atol=1e-12)
    np.testing.assert_allclose(second / p_k1, _norm(P2), atol=1e-12)
    np.testing.assert_allclose(third / p_k2, _norm(P3), atol=1e-12)
    # the accept probabilities of the first position against the hand-worked q'_1
    r = O.verify_sequence(zq, zp, [0, 0], [0.5, 0.5, 0.5], 1.0, [[0], [0]], [1.0 / 3.0, 0.5])
    assert r.a[0] == pytest.approx(0.75, abs=1e-15)


def test_accepted_length_is_geometric_with_identical_rows():
    """[SSD] 最优扇出度分配: with the same acceptance rate a at every position the accepted
    length is geometric, P(k) = (1-a) a^k (k < K), a^K (k = K)."""
    p, q = [3, 2, 1], [2, 3, 1]        # a(x) = [1, 2/3, 1]; acceptance rate 5/6
    K, G = 3, 6
    zq, zp = _logits([q] * K), _logits([p] * (K + 1))
    qn = _norm(q)
    hist = np.zeros(K + 1)
    g = _grid(G)
    for xs in itertools.product(range(3), repeat=K):
        w = np.prod(qn[list(xs)]) / G ** K
        for us in itertools.product(g, repeat=K):
            hist[O.verify_sequence(zq, zp, list(xs), list(us) + [0.5], 1.0).k] += w
    alpha = 5.0 / 6.0
    expect = [(1 - alpha) * alpha ** k for k in range(K)] + [alpha ** K]
    np.testing.assert_allclose(hist, expect, atol=1e-12)
    np.testing.assert_allclose(O.geometric_pk(K, alpha), expect, atol=1e-15)


def test_residual_mass_is_one_minus_acceptance_rate():
    rng = np.random.default_rng(5)
    for trial in range(20):
        V = 64
        zq = rng.normal(0, 2, size=(1, V))
        zp = np.vstack([zq[0] + rng.normal(0, 0.7, size=V), rng.normal(0, 2, size=V)])
        p, q = sp_softmax(zp[0]), sp_softmax(zq[0])
        x = int(np.argmax(q - p))                       # p(x) < q(x): rejectable
        r = O.verify_sequence(zq, zp, [x], [np.float32(1 - 2 ** -24), 0.3], 1.0)
        assert r.k == 0
        assert abs(r.R - (1.0 - np.minimum(p, q).sum())) < 1e-12


def test_bonus_inverse_cdf_closed_forms():
    # Residual uniform on {1, 2} (tokens 0 and 3 carry none): bonus = 1 for u < 1/2, else 2.
    zq, zp = _logits([Q1]), _logits([P1, P3])
    for u in _grid(40):
        r = O.verify_sequence(zq, zp, [0], [0.99, u], 1.0)
        assert r.k == 0 and r.bonus == (1 if u < 0.5 else 2)
    # All drafts accepted, uniform target row over V: bonus = floor(u V).
    V = 10
    zq = np.zeros((2, V))
    zp = np.zeros((3, V))
    zp[:2] = np.random.default_rng(11).normal(0, 3, size=(2, V))   # only row K is uniform
    for u in _grid(97):
        r = O.verify_sequence(zq, zp, [3, 7], [0.0, 0.0, u], 1.0)
        assert r.k == 2 and r.bonus == int(math.floor(u * V))
        assert abs(r.c_lo - r.bonus / V) < 1e-15 and abs(r.c_hi - (r.bonus + 1) / V) < 1e-15
    # Residual concentrated on one token: the bonus is that token for every u.
    zq = _logits([[1, 1, 0, 1]])
    zp = _logits([[1, 1, 5, 1], P3])
    for u in _grid(31):
        r = O.verify_sequence(zq, zp, [1], [0.999, u], 1.0)
        assert r.k == 0 and r.bonus == 2


def test_bonus_never_lands_on_zero_mass_tokens():
    rng = np.random.default_rng(6)
    V = 300
    for trial in range(30):
        zq = rng.normal(0, 2, size=(1, V))
        zp = np.vstack([zq[0] + rng.normal(0, 0.5, size=V), rng.normal(0, 2, size=V)])
        p, q = sp_softmax(zp[0]), sp_softmax(zq[0])
        x = int(np.argmax(q - p))
        r = O.verify_sequence(zq, zp, [x], [0.9999999, rng.random()], 1.0)
        assert r.k == 0 and p[r.bonus] > q[r.bonus]


# ------------------------------------------------------------------------------------------
# top-F
# ------------------------------------------------------------------------------------------
def test_topf_matches_python_sort_with_ties_and_masking():
    rng = np.random.default_rng(7)
    for trial in range(200):
        V = int(rng.integers(1, 60))
        z = rng.integers(-3, 4, size=V).astype(np.float64)     # many ties
        z[rng.random(V) < 0.1] = -np.inf
        F = int(rng.integers(0, V + 3))
        ex = int(rng.integers(-1, V))
        want = [v for v in sorted(range(V), key=lambda v: (-z[v], v)) if v != ex and z[v] != -np.inf][:F]
        want += [-1] * (F - len(want))
        assert list(O.topf(z, F, ex)) == want


def test_topf_distinct_values_is_argsort():
    rng = np.random.default_rng(8)
    z = rng.permutation(1000).astype(np.float64)
    assert list(O.topf(z, 5)) == list(np.argsort(-z)[:5])
    assert list(O.topf(z, 5, int(np.argmax(z)))) == list(np.argsort(-z)[1:6])


# ------------------------------------------------------------------------------------------
# draft-side Saguaro sampling
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("F,C,T", [(0, 1.0, 1.0), (3, 0.2, 0.8), (7, 0.0, 1.3), (5, 1.0, 0.5)])
def test_saguaro_sample_is_the_library_inverse_cdf(F, C, T):
    """x is scipy's discrete quantile function of q' (the pinned saguaro() over the pinned top-F
    set), for random u; the reported set, mass and normaliser are those of the same q'."""
    from scipy.stats import rv_discrete
    rng = np.random.default_rng(11 + F)
    V = 300
    z = rng.normal(0, 2, size=V)
    z[rng.random(V) < 0.05] = -np.inf
    S = O.topf(z, F)
    qs, sig, N = O.saguaro(O.softmax_t(z, T), [int(v) for v in S if v >= 0], C)
    dist = rv_discrete(values=(np.arange(V), qs / qs.sum()))
    for u in rng.random(200):
        r = O.saguaro_sample(z, T, F, C, float(u))
        assert r.x == int(dist.ppf(u))
        assert list(r.S) == list(S) and r.sigma == sig and r.N == N
        assert r.qx == qs[r.x] and r.c_lo <= u < r.c_hi


def test_saguaro_sample_grid_frequencies_are_q_prime():
    """Uniforms on a midpoint grid of G points land on token v about G q'(v) times (within one
    point per boundary): the inverse CDF carries the uniform onto q'."""
    w = np.array([3, 1, 4, 1, 5, 9, 2, 6, 5, 3, 5, 8], dtype=np.float64)
    z = _logits(w)
    G = 20000
    xs = np.array([O.saguaro_sample(z, 1.0, 3, 0.25, u).x for u in _grid(G)])
    top3 = {5, 11, 7}  # weights 9, 8, 6
    ww = np.array([wi * (0.25 if v in top3 else 1.0) for v, wi in enumerate(w)])
    want = G * ww / ww.sum()
    assert np.abs(np.bincount(xs, minlength=len(w)) - want).max() <= 1.0


def test_saguaro_sample_edges():
    """u = 0 gives the first token of positive mass; u at or past 1 the last; C = 0 never draws a
    set member; a masked token is never drawn."""
    z = np.array([-np.inf, 0.5, 2.0, -np.inf, 1.0, 3.0, -1.0, -np.inf])
    assert O.saguaro_sample(z, 1.0, 2, 0.5, 0.0).x == 1
    assert O.saguaro_sample(z, 1.0, 2, 0.5, 1.0).x == 6
    assert O.saguaro_sample(z, 1.0, 2, 0.5, 1.0 - 1e-15).x == 6
    xs = {O.saguaro_sample(z, 0.7, 2, 0.0, u).x for u in _grid(5000)}
    assert xs == {1, 4, 6}  # every unmasked token outside the top two {5, 2}
    xs = {O.saguaro_sample(z, 0.7, 0, 0.0, u).x for u in _grid(5000)}
    assert xs == {1, 2, 4, 5, 6}


# ------------------------------------------------------------------------------------------
# fan-out
# ------------------------------------------------------------------------------------------
def _objective(P, F, r):
    return sum(P[k] * F[k] ** (-r) for k in range(len(P)))


def _brute_force(P, r, budget):
    best, arg = None, None
    n = len(P)
    for cut in itertools.combinations(range(1, budget), n - 1):   # compositions with F_k >= 1
        F = np.diff((0,) + cut + (budget,))
        v = _objective(P, F, r)
        if best is None or v < best - 1e-15:
            best, arg = v, F
    return arg, best


@pytest.mark.parametrize("budget", [12, 32])
def test_fanout_integer_matches_brute_force_optimum(budget):
    K, a, r = 4, 0.7, 1.0
    F, Fc = O.fanout(K, a, r, budget)
    P = O.geometric_pk(K, a)
    arg, best = _brute_force(P, r, budget)
    assert int(F.sum()) == budget
    assert abs(_objective(P, F, r) - best) < 1e-12
    assert list(F) == list(arg)


@pytest.mark.parametrize("K,a,r,budget", [(4, 0.7, 1.0, 12), (4, 0.7, 1.0, 32), (8, 0.55, 0.5, 100),
                                          (2, 0.9, 2.0, 7)])
def test_fanout_continuous_is_the_lagrange_stationary_point(K, a, r, budget):
    F, Fc = O.fanout(K, a, r, budget)
    P = O.geometric_pk(K, a)
    assert abs(Fc.sum() - budget) < 1e-9
    # stationarity of sum_k P(k) F_k^-r + lambda sum_k F_k: P(k) F_k^-(1+r) is one constant
    g = P * Fc ** (-(1 + r))
    np.testing.assert_allclose(g, g[0], rtol=1e-12)
    # for k < K the page's closed form F_k = F_0 a^(k/(1+r))
    np.testing.assert_allclose(Fc[1:K] / Fc[:K - 1], a ** (1 / (1 + r)), rtol=1e-12)
    # integers are a rounding of the continuous optimum
    assert int(F.sum()) == budget and np.all(np.abs(F - Fc) < 1.0)


def test_fanout_twelve_branch_case_and_edges():
    g = json.load(open(os.path.join(GOLDEN, "ssd_branch_build.json")))
    F, _ = O.fanout(g["K"], 0.7, 1.0, g["branches"])
    assert len(F) == g["K"] + 1 and int(F.sum()) == g["branches"]
    assert list(O.fanout(4, 0.7, 1.0, 0)[0]) == [0] * 5
    for bad in [(4, 1.0, 1.0, 3), (4, 0.5, 0.0, 3), (4, 0.5, 1.0, -1)]:
        with pytest.raises(ValueError):
            O.fanout(*bad)


def test_branch_build_shape_from_the_page():
    g = json.load(open(os.path.join(GOLDEN, "ssd_branch_build.json")))
    lay = O.branch_layout(g["branches"], g["K"])
    assert lay["serial_forwards"] == g["serial_forwards"]
    assert lay["batched_forwards"] == g["batched_forwards"]
    assert lay["batch_size"] == g["batch_size"]


# ------------------------------------------------------------------------------------------
# speculation cache
# ------------------------------------------------------------------------------------------
def test_cache_keys_layout_and_lookup_against_a_dict():
    rng = np.random.default_rng(9)
    K, F = 4, [3, 2, 2, 2, 3]
    for trial in range(50):
        guesses = [list(rng.permutation(20)[:Fk]) for Fk in F]
        if trial % 5 == 0:
            guesses[1][1] = -1
        kk, tt = O.cache_keys(guesses, F)
        assert len(kk) == sum(F)
        table = {}
        j = 0
        for k, Fk in enumerate(F):
            for rank in range(Fk):
                t = guesses[k][rank]
                if t >= 0:
                    table.setdefault((k, t), j)
                    assert (kk[j], tt[j]) == (k, t)
                else:
                    assert (kk[j], tt[j]) == (-1, -1)
                j += 1
        for k in range(K + 1):
            for t in range(20):
                assert O.cache_lookup(kk, tt, k, t) == table.get((k, t), -1)
        assert O.cache_lookup(kk, tt, -1, -1) == -1 or (-1, -1) in [(a, b) for a, b in zip(kk, tt)]


def test_all_hit_fraction_decays_as_h_to_the_b():
    rng = np.random.default_rng(10)
    h, B, rounds = 0.8, 6, 20000
    all_hit = 0
    for _ in range(rounds):
        miss = 0
        for b in range(B):
            k, t = int(rng.integers(0, 5)), int(rng.integers(0, 100))
            kk = np.array([k if rng.random() < h else (k + 1) % 5])
            tt = np.array([t])
            miss += O.cache_lookup(kk, tt, k, t) < 0
        all_hit += miss == 0
    frac = all_hit / rounds
    expect = O.all_hit_probability(h, B)
    assert abs(expect - h ** B) < 1e-15
    assert abs(frac - expect) < 4 * math.sqrt(expect * (1 - expect) / rounds)


def test_ninety_two_percent_example():
    g = json.load(open(os.path.join(GOLDEN, "all_hit_92.json")))
    miss = 1.0 - O.all_hit_probability(g["h"], g["B"])
    assert abs(miss - g["fraction_rounds_with_miss"]) < g["abs_tol"]


# ------------------------------------------------------------------------------------------
# batch speedup and the backup speculator's crossover
# ------------------------------------------------------------------------------------------
def test_batch_speedup_hand_values_and_limits():
    # h = 0.9, E_hit = 4, E_miss = 2, T_p = 0.5, T_b = 1: tokens 3.6 + 0.2 = 3.8 per round;
    # b = 1 waits 0.1, b = 2 waits 1 - 0.81 = 0.19 of a verification for the backup
    assert abs(O.batch_speedup(0.9, 4, 2, 0.5, 1.0, 1) - 3.8 / 1.1) < 1e-12
    assert abs(O.batch_speedup(0.9, 4, 2, 0.5, 1.0, 2) - 3.8 / 1.19) < 1e-12
    # a primary speculator slower than the verification sets the round: 3.8 / (1.5 + 0.1)
    assert abs(O.batch_speedup(0.9, 4, 2, 1.5, 1.0, 1) - 3.8 / 1.6) < 1e-12
    # every sequence hits: no wait at any batch size; every one misses: always the backup
    for b in (1, 7, 1000):
        assert O.batch_speedup(1.0, 5, 1, 0.2, 3.0, b) == 5.0
        assert abs(O.batch_speedup(0.0, 5, 1.5, 0.2, 0.5, b) - 1.5 / 1.5) < 1e-12
    # large batches: the backup's latency alone bounds it (the page's limit)
    assert abs(O.batch_speedup(0.9, 4, 2, 0.5, 1.0, 10 ** 4) - 3.8 / 2.0) < 1e-12


def test_batch_speedup_falls_with_the_batch_as_all_hit_probability_does():
    S = [O.batch_speedup(0.93, 4.5, 2.0, 0.8, 0.7, b) for b in range(1, 200)]
    assert all(a >= c for a, c in zip(S, S[1:]))
    # the wait term is exactly the probability that not all sequences hit (the 92 % example)
    s24 = O.batch_speedup(0.9, 1.0, 1.0, 0.0, 1.0, 24)
    assert abs((1.0 / s24 - 1.0) - (1.0 - O.all_hit_probability(0.9, 24))) < 1e-12


@pytest.mark.parametrize("seed", range(6))
def test_backup_crossover_is_the_first_batch_where_the_fast_backup_wins(seed):
    """Brute force over integer batch sizes against the analytic crossover."""
    rng = np.random.default_rng(seed)
    found = 0
    while found < 20:
        h = rng.uniform(0.5, 0.99)
        E_hit = rng.uniform(2, 6)
        En, Ef = rng.uniform(1.5, 4), rng.uniform(1.0, 1.5)   # the neural backup drafts better
        Tn, Tf = rng.uniform(0.3, 2.0), rng.uniform(0.0, 0.1)  # and takes longer
        Tp = rng.uniform(0.1, 1.5)
        bs, fast_large = O.backup_crossover(h, E_hit, En, Tn, Ef, Tf, Tp)
        wins = [O.batch_speedup(h, E_hit, Ef, Tp, Tf, b) >= O.batch_speedup(h, E_hit, En, Tp, Tn, b)
                for b in range(1, 3001)]
        assert fast_large == (O.batch_speedup(h, E_hit, Ef, Tp, Tf, 10 ** 6)
                              >= O.batch_speedup(h, E_hit, En, Tp, Tn, 10 ** 6))
        if math.isnan(bs) or bs > 2500:
            assert all(w == wins[0] for w in wins) or bs > 2500
            continue
        found += 1
        first = wins.index(True) + 1 if fast_large else None
        if fast_large:
            assert first == max(1, math.ceil(bs)), (bs, first)
            assert all(wins[first - 1:])
        # the two speedups agree at the real crossing
        assert abs(O.batch_speedup(h, E_hit, Ef, Tp, Tf, bs) - O.batch_speedup(h, E_hit, En, Tp, Tn, bs)) < 1e-9


def test_batch_speedup_matches_a_simulated_two_gpu_schedule():
    """[SSD] "SSD 的核心思想": the speculator runs on its own GPU while the target verifies, so a round
    ends when both have finished; a batch with any miss then waits for the backup. An event-by-event
    simulation of that schedule (per-sequence random hits, the two GPUs' finish times, the backup's
    wait) gives tokens per unit of verification time; over many rounds it must approach
    batch_speedup, for a primary faster and slower than the verification."""
    rng = np.random.default_rng(17)
    for h, E_hit, E_miss, T_p, T_b, b in [(0.9, 4.0, 2.0, 0.5, 1.0, 4), (0.8, 3.0, 1.5, 1.7, 0.6, 3),
                                           (0.95, 5.0, 1.0, 1.0, 2.0, 16)]:
        rounds = 200000
        tokens = 0.0
        clock = 0.0
        hits = rng.random((rounds, b)) < h
        for r in range(rounds):
            start = clock
            verify_done = start + 1.0          # the target's verification, one unit
            spec_done = start + T_p            # the speculator's cache, on the other GPU
            clock = max(verify_done, spec_done)
            if not hits[r].all():              # some sequence missed: everyone waits for the backup
                clock += T_b
            tokens += np.where(hits[r], E_hit, E_miss).sum() / b  # per sequence
        sim = tokens / clock
        assert abs(sim - O.batch_speedup(h, E_hit, E_miss, T_p, T_b, b)) < 0.01 * sim, (h, T_p, b, sim)


def test_ssd_round_keys_outcome_k_with_the_guesses_of_draft_row_k():
    """[SSD] "怎么猜奖励 token" with "SSD 的核心思想": the outcome (k, t) is looked up among the guesses
    of draft position k (the extra draft row for k = K), which exclude the sampled token x_k. Rows
    built so that the round ends at (k, t_k), t_k the best token of draft row k other than x_k and of
    no other row: the lookup hits, at the first slot of position k (the second for the extra row,
    whose favourite is not excluded), for every k."""
    K, V, T = 3, 9, 1.0
    F = [2, 2, 2, 2]
    for k in range(K + 1):
        draft = np.full((1, K + 1, V), -4.0, dtype=np.float32)
        target = np.full((1, K + 1, V), -4.0, dtype=np.float32)
        x = np.zeros((1, K), dtype=np.int64)             # every draft token is 0, the draft's favourite
        for i in range(K + 1):
            draft[0, i, 0] = 3.0
            draft[0, i, 3 + i] = 2.0                     # t_i = 3 + i: row i's best other token
            draft[0, i, 1] = 1.0
        for i in range(k):
            target[0, i] = draft[0, i]                   # p = q: accepted for any u < 1
        # the target at position k (k < K: reject x_k = 0, residual on t_k; k = K: bonus drawn
        # from p_K) puts its mass on t_k
        target[0, k, :] = -20.0
        target[0, k, 3 + k] = 20.0
        u = np.full((1, K + 1), 0.5, dtype=np.float32)
        res = O.ssd_round(draft, target, "f32", x, u, T, None, 1.0, F)[0]
        assert (res["k"], res["bonus"]) == (k, 3 + k)
        # row K has no sampled token to exclude: its favourite, token 0, is its first guess
        want = sum(F[:k]) + (1 if k == K else 0)
        assert res["slot"] == want, (k, res["slot"], res["keys_k"], res["keys_t"])
        assert res["keys_k"][res["slot"]] == k and res["keys_t"][res["slot"]] == 3 + k
