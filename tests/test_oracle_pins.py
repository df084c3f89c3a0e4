"""Pins for the fp64 oracle: each test checks it against a route that does not
share its arithmetic (matrix exponential of the ODE, RK4 integration, closed
forms, 60-digit evaluation, invariants the pages state).

Source: "Exact Flow Linear Attention: Exact Solution from Continuous-Time
Dynamics", gist.science summary pages, Method steps 1-3 and Key Contributions
(stability).  Readout o_t = S_t^T q_t is the definition this project uses.
"""
import math

import mpmath
import numpy as np
import pytest
import scipy.linalg

import oracle

mpmath.mp.dps = 60


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# Coefficient alpha = (1 - exp(-beta*lambda)) / lambda   (Method step 3)
# ---------------------------------------------------------------------------

def _alpha_mp(beta, lam):
    """The plain definition, evaluated with enough digits to survive the
    cancellation in 1 - exp(-x) for x down to 1e-340."""
    if lam == 0:
        return mpmath.mpf(beta)
    with mpmath.workdps(420):
        b, l = mpmath.mpf(beta), mpmath.mpf(lam)
        return +((1 - mpmath.exp(-b * l)) / l)


@pytest.mark.parametrize("beta", [0.0, 1e-30, 1e-8, 0.05, 0.5, 1.0, 3.0, 10.0])
def test_alpha_matches_60_digit_evaluation(beta):
    lams = [0.0, 1e-300, 1e-30, 1e-12, 1e-6, 1e-3, 0.1, 1.0, 16.0, 88.0, 900.0, 1e4, 1e8]
    for lam in lams:
        got = oracle.alpha(beta, lam)
        ref = float(_alpha_mp(beta, lam))
        if ref == 0.0:
            assert got == 0.0
        else:
            assert abs(got - ref) <= 6e-16 * abs(ref), (beta, lam, got, ref)


def test_alpha_limits():
    # lambda -> 0 recovers beta (the DeltaNet / Euler coefficient)
    assert oracle.alpha(0.37, 0.0) == 0.37
    # beta*lambda -> infinity: alpha -> 1/lambda (exact overwrite along k)
    assert oracle.alpha(math.inf, 4.0) == 0.25
    assert abs(oracle.alpha(1e6, 3.0) - 1.0 / 3.0) <= 1e-16
    # beta = 0 is the identity step
    assert oracle.alpha(0.0, 5.0) == 0.0


def test_coeff_lambda_is_squared_norm():
    rng = _rng(1)
    k = rng.standard_normal((7, 5))
    beta = rng.uniform(0, 3, 7)
    lam, alp = oracle.coeff(k, beta)
    for t in range(7):
        ref_lam = mpmath.fsum(mpmath.mpf(x) ** 2 for x in k[t])
        assert abs(lam[t] - float(ref_lam)) <= 1e-15 * float(ref_lam)
        assert abs(alp[t] - float(_alpha_mp(beta[t], ref_lam))) <= 1e-15 * alp[t]


# ---------------------------------------------------------------------------
# P1: e^{-beta A} = I - alpha A for A = k k^T  (Method step 2), against a
# brute-force Taylor series with scaling and squaring, and scipy's expm.
# ---------------------------------------------------------------------------

def _taylor_expm(M):
    """exp(M) by scaling and squaring around a plain Taylor series."""
    nrm = np.abs(M).sum(axis=1).max()
    s = max(0, int(math.ceil(math.log2(nrm))) + 1) if nrm > 0 else 0
    X = M / (2.0 ** s)
    E = np.eye(M.shape[0])
    term = np.eye(M.shape[0])
    for n in range(1, 60):
        term = term @ X / n
        E = E + term
        if np.abs(term).max() < 1e-20:
            break
    for _ in range(s):
        E = E @ E
    return E


@pytest.mark.parametrize("seed,scale,beta", [(11, 1.0, 0.7), (12, 4.0, 1.1), (13, 0.05, 2.0),
                                             (14, 3.0, 0.01), (15, 2.0, 1.9)])
def test_P1_closed_form_matches_taylor_expm(seed, scale, beta):
    rng = _rng(seed)
    d = 6
    k = scale * rng.standard_normal(d)
    A = np.outer(k, k)
    # one oracle step from S = I with v = 0 gives (I - alpha k k^T)
    o, S1 = oracle.step(np.zeros((1, 1, d)), k[None, None], np.zeros((1, 1, d)),
                        np.array([[beta]]), np.eye(d)[None, None])
    ref = _taylor_expm(-beta * A)
    assert np.abs(S1[0, 0] - ref).max() <= 1e-12
    assert np.abs(S1[0, 0] - scipy.linalg.expm(-beta * A)).max() <= 1e-12


# ---------------------------------------------------------------------------
# P2: the exact step integrates dS/dt = -A S + k v^T for time beta
# (ZOH ODE of Method step 1).  Fine-step RK4 must agree to 1e-8.
# ---------------------------------------------------------------------------

def _rk4_token(S, k, v, beta):
    lam = float(k @ k)
    n = max(50, int(math.ceil(beta * lam / 0.02)))
    h = beta / n
    kv = np.outer(k, v)

    def f(X):
        return -np.outer(k, k @ X) + kv

    for _ in range(n):
        a = f(S)
        b = f(S + 0.5 * h * a)
        c = f(S + 0.5 * h * b)
        d = f(S + h * c)
        S = S + (h / 6.0) * (a + 2 * b + 2 * c + d)
    return S


@pytest.mark.parametrize("seed,kscale,beta", [(21, 1.0, 0.6), (22, 4.0, 0.9), (23, 0.3, 3.0),
                                              (24, 2.5, 0.4)])
def test_P2_exact_step_matches_rk4(seed, kscale, beta):
    rng = _rng(seed)
    dk, dv = 5, 3
    S0 = rng.standard_normal((dk, dv))
    k = kscale * rng.standard_normal(dk)
    v = rng.standard_normal(dv)
    _, S1 = oracle.step(np.zeros((1, 1, dk)), k[None, None], v[None, None],
                        np.array([[beta]]), S0[None, None])
    ref = _rk4_token(S0.copy(), k, v, beta)
    assert np.abs(S1[0, 0] - ref).max() <= 1e-8 * max(1.0, np.abs(ref).max())


def _ode_trajectory(q, k, v, beta, s0):
    """Exact solution of the ZOH ODE over each token (block matrix exponential).

    For Y = [S; I_dv], dY/dt = [[-k k^T, k v^T], [0, 0]] Y, so
    Y(beta) = expm(beta * M) Y(0): the top-right block is the input integral.
    """
    L, dk = k.shape
    dv = v.shape[1]
    S = s0.copy()
    outs = np.zeros((L, dv))
    for t in range(L):
        M = np.zeros((dk + dv, dk + dv))
        M[:dk, :dk] = -np.outer(k[t], k[t])
        M[:dk, dk:] = np.outer(k[t], v[t])
        E = scipy.linalg.expm(beta[t] * M)
        S = E[:dk, :dk] @ S + E[:dk, dk:]
        outs[t] = S.T @ q[t]
    return outs, S


def test_P2b_forward_matches_ode_solution_all_heads():
    """Whole forward pass, several (b, h) with dk != dv, vs the ODE solved by expm."""
    rng = _rng(31)
    B, L, H, dk, dv = 2, 12, 3, 5, 4
    q = rng.standard_normal((B, L, H, dk))
    k = 1.5 * rng.standard_normal((B, L, H, dk))
    v = rng.standard_normal((B, L, H, dv))
    beta = rng.uniform(0.0, 2.0, (B, L, H))
    s0 = rng.standard_normal((B, H, dk, dv))
    o, sf = oracle.forward(q, k, v, beta, s0)
    for b in range(B):
        for h in range(H):
            ro, rs = _ode_trajectory(q[b, :, h], k[b, :, h], v[b, :, h], beta[b, :, h], s0[b, h])
            scale = max(1.0, np.abs(ro).max())
            assert np.abs(o[b, :, h] - ro).max() <= 1e-12 * scale
            assert np.abs(sf[b, h] - rs).max() <= 1e-12 * max(1.0, np.abs(rs).max())


# ---------------------------------------------------------------------------
# P3: projection invariant along the key (Key Contributions: the exact flow
# contracts the key-aligned memory component by exp(-beta*lambda)).
#   k^T S_t = e^{-beta lambda} k^T S_{t-1} + (1 - e^{-beta lambda}) v^T
# P5: directions orthogonal to k are untouched.
# ---------------------------------------------------------------------------

def test_P3_P5_projection_invariants():
    rng = _rng(41)
    dk, dv = 7, 5
    for trial in range(20):
        S0 = rng.standard_normal((dk, dv))
        k = rng.uniform(0.2, 3.0) * rng.standard_normal(dk)
        v = rng.standard_normal(dv)
        beta = rng.uniform(0.0, 4.0)
        _, S1 = oracle.step(np.zeros((1, 1, dk)), k[None, None], v[None, None],
                            np.array([[beta]]), S0[None, None])
        S1 = S1[0, 0]
        e = math.exp(-beta * float(k @ k))
        lhs = k @ S1
        rhs = e * (k @ S0) + (1.0 - e) * v
        assert np.abs(lhs - rhs).max() <= 1e-12 * max(1.0, np.abs(rhs).max())
        # u orthogonal to k
        u = rng.standard_normal(dk)
        u -= (u @ k) / (k @ k) * k
        assert np.abs(u @ S1 - u @ S0).max() <= 1e-12 * max(1.0, np.abs(u @ S0).max())


# ---------------------------------------------------------------------------
# P4: Euler limit.  The explicit-Euler (DeltaNet) step uses beta in place of
# alpha (Problem / Key Contributions: the delta rule is the Euler discretisation).
# |alpha - beta| <= beta^2 lambda / 2, and the states converge as beta*lambda -> 0.
# ---------------------------------------------------------------------------

def test_P4_euler_limit():
    rng = _rng(51)
    dk, dv = 4, 3
    S0 = rng.standard_normal((dk, dv))
    k = rng.standard_normal(dk)
    v = rng.standard_normal(dv)
    lam = float(k @ k)
    prev = None
    for x in [1e-2, 1e-4, 1e-6, 1e-8]:
        beta = x / lam
        a = oracle.alpha(beta, lam)
        assert -4 * np.spacing(beta) <= beta - a <= beta * beta * lam / 2 + 4 * np.spacing(beta)
        _, S1 = oracle.step(np.zeros((1, 1, dk)), k[None, None], v[None, None],
                            np.array([[beta]]), S0[None, None])
        euler = S0 - beta * np.outer(k, k @ S0) + beta * np.outer(k, v)
        diff = np.abs(S1[0, 0] - euler).max()
        assert diff <= (beta * beta * lam / 2) * np.abs(k).max() * (
            np.abs(k @ S0).max() + np.abs(v).max()) * 1.01 + 1e-15
        if prev is not None:
            assert diff <= prev
        prev = diff


# ---------------------------------------------------------------------------
# P6: stiff limit beta*lambda -> infinity: the key-aligned component is
# overwritten by v exactly (the contraction factor e^{-beta lambda} vanishes).
# ---------------------------------------------------------------------------

def test_P6_stiff_limit_overwrites():
    rng = _rng(61)
    dk, dv = 6, 4
    S0 = rng.standard_normal((dk, dv))
    k = 3.0 * rng.standard_normal(dk)
    v = rng.standard_normal(dv)
    beta = 50.0 / float(k @ k) * 2  # beta*lambda = 100
    _, S1 = oracle.step(np.zeros((1, 1, dk)), k[None, None], v[None, None],
                        np.array([[beta]]), S0[None, None])
    assert np.abs(k @ S1[0, 0] - v).max() <= 1e-12 * max(1.0, np.abs(v).max())
    assert abs(oracle.alpha(beta, float(k @ k)) * float(k @ k) - 1.0) <= 1e-15


# ---------------------------------------------------------------------------
# P7: the exact flow is non-expansive (Key Contributions, stability): two
# trajectories driven by the same tokens never move apart in spectral norm.
# ---------------------------------------------------------------------------

def test_P7_non_expansive():
    rng = _rng(71)
    dk, dv, L = 8, 5, 64
    ks = rng.standard_normal((L, dk)) * np.exp(rng.uniform(np.log(0.1), np.log(30.0), (L, 1)))
    vs = rng.standard_normal((L, dv))
    betas = rng.uniform(0.0, 10.0, L)
    Sa = rng.standard_normal((1, 1, dk, dv))
    Sb = rng.standard_normal((1, 1, dk, dv))
    prev = np.linalg.norm(Sa[0, 0] - Sb[0, 0], 2)
    for t in range(L):
        args = (np.zeros((1, 1, dk)), ks[t][None, None], vs[t][None, None], np.array([[betas[t]]]))
        _, Sa = oracle.step(*args, Sa)
        _, Sb = oracle.step(*args, Sb)
        cur = np.linalg.norm(Sa[0, 0] - Sb[0, 0], 2)
        assert cur <= prev * (1 + 1e-12) + 1e-14
        prev = cur


# ---------------------------------------------------------------------------
# P9: scalar case d = 1 has the textbook linear-ODE solution
#   s_t = e^{-beta k^2} s_{t-1} + (1 - e^{-beta k^2}) v / k,   o_t = q s_t
# ---------------------------------------------------------------------------

def test_P9_scalar_closed_form():
    rng = _rng(91)
    L = 40
    k = rng.uniform(0.1, 5.0, L) * rng.choice([-1, 1], L)
    v = rng.standard_normal(L)
    q = rng.standard_normal(L)
    beta = rng.uniform(0.0, 3.0, L)
    o, sf = oracle.forward(q.reshape(1, L, 1, 1), k.reshape(1, L, 1, 1), v.reshape(1, L, 1, 1),
                           beta.reshape(1, L, 1), np.full((1, 1, 1, 1), 0.3))
    s = 0.3
    for t in range(L):
        e = math.exp(-beta[t] * k[t] ** 2)
        s = e * s + (1.0 - e) * v[t] / k[t]
        assert abs(o[0, t, 0, 0] - q[t] * s) <= 1e-14 * max(1.0, abs(q[t] * s))
    assert abs(sf[0, 0, 0, 0] - s) <= 1e-14 * max(1.0, abs(s))


# ---------------------------------------------------------------------------
# P10: split / resume and step-by-step equivalence; threading and layout.
# ---------------------------------------------------------------------------

def _rand_inputs(seed, B, L, H, dk, dv):
    rng = _rng(seed)
    return (rng.standard_normal((B, L, H, dk)), rng.standard_normal((B, L, H, dk)),
            rng.standard_normal((B, L, H, dv)), rng.uniform(0, 1, (B, L, H)),
            rng.standard_normal((B, H, dk, dv)))


def test_P10_split_resume_and_steps():
    q, k, v, beta, s0 = _rand_inputs(101, 2, 30, 2, 4, 3)
    o, sf = oracle.forward(q, k, v, beta, s0)
    o1, s1 = oracle.forward(q[:, :13], k[:, :13], v[:, :13], beta[:, :13], s0)
    o2, s2 = oracle.forward(q[:, 13:], k[:, 13:], v[:, 13:], beta[:, 13:], s1)
    assert np.array_equal(np.concatenate([o1, o2], axis=1), o)
    assert np.array_equal(s2, sf)
    st = s0.copy()
    for t in range(30):
        ot, st = oracle.step(q[:, t], k[:, t], v[:, t], beta[:, t], st)
        assert np.array_equal(ot, o[:, t])
    assert np.array_equal(st, sf)


def test_forward_threads_and_layout():
    q, k, v, beta, s0 = _rand_inputs(111, 3, 17, 5, 6, 2)
    o1, s1 = oracle.forward(q, k, v, beta, s0, nthreads=1)
    o8, s8 = oracle.forward(q, k, v, beta, s0, nthreads=8)
    assert np.array_equal(o1, o8) and np.array_equal(s1, s8)
    # every (b, h) slice run on its own gives the same numbers
    for b in range(3):
        for h in range(5):
            ob, sb = oracle.forward(q[b:b + 1, :, h:h + 1], k[b:b + 1, :, h:h + 1],
                                    v[b:b + 1, :, h:h + 1], beta[b:b + 1, :, h:h + 1],
                                    s0[b:b + 1, h:h + 1])
            assert np.array_equal(ob[0, :, 0], o1[b, :, h])
            assert np.array_equal(sb[0, 0], s1[b, h])


def test_zero_initial_state_and_degenerate_tokens():
    q, k, v, beta, _ = _rand_inputs(121, 1, 9, 1, 3, 3)
    o_none, s_none = oracle.forward(q, k, v, beta, None)
    o_zero, s_zero = oracle.forward(q, k, v, beta, np.zeros((1, 1, 3, 3)))
    assert np.array_equal(o_none, o_zero) and np.array_equal(s_none, s_zero)
    # beta = 0 and k = 0 are identity steps; the readout then uses S_{t-1}
    rng = _rng(122)
    S0 = rng.standard_normal((1, 1, 3, 3))
    qq = rng.standard_normal((1, 1, 3))
    for kk, bb in [(rng.standard_normal((1, 1, 3)), 0.0), (np.zeros((1, 1, 3)), 0.8)]:
        o, S1 = oracle.step(qq, kk, rng.standard_normal((1, 1, 3)), np.array([[bb]]), S0)
        assert np.array_equal(S1, S0)
        assert np.allclose(o[0, 0], S0[0, 0].T @ qq[0, 0], rtol=0, atol=1e-15)


def test_empty_sequence():
    q, k, v, beta, s0 = _rand_inputs(131, 2, 0, 3, 4, 4)
    o, sf = oracle.forward(q, k, v, beta, s0)
    assert o.shape == (2, 0, 3, 4)
    assert np.array_equal(sf, s0)


# ---------------------------------------------------------------------------
# P11: the Euler (delta-rule) update, the baseline the pages compare against
# (Problem statement; Key Contributions 1: the delta rule is one explicit Euler
# step of the same ODE).  A rank-1 update is fixed by what it does along k and
# on the complement of k, so these pins determine the Euler step completely:
#   k^T S_t - v^T = (1 - beta lambda) (k^T S_{t-1} - v^T),   u^T S_t = u^T S_{t-1} (u _|_ k).
# At beta*lambda = 1 the key direction is overwritten by v; at beta*lambda = 3
# the Euler step expands the error by 2 where the exact flow contracts it by e^-3.
# ---------------------------------------------------------------------------

def _one_step(S0, k, v, beta, rule):
    dk, dv = S0.shape
    _, S1 = oracle.step(np.zeros((1, 1, dk)), k[None, None], v[None, None],
                        np.array([[beta]]), S0[None, None], rule=rule)
    return S1[0, 0]


def test_P11_euler_coefficient_is_beta():
    rng = _rng(151)
    k = rng.standard_normal((9, 5)) * rng.uniform(0.1, 4.0, (9, 1))
    beta = rng.uniform(0.0, 5.0, 9)
    lam_e, a_e = oracle.coeff(k, beta, rule="euler")
    lam_x, a_x = oracle.coeff(k, beta)
    assert np.array_equal(a_e, beta)
    assert np.array_equal(lam_e, lam_x)
    assert not np.allclose(a_e, a_x)


def test_P11_euler_projection_invariants():
    rng = _rng(152)
    dk, dv = 7, 5
    for trial in range(20):
        S0 = rng.standard_normal((dk, dv))
        k = rng.uniform(0.2, 3.0) * rng.standard_normal(dk)
        v = rng.standard_normal(dv)
        lam = float(k @ k)
        # beta*lambda spread over (0, 1), around 1 and the expanding range up to 3
        beta = rng.uniform(0.0, 3.0) / lam
        S1 = _one_step(S0, k, v, beta, "euler")
        lhs = k @ S1 - v
        rhs = (1.0 - beta * lam) * (k @ S0 - v)
        tol = 1e-12 * max(1.0, np.abs(k @ S0).max(), np.abs(v).max())
        assert np.abs(lhs - rhs).max() <= tol
        u = rng.standard_normal(dk)
        u -= (u @ k) / (k @ k) * k
        assert np.abs(u @ S1 - u @ S0).max() <= 1e-12 * max(1.0, np.abs(u @ S0).max())


def test_P11_euler_unit_step_overwrites_and_large_step_expands():
    rng = _rng(153)
    dk, dv = 6, 4
    S0 = rng.standard_normal((dk, dv))
    k = rng.standard_normal(dk)
    v = rng.standard_normal(dv)
    lam = float(k @ k)
    err0 = k @ S0 - v
    S1 = _one_step(S0, k, v, 1.0 / lam, "euler")
    assert np.abs(k @ S1 - v).max() <= 1e-12 * max(1.0, np.abs(v).max(), np.abs(err0).max())
    S3 = _one_step(S0, k, v, 3.0 / lam, "euler")
    X3 = _one_step(S0, k, v, 3.0 / lam, "exact")
    assert np.allclose(k @ S3 - v, -2.0 * err0, rtol=1e-12, atol=1e-12)
    assert np.allclose(k @ X3 - v, math.exp(-3.0) * err0, rtol=1e-12, atol=1e-12)


def test_P11_euler_orthonormal_keys_store_values():
    """Associative memory with orthonormal keys and beta = 1: each Euler write
    stores v_t under k_t exactly and leaves the other keys' slots alone, so
    S_L = S_0 projected off span(K) + sum_t k_t v_t^T (keys used once each)."""
    rng = _rng(154)
    dk, dv, L = 8, 3, 5
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm[:, :L].T                       # L orthonormal rows
    v = rng.standard_normal((L, dv))
    q = rng.standard_normal((L, dk))
    S0 = rng.standard_normal((dk, dv))
    o, sf = oracle.forward(q[None, :, None], keys[None, :, None], v[None, :, None],
                           np.ones((1, L, 1)), S0[None, None], rule="euler")
    P_perp = np.eye(dk) - keys.T @ keys
    want = P_perp @ S0 + keys.T @ v
    assert np.abs(sf[0, 0] - want).max() <= 1e-12
    for t in range(L):
        assert np.abs(keys[t] @ sf[0, 0] - v[t]).max() <= 1e-12
        # after token t: the first t+1 keys hold their values, the rest still hold S0
        St = np.eye(dk) @ S0 - keys[:t + 1].T @ (keys[:t + 1] @ S0) + keys[:t + 1].T @ v[:t + 1]
        assert np.abs(o[0, t, 0] - St.T @ q[t]).max() <= 1e-12


def test_P11_euler_forward_equals_euler_steps_and_limits():
    q, k, v, beta, s0 = _rand_inputs(155, 2, 21, 3, 5, 4)
    o, sf = oracle.forward(q, k, v, beta, s0, rule="euler")
    st = s0.copy()
    for t in range(21):
        ot, st = oracle.step(q[:, t], k[:, t], v[:, t], beta[:, t], st, rule="euler")
        assert np.array_equal(ot, o[:, t])
    assert np.array_equal(st, sf)
    # the two rules differ at O((beta lambda)^2) per token and agree as beta -> 0
    ox, _ = oracle.forward(q, k, v, beta, s0)
    assert np.abs(ox - o).max() > 1e-3
    prev = None
    for scale in [1e-2, 1e-3, 1e-4]:
        oe, _ = oracle.forward(q, k, v, beta * scale, s0, rule="euler")
        ox, _ = oracle.forward(q, k, v, beta * scale, s0)
        d = np.abs(oe - ox).max()
        if prev is not None:
            # one decade less beta, two decades less gap: second order
            assert 0.01 / 1.5 <= d / prev <= 0.01 * 1.5
        prev = d


def test_rule_argument_is_checked():
    with pytest.raises(ValueError):
        oracle.coeff(np.ones((1, 2)), np.ones(1), rule="rk4")


# ---------------------------------------------------------------------------
# Packed variable-length batches: each sequence is an independent run.
# ---------------------------------------------------------------------------

def test_varlen_equal_lengths_is_the_dense_batch():
    q, k, v, beta, s0 = _rand_inputs(161, 3, 11, 2, 4, 3)
    o, sf = oracle.forward(q, k, v, beta, s0)
    cu = np.arange(4) * 11
    ov, sv = oracle.forward_varlen(q.reshape(33, 2, 4), k.reshape(33, 2, 4), v.reshape(33, 2, 3),
                                   beta.reshape(33, 2), cu, s0)
    assert np.array_equal(ov, o.reshape(33, 2, 3)) and np.array_equal(sv, sf)


def test_varlen_sequences_are_independent_and_empty_ones_keep_state():
    rng = _rng(162)
    lengths = [5, 0, 9, 1]
    T, H, dk, dv = 2 + sum(lengths) + 3, 2, 3, 2
    cu = 2 + np.concatenate([[0], np.cumsum(lengths)])
    q, k = rng.standard_normal((T, H, dk)), rng.standard_normal((T, H, dk))
    v, beta = rng.standard_normal((T, H, dv)), rng.uniform(0, 1, (T, H))
    s0 = rng.standard_normal((4, H, dk, dv))
    o, sf = oracle.forward_varlen(q, k, v, beta, cu, s0)
    assert np.array_equal(sf[1], s0[1])                      # empty sequence
    assert not o[:2].any() and not o[-3:].any()              # tokens outside every sequence
    k2 = k.copy()
    k2[cu[2]:cu[3]] += 1.0                                   # perturb sequence 2 only
    o2, sf2 = oracle.forward_varlen(q, k2, v, beta, cu, s0)
    for i in (0, 1, 3):
        assert np.array_equal(o2[cu[i]:cu[i + 1]], o[cu[i]:cu[i + 1]]) and np.array_equal(sf2[i], sf[i])
    assert not np.array_equal(sf2[2], sf[2])


# ---------------------------------------------------------------------------
# P12: the backward pass against central finite differences of the forward
# pass (the pages give no gradient; the gradient of a scalar loss
# L = sum(o * W) + sum(S_L * Wf) is fixed by the forward pass alone).
# ---------------------------------------------------------------------------

def _fd_inputs(seed, B, L, H, dk, dv, regime):
    rng = _rng(seed)
    q = rng.standard_normal((B, L, H, dk))
    k = rng.standard_normal((B, L, H, dk))
    v = rng.standard_normal((B, L, H, dv))
    beta = rng.uniform(0.1, 1.0, (B, L, H))
    if regime == "stiff":      # beta * lambda up to ~100: the contraction saturates
        k *= rng.uniform(1.5, 4.0, (B, L, H, 1))
        beta = rng.uniform(0.5, 3.0, (B, L, H))
    elif regime == "small":    # beta * lambda ~ 1e-5: the series branch of the lambda derivative
        beta = rng.uniform(1e-6, 3e-6, (B, L, H))
    s0 = rng.standard_normal((B, H, dk, dv))
    W = rng.standard_normal((B, L, H, dv))
    Wf = rng.standard_normal((B, H, dk, dv))
    return q, k, v, beta, s0, W, Wf


def _fd_check(inputs, rule, sample=None, seed=0):
    q, k, v, beta, s0, W, Wf = inputs
    args = [q, k, v, beta, s0]
    grads = oracle.backward(q, k, v, beta, s0, W, Wf, nthreads=1, rule=rule)
    grads = list(grads[:4]) + [grads[4]]

    def loss(a):
        o, sf = oracle.forward(*a, nthreads=1, rule=rule)
        return float((o * W).sum() + (sf * Wf).sum())

    # rounding floor of a central difference: a few ulps of the loss over 2h
    floor = 64 * np.finfo(float).eps * max(1.0, abs(loss(args))) / 1e-5
    rng = _rng(seed)
    for which, (x, g) in enumerate(zip(args, grads)):
        idx = list(np.ndindex(x.shape))
        if sample is not None and len(idx) > sample:
            idx = [idx[i] for i in rng.choice(len(idx), sample, replace=False)]
        fd = []
        for ix in idx:
            h = 1e-5 * max(1.0, abs(x[ix]))
            a_p = [a.copy() for a in args]
            a_m = [a.copy() for a in args]
            a_p[which][ix] += h
            a_m[which][ix] -= h
            fd.append((loss(a_p) - loss(a_m)) / (2 * h))
        fd = np.array(fd)
        got = np.array([g[ix] for ix in idx])
        scale = max(np.abs(fd).max(), 1e-12)
        assert np.abs(fd - got).max() <= 2e-6 * scale + floor, (which, np.abs(fd - got).max(), scale)


@pytest.mark.parametrize("rule", ["exact", "euler"])
@pytest.mark.parametrize("regime", ["moderate", "stiff", "small"])
def test_P12_backward_matches_finite_differences(rule, regime):
    if rule == "euler" and regime == "stiff":
        pytest.skip("the Euler step diverges for beta*lambda > 2; nothing to differentiate")
    _fd_check(_fd_inputs(171, 2, 5, 2, 3, 2, regime), rule)


def test_P12_backward_across_recompute_segments():
    # 150 tokens: three 64-token recompute segments of the oracle's reverse sweep
    _fd_check(_fd_inputs(172, 1, 150, 1, 2, 2, "moderate"), "exact", sample=12, seed=5)


def test_P12_backward_without_final_state_gradient_and_state():
    q, k, v, beta, s0, W, _ = _fd_inputs(173, 1, 4, 1, 3, 3, "moderate")
    g0 = oracle.backward(q, k, v, beta, None, W, None, nthreads=1)
    g1 = oracle.backward(q, k, v, beta, np.zeros_like(s0), W, np.zeros_like(s0), nthreads=1)
    for a, b in zip(g0, g1):
        assert np.array_equal(a, b)
    # o_t is linear in q_t: dq_t = S_t do_t exactly
    o, _ = oracle.forward(q, k, v, beta, None)
    gq = g0[0]
    assert np.allclose((gq * q).sum(), (o * W).sum(), rtol=1e-12)


@pytest.mark.parametrize("x", [0.0, 1e-300, 1e-12, 1e-6, 1e-3, 0.02, 0.049, 0.051, 0.3, 1.0, 7.0, 40.0, 700.0])
@pytest.mark.parametrize("lam", [1e-3, 1.0, 37.0])
def test_P12_alpha_derivatives_against_60_digit_differentiation(x, lam):
    """d alpha / d beta and d alpha / d lambda of (1 - exp(-beta lambda)) / lambda,
    differentiated by mpmath at 60 digits, across both branches of the
    oracle's evaluation (series below beta*lambda = 0.05)."""
    beta = x / lam
    b, l = mpmath.mpf(beta), mpmath.mpf(lam)
    f_b = lambda bb: (1 - mpmath.exp(-bb * l)) / l if bb * l != 0 else bb
    f_l = lambda ll: (1 - mpmath.exp(-b * ll)) / ll
    want_b = mpmath.diff(f_b, b) if x > 0 else mpmath.mpf(1)
    want_l = mpmath.diff(f_l, l) if x > 0 else -b * b / 2
    got_b, got_l = oracle.alpha_grad(beta, lam)
    assert abs(got_b - float(want_b)) <= 4e-15 * max(1.0, abs(float(want_b)))
    assert abs(got_l - float(want_l)) <= 1e-13 * abs(float(want_l)) + 1e-300
    assert oracle.alpha_grad(beta, lam, rule="euler") == (1.0, 0.0)
