"""Offline factor solve on the GPU (glowq_solve_factors) against the fp64 oracle
(oracle.solve.core_factors with the Cholesky factor of Sigma_x as the square root, and
oracle.solve.randomized_svd for the singular values), the same test matrix on both sides.

Bar: both sides run the same fp64 algorithm up to the orthonormalisation method (two Cholesky-QR
passes here, Householder QR in the oracle) and the left factor of the QR reduction, so the lifted
products A B agree to 1e-8 relative Frobenius norm and the singular values to 1e-9 relative
where the spectrum has a gap at r; an exactly rank-r0 whitened error (r0 <= r) is reproduced:
A B = E_cat to 1e-9."""
import numpy as np
import pytest
import torch

from gpu_util import glowq
from oracle import solve as S

pytestmark = pytest.mark.gpu


def covariance(d, alpha, seed):
    rng = np.random.default_rng(seed)
    Q, R = np.linalg.qr(rng.standard_normal((d, d)))
    Q = Q * np.sign(np.diag(R))
    lam = np.arange(1, d + 1, dtype=np.float64) ** (-alpha)
    lam *= d / lam.sum()
    return (Q * lam) @ Q.T


def run(g, E, Sigma, r, p, q, seed):
    d = E.shape[1]
    k = min(r + p, d)
    omega = np.random.default_rng(seed).standard_normal((d, k))
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    A, B, Sv = g.solve_factors(t(E), t(Sigma), t(omega), r, q)
    return A.cpu().numpy(), B.cpu().numpy(), Sv.cpu().numpy()


def oracle(E, Sigma, r, p, q, seed):
    L = np.linalg.cholesky(Sigma)
    A_list, B = S.core_factors([E], L, np.linalg.inv(L), r, p=p, q=q, seed=seed)
    M = S.qr_core(E, L)[1]
    _, s, _ = S.randomized_svd(M, r, p, q, np.random.default_rng(seed))
    return np.vstack(A_list) @ B, s[:r]


def rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.mark.parametrize("m,d,r0,r,p,q", [(96, 128, 6, 8, 8, 1), (40, 200, 3, 4, 4, 0), (300, 256, 16, 16, 16, 2)])
def test_exact_rank_error_is_reproduced(m, d, r0, r, p, q):
    g = glowq()
    rng = np.random.default_rng(m + d)
    Sigma = covariance(d, 1.19, d)
    L = np.linalg.cholesky(Sigma)
    U0, _ = np.linalg.qr(rng.standard_normal((m, r0)))
    V0, _ = np.linalg.qr(rng.standard_normal((d, r0)))
    s0 = np.linspace(3.0, 1.0, r0)
    E = (U0 * s0) @ V0.T @ np.linalg.inv(L)  # whitened error E L has rank r0 and singular values s0
    A, B, Sv = run(g, E, Sigma, r, p, q, seed=3)
    assert rel(A @ B, E) <= 1e-9
    assert np.max(np.abs(Sv[:r0] - s0)) <= 1e-9 * s0[0]
    P_ref, _ = oracle(E, Sigma, r, p, q, seed=3)
    assert rel(A @ B, P_ref) <= 1e-9


# the last shape has GEMMs with K split over up to 16 ranges and ten column blocks in the lift
@pytest.mark.parametrize("m,d,r,p,q", [(200, 256, 16, 8, 2), (96, 128, 8, 24, 1), (160, 192, 32, 32, 3),
                                       (2048, 640, 16, 8, 1)])
def test_matches_oracle_with_gap(m, d, r, p, q):
    g = glowq()
    rng = np.random.default_rng(7 * m + d)
    Sigma = covariance(d, 0.77, d + 1)
    # a dominant rank-r part plus small full-rank noise: a clear gap at r
    E = rng.standard_normal((m, r)) @ rng.standard_normal((r, d)) + 1e-3 * rng.standard_normal((m, d))
    A, B, Sv = run(g, E, Sigma, r, p, q, seed=11)
    P_ref, s_ref = oracle(E, Sigma, r, p, q, seed=11)
    assert rel(A @ B, P_ref) <= 1e-8
    assert np.max(np.abs(Sv - s_ref)) <= 1e-9 * s_ref[0]


@pytest.mark.parametrize("d,n_zero,m,r,p,q", [(384, 20, 200, 16, 16, 2), (256, 3, 96, 8, 8, 1), (160, 96, 64, 4, 4, 1)])
def test_singular_sigma_pseudo_inverse_lift(d, n_zero, m, r, p, q):
    """Singular Sigma_x (n_zero zero eigenvalues, null directions spread over several Cholesky blocks)
    and an error with a part in its null space, which whitening cannot see: the solve succeeds,
    B's rows lie in range(Sigma_x) (pseudo-inverse lift), and A B equals the oracle's
    S_r^{1/2} V_r^T Sigma_x^{+1/2} product -- here the error's part inside the range, whose
    whitened form has rank r0 <= r (so the randomized solve is exact)."""
    g = glowq()
    rng = np.random.default_rng(d + n_zero)
    Q, R = np.linalg.qr(rng.standard_normal((d, d)))
    Q = Q * np.sign(np.diag(R))
    lam = np.arange(1, d + 1, dtype=np.float64) ** (-1.19)
    lam *= d / lam.sum()
    lam[d - n_zero:] = 0.0
    Sigma = (Q * lam) @ Q.T
    Sigma = 0.5 * (Sigma + Sigma.T)
    Nq = Q[:, d - n_zero:]
    P = np.eye(d) - Nq @ Nq.T
    r0 = r - 2
    U0, _ = np.linalg.qr(rng.standard_normal((m, r0)))
    V0, _ = np.linalg.qr(P @ rng.standard_normal((d, r0)))
    E_in = (U0 * np.linspace(2.0, 0.5, r0)) @ V0.T          # rows in range(Sigma_x)
    E = E_in + rng.standard_normal((m, n_zero)) @ Nq.T       # plus a null-space part
    A, B, Sv = run(g, E, Sigma, r, p, q, seed=5)
    # rows of B with nonzero singular values lie in range(Sigma_x); the last r - r0 rows belong to
    # numerically zero singular values (S^{-1/2} amplifies rounding there, and A's columns are ~0)
    assert np.linalg.norm(B[:r0] @ Nq) <= 1e-9 * np.linalg.norm(B[:r0])
    assert np.linalg.norm(A @ B @ Nq) <= 1e-9 * np.linalg.norm(A @ B)
    A_list, B_ref, s_ref = S.whitened_factors([E], S.sqrt_psd(Q, lam), S.pinv_sqrt_psd(Q, lam), r)
    P_ref = np.vstack(A_list) @ B_ref
    assert rel(P_ref, E_in) <= 1e-9                          # the oracle's product: E's range part
    assert rel(A @ B, P_ref) <= 1e-9
    assert np.max(np.abs(Sv[:r0] - s_ref[:r0])) <= 1e-9 * s_ref[0]


def test_too_many_null_directions_is_unsupported():
    g = glowq()
    d, m, r = 256, 32, 4
    rng = np.random.default_rng(3)
    Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    lam = np.ones(d)
    lam[:100] = 0.0
    Sigma = (Q * lam) @ Q.T
    with pytest.raises(g.GlowQError) as ei:
        run(g, rng.standard_normal((m, d)), 0.5 * (Sigma + Sigma.T), r, 4, 0, seed=1)
    assert ei.value.status == g.ERR_UNSUPPORTED


def test_not_positive_definite_is_reported():
    g = glowq()
    d, m, r = 64, 32, 4
    E = np.random.default_rng(1).standard_normal((m, d))
    Sigma = -np.eye(d)
    with pytest.raises(g.GlowQError) as ei:
        run(g, E, Sigma, r, 4, 0, seed=1)
    assert ei.value.status == g.ERR_RANGE


def test_deterministic():
    """Split-K partial products are added in range order: two solves give identical bits."""
    g = glowq()
    m, d, r, p, q = 2048, 640, 16, 8, 1
    rng = np.random.default_rng(5)
    Sigma = covariance(d, 1.19, 9)
    E = rng.standard_normal((m, r)) @ rng.standard_normal((r, d)) + 1e-3 * rng.standard_normal((m, d))
    A1, B1, S1 = run(g, E, Sigma, r, p, q, seed=2)
    A2, B2, S2 = run(g, E, Sigma, r, p, q, seed=2)
    assert np.array_equal(A1, A2) and np.array_equal(B1, B2) and np.array_equal(S1, S2)


# ------------------------------------------------------------------ restore score g_ec
def _ec_case(m, d, r, noise, seed):
    rng = np.random.default_rng(seed)
    Sigma = covariance(d, 0.77, d + 2)
    sv = np.linspace(3.0, 1.0, r)
    E = (rng.standard_normal((m, r)) * sv) @ rng.standard_normal((r, d)) + noise * rng.standard_normal((m, d))
    return E, Sigma


@pytest.mark.parametrize("m,d,r,p,q,noise", [(200, 256, 16, 8, 2, 2.0), (300, 384, 24, 16, 2, 3.0),
                                             (2048, 640, 16, 8, 1, 4.0)])
def test_ec_score_matches_oracle(m, d, r, p, q, noise):
    """g_ec on the GPU (glowq_ec_score fed with the solve's singular values) against the oracle:
    the energy equals ||M||_F^2 of the oracle's whitened core M = R_e L (the same terms summed in
    another order: 1e-11 relative), the captured energy equals the oracle's randomized SVD with
    the same test matrix (1e-9 relative), and the score lies at most at the exact best-rank-r
    share, oracle.solve.g_ec (Eckart-Young: no rank-r approximation captures more), within the
    randomized range finder's shortfall (g_ec 0.83-0.96 here, the gap at r small)."""
    g = glowq()
    E, Sigma = _ec_case(m, d, r, noise, 13 * m + d)
    _, _, Sv = run(g, E, Sigma, r, p, q, seed=11)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    out = g.ec_score(t(E), t(Sigma), t(Sv), r).cpu().numpy()
    M = S.qr_core(E, np.linalg.cholesky(Sigma))[1]
    _, s_ref = oracle(E, Sigma, r, p, q, seed=11)
    energy = float(np.sum(M ** 2))
    captured = float(np.sum(s_ref[:r] ** 2))
    assert abs(out[0] - energy) <= 1e-11 * energy
    assert abs(out[1] - captured) <= 1e-9 * captured
    assert abs(out[2] - captured / energy) <= 1e-9
    exact = S.g_ec(M, r)
    assert -1e-12 <= exact - out[2] <= 1e-3


def test_ec_score_special_cases():
    """An error whose whitened form has rank r0 <= r scores 1; r = 0 (no singular values) and an
    all-zero error score 0; two calls give identical bits (fixed-order sums)."""
    g = glowq()
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    m, d, r0, r = 96, 128, 6, 8
    rng = np.random.default_rng(21)
    Sigma = covariance(d, 1.19, d)
    L = np.linalg.cholesky(Sigma)
    U0, _ = np.linalg.qr(rng.standard_normal((m, r0)))
    V0, _ = np.linalg.qr(rng.standard_normal((d, r0)))
    s0 = np.linspace(3.0, 1.0, r0)
    E = (U0 * s0) @ V0.T @ np.linalg.inv(L)
    _, _, Sv = run(g, E, Sigma, r, 8, 1, seed=3)
    out = g.ec_score(t(E), t(Sigma), t(Sv), r).cpu().numpy()
    assert abs(out[0] - np.sum(s0 ** 2)) <= 1e-10 * np.sum(s0 ** 2)
    assert abs(out[2] - 1.0) <= 1e-9
    none = g.ec_score(t(E), t(Sigma), None, 0).cpu().numpy()
    assert none[1] == 0.0 and none[2] == 0.0 and abs(none[0] - out[0]) <= 1e-12 * out[0]
    zero = g.ec_score(t(np.zeros((m, d))), t(Sigma), t(np.zeros(r)), r).cpu().numpy()
    assert np.array_equal(zero, np.zeros(3))
    E2, Sigma2 = _ec_case(300, 384, 24, 3.0, 5)
    a = g.ec_score(t(E2), t(Sigma2), t(np.linspace(2.0, 1.0, 24)), 24).cpu().numpy()
    b = g.ec_score(t(E2), t(Sigma2), t(np.linspace(2.0, 1.0, 24)), 24).cpu().numpy()
    assert np.array_equal(a, b)
