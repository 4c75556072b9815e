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
