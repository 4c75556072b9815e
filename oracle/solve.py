"""fp64 CPU oracle of GlowQ's offline factor solve and restore scores (TEST INFRASTRUCTURE
ONLY; imported by tests, the smoke check and the benchmark's CPU-baseline leg, never by
the HIP library).

The inference path consumes (A_i, B_shared); this module produces exact ones for the tiny
workload and states the optimisation the pages define, so that the inference oracle can
be pinned end to end (an exactly rank-r error is reproduced to rounding):

  * key design 1 (GlowQ paper note) and the notation table (Table 6, arXiv page):
    stack the errors of an input-sharing group row-wise, E_cat = [E_1; ...; E_m]
    (m modules, sum_i O_i rows, d columns), and fit one right factor:
    min ||E_cat - A B||_F^2; the optimum B spans the top-r right singular subspace
    (Eckart-Young-Mirsky); per-module B_i add no expressivity.
  * key design 2: the usage-weighted risk E||M x||^2 equals ||M Sigma_x^{1/2}||_F^2, so the
    covariance-aligned fit is min ||(E_cat - A B) Sigma_x^{1/2}||_F^2, solved by the rank-r
    SVD of the whitened error E_cat Sigma_x^{1/2}; isotropic Sigma_x gives the plain
    stacked SVD.
  * key design 3: thin QR E_cat = Q_e R_e reduces the tall problem to the core
    M = R_e Sigma_x^{1/2} (Frobenius norm is invariant under the left orthogonal
    factor); a randomized SVD with oversampling p and q power iterations extracts the
    dominant subspace; balanced factors A = U_r S_r^{1/2}, B = S_r^{1/2} V_r^T are lifted
    back to the original variables (pseudo-inverse square root when Sigma_x is singular).
  * Sigma_x is the uncentred second moment of the calibration inputs, X^T X / N (the
    identity of key design 2 needs E[x x^T]).
  * key design 4: restore scores g_ec(u) = sum_{j<=r} sigma_j(M_u)^2 / ||M_u||_F^2 and
    g_ner(u) = ||E_u||_F^2 / ||W_u||_F^2; the top-k units are restored, layer order
    breaking ties (the pages fall back to layer order when the signal is weak).
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np


def second_moment(X) -> np.ndarray:
    """Input second moment Sigma_x = E[x x^T] over calibration tokens: X is [N][d] (one token
    per row), Sigma_x = X^T X / N in fp64.  key design 2 (GlowQ paper note): the usage-weighted
    risk E||M x||^2 = ||M Sigma_x^{1/2}||_F^2 holds for this uncentred moment; Figure 2 of the
    arXiv page streams calibration samples and takes the empirical input covariance."""
    X = np.asarray(X, dtype=np.float64)
    return (X.T @ X) / X.shape[0]


def stack_errors(E_list: Sequence[np.ndarray]) -> np.ndarray:
    return np.vstack([np.asarray(e, dtype=np.float64) for e in E_list])


def split_rows(A: np.ndarray, n_outs: Sequence[int]) -> List[np.ndarray]:
    out, o = [], 0
    for n in n_outs:
        out.append(A[o:o + n])
        o += n
    assert o == A.shape[0]
    return out


def sqrt_psd(Q: np.ndarray, lam: np.ndarray) -> np.ndarray:
    """Symmetric square root Q diag(sqrt(lam)) Q^T of Sigma = Q diag(lam) Q^T."""
    lam = np.asarray(lam, dtype=np.float64)
    return (Q * np.sqrt(np.clip(lam, 0, None))) @ Q.T


def pinv_sqrt_psd(Q: np.ndarray, lam: np.ndarray, rtol: float = 1e-12) -> np.ndarray:
    """Pseudo-inverse of the symmetric square root (zero on the null space)."""
    lam = np.asarray(lam, dtype=np.float64)
    cut = rtol * float(lam.max())
    inv = np.where(lam > cut, 1.0 / np.sqrt(np.where(lam > cut, lam, 1.0)), 0.0)
    return (Q * inv) @ Q.T


def balanced_factors(U: np.ndarray, S: np.ndarray, Vt: np.ndarray, r: int
                     ) -> Tuple[np.ndarray, np.ndarray]:
    """A = U_r S_r^{1/2}, B = S_r^{1/2} V_r^T."""
    sq = np.sqrt(S[:r])
    return U[:, :r] * sq, sq[:, None] * Vt[:r]


def whitened_factors(E_list: Sequence[np.ndarray], S_half: np.ndarray, S_half_lift: np.ndarray,
                     r: int) -> Tuple[List[np.ndarray], np.ndarray, np.ndarray]:
    """Covariance-aligned shared factors by a full SVD of E_cat S_half.

    S_half is a square root of Sigma_x (symmetric, or a Cholesky factor L with
    Sigma = L L^T); S_half_lift maps back to the original variables (its (pseudo-)inverse).
    Returns (A_i list, B, singular values of the whitened error)."""
    n_outs = [np.asarray(e).shape[0] for e in E_list]
    E_cat = stack_errors(E_list)
    Ew = E_cat @ S_half
    U, S, Vt = np.linalg.svd(Ew, full_matrices=False)
    A, Bw = balanced_factors(U, S, Vt, r)
    B = Bw @ S_half_lift
    return split_rows(A, n_outs), B, S


def qr_core(E_cat: np.ndarray, S_half: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Thin QR E_cat = Q_e R_e and the core M = R_e S_half."""
    Qe, Re = np.linalg.qr(np.asarray(E_cat, dtype=np.float64), mode="reduced")
    return Qe, Re @ S_half


def randomized_svd(M: np.ndarray, r: int, p: int, q: int, rng: np.random.Generator
                   ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Randomized range finder with p oversampling columns and q power iterations, then an
    exact SVD of the small projected matrix (Halko, Martinsson and Tropp)."""
    n = M.shape[1]
    k = min(r + p, min(M.shape))
    Omega = rng.standard_normal((n, k))
    Y = M @ Omega
    Qy, _ = np.linalg.qr(Y)
    for _ in range(q):
        Z, _ = np.linalg.qr(M.T @ Qy)
        Qy, _ = np.linalg.qr(M @ Z)
    Bsmall = Qy.T @ M
    Ub, S, Vt = np.linalg.svd(Bsmall, full_matrices=False)
    return Qy @ Ub, S, Vt


def core_factors(E_list: Sequence[np.ndarray], S_half: np.ndarray, S_half_lift: np.ndarray, r: int,
                 p: Optional[int] = None, q: int = 0, seed: int = 0
                 ) -> Tuple[List[np.ndarray], np.ndarray]:
    """The QR-reduced solve: core M = R_e S_half, (randomized when p is given) SVD of M,
    balanced factors, left factor lifted by Q_e, right factor by S_half_lift."""
    n_outs = [np.asarray(e).shape[0] for e in E_list]
    E_cat = stack_errors(E_list)
    Qe, M = qr_core(E_cat, S_half)
    if p is None:
        U, S, Vt = np.linalg.svd(M, full_matrices=False)
    else:
        U, S, Vt = randomized_svd(M, r, p, q, np.random.default_rng(seed))
    A_core, Bw = balanced_factors(U, S, Vt, r)
    return split_rows(Qe @ A_core, n_outs), Bw @ S_half_lift


# ------------------------------------------------------------------ restore selection
def g_ec(M_u: np.ndarray, r: int) -> float:
    """Energy captured by the best rank r of the (whitened) core M_u."""
    s = np.linalg.svd(np.asarray(M_u, dtype=np.float64), compute_uv=False)
    tot = float(np.sum(s ** 2))
    return float(np.sum(s[:r] ** 2)) / tot if tot > 0 else 0.0


def g_ner(E_u: np.ndarray, W_u: np.ndarray) -> float:
    """Normalised error ratio ||E_u||_F^2 / ||W_u||_F^2."""
    w2 = float(np.sum(np.asarray(W_u, dtype=np.float64) ** 2))
    return float(np.sum(np.asarray(E_u, dtype=np.float64) ** 2)) / w2 if w2 > 0 else 0.0


def topk_restore(scores: Sequence[float], k: int) -> List[bool]:
    """Restore the k highest-scoring units; equal scores go to the lower unit index."""
    order = sorted(range(len(scores)), key=lambda u: (-float(scores[u]), u))
    chosen = set(order[:k])
    return [u in chosen for u in range(len(scores))]


def topk_restore_tol(scores: Sequence[float], k: int, rel_tol: float) -> List[bool]:
    """GlowQ-S selection with the layer-order fallback of key design 4 when the signal is weak:
    a unit's distance from the best score is measured in steps of rel_tol times the best score,
    key(u) = floor((max - score(u)) / (rel_tol * max)) in fp64; units with the same key count as
    equal, and among them the lower index (layer order) goes first.  When every score lies within
    one step of the best the choice is the first k units; rel_tol = 0 is the exact ranking
    (topk_restore)."""
    s = [float(v) for v in scores]
    mx = max(s) if s else 0.0
    if rel_tol > 0.0 and mx > 0.0:
        step = rel_tol * mx
        keys = [math.floor((mx - v) / step) for v in s]
        order = sorted(range(len(s)), key=lambda u: (keys[u], u))
    else:
        order = sorted(range(len(s)), key=lambda u: (-s[u], u))
    chosen = set(order[:k])
    return [u in chosen for u in range(len(s))]
