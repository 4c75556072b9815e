"""Checks that pin the fp64 oracle to facts outside itself: exact rational arithmetic,
hand-worked fixtures, closed forms (Eckart-Young-Mirsky), special cases that reduce to a
textbook SVD, brute-force loops and invariants.

Each check takes the oracle as a namespace (``ref`` for the inference definitions,
``sol`` for the factor solve) so that ``test_oracle_mutations.py`` can hand it a copy
with a planted mistake and confirm that some check fails.
"""
from __future__ import annotations

import itertools
import math
import os
from fractions import Fraction
from types import SimpleNamespace

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def oracle_namespaces():
    from oracle import glowq_ref, solve
    ref = SimpleNamespace(**{k: getattr(glowq_ref, k) for k in dir(glowq_ref) if not k.startswith("__")})
    sol = SimpleNamespace(**{k: getattr(solve, k) for k in dir(solve) if not k.startswith("__")})
    return ref, sol


# ------------------------------------------------------------------ helpers (test side)
def pack_words(q: np.ndarray) -> np.ndarray:
    """uint values [O][K] -> int32 words, input 8w+j in bits 4j..4j+3 (python ints)."""
    O, K = q.shape
    out = np.zeros((O, K // 8), dtype=np.int64)
    for o in range(O):
        for w in range(K // 8):
            v = 0
            for j in range(8):
                v |= int(q[o, 8 * w + j]) << (4 * j)
            out[o, w] = v - (1 << 32) if v >= (1 << 31) else v
    return out.astype(np.int32)


def fp16_from_bits(h: int) -> np.float16:
    return np.array([h], dtype=np.uint16).view(np.float16)[0]


# ------------------------------------------------------------------ P1: dequantisation
S_SWEEP_BITS = [0x0001, 0x0003, 0x0200, 0x0400, 0x1F60, 0x2E66, 0x3800, 0x3C00, 0x3E00,
                0x4248, 0x63D0, 0x7800, 0x7BFF]


def check_dequant_exhaustive(ref):
    """Every q in 0..15, every z in -16..31 and a sweep of fp16 scales (subnormal, min
    normal, 1, max): the oracle's fp64 value equals the exact rational (q - z) * s and is
    exactly representable in fp32."""
    zs = list(range(-16, 32))
    rows = [(z, sb) for z in zs for sb in S_SWEEP_BITS]
    O, K = len(rows), 256
    q = np.zeros((O, K), dtype=np.int64)
    s = np.zeros((O, 2), dtype=np.float16)
    z = np.zeros((O, 2), dtype=np.float16)
    for o, (zz, sb) in enumerate(rows):
        for k in range(K):
            q[o, k] = (k + o) % 16
        s[o, 0] = fp16_from_bits(sb)
        s[o, 1] = fp16_from_bits(S_SWEEP_BITS[(S_SWEEP_BITS.index(sb) + 5) % len(S_SWEEP_BITS)])
        z[o, 0] = zz
        z[o, 1] = -zz + 7
    words = pack_words(q)
    W = ref.dequant(words, s, z, O, K)
    assert W.shape == (O, K) and W.dtype == np.float64
    for o in range(O):
        for k in range(K):
            g = k // 128
            exact = (Fraction(int(q[o, k])) - Fraction(float(z[o, g]))) * Fraction(float(s[o, g]))
            assert Fraction(float(W[o, k])) == exact, (o, k)
            assert float(np.float32(W[o, k])) == float(W[o, k]), (o, k)


def check_dequant_golden(ref):
    """Hand-worked rows of the canonical format (tests/golden/dequant_nibbles.txt)."""
    rows, expects = {}, {}
    with open(os.path.join(GOLDEN, "dequant_nibbles.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            tok = line.split()
            if tok[0] == "row":
                r = int(tok[1])
                sb = int(tok[2].split("=")[1], 16)
                zz = int(tok[3].split("=")[1])
                words = [int(tok[4].split("=")[1], 16)] + [int(t, 16) for t in tok[5:]]
                rows[r] = (sb, zz, words)
            elif tok[0] == "expect":
                r = int(tok[1])
                expects[r] = [(int(p.split(":")[0]), float(p.split(":")[1])) for p in tok[2:]]
    assert rows and set(rows) == set(expects)
    for r, (sb, zz, words) in rows.items():
        w = np.array([[v - (1 << 32) if v >= (1 << 31) else v for v in words]], dtype=np.int64).astype(np.int32)
        s = np.array([[fp16_from_bits(sb)]], dtype=np.float16)
        z = np.array([[zz]], dtype=np.float16)
        W = ref.dequant(w, s, z, 1, 128)
        listed = dict(expects[r])
        for k in range(128):
            want = listed.get(k, (0 - zz) * float(s[0, 0]))
            assert float(W[0, k]) == want, (r, k, float(W[0, k]), want)


# ------------------------------------------------------------------ tiny random problem
def tiny_problem(seed=0, T=3, d=256, n_outs=(24, 40, 16), r=5, z_range=(0, 16)):
    rng = np.random.default_rng(seed)
    G = d // 128
    qs, ss, zs, words = [], [], [], []
    for O in n_outs:
        q = rng.integers(0, 16, size=(O, d))
        s = (rng.uniform(0.002, 0.05, size=(O, G))).astype(np.float16)
        z = rng.integers(z_range[0], z_range[1], size=(O, G)).astype(np.float16)
        qs.append(q)
        ss.append(s)
        zs.append(z)
        words.append(pack_words(q))
    x = rng.standard_normal((T, d)).astype(np.float16)
    b = (rng.standard_normal((r, d)) / math.sqrt(d)).astype(np.float16)
    a = [(rng.standard_normal((O, r)) * 0.05).astype(np.float16) for O in n_outs]
    return SimpleNamespace(x=x, b=b, a=a, q=qs, s=ss, z=zs, words=words, n_outs=list(n_outs), d=d,
                           T=T, r=r)


def _w_hats(ref, p):
    return [ref.dequant(w, s, z, O, p.d) for w, s, z, O in zip(p.words, p.s, p.z, p.n_outs)]


# ------------------------------------------------------------------ P3: restore off / r = 0
def check_restore_off(ref):
    p = tiny_problem(1)
    wh = _w_hats(ref, p)
    bf = ref.bruteforce_group(p.x, p.words, p.s, p.z, p.n_outs, p.d, None, p.a, restore=False)
    for restore, b in ((False, p.b), (True, None), (True, p.b[:0])):
        ys = ref.group_forward(p.x, wh, b, p.a, restore=restore)
        for y, w, yb in zip(ys, wh, bf):
            base = p.x.astype(np.float64) @ w.T
            assert np.array_equal(y, base)
            assert np.max(np.abs(y - yb)) <= 1e-15 * max(1.0, np.max(np.abs(yb)))


# ------------------------------------------------------------------ P4: associativity
def check_associativity_small_int(ref):
    """Small integers make every product and sum exact in fp64, so
    X W_hat^T + (X B^T) A^T must equal X (W_hat + A B)^T bit for bit; unequal
    dimensions expose a transposed operand, a wrong sign or a dropped term."""
    rng = np.random.default_rng(7)
    T, d, r = 5, 256, 3
    n_outs = [16, 32]
    words, ss, zs, qs = [], [], [], []
    for O in n_outs:
        q = rng.integers(0, 16, size=(O, d))
        qs.append(q)
        words.append(pack_words(q))
        ss.append(np.ones((O, 2), dtype=np.float16))
        zs.append(rng.integers(0, 16, size=(O, 2)).astype(np.float16))
    x = rng.integers(-3, 4, size=(T, d)).astype(np.float16)
    b = rng.integers(-2, 3, size=(r, d)).astype(np.float16)
    a = [rng.integers(-2, 3, size=(O, r)).astype(np.float16) for O in n_outs]
    wh = [ref.dequant(w, s, z, O, d) for w, s, z, O in zip(words, ss, zs, n_outs)]
    ys = ref.group_forward(x, wh, b, a, restore=True)
    for i, O in enumerate(n_outs):
        g = np.arange(d) // 128
        w_int = qs[i] - zs[i].astype(np.int64)[:, g]
        merged = w_int + a[i].astype(np.int64) @ b.astype(np.int64)
        want = x.astype(np.int64) @ merged.T
        assert ys[i].shape == (T, O)
        assert np.array_equal(ys[i], want.astype(np.float64)), i
    # solo = group of one with its private B; layerwise = one solo per module
    ysolo = ref.solo_forward(x, wh[1], b, a[1], restore=True)
    assert np.array_equal(ysolo, ys[1])
    ylw = ref.layerwise_forward(x, wh, [b, b], a, restore=True)
    for u, v in zip(ylw, ys):
        assert np.array_equal(u, v)


# ------------------------------------------------------------------ P11: brute force
def check_bruteforce(ref):
    for seed, kw in ((2, {}), (3, dict(T=2, d=128, n_outs=(8,), r=2, z_range=(-5, 20)))):
        p = tiny_problem(seed, **kw)
        wh = _w_hats(ref, p)
        ys = ref.group_forward(p.x, wh, p.b, p.a, restore=True)
        bf = ref.bruteforce_group(p.x, p.words, p.s, p.z, p.n_outs, p.d, p.b, p.a, restore=True)
        for y, yb in zip(ys, bf):
            scale = float(np.max(np.abs(yb)))
            assert np.max(np.abs(y - yb)) <= 1e-13 * scale, np.max(np.abs(y - yb)) / scale


# ------------------------------------------------------------------ P12: row independence
def check_row_independence(ref):
    p = tiny_problem(4, T=6)
    wh = _w_hats(ref, p)
    y_all = ref.group_forward(p.x, wh, p.b, p.a, restore=True)
    y_1 = ref.group_forward(p.x[:2], wh, p.b, p.a, restore=True)
    y_2 = ref.group_forward(p.x[2:], wh, p.b, p.a, restore=True)
    for ya, y1, y2 in zip(y_all, y_1, y_2):
        scale = float(np.max(np.abs(ya)))
        assert np.max(np.abs(ya - np.vstack([y1, y2]))) <= 1e-14 * scale


# ------------------------------------------------------------------ mask path
def check_path_mask(ref):
    """A layer outside the restore set returns the quantised product alone; a restored
    layer gets the correction; units run in the stated order."""
    units = {}
    for l in range(3):
        us = []
        for u, n_outs in enumerate(((24, 16, 16), (32,))):
            p = tiny_problem(10 + 3 * l + u, n_outs=n_outs)
            us.append(SimpleNamespace(x=p.x, b=p.b, a=p.a, weights=[
                SimpleNamespace(q_packed=w, s=s, z=z, n_out=O, k_in=p.d)
                for w, s, z, O in zip(p.words, p.s, p.z, p.n_outs)], p=p))
        units[l] = us
    mask = [True, False, True]
    out = ref.path_forward(units, mask)
    for l, us in units.items():
        for ui, u in enumerate(us):
            wh = _w_hats(ref, u.p)
            for i, w in enumerate(wh):
                base = u.x.astype(np.float64) @ w.T
                y = out[l][ui][i]
                if mask[l]:
                    corr = (u.x.astype(np.float64) @ u.b.astype(np.float64).T) @ u.a[i].astype(np.float64).T
                    assert np.max(np.abs(y - base - corr)) <= 1e-14 * np.max(np.abs(y))
                    assert np.max(np.abs(corr)) > 0
                else:
                    assert np.array_equal(y, base)


# ------------------------------------------------------------------ solver pins
def _cov(d, alpha, seed, n_zero=0):
    rng = np.random.default_rng(seed)
    Q, R = np.linalg.qr(rng.standard_normal((d, d)))
    Q = Q * np.sign(np.diag(R))
    lam = np.arange(1, d + 1, dtype=np.float64) ** (-alpha)
    lam *= d / lam.sum()
    if n_zero:
        lam[-n_zero:] = 0.0
    return Q, lam


def check_exact_rank(ref, sol, singular=False):
    """E_cat exactly rank r, W_i = W_hat_i + E_i: the covariance-aligned shared factors make
    the inference output reproduce X W_i^T to 1e-10 (full-rank or singular Sigma_x)."""
    rng = np.random.default_rng(11 + singular)
    d, r, T = 128, 6, 7
    n_outs = [40, 24, 16]
    m = sum(n_outs)
    Q, lam = _cov(d, 1.19, 5, n_zero=20 if singular else 0)
    U0, _ = np.linalg.qr(rng.standard_normal((m, r)))
    V0, _ = np.linalg.qr(rng.standard_normal((d, r)))
    if singular:  # restrict E to range(Sigma_x)
        P = (Q[:, :d - 20]) @ Q[:, :d - 20].T
        V0, _ = np.linalg.qr(P @ V0)
    sig = np.linspace(2.0, 0.3, r)
    E_cat = (U0 * sig) @ V0.T
    E_list = sol.split_rows(E_cat, n_outs)
    S_half = sol.sqrt_psd(Q, lam)
    S_lift = sol.pinv_sqrt_psd(Q, lam)
    A_list, B, _ = sol.whitened_factors(E_list, S_half, S_lift, r)
    p = tiny_problem(21, T=T, d=d, n_outs=tuple(n_outs), r=r)
    wh = _w_hats(ref, p)
    Z = rng.standard_normal((T, d))
    X = (Z * np.sqrt(lam)) @ Q.T  # rows in range(Sigma_x)
    ys = ref.group_forward(X, wh, B, A_list, restore=True)
    for y, w, E in zip(ys, wh, E_list):
        want = X @ (w + E).T
        assert np.linalg.norm(y - want) <= 1e-10 * np.linalg.norm(want)
    # the QR-reduced core route gives the same product
    A2, B2 = sol.core_factors(E_list, S_half, S_lift, r)
    AB1 = np.vstack(A_list) @ B
    AB2 = np.vstack(A2) @ B2
    assert np.linalg.norm(AB1 - AB2) <= 1e-10 * np.linalg.norm(AB1)


def check_pinv_lift(sol):
    """Singular Sigma_x with an error that also has a part outside its range (the case the
    pseudo-inverse lift of key design 3 exists for): the Moore-Penrose inverse of the symmetric
    root agrees with numpy's SVD-based pinv; B's rows lie in range(Sigma_x) (the minimum-norm
    lift); the factors equal those of the error projected onto that range (whitening cannot see
    the rest); and the whitened residual is the Eckart-Young optimum."""
    rng = np.random.default_rng(41)
    d, n_zero, r, m = 96, 12, 5, 60
    Q, lam = _cov(d, 1.19, 17, n_zero=n_zero)
    S_half = sol.sqrt_psd(Q, lam)
    S_lift = sol.pinv_sqrt_psd(Q, lam)
    assert np.linalg.norm(S_lift - np.linalg.pinv(S_half)) <= 1e-9 * np.linalg.norm(S_lift)
    E = rng.standard_normal((m, d))
    A_list, B, s = sol.whitened_factors([E], S_half, S_lift, r)
    N = Q[:, d - n_zero:]                      # orthonormal basis of the null space
    assert np.linalg.norm(B @ N) <= 1e-12 * np.linalg.norm(B)
    P = np.eye(d) - N @ N.T
    A2, B2, s2 = sol.whitened_factors([E @ P], S_half, S_lift, r)
    AB, AB2 = np.vstack(A_list) @ B, np.vstack(A2) @ B2
    assert np.linalg.norm(AB - AB2) <= 1e-10 * np.linalg.norm(AB)
    assert np.max(np.abs(s - s2)) <= 1e-12 * s[0]
    resid = np.linalg.norm((E - AB) @ S_half) ** 2
    assert abs(resid - float(np.sum(s[r:] ** 2))) <= 1e-10 * float(np.sum(s ** 2))


def check_eckart_young(sol):
    """Whitened residual of the shared factors equals sum_{j>r} sigma_j^2 of the whitened
    error (closed form), and no other rank-r pair tried does better."""
    rng = np.random.default_rng(31)
    d, r = 96, 5
    n_outs = [30, 20, 50]
    E_list = [rng.standard_normal((O, d)) * (1 + 0.3 * i) for i, O in enumerate(n_outs)]
    Q, lam = _cov(d, 0.77, 6)
    S_half = sol.sqrt_psd(Q, lam)
    S_lift = sol.pinv_sqrt_psd(Q, lam)
    A_list, B, S = sol.whitened_factors(E_list, S_half, S_lift, r)
    E_cat = np.vstack(E_list)
    resid = np.linalg.norm((E_cat - np.vstack(A_list) @ B) @ S_half) ** 2
    s_ref = np.linalg.svd(E_cat @ S_half, compute_uv=False)
    closed = float(np.sum(s_ref[r:] ** 2))
    assert abs(resid - closed) <= 1e-12 * closed
    for t in range(20):
        A_alt = np.vstack(A_list) + 0.05 * rng.standard_normal((sum(n_outs), r))
        B_alt = B + 0.05 * rng.standard_normal(B.shape)
        alt = np.linalg.norm((E_cat - A_alt @ B_alt) @ S_half) ** 2
        assert alt >= resid * (1 - 1e-12)
    # per-module right factors add nothing: the best per-module fit with the shared row
    # space B is what the shared solve already gives (A_i = E_i S B^T (B S B^T)^-1 ...)
    Bw = B @ S_half  # whitened shared basis
    for Ei, Ai in zip(E_list, A_list):
        Ai_ls = (Ei @ S_half) @ np.linalg.pinv(Bw)
        assert np.linalg.norm(Ai_ls - Ai) <= 1e-9 * np.linalg.norm(Ai)


def check_isotropic(sol):
    """Sigma_x = c I: the covariance-aligned product equals the plain stacked-SVD product."""
    rng = np.random.default_rng(41)
    d, r = 64, 4
    E_list = [rng.standard_normal((O, d)) for O in (20, 30)]
    c = 2.5
    S_half = np.sqrt(c) * np.eye(d)
    S_lift = np.eye(d) / np.sqrt(c)
    A_list, B, _ = sol.whitened_factors(E_list, S_half, S_lift, r)
    E_cat = np.vstack(E_list)
    U, S, Vt = np.linalg.svd(E_cat, full_matrices=False)
    plain = (U[:, :r] * S[:r]) @ Vt[:r]
    got = np.vstack(A_list) @ B
    assert np.linalg.norm(got - plain) <= 1e-12 * np.linalg.norm(plain)


def check_usage_weighted_risk(sol):
    """E||M x||^2 = tr(M Sigma M^T) = ||M Sigma^{1/2}||_F^2, algebraically and by Monte Carlo."""
    rng = np.random.default_rng(51)
    d, o = 32, 12
    Q, lam = _cov(d, 1.19, 8)
    Sigma = (Q * lam) @ Q.T
    S_half = sol.sqrt_psd(Q, lam)
    assert np.linalg.norm(S_half @ S_half - Sigma) <= 1e-12 * np.linalg.norm(Sigma)
    M = rng.standard_normal((o, d))
    lhs = float(np.trace(M @ Sigma @ M.T))
    rhs = float(np.linalg.norm(M @ S_half) ** 2)
    assert abs(lhs - rhs) <= 1e-12 * lhs
    n = 200000
    X = (rng.standard_normal((n, d)) * np.sqrt(lam)) @ Q.T
    v = np.sum((X @ M.T) ** 2, axis=1)
    mc, se = float(v.mean()), float(v.std() / math.sqrt(n))
    assert abs(mc - lhs) <= 4 * se


def check_second_moment(sol):
    """Sigma_x = X^T X / N: brute force with correctly rounded sums on a tiny input; the
    usage-weighted risk identity on the sample itself (mean of ||M x_t||^2 over the tokens equals
    tr(M Sigma_x M^T)); a closed form (tokens that are scaled basis vectors give a diagonal);
    symmetry and invariance to the token order."""
    rng = np.random.default_rng(61)
    X = rng.standard_normal((7, 5))
    S = sol.second_moment(X)
    for i in range(5):
        for j in range(5):
            want = math.fsum(X[t, i] * X[t, j] for t in range(7)) / 7
            assert abs(S[i, j] - want) <= 1e-15 * (1 + abs(want)), (i, j)
    X = rng.standard_normal((300, 16))
    M = rng.standard_normal((6, 16))
    S = sol.second_moment(X)
    risk = math.fsum(float(np.sum((M @ X[t]) ** 2)) for t in range(300)) / 300
    assert abs(risk - float(np.trace(M @ S @ M.T))) <= 1e-12 * risk
    assert np.array_equal(S, S.T) or np.max(np.abs(S - S.T)) <= 1e-15 * np.max(np.abs(S))
    perm = rng.permutation(300)
    assert np.max(np.abs(sol.second_moment(X[perm]) - S)) <= 1e-13 * np.max(np.abs(S))
    E = np.zeros((6, 3))
    E[0, 0], E[1, 1], E[2, 1], E[3, 2], E[4, 2], E[5, 2] = 2.0, 1.0, -3.0, 1.0, 1.0, 2.0
    assert np.array_equal(sol.second_moment(E), np.diag([4.0 / 6, 10.0 / 6, 6.0 / 6]))


def check_qr_core(sol):
    """sigma(R_e Sigma^{1/2}) = sigma(E_cat Sigma^{1/2}) (left-orthogonal invariance)."""
    rng = np.random.default_rng(61)
    d = 48
    E_cat = rng.standard_normal((150, d))
    Q, lam = _cov(d, 1.19, 9)
    S_half = sol.sqrt_psd(Q, lam)
    Qe, M = sol.qr_core(E_cat, S_half)
    assert M.shape == (d, d)
    assert np.linalg.norm(Qe.T @ Qe - np.eye(d)) <= 1e-12 * d
    s1 = np.linalg.svd(M, compute_uv=False)
    s2 = np.linalg.svd(E_cat @ S_half, compute_uv=False)
    assert np.max(np.abs(s1 - s2)) <= 1e-12 * s2[0]


def check_cholesky_vs_symmetric(sol):
    """The lifted product A B does not depend on which square root of Sigma_x is used."""
    rng = np.random.default_rng(71)
    d, r = 64, 6
    E_list = [rng.standard_normal((O, d)) for O in (30, 34)]
    Q, lam = _cov(d, 0.77, 10)
    Sigma = (Q * lam) @ Q.T
    L = np.linalg.cholesky(Sigma)
    A1, B1, _ = sol.whitened_factors(E_list, sol.sqrt_psd(Q, lam), sol.pinv_sqrt_psd(Q, lam), r)
    A2, B2, _ = sol.whitened_factors(E_list, L, np.linalg.inv(L), r)
    P1 = np.vstack(A1) @ B1
    P2 = np.vstack(A2) @ B2
    assert np.linalg.norm(P1 - P2) <= 1e-10 * np.linalg.norm(P1)


def check_randomized_svd(sol):
    """Randomized SVD: exact on an exactly rank-r core with p = q = 0; with oversampling and
    power iterations it reaches the exact top-r subspace of a decaying spectrum."""
    rng = np.random.default_rng(81)
    d, r = 80, 6
    U0, _ = np.linalg.qr(rng.standard_normal((d, r)))
    V0, _ = np.linalg.qr(rng.standard_normal((d, r)))
    M = (U0 * np.linspace(3, 1, r)) @ V0.T
    U, S, Vt = sol.randomized_svd(M, r, 0, 0, np.random.default_rng(1))
    P = (U[:, :r] * S[:r]) @ Vt[:r]
    assert np.linalg.norm(P - M) <= 1e-12 * np.linalg.norm(M)
    sv = 1.0 / np.arange(1, d + 1) ** 1.5
    Ua, _ = np.linalg.qr(rng.standard_normal((d, d)))
    Va, _ = np.linalg.qr(rng.standard_normal((d, d)))
    M2 = (Ua * sv) @ Va.T
    U, S, Vt = sol.randomized_svd(M2, r, 10, 3, np.random.default_rng(2))
    assert np.max(np.abs(S[:r] - sv[:r]) / sv[:r]) <= 1e-6
    best = np.sqrt(np.sum(sv[r:] ** 2))
    got = np.linalg.norm(M2 - (U[:, :r] * S[:r]) @ Vt[:r])
    assert got <= best * (1 + 1e-6)


def check_scores(sol):
    """g_ec is 1 for a core of rank <= r and the captured fraction otherwise; g_ner is the
    error-to-weight energy ratio; top-k matches exhaustive search with index tie-break."""
    rng = np.random.default_rng(91)
    M = (rng.standard_normal((20, 3))) @ rng.standard_normal((3, 20))
    assert abs(sol.g_ec(M, 3) - 1.0) <= 1e-12
    D = np.diag([4.0, 3.0, 2.0, 1.0])
    assert abs(sol.g_ec(D, 2) - (16 + 9) / 30.0) <= 1e-15
    W = np.full((3, 4), 2.0)
    E = np.full((3, 4), 0.5)
    assert abs(sol.g_ner(E, W) - 0.0625) <= 1e-15
    scores = [0.3, 0.9, 0.3, 0.1, 0.9, 0.5]
    for k in range(len(scores) + 1):
        best = None
        for comb in itertools.combinations(range(len(scores)), k):
            key = (sum(scores[i] for i in comb), [-i for i in sorted(comb)])
            if best is None or key > best[0]:
                best = (key, comb)
        want = [u in best[1] for u in range(len(scores))]
        assert sol.topk_restore(scores, k) == want, k


# ------------------------------------------------------------------ W4A8 (8-bit activations)
def check_w4a8_quantizer_hand(ref):
    """Hand-worked per-token codes in exact fp32 cases: a row whose max is 127 (scale 1, ties to
    even: -63.5 -> -64, 62.5 -> 62, 1.5 -> 2, -0.5 -> 0), a zero row (scale 0, codes 0) and a row
    whose max is 254 (scale 2: 63.5 -> 64, -31.5 -> -32, 0.5 -> 0, 3 -> 2)."""
    x = np.array([[127, -63.5, 62.5, 0.25, -0.5, 1.5, -127, 3],
                  [0, 0, 0, 0, 0, 0, 0, 0],
                  [254, 127, -63, 1, 6, -254, 0.5, 5]], dtype=np.float16)
    codes, scale = ref.quantize_x_int8(x)
    assert [float(v) for v in scale] == [1.0, 0.0, 2.0], scale
    assert codes[0].tolist() == [127, -64, 62, 0, 0, 2, -127, 3], codes[0]
    assert codes[1].tolist() == [0] * 8
    assert codes[2].tolist() == [127, 64, -32, 0, 3, -127, 0, 2], codes[2]


def check_w4a8_quantizer_invariants(ref):
    """Round to nearest: |x - scale * code| <= scale / 2 (up to the fp32 rounding of the ratio);
    codes in -127..127; every nonzero row's largest |x| maps to +-127."""
    rng = np.random.default_rng(61)
    x = (rng.standard_normal((9, 384)) * np.exp(rng.uniform(-6, 6, (9, 1)))).astype(np.float16)
    codes, scale = ref.quantize_x_int8(x)
    xf = x.astype(np.float64)
    assert codes.min() >= -127 and codes.max() <= 127
    err = np.abs(xf - scale.astype(np.float64)[:, None] * codes)
    assert np.all(err <= scale.astype(np.float64)[:, None] * (0.5 + 1e-6))
    amax_idx = np.abs(xf).argmax(axis=1)
    assert np.all(np.abs(codes[np.arange(9), amax_idx]) == 127)


def _w4a8_problem(seed, T=3, d=256, n_outs=(24, 16), r=4):
    p = tiny_problem(seed, T=T, d=d, n_outs=n_outs, r=r)
    rng = np.random.default_rng(seed + 100)
    p.x = (rng.standard_normal((T, d)) * 3).astype(np.float16)
    return p


def check_w4a8_bruteforce(ref):
    """The numpy W4A8 forward against element-by-element fsum loops (each code from its own fp32
    division and rounding; products exact in fp64), restore on and off."""
    p = _w4a8_problem(71)
    wh = _w_hats(ref, p)
    for restore in (True, False):
        ys = ref.group_forward_w4a8(p.x, wh, p.b, p.a, restore=restore)
        bf = ref.bruteforce_group_w4a8(p.x, p.words, p.s, p.z, p.n_outs, p.d, p.b, p.a, restore=restore)
        for y, yb in zip(ys, bf):
            assert np.linalg.norm(y - yb) <= 1e-13 * np.linalg.norm(yb), restore


def check_w4a8_lossless_and_scale(ref):
    """Integer activations whose row maximum is 127 quantise losslessly (scale 1, codes = X): the
    W4A8 forward then equals the pinned W4A16 forward exactly.  Doubling X (exact in fp16) keeps
    the codes, doubles the scales and so exactly doubles the quantised product."""
    p = _w4a8_problem(73)
    rng = np.random.default_rng(5)
    xi = rng.integers(-127, 128, size=(3, p.d)).astype(np.float64)
    xi[:, 7] = 127.0
    x16 = xi.astype(np.float16)
    wh = _w_hats(ref, p)
    y8 = ref.group_forward_w4a8(x16, wh, p.b, p.a, restore=True)
    y16 = ref.group_forward(x16, wh, p.b, p.a, restore=True)
    for a, b in zip(y8, y16):
        assert np.array_equal(a, b)
    base = ref.group_forward_w4a8(p.x, wh, None, p.a, restore=False)
    dbl = ref.group_forward_w4a8((p.x.astype(np.float32) * 2).astype(np.float16), wh, None, p.a, restore=False)
    for a, b in zip(base, dbl):
        assert np.array_equal(2.0 * a, b)


# ------------------------------------------------------------------ mixture of experts
def _moe_problem(seed, n_exp=5, T=7, d=256, n_outs=(24, 16), r=4, top=2):
    rng = np.random.default_rng(seed)
    G = d // 128
    experts = []
    for e in range(n_exp):
        mods = []
        for O in n_outs:
            q = rng.integers(0, 16, size=(O, d))
            s = rng.uniform(0.002, 0.05, size=(O, G)).astype(np.float16)
            z = rng.integers(0, 16, size=(O, G)).astype(np.float16)
            mods.append((pack_words(q), s, z, O))
        experts.append(mods)
    x = rng.standard_normal((T, d)).astype(np.float16)
    b = [(rng.standard_normal((r, d)) / math.sqrt(d)).astype(np.float16) for _ in range(n_exp)]
    a = [[(rng.standard_normal((O, r)) * 0.05).astype(np.float16) for O in n_outs] for _ in range(n_exp)]
    # top-`top` routing of every token to distinct experts; expert 1 receives no token
    pairs = []
    for t in range(T):
        choice = rng.permutation([e for e in range(n_exp) if e != 1])[:top]
        pairs += [(int(e), t) for e in choice]
    pairs.sort()
    row_token = np.array([t for _, t in pairs], dtype=np.int32)
    counts = np.bincount([e for e, _ in pairs], minlength=n_exp)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return SimpleNamespace(experts=experts, x=x, b=b, a=a, row_token=row_token, offsets=offsets, d=d,
                           n_exp=n_exp, n_outs=list(n_outs), r=r)


def _moe_w_hats(ref, p):
    return [[ref.dequant(w, s, z, O, p.d) for (w, s, z, O) in mods] for mods in p.experts]


def check_moe_rows(ref):
    """Every routed row equals the single-token group forward of its token through its expert's
    modules (rows are independent, so this is computed one row at a time, by a route that shares
    no blocking with the per-expert batches); an expert without rows changes nothing; with every
    expert holding the same B, one B for all experts gives the same outputs; permuting the rows
    inside an expert's range permutes the outputs."""
    p = _moe_problem(81)
    wh = _moe_w_hats(ref, p)
    ys = ref.moe_forward(p.x, p.row_token, p.offsets, wh, p.b, p.a, restore=True, share="expert")
    owner = np.repeat(np.arange(p.n_exp), np.diff(p.offsets))
    for j in range(len(p.row_token)):
        e, t = int(owner[j]), int(p.row_token[j])
        one = ref.group_forward(p.x[t:t + 1], wh[e], p.b[e], p.a[e], restore=True)
        for i in range(len(p.n_outs)):
            assert np.allclose(ys[i][j], one[i][0], rtol=1e-13, atol=1e-13 * np.abs(one[i]).max())
    assert p.offsets[1] == p.offsets[2]  # expert 1 has no rows
    # one B for all experts == every expert with that same B
    b0 = p.b[0]
    y_all = ref.moe_forward(p.x, p.row_token, p.offsets, wh, b0, p.a, restore=True, share="all")
    y_same = ref.moe_forward(p.x, p.row_token, p.offsets, wh, [b0] * p.n_exp, p.a, restore=True, share="expert")
    for u, v in zip(y_all, y_same):
        assert np.allclose(u, v, rtol=1e-13, atol=1e-13 * np.abs(v).max())
    # restore off: the quantised products alone, in both sharing modes
    y0 = ref.moe_forward(p.x, p.row_token, p.offsets, wh, p.b, p.a, restore=False, share="expert")
    y0a = ref.moe_forward(p.x, p.row_token, p.offsets, wh, b0, p.a, restore=False, share="all")
    for j in range(len(p.row_token)):
        e, t = int(owner[j]), int(p.row_token[j])
        for i in range(len(p.n_outs)):
            want = p.x[t].astype(np.float64) @ wh[e][i].T
            assert np.array_equal(y0[i][j], y0a[i][j])
            assert np.allclose(y0[i][j], want, rtol=1e-13, atol=1e-13 * np.abs(want).max())
    # a permutation of expert 3's rows permutes its outputs
    lo, hi = int(p.offsets[3]), int(p.offsets[4])
    perm = np.arange(len(p.row_token))
    perm[lo:hi] = perm[lo:hi][::-1]
    yp = ref.moe_forward(p.x, p.row_token[perm], p.offsets, wh, p.b, p.a, restore=True, share="expert")
    for u, v in zip(ys, yp):
        assert np.allclose(u[perm], v, rtol=1e-13, atol=1e-13 * np.abs(u).max())


# ------------------------------------------------------------------ the parity comparator
def check_parity_errors(ref):
    """The comparator behind every GPU parity assertion, against values worked by hand: the
    relative Frobenius error ||y - y_ref||_F / ||y_ref||_F and the largest elementwise error
    over max|y_ref| (the two bounds of the parity bar), with a negative difference, several
    rows, and a zero reference, where the bound becomes an equality."""
    def near(a, b):
        assert abs(a - b) <= 1e-15 * max(1.0, abs(b)), (a, b)

    e = ref.parity_errors(np.array([[3.0, 4.5]]), np.array([[3.0, 4.0]]))
    near(e["rel_fro"], 0.1)            # |0.5| / 5
    near(e["max_abs_rel"], 0.125)      # 0.5 / 4
    e = ref.parity_errors(np.array([[-2.5, 1.0], [0.0, 0.0]]), np.array([[-2.0, 1.0], [0.0, 0.0]]))
    near(e["rel_fro"], 0.5 / math.sqrt(5.0))
    near(e["max_abs_rel"], 0.25)       # |-0.5| / |-2|
    y_ref = np.array([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0]])
    y = y_ref + np.array([[0.0, 0.1], [-0.3, 0.0], [0.0, 0.0]])
    e = ref.parity_errors(y, y_ref)
    near(e["rel_fro"], math.sqrt((0.1 ** 2 + 0.3 ** 2) / 91.0))
    near(e["max_abs_rel"], 0.3 / 6.0)
    z = np.zeros((2, 3))
    e = ref.parity_errors(z, z)
    assert e["rel_fro"] == 0.0 and e["max_abs_rel"] == 0.0, e
    zt = z.copy()
    zt[1, 2] = 1e-30
    e = ref.parity_errors(zt, z)
    assert math.isinf(e["rel_fro"]) and math.isinf(e["max_abs_rel"]), e
    e = ref.parity_errors(y_ref, y_ref)
    assert e["rel_fro"] == 0.0 and e["max_abs_rel"] == 0.0, e


def check_restore_tol(sol):
    """Layer-order fallback: a hand-worked case (scores within 1 % of the best count as equal, the
    lower index first), every score within one step -> the first k units, rel_tol = 0 and any
    tolerance on well-separated scores equal the exact ranking (exhaustive search pins that one),
    an all-zero score vector -> the first k."""
    sc = [0.5, 0.503, 0.501, 0.2, 0.5029]
    assert sol.topk_restore_tol(sc, 2, 0.01) == [True, True, False, False, False]
    assert sol.topk_restore_tol(sc, 4, 0.01) == [True, True, True, False, True]
    assert sol.topk_restore_tol(sc, 2, 0.0) == [False, True, False, False, True]
    near = [1.0 + 1e-5 * u for u in range(12)]  # the best is the last unit, all within one step
    assert sol.topk_restore_tol(near, 5, 1e-3) == [u < 5 for u in range(12)]
    rng = np.random.default_rng(17)
    for _ in range(20):
        v = list(rng.uniform(0, 1, 9))
        for k in range(10):
            assert sol.topk_restore_tol(v, k, 0.0) == sol.topk_restore(v, k)
    spaced = [0.1 * (u % 7) + 0.05 for u in range(7)]  # distinct scores 0.1 apart, max 0.65
    for k in range(8):
        assert sol.topk_restore_tol(spaced, k, 0.05) == sol.topk_restore(spaced, k)
    assert sol.topk_restore_tol([0.0] * 6, 3, 0.01) == [True, True, True, False, False, False]


# ------------------------------------------------------------------ MX weight formats
MX_BITS = {"mxfp4": (2, 1), "mxfp6_e2m3": (2, 3), "mxfp6_e3m2": (3, 2)}


def _mx_golden():
    full, props = {}, {}
    with open(os.path.join(GOLDEN, "mx_elements.txt")) as f:
        for line in f:
            tok = line.split()
            if not tok or tok[0].startswith("#"):
                continue
            if tok[0] == "all":
                full[tok[1]] = [float(v) for v in tok[2:]]
            elif tok[0] == "props":
                props[tok[1]] = {kv.split("=")[0]: float(kv.split("=")[1]) for kv in tok[2:]}
    return full, props


def check_mx_elements(ref):
    """Every element code of the three MX element formats against the specification's printed
    values (tests/golden/mx_elements.txt): FP4's full table; for the FP6 formats the largest and
    smallest normal and subnormal magnitudes; magnitudes strictly increase with the code, the
    sign bit negates (code 100..0 is -0), and the exponent field 0 codes are the subnormals."""
    full, props = _mx_golden()
    for fmt, (eb, mb) in MX_BITS.items():
        n = 1 + eb + mb
        mags = [ref.mx_element_value(c, fmt) for c in range(1 << (n - 1))]
        if fmt in full:
            assert mags == full[fmt], (fmt, mags)
        assert all(a < b for a, b in zip(mags, mags[1:])), fmt
        sub = [m for c, m in enumerate(mags) if c >> mb == 0 and c > 0]
        nor = [m for c, m in enumerate(mags) if c >> mb > 0]
        pr = props[fmt]
        assert max(nor) == pr["max_normal"] and min(nor) == pr["min_normal"], fmt
        assert max(sub) == pr["max_subnormal"] and min(sub) == pr["min_subnormal"], fmt
        for c in range(1 << (n - 1)):
            neg = ref.mx_element_value(c | (1 << (n - 1)), fmt)
            assert neg == -mags[c] and math.copysign(1.0, neg) == -1.0, (fmt, c)


def check_mx_scales(ref):
    """E8M0 scales against torch's float8_e8m0fnu conversion (all 256 bytes; 255 is NaN)."""
    import torch
    want = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64)
    for s in range(256):
        got = ref.e8m0_value(s)
        if s == 255:
            assert math.isnan(got) and math.isnan(float(want[s]))
        else:
            assert got == float(want[s]), (s, got, float(want[s]))


def check_mx_dequant_hand(ref):
    """dequant_mx on 3 rows x 96 inputs (three blocks per row, each (row, block) its own
    scale): element k of row o is the printed FP4 magnitude of its code, negated when the code's
    sign bit is set, times 2^(S[o][k // 32] - 127)."""
    full, _ = _mx_golden()
    table = full["mxfp4"]
    O, K = 3, 96
    codes = np.array([[(5 * k + 3 * o) % 16 for k in range(K)] for o in range(O)], dtype=np.uint8)
    scales = np.array([[127, 130, 119], [126, 140, 104], [127, 127, 128]], dtype=np.uint8)
    W = ref.dequant_mx(codes, scales, "mxfp4", O, K)
    assert W.shape == (O, K)
    for o in range(O):
        for k in range(K):
            c = int(codes[o, k])
            v = table[c & 7] * (-1.0 if c & 8 else 1.0)
            assert W[o, k] == v * 2.0 ** (int(scales[o, k // 32]) - 127), (o, k)
    # every format's dequantised codes at scale 2^0 are the element values, in code order
    for fmt, (eb, mb) in MX_BITS.items():
        n = 1 << (1 + eb + mb)
        c = np.array([[v % n for v in range(128)]], dtype=np.uint8)
        Wf = ref.dequant_mx(c, np.full((1, 4), 127, dtype=np.uint8), fmt, 1, 128)
        assert [float(v) for v in Wf[0]] == [ref.mx_element_value(v % n, fmt) for v in range(128)], fmt


# ------------------------------------------------------------------ MXFP8 activations
def check_fp8_e4m3_codes(ref):
    """Every E4M3 code against torch's float8_e4m3fn conversion (0x7F and 0xFF are NaN)."""
    import torch
    want = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    for c in range(256):
        got, w = ref.fp8_e4m3_value(c), float(want[c])
        assert (math.isnan(got) and math.isnan(w)) or got == w, (c, got, w)


def check_mx8_quantizer_hand(ref):
    """A block whose largest magnitude is 1.9: shared exponent floor(log2 1.9) - 8 = -8 (scale byte
    119); 1.0 -> 256 (code 0x78), 0.5 -> 128 (0x70), 1.0625 -> 272, halfway between 256 and 288,
    -> 256 (even mantissa), 1.9 -> 486.4 -> saturated to 448 (0x7E), -0.25 -> -64 (0xE8); a block
    of zeros: scale byte 0, codes 0."""
    x = np.zeros((2, 64), dtype=np.float16)
    x[0, :5] = [1.0, 0.5, 1.0625, 1.9, -0.25]
    codes, scales = ref.quantize_x_mxfp8(x)
    assert scales.tolist() == [[119, 0], [0, 0]], scales
    assert codes[0, :5].tolist() == [0x78, 0x70, 0x78, 0x7E, 0xE8], codes[0, :5]
    assert not codes[0, 5:].any() and not codes[1].any()
    xq = ref.dequant_mxfp8(codes, scales)
    assert xq[0, :5].tolist() == [1.0, 0.5, 1.0, 1.75, -0.25]


def check_mx8_quantizer_vs_torch(ref):
    """Random fp16 activations (several magnitudes): each block's scale is 2^(floor(log2 max|x|) - 8)
    (from torch.frexp) and each element is torch's round-to-nearest-even float8_e4m3fn cast of
    x / scale wherever that cast is finite, 448 with x's sign where it overflows."""
    import torch
    g = torch.Generator().manual_seed(5)
    x = (torch.randn(24, 256, generator=g) * torch.logspace(-3, 3, 24).unsqueeze(1)).to(torch.float16)
    x[3, 32:64] = 0
    codes, scales = ref.quantize_x_mxfp8(x)
    xb = x.double().reshape(24, 8, 32)
    amax = xb.abs().amax(dim=2)
    _, e = torch.frexp(amax)
    want_s = torch.where(amax > 0, e - 1 - 8 + 127, torch.zeros_like(e))
    assert np.array_equal(scales.astype(np.int64), want_s.numpy()), "block scales"
    sc = torch.ldexp(torch.ones_like(amax), want_s - 127).repeat_interleave(32, dim=1)
    t = (x.double() / sc).to(torch.float8_e4m3fn).to(torch.float64)
    xq = torch.from_numpy(ref.dequant_mxfp8(codes, scales)) / sc
    fin = torch.isfinite(t)
    assert torch.equal(xq[fin], t[fin])
    assert torch.equal(xq[~fin], 448.0 * torch.sign(x.double()[~fin]))


def check_mx8_bruteforce(ref):
    """group_forward_mx8 on a tiny problem against explicit loops (math.fsum): every activation
    dequantised element by element from its code and block scale, the correction from the fp16
    activations."""
    rng = np.random.default_rng(9)
    T, d, r, n_outs = 3, 64, 4, (5, 3)
    x = (rng.standard_normal((T, d)) * 2).astype(np.float16)
    w_hats = [rng.integers(-7, 8, (O, d)).astype(np.float64) / 8 for O in n_outs]
    b = (rng.standard_normal((r, d)) / 8).astype(np.float16)
    a_list = [(rng.standard_normal((O, r)) / 4).astype(np.float16) for O in n_outs]
    ys = ref.group_forward_mx8(x, w_hats, b, a_list, True)
    codes, scales = ref.quantize_x_mxfp8(x)
    for i, O in enumerate(n_outs):
        for t in range(T):
            for o in range(O):
                base = math.fsum(ref.fp8_e4m3_value(int(codes[t, k])) * 2.0 ** (int(scales[t, k // 32]) - 127)
                                 * w_hats[i][o, k] for k in range(d))
                rr = [math.fsum(float(x[t, k]) * float(b[j, k]) for k in range(d)) for j in range(r)]
                corr = math.fsum(rr[j] * float(a_list[i][o, j]) for j in range(r))
                want = base + corr
                assert abs(ys[i][t, o] - want) <= 1e-12 * (1 + abs(want)), (i, t, o)


ALL_REF_CHECKS = [check_dequant_exhaustive, check_dequant_golden, check_restore_off,
                  check_associativity_small_int, check_bruteforce, check_row_independence,
                  check_path_mask, check_parity_errors, check_w4a8_quantizer_hand,
                  check_w4a8_quantizer_invariants, check_w4a8_bruteforce, check_w4a8_lossless_and_scale,
                  check_moe_rows, check_mx_elements, check_mx_scales, check_mx_dequant_hand,
                  check_fp8_e4m3_codes, check_mx8_quantizer_hand, check_mx8_quantizer_vs_torch, check_mx8_bruteforce]
ALL_SOL_CHECKS = [check_eckart_young, check_isotropic, check_usage_weighted_risk, check_qr_core,
                  check_cholesky_vs_symmetric, check_randomized_svd, check_scores, check_second_moment,
                  check_pinv_lift, check_restore_tol]
