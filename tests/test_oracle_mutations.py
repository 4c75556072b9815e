"""Plant plausible mistakes in copies of the oracle (on the CPU) and confirm that at least
one pin check fails for each: the pins are strong enough to catch a dropped term, a wrong
sign or index, a transposed operand or a wrong nibble order."""
import numpy as np
import pytest

import pins
from oracle import glowq_ref as G

REF, SOL = pins.oracle_namespaces()


def _mut_ref(**over):
    ns = type(REF)(**vars(REF))
    for k, v in over.items():
        setattr(ns, k, v)
    return ns


def _mut_sol(**over):
    ns = type(SOL)(**vars(SOL))
    for k, v in over.items():
        setattr(ns, k, v)
    return ns


def dequant_plus_z(q_packed, s, z, n_out, k_in):
    q = G.unpack_int4(q_packed, n_out, k_in).astype(np.float64)
    g = np.arange(k_in) // 128
    return (q + G._f64(z)[:, g]) * G._f64(s)[:, g]


def dequant_group64(q_packed, s, z, n_out, k_in):
    q = G.unpack_int4(q_packed, n_out, k_in).astype(np.float64)
    g = np.minimum(np.arange(k_in) // 64, k_in // 128 - 1)
    return (q - G._f64(z)[:, g]) * G._f64(s)[:, g]


def dequant_high_nibble_first(q_packed, s, z, n_out, k_in):
    words = G._np(q_packed).astype(np.int64) & 0xFFFFFFFF
    out = np.empty((n_out, k_in // 8, 8))
    for j in range(8):
        out[:, :, j] = (words >> (4 * (7 - j))) & 0xF
    q = out.reshape(n_out, k_in)
    g = np.arange(k_in) // 128
    return (q - G._f64(z)[:, g]) * G._f64(s)[:, g]


def dequant_zs_fp16(q_packed, s, z, n_out, k_in):
    # q*s - z*s with the product z*s rounded to fp16 first
    q = G.unpack_int4(q_packed, n_out, k_in).astype(np.float64)
    g = np.arange(k_in) // 128
    s64 = G._f64(s)[:, g]
    zs = (G._f64(z)[:, g] * s64).astype(np.float16).astype(np.float64)
    return q * s64 - zs


def group_drop_correction(x, w_hats, b, a_list, restore=True):
    return [G._f64(x) @ w.T for w in w_hats]


def group_minus_correction(x, w_hats, b, a_list, restore=True):
    x64 = G._f64(x)
    outs = [x64 @ w.T for w in w_hats]
    if restore and b is not None and G._np(b).shape[0] > 0:
        R = x64 @ G._f64(b).T
        outs = [y - R @ G._f64(a).T for y, a in zip(outs, a_list)]
    return outs


def group_anchor_a_for_all(x, w_hats, b, a_list, restore=True):
    x64 = G._f64(x)
    outs = [x64 @ w.T for w in w_hats]
    if restore and b is not None and G._np(b).shape[0] > 0:
        R = x64 @ G._f64(b).T
        a0 = G._f64(a_list[0])
        outs = [y + R @ (a0[: y.shape[1]] if a0.shape[0] >= y.shape[1] else np.resize(a0, (y.shape[1], a0.shape[1]))).T
                for y in outs]
    return outs


def group_ignores_restore(x, w_hats, b, a_list, restore=True):
    return G.group_forward(x, w_hats, b, a_list, restore=True)


def group_transposed_b(x, w_hats, b, a_list, restore=True):
    x64 = G._f64(x)
    outs = [x64 @ w.T for w in w_hats]
    if restore and b is not None and G._np(b).shape[0] > 0:
        bb = G._f64(b)
        R = x64[:, : bb.shape[0]] @ bb[:, : bb.shape[0]].T  # projects on the wrong axis
        outs = [y + R @ G._f64(a).T for y, a in zip(outs, a_list)]
    return outs


def path_inverted_mask(layers, mask):
    return G.path_forward(layers, [not m for m in mask])


def whitened_lift_with_sqrt(E_list, S_half, S_half_lift, r):
    return SOL.whitened_factors(E_list, S_half, S_half, r)


def whitened_full_s(E_list, S_half, S_half_lift, r):
    n_outs = [np.asarray(e).shape[0] for e in E_list]
    Ew = np.vstack(E_list) @ S_half
    U, S, Vt = np.linalg.svd(Ew, full_matrices=False)
    A = U[:, :r] * S[:r]
    B = (S[:r, None] * Vt[:r]) @ S_half_lift
    return SOL.split_rows(A, n_outs), B, S


def whitened_unwhitened(E_list, S_half, S_half_lift, r):
    n_outs = [np.asarray(e).shape[0] for e in E_list]
    U, S, Vt = np.linalg.svd(np.vstack(E_list), full_matrices=False)
    A, B = SOL.balanced_factors(U, S, Vt, r)
    return SOL.split_rows(A, n_outs), B, S


def topk_lowest(scores, k):
    order = sorted(range(len(scores)), key=lambda u: (float(scores[u]), u))
    chosen = set(order[:k])
    return [u in chosen for u in range(len(scores))]


def moment_centred(X):
    X = np.asarray(X, dtype=np.float64)
    Xc = X - X.mean(axis=0)
    return (Xc.T @ Xc) / X.shape[0]


def moment_unbiased(X):
    X = np.asarray(X, dtype=np.float64)
    return (X.T @ X) / (X.shape[0] - 1)


def moment_token_gram(X):
    X = np.asarray(X, dtype=np.float64)
    G = X @ X.T / X.shape[1]
    return G[:X.shape[1], :X.shape[1]] if G.shape[0] >= X.shape[1] else np.pad(G, (0, X.shape[1] - G.shape[0]))


REF_MUTANTS = {
    "dequant_plus_z": dict(dequant=dequant_plus_z),
    "dequant_group64": dict(dequant=dequant_group64),
    "dequant_high_nibble_first": dict(dequant=dequant_high_nibble_first),
    "dequant_zs_fp16": dict(dequant=dequant_zs_fp16),
    "group_drop_correction": dict(group_forward=group_drop_correction),
    "group_minus_correction": dict(group_forward=group_minus_correction),
    "group_anchor_a_for_all": dict(group_forward=group_anchor_a_for_all),
    "group_ignores_restore": dict(group_forward=group_ignores_restore),
    "group_transposed_b": dict(group_forward=group_transposed_b),
    "path_inverted_mask": dict(path_forward=path_inverted_mask),
}

SOL_MUTANTS = {
    "lift_with_sqrt": dict(whitened_factors=whitened_lift_with_sqrt),
    "unbalanced_full_s": dict(whitened_factors=whitened_full_s),
    "no_whitening": dict(whitened_factors=whitened_unwhitened),
    "topk_lowest": dict(topk_restore=topk_lowest),
    "moment_centred": dict(second_moment=moment_centred),
    "moment_unbiased": dict(second_moment=moment_unbiased),
    "moment_token_gram": dict(second_moment=moment_token_gram),
}


def _any_fails(checks):
    for c in checks:
        try:
            c()
        except Exception:
            return True
    return False


@pytest.mark.parametrize("name", sorted(REF_MUTANTS))
def test_ref_mutant_is_caught(name):
    ref = _mut_ref(**REF_MUTANTS[name])
    checks = [lambda c=c: c(ref) for c in pins.ALL_REF_CHECKS]
    checks.append(lambda: pins.check_exact_rank(ref, SOL))
    assert _any_fails(checks), f"no pin caught mutant {name}"


@pytest.mark.parametrize("name", sorted(SOL_MUTANTS))
def test_sol_mutant_is_caught(name):
    sol = _mut_sol(**SOL_MUTANTS[name])
    checks = [lambda c=c: c(sol) for c in pins.ALL_SOL_CHECKS]
    checks.append(lambda: pins.check_exact_rank(REF, sol))
    checks.append(lambda: pins.check_exact_rank(REF, sol, singular=True))
    assert _any_fails(checks), f"no pin caught mutant {name}"
