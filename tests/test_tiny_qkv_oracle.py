"""The tiny QKV workload end to end in the oracle (CPU): exact whitened shared factors,
brute-force agreement and the correction's effect."""
import numpy as np
import pytest

import workload as W
from oracle import glowq_ref as G
from oracle import solve as S


@pytest.fixture(scope="module")
def tiny():
    c = W.tiny_qkv_inputs()
    w_hats = [G.dequant_qw(q) for q in c["qw"]]
    E = [G._f64(w16) - wh for w16, wh in zip(c["w16"], w_hats)]
    Q, lam = c["Q"].numpy(), c["lam"].numpy()
    A, B, sv = S.whitened_factors(E, S.sqrt_psd(Q, lam), S.pinv_sqrt_psd(Q, lam), c["r"])
    return c, w_hats, E, A, B, sv


def test_tiny_qkv_bruteforce(tiny):
    c, w_hats, E, A, B, _ = tiny
    a16 = [a.astype(np.float16) for a in A]
    b16 = B.astype(np.float16)
    ys = G.group_forward(c["x"], w_hats, b16, a16, restore=True)
    bf = G.bruteforce_group(c["x"], [q.q_packed for q in c["qw"]], [q.s for q in c["qw"]],
                            [q.z for q in c["qw"]], [256] * 3, 256, b16, a16, restore=True)
    for y, yb in zip(ys, bf):
        assert np.max(np.abs(y - yb)) <= 1e-13 * np.max(np.abs(yb))


def test_tiny_qkv_correction_reduces_error(tiny):
    """With covariance-aligned factors the corrected output is closer to the fp16 model's
    output than the quantised product alone."""
    c, w_hats, E, A, B, sv = tiny
    x = G._f64(c["x"])
    ys = G.group_forward(c["x"], w_hats, B, A, restore=True)
    y0 = G.group_forward(c["x"], w_hats, B, A, restore=False)
    for y, yq, w16 in zip(ys, y0, c["w16"]):
        ref = x @ G._f64(w16).T
        assert np.linalg.norm(y - ref) < 0.95 * np.linalg.norm(yq - ref)
    # factors are balanced: A^T A = B Sigma B^T = diag(top-r singular values)
    Q, lam = c["Q"].numpy(), c["lam"].numpy()
    Sig = (Q * lam) @ Q.T
    At = np.vstack(A)
    assert np.allclose(At.T @ At, np.diag(sv[:16]), atol=1e-10 * sv[0])
    assert np.allclose(B @ Sig @ B.T, np.diag(sv[:16]), atol=1e-8 * sv[0])
