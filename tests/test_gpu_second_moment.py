"""Input second moment Sigma_x = X^T X / N on the GPU (glowq_second_moment) against the fp64
oracle (oracle.solve.second_moment).

Bar (derived from the arithmetic): products of fp16 values are exact in fp32; each token range of
at most N tokens is summed in fp32 and at most 16 ranges are added, then scaled, so
|Sigma_gpu - Sigma| <= (N + 18) 2^-24 (1/N) sum_t |x_ti x_tj| <= (N + 18) 2^-24 sqrt(S_ii S_jj)
element by element (Cauchy-Schwarz); the result is exactly symmetric and bitwise repeatable."""
import numpy as np
import pytest
import torch

import workload as W
from gpu_util import glowq, log
from oracle import solve as S

pytestmark = pytest.mark.gpu
U32 = 2.0 ** -24


def check(sig_gpu, ref, N, cols=None):
    g = sig_gpu.double().cpu().numpy()
    diag = np.diag(ref) if cols is None else None
    if cols is None:
        scale = np.sqrt(np.outer(diag, diag))
        got = g
    else:
        d_all = ref[1]
        ref = ref[0]
        scale = np.sqrt(np.outer(d_all, d_all[cols]))
        got = g[:, cols]
    bound = (N + 18) * U32 * scale + 1e-30
    err = np.abs(got - ref)
    assert np.all(err <= bound), float(np.max(err / bound))


@pytest.mark.parametrize("N,d", [(1, 128), (31, 128), (32, 256), (100, 384), (1000, 256), (4133, 512)])
def test_second_moment_matches_oracle(N, d):
    g = glowq()
    x = W.make_x(N, d, 1.19, (41, N, d))
    s1 = g.second_moment(x.cuda())
    s2 = g.second_moment(x.cuda())
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)          # fixed order of the token ranges
    assert torch.equal(s1, s1.t())      # one writer per mirrored pair
    check(s1, S.second_moment(x.numpy()), N)


def test_second_moment_calibration_shape_sampled():
    """64 calibration sequences of 2048 tokens at d = 4096 (the LLaMA-2-7B attention input):
    64 sampled columns against the oracle, every diagonal element, and symmetry."""
    g = glowq()
    d, seqs, L = 4096, 64, 2048
    log("generating 64 x 2048 calibration tokens")
    basis = W.haar_basis(d, 42, 0)
    x = torch.cat([W.make_x(L, d, 1.19, (42, q), device="cuda", basis=basis) for q in range(seqs)])
    N = x.shape[0]
    sig = g.second_moment(x)
    torch.cuda.synchronize()
    assert torch.equal(sig, sig.t())
    cols = np.sort(np.random.default_rng(5).choice(d, 64, replace=False))
    X64 = x.double().cpu().numpy()
    log("oracle on sampled columns")
    ref_cols = (X64.T @ X64[:, cols]) / N
    diag = np.einsum("ti,ti->i", X64, X64) / N
    # the sampled columns are the oracle's second moment restricted to them: check that on a block
    blk = S.second_moment(X64[:, cols[:8]])
    assert np.max(np.abs(blk - ref_cols[cols[:8]][:, :8])) <= 1e-12 * np.max(np.abs(blk))
    check(sig, (ref_cols, diag), N, cols=cols)


def test_second_moment_validates():
    g = glowq()
    L = g.lib()
    assert L.glowq_second_moment_workspace_bytes(0, 128) == 0
    assert L.glowq_second_moment_workspace_bytes(10, 100) == 0
    x = torch.zeros(4, 128, dtype=torch.float16, device="cuda")
    with pytest.raises(g.GlowQError):
        g.second_moment(x[:, :100])
