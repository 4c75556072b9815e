"""The seeded synthetic workload (CPU): base-quantiser invariants, canonical packing against
the oracle's unpacker, seeding, spectra and factor scaling."""
import math

import numpy as np
import torch

import workload as W
from oracle import glowq_ref


def test_rtn_invariants():
    """Round-to-nearest INT4-g128: every unclamped weight lies within s/2 of its dequantised
    value, the group minimum maps to q = 0, the maximum to 14 or 15, z is an integer."""
    cols = W.outlier_columns(512, (9, 9))
    w = W.make_w(64, 512, (9, 9, 0), cols)
    qw = W.rtn_quantize(w)
    q = qw.q.to(torch.int64).numpy()
    s = qw.s.to(torch.float64).numpy()
    z = qw.z.to(torch.float64).numpy()
    assert np.all(z == np.round(z))
    wf = w.to(torch.float64).numpy()
    g = np.arange(512) // 128
    w_hat = (q - z[:, g]) * s[:, g]
    inner = (q > 0) & (q < 15)
    assert np.all(np.abs(wf - w_hat)[inner] <= s[:, g][inner] / 2)
    wg = wf.reshape(64, 4, 128)
    qg = q.reshape(64, 4, 128)
    amin = wg.argmin(axis=2)
    amax = wg.argmax(axis=2)
    assert np.all(np.take_along_axis(qg, amin[..., None], 2) == 0)
    assert np.all(np.isin(np.take_along_axis(qg, amax[..., None], 2), [14, 15]))
    assert abs(qw.err_sq - float(((wf - w_hat) ** 2).sum())) <= 1e-9 * qw.err_sq


def test_packing_matches_oracle_unpack():
    rng = np.random.default_rng(0)
    q = torch.from_numpy(rng.integers(0, 16, size=(37, 384)).astype(np.uint8))
    words = W.pack_canonical(q)
    assert words.dtype == torch.int32 and words.shape == (37, 48)
    back = glowq_ref.unpack_int4(words, 37, 384)
    assert np.array_equal(back, q.numpy())


def test_seeding_is_deterministic_and_keyed():
    a = W.make_x(4, 256, 1.19, (1, 2, 3))
    b = W.make_x(4, 256, 1.19, (1, 2, 3))
    c = W.make_x(4, 256, 1.19, (1, 2, 4))
    assert torch.equal(a, b) and not torch.equal(a, c)
    assert W.seed_of(0, 1) != W.seed_of(1, 0)


def test_powerlaw_spectrum_and_basis():
    lam = W.powerlaw_spectrum(300, 1.19)
    assert abs(float(lam.sum()) - 300) < 1e-9
    ratio = lam[:-1] / lam[1:]
    k = torch.arange(1, 300, dtype=torch.float64)
    assert torch.allclose(ratio, ((k + 1) / k) ** 1.19)
    Q = W.haar_basis(128, 5)
    assert torch.allclose(Q.t() @ Q, torch.eye(128, dtype=Q.dtype), atol=1e-12)


def test_activation_covariance_follows_spectrum():
    d = 128
    lam = W.powerlaw_spectrum(d, 0.77)
    Q = W.haar_basis(d, 3)
    x = W.make_x(20000, d, 0.77, (3,), basis=Q, lam=lam).to(torch.float64)
    C = x.t() @ x / x.shape[0]
    ev = torch.linalg.eigvalsh(C).flip(0)
    assert torch.allclose(ev[:8], lam[:8], rtol=0.08)


def test_factor_scaling_matches_error_norm():
    unit = W.make_unit("qkv", "group", W.make_x(2, 256, 1.19, (5,)), [64, 32, 48], 8, (5, 0))
    for a, qw in zip(unit.a, unit.weights):
        ab = a.to(torch.float64) @ unit.b.to(torch.float64)
        assert abs(float(ab.norm()) - math.sqrt(qw.err_sq)) <= 2e-3 * math.sqrt(qw.err_sq)
    assert unit.b.shape == (8, 256)


def test_restore_mask_counts():
    m = W.restore_mask(32, 16, (0, 3, 0, 0))
    assert sum(m) == 16 and len(m) == 32
    assert m == W.restore_mask(32, 16, (0, 3, 0, 0))


def test_outlier_columns_shared_within_group():
    unit = W.make_unit("g", "group", W.make_x(1, 256, 1.19, (6,)), [16, 16], 4, (6, 1))
    cols = W.outlier_columns(256, (6, 1))
    assert cols.numel() == 4
    # the outlier columns carry ~10x larger quantisation scales in every module
    for qw in unit.weights:
        assert qw.s.shape == (16, 2)


def test_mx_quantizer_nearest_element_and_ranges():
    """Microscaling quantisation: every code is the element nearest to w / 2^X (the oracle's
    element table, brute force), the block exponent puts the block maximum in the element's top
    binade (inside the exact-fp16 range), codes fit their width, an all-zero block gets the
    range's low end and zero codes, and err_sq is ||W - dequant||^2."""
    cols = W.outlier_columns(256, (8,))
    w = W.make_w(24, 256, (8,), cols)
    w[3, :32] = 0
    for fmt, (eb, mb, bias) in W.MX_FORMATS.items():
        q = W.mx_quantize(w, fmt)
        lo, hi = W.MX_EXP_RANGE[fmt]
        n = 1 << (1 + eb + mb)
        vals = np.array([glowq_ref.mx_element_value(c, fmt) for c in range(n)])
        codes, X = q.codes.numpy().astype(np.int64), q.scales.numpy().astype(np.int64) - 127
        assert codes.max() < n and X.min() >= lo and X.max() <= hi
        assert X[3, 0] == lo and np.all(codes[3, :32] % (n // 2) == 0)
        wb = w.double().numpy()
        u = wb / np.ldexp(1.0, X)[:, np.arange(256) // 32]
        dist = np.abs(vals[None, None, :] - u[:, :, None])
        assert np.all(np.abs(vals[codes] - u) == dist.min(axis=2))
        emax = (1 << eb) - 1 - bias
        amax = np.abs(wb).reshape(24, 8, 32).max(axis=2)
        nz = amax > 0
        assert np.all(np.floor(np.log2(amax[nz])) - emax == X[nz])
        wh = glowq_ref.dequant_mx(q.codes, q.scales, fmt, 24, 256)
        assert abs(((wb - wh) ** 2).sum() - q.err_sq) <= 1e-12 * q.err_sq


def test_mx_quantizer_ties_to_even():
    """A value halfway between two FP4 elements rounds to the one with the even mantissa
    (1.25 -> 1.0, 1.75 -> 2.0, 2.5 -> 2.0, 5.0 -> 4.0) and values past the largest element
    saturate to 6."""
    row = torch.zeros(1, 32, dtype=torch.float16)
    row[0, :6] = torch.tensor([1.25, 1.75, 2.5, 5.0, -5.0, 7.5])
    q = W.mx_quantize(row, "mxfp4")
    assert int(q.scales[0, 0]) == 127  # max 7.5 -> floor(log2 7.5) - 2 = 0
    got = [glowq_ref.mx_element_value(int(c), "mxfp4") for c in q.codes[0, :6]]
    assert got == [1.0, 2.0, 2.0, 4.0, -4.0, 6.0]


def test_module_weights_follow_unit_keys():
    """make_unit draws module i's weight from keys + (i,) with the unit's outlier columns (the
    convention llama2_path_weights relies on to regenerate the path's fp16 weights)."""
    keys = (0, 3, 7, 2)
    unit = W.make_unit("t", "group", W.make_x(1, 256, 0.77, (1,)), [32, 16], 8, keys)
    cols = W.outlier_columns(256, keys)
    for i, O in enumerate([32, 16]):
        q = W.rtn_quantize(W.make_w(O, 256, list(keys) + [i], cols))
        assert torch.equal(q.q, unit.weights[i].q) and torch.equal(q.s, unit.weights[i].s)
    assert [u[3] for u in W.LLAMA2_PATH_UNITS] == [[4096] * 3, [4096], [11008] * 2, [4096]]
