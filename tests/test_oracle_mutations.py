"""Plant plausible mistakes in copies of the oracle (on the CPU) and confirm that at least
one pin check fails for each: the pins are strong enough to catch a dropped term, a wrong
sign or index, a transposed operand or a wrong nibble order."""
import math

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


def pinv_identity_on_null(Q, lam, rtol=1e-12):
    # a generalised inverse of the root that is not the Moore-Penrose one (1 on the null space)
    lam = np.asarray(lam, dtype=np.float64)
    cut = rtol * float(lam.max())
    inv = np.where(lam > cut, 1.0 / np.sqrt(np.where(lam > cut, lam, 1.0)), 1.0)
    return (Q * inv) @ Q.T


def topk_tol_relative_to_score(scores, k, rel_tol):
    # steps measured from zero rather than from the best score
    if rel_tol <= 0:
        return SOL.topk_restore(scores, k)
    mx = max(float(v) for v in scores)
    keys = [-math.floor(float(v) / (rel_tol * mx)) if mx > 0 else 0 for v in scores]
    order = sorted(range(len(scores)), key=lambda u: (keys[u], u))
    return [u in set(order[:k]) for u in range(len(scores))]


def topk_tol_upper_index(scores, k, rel_tol):
    # ties within a step go to the higher index
    mx = max(float(v) for v in scores) if len(scores) else 0.0
    if rel_tol <= 0 or mx <= 0:
        order = sorted(range(len(scores)), key=lambda u: (-float(scores[u]), -u))
    else:
        keys = [math.floor((mx - float(v)) / (rel_tol * mx)) for v in scores]
        order = sorted(range(len(scores)), key=lambda u: (keys[u], -u))
    return [u in set(order[:k]) for u in range(len(scores))]


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


def parity_by_test_norm(y_test, y_ref):
    yt, yr = G._f64(y_test), G._f64(y_ref)
    d = np.abs(yt - yr)
    return dict(rel_fro=float(np.linalg.norm(d) / np.linalg.norm(yt)), max_abs_rel=float(d.max() / np.abs(yt).max()))


def parity_mean_not_max(y_test, y_ref):
    yt, yr = G._f64(y_test), G._f64(y_ref)
    d = np.abs(yt - yr)
    nref, mref = np.linalg.norm(yr), np.abs(yr).max()
    return dict(rel_fro=float(np.linalg.norm(d) / nref) if nref > 0 else 0.0,
                max_abs_rel=float(d.mean() / mref) if mref > 0 else 0.0)


def parity_no_abs(y_test, y_ref):
    yt, yr = G._f64(y_test), G._f64(y_ref)
    d = yt - yr
    nref, mref = np.linalg.norm(yr), yr.max()
    return dict(rel_fro=float(np.linalg.norm(d) / nref) if nref > 0 else 0.0,
                max_abs_rel=float(d.max() / mref) if mref > 0 else 0.0)


def parity_zero_ref_passes(y_test, y_ref):
    yt, yr = G._f64(y_test), G._f64(y_ref)
    d = np.abs(yt - yr)
    nref, mref = np.linalg.norm(yr), np.abs(yr).max()
    return dict(rel_fro=float(np.linalg.norm(d) / nref) if nref > 0 else 0.0,
                max_abs_rel=float(d.max() / mref) if mref > 0 else 0.0)


def _quant_with(x, rnd=np.rint, per_tensor=False, div=127.0, lo=-127):
    xf = G._np(x).astype(np.float32)
    amax = np.abs(xf).max() * np.ones(xf.shape[0], np.float32) if per_tensor else np.abs(xf).max(axis=1)
    scale = (amax.astype(np.float32) / np.float32(div)).astype(np.float32)
    codes = np.zeros(xf.shape, dtype=np.int64)
    nz = scale > 0
    codes[nz] = np.clip(rnd((xf[nz] / scale[nz, None]).astype(np.float32)), lo, -lo).astype(np.int64)
    return codes, scale


def quant_half_away(x):
    return _quant_with(x, rnd=lambda v: np.sign(v) * np.floor(np.abs(v) + 0.5))


def quant_per_tensor(x):
    return _quant_with(x, per_tensor=True)


def quant_div128(x):
    return _quant_with(x, div=128.0)


def quant_unsigned_range(x):
    # an 8-bit range taken as 255 steps (the unsigned width) on a symmetric code
    return _quant_with(x, div=255.0, lo=-255)


def w4a8_no_scale(x, w_hats, b, a_list, restore=True):
    codes, _ = G.quantize_x_int8(x)
    outs = [codes.astype(np.float64) @ wh.T for wh in w_hats]
    if restore and b is not None and G._np(b).shape[0] > 0:
        R = G._f64(x) @ G._f64(b).T
        outs = [y + R @ G._f64(a).T for y, a in zip(outs, a_list)]
    return outs


def w4a8_corr_on_codes(x, w_hats, b, a_list, restore=True):
    codes, scale = G.quantize_x_int8(x)
    xh = scale.astype(np.float64)[:, None] * codes
    outs = [xh @ wh.T for wh in w_hats]
    if restore and b is not None and G._np(b).shape[0] > 0:
        R = xh @ G._f64(b).T  # correction from the dequantised activations
        outs = [y + R @ G._f64(a).T for y, a in zip(outs, a_list)]
    return outs


def moe_next_expert_b(x, row_token, offsets, w_hats, b, a, restore=True, share="expert"):
    n = len(w_hats)
    if share == "expert" and b is not None:
        b = [b[(e + 1) % n] for e in range(n)]  # expert e corrects with its neighbour's B
    return G.moe_forward(x, row_token, offsets, w_hats, b, a, restore, share)


def moe_no_gather(x, row_token, offsets, w_hats, b, a, restore=True, share="expert"):
    xx = G._f64(x)
    n_rows = int(G._np(offsets)[-1])
    idx = np.arange(n_rows) % xx.shape[0]
    return G.moe_forward(xx[idx], None, offsets, w_hats, b, a, restore, share)


def moe_offsets_shifted(x, row_token, offsets, w_hats, b, a, restore=True, share="expert"):
    o = np.array(G._np(offsets), dtype=np.int64).copy()
    o[1:-1] = np.minimum(o[1:-1] + 1, o[-1])  # every boundary one row late
    return G.moe_forward(x, row_token, o, w_hats, b, a, restore, share)


def _mx_value_with(bias_over=None, implicit_sub=False, swap=False):
    def f(code, fmt):
        eb, mb, bias = G.MX_ELEM[fmt]
        if bias_over is not None:
            bias = bias_over
        n = 1 + eb + mb
        sign = -1.0 if (code >> (n - 1)) & 1 else 1.0
        if swap:
            m, e = (code >> eb) & ((1 << mb) - 1), code & ((1 << eb) - 1)
        else:
            e, m = (code >> mb) & ((1 << eb) - 1), code & ((1 << mb) - 1)
        if e == 0 and not implicit_sub:
            mag = math.ldexp(m / (1 << mb), 1 - bias)
        else:
            mag = math.ldexp(1.0 + m / (1 << mb), max(e, 1) - bias)
        return sign * mag
    return f


def mx_dequant_block_mod(codes, scales, fmt, n_out, k_in):
    W = G.dequant_mx(codes, scales, fmt, n_out, k_in)
    s = G._np(scales).astype(np.int64)
    nb = k_in // 32
    good = 2.0 ** (s[:, np.arange(k_in) // 32] - 127)
    bad = 2.0 ** (s[:, np.arange(k_in) % nb] - 127)
    return W / good * bad


def mx_dequant_block16(codes, scales, fmt, n_out, k_in):
    W = G.dequant_mx(codes, scales, fmt, n_out, k_in)
    s = G._np(scales).astype(np.int64)
    idx = np.minimum(np.arange(k_in) // 16, k_in // 32 - 1)
    return W / 2.0 ** (s[:, np.arange(k_in) // 32] - 127) * 2.0 ** (s[:, idx] - 127)


def e8m0_bias128(s):
    return math.nan if s == 255 else math.ldexp(1.0, int(s) - 128)


def e8m0_no_nan(s):
    return math.ldexp(1.0, int(s) - 127)


def _mx8_with(emax=8, ties_away=False, nan_overflow=False, block=32, no_sign=False):
    def q(x):
        xf = G._f64(x)
        T, d = xf.shape
        blocks = xf.reshape(T, d // block, block)
        amax = np.abs(blocks).max(axis=2)
        X = np.full(amax.shape, -127, dtype=np.int64)
        for idx in zip(*np.nonzero(amax)):
            X[idx] = math.frexp(float(amax[idx]))[1] - 1 - emax
        u = np.abs(blocks) / np.ldexp(1.0, X)[:, :, None]
        mags = np.array([G.fp8_e4m3_value(c) for c in range(0x7F)])
        dist = np.abs(u[..., None] - mags)
        best = dist.min(axis=-1, keepdims=True)
        tie = dist == best
        pick = np.where(tie, np.arange(0x7F), -1).max(axis=-1) if ties_away else None
        if pick is None:
            cand = np.where(tie, np.arange(0x7F), 1 << 20)
            even = np.where(tie & (np.arange(0x7F) % 2 == 0), np.arange(0x7F), 1 << 20)
            pick = np.where(tie.sum(axis=-1) > 1, even.min(axis=-1), cand.min(axis=-1))
        if nan_overflow:
            pick = np.where(u > 464, 0x7F, pick)
        if not no_sign:
            pick = np.where((blocks < 0) & (pick > 0), pick | 0x80, pick)
        codes = pick.reshape(T, d).astype(np.uint8)
        sc = (X + 127).astype(np.uint8)
        if block != 32:
            sc = sc[:, ::32 // block]
        return codes, sc
    return q


def mx8_corr_on_quantised(x, w_hats, b, a_list, restore=True):
    xq = G.dequant_mxfp8(*G.quantize_x_mxfp8(x))
    outs = [xq @ wh.T for wh in w_hats]
    if restore and b is not None:
        R = xq @ G._f64(b).T
        outs = [y + R @ G._f64(a).T for y, a in zip(outs, a_list)]
    return outs


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
    "parity_by_test_norm": dict(parity_errors=parity_by_test_norm),
    "parity_mean_not_max": dict(parity_errors=parity_mean_not_max),
    "parity_no_abs": dict(parity_errors=parity_no_abs),
    "parity_zero_ref_passes": dict(parity_errors=parity_zero_ref_passes),
    "quant_half_away": dict(quantize_x_int8=quant_half_away),
    "quant_per_tensor": dict(quantize_x_int8=quant_per_tensor),
    "quant_div128": dict(quantize_x_int8=quant_div128),
    "quant_unsigned_range": dict(quantize_x_int8=quant_unsigned_range),
    "w4a8_no_scale": dict(group_forward_w4a8=w4a8_no_scale),
    "w4a8_corr_on_codes": dict(group_forward_w4a8=w4a8_corr_on_codes),
    "moe_next_expert_b": dict(moe_forward=moe_next_expert_b),
    "moe_no_gather": dict(moe_forward=moe_no_gather),
    "moe_offsets_shifted": dict(moe_forward=moe_offsets_shifted),
    "mx_bias_one_for_all": dict(mx_element_value=_mx_value_with(bias_over=1)),
    "mx_subnormal_implicit_one": dict(mx_element_value=_mx_value_with(implicit_sub=True)),
    "mx_fields_swapped": dict(mx_element_value=_mx_value_with(swap=True)),
    "mx_dequant_block_mod": dict(dequant_mx=mx_dequant_block_mod),
    "mx_dequant_block16": dict(dequant_mx=mx_dequant_block16),
    "e8m0_bias128": dict(e8m0_value=e8m0_bias128),
    "e8m0_no_nan": dict(e8m0_value=e8m0_no_nan),
    "mx8_emax_7": dict(quantize_x_mxfp8=_mx8_with(emax=7)),
    "mx8_ties_away": dict(quantize_x_mxfp8=_mx8_with(ties_away=True)),
    "mx8_nan_on_overflow": dict(quantize_x_mxfp8=_mx8_with(nan_overflow=True)),
    "mx8_block16": dict(quantize_x_mxfp8=_mx8_with(block=16)),
    "mx8_no_sign": dict(quantize_x_mxfp8=_mx8_with(no_sign=True)),
    "mx8_corr_on_quantised": dict(group_forward_mx8=mx8_corr_on_quantised),
}

SOL_MUTANTS = {
    "lift_with_sqrt": dict(whitened_factors=whitened_lift_with_sqrt),
    "unbalanced_full_s": dict(whitened_factors=whitened_full_s),
    "no_whitening": dict(whitened_factors=whitened_unwhitened),
    "topk_lowest": dict(topk_restore=topk_lowest),
    "topk_tol_relative_to_score": dict(topk_restore_tol=topk_tol_relative_to_score),
    "topk_tol_upper_index": dict(topk_restore_tol=topk_tol_upper_index),
    "pinv_identity_on_null": dict(pinv_sqrt_psd=pinv_identity_on_null),
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
