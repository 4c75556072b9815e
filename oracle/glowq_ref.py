"""fp64 CPU oracle of the GlowQ inference path (TEST INFRASTRUCTURE ONLY).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import this
module.  It shares no code with the HIP library and the library never imports it.

What it computes is the plain definition of the method's inference result; the method
reaches exactly this result (up to rounding order), its speed coming from computing the
shared projection once per group:

  * dequantisation of the W4A16 "INT4, g128" weights (GlowQ paper note, "Experimental
    setup"): W_hat[o, k] = (q[o, k] - z[o, g]) * s[o, g] with g = floor(k / 128);
  * the low-rank error-compensation paradigm W - W_q ~ A B, the output gaining A (B X)
    (GlowQ paper note, "Research background and motivation");
  * the group-shared form: for an input-sharing group the right projection
    R = X B_shared^T is formed once, by the anchor, and every module i of the group,
    the anchor included, returns y_i = X W_hat_i^T + R A_i^T (GlowQ paper note, key
    design 4 and the flowchart's final node; GlowQ arXiv abstract);
  * solo modules (o_proj, down_proj) do the same with a private B, on the fly
    (key design 4);
  * GlowQ-S: a unit outside the restore set returns the quantised product alone
    (key design 4; "Efficiency and selective restoration" bullets);
  * the layerwise baseline: every module has its own (A_i, B_i) and its own
    projection X B_i^T (GlowQ paper note, motivation; the "Layerwise" rows of the
    latency table, Table 3 of the arXiv page).

Activations are token-major (X is T x d, y_i is T x O_i): the pages write y = W X with
X as columns; both describe the same numbers.

Every input is converted to fp64 exactly; every product and sum is fp64.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np

GROUP = 128


def _np(t) -> np.ndarray:
    if hasattr(t, "detach"):
        t = t.detach().cpu()
        if str(t.dtype) == "torch.float16":
            return t.numpy()
        return t.numpy()
    return np.asarray(t)


def _f64(t) -> np.ndarray:
    return _np(t).astype(np.float64)


# --------------------------------------------------------------------------- format
def unpack_int4(q_packed, n_out: int, k_in: int) -> np.ndarray:
    """Canonical packed words -> uint8 [n_out][k_in].

    Word w of row o holds q[o][8w + j] in bits 4j..4j+3 (low nibble first)."""
    words = _np(q_packed).astype(np.int64) & 0xFFFFFFFF
    assert words.shape == (n_out, k_in // 8), words.shape
    out = np.empty((n_out, k_in // 8, 8), dtype=np.uint8)
    for j in range(8):
        out[:, :, j] = (words >> (4 * j)) & 0xF
    return out.reshape(n_out, k_in)


def dequant(q_packed, s, z, n_out: int, k_in: int) -> np.ndarray:
    """W_hat = (q - z) * s per 128-input group, in fp64 (exact: |q - z| < 2^12 and s has an
    11-bit significand, so the product has at most 24 significant bits)."""
    q = unpack_int4(q_packed, n_out, k_in).astype(np.float64)
    s64 = _f64(s)
    z64 = _f64(z)
    assert s64.shape == (n_out, k_in // GROUP) and z64.shape == s64.shape
    g = np.arange(k_in) // GROUP
    return (q - z64[:, g]) * s64[:, g]


def dequant_qw(qw) -> np.ndarray:
    """Dequantise a workload QuantWeight-like object (q_packed, s, z, n_out, k_in)."""
    if getattr(qw, "fmt", "int4") != "int4":
        return dequant_mx(qw.codes, qw.scales, qw.fmt, qw.n_out, qw.k_in)
    return dequant(qw.q_packed, qw.s, qw.z, qw.n_out, qw.k_in)


# --------------------------------------------------------------------------- MX weights
# GlowQ on microscaling weight formats (GlowQ arXiv page, Table 13: MXFP4 and MXFP6 rows,
# quantised alone and with the correction).  The formats themselves are those of the OCP
# Microscaling (MX) Formats specification v1.0: blocks of 32 consecutive elements along a row
# share one E8M0 scale 2^(S - 127) (S = 255 encodes NaN); an element is a sign bit, ebits
# exponent bits and mbits mantissa bits with the given bias, no infinities or NaNs; exponent
# field 0 is subnormal.  The pages do not say which 6-bit element MXFP6 means: both the E2M3
# and the E3M2 element are covered.
MX_BLOCK = 32
MX_ELEM = {"mxfp4": (2, 1, 1), "mxfp6_e2m3": (2, 3, 1), "mxfp6_e3m2": (3, 2, 3)}  # ebits, mbits, bias


def mx_element_value(code: int, fmt: str) -> float:
    """Value of one element code: (-1)^sign 2^(E - bias) (1 + M / 2^mbits) for E > 0,
    (-1)^sign 2^(1 - bias) (M / 2^mbits) for E = 0."""
    ebits, mbits, bias = MX_ELEM[fmt]
    nbits = 1 + ebits + mbits
    assert 0 <= code < (1 << nbits)
    sign = -1.0 if (code >> (nbits - 1)) & 1 else 1.0
    e = (code >> mbits) & ((1 << ebits) - 1)
    m = code & ((1 << mbits) - 1)
    if e == 0:
        mag = math.ldexp(m / (1 << mbits), 1 - bias)
    else:
        mag = math.ldexp(1.0 + m / (1 << mbits), e - bias)
    return sign * mag


def e8m0_value(s: int) -> float:
    """The shared scale of an MX block: 2^(s - 127); s = 255 is NaN."""
    return math.nan if s == 255 else math.ldexp(1.0, int(s) - 127)


def dequant_mx(codes, scales, fmt: str, n_out: int, k_in: int) -> np.ndarray:
    """W_hat[o, k] = element(codes[o, k]) * 2^(scales[o, k // 32] - 127) in fp64 (exact).

    codes: uint8 [n_out][k_in], one element code per byte in its low bits;
    scales: uint8 [n_out][k_in / 32], E8M0."""
    c = _np(codes).astype(np.int64)
    s = _np(scales).astype(np.int64)
    assert c.shape == (n_out, k_in) and s.shape == (n_out, k_in // MX_BLOCK), (c.shape, s.shape)
    ebits, mbits, _ = MX_ELEM[fmt]
    table = np.array([mx_element_value(v, fmt) for v in range(1 << (1 + ebits + mbits))])
    scale = np.array([e8m0_value(v) for v in range(256)])
    return table[c] * scale[s][:, np.arange(k_in) // MX_BLOCK]


# --------------------------------------------------------------------------- forward
def shared_projection(x, b) -> np.ndarray:
    """R = X B^T, fp64 [T][r] (formed once per group by the anchor)."""
    return _f64(x) @ _f64(b).T


def group_forward(x, w_hats: Sequence[np.ndarray], b, a_list: Sequence, restore: bool = True
                  ) -> List[np.ndarray]:
    """Outputs y_i = X W_hat_i^T + [restore and r > 0] (X B^T) A_i^T for every module of an
    input-sharing group (module 0 the anchor).  R is formed once and shared."""
    x64 = _f64(x)
    outs = [x64 @ wh.T for wh in w_hats]
    r = 0 if b is None else _np(b).shape[0]
    if restore and r > 0:
        R = shared_projection(x64, b)
        outs = [y + R @ _f64(a).T for y, a in zip(outs, a_list)]
    return outs


def solo_forward(x, w_hat: np.ndarray, b, a, restore: bool = True) -> np.ndarray:
    """Solo module: y = X W_hat^T + (X B^T) A^T with its private B, nothing kept."""
    return group_forward(x, [w_hat], b, [a], restore)[0]


def layerwise_forward(x, w_hats: Sequence[np.ndarray], b_list: Sequence, a_list: Sequence,
                      restore: bool = True) -> List[np.ndarray]:
    """Baseline: every module projects with its own B_i (m projections per group)."""
    return [solo_forward(x, wh, b, a, restore) for wh, b, a in zip(w_hats, b_list, a_list)]


def path_forward(layers: Dict[int, list], mask: Sequence[bool]) -> Dict[int, List[List[np.ndarray]]]:
    """Decoder-linear path: per layer, in order, the QKV group, the o_proj solo, the gate/up
    group and the down_proj solo; a layer outside the restore set runs every unit with
    restore off (GlowQ paper note, key design 4)."""
    out = {}
    for l, units in layers.items():
        res = []
        for u in units:
            w_hats = [dequant_qw(q) for q in u.weights]
            res.append(group_forward(u.x, w_hats, u.b, u.a, bool(mask[l])))
        out[l] = res
    return out


# --------------------------------------------------------------------------- W4A8
# The arXiv page (Tables 14 and 15) and the paper note's results bullets run the method with 8-bit
# activations as well ("W4A8"): the quantised weight product then takes 8-bit activations while
# the correction branch stays high precision.  The pages give no activation quantiser; this oracle
# takes the plainest one: per token (row of X), symmetric, round-to-nearest-even to the integers
# -127..127, the scale a / 127 with a = max_k |x[t, k]|.  Every step of it is fp32 (the fp16
# inputs are exact in fp32; the division and the rounding are IEEE operations), so that the
# integer codes are decided in one fixed precision; a zero row gets scale 0 and codes 0.
def quantize_x_int8(x):
    """Per-token symmetric int8 codes of fp16 activations: (codes int64 [T][d] in -127..127,
    scales fp32 [T]); x ~ scale[t] * codes[t]."""
    xf = _np(x).astype(np.float32)
    amax = np.abs(xf).max(axis=1) if xf.size else np.zeros(xf.shape[0], np.float32)
    scale = (amax.astype(np.float32) / np.float32(127.0)).astype(np.float32)
    codes = np.zeros(xf.shape, dtype=np.int64)
    nz = scale > 0
    if np.any(nz):
        ratio = (xf[nz] / scale[nz, None]).astype(np.float32)
        codes[nz] = np.clip(np.rint(ratio), -127, 127).astype(np.int64)
    return codes, scale


def group_forward_w4a8(x, w_hats: Sequence[np.ndarray], b, a_list, restore: bool = True
                       ) -> List[np.ndarray]:
    """W4A8 group forward: y_i = scale_t * (codes_t . W_hat_i^T) + [restore and r > 0]
    (X B^T) A_i^T, with (codes, scale) = quantize_x_int8(X), the quantised product in fp64
    (exact products of integers and exact weights), and the shared projection R = X B^T formed
    once from the fp16 activations (the high-precision branch)."""
    codes, scale = quantize_x_int8(x)
    xq = codes.astype(np.float64)
    sc = scale.astype(np.float64)[:, None]
    outs = [sc * (xq @ wh.T) for wh in w_hats]
    r = 0 if b is None else _np(b).shape[0]
    if restore and r > 0:
        R = shared_projection(x, b)
        outs = [y + R @ _f64(a).T for y, a in zip(outs, a_list)]
    return outs


def bruteforce_group_w4a8(x, q_packed_list, s_list, z_list, n_outs, k_in, b, a_list,
                          restore: bool = True) -> List[np.ndarray]:
    """W4A8 element by element: per token the code of every input from its own fp32 division
    and rounding, the quantised sum over groups of s * sum (q - z) * code (nibbles read from the
    packed words), times the token's scale, plus the correction; correctly rounded sums (fsum).
    Tiny shapes only."""
    xs = _np(x).astype(np.float32)
    T = xs.shape[0]
    r = 0 if b is None else _np(b).shape[0]
    R = None
    if restore and r > 0:
        bb = _f64(b)
        R = [[math.fsum(float(xs[t, k]) * float(bb[j, k]) for k in range(k_in)) for j in range(r)]
             for t in range(T)]
    codes, scales = [], []
    for t in range(T):
        amax = np.float32(0.0)
        for k in range(k_in):
            amax = max(amax, np.float32(abs(xs[t, k])))
        sc = np.float32(amax / np.float32(127.0))
        row = []
        for k in range(k_in):
            if sc == 0:
                row.append(0)
            else:
                v = float(np.rint(np.float32(xs[t, k] / sc)))
                row.append(int(min(127.0, max(-127.0, v))))
        codes.append(row)
        scales.append(float(sc))
    outs = []
    for qp, s, z, O, a in zip(q_packed_list, s_list, z_list, n_outs, a_list):
        words = _np(qp).astype(np.int64) & 0xFFFFFFFF
        s64, z64 = _f64(s), _f64(z)
        aa = None if R is None else _f64(a)
        y = np.zeros((T, O))
        for t in range(T):
            for o in range(O):
                terms = []
                for k in range(k_in):
                    q = (int(words[o, k // 8]) >> (4 * (k % 8))) & 0xF
                    g = k // GROUP
                    terms.append(scales[t] * float(s64[o, g]) * (q - float(z64[o, g])) * codes[t][k])
                if R is not None:
                    terms.extend(R[t][j] * float(aa[o, j]) for j in range(r))
                y[t, o] = math.fsum(terms)
        outs.append(y)
    return outs


# --------------------------------------------------------------------------- MX weights x MXFP8 activations
# The 8-bit-activation form of the method (arXiv page, Tables 14 and 15: W4A8) on microscaling
# weights (Table 13), with the activations in the same family: MXFP8, i.e. FP8 E4M3 elements
# sharing one E8M0 scale per 32 consecutive inputs of a token (OCP Microscaling v1.0).  The
# conversion is the specification's: the block's shared exponent is floor(log2 max|x|) minus the
# element's largest exponent (8 for E4M3, whose largest value is 1.75 * 2^8 = 448), and each
# x / 2^X becomes the nearest E4M3 value, ties to the even mantissa, saturating at 448 (a block of
# zeros gets the smallest scale, 2^-127, and zero codes).  The correction branch stays high
# precision, as for W4A8: R = X B^T from the fp16 activations.
E4M3_MAX = 448.0


def fp8_e4m3_value(code: int) -> float:
    """Value of an E4M3 code: bias 7, exponent field 0 subnormal (2^-6 * m/8); exponent field 15
    with mantissa 7 is NaN (no infinities)."""
    assert 0 <= code < 256
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return math.nan
    if e == 0:
        return sign * math.ldexp(m / 8.0, -6)
    return sign * math.ldexp(1.0 + m / 8.0, e - 7)


def quantize_x_mxfp8(x):
    """MXFP8 codes of fp16 activations: (codes uint8 [T][d], E4M3; scales uint8 [T][d/32], E8M0).
    Every step is exact: x is fp16, x / 2^X a power-of-two scaling, and the element is chosen by
    distance to each finite E4M3 magnitude."""
    xf = _f64(x)
    T, d = xf.shape
    assert d % MX_BLOCK == 0
    blocks = xf.reshape(T, d // MX_BLOCK, MX_BLOCK)
    amax = np.abs(blocks).max(axis=2) if T else np.zeros((0, d // MX_BLOCK))
    X = np.full(amax.shape, -127, dtype=np.int64)
    for idx in zip(*np.nonzero(amax)):
        X[idx] = math.frexp(float(amax[idx]))[1] - 1 - 8  # floor(log2 amax) - 8
    u = np.abs(blocks) / np.ldexp(1.0, X)[:, :, None]
    mags = np.array([fp8_e4m3_value(c) for c in range(0x7F)])  # finite non-negative values, code order
    dist = np.abs(u[..., None] - mags)
    best = dist.min(axis=-1, keepdims=True)
    tie = dist == best
    # nearest value; of two equally near ones, the even code (even mantissa)
    cand = np.where(tie, np.arange(0x7F), 1 << 20)
    even = np.where(tie & (np.arange(0x7F) % 2 == 0), np.arange(0x7F), 1 << 20)
    code = np.where(tie.sum(axis=-1) > 1, even.min(axis=-1), cand.min(axis=-1))
    code = np.where((blocks < 0) & (code > 0), code | 0x80, code)
    return code.reshape(T, d).astype(np.uint8), (X + 127).astype(np.uint8)


def dequant_mxfp8(codes, scales) -> np.ndarray:
    """fp64 values of MXFP8 activations: E4M3 element times 2^(S - 127)."""
    c = _np(codes).astype(np.int64)
    s = _np(scales).astype(np.int64)
    table = np.array([fp8_e4m3_value(v) for v in range(256)])
    return table[c] * np.ldexp(1.0, s - 127)[:, np.arange(c.shape[1]) // MX_BLOCK]


def group_forward_mx8(x, w_hats: Sequence[np.ndarray], b, a_list, restore: bool = True) -> List[np.ndarray]:
    """MX weights x MXFP8 activations: y_i = X_q W_hat_i^T + [restore and r > 0] (X B^T) A_i^T with
    X_q = dequant_mxfp8(quantize_x_mxfp8(X)) (fp64, exact products of the element values) and the
    shared projection from the fp16 activations."""
    xq = dequant_mxfp8(*quantize_x_mxfp8(x))
    outs = [xq @ wh.T for wh in w_hats]
    r = 0 if b is None else _np(b).shape[0]
    if restore and r > 0:
        R = shared_projection(x, b)
        outs = [y + R @ _f64(a).T for y, a in zip(outs, a_list)]
    return outs


# --------------------------------------------------------------------------- mixture of experts
# The arXiv page's Figures 7-9 (Qwen1.5-MoE-A2.7B) show the covariance-aligned shared basis for
# the MLP gate/up projections both aggregated over all experts (Fig. 8) and for one expert alone
# (Fig. 9).  An MoE layer routes every token to a few experts; each expert's gate and up form an
# input-sharing group over the tokens routed to it, and its down projection is a solo module on
# its own hidden rows.  Routed rows are listed grouped by expert: rows offsets[e] ..
# offsets[e + 1] - 1 belong to expert e, and row j reads token row_token[j] of X (or row j of X
# when row_token is None, as for the down projection whose input is already in routed order).
# Sharing: "expert" -- each expert e forms R_e = X_e B_e^T from its own rows with its own B_e
# (Fig. 9); "all" -- one B for every expert, R = X B^T per token, consumed by every expert that
# token is routed to (Fig. 8).
def moe_forward(x, row_token, offsets, w_hats, b, a, restore: bool = True, share: str = "expert"
                ) -> List[np.ndarray]:
    """Outputs y_i [n_rows][O_i] in routed-row order for m modules per expert.

    w_hats[e][i] is expert e's dequantised module i, a[e][i] its left factor; b[e] is expert e's
    right factor (share == "expert") or b is the one right factor of all experts (share == "all")."""
    x64 = _f64(x)
    offs = [int(v) for v in _np(offsets)]
    n_rows = offs[-1]
    rows_x = x64[np.asarray(_np(row_token), dtype=np.int64)] if row_token is not None else x64[:n_rows]
    m = len(w_hats[0])
    outs = [np.zeros((n_rows, w_hats[0][i].shape[0])) for i in range(m)]
    R_all = None
    if restore and share == "all" and b is not None and _np(b).shape[0] > 0:
        R_all = shared_projection(rows_x, b)  # per routed row: the row's token times B^T
    for e in range(len(w_hats)):
        lo, hi = offs[e], offs[e + 1]
        if hi <= lo:
            continue
        xe = rows_x[lo:hi]
        if share == "all":
            ys = group_forward(xe, w_hats[e], None, a[e], restore=False)
            if R_all is not None:
                ys = [y + R_all[lo:hi] @ _f64(ai).T for y, ai in zip(ys, a[e])]
        else:
            ys = group_forward(xe, w_hats[e], b[e] if restore else None, a[e], restore=restore)
        for i in range(m):
            outs[i][lo:hi] = ys[i]
    return outs


# --------------------------------------------------------------------------- brute force
def bruteforce_group(x, q_packed_list, s_list, z_list, n_outs, k_in, b, a_list,
                     restore: bool = True) -> List[np.ndarray]:
    """Element-by-element loops with correctly rounded sums (math.fsum); each nibble is
    read straight from its packed word.  For tiny shapes only."""
    xs = _f64(x)
    T = xs.shape[0]
    r = 0 if b is None else _np(b).shape[0]
    R = None
    if restore and r > 0:
        bb = _f64(b)
        R = [[math.fsum(float(xs[t, k]) * float(bb[j, k]) for k in range(k_in)) for j in range(r)]
             for t in range(T)]
    outs = []
    for qp, s, z, O, a in zip(q_packed_list, s_list, z_list, n_outs, a_list):
        words = _np(qp).astype(np.int64) & 0xFFFFFFFF
        s64, z64 = _f64(s), _f64(z)
        aa = None if R is None else _f64(a)
        y = np.zeros((T, O))
        for t in range(T):
            for o in range(O):
                terms = []
                for k in range(k_in):
                    q = (int(words[o, k // 8]) >> (4 * (k % 8))) & 0xF
                    g = k // GROUP
                    terms.append(float(xs[t, k]) * ((q - float(z64[o, g])) * float(s64[o, g])))
                if R is not None:
                    terms.extend(R[t][j] * float(aa[o, j]) for j in range(r))
                y[t, o] = math.fsum(terms)
        outs.append(y)
    return outs


# --------------------------------------------------------------------------- comparison
def parity_errors(y_test, y_ref) -> Dict[str, float]:
    """The two measures of the parity bar, per module output:

      rel_fro     = ||y_test - y_ref||_F / ||y_ref||_F
      max_abs_rel = max_elem |y_test - y_ref| / max_elem |y_ref|

    Both are normalised by the reference alone.  A zero reference makes the bound an
    equality: the measure is 0 when y_test equals it and inf otherwise (likewise for empty
    outputs, which are equal)."""
    yt = _f64(y_test)
    yr = _f64(y_ref)
    assert yt.shape == yr.shape, (yt.shape, yr.shape)
    diff = np.abs(yt - yr)
    if diff.size == 0:
        return dict(rel_fro=0.0, max_abs_rel=0.0)
    dfro = float(np.sqrt(np.sum(diff * diff)))
    dmax = float(diff.max())
    nref = float(np.sqrt(np.sum(yr * yr)))
    mref = float(np.abs(yr).max())

    def ratio(num, den):
        if den > 0:
            return num / den
        return 0.0 if num == 0 else math.inf

    return dict(rel_fro=ratio(dfro, nref), max_abs_rel=ratio(dmax, mref))
