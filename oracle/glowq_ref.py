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
    return dequant(qw.q_packed, qw.s, qw.z, qw.n_out, qw.k_in)


# --------------------------------------------------------------------------- forward
def base_product(x, w_hat: np.ndarray) -> np.ndarray:
    """Y0 = X W_hat^T, fp64 [T][O]."""
    return _f64(x) @ w_hat.T


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


def unit_forward(unit, layerwise: bool = False) -> List[np.ndarray]:
    """Forward of a workload Unit (group or solo) through the definitions above."""
    w_hats = [dequant_qw(q) for q in unit.weights]
    if layerwise and unit.kind == "group":
        return layerwise_forward(unit.x, w_hats, unit.b_layerwise, unit.a, unit.restore)
    return group_forward(unit.x, w_hats, unit.b, unit.a, unit.restore)


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
    """Relative Frobenius error and max-abs error relative to max|y_ref|."""
    yt = _f64(y_test)
    yr = _f64(y_ref)
    diff = yt - yr
    nref = float(np.linalg.norm(yr))
    mref = float(np.abs(yr).max()) if yr.size else 0.0
    return dict(
        rel_fro=float(np.linalg.norm(diff)) / nref if nref > 0 else float(np.linalg.norm(diff)),
        max_abs_rel=float(np.abs(diff).max()) / mref if (mref > 0 and diff.size) else 0.0,
    )
