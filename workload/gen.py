"""Seeded synthetic workloads for the GlowQ group-shared low-rank correction path.

This module draws every random input that both the fp64 oracle (``oracle/``) and the
HIP library consume: activations X with a power-law covariance spectrum, fp16 weights
with outlier input columns, the round-to-nearest INT4-g128 base quantisation of those
weights (packed in the library's canonical nibble format) or their microscaling (MXFP4 /
MXFP6) quantisation, seeded Gaussian low-rank
factors rescaled to the size of the quantisation error, and the GlowQ-S restore mask.

It holds none of the correction method's arithmetic: no shared projection, no
correction epilogue and no factor solve (the whitened SVD that yields exact factors
lives in the oracle).  The base quantiser here is the W4A16 "INT4, g128" weight format
that the correction is applied on top of (GlowQ paper note, "Experimental setup";
GlowQ arXiv page, Table 1 header "INT4, g128"); its rounding rules (half-to-even, zero
point from the fp16 scale, q clipped to 0..15, z not clamped) are this recipe's reading of
that format.

All functions take a ``device`` so that large workloads can be drawn directly on the
GPU (random streams then differ from the CPU ones; both sides of a parity test always
read the same tensors).
"""
from __future__ import annotations

import functools
import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

GROUP = 128  # inputs per quantisation group (INT4 "g128")

# stable integer codes for seed keys
KIND = {"x": 1, "w": 2, "outlier": 3, "a": 4, "b": 5, "basis": 6, "mask": 7, "z": 8, "route": 9}


def seed_of(*keys: int) -> int:
    """64-bit seed from a tuple of non-negative integer keys (numpy SeedSequence)."""
    ss = np.random.SeedSequence([int(k) for k in keys])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def generator(device, *keys: int) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(seed_of(*keys))
    return g


# ----------------------------------------------------------------------------------
# activations: rows ~ N(0, Sigma_x), Sigma_x = Q diag(lam) Q^T, lam_k ∝ k^-alpha
# (GlowQ paper note, key design 2: input covariance spectra decay as a power law with
#  exponent about 0.77 for MLP inputs and 1.19 for QKV inputs; GlowQ arXiv page, Fig. 2)
# ----------------------------------------------------------------------------------
def powerlaw_spectrum(d: int, alpha: float) -> torch.Tensor:
    """lam_k = k^-alpha for k = 1..d, rescaled so that sum(lam) = d (fp64, CPU)."""
    k = torch.arange(1, d + 1, dtype=torch.float64)
    lam = k.pow(-alpha)
    return lam * (d / lam.sum())


@functools.lru_cache(maxsize=8)
def _haar_basis_cpu(d: int, seed: int, dtype_name: str) -> torch.Tensor:
    dtype = getattr(torch, dtype_name)
    g = torch.Generator().manual_seed(seed)
    a = torch.randn(d, d, generator=g, dtype=dtype)
    q, r = torch.linalg.qr(a)
    sgn = torch.sign(torch.diagonal(r))
    sgn[sgn == 0] = 1
    return (q * sgn.unsqueeze(0)).contiguous()


def haar_basis(d: int, *keys: int) -> torch.Tensor:
    """Seeded Haar-random orthogonal d x d matrix (QR of a Gaussian, column signs fixed
    by sign(diag R)).  fp64 for d <= 4096, fp32 above (only the activation distribution
    depends on it).  Always built on the CPU and cached per process."""
    return _haar_basis_cpu(d, seed_of(*keys), "float64" if d <= 4096 else "float32")


def make_x(T: int, d: int, alpha: float, keys: Sequence[int], device="cpu",
           basis: Optional[torch.Tensor] = None, lam: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp16 [T][d]: fp16_RNE(Z diag(sqrt lam) Q^T), Z ~ N(0,1)."""
    if lam is None:
        lam = powerlaw_spectrum(d, alpha)
    if basis is None:
        basis = haar_basis(d, *keys, KIND["basis"])
    g = generator(device, *keys, KIND["x"])
    z = torch.randn(T, d, generator=g, device=device, dtype=torch.float32)
    dt = basis.dtype
    zs = z.to(dt) * lam.to(device=device, dtype=dt).sqrt().unsqueeze(0)
    x = zs @ basis.to(device).t()
    return x.to(torch.float16).contiguous()


# ----------------------------------------------------------------------------------
# weights: W ~ N(0, 0.02^2), four outlier input columns x10, rounded to fp16
# ----------------------------------------------------------------------------------
def outlier_columns(d: int, keys: Sequence[int], n: int = 4) -> torch.Tensor:
    g = generator("cpu", *keys, KIND["outlier"])
    return torch.randperm(d, generator=g)[:n].sort().values


def make_w(O: int, d: int, keys: Sequence[int], cols: torch.Tensor, device="cpu",
           std: float = 0.02, outlier_gain: float = 10.0) -> torch.Tensor:
    g = generator(device, *keys, KIND["w"])
    w = torch.randn(O, d, generator=g, device=device, dtype=torch.float32) * std
    if cols.numel():
        w[:, cols.to(device)] *= outlier_gain
    return w.to(torch.float16).contiguous()


# ----------------------------------------------------------------------------------
# base quantiser: asymmetric round-to-nearest INT4 per 128-input group
#   s = fp16_RNE((max - min) / 15), z = RNE(-min / s), q = clip(RNE(w / s) + z, 0, 15)
# (RNE = round half to even; z from the fp16-rounded s; z is not clamped)
# ----------------------------------------------------------------------------------
@dataclass
class QuantWeight:
    q: torch.Tensor        # uint8 [O][d], values 0..15
    s: torch.Tensor        # fp16 [O][d/128]
    z: torch.Tensor        # fp16 [O][d/128], integer valued
    q_packed: torch.Tensor  # int32 [O][d/8], canonical nibble packing
    err_sq: float          # ||W - W_hat||_F^2 (fp64)
    w_sq: float            # ||W||_F^2 (fp64)

    @property
    def n_out(self) -> int:
        return int(self.q.shape[0])

    @property
    def k_in(self) -> int:
        return int(self.q.shape[1])


def rtn_quantize(w: torch.Tensor) -> QuantWeight:
    O, d = w.shape
    assert d % GROUP == 0
    wg = w.to(torch.float64).reshape(O, d // GROUP, GROUP)
    mn = wg.amin(dim=2)
    mx = wg.amax(dim=2)
    s = ((mx - mn) / 15.0).to(torch.float16).to(torch.float64)
    degenerate = s == 0
    s = torch.where(degenerate, torch.ones_like(s), s)
    z = torch.round(-mn / s)
    q = torch.clamp(torch.round(wg / s.unsqueeze(2)) + z.unsqueeze(2), 0, 15)
    w_hat = (q - z.unsqueeze(2)) * s.unsqueeze(2)
    err_sq = float(((wg - w_hat) ** 2).sum())
    w_sq = float((wg ** 2).sum())
    q8 = q.reshape(O, d).to(torch.uint8).contiguous()
    return QuantWeight(q=q8, s=s.to(torch.float16).contiguous(), z=z.to(torch.float16).contiguous(),
                       q_packed=pack_canonical(q8), err_sq=err_sq, w_sq=w_sq)


MX_BLOCK = 32
# element formats (exponent bits, mantissa bits, bias) of the OCP MX v1.0 specification
MX_FORMATS = {"mxfp4": (2, 1, 1), "mxfp6_e2m3": (2, 3, 1), "mxfp6_e3m2": (3, 2, 3)}
# block exponents X for which every element times 2^X is an exact fp16 (the device layout's
# range): the finest element step times 2^X must reach 2^-24, the largest element must stay
# below 65520
MX_EXP_RANGE = {"mxfp4": (-23, 13), "mxfp6_e2m3": (-21, 13), "mxfp6_e3m2": (-20, 11)}


@dataclass
class MxWeight:
    fmt: str
    codes: torch.Tensor    # uint8 [O][d], one element code per byte (low 4 or 6 bits)
    scales: torch.Tensor   # uint8 [O][d/32], E8M0 biased block exponents
    err_sq: float          # ||W - W_hat||_F^2 (fp64)
    w_sq: float            # ||W||_F^2 (fp64)

    @property
    def n_out(self) -> int:
        return int(self.codes.shape[0])

    @property
    def k_in(self) -> int:
        return int(self.codes.shape[1])


def floor_log2(v: torch.Tensor) -> torch.Tensor:
    """floor(log2 v) of positive fp64 values, exactly (from the binary exponent; a device log2 may
    land just below an integer at powers of two); 0 where v == 0."""
    _, e = torch.frexp(v)
    return torch.where(v > 0, (e - 1).to(v.dtype), torch.zeros_like(v))


def pow2(e: torch.Tensor) -> torch.Tensor:
    """2^e in fp64 for integer-valued e in the normal range, exactly (built from the exponent bits;
    a device pow is not always exact)."""
    return ((e.to(torch.int64) + 1023) << 52).view(torch.float64)


def mx_quantize(w: torch.Tensor, fmt: str) -> MxWeight:
    """Microscaling quantisation of the generated weights (the conversion of the OCP MX v1.0
    specification): per block of 32 inputs the shared exponent is floor(log2 max|w|) minus the
    element's largest exponent, kept inside MX_EXP_RANGE (an all-zero block takes the range's
    low end); each w / 2^X is rounded to the nearest element, ties to the even mantissa,
    saturating at the largest element.  Runs in fp64 on w's device; codes and scales are
    returned on the CPU."""
    eb, mb, bias = MX_FORMATS[fmt]
    lo, hi = MX_EXP_RANGE[fmt]
    emax = (1 << eb) - 1 - bias
    emin = 1 - bias
    top = math.ldexp(2.0 - 2.0 ** -mb, emax)
    O, d = w.shape
    assert d % MX_BLOCK == 0
    wb = w.detach().to(torch.float64).reshape(O, d // MX_BLOCK, MX_BLOCK)
    amax = wb.abs().amax(dim=2)
    X = torch.where(amax > 0, floor_log2(amax) - emax, torch.full_like(amax, float(lo))).clamp(lo, hi)
    u = wb.abs() / pow2(X).unsqueeze(2)
    k = floor_log2(u).clamp(emin, emax)  # below the normal range the step is the subnormal one
    step = pow2(k - mb)
    mag = torch.minimum(torch.round(u / step) * step, torch.tensor(top, dtype=torch.float64, device=wb.device))
    # encode: subnormal when below 2^emin, else exponent field and mantissa of the magnitude
    sub = mag < math.ldexp(1.0, emin)
    kk = floor_log2(torch.where(sub, 1.0, mag))
    e_field = torch.where(sub, torch.zeros_like(kk), kk + bias)
    m_field = torch.where(sub, mag / math.ldexp(1.0, emin - mb), (mag / pow2(kk) - 1.0) * (1 << mb))
    assert bool(torch.all(m_field == torch.round(m_field))) and bool(torch.all(m_field < (1 << mb)))
    sign = (wb < 0) & (mag > 0)
    codes = (sign.to(torch.int64) << (eb + mb)) | (e_field.to(torch.int64) << mb) | m_field.to(torch.int64)
    w_hat = torch.where(sign, -mag, mag) * pow2(X).unsqueeze(2)
    err_sq = float(((wb - w_hat) ** 2).sum())
    w_sq = float((wb ** 2).sum())
    return MxWeight(fmt=fmt, codes=codes.reshape(O, d).to(torch.uint8).cpu().contiguous(),
                    scales=(X + 127).to(torch.uint8).cpu().contiguous(), err_sq=err_sq, w_sq=w_sq)


def pack_canonical(q: torch.Tensor) -> torch.Tensor:
    """uint8 [O][d] (0..15) -> int32 [O][d/8]; nibble j (bits 4j..4j+3) of word w holds
    q[o][8w + j] (low nibble first).  The int32 holds the uint32 bit pattern."""
    O, d = q.shape
    assert d % 8 == 0
    v = q.to(torch.int64).reshape(O, d // 8, 8)
    shifts = torch.arange(0, 32, 4, device=q.device, dtype=torch.int64)
    word = (v << shifts).sum(dim=2)  # < 2^32
    word = torch.where(word >= 2 ** 31, word - 2 ** 32, word)
    return word.to(torch.int32).contiguous()


# ----------------------------------------------------------------------------------
# seeded Gaussian factors rescaled so that ||A_i B||_F = ||E_i||_F
# ----------------------------------------------------------------------------------
def gaussian_factors(n_outs: Sequence[int], d: int, r: int, err_sq: Sequence[float],
                     keys: Sequence[int], device="cpu", per_module_b: bool = False):
    """Returns (A list fp16 [O_i][r], B fp16 [r][d]) or, with per_module_b, a list of B_i.
    B <- B / sqrt(d); A_i <- A_i * ||E_i||_F / ||A_i B||_F (product norm in fp64)."""
    def draw_b(tag):
        gb = generator(device, *keys, KIND["b"], tag)
        return torch.randn(r, d, generator=gb, device=device, dtype=torch.float64) / math.sqrt(d)

    b_shared = draw_b(0)
    A, Bs = [], []
    for i, (O, e2) in enumerate(zip(n_outs, err_sq)):
        b = draw_b(1 + i) if per_module_b else b_shared
        ga = generator(device, *keys, KIND["a"], i)
        a = torch.randn(O, r, generator=ga, device=device, dtype=torch.float64)
        # ||A B||_F^2 = sum((A^T A) * (B B^T))
        nrm2 = float(((a.t() @ a) * (b @ b.t())).sum())
        scale = math.sqrt(e2 / nrm2) if nrm2 > 0 else 0.0
        A.append((a * scale).to(torch.float16).contiguous())
        Bs.append(b.to(torch.float16).contiguous())
    if per_module_b:
        return A, Bs
    return A, Bs[0]


def restore_mask(n_units: int, n_restore: int, keys: Sequence[int]) -> List[bool]:
    """GlowQ-S restore set drawn from a seeded score: one uniform score per unit, the
    n_restore highest are restored; equal scores go to the lower index."""
    g = generator("cpu", *keys, KIND["mask"])
    score = torch.rand(n_units, generator=g, dtype=torch.float64)
    order = sorted(range(n_units), key=lambda u: (-float(score[u]), u))
    chosen = set(order[:n_restore])
    return [u in chosen for u in range(n_units)]


def moe_routing(T: int, n_exp: int, top_k: int, keys: Sequence[int], skip: Sequence[int] = ()):
    """Top-k routing of T tokens to n_exp experts from seeded uniform scores (experts in `skip`
    receive no token), listed grouped by expert and, within an expert, by token:
    (row_token int32 [T top_k], offsets int32 [n_exp + 1])."""
    g = generator("cpu", *keys, KIND["route"])
    score = torch.rand(T, n_exp, generator=g, dtype=torch.float64)
    if len(skip):
        score[:, list(skip)] = -1.0
    top = torch.topk(score, top_k, dim=1).indices  # distinct experts per token
    pairs = sorted((int(top[t, k]), t) for t in range(T) for k in range(top_k))
    row_token = torch.tensor([t for _, t in pairs], dtype=torch.int32)
    counts = torch.bincount(torch.tensor([e for e, _ in pairs], dtype=torch.int64), minlength=n_exp)
    offsets = torch.zeros(n_exp + 1, dtype=torch.int32)
    offsets[1:] = torch.cumsum(counts, 0).to(torch.int32)
    return row_token, offsets


# ----------------------------------------------------------------------------------
# workload descriptions
# ----------------------------------------------------------------------------------
@dataclass
class Unit:
    """One call of the path: an input-sharing group (m >= 1 modules with one shared B,
    module 0 the anchor) or a solo module (m == 1, private B)."""
    name: str
    kind: str                 # "group" | "solo"
    x: torch.Tensor           # fp16 [T][d]
    weights: List[QuantWeight]
    a: List[torch.Tensor]     # fp16 [O_i][r]
    b: torch.Tensor           # fp16 [r][d]
    r: int
    restore: bool = True
    b_layerwise: Optional[List[torch.Tensor]] = None  # per-module B_i for the baseline
    extra: Dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return int(self.x.shape[0])

    @property
    def d(self) -> int:
        return int(self.x.shape[1])

    @property
    def n_outs(self) -> List[int]:
        return [w.n_out for w in self.weights]


def make_unit(name: str, kind: str, x: torch.Tensor, n_outs: Sequence[int], r: int,
              keys: Sequence[int], device="cpu", restore: bool = True,
              layerwise: bool = False, w_override: Optional[List[torch.Tensor]] = None,
              fmt: str = "int4") -> Unit:
    d = x.shape[1]
    cols = outlier_columns(d, keys)  # shared by the modules of one group (an input property)
    weights = []
    for i, O in enumerate(n_outs):
        w = w_override[i] if w_override is not None else make_w(O, d, list(keys) + [i], cols, device)
        weights.append(rtn_quantize(w) if fmt == "int4" else mx_quantize(w, fmt))
    a, b = gaussian_factors(n_outs, d, r, [q.err_sq for q in weights], keys, device)
    b_lw = None
    if layerwise:
        _, b_lw = gaussian_factors(n_outs, d, r, [q.err_sq for q in weights], keys, device,
                                   per_module_b=True)
    return Unit(name=name, kind=kind, x=x, weights=weights, a=a, b=b, r=r, restore=restore,
                b_layerwise=b_lw)


ALPHA_QKV = 1.19
ALPHA_MLP = 0.77


def tiny_qkv_inputs(device="cpu"):
    """Tiny QKV group, d = 256, 3 x 256 outputs, T = 8, r = 16.  Returns the fp16
    weights before quantisation, the quantised weights, X and the covariance (Q, lam)
    so that exact whitened factors can be solved by the caller."""
    keys = (0, 0, 0, 0)
    d, T = 256, 8
    lam = powerlaw_spectrum(d, ALPHA_QKV)
    Q = haar_basis(d, *keys, KIND["basis"])
    x = make_x(T, d, ALPHA_QKV, keys, device, basis=Q, lam=lam)
    cols = outlier_columns(d, keys)
    w16 = [make_w(256, d, list(keys) + [i], cols, device) for i in range(3)]
    qw = [rtn_quantize(w) for w in w16]
    return dict(x=x, w16=w16, qw=qw, Q=Q, lam=lam, r=16, d=d, T=T)


def llama2_qkv_unit(T: int, device="cpu", layerwise=False, fmt: str = "int4") -> Unit:
    keys = (0, 1, 0, 0)
    x = make_x(T, 4096, ALPHA_QKV, keys, device)
    return make_unit("qkv", "group", x, [4096, 4096, 4096], 64, keys, device, layerwise=layerwise, fmt=fmt)


def llama2_gateup_unit(T: int = 2048, device="cpu", layerwise=False, fmt: str = "int4") -> Unit:
    keys = (0, 2, 0, 0)
    x = make_x(T, 4096, ALPHA_MLP, keys, device)
    return make_unit("gateup", "group", x, [11008, 11008], 64, keys, device, layerwise=layerwise, fmt=fmt)


LLAMA2_7B = dict(d=4096, inter=11008, n_layers=32)


# The modules of layer l of the 32-layer path: (unit index, unit name, kind, n_outs, d_in); module i
# of unit u draws its fp16 weight from the keys (0, 3, l, u, i) with the unit's outlier columns.
LLAMA2_PATH_UNITS = [(0, "qkv", "group", [4096] * 3, 4096), (1, "o_proj", "solo", [4096], 4096),
                     (2, "gateup", "group", [11008] * 2, 4096), (3, "down_proj", "solo", [4096], 11008)]


def llama2_path_weights(l: int, device="cpu") -> List[torch.Tensor]:
    """The fp16 weights of layer l's seven modules in unit order (q, k, v, o, gate, up, down), as
    llama2_path_inputs draws them (for restore scores that need W itself)."""
    out = []
    for u, _, _, n_outs, d_in in LLAMA2_PATH_UNITS:
        keys = (0, 3, l, u)
        cols = outlier_columns(d_in, keys)
        out += [make_w(O, d_in, list(keys) + [i], cols, device) for i, O in enumerate(n_outs)]
    return out


def llama2_path_inputs(T: int, device="cpu", layers: Optional[Sequence[int]] = None, r: int = 64,
                       layerwise=False, mask: Optional[Sequence[bool]] = None):
    """32-layer LLaMA-2-7B linear path.  One activation per input kind, shared by all
    layers (the layers are not chained).  Returns (units per layer, mask per layer).  Without a
    given mask the restore set is the seeded one of restore_mask (16 of 32 layers)."""
    d, inter, L = LLAMA2_7B["d"], LLAMA2_7B["inter"], LLAMA2_7B["n_layers"]
    x_attn = make_x(T, d, ALPHA_QKV, (0, 3, 100, 0), device)
    x_o = make_x(T, d, ALPHA_QKV, (0, 3, 101, 0), device)
    x_mlp = make_x(T, d, ALPHA_MLP, (0, 3, 102, 0), device)
    x_down = make_x(T, inter, ALPHA_MLP, (0, 3, 103, 0), device)
    mask = restore_mask(L, 16, (0, 3, 0, 0)) if mask is None else [bool(v) for v in mask]
    xs = {0: x_attn, 1: x_o, 2: x_mlp, 3: x_down}
    layers = range(L) if layers is None else layers
    out = {}
    for l in layers:
        rs = mask[l]
        out[l] = [make_unit(name, kind, xs[u], n_outs, r, (0, 3, l, u), device, rs, layerwise)
                  for u, name, kind, n_outs, _ in LLAMA2_PATH_UNITS]
    return out, mask


def llama3_gqa_units(T: int, r: int, device="cpu", layerwise=False, which=("qkv", "gateup", "down")):
    """LLaMA-3.1-8B GQA shapes: QKV 4096 -> 4096 + 1024 + 1024, gate/up 4096 -> 2 x 14336,
    solo down 14336 -> 4096."""
    units = []
    if "qkv" in which:
        x = make_x(T, 4096, ALPHA_QKV, (0, 4, 0, 0), device)
        units.append(make_unit("qkv", "group", x, [4096, 1024, 1024], r, (0, 4, 0, r), device,
                               layerwise=layerwise))
    if "gateup" in which:
        x = make_x(T, 4096, ALPHA_MLP, (0, 4, 1, 0), device)
        units.append(make_unit("gateup", "group", x, [14336, 14336], r, (0, 4, 1, r), device,
                               layerwise=layerwise))
    if "down" in which:
        x = make_x(T, 14336, ALPHA_MLP, (0, 4, 2, 0), device)
        units.append(make_unit("down_proj", "solo", x, [4096], r, (0, 4, 2, r), device,
                               layerwise=layerwise))
    return units
