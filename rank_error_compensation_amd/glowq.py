"""Thin ctypes binding of libglowq (include/glowq.h).

Argument marshalling only: every step of the path runs in the library's HIP kernels.  torch is
used for device memory and the current stream (plumbing); tensors are passed as raw pointers.
There is no fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libglowq.so")

OK = 0
ERR_INVALID_ARG = -1
ERR_SHAPE = -2
ERR_ALIGN = -3
ERR_UNSUPPORTED = -4
ERR_WORKSPACE = -5
ERR_HIP = -6
ERR_RANGE = -7
ERR_HANDOFF = -8
ERR_ROUTING = -9
MOE_SHARE_EXPERT = 0
MOE_SHARE_ALL = 1
FMT_INT4_G128 = 0
FMT_MXFP4 = 1
FMT_MXFP6_E2M3 = 2
FMT_MXFP6_E3M2 = 3
FORMATS = {"int4": FMT_INT4_G128, "mxfp4": FMT_MXFP4, "mxfp6_e2m3": FMT_MXFP6_E2M3, "mxfp6_e3m2": FMT_MXFP6_E3M2}

DTYPE_F32 = 0
DTYPE_F16 = 1
UNIT_GROUP = 0
UNIT_SOLO = 1
MAX_MODULES = 8

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t


class QWeightC(ctypes.Structure):
    _fields_ = [("q", _vp), ("sz", _vp), ("n_out", _i64), ("k_in", _i64), ("format", _i32), ("reserved", _i32)]


class MoeModuleC(ctypes.Structure):
    _fields_ = [("q", _vp), ("sz", _vp), ("a", _vp), ("y", _vp), ("n_out", _i64), ("k_in", _i64)]


class UnitC(ctypes.Structure):
    _fields_ = [("kind", _i32), ("m", _i32), ("x", _vp), ("T", _i64), ("d", _i64),
                ("w", ctypes.POINTER(QWeightC)), ("b", _vp), ("a", ctypes.POINTER(_vp)),
                ("r", _i32), ("restore", _i32), ("y", ctypes.POINTER(_vp))]


EXPORTS = {
    "glowq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "glowq_version": (ctypes.c_int, []),
    "glowq_q_bytes": (_sz, [_i64, _i64]),
    "glowq_sz_bytes": (_sz, [_i64, _i64]),
    "glowq_repack": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp]),
    "glowq_mx_q_bytes": (_sz, [_i32, _i64, _i64]),
    "glowq_repack_mx": (ctypes.c_int, [_i32, _vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp]),
    "glowq_dequant": (ctypes.c_int, [ctypes.POINTER(QWeightC), _vp, _i32, _vp]),
    "glowq_workspace_bytes": (_sz, [_i64, _i32, _i32]),
    "glowq_workspace_init": (ctypes.c_int, [_vp, _sz, _vp]),
    "glowq_workspace_status": (ctypes.c_int, [_vp, _sz, _vp]),
    "glowq_group_forward": (ctypes.c_int, [_vp, _i64, _i64, _i32, ctypes.POINTER(QWeightC), _vp,
                                           ctypes.POINTER(_vp), _i32, _i32, _vp, _sz,
                                           ctypes.POINTER(_vp), _vp]),
    "glowq_static_scratch_bytes": (_sz, []),
    "glowq_group_forward_static": (ctypes.c_int, [_vp, _i64, _i64, _i32, ctypes.POINTER(QWeightC), _vp,
                                                  ctypes.POINTER(_vp), _i32, _i32, ctypes.POINTER(_vp), _vp]),
    "glowq_w4a8_workspace_bytes": (_sz, [_i64, _i64, _i32]),
    "glowq_mx8_workspace_bytes": (_sz, [_i64, _i64, _i32]),
    "glowq_group_forward_w4a8": (ctypes.c_int, [_vp, _i64, _i64, _i32, ctypes.POINTER(QWeightC), _vp,
                                                ctypes.POINTER(_vp), _i32, _i32, _vp, _sz, ctypes.POINTER(_vp), _vp]),
    "glowq_group_forward_mx8": (ctypes.c_int, [_vp, _i64, _i64, _i32, ctypes.POINTER(QWeightC), _vp,
                                                ctypes.POINTER(_vp), _i32, _i32, _vp, _sz, ctypes.POINTER(_vp), _vp]),
    "glowq_moe_workspace_bytes": (_sz, [_i64, _i64, _i32, _i32]),
    "glowq_moe_forward": (ctypes.c_int, [_vp, _i64, _i64, _i32, _i32, ctypes.POINTER(MoeModuleC), _vp, _i32, _i32,
                                         _i32, _vp, _vp, _i64, _vp, _sz, _vp]),
    "glowq_solo_forward": (ctypes.c_int, [_vp, _i64, _i64, ctypes.POINTER(QWeightC), _vp, _vp, _i32,
                                          _i32, _vp, _sz, _vp, _vp]),
    "glowq_layerwise_forward": (ctypes.c_int, [_vp, _i64, _i64, _i32, ctypes.POINTER(QWeightC),
                                               ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i32, _i32,
                                               _vp, _sz, ctypes.POINTER(_vp), _vp]),
    "glowq_path_forward": (ctypes.c_int, [ctypes.POINTER(UnitC), _i32, _vp, _sz, _vp]),
    "glowq_ner_workspace_bytes": (_sz, [_i64]),
    "glowq_ner_sums": (ctypes.c_int, [_vp, ctypes.POINTER(QWeightC), _vp, _sz, _vp, _vp]),
    "glowq_ner_sums_batch": (ctypes.c_int, [_i32, ctypes.POINTER(_vp), ctypes.POINTER(QWeightC), _vp, _sz,
                                            _vp, _vp]),
    "glowq_restore_topk": (ctypes.c_int, [_vp, _i32, _i32, _i32, _vp, _vp, _vp]),
    "glowq_restore_select": (ctypes.c_int, [_vp, _i32, _i32, _i32, ctypes.c_double, _vp, _vp, _vp]),
    "glowq_second_moment_workspace_bytes": (_sz, [_i64, _i64]),
    "glowq_second_moment": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _sz, _vp]),
    "glowq_solve_workspace_bytes": (_sz, [_i64, _i64, _i32, _i32]),
    "glowq_solve_factors": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz,
                                           _vp]),
    "glowq_ec_score_workspace_bytes": (_sz, [_i64, _i64]),
    "glowq_ec_score": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _i32, _vp, _vp, _sz, _vp]),
}

_lib = None


def lib():
    """Load libglowq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build the HIP library first "
                               "(python -m rank_error_compensation_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


class GlowQError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {lib().glowq_status_string(status).decode()} ({status})")


def check(status: int, what: str) -> None:
    if status != OK:
        raise GlowQError(status, what)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# --------------------------------------------------------------------------- weights
@dataclass
class QWeight:
    """One module (INT4-g128 or MX) in the library's device layout."""
    q: torch.Tensor     # uint8, glowq_q_bytes (MX: glowq_mx_q_bytes)
    sz: torch.Tensor    # uint8, glowq_sz_bytes
    n_out: int
    k_in: int
    fmt: int = FMT_INT4_G128

    def c(self) -> QWeightC:
        return QWeightC(self.q.data_ptr(), self.sz.data_ptr(), self.n_out, self.k_in, self.fmt, 0)

    @staticmethod
    def from_mx(fmt, codes: torch.Tensor, scales: torch.Tensor, device=None, stream=None) -> "QWeight":
        """Repack MX codes (uint8 [n_out][k_in], one code per byte) and E8M0 scales (uint8
        [n_out][k_in/32]) into the device layout (glowq_repack_mx; synchronises the stream)."""
        device = device or torch.device("cuda")
        f = FORMATS[fmt] if isinstance(fmt, str) else int(fmt)
        n_out, k_in = codes.shape
        c = codes.to(device=device, dtype=torch.uint8).contiguous()
        s = scales.to(device=device, dtype=torch.uint8).contiguous()
        L = lib()
        qb, zb = L.glowq_mx_q_bytes(f, n_out, k_in), L.glowq_sz_bytes(n_out, k_in)
        if qb == 0 or zb == 0:
            raise GlowQError(ERR_SHAPE, "glowq_mx_q_bytes")
        q_dev = torch.empty(qb, dtype=torch.uint8, device=device)
        sz_dev = torch.empty(zb, dtype=torch.uint8, device=device)
        flag = torch.empty(1, dtype=torch.int32, device=device)
        check(L.glowq_repack_mx(f, _ptr(c), _ptr(s), n_out, k_in, _ptr(q_dev), _ptr(sz_dev), _ptr(flag),
                                _stream(stream)), "glowq_repack_mx")
        return QWeight(q_dev, sz_dev, int(n_out), int(k_in), f)

    @staticmethod
    def from_canonical(q_packed: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
                       device=None, stream=None) -> "QWeight":
        """Repack canonical (q_packed int32 [n_out][k_in/8], scales/zeros fp16 [n_out][k_in/128])
        into the device layout (glowq_repack; synchronises the stream)."""
        device = device or torch.device("cuda")
        n_out, kw = q_packed.shape
        k_in = kw * 8
        qc = q_packed.to(device).contiguous()
        s = scales.to(device=device, dtype=torch.float16).contiguous()
        z = zeros.to(device=device, dtype=torch.float16).contiguous()
        L = lib()
        qb, zb = L.glowq_q_bytes(n_out, k_in), L.glowq_sz_bytes(n_out, k_in)
        if qb == 0 or zb == 0:
            raise GlowQError(ERR_SHAPE, "glowq_q_bytes")
        q_dev = torch.empty(qb, dtype=torch.uint8, device=device)
        sz_dev = torch.empty(zb, dtype=torch.uint8, device=device)
        flag = torch.empty(1, dtype=torch.int32, device=device)
        check(L.glowq_repack(_ptr(qc), _ptr(s), _ptr(z), n_out, k_in, _ptr(q_dev), _ptr(sz_dev),
                             _ptr(flag), _stream(stream)), "glowq_repack")
        return QWeight(q_dev, sz_dev, int(n_out), int(k_in))

    @staticmethod
    def from_workload(qw, device=None, stream=None) -> "QWeight":
        if getattr(qw, "fmt", "int4") != "int4":
            return QWeight.from_mx(qw.fmt, qw.codes, qw.scales, device, stream)
        return QWeight.from_canonical(qw.q_packed, qw.s, qw.z, device, stream)


def dequant(w: QWeight, dtype=torch.float32, stream=None) -> torch.Tensor:
    out = torch.empty(w.n_out, w.k_in, dtype=dtype, device=w.q.device)
    code = DTYPE_F32 if dtype == torch.float32 else DTYPE_F16
    wc = w.c()
    check(lib().glowq_dequant(ctypes.byref(wc), _ptr(out), code, _stream(stream)), "glowq_dequant")
    return out


# --------------------------------------------------------------------------- restore selection
def ner_sums(w: torch.Tensor, qw: QWeight, out: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """fp64 [2]: ||W - W_hat||_F^2 and ||W||_F^2 of one module (glowq_ner_sums); `out` may be a
    16-byte aligned fp64 view of two elements."""
    w = w.contiguous()
    if out is None:
        out = torch.empty(2, dtype=torch.float64, device=w.device)
    if workspace is None:
        workspace = torch.empty(int(lib().glowq_ner_workspace_bytes(qw.n_out)), dtype=torch.uint8,
                                device=w.device)
    wc = qw.c()
    check(lib().glowq_ner_sums(_ptr(w), ctypes.byref(wc), _ptr(workspace), workspace.numel(), _ptr(out),
                               _stream(stream)), "glowq_ner_sums")
    return out


def ner_workspace_bytes_batch(n_outs: Sequence[int]) -> int:
    return int(sum(lib().glowq_ner_workspace_bytes(n) for n in n_outs))


def ner_sums_batch(ws_and_qws: Sequence, out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """fp64 [n][2] pairs of glowq_ner_sums for (fp16 W, QWeight) pairs, in one batch call."""
    items = [(w.contiguous(), qw) for w, qw in ws_and_qws]
    dev = items[0][0].device
    if out is None:
        out = torch.empty(len(items), 2, dtype=torch.float64, device=dev)
    if workspace is None:
        workspace = torch.empty(ner_workspace_bytes_batch([qw.n_out for _, qw in items]), dtype=torch.uint8,
                                device=dev)
    wp = _arr(_vp, [w.data_ptr() for w, _ in items])
    wc = _arr(QWeightC, [qw.c() for _, qw in items])
    check(lib().glowq_ner_sums_batch(len(items), wp, wc, _ptr(workspace), workspace.numel(), _ptr(out),
                                     _stream(stream)), "glowq_ner_sums_batch")
    return out


def restore_select(sums: torch.Tensor, k: int, rel_tol: float, stream=None):
    """glowq_restore_select: (scores fp64 [n_units], mask int32 [n_units]) with the layer-order
    fallback for scores within rel_tol steps of the best."""
    sums = sums.contiguous()
    n_units, n_per = int(sums.shape[0]), int(sums.shape[1])
    scores = torch.empty(n_units, dtype=torch.float64, device=sums.device)
    mask = torch.empty(n_units, dtype=torch.int32, device=sums.device)
    check(lib().glowq_restore_select(_ptr(sums), n_units, n_per, k, float(rel_tol), _ptr(scores), _ptr(mask),
                                     _stream(stream)), "glowq_restore_select")
    return scores, mask


def restore_topk(sums: torch.Tensor, k: int, stream=None):
    """sums fp64 [n_units][n_per_unit][2] -> (scores fp64 [n_units], mask int32 [n_units])."""
    sums = sums.contiguous()
    n_units, n_per = int(sums.shape[0]), int(sums.shape[1])
    scores = torch.empty(n_units, dtype=torch.float64, device=sums.device)
    mask = torch.empty(n_units, dtype=torch.int32, device=sums.device)
    check(lib().glowq_restore_topk(_ptr(sums), n_units, n_per, k, _ptr(scores), _ptr(mask),
                                   _stream(stream)), "glowq_restore_topk")
    return scores, mask


# --------------------------------------------------------------------------- offline factor solve
def second_moment(x: torch.Tensor, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """fp32 [d][d] Sigma_x = X^T X / N of fp16 calibration activations x [N][d]."""
    x = x.contiguous()
    N, d = int(x.shape[0]), int(x.shape[1])
    if out is None:
        out = torch.empty(d, d, dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = torch.empty(int(lib().glowq_second_moment_workspace_bytes(N, d)), dtype=torch.uint8,
                                device=x.device)
    check(lib().glowq_second_moment(_ptr(x), N, d, _ptr(out), _ptr(workspace), workspace.numel(),
                                    _stream(stream)), "glowq_second_moment")
    return out


def solve_factors(e: torch.Tensor, sigma: torch.Tensor, omega: torch.Tensor, r: int, q: int = 0,
                  workspace: Optional[torch.Tensor] = None, stream=None):
    """fp64 stacked errors e [m][d], Sigma_x [d][d], test matrix omega [d][k] -> (A [m][r],
    B [r][d], S [r]) (glowq_solve_factors; synchronises the stream)."""
    e, sigma, omega = e.contiguous(), sigma.contiguous(), omega.contiguous()
    m, d = int(e.shape[0]), int(e.shape[1])
    k = int(omega.shape[1])
    A = torch.empty(m, r, dtype=torch.float64, device=e.device)
    B = torch.empty(r, d, dtype=torch.float64, device=e.device)
    S = torch.empty(r, dtype=torch.float64, device=e.device)
    if workspace is None:
        workspace = torch.empty(int(lib().glowq_solve_workspace_bytes(m, d, k, r)), dtype=torch.uint8, device=e.device)
    check(lib().glowq_solve_factors(_ptr(e), m, d, _ptr(sigma), _ptr(omega), r, k, q, _ptr(A), _ptr(B), _ptr(S),
                                    _ptr(workspace), workspace.numel(), _stream(stream)), "glowq_solve_factors")
    return A, B, S


def ec_score(e: torch.Tensor, sigma: torch.Tensor, s: Optional[torch.Tensor], r: int,
             workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """fp64 [3]: ||E_cat L||_F^2, sum of the first r squared singular values s, and g_ec, their
    ratio (glowq_ec_score)."""
    e, sigma = e.contiguous(), sigma.contiguous()
    m, d = int(e.shape[0]), int(e.shape[1])
    out = torch.empty(3, dtype=torch.float64, device=e.device)
    if workspace is None:
        workspace = torch.empty(int(lib().glowq_ec_score_workspace_bytes(m, d)), dtype=torch.uint8, device=e.device)
    s = s.contiguous() if s is not None else None
    check(lib().glowq_ec_score(_ptr(e), m, d, _ptr(sigma), _ptr(s), r, _ptr(out), _ptr(workspace), workspace.numel(),
                               _stream(stream)), "glowq_ec_score")
    return out


# --------------------------------------------------------------------------- forward
def workspace_bytes(T: int, r: int, n_proj: int = 1) -> int:
    return int(lib().glowq_workspace_bytes(T, r, n_proj))


def init_workspace(ws: torch.Tensor, stream=None) -> torch.Tensor:
    """Zero-fill a workspace with the library's fill kernel (glowq_workspace_init)."""
    check(lib().glowq_workspace_init(_ptr(ws), ws.numel(), _stream(stream)), "glowq_workspace_init")
    return ws


def workspace_status(ws: torch.Tensor, stream=None) -> int:
    """glowq_workspace_status: synchronises, returns OK or ERR_HANDOFF and clears the word."""
    st = int(lib().glowq_workspace_status(_ptr(ws), ws.numel(), _stream(stream)))
    if st not in (OK, ERR_HANDOFF, ERR_ROUTING):
        check(st, "glowq_workspace_status")
    return st


def make_workspace(T: int, r: int, n_proj: int = 1, device=None, min_bytes: int = 0) -> Optional[torch.Tensor]:
    n = max(workspace_bytes(T, r, n_proj), min_bytes)
    if n == 0:
        return None
    ws = torch.empty(n, dtype=torch.uint8, device=device or torch.device("cuda"))
    return init_workspace(ws)


def _arr(kind, items):
    return (kind * max(1, len(items)))(*items)


def _outs(x: torch.Tensor, weights: Sequence[QWeight], y):
    if y is None:
        y = [torch.empty(x.shape[0], w.n_out, dtype=torch.float16, device=x.device) for w in weights]
    return y


def group_forward(x: torch.Tensor, weights: Sequence[QWeight], b: Optional[torch.Tensor],
                  a: Sequence[torch.Tensor], r: int, restore: bool = True,
                  workspace: Optional[torch.Tensor] = None, y: Optional[List[torch.Tensor]] = None,
                  stream=None) -> List[torch.Tensor]:
    m = len(weights)
    y = _outs(x, weights, y)
    if workspace is None and restore and r > 0:
        workspace = make_workspace(x.shape[0], r, 1, x.device)
    wc = _arr(QWeightC, [w.c() for w in weights])
    ac = _arr(_vp, [t.data_ptr() for t in a]) if a else None
    yc = _arr(_vp, [t.data_ptr() for t in y])
    ws_n = 0 if workspace is None else workspace.numel()
    check(lib().glowq_group_forward(_ptr(x), x.shape[0], x.shape[1], m, wc, _ptr(b), ac, r,
                                    int(bool(restore)), _ptr(workspace), ws_n, yc, _stream(stream)),
          "glowq_group_forward")
    return y


def group_forward_static(x: torch.Tensor, weights: Sequence[QWeight], b: Optional[torch.Tensor],
                         a: Sequence[torch.Tensor], r: int, restore: bool = True,
                         y: Optional[List[torch.Tensor]] = None, stream=None) -> List[torch.Tensor]:
    """glowq_group_forward_static: no workspace argument; the library's per-device scratch."""
    m = len(weights)
    y = _outs(x, weights, y)
    wc = _arr(QWeightC, [w.c() for w in weights])
    ac = _arr(_vp, [t.data_ptr() for t in a]) if a else None
    yc = _arr(_vp, [t.data_ptr() for t in y])
    check(lib().glowq_group_forward_static(_ptr(x), x.shape[0], x.shape[1], m, wc, _ptr(b), ac, r,
                                           int(bool(restore)), yc, _stream(stream)),
          "glowq_group_forward_static")
    return y


def w4a8_workspace_bytes(T: int, d: int, r: int) -> int:
    return int(lib().glowq_w4a8_workspace_bytes(T, d, r))


def group_forward_w4a8(x: torch.Tensor, weights: Sequence[QWeight], b: Optional[torch.Tensor],
                       a: Sequence[torch.Tensor], r: int, restore: bool = True,
                       workspace: Optional[torch.Tensor] = None, y: Optional[List[torch.Tensor]] = None,
                       stream=None) -> List[torch.Tensor]:
    """glowq_group_forward_w4a8: per-token 8-bit activations for the quantised product, the
    correction on the fp16 activations."""
    m = len(weights)
    y = _outs(x, weights, y)
    if workspace is None and x.shape[0] > 0:
        n = w4a8_workspace_bytes(x.shape[0], x.shape[1], r if restore else 0)
        workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=x.device)
    wc = _arr(QWeightC, [w.c() for w in weights])
    ac = _arr(_vp, [t.data_ptr() for t in a]) if a else None
    yc = _arr(_vp, [t.data_ptr() for t in y])
    ws_n = 0 if workspace is None else workspace.numel()
    check(lib().glowq_group_forward_w4a8(_ptr(x), x.shape[0], x.shape[1], m, wc, _ptr(b), ac, r,
                                         int(bool(restore)), _ptr(workspace), ws_n, yc, _stream(stream)),
          "glowq_group_forward_w4a8")
    return y


def mx8_workspace_bytes(T: int, d: int, r: int) -> int:
    return int(lib().glowq_mx8_workspace_bytes(T, d, r))


def group_forward_mx8(x: torch.Tensor, weights: Sequence[QWeight], b: Optional[torch.Tensor],
                      a: Sequence[torch.Tensor], r: int, restore: bool = True,
                      workspace: Optional[torch.Tensor] = None, y: Optional[List[torch.Tensor]] = None,
                      stream=None) -> List[torch.Tensor]:
    """glowq_group_forward_mx8: MXFP4 weights against MXFP8 activations on the block-scaled matrix
    cores, the correction on the fp16 activations."""
    m = len(weights)
    y = _outs(x, weights, y)
    if workspace is None and x.shape[0] > 0:
        n = mx8_workspace_bytes(x.shape[0], x.shape[1], r if restore else 0)
        workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=x.device)
    wc = _arr(QWeightC, [w.c() for w in weights])
    ac = _arr(_vp, [t.data_ptr() for t in a]) if a else None
    yc = _arr(_vp, [t.data_ptr() for t in y])
    ws_n = 0 if workspace is None else workspace.numel()
    check(lib().glowq_group_forward_mx8(_ptr(x), x.shape[0], x.shape[1], m, wc, _ptr(b), ac, r,
                                        int(bool(restore)), _ptr(workspace), ws_n, yc, _stream(stream)),
          "glowq_group_forward_mx8")
    return y


# --------------------------------------------------------------------------- mixture of experts
@dataclass
class MoeModule:
    """One module (gate, up or down) of every expert, stacked: expert e's device layout at
    e * q_bytes / e * sz_bytes, its left factor a[e] fp16 [n_out][r]."""
    q: torch.Tensor
    sz: torch.Tensor
    a: Optional[torch.Tensor]   # fp16 [n_exp][n_out][r]
    n_out: int
    k_in: int

    @staticmethod
    def stack(weights: Sequence[QWeight], a: Optional[Sequence[torch.Tensor]]) -> "MoeModule":
        q = torch.cat([w.q for w in weights]).contiguous()
        sz = torch.cat([w.sz for w in weights]).contiguous()
        a_st = torch.stack(list(a)).contiguous() if a is not None else None
        return MoeModule(q, sz, a_st, weights[0].n_out, weights[0].k_in)


def moe_workspace_bytes(n_rows: int, T: int, r: int, share: int) -> int:
    return int(lib().glowq_moe_workspace_bytes(n_rows, T, r, share))


def moe_forward(x: torch.Tensor, n_exp: int, modules: Sequence[MoeModule], b: Optional[torch.Tensor], share: int,
                r: int, restore: bool, row_token: Optional[torch.Tensor], offsets: torch.Tensor, n_rows: int,
                workspace: Optional[torch.Tensor] = None, y: Optional[List[torch.Tensor]] = None,
                stream=None) -> List[torch.Tensor]:
    """glowq_moe_forward: outputs y_i fp16 [n_rows][n_out_i] in routed-row order."""
    if y is None:
        y = [torch.empty(n_rows, mm.n_out, dtype=torch.float16, device=x.device) for mm in modules]
    if workspace is None:
        workspace = make_workspace(1, 8, 1, x.device,
                                   min_bytes=moe_workspace_bytes(n_rows, x.shape[0], r if restore else 0, share))
    mc = _arr(MoeModuleC, [MoeModuleC(mm.q.data_ptr(), mm.sz.data_ptr(),
                                      None if mm.a is None else mm.a.data_ptr(), yy.data_ptr(), mm.n_out, mm.k_in)
                           for mm, yy in zip(modules, y)])
    check(lib().glowq_moe_forward(_ptr(x), x.shape[0], x.shape[1], n_exp, len(modules), mc, _ptr(b), share, r,
                                  int(bool(restore)), _ptr(row_token), _ptr(offsets), n_rows, _ptr(workspace),
                                  workspace.numel(), _stream(stream)), "glowq_moe_forward")
    return y


def solo_forward(x: torch.Tensor, w: QWeight, b: Optional[torch.Tensor], a: Optional[torch.Tensor],
                 r: int, restore: bool = True, workspace: Optional[torch.Tensor] = None,
                 y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    if y is None:
        y = torch.empty(x.shape[0], w.n_out, dtype=torch.float16, device=x.device)
    if workspace is None and restore and r > 0:
        workspace = make_workspace(x.shape[0], r, 1, x.device)
    wc = w.c()
    ws_n = 0 if workspace is None else workspace.numel()
    check(lib().glowq_solo_forward(_ptr(x), x.shape[0], x.shape[1], ctypes.byref(wc), _ptr(b), _ptr(a),
                                   r, int(bool(restore)), _ptr(workspace), ws_n, _ptr(y), _stream(stream)),
          "glowq_solo_forward")
    return y


def layerwise_forward(x: torch.Tensor, weights: Sequence[QWeight], b: Sequence[torch.Tensor],
                      a: Sequence[torch.Tensor], r: int, restore: bool = True,
                      workspace: Optional[torch.Tensor] = None, y: Optional[List[torch.Tensor]] = None,
                      stream=None) -> List[torch.Tensor]:
    m = len(weights)
    y = _outs(x, weights, y)
    if workspace is None and restore and r > 0:
        workspace = make_workspace(x.shape[0], r, m, x.device)
    wc = _arr(QWeightC, [w.c() for w in weights])
    bc = _arr(_vp, [t.data_ptr() for t in b]) if b else None
    ac = _arr(_vp, [t.data_ptr() for t in a]) if a else None
    yc = _arr(_vp, [t.data_ptr() for t in y])
    ws_n = 0 if workspace is None else workspace.numel()
    check(lib().glowq_layerwise_forward(_ptr(x), x.shape[0], x.shape[1], m, wc, bc, ac, r,
                                        int(bool(restore)), _ptr(workspace), ws_n, yc, _stream(stream)),
          "glowq_layerwise_forward")
    return y


@dataclass
class PathUnit:
    """One unit of a decoder-layer schedule (a group or a solo module) with its restore bit."""
    kind: int
    x: torch.Tensor
    weights: List[QWeight]
    b: Optional[torch.Tensor]
    a: List[torch.Tensor]
    r: int
    restore: bool
    y: List[torch.Tensor]


class PathPlan:
    """Marshalled glowq_unit array for repeated glowq_path_forward calls (keeps the ctypes
    arrays alive)."""

    def __init__(self, units: Sequence[PathUnit]):
        self.units = list(units)
        self._keep = []
        arr = (UnitC * max(1, len(self.units)))()
        for i, u in enumerate(self.units):
            wc = _arr(QWeightC, [w.c() for w in u.weights])
            ac = _arr(_vp, [t.data_ptr() for t in u.a]) if u.a else None
            yc = _arr(_vp, [t.data_ptr() for t in u.y])
            self._keep += [wc, ac, yc]
            arr[i] = UnitC(u.kind, len(u.weights), u.x.data_ptr(), u.x.shape[0], u.x.shape[1],
                           ctypes.cast(wc, ctypes.POINTER(QWeightC)),
                           None if u.b is None else u.b.data_ptr(),
                           None if ac is None else ctypes.cast(ac, ctypes.POINTER(_vp)),
                           u.r, int(bool(u.restore)), ctypes.cast(yc, ctypes.POINTER(_vp)))
        self.arr = arr
        need = max([workspace_bytes(u.x.shape[0], u.r, 1) for u in self.units if u.restore] + [0])
        dev = self.units[0].x.device if self.units else torch.device("cuda")
        self.workspace = make_workspace(1, 8, 1, dev, min_bytes=need)

    def run(self, stream=None) -> None:
        check(lib().glowq_path_forward(self.arr, len(self.units), _ptr(self.workspace),
                                       self.workspace.numel(), _stream(stream)), "glowq_path_forward")
