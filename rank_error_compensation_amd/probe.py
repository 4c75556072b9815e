"""ctypes binding of libglowq_probe.so (include/glowq_probe.h): the achievable-peak probes used
by the benchmark and the hand-off protocol probe used by the tests.  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libglowq_probe.so")
_vp, _sz, _i32, _i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
EXPORTS = {
    "glowq_probe_read": (ctypes.c_int, [_vp, _sz, _vp, _i32, _vp]),
    "glowq_probe_mfma_f16": (ctypes.c_int, [_i64, _vp, _i32, _vp]),
    "glowq_probe_mfma_f16_flops": (ctypes.c_double, [_i64, _i32]),
    "glowq_probe_mfma_shape": (ctypes.c_int, [_i32, _i32, _i64, _vp, _i32, _vp]),
    "glowq_probe_mfma_shape_flops": (ctypes.c_double, [_i32, _i32, _i64, _i32]),
    "glowq_probe_read_sequence": (ctypes.c_int, [_vp, ctypes.POINTER(_i64), _i32, _vp, _vp]),
    "glowq_probe_handoff": (ctypes.c_int, [_vp, _sz, _i32, _i32, _i32, _i64, _i32, ctypes.c_float, _vp, _vp]),
}
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build the HIP libraries first "
                               "(python -m rank_error_compensation_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def read(src: torch.Tensor, sink: torch.Tensor, blocks: int) -> None:
    rc = lib().glowq_probe_read(src.data_ptr(), src.numel() * src.element_size(), sink.data_ptr(), blocks,
                                _stream())
    if rc != 0:
        raise RuntimeError(f"glowq_probe_read failed ({rc})")


def mfma_shape(shape: int, chains: int, iters: int, sink: torch.Tensor, blocks: int) -> float:
    """One launch of the shape probe; returns its fp16 flops."""
    rc = lib().glowq_probe_mfma_shape(shape, chains, iters, sink.data_ptr(), blocks, _stream())
    if rc != 0:
        raise RuntimeError(f"glowq_probe_mfma_shape failed ({rc})")
    return lib().glowq_probe_mfma_shape_flops(shape, chains, iters, blocks)


def mfma_f16(iters: int, sink: torch.Tensor, blocks: int) -> float:
    """Launch the matrix-core loop; returns the dense fp16 flops it performs."""
    rc = lib().glowq_probe_mfma_f16(iters, sink.data_ptr(), blocks, _stream())
    if rc != 0:
        raise RuntimeError(f"glowq_probe_mfma_f16 failed ({rc})")
    return lib().glowq_probe_mfma_f16_flops(iters, blocks)


class ReadSequence:
    """Marshalled size array for repeated glowq_probe_read_sequence calls over one buffer."""

    def __init__(self, sizes):
        self.n = len(sizes)
        self.arr = (_i64 * self.n)(*[int(b) for b in sizes])
        self.total = sum(int(b) for b in sizes)

    def run(self, src: torch.Tensor, sink: torch.Tensor) -> None:
        if src.numel() * src.element_size() < self.total:
            raise ValueError("source buffer smaller than the sequence")
        rc = lib().glowq_probe_read_sequence(src.data_ptr(), self.arr, self.n, sink.data_ptr(), _stream())
        if rc != 0:
            raise RuntimeError(f"glowq_probe_read_sequence failed ({rc})")


def handoff(ws: torch.Tensor, n_prod: int, n_cons: int, n_pairs: int, delay: int, publish: bool, salt: float,
            counts: torch.Tensor) -> None:
    """One launch of the hand-off protocol probe on workspace `ws` (counts: int32 [2], accumulated)."""
    rc = lib().glowq_probe_handoff(ws.data_ptr(), ws.numel() * ws.element_size(), n_prod, n_cons, n_pairs, delay,
                                   int(publish), salt, counts.data_ptr(), _stream())
    if rc != 0:
        raise RuntimeError(f"glowq_probe_handoff failed ({rc})")
