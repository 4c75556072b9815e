"""The C ABI without a GPU: the library loads, exports every function that include/glowq.h
declares, sizes its buffers as documented and rejects invalid arguments before any HIP call."""
import ctypes
import os
import re

import pytest

from rank_error_compensation_amd import glowq as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "glowq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(glowq_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    L = g.lib()
    names = header_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(g.EXPORTS), set(names) ^ set(g.EXPORTS)


def test_status_strings_and_version():
    L = g.lib()
    assert L.glowq_version() == 300
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -8):
        assert L.glowq_status_string(code).startswith(b"GLOWQ_")
    assert L.glowq_status_string(12345) == b"GLOWQ_ERR_UNKNOWN"


def test_buffer_sizes():
    L = g.lib()
    assert L.glowq_q_bytes(4096, 4096) == 4096 * 4096 // 2
    assert L.glowq_sz_bytes(4096, 4096) == 4096 * 32 * 4
    assert L.glowq_q_bytes(17, 256) == 2 * 2 * 1024  # rows padded to 32
    assert L.glowq_q_bytes(16, 100) == 0 and L.glowq_q_bytes(0, 128) == 0
    assert L.glowq_workspace_bytes(0, 64, 1) == 0
    assert L.glowq_workspace_bytes(4, 0, 1) == 0
    hdr = 8192  # synchronisation words of the decode hand-off
    r256 = lambda n: (n + 255) // 256 * 256
    # the fixed decode area ((fp32, tag) pairs for T <= 64, r <= 256, 8 projections, 8 copies),
    # then for calls that may take the prefill path (T > 16) the projection in fp16 (r padded to
    # 32) and its fp32 split-K partials (up to 8 splits), and for 17 .. 64 tokens the fp32 partial
    # outputs of a K-split call (ranges x rows at most 28672, times T)
    area = 64 * 256 * 8 * 8 * 8
    ws = lambda T, r, p: hdr + area + (0 if T <= 16 else
                                       r256(T * ((r + 31) // 32 * 32) * 2 * p) +
                                       r256(8 * T * ((r + 31) // 32 * 32) * 4 * p) +
                                       (r256(28672 * T * 4) if T <= 64 else 0))
    assert L.glowq_workspace_bytes(1, 64, 1) == hdr + area
    assert L.glowq_workspace_bytes(16, 256, 8) == hdr + area
    assert L.glowq_workspace_bytes(64, 256, 8) == ws(64, 256, 8)
    assert L.glowq_workspace_bytes(2048, 64, 1) == hdr + area + 2048 * 64 * 2 + 8 * 2048 * 64 * 4
    assert L.glowq_workspace_bytes(100, 8, 3) == ws(100, 8, 3)


FAKE = 0x10000  # 64 KiB-aligned fake device address: never dereferenced, validation fails first


def _w(n_out=32, k_in=256, q=FAKE, sz=FAKE, fmt=0, reserved=0):
    return g.QWeightC(q, sz, n_out, k_in, fmt, reserved)


def call_group(x=FAKE, T=4, d=256, m=1, w=None, b=FAKE, a=None, r=8, restore=1, ws=FAKE,
               ws_bytes=1 << 24, y=None):
    L = g.lib()
    w = w if w is not None else [_w() for _ in range(m)]
    wc = (g.QWeightC * max(1, len(w)))(*w)
    a = a if a is not None else [FAKE] * m
    y = y if y is not None else [FAKE] * m
    ac = (ctypes.c_void_p * max(1, len(a)))(*a)
    yc = (ctypes.c_void_p * max(1, len(y)))(*y)
    return L.glowq_group_forward(x, T, d, m, wc, b, ac, r, restore, ws, ws_bytes, yc, None)


@pytest.mark.parametrize("kw,code", [
    (dict(m=0), g.ERR_SHAPE),
    (dict(m=9), g.ERR_UNSUPPORTED),
    (dict(T=-1), g.ERR_SHAPE),
    (dict(d=100), g.ERR_SHAPE),
    (dict(d=0), g.ERR_SHAPE),
    (dict(r=-8), g.ERR_SHAPE),
    (dict(r=264), g.ERR_UNSUPPORTED),
    (dict(r=12), g.ERR_UNSUPPORTED),
    (dict(x=None), g.ERR_INVALID_ARG),
    (dict(w=[_w(q=0)]), g.ERR_INVALID_ARG),
    (dict(w=[_w(n_out=0)]), g.ERR_SHAPE),
    (dict(w=[_w(k_in=384)]), g.ERR_SHAPE),
    (dict(b=None), g.ERR_INVALID_ARG),
    (dict(a=[0]), g.ERR_INVALID_ARG),
    (dict(y=[0]), g.ERR_INVALID_ARG),
    (dict(x=FAKE + 8), g.ERR_ALIGN),
    (dict(y=[FAKE + 2]), g.ERR_ALIGN),
    (dict(a=[FAKE + 4]), g.ERR_ALIGN),
    (dict(w=[_w(q=FAKE + 8)]), g.ERR_ALIGN),
    (dict(ws=None), g.ERR_WORKSPACE),
    (dict(ws_bytes=100), g.ERR_WORKSPACE),
    (dict(ws=FAKE + 16), g.ERR_ALIGN),
    # activation offsets T d 2 are 32-bit in the kernels: T d above 2^30 is refused
    (dict(T=1 << 19, d=4096), g.ERR_UNSUPPORTED),
    (dict(T=262144, d=8192), g.ERR_UNSUPPORTED),
    (dict(T=(1 << 30) // 4096 + 1, d=4096), g.ERR_UNSUPPORTED),
    # int32 work-tile numbering: (T / 16) x (rows / 16) tiles above 2^31 - 1 are refused
    (dict(T=1 << 16, d=128, m=8, w=[_w(n_out=1 << 24, k_in=128)] * 8), g.ERR_UNSUPPORTED),
])
def test_group_validation_rejects_before_any_hip_call(kw, code):
    assert call_group(**kw) == code


def test_activation_block_bound_rejects_before_any_hip_call():
    # restore off, no workspace: T d one row above 2^30 is still refused before any launch
    L = g.lib()
    wc = (g.QWeightC * 1)(_w(n_out=16, k_in=4096))
    assert L.glowq_group_forward(FAKE, (1 << 30) // 4096 + 1, 4096, 1, wc, None, None, 0, 0, None, 0,
                                 (ctypes.c_void_p * 1)(FAKE), None) == g.ERR_UNSUPPORTED


def test_workspace_init_and_status_validate():
    L = g.lib()
    for fn in (L.glowq_workspace_init, L.glowq_workspace_status):
        assert fn(None, 1 << 20, None) == g.ERR_INVALID_ARG
        assert fn(FAKE + 16, 1 << 20, None) == g.ERR_ALIGN
        assert fn(FAKE, 8191, None) == g.ERR_WORKSPACE


def test_restore_off_needs_no_factors_and_t0_is_noop():
    # restore off with null b / a / workspace validates; T = 0 returns OK without launching
    assert call_group(T=0, b=None, a=[0], ws=None, restore=0) == g.OK
    assert call_group(T=0, r=0, b=None, a=[0], ws=None) == g.OK
    assert call_group(T=0, x=None, y=[0]) == g.OK


def test_other_entry_points_validate():
    L = g.lib()
    wc = _w()
    assert L.glowq_solo_forward(FAKE, 4, 256, ctypes.byref(wc), None, FAKE, 8, 1, FAKE, 1 << 20, FAKE,
                                None) == g.ERR_INVALID_ARG
    assert L.glowq_solo_forward(FAKE, 4, 256, None, FAKE, FAKE, 8, 1, FAKE, 1 << 20, FAKE, None) == g.ERR_INVALID_ARG
    ws = (g.QWeightC * 2)(_w(), _w())
    bc = (ctypes.c_void_p * 2)(FAKE, 0)
    ac = (ctypes.c_void_p * 2)(FAKE, FAKE)
    yc = (ctypes.c_void_p * 2)(FAKE, FAKE)
    assert L.glowq_layerwise_forward(FAKE, 4, 256, 2, ws, bc, ac, 8, 1, FAKE, 1 << 20, yc, None) == g.ERR_INVALID_ARG
    bc2 = (ctypes.c_void_p * 2)(FAKE, FAKE)
    need = L.glowq_workspace_bytes(4, 8, 2)
    assert L.glowq_layerwise_forward(FAKE, 4, 256, 2, ws, bc2, ac, 8, 1, FAKE, need - 1, yc, None) == g.ERR_WORKSPACE
    assert L.glowq_dequant(None, FAKE, 0, None) == g.ERR_INVALID_ARG
    assert L.glowq_dequant(ctypes.byref(wc), FAKE, 7, None) == g.ERR_INVALID_ARG
    bad = _w(k_in=200)
    assert L.glowq_dequant(ctypes.byref(bad), FAKE, 0, None) == g.ERR_SHAPE
    assert L.glowq_repack(FAKE, FAKE, FAKE, 16, 100, FAKE, FAKE, FAKE, None) == g.ERR_SHAPE
    assert L.glowq_repack(None, FAKE, FAKE, 16, 128, FAKE, FAKE, FAKE, None) == g.ERR_INVALID_ARG
    assert L.glowq_repack(FAKE, FAKE, FAKE, 16, 128, FAKE + 4, FAKE, FAKE, None) == g.ERR_ALIGN


def test_restore_selection_validates():
    """glowq_ner_sums / glowq_restore_topk / glowq_restore_select reject bad arguments before any HIP call."""
    L = g.lib()
    wc = _w()
    assert L.glowq_ner_workspace_bytes(0) == 0
    assert L.glowq_ner_workspace_bytes(17) == 256 and L.glowq_ner_workspace_bytes(4096) == 4096
    need = L.glowq_ner_workspace_bytes(wc.n_out)
    assert L.glowq_ner_sums(None, ctypes.byref(wc), FAKE, need, FAKE, None) == g.ERR_INVALID_ARG
    assert L.glowq_ner_sums(FAKE, None, FAKE, need, FAKE, None) == g.ERR_INVALID_ARG
    assert L.glowq_ner_sums(FAKE, ctypes.byref(wc), FAKE, need, None, None) == g.ERR_INVALID_ARG
    assert L.glowq_ner_sums(FAKE, ctypes.byref(_w(k_in=200)), FAKE, 1 << 20, FAKE, None) == g.ERR_SHAPE
    assert L.glowq_ner_sums(FAKE + 8, ctypes.byref(wc), FAKE, need, FAKE, None) == g.ERR_ALIGN
    assert L.glowq_ner_sums(FAKE, ctypes.byref(wc), FAKE + 16, need, FAKE, None) == g.ERR_ALIGN
    assert L.glowq_ner_sums(FAKE, ctypes.byref(wc), FAKE, need - 1, FAKE, None) == g.ERR_WORKSPACE
    wp = (ctypes.c_void_p * 2)(FAKE, 0)
    wqs = (g.QWeightC * 2)(_w(), _w())
    assert L.glowq_ner_sums_batch(0, wp, wqs, FAKE, 1 << 20, FAKE, None) == g.ERR_INVALID_ARG
    assert L.glowq_ner_sums_batch(2, wp, wqs, FAKE, 1 << 20, FAKE, None) == g.ERR_INVALID_ARG
    wp2 = (ctypes.c_void_p * 2)(FAKE, FAKE)
    assert L.glowq_ner_sums_batch(2, wp2, wqs, FAKE, 2 * need - 1, FAKE, None) == g.ERR_WORKSPACE
    wqs_bad = (g.QWeightC * 2)(_w(), _w(n_out=0))
    assert L.glowq_ner_sums_batch(2, wp2, wqs_bad, FAKE, 1 << 20, FAKE, None) == g.ERR_SHAPE
    assert L.glowq_restore_topk(None, 4, 1, 2, FAKE, FAKE, None) == g.ERR_INVALID_ARG
    assert L.glowq_restore_topk(FAKE, 0, 1, 0, FAKE, FAKE, None) == g.ERR_SHAPE
    assert L.glowq_restore_topk(FAKE, 4097, 1, 2, FAKE, FAKE, None) == g.ERR_SHAPE
    assert L.glowq_restore_topk(FAKE, 4, 0, 2, FAKE, FAKE, None) == g.ERR_SHAPE
    assert L.glowq_restore_topk(FAKE, 4, 1, 5, FAKE, FAKE, None) == g.ERR_SHAPE
    assert L.glowq_restore_topk(FAKE, 4, 1, -1, FAKE, FAKE, None) == g.ERR_SHAPE
    assert L.glowq_restore_topk(FAKE, 4, 1, 2, FAKE, FAKE + 4, None) == g.ERR_ALIGN
    for bad in (-1e-3, 1.5, float("nan"), float("inf")):
        assert L.glowq_restore_select(FAKE, 4, 1, 2, bad, FAKE, FAKE, None) == g.ERR_INVALID_ARG
    assert L.glowq_restore_select(FAKE, 4, 1, 5, 0.01, FAKE, FAKE, None) == g.ERR_SHAPE
    assert L.glowq_restore_select(None, 4, 1, 2, 0.01, FAKE, FAKE, None) == g.ERR_INVALID_ARG


def test_second_moment_validates():
    L = g.lib()
    assert L.glowq_second_moment_workspace_bytes(0, 128) == 0
    assert L.glowq_second_moment_workspace_bytes(4, 100) == 0
    assert L.glowq_second_moment_workspace_bytes(4, 16512) == 0
    need = L.glowq_second_moment_workspace_bytes(1000, 256)
    assert need > 0 and need % 256 == 0
    assert L.glowq_second_moment(None, 1000, 256, FAKE, FAKE, need, None) == g.ERR_INVALID_ARG
    assert L.glowq_second_moment(FAKE, 1000, 200, FAKE, FAKE, need, None) == g.ERR_SHAPE
    assert L.glowq_second_moment(FAKE, 0, 256, FAKE, FAKE, need, None) == g.ERR_SHAPE
    assert L.glowq_second_moment(FAKE, 1000, 256, FAKE + 8, FAKE, need, None) == g.ERR_ALIGN
    assert L.glowq_second_moment(FAKE, 1000, 256, FAKE, FAKE, need - 1, None) == g.ERR_WORKSPACE
    assert L.glowq_second_moment(FAKE, 1 << 20, 4096, FAKE, FAKE, 1 << 40, None) == g.ERR_UNSUPPORTED


def test_solve_validates():
    L = g.lib()
    assert L.glowq_solve_workspace_bytes(0, 128, 16, 8) == 0
    assert L.glowq_solve_workspace_bytes(96, 128, 8, 16) == 0     # k < r
    assert L.glowq_solve_workspace_bytes(96, 128, 97, 8) == 0     # k > 96
    need = L.glowq_solve_workspace_bytes(96, 128, 16, 8)
    assert need > 0 and need % 256 == 0
    args = lambda **kw: [kw.get(n, v) for n, v in (("e", FAKE), ("m", 96), ("d", 128), ("s", FAKE), ("o", FAKE),
                                                       ("r", 8), ("k", 16), ("q", 1), ("a", FAKE), ("b", FAKE),
                                                       ("sv", FAKE), ("ws", FAKE), ("n", need), ("st", None))]
    assert L.glowq_solve_factors(*args(e=None)) == g.ERR_INVALID_ARG
    assert L.glowq_solve_factors(*args(k=4)) == g.ERR_SHAPE
    assert L.glowq_solve_factors(*args(q=-1)) == g.ERR_SHAPE
    assert L.glowq_solve_factors(*args(k=100)) == g.ERR_UNSUPPORTED
    assert L.glowq_solve_factors(*args(a=FAKE + 8)) == g.ERR_ALIGN
    assert L.glowq_solve_factors(*args(n=need - 1)) == g.ERR_WORKSPACE


def test_ec_score_validates():
    L = g.lib()
    assert L.glowq_ec_score_workspace_bytes(0, 128) == 0
    assert L.glowq_ec_score_workspace_bytes(96, 0) == 0
    need = L.glowq_ec_score_workspace_bytes(96, 128)
    assert need == (128 * 128 + 128) * 8  # E^T E (d x d) and one partial sum per row
    args = lambda **kw: [kw.get(n, v) for n, v in (("e", FAKE), ("m", 96), ("d", 128), ("s", FAKE), ("sv", FAKE),
                                                       ("r", 8), ("o", FAKE), ("ws", FAKE), ("n", need),
                                                       ("st", None))]
    assert L.glowq_ec_score(*args(e=None)) == g.ERR_INVALID_ARG
    assert L.glowq_ec_score(*args(sv=None)) == g.ERR_INVALID_ARG
    assert L.glowq_ec_score(*args(r=-1)) == g.ERR_SHAPE
    assert L.glowq_ec_score(*args(r=97)) == g.ERR_SHAPE        # r > m
    assert L.glowq_ec_score(*args(m=0)) == g.ERR_SHAPE
    assert L.glowq_ec_score(*args(d=1 << 20, n=1 << 40)) == g.ERR_UNSUPPORTED
    assert L.glowq_ec_score(*args(o=FAKE + 8)) == g.ERR_ALIGN
    assert L.glowq_ec_score(*args(ws=FAKE + 16)) == g.ERR_ALIGN
    assert L.glowq_ec_score(*args(n=need - 1)) == g.ERR_WORKSPACE


def test_path_validates_every_unit_first():
    L = g.lib()
    wq = (g.QWeightC * 1)(_w())
    ac = (ctypes.c_void_p * 1)(FAKE)
    yc = (ctypes.c_void_p * 1)(FAKE)
    P = ctypes.POINTER
    good = g.UnitC(g.UNIT_GROUP, 1, FAKE, 0, 256, ctypes.cast(wq, P(g.QWeightC)), FAKE,
                   ctypes.cast(ac, P(ctypes.c_void_p)), 8, 1, ctypes.cast(yc, P(ctypes.c_void_p)))
    bad = g.UnitC(g.UNIT_SOLO, 2, FAKE, 0, 256, ctypes.cast(wq, P(g.QWeightC)), FAKE,
                  ctypes.cast(ac, P(ctypes.c_void_p)), 8, 1, ctypes.cast(yc, P(ctypes.c_void_p)))
    arr = (g.UnitC * 2)(good, bad)
    assert L.glowq_path_forward(arr, 2, FAKE, 1 << 20, None) == g.ERR_SHAPE
    arr2 = (g.UnitC * 2)(good, good)
    assert L.glowq_path_forward(arr2, 2, FAKE, 1 << 20, None) == g.OK  # T = 0 units
    bad_kind = g.UnitC(7, 1, FAKE, 0, 256, ctypes.cast(wq, P(g.QWeightC)), FAKE,
                       ctypes.cast(ac, P(ctypes.c_void_p)), 8, 1, ctypes.cast(yc, P(ctypes.c_void_p)))
    assert L.glowq_path_forward((g.UnitC * 1)(bad_kind), 1, FAKE, 1 << 20, None) == g.ERR_INVALID_ARG
    assert L.glowq_path_forward(None, 3, FAKE, 1 << 20, None) == g.ERR_INVALID_ARG


def test_probe_library_exports_and_rejects_bad_arguments():
    """The measurement probes (libglowq_probe.so, include/glowq_probe.h): every declared function
    is exported, and invalid arguments are rejected before any HIP call."""
    from rank_error_compensation_amd import probe
    src = open(os.path.join(ROOT, "include", "glowq_probe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = sorted(set(re.findall(r"\b(glowq_[a-z_0-9]+)\s*\(", src)))
    L = probe.lib()
    assert set(names) == set(probe.EXPORTS), set(names) ^ set(probe.EXPORTS)
    for n in names:
        assert hasattr(L, n), n
    assert L.glowq_probe_read(None, 1024, FAKE, 4, None) == -1
    assert L.glowq_probe_read(FAKE, 1000, FAKE, 4, None) == -1      # not a multiple of 16
    assert L.glowq_probe_read(FAKE, 1024, FAKE, 0, None) == -1
    assert L.glowq_probe_mfma_f16(10, None, 4, None) == -1
    assert L.glowq_probe_mfma_f16(-1, FAKE, 4, None) == -1
    assert L.glowq_probe_mfma_f16_flops(3, 2) == 2 * 4 * 3 * 4 * 32 * 32 * 16 * 2
    sizes = (ctypes.c_int64 * 3)(1024, 1000, 2048)                   # 1000: not a multiple of 16
    assert L.glowq_probe_read_sequence(FAKE, sizes, 3, FAKE, None) == -1
    sizes = (ctypes.c_int64 * 1)(257 << 20)                          # beyond 256 MiB per read
    assert L.glowq_probe_read_sequence(FAKE, sizes, 1, FAKE, None) == -1
    assert L.glowq_probe_read_sequence(FAKE, sizes, 0, FAKE, None) == -1

    def handoff(ws=FAKE, nbytes=8192 + 8 * 256, n_prod=4, n_cons=8, n_pairs=256, delay=0, publish=1, cnt=FAKE):
        return L.glowq_probe_handoff(ws, nbytes, n_prod, n_cons, n_pairs, delay, publish, 1.0, cnt, None)
    assert handoff(ws=None) == -1
    assert handoff(cnt=None) == -1
    assert handoff(ws=FAKE + 16) == -1                               # workspace not 256-byte aligned
    assert handoff(nbytes=8192 + 8 * 255) == -1                      # pairs beyond the workspace
    assert handoff(n_prod=0) == -1 and handoff(n_prod=1025) == -1
    assert handoff(n_cons=0) == -1 and handoff(n_cons=65537) == -1
    assert handoff(n_pairs=0) == -1 and handoff(n_pairs=65537, nbytes=1 << 20) == -1
    assert handoff(delay=-1) == -1 and handoff(delay=4097) == -1
    assert handoff(publish=2) == -1
    assert handoff(publish=0, n_pairs=257, nbytes=1 << 20) == -1     # silent producers: one wait per thread
    assert handoff(publish=0, n_cons=65) == -1


def test_moe_validation_rejects_before_any_hip_call():
    L = g.lib()
    mod = (g.MoeModuleC * 2)(g.MoeModuleC(FAKE, FAKE, FAKE, FAKE, 64, 256), g.MoeModuleC(FAKE, FAKE, FAKE, FAKE, 64, 256))

    def call(x=FAKE, T=8, d=256, n_exp=4, m=2, mods=mod, b=FAKE, share=0, r=16, restore=1, tok=FAKE, off=FAKE,
             n_rows=16, ws=FAKE, ws_bytes=1 << 24):
        return L.glowq_moe_forward(x, T, d, n_exp, m, mods, b, share, r, restore, tok, off, n_rows, ws, ws_bytes, None)

    assert call(n_exp=0) == g.ERR_UNSUPPORTED
    assert call(n_exp=257) == g.ERR_UNSUPPORTED
    assert call(m=5) == g.ERR_UNSUPPORTED
    assert call(share=2) == g.ERR_INVALID_ARG
    assert call(d=100) == g.ERR_SHAPE
    assert call(r=12) == g.ERR_UNSUPPORTED
    assert call(n_rows=0) == g.OK                      # no routed rows: nothing to do
    assert call(off=None) == g.ERR_INVALID_ARG
    assert call(tok=None, T=8, n_rows=16) == g.ERR_SHAPE  # rows read x[j]: T must equal n_rows
    assert call(b=None) == g.ERR_INVALID_ARG
    assert call(ws_bytes=100) == g.ERR_WORKSPACE
    assert call(ws=FAKE + 16) == g.ERR_ALIGN
    assert call(x=FAKE + 2) == g.ERR_ALIGN
    bad = (g.MoeModuleC * 2)(g.MoeModuleC(FAKE, FAKE, FAKE, FAKE, 64, 384), g.MoeModuleC(FAKE, FAKE, FAKE, FAKE, 64, 256))
    assert call(mods=bad) == g.ERR_SHAPE
    assert L.glowq_moe_workspace_bytes(16, 8, 16, 0) == 8192 + 16 * 32 * 2 + 0 * 256 + (256 - 16 * 32 * 2 % 256) % 256
    assert L.glowq_moe_workspace_bytes(16, 8, 0, 0) == 8192
    assert L.glowq_moe_workspace_bytes(16, 8, 16, 3) == 0


def test_mx_sizes_and_repack_validation():
    """MX device-layout sizes (1024 / 1536 bytes per 16 rows x 128 inputs, scales in the INT4
    geometry) and glowq_repack_mx's checks before any HIP call."""
    L = g.lib()
    assert L.glowq_mx_q_bytes(g.FMT_MXFP4, 32, 256) == L.glowq_q_bytes(32, 256) == 2 * 2 * 1024
    assert L.glowq_mx_q_bytes(g.FMT_MXFP6_E2M3, 17, 384) == 2 * 3 * 1536
    assert L.glowq_mx_q_bytes(g.FMT_MXFP6_E3M2, 16, 128) == 1536
    assert L.glowq_mx_q_bytes(g.FMT_INT4_G128, 16, 128) == 0 and L.glowq_mx_q_bytes(7, 16, 128) == 0
    assert L.glowq_mx_q_bytes(g.FMT_MXFP4, 16, 100) == 0 and L.glowq_mx_q_bytes(g.FMT_MXFP4, 0, 128) == 0
    R = L.glowq_repack_mx
    assert R(g.FMT_INT4_G128, FAKE, FAKE, 16, 128, FAKE, FAKE, FAKE, None) == g.ERR_INVALID_ARG
    assert R(4, FAKE, FAKE, 16, 128, FAKE, FAKE, FAKE, None) == g.ERR_INVALID_ARG
    assert R(g.FMT_MXFP4, None, FAKE, 16, 128, FAKE, FAKE, FAKE, None) == g.ERR_INVALID_ARG
    assert R(g.FMT_MXFP4, FAKE, FAKE, 16, 128, FAKE, FAKE, None, None) == g.ERR_INVALID_ARG
    assert R(g.FMT_MXFP4, FAKE, FAKE, 16, 96, FAKE, FAKE, FAKE, None) == g.ERR_SHAPE
    assert R(g.FMT_MXFP4, FAKE, FAKE, 0, 128, FAKE, FAKE, FAKE, None) == g.ERR_SHAPE
    assert R(g.FMT_MXFP6_E2M3, FAKE + 8, FAKE, 16, 128, FAKE, FAKE, FAKE, None) == g.ERR_ALIGN
    assert R(g.FMT_MXFP6_E2M3, FAKE, FAKE + 2, 16, 128, FAKE, FAKE, FAKE, None) == g.ERR_ALIGN
    assert R(g.FMT_MXFP6_E3M2, FAKE, FAKE, 16, 128, FAKE + 4, FAKE, FAKE, None) == g.ERR_ALIGN


def test_forward_format_validation():
    """Forward calls: an unknown format or a nonzero reserved word is INVALID_ARG, modules of
    different formats in one call UNSUPPORTED; W4A8 takes INT4 only; the dequant export and the
    restore scores validate the format too."""
    L = g.lib()
    assert call_group(w=[_w(fmt=4)]) == g.ERR_INVALID_ARG
    assert call_group(w=[_w(fmt=-1)]) == g.ERR_INVALID_ARG
    assert call_group(w=[_w(fmt=1, reserved=3)]) == g.ERR_INVALID_ARG
    mixed = (g.QWeightC * 2)(_w(fmt=1), _w(fmt=2))
    ys = (ctypes.c_void_p * 2)(FAKE, FAKE)
    as_ = (ctypes.c_void_p * 2)(FAKE, FAKE)
    assert L.glowq_group_forward(FAKE, 4, 256, 2, mixed, FAKE, as_, 8, 1, FAKE, 1 << 20, ys, None) == g.ERR_UNSUPPORTED
    w8 = (g.QWeightC * 1)(_w(fmt=g.FMT_MXFP4))
    a1 = (ctypes.c_void_p * 1)(FAKE)
    y1 = (ctypes.c_void_p * 1)(FAKE)
    assert L.glowq_group_forward_w4a8(FAKE, 4, 256, 1, w8, FAKE, a1, 8, 1, FAKE, 1 << 24, y1, None) == g.ERR_UNSUPPORTED
    assert L.glowq_dequant(ctypes.byref(_w(fmt=9)), FAKE, 0, None) == g.ERR_INVALID_ARG
    need = L.glowq_ner_workspace_bytes(32)
    assert L.glowq_ner_sums(FAKE, ctypes.byref(_w(fmt=g.FMT_MXFP4)), FAKE, need, FAKE, None) == g.ERR_UNSUPPORTED


def test_mx8_validation():
    """glowq_group_forward_mx8: MX weight modules only (MXFP4, MXFP6 E2M3 or E3M2); the workspace
    holds the codes, the block scales and the projection; checks before any HIP call."""
    L = g.lib()
    r256 = lambda n: (n + 255) // 256 * 256
    # codes [T][d] | one 512-byte scale record per (128-token block, 128-input group)
    assert L.glowq_mx8_workspace_bytes(4, 256, 0) == r256(4 * 256) + 1 * 2 * 512
    assert L.glowq_mx8_workspace_bytes(129, 384, 0) == r256(129 * 384) + 2 * 3 * 512
    assert L.glowq_mx8_workspace_bytes(4, 256, 8) > L.glowq_mx8_workspace_bytes(4, 256, 0)
    assert L.glowq_mx8_workspace_bytes(0, 256, 8) == 0 and L.glowq_mx8_workspace_bytes(4, 200, 8) == 0
    a1 = (ctypes.c_void_p * 1)(FAKE)
    y1 = (ctypes.c_void_p * 1)(FAKE)
    w1 = (g.QWeightC * 1)(_w(fmt=g.FMT_INT4_G128))
    assert L.glowq_group_forward_mx8(FAKE, 4, 256, 1, w1, FAKE, a1, 8, 1, FAKE, 1 << 24, y1, None) == g.ERR_UNSUPPORTED
    w2 = (g.QWeightC * 2)(_w(fmt=g.FMT_MXFP4), _w(fmt=g.FMT_MXFP6_E2M3))  # one format per call
    a2 = (ctypes.c_void_p * 2)(FAKE, FAKE)
    y2 = (ctypes.c_void_p * 2)(FAKE, FAKE)
    assert L.glowq_group_forward_mx8(FAKE, 4, 256, 2, w2, FAKE, a2, 8, 1, FAKE, 1 << 24, y2, None) == g.ERR_UNSUPPORTED
    w1 = (g.QWeightC * 1)(_w(fmt=g.FMT_MXFP4))
    need = L.glowq_mx8_workspace_bytes(4, 256, 8)
    assert L.glowq_group_forward_mx8(FAKE, 4, 256, 1, w1, FAKE, a1, 8, 1, FAKE, need - 1, y1, None) == g.ERR_WORKSPACE
    assert L.glowq_group_forward_mx8(FAKE, 4, 256, 1, w1, FAKE, a1, 8, 1, FAKE + 16, need, y1, None) == g.ERR_ALIGN
    assert L.glowq_group_forward_mx8(FAKE, 4, 256, 1, w1, None, a1, 8, 1, FAKE, need, y1, None) == g.ERR_INVALID_ARG
