"""The allocation-free group forward (glowq_group_forward_static) through the C ABI: the same
results as glowq_group_forward with a caller workspace, call after call on the shared per-device
scratch (the second call of each pair smaller than the first), and size rejection before any
HIP call."""
import ctypes

import numpy as np
import pytest
import torch

import workload as W
from gpu_util import DevUnit, assert_parity, glowq, log, oracle_unit

FAKE = 0x10000  # aligned fake device address: never dereferenced, validation fails first


def test_static_rejects_calls_larger_than_the_scratch():
    from rank_error_compensation_amd import glowq as g
    L = g.lib()
    cap = int(L.glowq_static_scratch_bytes())
    assert cap == 16 << 20
    T = 8192  # prefill projection and its split partials exceed 16 MiB at r = 256
    assert int(L.glowq_workspace_bytes(T, 256, 1)) > cap
    wc = (g.QWeightC * 1)(g.QWeightC(FAKE, FAKE, 32, 256))
    ac = (ctypes.c_void_p * 1)(FAKE)
    yc = (ctypes.c_void_p * 1)(FAKE)
    assert L.glowq_group_forward_static(FAKE, T, 256, 1, wc, FAKE, ac, 256, 1, yc, None) == g.ERR_WORKSPACE
    assert L.glowq_group_forward_static(FAKE, 4, 100, 1, wc, FAKE, ac, 8, 1, yc, None) == g.ERR_SHAPE
    assert L.glowq_group_forward_static(FAKE, 0, 256, 1, wc, FAKE, ac, 8, 1, yc, None) == g.OK


# (label, T, d, module rows, r): decode (1, 4, 16 tokens), a narrow K-split call (40 tokens at
# d = 8192), the one-token-block tile split over K (64 and 48 tokens, 64 and 65 input groups),
# prefill (200 and 130 tokens); each followed by a smaller call of the same kind
CASES = [
    ("prefill", [(200, 512, [96, 64, 40], 32), (130, 384, [48, 32], 16)]),
    ("decode16", [(16, 1024, [256, 128, 128], 64), (4, 512, [64, 32, 32], 32)]),
    ("decode1", [(1, 4096, [512, 256, 256], 64), (1, 256, [40, 24], 16)]),
    ("narrow_split", [(40, 8192, [256], 64), (17, 8192, [128], 32)]),
    ("mid_split", [(64, 8192, [2048], 64), (48, 8320, [2048], 32)]),
    ("solo", [(4, 2048, [300], 64), (1, 1024, [100], 8)]),
]


@pytest.mark.gpu
@pytest.mark.parametrize("idx", range(len(CASES)), ids=[c[0] for c in CASES])
def test_static_matches_workspace_path(idx):
    label, calls = CASES[idx]
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g = glowq()
    for rep in range(2):  # the same pair twice: the scratch keeps the last call's contents
        for k, (T, d, rows, r) in enumerate(calls):
            keys = (40, idx, k)
            x = W.make_x(T, d, 1.19, (40, idx))  # one activation basis per case
            kind = "solo" if len(rows) == 1 else "group"
            unit = W.make_unit("s", kind, x, rows, r, keys)
            du = DevUnit(unit)
            log(f"static {label} rep {rep} call {k}: T={T} d={d} rows={rows} r={r}")
            ref_ws = du.forward()
            ys = g.group_forward_static(du.x, du.w, du.b, du.a, r, True)
            torch.cuda.synchronize()
            for i, (a, b) in enumerate(zip(ys, ref_ws)):
                assert torch.equal(a, b), (label, rep, k, i)
            for i, (y, yr) in enumerate(zip(ys, oracle_unit(unit))):
                assert_parity(y, yr, f"static {label} call {k} module {i}")
            # restore off through the static entry: the quantised product alone
            ys0 = g.group_forward_static(du.x, du.w, None, [], r, False)
            torch.cuda.synchronize()
            for i, (y, yr) in enumerate(zip(ys0, oracle_unit(unit, restore=False))):
                assert_parity(y, yr, f"static {label} call {k} restore off module {i}")
