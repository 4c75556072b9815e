"""Correcting calls of 17 to 64 tokens with INT4 weights on the one-token-block tile (every weight
byte read once, all operands staged in LDS by the load unit, the projection formed in the same
launch and handed over as tagged pairs): every module against the fp64 oracle, group, solo and
layerwise, 32- and 64-token tiles, ragged row counts, a single input group, rank 256 and the
LLaMA-3.1-8B gate/up shape.  Calls with fewer than 160 workgroups of 128 rows, at least 48 tokens
and at least 64 input groups split K over ranges of workgroups, the projection's producers over the
same ranges (the ranges' fp32 sums added by a second launch): even and uneven ranges, ragged rows
and tokens, ranks 24 and 256, layerwise projections and the LLaMA-3.1-8B down_proj.  The same
shapes without the correction (other tiles) are checked beside them.

Bar: relative Frobenius error <= 1e-3 and max-abs error <= 1e-2 max|y| per module."""
import pytest
import torch

import workload as W
from gpu_util import DevUnit, assert_handoff_ok, assert_parity, glowq, log, oracle_unit

pytestmark = pytest.mark.gpu
WS_HEADER = 8192

# (T, d, rows, r): every case has at least 160 row blocks of 128 rows
CASES = [
    (64, 256, [11008, 11008], 16),       # 64-token tile, 172 workgroups
    (24, 256, [12000, 10000], 8),        # 32-token tile, ragged rows, T past a token tile
    (50, 640, [14000, 6000, 1000], 32),  # three modules, one ragged
    (17, 128, [21000], 64),              # solo, one input group, 17 tokens (16 + 1)
    (33, 1024, [11000, 11000], 256),     # rank 256
]
# (T, d, rows, r): fewer than 160 row blocks, K split (ranges of input groups as the library picks)
SPLIT_CASES = [
    (48, 8320, [3000, 1500, 700], 16),   # 65 groups in five ranges of 13, ragged rows and tokens
    (57, 9600, [4096], 64),              # solo, 75 groups in ranges 6 x 11 + 9; 57 tokens
    (64, 8192, [4096], 256),             # rank 256, ranges 6 x 10 + 4
    (50, 8192, [3000, 1500, 1500], 64),  # three modules (layerwise: three projections), four ranges
    (56, 8192, [3000], 24),              # rank 24: a half-filled rank tile in every producer range
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    glowq()
    yield
    torch.cuda.synchronize()


def _call(g, unit, du, r, restore, ws):
    if unit.kind == "solo":
        return [g.solo_forward(du.x, du.w[0], du.b, du.a[0], r, restore, workspace=ws)]
    return g.group_forward(du.x, du.w, du.b, du.a, r, restore, workspace=ws)


@pytest.mark.parametrize("T,d,rows,r", CASES + SPLIT_CASES)
def test_mid_tile_matches_oracle(T, d, rows, r):
    g = glowq()
    log(f"mid tile T={T} d={d} rows={rows} r={r}")
    keys = (90, T, d)
    x = W.make_x(T, d, 0.81, keys, device="cuda")
    unit = W.make_unit("m", "group" if len(rows) > 1 else "solo", x, rows, r, keys, device="cuda",
                       layerwise=len(rows) > 1)
    du = DevUnit(unit, layerwise=len(rows) > 1)
    ws = g.make_workspace(T, r, len(rows))
    for restore in (True, False):
        ref = oracle_unit(unit, restore=restore)
        for rep in range(2):
            e0 = int(ws[:4].view(torch.int32).item())
            ys = _call(g, unit, du, r, restore, ws)
            torch.cuda.synchronize()
            assert int(ws[:4].view(torch.int32).item()) == e0 + (1 if restore else 0)
            for i, (y, yr) in enumerate(zip(ys, ref)):
                assert_parity(y, yr, f"mid T={T} d={d} r={r} restore={restore} rep {rep} module {i}")
            assert_handoff_ok(ws)
        # no workspace at all when not correcting
        if not restore:
            ys = _call(g, unit, du, r, False, None)
            for i, (y, yr) in enumerate(zip(ys, ref)):
                assert_parity(y, yr, f"mid T={T} no workspace module {i}")
    if unit.kind == "group":
        ref_lw = oracle_unit(unit, layerwise=True)
        ys = g.layerwise_forward(du.x, du.w, du.b_lw, du.a, r, True, workspace=ws)
        torch.cuda.synchronize()
        for i, (y, yr) in enumerate(zip(ys, ref_lw)):
            assert_parity(y, yr, f"mid layerwise T={T} module {i}")
        assert_handoff_ok(ws)
    hdr = ws[:WS_HEADER].view(torch.int32).cpu()
    assert int(hdr[1:].abs().sum()) == 0  # arrival counters back to zero


def test_mid_tile_is_deterministic():
    """Two calls on the same inputs give bitwise equal outputs (fixed-order sums)."""
    g = glowq()
    T, d, rows, r = 64, 512, [14000, 8000], 64
    keys = (91,)
    x = W.make_x(T, d, 1.05, keys, device="cuda")
    unit = W.make_unit("md", "group", x, rows, r, keys, device="cuda")
    du = DevUnit(unit)
    ws = g.make_workspace(T, r, 1)
    a = [y.clone() for y in g.group_forward(du.x, du.w, du.b, du.a, r, True, workspace=ws)]
    b = g.group_forward(du.x, du.w, du.b, du.a, r, True, workspace=ws)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    assert_handoff_ok(ws)


def test_mid_tile_llama3_gateup():
    """LLaMA-3.1-8B gate/up (4096 -> 2 x 14336) at T = 64, r = 64, correcting and not."""
    g = glowq()
    log("mid tile LLaMA-3.1-8B gate/up T=64")
    unit = W.llama3_gqa_units(64, 64, device="cuda", which=("gateup",))[0]
    du = DevUnit(unit)
    ws = g.make_workspace(64, 64, 1)
    for restore in (True, False):
        ref = oracle_unit(unit, restore=restore)
        ys = _call(g, unit, du, 64, restore, ws)
        torch.cuda.synchronize()
        for i, (y, yr) in enumerate(zip(ys, ref)):
            assert_parity(y, yr, f"mid gate/up restore={restore} module {i}")
        assert_handoff_ok(ws)


@pytest.mark.parametrize("which", ["down"])
def test_mid_split_llama3_units(which):
    """LLaMA-3.1-8B down_proj (14336 -> 4096) at T = 64, r = 64 and 128, on the K-split tile,
    correcting and not; twice in a row on one workspace."""
    g = glowq()
    for r in (64, 128):
        log(f"mid split LLaMA-3.1-8B {which} T=64 r={r}")
        unit = W.llama3_gqa_units(64, r, device="cuda", which=(which,))[0]
        du = DevUnit(unit)
        ws = g.make_workspace(64, r, 1)
        for restore in (True, False):
            ref = oracle_unit(unit, restore=restore)
            for rep in range(2):
                ys = _call(g, unit, du, r, restore, ws)
                torch.cuda.synchronize()
                for i, (y, yr) in enumerate(zip(ys, ref)):
                    assert_parity(y, yr, f"mid split {which} r={r} restore={restore} rep {rep} module {i}")
                assert_handoff_ok(ws)


def test_mid_split_is_deterministic():
    """K-split calls give bitwise equal outputs call after call (ranges added in a fixed order)."""
    g = glowq()
    T, d, rows, r = 48, 8192, [2048, 1024], 64
    keys = (92,)
    x = W.make_x(T, d, 0.77, keys, device="cuda")
    unit = W.make_unit("ms", "group", x, rows, r, keys, device="cuda")
    du = DevUnit(unit)
    ws = g.make_workspace(T, r, 1)
    a = [y.clone() for y in g.group_forward(du.x, du.w, du.b, du.a, r, True, workspace=ws)]
    b = g.group_forward(du.x, du.w, du.b, du.a, r, True, workspace=ws)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    assert_handoff_ok(ws)
