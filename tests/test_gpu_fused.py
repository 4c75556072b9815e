"""17 to 64 tokens on the prefill tiles with the projection formed inside the launch (producer
workgroups handing R over as tagged pairs): every module against the fp64 oracle, the epoch
advancing once per correcting call, group and layerwise, ranks up to 256, repeated calls on one
workspace and replays of a captured graph.

Bar: relative Frobenius error <= 1e-3 and max-abs error <= 1e-2 max|y| per module."""
import pytest
import torch

import workload as W
from gpu_util import DevUnit, assert_handoff_ok, assert_parity, glowq, log, oracle_unit

pytestmark = pytest.mark.gpu
WS_HEADER = 8192


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    glowq()
    yield
    torch.cuda.synchronize()


# (T, d, rows, r): >= 40 row tiles of 128, so these calls take the prefill tiles; T <= 64 fuses
CASES = [(17, 512, [3000, 2500], 16), (40, 1024, [2048, 2048, 1024], 64), (64, 384, [5200], 256),
         (33, 2048, [4096, 1024, 1024], 128), (64, 1024, [14336 // 2, 14336 // 2], 64)]


@pytest.mark.parametrize("T,d,rows,r", CASES)
def test_fused_matches_oracle_and_advances_epoch(T, d, rows, r):
    g = glowq()
    keys = (80, T, d)
    x = W.make_x(T, d, 0.77, keys, device="cuda")
    unit = W.make_unit("f", "group" if len(rows) > 1 else "solo", x, rows, r, keys, device="cuda", layerwise=True)
    du = DevUnit(unit, layerwise=True)
    ref = oracle_unit(unit)
    ws = g.make_workspace(T, r, len(rows))
    for rep in range(3):
        e0 = int(ws[:4].view(torch.int32).item())
        if unit.kind == "solo":
            ys = [g.solo_forward(du.x, du.w[0], du.b, du.a[0], r, True, workspace=ws)]
        else:
            ys = g.group_forward(du.x, du.w, du.b, du.a, r, True, workspace=ws)
        torch.cuda.synchronize()
        assert int(ws[:4].view(torch.int32).item()) == e0 + 1  # one epoch step per correcting call
        for i, (y, yr) in enumerate(zip(ys, ref)):
            assert_parity(y, yr, f"fused T={T} d={d} r={r} rep {rep} module {i}")
        assert_handoff_ok(ws)
    if unit.kind == "group":
        ref_lw = oracle_unit(unit, layerwise=True)
        ys = g.layerwise_forward(du.x, du.w, du.b_lw, du.a, r, True, workspace=ws)
        torch.cuda.synchronize()
        for i, (y, yr) in enumerate(zip(ys, ref_lw)):
            assert_parity(y, yr, f"fused layerwise T={T} module {i}")
        assert_handoff_ok(ws)
    hdr = ws[:WS_HEADER].view(torch.int32).cpu()
    assert int(hdr[1:].abs().sum()) == 0  # arrival counters back to zero


def test_fused_graph_replay_matches_eager():
    """A fused call captured in a HIP graph: every replay (eager work between replays) equals the
    eager result bitwise."""
    g = glowq()
    T, d, rows, r = 48, 1024, [3072, 3072], 64
    keys = (81,)
    x = W.make_x(T, d, 1.19, keys, device="cuda")
    unit = W.make_unit("fg", "group", x, rows, r, keys, device="cuda")
    du = DevUnit(unit)
    ws = g.make_workspace(T, r, 1)
    ys = [torch.empty(T, n, dtype=torch.float16, device="cuda") for n in rows]
    g.group_forward(du.x, du.w, du.b, du.a, r, True, workspace=ws, y=ys)
    torch.cuda.synchronize()
    eager = [y.clone() for y in ys]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g.group_forward(du.x, du.w, du.b, du.a, r, True, workspace=ws, y=ys)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g.group_forward(du.x, du.w, du.b, du.a, r, True, workspace=ws, y=ys)
    for rep in range(4):
        for y in ys:
            y.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(ys, eager):
            assert torch.equal(a, b), rep
        g.group_forward(du.x, du.w, du.b, du.a, r, False, workspace=ws)  # eager work between replays
    assert_handoff_ok(ws)
    for i, (y, yr) in enumerate(zip(eager, oracle_unit(unit))):
        assert_parity(y, yr, f"fused graph module {i}")
