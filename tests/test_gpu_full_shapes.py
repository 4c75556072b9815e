"""Full-size workloads through the C ABI against the fp64 oracle (needs gfx950).

* the 32-layer LLaMA-2-7B linear path's schedule (glowq_path_forward) on a window of layers with
  the restore mask, at decode T = 1 (every output) and prefill T = 512 (sampled tokens: rows of
  the output are independent, so the oracle computes only the sampled ones);
* LLaMA-3.1-8B GQA shapes at T = 64 (batched decode) and T = 4096 (sampled tokens), r = 64, 128;
* the layerwise baseline at full QKV decode shape.
Bar: relative Frobenius error <= 1e-3 and max-abs error <= 1e-2 max|y| per module.
"""
import numpy as np
import pytest
import torch

import workload as W
from gpu_util import DevUnit, assert_parity, glowq, log, oracle_unit
from oracle import glowq_ref as G

pytestmark = [pytest.mark.gpu]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    glowq()
    yield
    torch.cuda.synchronize()


def _sample_rows(T, n, seed):
    if T <= n:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(T, size=n, replace=False))
    rows[0], rows[-1] = 0, T - 1  # always include the first and last token (ragged tail)
    return np.unique(rows)


@pytest.mark.parametrize("T", [1, 512])
def test_llama2_path_window(T):
    """Layers 0..3 of the path run as one schedule (QKV group, o_proj solo, gate/up group,
    down_proj solo per layer) with the restore mask of the full 32-layer path."""
    g = glowq()
    layers = [0, 1, 2, 3]
    log(f"generating 32-layer path inputs, layers {layers} T={T}")
    units, mask = W.llama2_path_inputs(T, device="cuda", layers=layers)
    assert sum(mask) == 16
    assert any(mask[l] for l in layers) and not all(mask[l] for l in layers), "window mixes restored/unrestored"
    plan_units, devs = [], []
    for l in layers:
        for u in units[l]:
            du = DevUnit(u)
            ys = [torch.empty(T, q.n_out, dtype=torch.float16, device="cuda") for q in u.weights]
            kind = g.UNIT_GROUP if u.kind == "group" else g.UNIT_SOLO
            plan_units.append(g.PathUnit(kind, du.x, du.w, du.b, du.a, u.r, bool(mask[l]), ys))
            devs.append((l, u))
    plan = g.PathPlan(plan_units)
    plan.run()
    plan.run()  # twice: the schedule is re-runnable on one workspace
    torch.cuda.synchronize()
    rows = _sample_rows(T, 32, 3)
    for pu, (l, u) in zip(plan_units, devs):
        ref = oracle_unit(u, restore=bool(mask[l]), rows=rows)
        for i, (y, yr) in enumerate(zip(pu.y, ref)):
            assert_parity(y[torch.from_numpy(rows).cuda()], yr,
                          f"path T={T} layer {l} {u.name}[{i}] restore={mask[l]}")


@pytest.mark.parametrize("T,r", [(64, 64), (64, 128), (4096, 64), (4096, 128)])
def test_llama3_gqa(T, r):
    log(f"generating GQA units T={T} r={r}")
    units = W.llama3_gqa_units(T, r, device="cuda")
    rows = _sample_rows(T, 48, 4)
    for u in units:
        du = DevUnit(u)
        ys = du.forward()
        torch.cuda.synchronize()
        ref = oracle_unit(u, rows=rows)
        for i, (y, yr) in enumerate(zip(ys, ref)):
            assert_parity(y[torch.from_numpy(rows).cuda()], yr, f"gqa T={T} r={r} {u.name}[{i}]")


@pytest.mark.parametrize("T", [1, 16])
def test_llama2_qkv_layerwise_full(T):
    """The layerwise baseline (one projection per module) at the full QKV shape."""
    unit = W.llama2_qkv_unit(T, device="cuda", layerwise=True)
    du = DevUnit(unit, layerwise=True)
    ys = du.forward_layerwise()
    ref = oracle_unit(unit, layerwise=True)
    for i, (y, yr) in enumerate(zip(ys, ref)):
        assert_parity(y, yr, f"qkv layerwise T={T} module {i}")


def test_prefill_deterministic_and_row_independent():
    """Prefill results are bitwise repeatable, and a token's output does not depend on the other
    tokens of the batch (the first 300 tokens alone give the same rows as the full batch)."""
    g = glowq()
    unit = W.llama2_gateup_unit(700, device="cuda")
    du = DevUnit(unit)
    y1 = [t.clone() for t in du.forward()]
    y2 = du.forward()
    for a, b in zip(y1, y2):
        assert torch.equal(a, b)
    ys = du.forward(x=du.x[:300].contiguous())
    for a, b in zip(ys, y1):
        e = G.parity_errors(a.float().cpu().numpy(), b[:300].float().cpu().numpy().astype(np.float64))
        assert e["rel_fro"] <= 1e-3


def test_path_graph_replay_matches_eager():
    """The decode schedule (layers 0..3, T = 1, mixed restore bits) captured in a HIP graph: every
    replay, with eager work and synchronisation between replays, reproduces the eager outputs
    bitwise (the hand-off's epoch lives in the workspace, so replays never reuse a tag)."""
    g = glowq()
    layers, T = [0, 1, 2, 3], 1
    units, mask = W.llama2_path_inputs(T, device="cuda", layers=layers)
    plan_units = []
    for l in layers:
        for u in units[l]:
            du = DevUnit(u)
            ys = [torch.empty(T, q.n_out, dtype=torch.float16, device="cuda") for q in u.weights]
            kind = g.UNIT_GROUP if u.kind == "group" else g.UNIT_SOLO
            plan_units.append(g.PathUnit(kind, du.x, du.w, du.b, du.a, u.r, bool(mask[l]), ys))
    plan = g.PathPlan(plan_units)
    plan.run()
    torch.cuda.synchronize()
    ref = [y.clone() for pu in plan_units for y in pu.y]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan.run()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan.run()
    torch.cuda.synchronize()
    for rep in range(4):
        for pu in plan_units:
            for y in pu.y:
                y.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [y for pu in plan_units for y in pu.y]
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), f"replay {rep}: output {i} differs from the eager run"
