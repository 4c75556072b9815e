"""Helpers for GPU parity tests: move a workload unit to the device through the library's
repack, run it through the C ABI, compare with the fp64 oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import glowq_ref as G

REL_FRO_TOL = 1e-3   # relative Frobenius error bound on every module output
MAX_ABS_TOL = 1e-2   # max elementwise error bound, relative to max|y|


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def glowq():
    from rank_error_compensation_amd import glowq as g
    g.lib()
    return g


class DevUnit:
    """Device copies of a workload Unit."""

    def __init__(self, unit, layerwise: bool = False):
        g = glowq()
        self.unit = unit
        self.x = unit.x.cuda().contiguous()
        self.w = [g.QWeight.from_workload(q) for q in unit.weights]
        self.a = [t.cuda().contiguous() for t in unit.a]
        self.b = unit.b.cuda().contiguous()
        self.b_lw = [t.cuda().contiguous() for t in unit.b_layerwise] if (layerwise and unit.b_layerwise) else None
        self.r = unit.r

    def forward(self, restore=None, r=None, x=None):
        g = glowq()
        restore = self.unit.restore if restore is None else restore
        r = self.r if r is None else r
        x = self.x if x is None else x
        ws = g.make_workspace(x.shape[0], r, 1, x.device) if (restore and r > 0) else None
        if self.unit.kind == "solo":
            ys = [g.solo_forward(x, self.w[0], self.b, self.a[0], r, restore, workspace=ws)]
        else:
            ys = g.group_forward(x, self.w, self.b, self.a, r, restore, workspace=ws)
        assert_handoff_ok(ws)
        return ys

    def forward_layerwise(self, restore=True):
        g = glowq()
        ws = g.make_workspace(self.x.shape[0], self.r, len(self.w), self.x.device) if (restore and self.r > 0) else None
        ys = g.layerwise_forward(self.x, self.w, self.b_lw, self.a, self.r, restore, workspace=ws)
        assert_handoff_ok(ws)
        return ys


def assert_handoff_ok(ws):
    """No bounded wait of the projection hand-off expired in the calls on `ws` since the last
    check (glowq_workspace_status, which synchronises and clears the word)."""
    if ws is not None:
        g = glowq()
        assert g.workspace_status(ws) == g.OK, "a hand-off wait expired"


def oracle_unit(unit, restore=None, layerwise=False, rows=None, r=None):
    """fp64 oracle outputs; rows selects a subset of tokens (rows are independent)."""
    restore = unit.restore if restore is None else restore
    x = unit.x if rows is None else unit.x[rows]
    w_hats = [G.dequant_qw(q) for q in unit.weights]
    use_r = unit.r if r is None else r
    if layerwise:
        return G.layerwise_forward(x, w_hats, unit.b_layerwise, unit.a, restore and use_r > 0)
    b = unit.b if use_r > 0 else None
    return G.group_forward(x, w_hats, b, unit.a, restore and use_r > 0)


def assert_parity(y_gpu, y_ref, what: str):
    yg = y_gpu.float().cpu().numpy().astype(np.float64)
    assert yg.shape == y_ref.shape, (what, yg.shape, y_ref.shape)
    assert np.all(np.isfinite(yg)), what
    e = G.parity_errors(yg, y_ref)
    log(f"  {what}: rel_fro={e['rel_fro']:.3e} max_abs_rel={e['max_abs_rel']:.3e}")
    assert e["rel_fro"] <= REL_FRO_TOL, (what, e)
    assert e["max_abs_rel"] <= MAX_ABS_TOL, (what, e)
    return e
