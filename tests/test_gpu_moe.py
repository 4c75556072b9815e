"""Mixture-of-experts forward (glowq_moe_forward) against the fp64 oracle through the C ABI.

Bar: every routed row's outputs within relative Frobenius 1e-3 and max-abs 1e-2 * max|y| of
oracle.glowq_ref.moe_forward (per module, over all rows); at the Qwen1.5-MoE-A2.7B shapes the
oracle runs on the rows of sampled experts (rows are independent, and an expert's rows use that
expert's weights alone)."""
import numpy as np
import pytest
import torch

import workload as W
from gpu_util import assert_parity, glowq, log
from oracle import glowq_ref as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    glowq()
    yield
    torch.cuda.synchronize()


class MoeCase:
    """n_exp experts of m modules (rows n_outs) over d inputs, rank r, stacked on the device."""

    def __init__(self, n_exp, d, n_outs, r, keys, device="cpu", alpha=0.77):
        g = glowq()
        self.n_exp, self.d, self.n_outs, self.r = n_exp, d, list(n_outs), r
        self.units = []
        for e in range(n_exp):
            xdummy = torch.zeros(1, d, dtype=torch.float16, device=device)
            self.units.append(W.make_unit(f"e{e}", "group", xdummy, n_outs, r, tuple(keys) + (e,), device=device))
        self.qw = [[g.QWeight.from_workload(u.weights[i]) for u in self.units] for i in range(len(n_outs))]
        self.mods = [g.MoeModule.stack(self.qw[i], [u.a[i].cuda() for u in self.units]) for i in range(len(n_outs))]
        self.b_exp = torch.stack([u.b.cuda() for u in self.units]).contiguous()
        self.b_all = self.units[0].b.cuda().contiguous()

    def w_hats(self, experts):
        return {e: [G.dequant_qw(q) for q in self.units[e].weights] for e in experts}

    def run(self, x, row_token, offsets, share, restore=True, r=None):
        g = glowq()
        r = self.r if r is None else r
        n_rows = int(offsets[-1])
        b = self.b_all if share == g.MOE_SHARE_ALL else self.b_exp
        ws = g.make_workspace(1, 8, 1, min_bytes=g.moe_workspace_bytes(n_rows, x.shape[0], r if restore else 0, share))
        ys = g.moe_forward(x.cuda(), self.n_exp, self.mods, b, share, r, restore,
                           None if row_token is None else row_token.cuda(), offsets.cuda(), n_rows, workspace=ws)
        torch.cuda.synchronize()
        return ys, ws

    def oracle_rows(self, x, row_token, offsets, share, experts, restore=True):
        """Oracle outputs of the rows of `experts` (dict e -> list of module outputs)."""
        wh = self.w_hats(experts)
        out = {}
        for e in experts:
            lo, hi = int(offsets[e]), int(offsets[e + 1])
            rows = x[row_token[lo:hi].long()] if row_token is not None else x[lo:hi]
            if share == glowq().MOE_SHARE_ALL:
                b = self.units[0].b
            else:
                b = self.units[e].b
            # through the pinned MoE oracle on a one-expert routing of these rows
            off1 = np.array([0, hi - lo], dtype=np.int32)
            out[e] = G.moe_forward(rows, None, off1, [wh[e]], b if share == 1 else [b],
                                   [self.units[e].a], restore=restore, share="all" if share == 1 else "expert")
        return out


def check(case, ys, x, row_token, offsets, share, experts, restore=True, label=""):
    ref = case.oracle_rows(x, row_token, offsets, share, experts, restore)
    for e in experts:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        for i in range(len(case.n_outs)):
            assert_parity(ys[i][lo:hi], ref[e][i], f"{label} expert {e} module {i}")


@pytest.mark.parametrize("share", [0, 1], ids=["per_expert", "all_experts"])
@pytest.mark.parametrize("T,top", [(1, 2), (37, 2), (150, 3), (300, 2)])
def test_moe_small_all_rows(share, T, top):
    """8 experts (expert 2 receives no token), gate/up group of 96 + 80 rows at d = 512, r = 16:
    every routed row against the oracle, restore on and off."""
    case = MoeCase(8, 512, [96, 80], 16, (70, T))
    x = W.make_x(T, 512, 0.77, (70, T))
    row_token, offsets = W.moe_routing(T, 8, top, (70, T), skip=[2])
    for restore in (True, False):
        ys, ws = case.run(x, row_token, offsets, share, restore)
        assert glowq().workspace_status(ws) == glowq().OK
        check(case, ys, x, row_token, offsets, share, range(8), restore, f"T={T} share={share} restore={restore}")


@pytest.mark.parametrize("r", [128, 256])
def test_moe_projection_wide_rank_few_rows(r):
    """Few routed rows per expert (the projection splits the rank columns over the waves) at ranks
    that give each wave two and four 16-column tiles: every routed row against the oracle."""
    case = MoeCase(8, 512, [96, 80], r, (73, r))
    x = W.make_x(9, 512, 0.77, (73, r))
    row_token, offsets = W.moe_routing(9, 8, 2, (73, r), skip=[5])
    ys, ws = case.run(x, row_token, offsets, 0, True)
    assert glowq().workspace_status(ws) == glowq().OK
    check(case, ys, x, row_token, offsets, 0, range(8), True, f"few rows r={r}")


def test_moe_down_solo_routed_order():
    """The down projection: one module per expert on its hidden rows, already in routed order
    (no token indices), 6 experts of 64 rows at d = 384, r = 24."""
    case = MoeCase(6, 384, [64], 24, (71,))
    row_token, offsets = W.moe_routing(40, 6, 2, (71,))
    n_rows = int(offsets[-1])
    h = W.make_x(n_rows, 384, 0.77, (71, 1))
    ys, ws = case.run(h, None, offsets, 0, True)
    check(case, ys, h, None, offsets, 0, range(6), True, "down")


@pytest.mark.parametrize("T", [1, 64, 512, 2048])
def test_moe_qwen_gateup_sampled(T):
    """Qwen1.5-MoE-A2.7B MLP: 60 experts, gate/up 2 x 1408 rows over d = 2048, top-4 routing,
    r = 64, per-expert shared basis; the rows of 6 experts (the busiest, the last and some
    others) against the oracle."""
    g = glowq()
    case = MoeCase(60, 2048, [1408, 1408], 64, (72,), device="cuda")
    x = W.make_x(T, 2048, 0.77, (72, T), device="cuda")
    row_token, offsets = W.moe_routing(T, 60, 4, (72, T))
    counts = np.diff(offsets.numpy())
    experts = sorted(set([int(np.argmax(counts)), 59, 0, 17] + [int(e) for e in np.nonzero(counts)[0][:2]]))
    for share in (0, 1):
        ys, ws = case.run(x, row_token, offsets, share, True)
        assert g.workspace_status(ws) == g.OK
        log(f"qwen moe T={T} share={share} rows={int(offsets[-1])} experts checked {experts}")
        check(case, ys, x.cpu(), row_token, offsets, share, experts, True, f"qwen T={T} share={share}")


def test_moe_bad_routing_is_reported_and_clamped():
    """Routing data out of range -- a token index equal to T, offsets that end past n_rows -- is
    clamped inside the kernels (no out-of-bounds access) and reported as GLOWQ_ERR_ROUTING."""
    g = glowq()
    case = MoeCase(4, 256, [32, 32], 8, (73,))
    x = W.make_x(10, 256, 0.77, (73,))
    row_token, offsets = W.moe_routing(10, 4, 2, (73,))
    bad_tok = row_token.clone()
    bad_tok[3] = 10
    ys, ws = case.run(x, bad_tok, offsets, 0, True)
    assert g.workspace_status(ws) == g.ERR_ROUTING
    assert g.workspace_status(ws) == g.OK  # cleared
    bad_off = offsets.clone()
    bad_off[2] = int(offsets[-1]) + 5  # beyond n_rows (clamped)
    ys, ws = case.run(x, row_token, bad_off, 0, True)
    assert g.workspace_status(ws) == g.ERR_ROUTING


def test_moe_empty_and_deterministic():
    g = glowq()
    case = MoeCase(4, 256, [48, 32], 16, (74,))
    x = W.make_x(33, 256, 0.77, (74,))
    row_token, offsets = W.moe_routing(33, 4, 2, (74,))
    a, _ = case.run(x, row_token, offsets, 0, True)
    b, _ = case.run(x, row_token, offsets, 0, True)
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    zero_off = torch.zeros(5, dtype=torch.int32)
    ys, _ = case.run(x, row_token[:0], zero_off, 0, True)
    assert all(y.shape[0] == 0 for y in ys)
