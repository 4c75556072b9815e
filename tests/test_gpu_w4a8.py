"""W4A8 group forward (glowq_group_forward_w4a8) against the fp64 oracle through the C ABI.

Bar: the per-token integer codes, code sums and fp32 scales the library writes to its workspace
are bit-exact against oracle.glowq_ref.quantize_x_int8 (the quantiser's integer decisions are
taken in fp32 on both sides); outputs within relative Frobenius 1e-3 and max-abs 1e-2 * max|y| of
oracle.glowq_ref.group_forward_w4a8."""
import numpy as np
import pytest
import torch

import workload as W
from gpu_util import assert_parity, glowq, log
from oracle import glowq_ref as G

pytestmark = pytest.mark.gpu

PERM = [0, 4, 1, 5, 2, 6, 3, 7]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    glowq()
    yield
    torch.cuda.synchronize()


def natural_from_layout(codes_pos: np.ndarray, d: int) -> np.ndarray:
    """Undo the documented operand order: position 16 (4 m + g) + 8 h + b of each 128-input group
    holds input 64 m + 32 h + 8 g + PERM[b]."""
    T = codes_pos.shape[0]
    out = np.zeros_like(codes_pos)
    for pos in range(128):
        q, rem = divmod(pos, 16)
        m, g = divmod(q, 4)
        h, b = divmod(rem, 8)
        k = 64 * m + 32 * h + 8 * g + PERM[b]
        out[:, k::128] = codes_pos[:, pos::128]
    return out


def r256(n):
    return (n + 255) // 256 * 256


def run_unit(unit, restore=True, r=None):
    g = glowq()
    r = unit.r if r is None else r
    x = unit.x.cuda().contiguous()
    w = [g.QWeight.from_workload(q) for q in unit.weights]
    a = [t.cuda().contiguous() for t in unit.a]
    b = unit.b.cuda().contiguous()
    T, d = x.shape
    ws = torch.empty(max(g.w4a8_workspace_bytes(T, d, r if restore else 0), 256), dtype=torch.uint8, device="cuda")
    ys = g.group_forward_w4a8(x, w, b, a, r, restore, workspace=ws)
    torch.cuda.synchronize()
    return ys, ws


def oracle(unit, restore=True, r=None, rows=None):
    r = unit.r if r is None else r
    x = unit.x if rows is None else unit.x[rows]
    w_hats = [G.dequant_qw(q) for q in unit.weights]
    b = unit.b if r > 0 else None
    return G.group_forward_w4a8(x, w_hats, b, unit.a, restore and r > 0)


def check_codes(unit, ws):
    T, d = unit.x.shape
    Gn = d // 128
    codes_ref, scale_ref = G.quantize_x_int8(unit.x)
    raw = ws.cpu().numpy()
    codes = natural_from_layout(raw[: T * d].view(np.int8).reshape(T, d).astype(np.int64), d)
    assert np.array_equal(codes, codes_ref), np.argwhere(codes != codes_ref)[:5]
    o = r256(T * d)
    sums = raw[o: o + T * Gn * 4].view(np.int32).reshape(T, Gn)
    assert np.array_equal(sums, codes_ref.reshape(T, Gn, 128).sum(axis=2))
    o += r256(T * Gn * 4)
    scales = raw[o: o + T * 4].view(np.float32)
    assert np.array_equal(scales.view(np.uint32), scale_ref.astype(np.float32).view(np.uint32))


# (T, d, rows, r): decode-sized (one token tile), 17-32 and 33+ token tiles, ragged tokens and
# rows, every tile shape the planner picks (128 / 64 rows, one, two or four wave groups)
SHAPES = [(1, 256, [256, 256, 256], 16), (3, 384, [40, 24], 8), (16, 1024, [520, 17], 64),
          (17, 512, [96, 64, 40], 32), (33, 640, [100], 24), (64, 1024, [1024, 512, 512], 64),
          (65, 256, [48, 32], 16), (130, 384, [300, 200], 40), (300, 512, [2048, 2048], 128),
          (8, 2048, [64], 256)]


@pytest.mark.parametrize("T,d,rows,r", SHAPES)
def test_w4a8_matches_oracle(T, d, rows, r):
    keys = (50, T, d)
    x = W.make_x(T, d, 1.19, keys)
    unit = W.make_unit("w8", "group", x, rows, r, keys)
    for restore in (True, False):
        ys, ws = run_unit(unit, restore)
        check_codes(unit, ws)
        for i, (y, yr) in enumerate(zip(ys, oracle(unit, restore))):
            assert_parity(y, yr, f"w4a8 T={T} d={d} r={r} restore={restore} module {i}")


def test_w4a8_rank_zero_zero_rows_and_empty():
    g = glowq()
    keys = (51,)
    T, d = 24, 512
    x = W.make_x(T, d, 0.77, keys)
    x[5] = 0          # a zero token: scale 0, codes 0, output = its correction only
    x[17, :] = 0
    x[17, 3] = 2.0    # a one-hot token
    unit = W.make_unit("w8z", "group", x, [96, 33], 16, keys)
    ys, ws = run_unit(unit, True)
    check_codes(unit, ws)
    for i, (y, yr) in enumerate(zip(ys, oracle(unit, True))):
        assert_parity(y, yr, f"w4a8 zero rows module {i}")
    ys, ws = run_unit(unit, True, r=0)
    for i, (y, yr) in enumerate(zip(ys, oracle(unit, True, r=0))):
        assert_parity(y, yr, f"w4a8 r=0 module {i}")
    e = unit.x[:0]
    w = [g.QWeight.from_workload(q) for q in unit.weights]
    out = g.group_forward_w4a8(e.cuda(), w, unit.b.cuda(), [t.cuda() for t in unit.a], 16, True)
    assert all(o.shape[0] == 0 for o in out)


def test_w4a8_widest_input():
    """d = 16384, the largest the quantiser holds in registers, with a ragged token count."""
    keys = (52,)
    x = W.make_x(5, 16384, 0.77, keys)
    unit = W.make_unit("w8w", "solo", x, [272], 64, keys)
    ys, ws = run_unit(unit, True)
    check_codes(unit, ws)
    assert_parity(ys[0], oracle(unit, True)[0], "w4a8 d=16384")


@pytest.mark.parametrize("T", [1, 16, 64])
def test_w4a8_llama_qkv(T):
    """LLaMA-2-7B QKV group (d = 4096, 3 x 4096 rows, r = 64) at decode and batched-decode sizes."""
    keys = (53, T)
    x = W.make_x(T, 4096, 1.19, keys, device="cuda")
    unit = W.make_unit("w8q", "group", x, [4096, 4096, 4096], 64, keys, device="cuda")
    ys, ws = run_unit(unit, True)
    check_codes(unit, ws)
    for i, (y, yr) in enumerate(zip(ys, oracle(unit, True))):
        assert_parity(y, yr, f"w4a8 qkv T={T} module {i}")


def test_w4a8_gateup_prefill_sampled():
    """LLaMA-2-7B gate/up group at T = 2048 (r = 64), 40 sampled tokens against the oracle (rows
    are independent: each token's codes, product and correction use that token alone)."""
    keys = (54,)
    T = 2048
    x = W.make_x(T, 4096, 0.77, keys, device="cuda")
    unit = W.make_unit("w8g", "group", x, [11008, 11008], 64, keys, device="cuda")
    ys, ws = run_unit(unit, True)
    rows = np.sort(np.random.default_rng(3).choice(T, 40, replace=False))
    rows[-1] = T - 1
    ref = oracle(unit, True, rows=torch.from_numpy(rows).cuda())
    for i, (y, yr) in enumerate(zip(ys, ref)):
        assert_parity(y[rows], yr, f"w4a8 gate/up T=2048 module {i}")
    codes_ref, scale_ref = G.quantize_x_int8(unit.x[torch.from_numpy(rows).cuda()])
    raw = ws.cpu().numpy()
    o = r256(T * 4096) + r256(T * 32 * 4)
    scales = raw[o: o + T * 4].view(np.float32)[rows]
    assert np.array_equal(scales.view(np.uint32), scale_ref.astype(np.float32).view(np.uint32))


def test_w4a8_deterministic():
    keys = (55,)
    x = W.make_x(200, 1024, 0.77, keys)
    unit = W.make_unit("w8d", "group", x, [640, 320], 32, keys)
    a, _ = run_unit(unit, True)
    b, _ = run_unit(unit, True)
    for u, v in zip(a, b):
        assert torch.equal(u, v)
