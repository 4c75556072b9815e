"""MX weights (MXFP4, MXFP6 E2M3 / E3M2) x MXFP8 activations (glowq_group_forward_mx8) against the
fp64 oracle through the C ABI.

Bar: the E4M3 codes and E8M0 block scales the library writes to its workspace are bit-exact
against oracle.glowq_ref.quantize_x_mxfp8 (every step of the conversion is exact on both sides);
outputs within relative Frobenius 1e-3 and max-abs 1e-2 * max|y| of
oracle.glowq_ref.group_forward_mx8 on the dequantised MX weights."""
import numpy as np
import pytest
import torch

import workload as W
from gpu_util import assert_parity, glowq
from oracle import glowq_ref as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    glowq()
    yield
    torch.cuda.synchronize()


def r256(n):
    return (n + 255) // 256 * 256


def natural_from_operand_order(pos: np.ndarray) -> np.ndarray:
    """Undo the documented operand order: byte 32 h + p of each 128-input group holds input
    32 g + n with g = 2 (p / 16) + h / 2 and n = 16 (h % 2) + p % 16."""
    out = np.zeros_like(pos)
    for q in range(128):
        h, p = divmod(q, 32)
        g, n = 2 * (p // 16) + h // 2, 16 * (h % 2) + p % 16
        out[:, 32 * g + n::128] = pos[:, q::128]
    return out


def run_unit(unit, restore=True, r=None):
    g = glowq()
    r = unit.r if r is None else r
    x = unit.x.cuda().contiguous()
    w = [g.QWeight.from_workload(q) for q in unit.weights]
    a = [t.cuda().contiguous() for t in unit.a]
    b = unit.b.cuda().contiguous()
    T, d = x.shape
    ws = torch.empty(max(g.mx8_workspace_bytes(T, d, r if restore else 0), 256), dtype=torch.uint8, device="cuda")
    ys = g.group_forward_mx8(x, w, b, a, r, restore, workspace=ws)
    torch.cuda.synchronize()
    return ys, ws


def oracle(unit, restore=True, r=None, rows=None):
    r = unit.r if r is None else r
    x = unit.x if rows is None else unit.x[rows]
    w_hats = [G.dequant_qw(q) for q in unit.weights]
    return G.group_forward_mx8(x, w_hats, unit.b if r > 0 else None, unit.a, restore and r > 0)


def natural_scales(raw: np.ndarray, T: int, d: int) -> np.ndarray:
    """Undo the documented scale records: per 128-token block and group a 512-byte record, the scale
    of token t and block g of the group at byte 8 (16 g + t % 16) + (t % 128) / 16."""
    n_groups = d // 128
    t = np.arange(T)[:, None]
    b = np.arange(d // 32)[None, :]
    pos = ((t // 128) * n_groups + b // 4) * 512 + 8 * (16 * (b % 4) + t % 16) + (t % 128) // 16
    return raw[pos]


def check_codes(unit, ws, rows=None):
    T, d = unit.x.shape
    x = unit.x if rows is None else unit.x[torch.as_tensor(rows, device=unit.x.device)]
    codes_ref, scales_ref = G.quantize_x_mxfp8(x)
    raw = ws.cpu().numpy()
    codes = natural_from_operand_order(raw[: T * d].reshape(T, d))
    scales = natural_scales(raw[r256(T * d):], T, d)
    if rows is not None:
        codes, scales = codes[rows], scales[rows]
    assert np.array_equal(codes, codes_ref), np.argwhere(codes != codes_ref)[:5]
    assert np.array_equal(scales, scales_ref), np.argwhere(scales != scales_ref)[:5]


# (T, d, rows, r): decode-sized (one token tile), 17-32 and 33+ token tiles, ragged tokens and
# rows, each tile shape the planner picks (128 / 64 rows, one, two or four wave groups)
SHAPES = [(1, 256, [256, 256, 256], 16), (3, 384, [40, 24], 8), (16, 1024, [520, 17], 64),
          (17, 512, [96, 64, 40], 32), (33, 640, [100], 24), (64, 1024, [1024, 512, 512], 64),
          (65, 256, [48, 32], 16), (130, 384, [300, 200], 40), (300, 512, [2048, 2048], 128),
          (8, 2048, [64], 256),
          # wide tiles (128 tokens x 512 rows, at least 256 of them): ragged tokens and rows, group
          # counts 2, 5, 6, 11 against the three-stage ring (tails of 2, 2, 0 and 2 groups)
          (260, 640, [22000, 21000, 1000], 64), (129, 256, [32784, 32760], 256),
          (200, 768, [33000, 33000], 32), (520, 1408, [13000, 13600], 24),
          # token blocks a multiple of 4 (the XCD quarter mapping), an odd number of row blocks
          (500, 256, [16400, 16000], 16)]


@pytest.mark.parametrize("T,d,rows,r", SHAPES)
def test_mx8_matches_oracle(T, d, rows, r):
    keys = (60, T, d)
    x = W.make_x(T, d, 1.19, keys)
    unit = W.make_unit("m8", "group", x, rows, r, keys, fmt="mxfp4")
    for restore in (True, False):
        ys, ws = run_unit(unit, restore)
        check_codes(unit, ws)
        for i, (y, yr) in enumerate(zip(ys, oracle(unit, restore))):
            assert_parity(y, yr, f"mx8 T={T} d={d} r={r} restore={restore} module {i}")


def test_mx8_zero_and_extreme_rows_rank_zero_and_empty():
    """A zero token (zero-scale blocks: smallest scale byte, zero codes), a one-hot token, a token of
    the largest fp16 magnitudes (saturation at 448 with a scale of 2^7) and one of fp16 subnormals;
    rank 0; an empty call."""
    g = glowq()
    keys = (61,)
    T, d = 24, 512
    x = W.make_x(T, d, 0.77, keys)
    x[5] = 0
    x[17, :] = 0
    x[17, 3] = 2.0
    x[9, :] = 65504.0
    x[9, 1::3] = -60000.0
    x[11, :] = torch.tensor(2.0 ** -24, dtype=torch.float16)
    unit = W.make_unit("m8z", "group", x, [96, 33], 16, keys, fmt="mxfp4")
    ys, ws = run_unit(unit, True)
    check_codes(unit, ws)
    for i, (y, yr) in enumerate(zip(ys, oracle(unit, True))):
        keep = [t for t in range(T) if t != 9]  # the saturated token's outputs overflow fp16
        assert_parity(y[keep], yr[keep], f"mx8 extreme rows module {i}")
    ys, ws = run_unit(unit, True, r=0)
    for i, (y, yr) in enumerate(zip(ys, oracle(unit, True, r=0))):
        keep = [t for t in range(T) if t != 9]
        assert_parity(y[keep], yr[keep], f"mx8 r=0 module {i}")
    e = unit.x[:0]
    w = [g.QWeight.from_workload(q) for q in unit.weights]
    out = g.group_forward_mx8(e.cuda(), w, unit.b.cuda(), [t.cuda() for t in unit.a], 16, True)
    assert all(o.shape[0] == 0 for o in out)


def test_mx8_rejects_int4_weights():
    g = glowq()
    keys = (62,)
    x = W.make_x(4, 256, 0.77, keys)
    unit = W.make_unit("m8f", "group", x, [32], 8, keys, fmt="int4")
    with pytest.raises(g.GlowQError) as e:
        run_unit(unit, True)
    assert e.value.status == g.ERR_UNSUPPORTED


# MXFP6 weights: the 16 + 8-byte operand of the block-scaled step, small tiles and both rings of the
# wide tile (two stages for MXFP6), ragged tokens and rows
SHAPES6 = [("mxfp6_e2m3", 3, 384, [40, 24], 8), ("mxfp6_e2m3", 33, 640, [100], 24),
           ("mxfp6_e2m3", 260, 640, [22000, 21000, 1000], 64), ("mxfp6_e2m3", 500, 256, [16400, 16000], 16),
           ("mxfp6_e3m2", 17, 512, [96, 64, 40], 32), ("mxfp6_e3m2", 129, 256, [32784, 32760], 256)]


@pytest.mark.parametrize("fmt,T,d,rows,r", SHAPES6)
def test_mx8_mxfp6_weights_match_oracle(fmt, T, d, rows, r):
    keys = (66, T, d)
    x = W.make_x(T, d, 1.19, keys)
    unit = W.make_unit("m86", "group", x, rows, r, keys, fmt=fmt)
    ys, ws = run_unit(unit, True)
    check_codes(unit, ws)
    for i, (y, yr) in enumerate(zip(ys, oracle(unit, True))):
        assert_parity(y, yr, f"mx8 {fmt} T={T} d={d} r={r} module {i}")


@pytest.mark.parametrize("T", [1, 16, 64])
def test_mx8_llama_qkv(T):
    """LLaMA-2-7B QKV group (d = 4096, 3 x 4096 rows, r = 64) at decode and batched-decode sizes."""
    keys = (63, T)
    x = W.make_x(T, 4096, 1.19, keys, device="cuda")
    unit = W.make_unit("m8q", "group", x, [4096, 4096, 4096], 64, keys, device="cuda", fmt="mxfp4")
    ys, ws = run_unit(unit, True)
    check_codes(unit, ws)
    for i, (y, yr) in enumerate(zip(ys, oracle(unit, True))):
        assert_parity(y, yr, f"mx8 qkv T={T} module {i}")


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp6_e2m3"])
def test_mx8_gateup_prefill_sampled(fmt):
    """LLaMA-2-7B gate/up group at T = 2048 (r = 64), 40 sampled tokens against the oracle (rows are
    independent: each token's codes, product and correction use that token alone)."""
    keys = (64,)
    T = 2048
    x = W.make_x(T, 4096, 0.77, keys, device="cuda")
    unit = W.make_unit("m8g", "group", x, [11008, 11008], 64, keys, device="cuda", fmt=fmt)
    ys, ws = run_unit(unit, True)
    rows = np.sort(np.random.default_rng(3).choice(T, 40, replace=False))
    rows[-1] = T - 1
    ref = oracle(unit, True, rows=torch.from_numpy(rows).cuda())
    for i, (y, yr) in enumerate(zip(ys, ref)):
        assert_parity(y[rows], yr, f"mx8 {fmt} gate/up T=2048 module {i}")
    check_codes(unit, ws, rows=rows)


def test_mx8_deterministic():
    keys = (65,)
    x = W.make_x(200, 1024, 0.77, keys)
    unit = W.make_unit("m8d", "group", x, [640, 320], 32, keys, fmt="mxfp4")
    a, _ = run_unit(unit, True)
    b, _ = run_unit(unit, True)
    for u, v in zip(a, b):
        assert torch.equal(u, v)
