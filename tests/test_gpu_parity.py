"""HIP path against the fp64 oracle, element by element, through the C ABI (needs gfx950).

Bar: dequantised weights bit-exact; outputs within relative Frobenius 1e-3 and max-abs
1e-2 * max|y| of the oracle."""
import math

import numpy as np
import pytest
import torch

import workload as W
from gpu_util import DevUnit, assert_parity, glowq, log, oracle_unit
from oracle import glowq_ref as G
from oracle import solve as S

# workspace header: synchronisation words of the decode hand-off (int32 word 0: the epoch; every
# other word is back to zero after each call)
WS_HEADER = 8192

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    glowq()
    yield
    torch.cuda.synchronize()


def _random_qweight(n_out, d, seed, z_lo=-20, z_hi=36):
    rng = np.random.default_rng(seed)
    q = torch.from_numpy(rng.integers(0, 16, size=(n_out, d)).astype(np.uint8))
    s = torch.from_numpy(rng.uniform(-0.05, 0.05, size=(n_out, d // 128)).astype(np.float16))
    z = torch.from_numpy(rng.integers(z_lo, z_hi, size=(n_out, d // 128)).astype(np.float16))
    return W.QuantWeight(q=q, s=s, z=z, q_packed=W.pack_canonical(q), err_sq=1.0, w_sq=1.0)


# ------------------------------------------------------------------ dequantisation export
@pytest.mark.parametrize("n_out,d,seed", [(40, 384, 0), (256, 256, 1), (1, 128, 2), (4096, 4096, 3)])
def test_dequant_bit_exact(n_out, d, seed):
    g = glowq()
    qw = _random_qweight(n_out, d, seed)
    w = g.QWeight.from_workload(qw)
    ref = G.dequant_qw(qw)
    f32 = g.dequant(w, torch.float32).cpu().numpy()
    assert np.array_equal(f32.astype(np.float64), ref)
    f16 = g.dequant(w, torch.float16).cpu().numpy()
    assert np.array_equal(f16.view(np.uint16), ref.astype(np.float16).view(np.uint16))
    torch.cuda.synchronize()


def test_dequant_extremes_bit_exact():
    """Zero points at the +-1024 limits, subnormal and maximal fp16 scales."""
    g = glowq()
    n_out, d = 32, 256
    rng = np.random.default_rng(5)
    q = torch.from_numpy(rng.integers(0, 16, size=(n_out, d)).astype(np.uint8))
    zs = np.array([-1024, 1024, 0, 15, -1, 1023, -1023, 7] * 8, dtype=np.float16).reshape(n_out, 2)
    sb = np.array([0x0001, 0x03FF, 0x0400, 0x7BFF, 0x3C00, 0x1400, 0x8001, 0xFBFF] * 8, dtype=np.uint16)
    s = sb.view(np.float16).reshape(n_out, 2)
    qw = W.QuantWeight(q=q, s=torch.from_numpy(s), z=torch.from_numpy(zs), q_packed=W.pack_canonical(q),
                       err_sq=1.0, w_sq=1.0)
    w = g.QWeight.from_workload(qw)
    ref = G.dequant_qw(qw)
    f32 = g.dequant(w, torch.float32).cpu().numpy()
    assert np.array_equal(f32.astype(np.float64), ref)
    with np.errstate(over="ignore"):
        ref16 = ref.astype(np.float16)
    f16 = g.dequant(w, torch.float16).cpu().numpy()
    assert np.array_equal(f16.view(np.uint16), ref16.view(np.uint16))


def test_repack_rejects_bad_zero_points():
    g = glowq()
    for bad in (1025.0, 0.5, float("inf")):
        qw = _random_qweight(16, 128, 9)
        z = qw.z.clone()
        z[3, 0] = bad
        with pytest.raises(g.GlowQError) as ei:
            g.QWeight.from_canonical(qw.q_packed, qw.s, z)
        assert ei.value.status == g.ERR_RANGE
    qw = _random_qweight(16, 128, 9)
    s = qw.s.clone()
    s[0, 0] = float("nan")
    with pytest.raises(g.GlowQError):
        g.QWeight.from_canonical(qw.q_packed, s, qw.z)


# ------------------------------------------------------------------ tiny QKV group (d = 256)
@pytest.fixture(scope="module")
def tiny_unit():
    c = W.tiny_qkv_inputs()
    w_hats = [G.dequant_qw(q) for q in c["qw"]]
    E = [G._f64(w16) - wh for w16, wh in zip(c["w16"], w_hats)]
    Q, lam = c["Q"].numpy(), c["lam"].numpy()
    A, B, _ = S.whitened_factors(E, S.sqrt_psd(Q, lam), S.pinv_sqrt_psd(Q, lam), c["r"])
    unit = W.Unit(name="qkv", kind="group", x=c["x"], weights=c["qw"],
                  a=[torch.from_numpy(a.astype(np.float16)) for a in A],
                  b=torch.from_numpy(B.astype(np.float16)), r=c["r"])
    return unit


def test_tiny_qkv_group(tiny_unit):
    du = DevUnit(tiny_unit)
    ys = du.forward()
    ref = oracle_unit(tiny_unit)
    for i, (y, yr) in enumerate(zip(ys, ref)):
        assert_parity(y, yr, f"tiny module {i}")


@pytest.mark.parametrize("restore,r", [(False, 16), (True, 0)])
def test_tiny_qkv_no_correction(tiny_unit, restore, r):
    du = DevUnit(tiny_unit)
    ys = du.forward(restore=restore, r=r)
    ref = oracle_unit(tiny_unit, restore=restore, r=r)
    for i, (y, yr) in enumerate(zip(ys, ref)):
        assert_parity(y, yr, f"tiny restore={restore} r={r} module {i}")


# ------------------------------------------------------------------ ragged shapes, both paths
RAGGED = [
    # T, d, n_outs, r
    (1, 128, (16,), 8),
    (3, 384, (40, 24, 8), 8),
    (17, 384, (40, 24, 8), 24),
    (33, 256, (1, 17, 31), 16),
    (64, 512, (48, 80), 32),
    (65, 384, (40, 24, 8), 24),
    (130, 256, (100, 36), 40),
    (300, 640, (272, 16, 48), 64),
    (257, 128, (520,), 256),
    # enough 32-token blocks that the prefill projection needs no K split (written directly)
    (8200, 128, (40, 24), 32),
    (8224, 256, (24,), 64),
    # prefill grids below the wide tile's threshold with 512 and 640 small tiles (two wave
    # groups, one wave group per workgroup); the smaller cases above take four
    (1024, 256, (4096,), 32),
    (1000, 256, (2560, 2560), 16),
]


@pytest.mark.parametrize("T,d,n_outs,r", RAGGED)
def test_ragged_group(T, d, n_outs, r):
    keys = (7, T, d, r)
    x = W.make_x(T, d, 1.19, keys)
    unit = W.make_unit("g", "group", x, list(n_outs), r, keys)
    du = DevUnit(unit)
    ys = du.forward()
    ref = oracle_unit(unit)
    for i, (y, yr) in enumerate(zip(ys, ref)):
        assert_parity(y, yr, f"T={T} d={d} O={n_outs[i]} r={r}")


@pytest.mark.parametrize("T", [6, 16])
def test_decode_two_row_tiles_without_lds(T):
    """6-16 tokens at d = 4096 (activations read from L2, not staged in LDS) with 513 16-row tiles:
    two row tiles per workgroup, the last module's last workgroup holding one real tile."""
    x = W.make_x(T, 4096, 1.19, (37, T))
    u = W.make_unit("wide", "group", x, [4096, 2064, 2048], 64, (37, T, 64))
    du = DevUnit(u)
    for restore in (True, False):
        ys = du.forward(restore=restore)
        for i, (y, yr) in enumerate(zip(ys, oracle_unit(u, restore=restore))):
            assert_parity(y, yr, f"T={T} restore={restore} module {i}")


@pytest.mark.parametrize("T", [17, 33, 64])
def test_decode_narrow_k_split(T):
    """17-64 tokens on a correcting narrow call (fewer than 40 128-row tiles) with long rows (at
    least 64 input groups): the groups split into 4 K ranges over 4-row-tile workgroups, the first
    range adding the correction, then a second launch sums the ranges.  A ragged module (520 rows:
    the last workgroup holds one real 16-row tile and a half-empty one), a solo module whose 65
    groups split 17 + 17 + 17 + 14, and a layerwise group (one projection per module); without
    restore the call takes the unsplit decode kernel.  (The solo and layerwise cases run at one
    token count: their factors at d >= 8192 take the oracle most of the test's time.)"""
    x = W.make_x(T, 8192, 1.19, (41, T))
    u = W.make_unit("nar", "group", x, [1024, 520, 256], 64, (41, T, 64))
    du = DevUnit(u)
    for restore in (True, False):
        ys = du.forward(restore=restore)
        for i, (y, yr) in enumerate(zip(ys, oracle_unit(u, restore=restore))):
            assert_parity(y, yr, f"T={T} restore={restore} module {i}")
    if T != 33:
        return
    xs = W.make_x(T, 8320, 0.77, (42, T))
    solo = W.make_unit("ns", "solo", xs, [200], 24, (42, T))
    assert_parity(DevUnit(solo).forward()[0], oracle_unit(solo)[0], f"solo T={T}")
    xl = W.make_x(T, 8192, 0.77, (43, T))
    lw = W.make_unit("nl", "group", xl, [64, 48, 16], 16, (43, T), layerwise=True)
    for i, (y, yr) in enumerate(zip(DevUnit(lw, layerwise=True).forward_layerwise(),
                                    oracle_unit(lw, layerwise=True))):
        assert_parity(y, yr, f"layerwise T={T} module {i}")


@pytest.mark.parametrize("T", [70, 130])
def test_prefill_small_grid_half_row_tiles(T):
    """Prefill calls with fewer than 128 tiles of 64 tokens x 128 rows take 64 x 64 tiles, and
    with fewer than 128 of those 32 x 64 tiles (one 16-row tile per wave, 4 wave groups splitting
    the 5 input groups 2 + 1 + 1 + 1), as here: ragged tokens, a 130-row module whose last wave
    holds a 2-row tile and waves past its end, with and without restore."""
    x = W.make_x(T, 640, 1.19, (47, T))
    u = W.make_unit("hr", "group", x, [256, 130, 64], 32, (47, T, 32))
    du = DevUnit(u)
    for restore in (True, False):
        ys = du.forward(restore=restore)
        for i, (y, yr) in enumerate(zip(ys, oracle_unit(u, restore=restore))):
            assert_parity(y, yr, f"T={T} restore={restore} module {i}")


def test_prefill_small_grid_64x64_tiles():
    """A wide group at T = 64 (72 row tiles of 128) with 72 tiles of 64 x 128 and 144 of 64 x 64:
    the 64 x 64 tiles (4 wave groups), with and without restore."""
    T = 64
    x = W.make_x(T, 256, 1.19, (48, T))
    u = W.make_unit("hr64", "group", x, [4096, 4096, 1024], 32, (48, T, 32))
    du = DevUnit(u)
    for restore in (True, False):
        ys = du.forward(restore=restore)
        for i, (y, yr) in enumerate(zip(ys, oracle_unit(u, restore=restore))):
            assert_parity(y, yr, f"restore={restore} module {i}")


@pytest.mark.parametrize("T", [40, 64])
def test_prefill_small_t_wide_group(T):
    """A wide group at 17-64 tokens with at least 128 tiles of 64 x 128 (two 8200-row modules,
    the last tile of each ragged): 32-token x 128-row tiles, with and without restore."""
    x = W.make_x(T, 256, 1.19, (49, T))
    u = W.make_unit("wg", "group", x, [8200, 8200], 32, (49, T, 32))
    du = DevUnit(u)
    for restore in (True, False):
        ys = du.forward(restore=restore)
        for i, (y, yr) in enumerate(zip(ys, oracle_unit(u, restore=restore))):
            assert_parity(y, yr, f"T={T} restore={restore} module {i}")


@pytest.mark.parametrize("T", [1, 5, 100])
def test_solo_and_layerwise(T):
    keys = (8, T)
    x = W.make_x(T, 384, 0.77, keys)
    unit = W.make_unit("g", "group", x, [64, 48, 16], 16, keys, layerwise=True)
    du = DevUnit(unit, layerwise=True)
    ys = du.forward_layerwise()
    ref = oracle_unit(unit, layerwise=True)
    for i, (y, yr) in enumerate(zip(ys, ref)):
        assert_parity(y, yr, f"layerwise T={T} module {i}")
    solo = W.make_unit("s", "solo", x, [96], 24, keys)
    ds = DevUnit(solo)
    assert_parity(ds.forward()[0], oracle_unit(solo)[0], f"solo T={T}")


def test_t_zero_is_noop():
    g = glowq()
    unit = W.make_unit("g", "group", W.make_x(2, 256, 1.19, (9,)), [32], 8, (9,))
    du = DevUnit(unit)
    x0 = du.x[:0]
    ys = g.group_forward(x0, du.w, du.b, du.a, 8, True)
    assert ys[0].shape == (0, 32)


# ------------------------------------------------------------------ LLaMA-2-7B QKV decode
@pytest.fixture(scope="module")
def qkv_units():
    return {T: W.llama2_qkv_unit(T) for T in (1, 4, 16)}


@pytest.mark.parametrize("T", [1, 4, 16])
def test_llama2_qkv_decode(qkv_units, T):
    unit = qkv_units[T]
    du = DevUnit(unit)
    ys = du.forward()
    ref = oracle_unit(unit)
    for i, (y, yr) in enumerate(zip(ys, ref)):
        assert_parity(y, yr, f"qkv T={T} module {i}")


def test_llama2_qkv_deterministic(qkv_units):
    du = DevUnit(qkv_units[4])
    first = [y.clone() for y in du.forward()]
    for _ in range(20):
        ys = du.forward()
        for a, b in zip(first, ys):
            assert torch.equal(a, b)


# ------------------------------------------------------------------ LLaMA-2-7B gate/up prefill
def test_llama2_gateup_prefill():
    log("generating gate/up T=2048")
    unit = W.llama2_gateup_unit(2048)
    du = DevUnit(unit)
    ys = du.forward()
    torch.cuda.synchronize()
    log("oracle gate/up T=2048")
    ref = oracle_unit(unit)
    for i, (y, yr) in enumerate(zip(ys, ref)):
        assert_parity(y, yr, f"gate/up T=2048 module {i}")
    # decode and prefill kernels agree on the same tokens (first 64 through the decode path)
    yd = du.forward(x=du.x[:64].contiguous())
    for i, (a, b) in enumerate(zip(yd, ys)):
        e = G.parity_errors(a.float().cpu().numpy(), b[:64].float().cpu().numpy().astype(np.float64))
        assert e["rel_fro"] <= 1e-3, (i, e)


def test_decode_workspace_state_after_calls():
    """After every decode call the hand-off's arrival counters are back to zero, no bounded wait
    expired, and the epoch word has advanced once per call that applied the correction."""
    g = glowq()
    keys = (10,)
    calls = 0
    T_max = 64
    ws = g.make_workspace(T_max, 24, 3)
    for T, lw in ((1, False), (7, True), (64, False), (3, True)):
        x = W.make_x(T, 512, 1.19, keys + (T,))
        unit = W.make_unit("g", "group", x, [64, 40, 32], 24, keys, layerwise=True)
        du = DevUnit(unit, layerwise=True)
        for _ in range(3):
            if lw:
                g.layerwise_forward(du.x, du.w, du.b_lw, du.a, 24, True, workspace=ws)
            else:
                g.group_forward(du.x, du.w, du.b, du.a, 24, True, workspace=ws)
            calls += 1
        g.group_forward(du.x, du.w, du.b, du.a, 24, False, workspace=ws)  # restore off: no hand-off
        torch.cuda.synchronize()
        hdr = ws[:WS_HEADER].view(torch.int32).cpu()
        assert int(hdr[0]) == calls, (int(hdr[0]), calls)          # epoch
        assert int(hdr[1:].abs().sum()) == 0, hdr[1:].nonzero()     # counters and error flag


def test_prefill_split_projection():
    """Prefill calls whose projection R = X B^T is split over K (fp32 partials summed in a fixed
    order) match the oracle call after call, group and layerwise, with token blocks ragged at T,
    and leave the workspace header untouched."""
    g = glowq()
    keys = (12,)
    ws = g.make_workspace(300, 40, 3)
    for T, d, lw in ((100, 512, False), (300, 640, True), (65, 1024, False), (300, 640, False)):
        x = W.make_x(T, d, 0.77, keys + (T, d))
        unit = W.make_unit("g", "group", x, [72, 40, 24], 40, keys + (T, d), layerwise=True)
        du = DevUnit(unit, layerwise=True)
        ref = oracle_unit(unit, layerwise=lw)
        for _ in range(2):
            if lw:
                ys = g.layerwise_forward(du.x, du.w, du.b_lw, du.a, 40, True, workspace=ws)
            else:
                ys = g.group_forward(du.x, du.w, du.b, du.a, 40, True, workspace=ws)
            torch.cuda.synchronize()
            for i, (y, yr) in enumerate(zip(ys, ref)):
                assert_parity(y, yr, f"T={T} d={d} layerwise={lw} module {i}")
            assert int(ws[:WS_HEADER].view(torch.int32).abs().sum()) == 0


def test_epoch_wrap_clears_stale_pairs():
    """The epoch skips 2^32 - 1 (tags are never 0), and the calls with the last and the first tag
    of a wrap (2^32 - 1 and 1) clear every pair outside their range: a pair planted there with the tag a later, larger
    call will use is gone before that call runs, and every result matches the oracle."""
    g = glowq()
    keys = (11,)
    r, n_out = 16, [48, 32]
    ws = g.make_workspace(4, r, 1)
    pairs = ws[WS_HEADER:].view(torch.int64)  # the decode area: (fp32 value, u32 tag) pairs
    hdr = ws[:WS_HEADER].view(torch.int32)
    hdr[0] = -2  # epoch 2^32 - 2: the next call uses tag 2^32 - 1
    # pair index 8 * 1 * 1 * r (first slot past a T=1 call's range) is inside a T=4 call's range;
    # plant a pair carrying tag 2 (what the T=4 call below will wait for) and a huge value
    planted = 8 * r + 5
    pairs[planted] = (2 << 32) | 0x7F000000
    units = {T: W.make_unit("w", "group", W.make_x(T, 256, 1.19, keys + (T,)), n_out, r, keys) for T in (1, 4)}
    devs = {T: DevUnit(u) for T, u in units.items()}
    def run(T):
        d = devs[T]
        return g.group_forward(d.x, d.w, d.b, d.a, r, True, workspace=ws)

    run(1)  # tag 2^32 - 1: the last tag of a wrap also clears the area outside its range
    torch.cuda.synchronize()
    assert int(hdr[0]) == 0, int(hdr[0])  # 2^32 - 1 skipped
    assert int(pairs[planted]) == 0
    pairs[planted] = (1 << 32) | 0x7F000000  # a pair left with tag 1, to be cleared by the tag-1 call
    ys = run(1)  # tag 1: clears the area outside its range
    torch.cuda.synchronize()
    assert int(hdr[0]) == 1
    assert int(pairs[planted]) == 0
    for y, yr in zip(ys, oracle_unit(units[1])):
        assert_parity(y, yr, "T=1 after wrap")
    ys = run(4)  # tag 2
    torch.cuda.synchronize()
    for y, yr in zip(ys, oracle_unit(units[4])):
        assert_parity(y, yr, "T=4 after wrap")
    assert int(hdr[1:].abs().sum()) == 0


def test_workspace_reuse_across_calls_and_paths():
    """One workspace reused by consecutive decode and prefill calls with different inputs: every
    result matches the oracle (no stale projection is ever consumed)."""
    g = glowq()
    ws = g.make_workspace(200, 32, 1)
    for i, T in enumerate((1, 1, 150, 1, 16, 200, 2, 2)):
        keys = (11, i)
        x = W.make_x(T, 384, 0.77, keys)
        unit = W.make_unit("g", "group", x, [48, 32], 32, keys)
        du = DevUnit(unit)
        ys = g.group_forward(du.x, du.w, du.b, du.a, 32, True, workspace=ws)
        ref = oracle_unit(unit)
        for j, (y, yr) in enumerate(zip(ys, ref)):
            assert_parity(y, yr, f"reuse call {i} T={T} module {j}")


@pytest.mark.parametrize("T,d,n_outs,r", [
    (1, 256, (16, 33, 8, 40, 24, 17, 64, 48), 16),          # decode, the most modules a call takes
    (12, 384, (130, 96, 33, 8, 64, 200, 17, 90), 24),       # decode, activations in LDS
    (40, 256, (700, 650, 720, 690, 700, 710, 640, 660), 32),  # fused 17-64-token tiles
    (300, 128, (100, 36, 48, 16, 80, 20, 64, 8), 40),       # prefill
])
def test_eight_modules_group_and_layerwise(T, d, n_outs, r):
    """GLOWQ_MAX_MODULES = 8 modules in one call: the group form (one shared projection) and the
    layerwise form (eight projections, eight right factors) against the oracle."""
    keys = (17, T, d, r)
    x = W.make_x(T, d, 0.77, keys)
    unit = W.make_unit("g8", "group", x, list(n_outs), r, keys, layerwise=True)
    du = DevUnit(unit, layerwise=True)
    for i, (y, yr) in enumerate(zip(du.forward(), oracle_unit(unit))):
        assert_parity(y, yr, f"8 modules T={T} module {i}")
    for i, (y, yr) in enumerate(zip(du.forward_layerwise(), oracle_unit(unit, layerwise=True))):
        assert_parity(y, yr, f"8 modules layerwise T={T} module {i}")
