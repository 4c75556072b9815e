"""MX weights (MXFP4, MXFP6 E2M3 / E3M2) through the C ABI against the fp64 oracle.

Bar: the dequantisation export is bit-exact against oracle.glowq_ref.dequant_mx (fp32, and fp16:
every admitted element times its scale is an fp16 value); the repack rejects codes wider than the
element and scales outside the exact range; forward outputs (decode, the K-split narrow decode,
fused 17-64-token tiles, small and wide prefill tiles, layerwise and solo calls) within relative
Frobenius 1e-3 and max-abs 1e-2 * max|y| of oracle.glowq_ref.group_forward on the MX weights."""
import numpy as np
import pytest
import torch

import workload as W
from gpu_util import DevUnit, assert_parity, glowq, log, oracle_unit
from oracle import glowq_ref as G

pytestmark = pytest.mark.gpu
FMTS = ["mxfp4", "mxfp6_e2m3", "mxfp6_e3m2"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    glowq()
    yield
    torch.cuda.synchronize()


def random_mx(fmt, n_out, k_in, seed):
    """Every code of the element (both zeros included) and every admitted scale."""
    rng = np.random.default_rng(seed)
    eb, mb, _ = W.MX_FORMATS[fmt]
    lo, hi = W.MX_EXP_RANGE[fmt]
    codes = rng.integers(0, 1 << (1 + eb + mb), size=(n_out, k_in)).astype(np.uint8)
    codes[0, : 1 << (1 + eb + mb)] = np.arange(1 << (1 + eb + mb))
    scales = rng.integers(lo + 127, hi + 128, size=(n_out, k_in // 32)).astype(np.uint8)
    scales[0, 0], scales[0, 1] = lo + 127, hi + 127
    return torch.from_numpy(codes), torch.from_numpy(scales)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n_out,k_in", [(16, 128), (37, 384), (300, 1024)])
def test_mx_dequant_bit_exact(fmt, n_out, k_in):
    g = glowq()
    codes, scales = random_mx(fmt, n_out, k_in, (n_out * 7 + k_in) % 1000)
    qw = g.QWeight.from_mx(fmt, codes, scales)
    ref = G.dequant_mx(codes, scales, fmt, n_out, k_in)
    w32 = g.dequant(qw, torch.float32).cpu().numpy().astype(np.float64)
    assert np.array_equal(w32, ref), np.argwhere(w32 != ref)[:5]
    w16 = g.dequant(qw, torch.float16).cpu().numpy()
    assert np.array_equal(w16.astype(np.float64), ref)
    # the sign of zero survives (codes 0 and the sign bit alone)
    neg0 = np.signbit(w32) & (w32 == 0)
    assert np.array_equal(neg0, np.signbit(ref) & (ref == 0))


@pytest.mark.parametrize("fmt", FMTS)
def test_mx_repack_rejects_out_of_range(fmt):
    g = glowq()
    eb, mb, _ = W.MX_FORMATS[fmt]
    lo, hi = W.MX_EXP_RANGE[fmt]
    codes, scales = random_mx(fmt, 20, 256, 5)
    for bad_scale in (lo + 126, hi + 128, 255):
        s = scales.clone()
        s[7, 3] = bad_scale
        with pytest.raises(g.GlowQError) as e:
            g.QWeight.from_mx(fmt, codes, s)
        assert e.value.status == g.ERR_RANGE
    c = codes.clone()
    c[19, 255] = 1 << (1 + eb + mb)
    with pytest.raises(g.GlowQError) as e:
        g.QWeight.from_mx(fmt, c, scales)
    assert e.value.status == g.ERR_RANGE
    g.QWeight.from_mx(fmt, codes, scales)  # in range: accepted


# (T, d, rows, r, what): which kernel the planner picks for that call
SHAPES = [(1, 512, [96, 80, 64], 16, "decode T=1"),
          (5, 640, [300, 17], 24, "decode, activations in LDS"),
          (2, 8192, [256, 200], 32, "decode, 8 waves"),
          (16, 2048, [4200, 4200], 64, "decode, two row tiles"),
          (40, 8192, [512], 32, "narrow decode with a K split"),
          (33, 512, [3000, 2500], 32, "fused 32 x 64 tiles"),
          (64, 256, [8192, 8192], 64, "fused 64 x 128 tiles"),
          (100, 384, [700, 300], 40, "small prefill tiles"),
          (256, 256, [4096, 4096], 32, "64 x 128 tiles, four wave groups"),
          (500, 256, [8192, 8000], 64, "wide prefill tile")]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("T,d,rows,r,what", SHAPES)
def test_mx_forward_matches_oracle(fmt, T, d, rows, r, what):
    keys = (90, T, d, FMTS.index(fmt))
    x = W.make_x(T, d, 0.77, keys)
    unit = W.make_unit("mx", "group", x, rows, r, keys, fmt=fmt, layerwise=True)
    du = DevUnit(unit, layerwise=True)
    for restore in (True, False):
        ys = du.forward(restore=restore)
        torch.cuda.synchronize()
        for i, (y, yr) in enumerate(zip(ys, oracle_unit(unit, restore=restore))):
            assert_parity(y, yr, f"{fmt} {what} restore={restore} module {i}")
    ys = du.forward_layerwise(True)
    torch.cuda.synchronize()
    for i, (y, yr) in enumerate(zip(ys, oracle_unit(unit, layerwise=True))):
        assert_parity(y, yr, f"{fmt} {what} layerwise module {i}")


@pytest.mark.parametrize("fmt", FMTS)
def test_mx_solo_ragged(fmt):
    keys = (91, FMTS.index(fmt))
    x = W.make_x(7, 896, 0.77, keys)
    unit = W.make_unit("mxs", "solo", x, [203], 48, keys, fmt=fmt)
    du = DevUnit(unit)
    ys = du.forward()
    torch.cuda.synchronize()
    assert_parity(ys[0], oracle_unit(unit)[0], f"{fmt} solo")


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp6_e2m3"])
def test_mx_llama_qkv_decode(fmt):
    """LLaMA-2-7B QKV group (d = 4096, 3 x 4096 rows, r = 64) at T = 1, whole outputs."""
    keys = (92, FMTS.index(fmt))
    x = W.make_x(1, 4096, 1.19, keys, device="cuda")
    unit = W.make_unit("mxq", "group", x, [4096] * 3, 64, keys, device="cuda", fmt=fmt)
    du = DevUnit(unit)
    ys = du.forward()
    torch.cuda.synchronize()
    for i, (y, yr) in enumerate(zip(ys, oracle_unit(unit))):
        assert_parity(y, yr, f"{fmt} qkv T=1 module {i}")


@pytest.mark.parametrize("fmt", FMTS)
def test_mx_llama_gateup_prefill_sampled(fmt):
    """LLaMA-2-7B gate/up group at T = 2048 (the wide tile), 24 sampled tokens against the oracle
    (rows are independent)."""
    keys = (93, FMTS.index(fmt))
    T = 2048
    x = W.make_x(T, 4096, 0.77, keys, device="cuda")
    unit = W.make_unit("mxg", "group", x, [11008, 11008], 64, keys, device="cuda", fmt=fmt)
    du = DevUnit(unit)
    ys = du.forward()
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(4).choice(T, 24, replace=False))
    rows[-1] = T - 1
    ref = oracle_unit(unit, rows=torch.from_numpy(rows).cuda())
    for i, (y, yr) in enumerate(zip(ys, ref)):
        assert_parity(y[torch.from_numpy(rows).cuda()], yr, f"{fmt} gate/up T=2048 module {i}")
