"""GlowQ-S restore selection on the GPU (glowq_ner_sums, glowq_restore_topk) against the fp64
oracle (oracle.solve.g_ner, oracle.solve.topk_restore; W_hat from oracle.glowq_ref.dequant_qw).

Bar: normalised error ratios within 1e-12 relative of the oracle (both sides sum exact fp64
terms, in different orders); masks bit-exact: equal to the oracle's top-k of the GPU's own
scores (the decision taken in the same precision), and to the oracle's top-k of the oracle's
scores wherever the k-th and (k+1)-th oracle scores differ by more than 1e-9 relative."""
import numpy as np
import pytest
import torch

import workload as W
from gpu_util import glowq, log
from oracle import glowq_ref as G
from oracle import solve as S

pytestmark = pytest.mark.gpu
REL = 1e-12


def make_module(O, d, keys, device="cpu", const_groups=0):
    cols = W.outlier_columns(d, keys)
    w = W.make_w(O, d, keys, cols, device)
    if const_groups:
        # constant groups (max == min): the quantiser turns their zero scale into 1
        w[:const_groups, :128] = w[:const_groups, :1]
    return w, W.rtn_quantize(w)


def oracle_err_w(w, qw):
    w64 = w.double().cpu().numpy()
    return w64 - G.dequant_qw(qw), w64


def gpu_sums(g, w, qw):
    dq = g.QWeight.from_workload(qw)
    return g.ner_sums(w.cuda(), dq)


@pytest.mark.parametrize("O,d,const_groups", [(40, 256, 0), (17, 384, 3), (64, 1024, 0), (16, 128, 16),
                                              (1, 128, 0), (300, 640, 5)])
def test_ner_ratio_matches_oracle(O, d, const_groups):
    g = glowq()
    w, qw = make_module(O, d, (21, O, d), const_groups=const_groups)
    s = gpu_sums(g, w, qw)
    s2 = gpu_sums(g, w, qw)
    torch.cuda.synchronize()
    assert torch.equal(s, s2)  # fixed summation order: bitwise repeatable
    E, W64 = oracle_err_w(w, qw)
    want = S.g_ner(E, W64)
    got = float(s[0]) / float(s[1])
    assert abs(got - want) <= REL * abs(want), (got, want)
    assert abs(float(s[1]) - float(np.sum(W64 ** 2))) <= REL * float(s[1])


def test_ner_ratio_llama_gate_shape():
    g = glowq()
    log("generating a 11008 x 4096 module")
    w, qw = make_module(11008, 4096, (22,), device="cuda")
    s = gpu_sums(g, w, qw)
    torch.cuda.synchronize()
    E, W64 = oracle_err_w(w, qw)
    want = S.g_ner(E, W64)
    got = float(s[0]) / float(s[1])
    assert abs(got - want) <= REL * abs(want), (got, want)


def test_batch_equals_single_calls():
    """40 modules of mixed shapes in one batch call (two launches of up to 32 modules) give the
    same pairs, bit for bit, as one call per module, and match the oracle."""
    g = glowq()
    shapes = [(16 + 8 * (i % 5), 128 * (1 + i % 3)) for i in range(40)]
    items = []
    for i, (O, d) in enumerate(shapes):
        w, qw = make_module(O, d, (24, i))
        items.append((w, qw, w.cuda(), g.QWeight.from_workload(qw)))
    batch = g.ner_sums_batch([(wd, dq) for _, _, wd, dq in items])
    single = torch.stack([g.ner_sums(wd, dq) for _, _, wd, dq in items])
    torch.cuda.synchronize()
    assert torch.equal(batch, single)
    for i, (w, qw, _, _) in enumerate(items):
        E, W64 = oracle_err_w(w, qw)
        want = S.g_ner(E, W64)
        got = float(batch[i, 0]) / float(batch[i, 1])
        assert abs(got - want) <= REL * abs(want), (i, got, want)


def check_masks(scores_gpu, mask_gpu, scores_ref, k):
    sg = [float(v) for v in scores_gpu.cpu()]
    mg = [bool(v) for v in mask_gpu.cpu()]
    assert mg == S.topk_restore(sg, k)
    order = sorted(scores_ref, reverse=True)
    if 0 < k < len(order) and order[k - 1] - order[k] > 1e-9 * abs(order[k - 1]):
        assert mg == S.topk_restore(scores_ref, k)


@pytest.mark.parametrize("k", [0, 1, 3, 8])
def test_layer_selection_end_to_end(k):
    """8 layers of three modules of different shapes: per-module sums on the GPU, then the
    layer scores and the top-k mask on the GPU, against the oracle's layer ratio (the error
    over the weight energy of the whole layer) and its top-k."""
    g = glowq()
    shapes = [(48, 256), (32, 256), (24, 384)]
    sums, ref = [], []
    for layer in range(8):
        errs, ws = [], []
        for i, (O, d) in enumerate(shapes):
            w, qw = make_module(O, d, (23, layer, i))
            sums.append(gpu_sums(g, w, qw))
            E, W64 = oracle_err_w(w, qw)
            errs.append(E.ravel())
            ws.append(W64.ravel())
        ref.append(S.g_ner(np.concatenate(errs), np.concatenate(ws)))
    st = torch.stack(sums).reshape(8, len(shapes), 2)
    scores, mask = g.restore_topk(st, k)
    torch.cuda.synchronize()
    for a, b in zip(scores.cpu().tolist(), ref):
        assert abs(a - b) <= REL * abs(b), (a, b)
    check_masks(scores, mask, ref, k)


def test_topk_ties_zero_weight_and_extremes():
    """Exact ties go to the lower unit; a unit with no weight energy scores 0; k = 0 and
    k = n restore nothing and everything."""
    g = glowq()
    pairs = [(1.0, 4.0), (3.0, 4.0), (1.0, 4.0), (0.0, 0.0), (3.0, 4.0), (2.0, 8.0), (0.5, 1.0)]
    st = torch.tensor(pairs, dtype=torch.float64, device="cuda").reshape(len(pairs), 1, 2)
    for k in range(len(pairs) + 1):
        scores, mask = g.restore_topk(st, k)
        torch.cuda.synchronize()
        ref = [e / w if w > 0 else 0.0 for e, w in pairs]
        assert scores.cpu().tolist() == ref
        assert [bool(v) for v in mask.cpu()] == S.topk_restore(ref, k), k
    # several modules per unit are summed before the division
    st2 = torch.tensor([[[1.0, 2.0], [1.0, 6.0]], [[0.0, 1.0], [2.0, 3.0]]], dtype=torch.float64, device="cuda")
    scores, mask = g.restore_topk(st2, 1)
    torch.cuda.synchronize()
    assert scores.cpu().tolist() == [2.0 / 8.0, 2.0 / 4.0]
    assert mask.cpu().tolist() == [0, 1]


@pytest.mark.parametrize("rel_tol", [0.0, 1e-3, 0.01, 0.2])
def test_select_with_layer_order_fallback(rel_tol):
    """glowq_restore_select against oracle.solve.topk_restore_tol on the GPU's own scores (the
    keys floor((max - s) / (rel_tol max)) are fp64 on both sides, bit-identical): near-equal
    scores fall back to layer order; separated ones keep the exact ranking."""
    g = glowq()
    rng = np.random.default_rng(29)
    base = [(1.0 + 1e-4 * rng.standard_normal(), 100.0) for _ in range(20)]          # weak signal
    sep = [(float(v), 1.0) for v in rng.uniform(0.1, 1.0, 12)]                       # strong signal
    mixed = base[:6] + [(50.0, 100.0), (0.2, 100.0)] + base[6:10]
    for pairs in (base, sep, mixed):
        st = torch.tensor(pairs, dtype=torch.float64, device="cuda").reshape(len(pairs), 1, 2)
        for k in (0, 1, 5, len(pairs) // 2, len(pairs)):
            scores, mask = g.restore_select(st, k, rel_tol)
            torch.cuda.synchronize()
            sg = [float(v) for v in scores.cpu()]
            assert [bool(v) for v in mask.cpu()] == S.topk_restore_tol(sg, k, rel_tol), (rel_tol, k)
            if rel_tol == 0.0:
                _, m0 = g.restore_topk(st, k)
                assert torch.equal(mask, m0)
    # weak signal with a tolerance above its spread: the first k layers exactly
    st = torch.tensor(base, dtype=torch.float64, device="cuda").reshape(len(base), 1, 2)
    _, mask = g.restore_select(st, 7, 0.01)
    torch.cuda.synchronize()
    assert [bool(v) for v in mask.cpu()] == [u < 7 for u in range(len(base))]
