"""The decode path's projection hand-off under slow and silent producers (GPU).

The probe (glowq_probe_handoff) runs the hand-off routines the decode kernel uses -- epoch read,
slot and launch arrivals, tagged pairs read through the bounded wait, the last arrival's epoch
advance -- with producer workgroups that sleep before they arrive and publish.  Consumers then
count slots, finish and wait while the previous launch's pairs (one tag behind) are still in
memory.  Every launch must deliver exactly this launch's values to every consumer, leave the
counters at zero and advance the epoch by one; producers that never publish must end in the
workspace error word (GLOWQ_ERR_HANDOFF), not a hang, and the workspace must work again after.
"""
import random

import pytest
import torch

from gpu_util import glowq, log

pytestmark = pytest.mark.gpu

MAX_PAIRS = 65536


def probe():
    from rank_error_compensation_amd import probe as P
    return P


def fresh_workspace():
    g = glowq()
    ws = torch.empty(8192 + 8 * MAX_PAIRS, dtype=torch.uint8, device="cuda")
    g.init_workspace(ws)
    return ws


def epoch(ws):
    return int(ws.view(torch.int32)[0].item()) & 0xFFFFFFFF


def header_clean(ws):
    """Status OK (which also clears the error word), then every header word but the epoch is 0:
    slot and launch counters reset by the last arrivals."""
    g = glowq()
    st = g.workspace_status(ws)
    h = ws[:8192].view(torch.int32)[1:].cpu()
    return st == g.OK and int(h.abs().sum()) == 0


def launch(ws, n_prod, n_cons, n_pairs, delay, salt, publish=True):
    counts = torch.zeros(4, dtype=torch.int32, device="cuda")
    probe().handoff(ws, n_prod, n_cons, n_pairs, delay, publish, salt, counts)
    return counts


CASES = [  # (producers, consumers, pairs, delay)
    (1, 1, 1, 0),
    (1, 63, 8, 200),        # grid 64: one workgroup per arrival slot
    (3, 62, 200, 500),      # grid 65: one slot holds two workgroups
    (7, 121, 1000, 1000),   # grid 128
    (16, 4000, 4096, 300),  # more consumers than the GPU holds at once
    (64, 2048, MAX_PAIRS, 50),
]


@pytest.mark.parametrize("n_prod,n_cons,n_pairs,delay", CASES)
def test_delayed_producers(n_prod, n_cons, n_pairs, delay):
    log(f"handoff delayed producers: n_prod={n_prod} n_cons={n_cons} n_pairs={n_pairs} delay={delay}")
    ws = fresh_workspace()
    e0 = epoch(ws)
    counts = [launch(ws, n_prod, n_cons, n_pairs, delay, 1000.0 * (i + 1)) for i in range(3)]
    torch.cuda.synchronize()
    for c in counts:
        assert int(c[0]) == 0, "a consumer read a value of another launch"
        assert int(c[1]) == n_cons * n_pairs
    assert epoch(ws) == (e0 + 3) & 0xFFFFFFFF
    assert header_clean(ws)


def test_back_to_back_mixed_launches():
    """24 launches of different shapes and delays queued without a synchronisation between them."""
    log("handoff back-to-back mixed launches")
    rng = random.Random(7)
    ws = fresh_workspace()
    runs = []
    for i in range(24):
        n_prod = rng.choice([1, 2, 5, 16, 64])
        n_cons = rng.choice([1, 3, 64, 65, 500, 2100])
        n_pairs = rng.choice([1, 7, 256, 1000, 4096])
        delay = rng.choice([0, 10, 200, 800])
        runs.append((n_cons * n_pairs, launch(ws, n_prod, n_cons, n_pairs, delay, 17.0 * i - 100.0)))
    torch.cuda.synchronize()
    for expect_seen, c in runs:
        assert int(c[0]) == 0
        assert int(c[1]) == expect_seen
    assert epoch(ws) == 24
    assert header_clean(ws)


def test_epoch_wrap_skips_the_zero_tag():
    """The epoch runs 2^32 - 3, 2^32 - 2, then 0 (2^32 - 1 is skipped so the tag epoch + 1 is never
    the 0 of zero-filled memory), 1, 2; every launch on the way delivers its own values."""
    log("handoff epoch wrap")
    ws = fresh_workspace()
    ws.view(torch.int32)[0] = -3  # epoch 2^32 - 3
    seen = []
    for i in range(4):
        c = launch(ws, 4, 300, 512, 100, 3.0 + i)
        torch.cuda.synchronize()
        assert int(c[0]) == 0 and int(c[1]) == 300 * 512
        seen.append(epoch(ws))
    assert seen == [0xFFFFFFFE, 0, 1, 2]
    assert header_clean(ws)


def test_silent_producers_raise_the_error_word():
    """Producers that arrive but never publish: every consumer wait expires (bounded), the launch
    still ends, advances the epoch and raises GLOWQ_ERR_HANDOFF once; the next launch is clean."""
    log("handoff silent producers (bounded waits expire)")
    g = glowq()
    ws = fresh_workspace()
    assert g.workspace_status(ws) == g.OK
    launch(ws, 2, 2, 64, 0, 5.0, publish=False)
    torch.cuda.synchronize()
    assert epoch(ws) == 1
    assert g.workspace_status(ws) == g.ERR_HANDOFF
    assert g.workspace_status(ws) == g.OK  # reading the status cleared it
    c = launch(ws, 2, 40, 64, 100, 6.0)
    torch.cuda.synchronize()
    assert int(c[0]) == 0 and int(c[1]) == 40 * 64
    assert epoch(ws) == 2
    assert header_clean(ws)
