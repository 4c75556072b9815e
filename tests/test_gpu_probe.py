"""The measurement probes (libglowq_probe.so) compute what they claim, so that the achievable
peaks the benchmark reports are rates of real work (needs gfx950)."""
import numpy as np
import pytest
import torch

pytestmark = [pytest.mark.gpu]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def test_mfma_probe_result():
    """Each wavefront's 8 chains accumulate iters copies of the 16x16x32 product A B^T of its
    fixed operands (lane l holds A[l % 16][8 (l / 16) + e] and B[l % 16][8 (l / 16) + e]); the
    sum over chains, in the output layout (lane l: rows 4 (l / 16) + i, column l % 16), must be
    8 iters (A B^T) exactly (all values are small dyadic rationals)."""
    from rank_error_compensation_amd import probe
    iters, blocks = 3, 2
    sink = torch.zeros(blocks * 256 * 16, dtype=torch.uint8, device="cuda")
    fl = probe.mfma_f16(iters, sink, blocks)
    torch.cuda.synchronize()
    assert fl == blocks * 4 * iters * 8 * 16 * 16 * 32 * 2
    out = sink.view(torch.float32).cpu().numpy().reshape(blocks * 4, 64, 4)
    A = np.zeros((16, 32))
    B = np.zeros((16, 32))
    for l in range(64):
        for e in range(8):
            A[l % 16, 8 * (l // 16) + e] = ((l + e) & 3) * 0.25
            B[l % 16, 8 * (l // 16) + e] = ((l * 3 + e) & 3) * 0.125
    D = 8 * iters * (A @ B.T)
    want = np.zeros((64, 4))
    for l in range(64):
        for i in range(4):
            want[l, i] = D[4 * (l // 16) + i, l % 16]
    for w in range(blocks * 4):
        np.testing.assert_array_equal(out[w], want)


def test_read_probe_folds_every_word():
    """The streaming read xors every 16-byte word of the buffer into exactly one thread's result:
    the xor over all threads equals the xor of the whole buffer."""
    from rank_error_compensation_amd import probe
    n16, blocks = 1 << 16, 8
    g = torch.Generator(device="cpu").manual_seed(7)
    words = torch.randint(0, 2**31 - 1, (n16 * 4,), generator=g, dtype=torch.int64).to(torch.int32)
    src = words.cuda()
    sink = torch.zeros(blocks * 256 * 16, dtype=torch.uint8, device="cuda")
    probe.read(src.view(torch.uint8), sink, blocks)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.view(torch.int32).cpu().numpy().reshape(-1, 4), axis=0)
    want = np.bitwise_xor.reduce(words.numpy().reshape(-1, 4), axis=0)
    np.testing.assert_array_equal(got, want)
