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
    """Each wavefront's 4 chains accumulate iters copies of the 32x32x16 product A B^T of its
    fixed operands (lane l holds A[l % 32][8 (l / 32) + e] and B[l % 32][8 (l / 32) + e]); the
    sum over chains, in the output layout (lane l: column l % 32, element i: row
    8 (i / 4) + 4 (l / 32) + i % 4), must be 4 iters (A B^T) exactly (small dyadic rationals)."""
    from rank_error_compensation_amd import probe
    iters, blocks = 3, 2
    sink = torch.zeros(blocks * 256 * 64, dtype=torch.uint8, device="cuda")
    fl = probe.mfma_f16(iters, sink, blocks)
    torch.cuda.synchronize()
    assert fl == blocks * 4 * iters * 4 * 32 * 32 * 16 * 2
    out = sink.view(torch.float32).cpu().numpy().reshape(blocks * 4, 64, 16)
    A = np.zeros((32, 16))
    B = np.zeros((32, 16))
    for l in range(64):
        for e in range(8):
            A[l % 32, 8 * (l // 32) + e] = ((l + e) & 3) * 0.25
            B[l % 32, 8 * (l // 32) + e] = ((l * 3 + e) & 3) * 0.125
    D = 4 * iters * (A @ B.T)
    want = np.zeros((64, 16))
    for l in range(64):
        for i in range(16):
            want[l, i] = D[8 * (i // 4) + 4 * (l // 32) + i % 4, l % 32]
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


def test_read_sequence_reads_consecutive_regions():
    """The launch-sequence probe reads region i right after region i - 1: with two regions of one
    size, the second launch overwrites every sink word, and the xor over the sink equals the xor
    of the second region alone."""
    from rank_error_compensation_amd import probe
    n16 = 1 << 12                                    # 64 KiB per region: 2 workgroups per read
    g = torch.Generator(device="cpu").manual_seed(11)
    words = torch.randint(0, 2**31 - 1, (2 * n16 * 4,), generator=g, dtype=torch.int64).to(torch.int32)
    src = words.cuda()
    sink = torch.zeros(2 * 256 * 16, dtype=torch.uint8, device="cuda")
    seq = probe.ReadSequence([n16 * 16, n16 * 16])
    seq.run(src.view(torch.uint8), sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.view(torch.int32).cpu().numpy().reshape(-1, 4), axis=0)
    want = np.bitwise_xor.reduce(words.numpy()[n16 * 4:].reshape(-1, 4), axis=0)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("chains", [4, 8, 16])
def test_mfma_shape_probe_results(chains):
    """The shape probe's two instructions compute what the kernels assume of them: for
    v_mfma_f32_16x16x32_f16 lane l holds A[l % 16][8 (l / 16) + e] and B[l % 16][8 (l / 16) + e] and
    returns D = A B^T at rows 4 (l / 16) + q, column l % 16; for 32x32x16 the layout of the test
    above (whose four outputs per quad are summed here).  Chains x iters copies, exact."""
    from rank_error_compensation_amd import probe
    iters, blocks = 3, 2
    for shape in (0, 1):
        sink = torch.zeros(blocks * 256 * 16, dtype=torch.uint8, device="cuda")
        fl = probe.mfma_shape(shape, chains, iters, sink, blocks)
        torch.cuda.synchronize()
        out = sink.view(torch.float32).cpu().numpy().reshape(blocks * 4, 64, 4)
        want = np.zeros((64, 4))
        if shape == 1:
            assert fl == blocks * 4 * iters * chains * 16 * 16 * 32 * 2
            A = np.zeros((16, 32))
            B = np.zeros((16, 32))
            for l in range(64):
                for e in range(8):
                    A[l % 16, 8 * (l // 16) + e] = ((l + e) & 3) * 0.25
                    B[l % 16, 8 * (l // 16) + e] = ((l * 3 + e) & 3) * 0.125
            D = chains * iters * (A @ B.T)
            for l in range(64):
                for q in range(4):
                    want[l, q] = D[4 * (l // 16) + q, l % 16]
        else:
            assert fl == blocks * 4 * iters * chains * 32 * 32 * 16 * 2
            A = np.zeros((32, 16))
            B = np.zeros((32, 16))
            for l in range(64):
                for e in range(8):
                    A[l % 32, 8 * (l // 32) + e] = ((l + e) & 3) * 0.25
                    B[l % 32, 8 * (l // 32) + e] = ((l * 3 + e) & 3) * 0.125
            D = chains * iters * (A @ B.T)
            for l in range(64):
                for i in range(16):
                    want[l, i & 3] += D[8 * (i // 4) + 4 * (l // 32) + i % 4, l % 32]
        for w in range(blocks * 4):
            np.testing.assert_array_equal(out[w], want)
