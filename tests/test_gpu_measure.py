"""The measurement hooks the bench's ceilings come from, run through the C ABI."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mxfp4_latent_mixture_amd as m
    return m


def test_read_stream_reads_every_word_once(lm):
    # the XOR of every workgroup's word is the XOR of every 32-bit word of the
    # buffer exactly when each word is read once
    rng = np.random.default_rng(7)
    words = rng.integers(0, 2**32, size=(3 << 20) // 4 + 4 * 37, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.uint8).copy()).cuda()
    want = np.bitwise_xor.reduce(words)
    for blocks in (1, 7, 256, 1000):
        sink = torch.zeros(blocks, dtype=torch.int32, device="cuda")
        lm.debug_read_stream(buf, sink, blocks)
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        assert got == want, blocks


def test_mfma_rate_runs_and_repeats(lm):
    sink = torch.zeros(64, dtype=torch.int32, device="cuda")
    lm.debug_mfma_rate(16, sink, 64)
    torch.cuda.synchronize()
    first = sink.cpu().numpy().copy()
    lm.debug_mfma_rate(16, sink, 64)
    torch.cuda.synchronize()
    assert np.array_equal(first, sink.cpu().numpy())
    assert np.count_nonzero(first) > 0
    lm.debug_mfma_rate(0, sink, 64)  # no rounds: every accumulator stays zero
    torch.cuda.synchronize()
    assert not sink.cpu().numpy().any()
