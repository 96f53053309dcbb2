"""The read-bandwidth reference (tq_stream_read) reads every byte: each
sink word equals the xor, computed on the host, of the 16-byte words its
thread visits (word j goes to thread j mod TQ_STREAM_READ_SINK)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import kv_cache_quantization_encode_amd as tq  # noqa: E402
from kv_cache_quantization_encode_amd import _lib as L  # noqa: E402


@pytest.mark.parametrize("n_words", [1, 1000, L.TQ_STREAM_READ_SINK * 9 + 77])
def test_stream_read_visits_every_word(n_words):
    rng = np.random.default_rng(n_words)
    host = rng.integers(0, 2**32, size=(n_words, 4), dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).to("cuda")
    sink = torch.full((L.TQ_STREAM_READ_SINK,), -1, dtype=torch.int32, device="cuda")
    tq.stream_read(src, sink)
    got = sink.cpu().numpy().view(np.uint32)
    w = np.bitwise_xor.reduce(host, axis=1)
    T = L.TQ_STREAM_READ_SINK
    pad = (-n_words) % T
    want = np.bitwise_xor.reduce(np.concatenate([w, np.zeros(pad, np.uint32)]).reshape(-1, T), axis=0)
    assert np.array_equal(got, want)
