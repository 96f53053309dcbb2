"""The Python binding rejects tensors the kernels must not be handed (host
tensors, wrong dtypes or shapes) with ValueError before any library call;
runs without a GPU."""
import pytest

torch = pytest.importorskip("torch")

import kv_cache_quantization_encode_amd as tq  # noqa: E402
from kv_cache_quantization_encode_amd import _lib as L  # noqa: E402


@pytest.fixture(scope="module")
def tables():
    return tq.Tables(L.key_config(mode="prod", bits=3, seed=1), "cpu")


def test_host_tensors_are_rejected(tables):
    keys = torch.zeros((16, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        tq.encode_keys(tables, keys)
    with pytest.raises(ValueError, match="GPU"):
        tq.encode_values(keys, 2)
    with pytest.raises(ValueError, match="GPU"):
        tq.append_kv(tables, keys, keys, 2, {}, {})
    with pytest.raises(ValueError, match="GPU"):
        tq.channel_moments(keys)
    with pytest.raises(ValueError, match="GPU"):
        tq.encode_keys_batched([tables, tables], [keys, keys])


def test_shape_and_count_errors(tables):
    with pytest.raises(ValueError):
        tq.encode_keys_batched([tables], [])                 # one Tables per key set
    with pytest.raises(ValueError):
        tq.encode_keys_batched([tables] * 33, [torch.zeros((1, 128))] * 33)   # at most 32 sets
    with pytest.raises(ValueError, match="GPU"):
        tq.encode_keys(tables, torch.zeros((16, 64)))        # checked before the shape: still host


def test_paged_store_rejects_mismatched_chunks(tables):
    store = tq.PagedKVCache.__new__(tq.PagedKVCache)         # only the argument check is exercised
    store.Hkv = 2
    with pytest.raises(ValueError):
        store.append(0, torch.zeros((4, 3, 128)), torch.zeros((4, 3, 128)))
