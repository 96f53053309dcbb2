"""Memory accounting of the packed records (host only)."""
import pytest

import oracle.tq_oracle as O

q = pytest.importorskip("kv_cache_quantization_encode_amd.quality")


@pytest.mark.parametrize("mode,bits", [("prod", 3), ("prod", 4), ("mse", 4), ("mse", 8), ("grouped", None),
                                       ("grouped_prod", None)])
def test_key_record_bytes_match_the_oracle(mode, bits):
    cfg = O.KeyConfig(mode=mode, bits=bits or 3, bits_outlier=4, bits_normal=2)
    assert q.key_record_bytes(mode, bits or 3) == O.record_bytes(cfg)


def test_memory_table_against_fp16():
    rows = q.memory_table(contexts=(32768,), kv_heads=8, layers=1, configs=(("prod", 3, 2),))
    r = rows[0]
    # 52-byte key (bit-packing article sec 四) + 32 B of 2-bit codes + 4 fp16 scales and zeros
    assert r["bytes"] == 32768 * 8 * (52 + 48)
    assert r["fp16_bytes"] == 32768 * 8 * 512
    assert abs(r["ratio"] - 5.12) < 1e-12
