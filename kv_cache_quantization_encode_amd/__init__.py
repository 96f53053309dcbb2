"""MI355X-native TurboQuant KV-cache path: key/value encode and packed-domain
decode attention, as HIP kernels for gfx950 behind the C ABI in include/tq.h.

The Python layer only marshals arguments (torch provides device memory and
streams); importing it requires the built libtq.so next to this file.
"""
from ._lib import (TQ_BF16, TQ_F16, TQ_F32, TQ_MODE_GROUPED, TQ_MODE_GROUPED_PROD, TQ_MODE_MSE, TQ_MODE_PROD, KeyConfig,
                   TqError, key_config, status_string)
from .api import (Decoder, KeyBatchEncoder, Tables, append_kv, build_codebook, channel_moments, decode_attention,
                  decode_attention_noalloc,
                  decode_workspace_bytes, dequantize_keys, dequantize_values, encode_keys, encode_keys_batched,
                  encode_values,
                  idx_row_bytes, key_planes, parse_tables, select_outlier_channels, stream_read, value_planes)
from .store import PagedKVCache
from . import quality

__all__ = ["KeyConfig", "TqError", "key_config", "status_string", "Tables", "Decoder",
           "build_codebook", "parse_tables", "encode_keys", "encode_keys_batched", "KeyBatchEncoder", "encode_values", "append_kv", "decode_attention",
           "decode_attention_noalloc",
           "decode_workspace_bytes", "key_planes", "value_planes", "idx_row_bytes", "PagedKVCache",
           "dequantize_keys", "dequantize_values", "quality",
           "channel_moments", "select_outlier_channels", "stream_read",
           "TQ_F32", "TQ_BF16", "TQ_F16", "TQ_MODE_MSE", "TQ_MODE_PROD", "TQ_MODE_GROUPED",
           "TQ_MODE_GROUPED_PROD"]
