"""tq_decode_attention_noalloc (the decode step for callers that cannot
allocate: the split-K partials live in the library's own per-GPU array)
against tq_decode_attention with a caller-provided workspace: bit-identical
outputs, LSE and scores on two calls in a row, the second with a smaller
input, and the size limit of the array reported as an error."""
import ctypes

import numpy as np
import pytest

import tq_workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU runs, skipped there
    pytest.skip("needs a GPU", allow_module_level=True)

import kv_cache_quantization_encode_amd as tq  # noqa: E402
from kv_cache_quantization_encode_amd import _lib as L  # noqa: E402

DEV = "cuda"


def _cache(T, v_bits, B, Hkv, max_ctx, wid):
    n = B * Hkv * max_ctx
    k = W.normal_bf16_device(wid, 1, (n, 128), DEV)
    v = W.normal_bf16_device(wid, 2, (n, 128), DEV)
    return tq.encode_keys(T, k), tq.encode_values(v, v_bits)


def _both(T, v_bits, B, Hq, Hkv, ctx, max_ctx, wid):
    kp, vp = _cache(T, v_bits, B, Hkv, max_ctx, wid)
    q = W.normal_bf16_device(wid, 3, (1, B, Hq, 128), DEV)[0].contiguous()
    cl = torch.tensor(ctx, dtype=torch.int32, device=DEV)
    dec = tq.Decoder(T, B, Hq, Hkv, max_ctx, v_bits, torch.bfloat16, DEV)
    ref_o = torch.empty((B, Hq, 128), dtype=torch.float32, device=DEV)
    ref_l = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    ref_s = torch.full((B, Hq, max_ctx), float("nan"), dtype=torch.float32, device=DEV)
    dec(q, cl, kp, vp, out=ref_o, lse=ref_l, scores=ref_s)
    o = torch.full_like(ref_o, float("nan"))
    lse = torch.full_like(ref_l, float("nan"))
    s = torch.full_like(ref_s, float("nan"))
    tq.decode_attention_noalloc(T, q, cl, kp, vp, v_bits, max_ctx, Hkv, o, lse=lse, scores=s)
    torch.cuda.synchronize()
    return (o, lse, s), (ref_o, ref_l, ref_s)


def _same(a, b):
    a, b = a.cpu().numpy(), b.cpu().numpy()
    return np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_noalloc_equals_workspace_decode_twice_second_smaller():
    print("noalloc: prod 3-bit, B=4 Hq=32 Hkv=8 max_ctx=3000, then mse 2-bit B=2 Hq=8 Hkv=2 max_ctx=700",
          flush=True)
    T = tq.Tables(tq.key_config(mode="prod", bits=3, seed=42), DEV)
    got, ref = _both(T, 2, 4, 32, 8, [3000, 1, 2047, 0], 3000, 41)
    for g, r in zip(got, ref):
        assert _same(g, r)
    T2 = tq.Tables(tq.key_config(mode="mse", bits=2, seed=7), DEV)
    got, ref = _both(T2, 4, 2, 8, 2, [700, 333], 700, 42)
    for g, r in zip(got, ref):
        assert _same(g, r)


def test_noalloc_rejects_shapes_beyond_its_array():
    """512 sequences x 64 query heads x 64 KV heads need 512*64*130*4 bytes of
    partials (17 MB) for one split: more than the 8 MiB array."""
    T = tq.Tables(tq.key_config(mode="prod", bits=3, seed=42), DEV)
    B, Hq, Hkv, max_ctx = 512, 64, 64, 64
    need = tq.decode_workspace_bytes(T, B, Hq, Hkv, max_ctx, torch.bfloat16, 2)
    assert need > 8 << 20
    dummy = torch.zeros(16, dtype=torch.uint8, device=DEV)
    p = dummy.data_ptr()
    st = L.lib.tq_decode_attention_noalloc(ctypes.byref(T.cfg), p, p, L.TQ_BF16, B, Hq, Hkv, p, max_ctx,
                                           p, p, p, p, 2, 32, p, p, p, ctypes.c_float(1.0), p, None, None,
                                           None)
    assert st == L.TQ_ERR_WORKSPACE
