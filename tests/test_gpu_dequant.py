"""GPU dequantisation (tq_dequantize_keys / tq_dequantize_values) against the
oracle's dense k_hat and v_hat, on records the oracle packed itself.

Tolerances.  Keys are evaluated in float32: the QJL term is a sum of 128
fp16 x (+-1) products and the codebook term one product, then a 128-point
Walsh-Hadamard transform adds 128 terms per output; each step is a float32
sum of at most 256 terms, so the error stays below 256 * 2^-24 of the sum of
magnitudes, which for these rows is < 2e-4 of the row's largest |k_hat|.
bf16 / fp16 outputs add half an ulp of the output type.  Values are one fma
of exact fp16 operands: bit-exact in float32.
"""
import math

import numpy as np
import pytest

import oracle.tq_oracle as O
import tq_workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import kv_cache_quantization_encode_amd as tq  # noqa: E402
from kv_cache_quantization_encode_amd import _lib as L  # noqa: E402

DEV = "cuda"

CFGS = [dict(mode="prod", bits=2), dict(mode="prod", bits=3), dict(mode="prod", bits=4),
        dict(mode="mse", bits=1), dict(mode="mse", bits=2), dict(mode="mse", bits=3), dict(mode="mse", bits=4),
        dict(mode="mse", bits=8), dict(mode="grouped", bits_outlier=4, bits_normal=2),
        dict(mode="grouped", bits_outlier=3, bits_normal=1),
        dict(mode="grouped_prod", bits_outlier=3, bits_normal=2),
        dict(mode="grouped_prod", bits_outlier=4, bits_normal=2)]


def _ocfg(kw):
    return O.KeyConfig(d=128, mode=kw["mode"], bits=kw.get("bits", 3), seed=5,
                       bits_outlier=kw.get("bits_outlier", 4), bits_normal=kw.get("bits_normal", 2))


def _planes(rec, mode):
    p = dict(idx=torch.from_numpy(rec["idx"]).to(DEV),
             norm=torch.from_numpy(np.ascontiguousarray(rec["norm"]).view(np.float16)).to(DEV))
    if mode in ("prod", "grouped_prod"):
        p["signs"] = torch.from_numpy(rec["signs"]).to(DEV)
        p["rnorm"] = torch.from_numpy(np.ascontiguousarray(rec["rnorm"]).view(np.float16)).to(DEV)
    return p


@pytest.mark.parametrize("kw", CFGS, ids=lambda k: "-".join(str(v) for v in k.values()))
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_dequantize_keys_matches_oracle(kw, dtype):
    n = 1000  # ragged: not a multiple of the 256-row block
    scale = W.w5_col_scale() if kw["mode"].startswith("grouped") else None
    kv, _ = W.kv_rows(31, 1, n, scale_cols=scale)
    To = O.build_tables(_ocfg(kw))
    enc = O.encode_keys(kv.astype(np.float64), To)
    ref = O.dequant_keys(enc, To)
    Tg = tq.Tables(L.key_config(seed=5, **kw), DEV)
    got = tq.dequantize_keys(Tg, _planes(O.pack_key_record(enc, To), kw["mode"]), dtype=dtype)
    torch.cuda.synchronize()
    got = got.float().cpu().numpy().astype(np.float64)
    rowmax = np.max(np.abs(ref), axis=1, keepdims=True)
    tol = 2e-4 * rowmax + 1e-7
    if dtype == torch.bfloat16:
        tol = tol + np.abs(ref) * 2.0 ** -8
    err = np.abs(got - ref)
    assert np.all(err <= tol), "worst %.3g (tol %.3g)" % (float(np.max(err - tol)), float(tol.ravel()[np.argmax(err - tol)]))


def test_dequantize_keys_gathers_slots():
    kw = dict(mode="prod", bits=3)
    n = 300
    kv, _ = W.kv_rows(32, 1, n)
    To = O.build_tables(_ocfg(kw))
    enc = O.encode_keys(kv.astype(np.float64), To)
    ref = O.dequant_keys(enc, To)
    Tg = tq.Tables(L.key_config(seed=5, **kw), DEV)
    slots = np.array([5, 299, -1, 0, 300, 17], dtype=np.int64)
    got = tq.dequantize_keys(Tg, _planes(O.pack_key_record(enc, To), "prod"),
                             slots=torch.from_numpy(slots).to(DEV)).cpu().numpy()
    for i, s in enumerate(slots):
        if 0 <= s < n:
            assert np.allclose(got[i], ref[s], rtol=0, atol=2e-4 * np.abs(ref[s]).max())
        else:
            assert np.all(got[i] == 0)


@pytest.mark.parametrize("bits", [2, 4])
def test_dequantize_values_exact(bits):
    n = 777
    vv, _ = W.kv_rows(33, 2, n)
    venc = O.encode_values(vv, bits)
    ref = O.dequant_values(venc)
    vrec = O.pack_value_record(venc, bits)
    vp = {k: torch.from_numpy(v).to(DEV) for k, v in vrec.items()}
    got = tq.dequantize_values(vp, bits).cpu().numpy()
    assert np.array_equal(got, ref.astype(np.float32))
    got16 = tq.dequantize_values(vp, bits, dtype=torch.bfloat16).float().cpu().numpy()
    assert np.array_equal(got16, W.bf16_values(W.bf16_bits(ref.astype(np.float32))))


def test_encode_then_dequantize_round_trip_error():
    """Prefill use: GPU encode then GPU dequantise gives k_hat whose error
    matches the method's distortion (Theorem-1 band for 3-bit MSE keys)."""
    n = 4096
    kv, kb = W.kv_rows(34, 1, n)
    Tg = tq.Tables(L.key_config(mode="mse", bits=3, seed=5), DEV)
    x = torch.from_numpy(kb.view(np.int16)).view(torch.bfloat16).to(DEV)
    kh = tq.dequantize_keys(Tg, tq.encode_keys(Tg, x)).cpu().numpy().astype(np.float64)
    k = kv.astype(np.float64)
    nrm = np.linalg.norm(k, axis=1, keepdims=True)
    mse = float(np.mean(np.sum(((kh - k) / nrm) ** 2, axis=1)))
    assert mse <= math.sqrt(3) * math.pi / 2 * 4.0 ** -3
    assert abs(mse - Tg.mse[0]) < 0.15 * Tg.mse[0]
