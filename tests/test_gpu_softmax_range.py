"""GPU decode against the oracle where the softmax weights span a wide range.

One key dominates (logit gap 15.5 for the first query head of the group) and
the other 131,071 keys have nearly equal, small weights (about e^-15.5 each),
so together they carry about 1.5 % of the mass.  Their p.V contributions
fall far below fp16's normal range unless the weights are rescaled; the
kernel carries p * 2^14 and renormalises each tile's value scales by a power
of two.  Values are shifted (mean 3) so that dropping the small weights'
code part, while keeping their zero-point part, would bias the output by
several hundredths.  Value magnitudes of 1e-4, 1 and 1000 exercise the
per-tile scale exponent; the output tolerance scales with them (1e-2 for
unit-scale values)."""
import math

import numpy as np
import pytest

import oracle.tq_oracle as O
import tq_workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU runs, skipped there
    pytest.skip("needs a GPU", allow_module_level=True)

import kv_cache_quantization_encode_amd as tq  # noqa: E402
from kv_cache_quantization_encode_amd import _lib as L  # noqa: E402

DEV = "cuda"
N = 131072


@pytest.fixture(scope="module")
def peaky_keys():
    """Oracle-encoded prod 3-bit keys: N(0, 0.05^2) keys plus one at 37 %
    depth along the first query head, with q.k / sqrt(d) = 15.5."""
    To = O.build_tables(O.KeyConfig(mode="prod", bits=3, seed=42))
    qv, qb = W.queries(31, 1, 4)
    kv, _ = W.kv_rows(31, 1, N)
    keys = kv.astype(np.float64) * 0.05
    q0 = qv[0, 0].astype(np.float64)            # bf16 values, as the GPU sees them
    pos = int(0.37 * N)
    keys[pos] = q0 / np.linalg.norm(q0) * (15.5 * math.sqrt(128) / np.linalg.norm(q0))
    enc = O.encode_keys(keys, To)
    rec = O.pack_key_record(enc, To)
    khat = O.dequant_keys(enc, To)
    kp = dict(idx=torch.from_numpy(rec["idx"]).to(DEV),
              norm=torch.from_numpy(np.ascontiguousarray(rec["norm"]).view(np.float16)).to(DEV),
              signs=torch.from_numpy(rec["signs"]).to(DEV), rnorm=torch.from_numpy(rec["rnorm"]).to(DEV))
    q = torch.from_numpy(qb.view(np.int16)).view(torch.bfloat16).to(DEV)
    return kp, khat, q, qv.astype(np.float64)


@pytest.mark.parametrize("vscale", [1e-4, 1.0, 1000.0])
def test_decode_dominant_token_128k_four_bit_values(peaky_keys, vscale):
    print("peaky softmax: 1 x 1 KV head x 4 q heads, ctx 131072, prod 3-bit keys, 4-bit values, scale %g"
          % vscale, flush=True)
    kp, khat, q, qf = peaky_keys
    vv, _ = W.kv_rows(31, 2, N)
    vals = ((vv.astype(np.float64) + 3.0) * vscale).astype(np.float32)
    venc = O.encode_values(vals, 4)
    vrec = O.pack_value_record(venc, 4)
    vhat = O.dequant_values(venc)
    vp = dict(codes=torch.from_numpy(vrec["codes"]).to(DEV), scale=torch.from_numpy(vrec["scale"]).to(DEV),
              zero=torch.from_numpy(vrec["zero"]).to(DEV))
    Tg = tq.Tables(L.key_config(mode="prod", bits=3, seed=42), DEV)
    ctx_t = torch.tensor([N], dtype=torch.int32, device=DEV)
    out, lse, _ = tq.decode_attention(Tg, q, ctx_t, kp, vp, 4, N, with_lse=True)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy()[0], lse.cpu().numpy()[0]
    s_ref, o_ref, lse_ref = O.decode_attention(qf[0], khat, vhat, N)
    # the regime the test is about: the dominant key takes ~98.5 % of head 0's
    # weight and the rest share the remainder in weights far below 2^-14
    x = s_ref[0] / math.sqrt(128)
    p = np.exp(x - x.max())
    rest = (p.sum() - 1.0) / p.sum()
    assert 0.005 < rest < 0.05 and np.median(p) < 2.0 ** -20, (rest, np.median(p))
    err = np.abs(out - o_ref)
    tol = 1e-2 * vscale
    assert np.all(err <= tol), "output error %.3g > %.3g (heads %s)" % (err.max(), tol, err.max(axis=1))
    assert np.all(np.abs(lse - lse_ref) <= 5e-3 * np.maximum(1.0, np.abs(lse_ref)))
