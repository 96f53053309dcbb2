"""GPU parity of tq_decode_attention_append: the step's new key and value are
encoded, stored and attended inside the decode launch.  Checked against the
CPU oracle on the same seeded inputs: the stored records by the encode rules
(tests/parity.py), every other record untouched, and the scores, lse and
outputs against the oracle's decode over the cache that now holds the
appended records."""
import numpy as np
import pytest

import oracle.tq_oracle as O
import tq_workloads as W
from tests import parity as P

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU runs, skipped there
    pytest.skip("needs a GPU", allow_module_level=True)

import kv_cache_quantization_encode_amd as tq  # noqa: E402
from kv_cache_quantization_encode_amd import _lib as L  # noqa: E402
from tests.test_gpu_parity import _oracle_cache  # noqa: E402

DEV = "cuda"


def _np(t):
    return t.detach().cpu().numpy()


def _new_rows(wid, n, dtype):
    """n keys and n values as (float64 oracle input, device tensor of dtype)."""
    out = []
    for kind in (1, 2):
        f32, b16 = W.kv_rows(wid, kind, n)
        if dtype == torch.bfloat16:
            t = torch.from_numpy(b16.view(np.int16)).view(torch.bfloat16).to(DEV)
            vals = t.float().cpu().numpy()
        else:
            t = torch.from_numpy(f32).to(DEV).to(dtype)
            vals = t.float().cpu().numpy()
        out.append((vals.astype(np.float64), t))
    return out


def _slots(B, Hkv, max_ctx, ctx):
    return [((b * Hkv + h) * max_ctx + ctx[b] - 1, b, h) for b in range(B) for h in range(Hkv) if ctx[b] > 0]


def _step(Tg, To, kw, vb, kp, vp, khat, vhat, B, Hq, Hkv, max_ctx, ctx, wid, kv_dtype, q_dtype=torch.bfloat16):
    """One appending decode step; checks it and updates khat / vhat in place."""
    (kf, kt), (vf, vt) = _new_rows(wid, B * Hkv, kv_dtype)
    qv, qb = W.queries(wid, B, Hq)
    if q_dtype == torch.bfloat16:
        q = torch.from_numpy(qb.view(np.int16)).view(torch.bfloat16).to(DEV)
    else:
        q = torch.from_numpy(qv).to(DEV).to(q_dtype)
        qv = q.float().cpu().numpy()
    slots = _slots(B, Hkv, max_ctx, ctx)
    # the records the call will write are garbage beforehand: nothing may read them
    for s, _, _ in slots:
        for p in list(kp.values()) + list(vp.values()):
            p.view(torch.uint8).view(p.shape[0], -1)[s] = 0xFF
    before_k = {k: _np(v).copy() for k, v in kp.items()}
    before_v = {k: _np(v).copy() for k, v in vp.items()}
    ctx_t = torch.tensor(ctx, dtype=torch.int32, device=DEV)
    dec = tq.Decoder(Tg, B, Hq, Hkv, max_ctx, vb, q.dtype, DEV)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    scores = torch.full((B, Hq, max_ctx), float("nan"), dtype=torch.float32, device=DEV)
    out = dec(q, ctx_t, kp, vp, lse=lse, scores=scores, k_new=kt.view(B, Hkv, 128), v_new=vt.view(B, Hkv, 128))
    torch.cuda.synchronize()
    out, lse, scores = _np(out), _np(lse), _np(scores)
    rows = np.array([s for s, _, _ in slots], dtype=np.int64)
    src = np.array([b * Hkv + h for _, b, h in slots], dtype=np.int64)
    # records written: the encode rules against the oracle
    after_k = {k: _np(v) for k, v in kp.items()}
    after_v = {k: _np(v) for k, v in vp.items()}
    if len(rows):
        g = P.unpack_gpu_keys(To, {k: v[rows] for k, v in after_k.items()})
        P.check_keys(kf[src], To, g)
        P.check_values(vf[src].astype(np.float32), vb, after_v["codes"][rows], after_v["scale"][rows],
                       after_v["zero"][rows])
        # the cache as a later call reads it: the stored records, dequantised
        kh = O.dequant_keys(g, To)
        venc = dict(codes=O.unpack_fields(after_v["codes"][rows], O.index_width(vb), 128),
                    scale16=after_v["scale"][rows].view(np.float16), zero16=after_v["zero"][rows].view(np.float16))
        vh = O.dequant_values(venc)
        for i, (_, b, h) in enumerate(slots):
            khat[b, h, ctx[b] - 1] = kh[i]
            vhat[b, h, ctx[b] - 1] = vh[i]
    # nothing else written
    mask = np.ones(B * Hkv * max_ctx, dtype=bool)
    mask[rows] = False
    for k in before_k:
        assert np.array_equal(after_k[k].reshape(B * Hkv * max_ctx, -1)[mask],
                              before_k[k].reshape(B * Hkv * max_ctx, -1)[mask]), "key plane %s changed" % k
    for k in before_v:
        assert np.array_equal(after_v[k].reshape(B * Hkv * max_ctx, -1)[mask],
                              before_v[k].reshape(B * Hkv * max_ctx, -1)[mask]), "value plane %s changed" % k
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hkv):
            heads = slice(h * G, (h + 1) * G)
            s_ref, o_ref, lse_ref = O.decode_attention(qv[b, heads].astype(np.float64), khat[b, h], vhat[b, h],
                                                       ctx[b])
            if ctx[b] > 0:
                P.check_scores(scores[b, heads, :ctx[b]], s_ref)
                assert np.all(np.abs(lse[b, heads] - lse_ref) <= 5e-3 * np.maximum(1.0, np.abs(lse_ref)))
            else:
                assert np.all(np.isneginf(lse[b, heads]))
            P.check_out(out[b, heads], o_ref)


def _run(kw, vb, B, Hq, Hkv, max_ctx, ctxs, kv_dtype=torch.bfloat16, q_dtype=torch.bfloat16, wid=21):
    To, kp, vp, khat, vhat = _oracle_cache(kw, vb, B, Hkv, max_ctx, wid=11)
    Tg = tq.Tables(L.key_config(seed=42, **kw), DEV)
    for i, ctx in enumerate(ctxs):
        _step(Tg, To, kw, vb, kp, vp, khat, vhat, B, Hq, Hkv, max_ctx, ctx, wid + i, kv_dtype, q_dtype)


APPEND_CASES = [
    (dict(mode="prod", bits=3), 2),
    (dict(mode="prod", bits=4), 4),
    (dict(mode="prod", bits=2), 2),
    (dict(mode="prod", bits=7), 4),
    (dict(mode="mse", bits=1), 4),
    (dict(mode="mse", bits=2), 2),
    (dict(mode="mse", bits=3), 4),
    (dict(mode="mse", bits=4), 2),
    (dict(mode="mse", bits=6), 4),
    (dict(mode="grouped", bits_outlier=4, bits_normal=2), 4),
    (dict(mode="grouped", bits_outlier=3, bits_normal=2), 2),
    (dict(mode="grouped", bits_outlier=2, bits_normal=2), 4),
    (dict(mode="grouped", bits_outlier=4, bits_normal=1), 2),
    (dict(mode="grouped_prod", bits_outlier=3, bits_normal=2), 2),
    (dict(mode="grouped_prod", bits_outlier=4, bits_normal=1), 4),
]


@pytest.mark.parametrize("kw,vb", APPEND_CASES, ids=lambda x: str(x))
def test_append_decode(kw, vb):
    # ragged lengths: a full context, one token, none, a ragged tile, and the
    # first token of the second split (alone in its split's range)
    _run(kw, vb, B=5, Hq=8, Hkv=2, max_ctx=2048, ctxs=[[2048, 1, 0, 65, 1025]])


@pytest.mark.parametrize("kv_dtype", [torch.float32, torch.float16], ids=str)
def test_append_decode_input_types(kv_dtype):
    _run(dict(mode="prod", bits=3), 2, B=2, Hq=4, Hkv=1, max_ctx=1500, ctxs=[[1500, 700]], kv_dtype=kv_dtype,
         q_dtype=kv_dtype)


def test_append_decode_two_quads_and_consecutive_steps():
    """Eight query heads per KV head (two workgroups hold the new token; one
    stores it), and three steps in a row, each attending the tokens the
    earlier steps appended."""
    _run(dict(mode="prod", bits=3), 2, B=2, Hq=16, Hkv=2, max_ctx=1200, ctxs=[[900, 1], [901, 2], [902, 3]])


def test_append_decode_rejects_8bit_indices():
    """8-bit MSE keys decode (scored directly) but are not appended inside the
    decode: the one-wave encoder holds at most 64 boundaries in its lanes."""
    kw = dict(mode="mse", bits=8)
    Tg = tq.Tables(L.key_config(seed=42, **kw), DEV)
    kp = tq.key_planes(Tg, 64, DEV)
    vp = tq.value_planes(2, 64, device=DEV)
    q = torch.zeros((1, 4, 128), dtype=torch.bfloat16, device=DEV)
    kn = torch.zeros((1, 1, 128), dtype=torch.bfloat16, device=DEV)
    dec = tq.Decoder(Tg, 1, 4, 1, 64, 2, q.dtype, DEV)
    with pytest.raises(L.TqError) as e:
        dec(q, torch.tensor([10], dtype=torch.int32, device=DEV), kp, vp, k_new=kn, v_new=kn)
    assert e.value.status == L.TQ_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(mode="prod", bits=3), dict(mode="mse", bits=4), dict(mode="mse", bits=1),
                                dict(mode="grouped", bits_outlier=4, bits_normal=2),
                                dict(mode="grouped_prod", bits_outlier=3, bits_normal=2)],
                         ids=["prod3", "mse4", "mse1", "grouped42", "grouped_prod32"])
def test_append_decode_extreme_norms(kw):
    """New keys of norm about 1e-30 and 1e30 (fp32 sums of their squares would
    underflow or overflow), keys whose halves differ by 60 decades and an
    all-zero key, appended inside the decode: index and sign bytes as the
    oracle's, stored fp16 norms 0, +inf (per half for the grouped modes) and
    0 as the oracle's rounding gives."""
    B, Hkv, Hq, max_ctx = 8, 6, 24, 128
    n = B * Hkv
    base, _ = W.kv_rows(82, 1, n)
    x = base.astype(np.float64) / np.sqrt(128.0)
    x[:16] *= 1e-30
    x[16:32] *= 1e30
    x[32:40, :64] *= 1e30
    x[32:40, 64:] *= 1e-30
    x[-1] = 0.0
    xv, xb = W.to_bf16(x.astype(np.float32))
    vv, vb = W.kv_rows(82, 2, n)
    To, kp, vp, _, _ = _oracle_cache(kw, 2, B, Hkv, max_ctx, wid=11)
    Tg = tq.Tables(L.key_config(seed=42, **kw), DEV)
    q = torch.from_numpy(W.queries(82, B, Hq)[1].view(np.int16)).view(torch.bfloat16).to(DEV)
    kn = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(DEV).view(B, Hkv, 128)
    vn = torch.from_numpy(vb.view(np.int16)).view(torch.bfloat16).to(DEV).view(B, Hkv, 128)
    ctx = torch.full((B,), 70, dtype=torch.int32, device=DEV)
    tq.decode_attention(Tg, q, ctx, kp, vp, 2, max_ctx, k_new=kn, v_new=vn)
    torch.cuda.synchronize()
    rows = np.arange(n) * max_ctx + 69
    g = P.unpack_gpu_keys(To, {k: _np(v)[rows] for k, v in kp.items()})
    P.check_keys(xv.astype(np.float64), To, g)
    nrm = g["norm16"].astype(np.float64).reshape(n, -1)
    assert np.all(nrm[:16] == 0) and np.all(np.isposinf(nrm[16:32])) and np.all(nrm[-1] == 0)
    P.check_values(vn.view(n, 128).float().cpu().numpy(), 2, _np(vp["codes"])[rows], _np(vp["scale"])[rows],
                   _np(vp["zero"])[rows])
