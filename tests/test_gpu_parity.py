"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Sizes span several tiles and ragged tails."""
import math

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

DEV = "cuda"


def _ocfg(kw, seed=42):
    return O.KeyConfig(d=128, mode=kw["mode"], bits=kw.get("bits", 3), seed=seed,
                       bits_outlier=kw.get("bits_outlier", 4), bits_normal=kw.get("bits_normal", 2))


def _tables(kw, seed=42):
    return tq.Tables(L.key_config(seed=seed, **kw), DEV), O.build_tables(_ocfg(kw, seed))


def _np(t):
    return t.detach().cpu().numpy()


def _gpu_key_fields(Tg, To, planes, rows=None):
    pl = {k: _np(v) for k, v in planes.items()}
    if rows is not None:
        pl = {k: v[rows] for k, v in pl.items()}
    return P.unpack_gpu_keys(To, pl)


# ------------------------------------------------------------------ encode

KEY_CFGS = [dict(mode="prod", bits=3), dict(mode="prod", bits=4), dict(mode="prod", bits=2),
            dict(mode="mse", bits=4), dict(mode="mse", bits=8), dict(mode="mse", bits=1), dict(mode="mse", bits=2),
            dict(mode="mse", bits=3), dict(mode="grouped", bits_outlier=4, bits_normal=2),
            dict(mode="grouped", bits_outlier=3, bits_normal=1),
            dict(mode="grouped_prod", bits_outlier=3, bits_normal=2),
            dict(mode="grouped_prod", bits_outlier=4, bits_normal=1)]


def _grouped(kw):
    return kw["mode"].startswith("grouped")


def test_encode_w1_unit_keys_fp32():
    """Tiny prod check: 4096 unit-norm fp32 keys, 3-bit prod, seed 42."""
    k, _, _ = W.w1_inputs()
    Tg, To = _tables(dict(mode="prod", bits=3))
    planes = tq.encode_keys(Tg, torch.from_numpy(k).to(DEV))
    torch.cuda.synchronize()
    rep = {}
    P.check_keys(k.astype(np.float64), To, _gpu_key_fields(Tg, To, planes), rep)
    print("w1 band cases:", rep)


@pytest.mark.parametrize("kw", KEY_CFGS, ids=lambda k: "-".join(str(v) for v in k.values()))
def test_encode_keys_modes_bf16(kw):
    n = 3001  # ragged: not a multiple of the 16-key tile
    kv, kb = W.kv_rows(9, 1, n, scale_cols=W.w5_col_scale() if _grouped(kw) else None)
    Tg, To = _tables(kw, seed=1234)
    x = torch.from_numpy(kb.view(np.int16)).view(torch.bfloat16).to(DEV)
    planes = tq.encode_keys(Tg, x)
    torch.cuda.synchronize()
    P.check_keys(kv.astype(np.float64), To, _gpu_key_fields(Tg, To, planes))


@pytest.mark.parametrize("kw", [dict(mode="prod", bits=3), dict(mode="mse", bits=4), dict(mode="mse", bits=2),
                                dict(mode="grouped", bits_outlier=4, bits_normal=2),
                                dict(mode="grouped_prod", bits_outlier=3, bits_normal=2)],
                         ids=["prod3", "mse4", "mse2", "grouped42", "grouped_prod32"])
@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_encode_keys_modes_f32_f16(kw, dtype):
    """The float32 and fp16 input paths (their own unpack and sign steps) in
    the direct-bucketize, hint-grid and grouped encoders."""
    n = 1000  # ragged
    rng = np.random.default_rng(17)
    scale = W.w5_col_scale() if _grouped(kw) else np.ones(128)
    x = (rng.standard_normal((n, 128)) * scale).astype(np.float32 if dtype == "f32" else np.float16)
    Tg, To = _tables(kw, seed=77)
    planes = tq.encode_keys(Tg, torch.from_numpy(x).to(DEV))
    torch.cuda.synchronize()
    P.check_keys(x.astype(np.float64), To, _gpu_key_fields(Tg, To, planes))


def test_encode_keys_strided_fp16_with_slots():
    """fp16 rows with a row stride, written through a slot map that permutes,
    skips (-1 and out-of-range) and leaves other records untouched."""
    kw = dict(mode="prod", bits=3)
    Tg, To = _tables(kw)
    n, nrec = 500, 700
    rng = np.random.default_rng(5)
    base = rng.standard_normal((n, 160)).astype(np.float16)
    x = torch.from_numpy(base).to(DEV)[:, :128]
    assert x.stride(0) == 160
    slots = rng.permutation(nrec)[:n].astype(np.int64)
    slots[7] = -1
    slots[8] = nrec + 3
    planes = tq.key_planes(Tg, nrec, DEV)
    for v in planes.values():
        v.view(torch.uint8).fill_(0xAB)
    tq.encode_keys(Tg, x, planes, slots=torch.from_numpy(slots).to(DEV), n_records=nrec)
    torch.cuda.synchronize()
    ok = (slots >= 0) & (slots < nrec)
    fields = _gpu_key_fields(Tg, To, planes, rows=slots[ok])
    P.check_keys(base[ok, :128].astype(np.float64), To, fields)
    untouched = np.setdiff1d(np.arange(nrec), slots[ok])
    assert np.all(_np(planes["idx"])[untouched] == 0xAB)
    assert np.all(_np(planes["signs"])[untouched] == 0xAB)


@pytest.mark.parametrize("kw,cell", [(dict(mode="prod", bits=3), 2), (dict(mode="prod", bits=2), 1),
                                     (dict(mode="mse", bits=2), 2), (dict(mode="mse", bits=4), 8)],
                         ids=["prod3", "prod2", "mse2", "mse4"])
def test_encode_zero_key(kw, cell):
    """A zero key: norms 0, every y = 0 in the cell just above the middle
    boundary (ties go up), and (prod) the signs of S(-c[idx]) as the oracle
    gives them."""
    Tg, To = _tables(kw)
    x = torch.zeros((16, 128), dtype=torch.bfloat16, device=DEV)
    planes = tq.encode_keys(Tg, x)
    torch.cuda.synchronize()
    f = _gpu_key_fields(Tg, To, planes)
    assert np.all(f["norm16"] == 0)
    assert np.all(f["idx"] == cell)
    if kw["mode"] == "prod":
        assert np.all(f["rnorm16"] == 0)
        P.check_keys(np.zeros((16, 128)), To, f)


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_encode_values_exact(bits, dtype):
    n = 1001
    vv, vb = W.kv_rows(9, 2, n)
    if dtype == "f32":
        vv = W.gaussian(9, 3, (n, 128))
        x = torch.from_numpy(vv).to(DEV)
    elif dtype == "f16":
        vh = W.gaussian(9, 4, (n, 128)).astype(np.float16)
        vv = vh.astype(np.float32)
        x = torch.from_numpy(vh).to(DEV)
    else:
        x = torch.from_numpy(vb.view(np.int16)).view(torch.bfloat16).to(DEV)
    vv = vv.copy()
    # a constant group and a group with repeated extremes
    if dtype == "f32":
        x[3, :32] = 1.5
        vv[3, :32] = 1.5
    # a group of exact rounding ties: min 0 and max 2^b - 1 give s = 1, z = 0,
    # so k + 1/2 must go to the even code (exact in every input type)
    top = (1 << bits) - 1
    tie_row = np.ones(32, dtype=np.float32)
    tie_row[0], tie_row[1] = 0.0, float(top)
    tie_row[2:2 + top] = np.arange(top, dtype=np.float32) + 0.5
    vv[5, 32:64] = tie_row
    x[5, 32:64] = torch.from_numpy(tie_row).to(DEV).to(x.dtype)
    planes = tq.encode_values(x, bits)
    torch.cuda.synchronize()
    enc = P.check_values(vv, bits, _np(planes["codes"]), _np(planes["scale"]), _np(planes["zero"]))
    even = [int(t - 0.5) if int(t - 0.5) % 2 == 0 else int(t + 0.5) for t in tie_row[2:2 + top]]
    assert list(enc["codes"][5, 34:34 + top]) == even


# ------------------------------------------------------------------ decode

def _oracle_cache(kw, v_bits, B, Hkv, max_ctx, wid=11, seed=42, key_scale=None):
    """Oracle-encoded planes [B*Hkv*max_ctx records] plus dense k_hat, v_hat."""
    To = O.build_tables(_ocfg(kw, seed))
    n = B * Hkv * max_ctx
    kv, _ = W.kv_rows(wid, 1, n, scale_cols=key_scale)
    vv, _ = W.kv_rows(wid, 2, n)
    enc = O.encode_keys(kv.astype(np.float64), To)
    rec = O.pack_key_record(enc, To)
    venc = O.encode_values(vv, v_bits)
    vrec = O.pack_value_record(venc, v_bits)
    khat = O.dequant_keys(enc, To).reshape(B, Hkv, max_ctx, 128)
    vhat = O.dequant_values(venc).reshape(B, Hkv, max_ctx, 128)
    planes = dict(idx=torch.from_numpy(rec["idx"]).to(DEV),
                  norm=torch.from_numpy(np.ascontiguousarray(rec["norm"]).view(np.float16)).to(DEV))
    if "signs" in rec:
        planes["signs"] = torch.from_numpy(rec["signs"]).to(DEV)
        planes["rnorm"] = torch.from_numpy(np.ascontiguousarray(rec["rnorm"]).view(np.float16)).to(DEV)
    vpl = dict(codes=torch.from_numpy(vrec["codes"]).to(DEV), scale=torch.from_numpy(vrec["scale"]).to(DEV),
               zero=torch.from_numpy(vrec["zero"]).to(DEV))
    return To, planes, vpl, khat, vhat


def _run_decode(kw, v_bits, B, Hq, Hkv, max_ctx, ctx, seed=42, q_dtype=torch.bfloat16, key_scale=None,
                wid=11):
    To, kp, vp, khat, vhat = _oracle_cache(kw, v_bits, B, Hkv, max_ctx, wid=wid, seed=seed,
                                           key_scale=key_scale)
    Tg = tq.Tables(L.key_config(seed=seed, **kw), DEV)
    qv, qb = W.queries(wid, B, Hq)
    if q_dtype == torch.bfloat16:
        q = torch.from_numpy(qb.view(np.int16)).view(torch.bfloat16).to(DEV)
    else:
        q = torch.from_numpy(qv).to(DEV).to(q_dtype)
        qv = q.float().cpu().numpy()
    ctx_t = torch.tensor(ctx, dtype=torch.int32, device=DEV)
    out, lse, scores = tq.decode_attention(Tg, q, ctx_t, kp, vp, v_bits, max_ctx, with_lse=True,
                                           with_scores=True)
    torch.cuda.synchronize()
    out, lse, scores = _np(out), _np(lse), _np(scores)
    G = Hq // Hkv
    worst = 0.0
    for b in range(B):
        for h in range(Hkv):
            heads = slice(h * G, (h + 1) * G)
            s_ref, o_ref, lse_ref = O.decode_attention(qv[b, heads].astype(np.float64), khat[b, h], vhat[b, h],
                                                       ctx[b])
            if ctx[b] > 0:
                worst = max(worst, P.check_scores(scores[b, heads, :ctx[b]], s_ref))
                assert np.all(np.abs(lse[b, heads] - lse_ref) <= 5e-3 * np.maximum(1.0, np.abs(lse_ref)))
            else:
                assert np.all(np.isneginf(lse[b, heads]))
            P.check_out(out[b, heads], o_ref)
    return worst


DEC_CASES = [
    (dict(mode="prod", bits=3), 2),
    (dict(mode="prod", bits=4), 4),
    (dict(mode="prod", bits=2), 2),
    (dict(mode="grouped", bits_outlier=4, bits_normal=2), 4),
    (dict(mode="mse", bits=2), 2),
    (dict(mode="mse", bits=3), 4),
    # every other supported key format, with the other value width
    (dict(mode="prod", bits=3), 4),
    (dict(mode="mse", bits=1), 4),
    (dict(mode="mse", bits=3), 2),
    (dict(mode="grouped", bits_outlier=3, bits_normal=2), 2),
    (dict(mode="grouped", bits_outlier=2, bits_normal=2), 4),
    (dict(mode="grouped", bits_outlier=4, bits_normal=1), 2),
    # grouped halves with the QJL sketch of the whole residual (three table classes)
    (dict(mode="grouped_prod", bits_outlier=3, bits_normal=2), 2),
    (dict(mode="grouped_prod", bits_outlier=3, bits_normal=2), 4),
    (dict(mode="grouped_prod", bits_outlier=4, bits_normal=1), 4),
    # indices of 4 to 6 bits: one lookup table per coordinate (nibbles or bytes)
    (dict(mode="mse", bits=4), 2),
    (dict(mode="mse", bits=5), 4),
    (dict(mode="mse", bits=6), 2),
    (dict(mode="prod", bits=5), 4),
    (dict(mode="prod", bits=6), 2),
    (dict(mode="prod", bits=7), 4),
    # indices of 7 and 8 bits: scored directly (float32, the codebook in LDS)
    (dict(mode="mse", bits=8), 2),
    (dict(mode="mse", bits=7), 4),
    (dict(mode="prod", bits=8), 4),
    (dict(mode="prod", bits=9), 2),
]


@pytest.mark.parametrize("kw,vb", DEC_CASES, ids=lambda x: str(x))
def test_decode_oracle_packed(kw, vb):
    key_scale = W.w5_col_scale() if _grouped(kw) else None
    worst = _run_decode(kw, vb, B=2, Hq=8, Hkv=2, max_ctx=2500, ctx=[2500, 1337], key_scale=key_scale)
    print("worst relative score error", worst)


def test_decode_w1_scores_all_keys():
    """Tiny prod check: 8 queries against one KV head of 4096 unit keys (fp32),
    scores for every key and the softmax-weighted values."""
    kw = dict(mode="prod", bits=3)
    k, v, qv = W.w1_inputs()
    To = O.build_tables(_ocfg(kw))
    Tg = tq.Tables(L.key_config(**kw), DEV)
    enc = O.encode_keys(k.astype(np.float64), To)
    rec = O.pack_key_record(enc, To)
    venc = O.encode_values(v, 2)
    vrec = O.pack_value_record(venc, 2)
    kp = dict(idx=torch.from_numpy(rec["idx"]).to(DEV), norm=torch.from_numpy(rec["norm"]).to(DEV),
              signs=torch.from_numpy(rec["signs"]).to(DEV), rnorm=torch.from_numpy(rec["rnorm"]).to(DEV))
    vp = {k2: torch.from_numpy(v2).to(DEV) for k2, v2 in vrec.items()}
    q = torch.from_numpy(qv).to(DEV).reshape(1, 8, 128)
    out, lse, scores = tq.decode_attention(Tg, q, torch.tensor([4096], dtype=torch.int32, device=DEV), kp, vp,
                                           2, 4096, with_lse=True, with_scores=True)
    torch.cuda.synchronize()
    s_ref, o_ref, _ = O.decode_attention(qv.astype(np.float64), O.dequant_keys(enc, To),
                                         O.dequant_values(venc), 4096)
    P.check_scores(_np(scores)[0], s_ref)
    P.check_out(_np(out)[0], o_ref)


@pytest.mark.parametrize("G", [1, 2, 8])
def test_decode_group_sizes(G):
    _run_decode(dict(mode="prod", bits=3), 2, B=1, Hq=2 * G, Hkv=2, max_ctx=700, ctx=[700])


def test_decode_short_and_empty_contexts():
    _run_decode(dict(mode="prod", bits=3), 2, B=4, Hq=4, Hkv=1, max_ctx=300, ctx=[0, 1, 65, 300])


@pytest.mark.parametrize("q_dtype", [torch.float32, torch.float16], ids=["f32", "f16"])
def test_decode_fp32_and_fp16_queries(q_dtype):
    _run_decode(dict(mode="prod", bits=3), 2, B=1, Hq=4, Hkv=1, max_ctx=1000, ctx=[999], q_dtype=q_dtype)


def test_decode_is_deterministic():
    kw = dict(mode="prod", bits=3)
    To, kp, vp, _, _ = _oracle_cache(kw, 2, 2, 2, 3000)
    Tg = tq.Tables(L.key_config(**kw), DEV)
    _, qb = W.queries(11, 2, 8)
    q = torch.from_numpy(qb.view(np.int16)).view(torch.bfloat16).to(DEV)
    ctx = torch.tensor([3000, 2000], dtype=torch.int32, device=DEV)
    a = tq.decode_attention(Tg, q, ctx, kp, vp, 2, 3000)[0].clone()
    b = tq.decode_attention(Tg, q, ctx, kp, vp, 2, 3000)[0]
    assert torch.equal(a, b)


def test_end_to_end_gpu_encode_then_decode():
    """GPU-encoded cache decoded on the GPU against the oracle's encode+decode
    of the same inputs (keys whose bytes differ in a band case are rare and
    move a score by at most one centroid step; outputs stay within 1e-2)."""
    kw = dict(mode="prod", bits=3)
    B, Hq, Hkv, N = 1, 8, 2, 2048
    Tg, To = _tables(kw)
    kv, kb = W.kv_rows(12, 1, B * Hkv * N)
    vv, vb = W.kv_rows(12, 2, B * Hkv * N)
    kp = tq.encode_keys(Tg, torch.from_numpy(kb.view(np.int16)).view(torch.bfloat16).to(DEV))
    vp = tq.encode_values(torch.from_numpy(vb.view(np.int16)).view(torch.bfloat16).to(DEV), 2)
    qv, qb = W.queries(12, B, Hq)
    q = torch.from_numpy(qb.view(np.int16)).view(torch.bfloat16).to(DEV)
    out, _, _ = tq.decode_attention(Tg, q, torch.tensor([N], dtype=torch.int32, device=DEV), kp, vp, 2, N)
    torch.cuda.synchronize()
    enc = O.encode_keys(kv.astype(np.float64), To)
    khat = O.dequant_keys(enc, To).reshape(B, Hkv, N, 128)
    vhat = O.dequant_values(O.encode_values(vv, 2)).reshape(B, Hkv, N, 128)
    out = _np(out)
    for h in range(Hkv):
        _, o_ref, _ = O.decode_attention(qv[0, 4 * h:4 * h + 4].astype(np.float64), khat[0, h], vhat[0, h], N)
        P.check_out(out[0, 4 * h:4 * h + 4], o_ref)


def test_decode_clamps_out_of_range_lengths():
    """ctx_len outside [0, max_ctx] is clamped on the device: a length past
    max_ctx decodes as max_ctx and a negative one as an empty sequence."""
    kw = dict(mode="prod", bits=3)
    B, Hq, Hkv, max_ctx = 2, 4, 1, 256
    Tg = tq.Tables(L.key_config(seed=3, **kw), DEV)
    n = B * Hkv * max_ctx
    keys = torch.from_numpy(W.kv_rows(81, 1, n)[0]).to(DEV).to(torch.bfloat16)
    vals = torch.from_numpy(W.kv_rows(81, 2, n)[0]).to(DEV).to(torch.bfloat16)
    kp, vp = tq.encode_keys(Tg, keys), tq.encode_values(vals, 2)
    q = torch.from_numpy(W.queries(81, B, Hq)[1].view(np.int16)).view(torch.bfloat16).to(DEV)
    dec = tq.Decoder(Tg, B, Hq, Hkv, max_ctx, 2)
    res = []
    for ctx in ([max_ctx + 50, -3], [max_ctx, 0]):
        lse = torch.empty((B, Hq), device=DEV)
        out = dec(q, torch.tensor(ctx, dtype=torch.int32, device=DEV), kp, vp, lse=lse)
        res.append((out.clone(), lse.clone()))
    torch.cuda.synchronize()
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])
    assert torch.all(res[0][0][1] == 0) and torch.all(torch.isinf(res[0][1][1]))


@pytest.mark.parametrize("kw", [dict(mode="mse", bits=4), dict(mode="mse", bits=1), dict(mode="prod", bits=3),
                                dict(mode="grouped", bits_outlier=4, bits_normal=2),
                                dict(mode="grouped_prod", bits_outlier=3, bits_normal=2)],
                         ids=["mse4", "mse1", "prod3", "grouped42", "grouped_prod32"])
def test_encode_extreme_norms(kw):
    """Finite bf16 keys of norm about 1e-30 and 1e30 (their fp32 sums of
    squares would underflow to 0 or overflow to inf), and grouped keys whose
    halves differ by 60 decades: index and sign bytes as the oracle's; the
    stored fp16 norms are 0 and +inf, as the oracle's fp16 rounding gives."""
    n = 48
    base, _ = W.kv_rows(81, 1, 3 * n)
    x = base.astype(np.float64) / np.sqrt(128.0)
    x[:n] *= 1e-30
    x[n:2 * n] *= 1e30
    x[2 * n:, :64] *= 1e30
    x[2 * n:, 64:] *= 1e-30
    xv, xb = W.to_bf16(x.astype(np.float32))
    assert np.all(np.isfinite(xv)) and np.all(np.abs(xv[:n]).max(axis=1) > 0)
    Tg, To = _tables(kw)
    planes = tq.encode_keys(Tg, torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(DEV))
    torch.cuda.synchronize()
    f = _gpu_key_fields(Tg, To, planes)
    P.check_keys(xv.astype(np.float64), To, f)
    nrm = f["norm16"].astype(np.float64).reshape(3 * n, -1)
    assert np.all(nrm[:n] == 0) and np.all(np.isposinf(nrm[n:2 * n]))


def test_encode_writes_nothing_with_foreign_tables():
    """Tables built for another configuration (8-bit MSE tables given with a
    2-bit MSE configuration, whose rows are four times shorter): the key
    encoder checks the tables' header against the configuration and leaves
    every plane untouched."""
    T2 = tq.Tables(L.key_config(mode="mse", bits=2), DEV)
    T8 = tq.Tables(L.key_config(mode="mse", bits=8), DEV)
    T2.dev = T8.dev
    planes = tq.key_planes(T2, 64, DEV)
    for v in planes.values():
        v.view(torch.uint8).fill_(0xAB)
    x = W.normal_bf16_device(5, 1, (64, 128), DEV)
    tq.encode_keys(T2, x, planes)
    torch.cuda.synchronize()
    for v in planes.values():
        assert torch.all(v.view(torch.uint8) == 0xAB)


def test_encode_zero_key_grouped_prod():
    """A zero key in grouped + QJL mode: both norms and rho 0, each half's
    y = 0 in the cell above its middle boundary, and every sign bit 1 (the
    weighted residual is 0, and [0 >= 0])."""
    kw = dict(mode="grouped_prod", bits_outlier=3, bits_normal=2)
    Tg, To = _tables(kw)
    planes = tq.encode_keys(Tg, torch.zeros((16, 128), dtype=torch.bfloat16, device=DEV))
    torch.cuda.synchronize()
    f = _gpu_key_fields(Tg, To, planes)
    assert np.all(f["norm16"] == 0) and np.all(f["rnorm16"] == 0)
    assert np.all(f["idx"][:, :64] == 4) and np.all(f["idx"][:, 64:] == 2)
    assert np.all(f["bits"] == 1)
    P.check_keys(np.zeros((16, 128)), To, f)
