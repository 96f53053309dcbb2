"""GPU parity at the full sizes of the five workloads.

Every GPU output here is produced at full size, in the launch configuration
the benchmark uses (one tq_decode_attention call over the whole batch); the
oracle recomputes sampled (sequence, KV head) groups or layers one by one:
  - encode: the sampled rows' index/sign bytes and norms under the band rule,
    value codes bit-exact;
  - decode on the oracle's packed cache: the sampled groups' records are
    overwritten with the oracle's own encoding, and their scores, outputs and
    log-sum-exp are compared with the oracle's attention over its k_hat, v_hat;
  - end to end (GPU-encoded cache): outputs within 1e-2 of the oracle's
    encode + decode of the same inputs.
"""
import math

import numpy as np
import pytest

import oracle.tq_oracle as O
import tq_workloads as W
from tests import parity as P

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import kv_cache_quantization_encode_amd as tq  # noqa: E402
from kv_cache_quantization_encode_amd import _lib as L  # noqa: E402

DEV = "cuda"
D = 128


def _np(t):
    return t.detach().cpu().numpy()


def _bf16_rows(x, rows):
    """float32 values of bf16 device rows."""
    return x[rows].float().cpu().numpy()


def _gpu_fields(To, kp, rows):
    pl = {k: _np(v[rows]) for k, v in kp.items()}
    return P.unpack_gpu_keys(To, pl)


def _overwrite(kp, vp, rows, rec, vrec):
    kp["idx"][rows] = torch.from_numpy(rec["idx"]).to(DEV)
    kp["norm"][rows] = torch.from_numpy(np.ascontiguousarray(rec["norm"]).view(np.float16)).to(DEV)
    if "signs" in kp:
        kp["signs"][rows] = torch.from_numpy(rec["signs"]).to(DEV)
        kp["rnorm"][rows] = torch.from_numpy(np.ascontiguousarray(rec["rnorm"]).view(np.float16)).to(DEV)
    for k in ("codes", "scale", "zero"):
        vp[k][rows] = torch.from_numpy(vrec[k]).to(DEV)


def _full_decode_case(kw, v_bits, B, Hkv, Hq, ctx, keys, vals, q, q_vals, samples, label):
    """keys/vals: [B*Hkv*ctx, D] bf16 device tensors; q: [B, Hq, D] bf16.
    Returns GPU scores of the GPU-encoded cache (for quality metrics) and the
    oracle's scores of the sampled groups ({(b, h): [G, ctx]})."""
    seed = 42
    Tg = tq.Tables(L.key_config(seed=seed, **kw), DEV)
    To = O.build_tables(O.KeyConfig(d=D, seed=seed, mode=kw["mode"], bits=kw.get("bits", 3),
                                    bits_outlier=kw.get("bits_outlier", 4),
                                    bits_normal=kw.get("bits_normal", 2)))
    n = B * Hkv * ctx
    kp = tq.encode_keys(Tg, keys)
    vp = tq.encode_values(vals, v_bits)
    ctx_t = torch.full((B,), ctx, dtype=torch.int32, device=DEV)
    dec = tq.Decoder(Tg, B, Hq, Hkv, ctx, v_bits, q.dtype, DEV)
    out_e2e = dec(q, ctx_t, kp, vp)
    scores_e2e = torch.empty((B, Hq, ctx), dtype=torch.float32, device=DEV)
    dec(q, ctx_t, kp, vp, scores=scores_e2e)
    torch.cuda.synchronize()
    out_e2e = _np(out_e2e)
    G = Hq // Hkv
    refs = {}
    for (b, h) in samples:
        g = b * Hkv + h
        rows = slice(g * ctx, (g + 1) * ctx)
        kv = _bf16_rows(keys, rows).astype(np.float64)
        vv = _bf16_rows(vals, rows)
        rep = {}
        enc = P.check_keys(kv, To, _gpu_fields(To, kp, rows), rep)          # encode parity
        venc = P.check_values(vv, v_bits, _np(vp["codes"][rows]), _np(vp["scale"][rows]),
                              _np(vp["zero"][rows]))
        khat, vhat = O.dequant_keys(enc, To), O.dequant_values(venc)
        heads = slice(h * G, (h + 1) * G)
        s_ref, o_ref, lse_ref = O.decode_attention(q_vals[b, heads].astype(np.float64), khat, vhat, ctx)
        P.check_out(out_e2e[b, heads], o_ref)                               # end to end
        refs[(b, h)] = (s_ref, o_ref, lse_ref)
        _overwrite(kp, vp, rows, O.pack_key_record(enc, To), O.pack_value_record(venc, v_bits))
        print("%s group (%d,%d): band cases %s" % (label, b, h, rep), flush=True)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    scores = torch.full((B, Hq, ctx), float("nan"), dtype=torch.float32, device=DEV)
    out = dec(q, ctx_t, kp, vp, lse=lse, scores=scores)
    torch.cuda.synchronize()
    out, lse = _np(out), _np(lse)
    worst = 0.0
    for (b, h), (s_ref, o_ref, lse_ref) in refs.items():
        heads = slice(h * G, (h + 1) * G)
        worst = max(worst, P.check_scores(_np(scores[b, heads]), s_ref))
        P.check_out(out[b, heads], o_ref)
        assert np.all(np.abs(lse[b, heads] - lse_ref) <= 5e-3 * np.maximum(1.0, np.abs(lse_ref)))
    print("%s: worst relative score error %.3g over %d sampled groups" % (label, worst, len(refs)), flush=True)
    del kp, vp
    return scores_e2e, {k: v[0] for k, v in refs.items()}


def test_gqa_decode_32k_full_size():
    """16 sequences x 8 KV heads x 32 query heads, context 32768, prod 3-bit
    keys, 2-bit values, bf16: the benchmark's inputs and launch."""
    B, Hkv, Hq, ctx = 16, 8, 32, 32768
    n = B * Hkv * ctx
    keys = W.normal_bf16_device(3, 1, (n, D), DEV)
    vals = W.normal_bf16_device(3, 2, (n, D), DEV)
    q = W.normal_bf16_device(3, 3, (1, B, Hq, D), DEV)[0].contiguous()
    _full_decode_case(dict(mode="prod", bits=3), 2, B, Hkv, Hq, ctx, keys, vals, q, _np(q.float()),
                      [(0, 0), (2, 5), (6, 3), (9, 1), (11, 6), (15, 7)], "gqa-decode-32k")


def test_gqa_decode_32k_append_step_full_size():
    """The benchmark's step at full size: one tq_decode_attention_append call
    over 16 x 8 KV heads x 32 query heads at context 32768 that appends token
    32767 of every (sequence, KV head).  All 128 appended records against the
    oracle's encoding of the new rows; on sampled groups, the scores (the new
    token's included), outputs and lse against the oracle's attention over the
    dequantised records the planes hold after the call."""
    B, Hkv, Hq, ctx = 16, 8, 32, 32768
    G = Hq // Hkv
    n = B * Hkv * ctx
    keys = W.normal_bf16_device(3, 1, (n, D), DEV)
    vals = W.normal_bf16_device(3, 2, (n, D), DEV)
    k_new = W.normal_bf16_device(3, 6, (1, B * Hkv, D), DEV)[0].contiguous()
    v_new = W.normal_bf16_device(3, 7, (1, B * Hkv, D), DEV)[0].contiguous()
    q = W.normal_bf16_device(3, 3, (1, B, Hq, D), DEV)[0].contiguous()
    kw = dict(mode="prod", bits=3)
    Tg = tq.Tables(L.key_config(seed=42, **kw), DEV)
    To = O.build_tables(O.KeyConfig(d=D, seed=42, mode="prod", bits=3))
    kp = tq.encode_keys(Tg, keys)
    vp = tq.encode_values(vals, 2)
    del keys, vals
    ctx_t = torch.full((B,), ctx, dtype=torch.int32, device=DEV)
    dec = tq.Decoder(Tg, B, Hq, Hkv, ctx, 2, q.dtype, DEV)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    scores = torch.full((B, Hq, ctx), float("nan"), dtype=torch.float32, device=DEV)
    out = dec(q, ctx_t, kp, vp, lse=lse, scores=scores, k_new=k_new.view(B, Hkv, D), v_new=v_new.view(B, Hkv, D))
    torch.cuda.synchronize()
    out, lse = _np(out), _np(lse)
    rows = np.arange(B * Hkv) * ctx + ctx - 1
    rep = {}
    P.check_keys(k_new.float().cpu().numpy().astype(np.float64), To, _gpu_fields(To, kp, rows), rep)
    P.check_values(v_new.float().cpu().numpy(), 2, _np(vp["codes"][rows]), _np(vp["scale"][rows]),
                   _np(vp["zero"][rows]))
    print("appended records: band cases %s" % rep, flush=True)
    qv = _np(q.float())
    worst = 0.0
    for (b, h) in [(0, 0), (7, 4), (15, 7)]:
        g = b * Hkv + h
        sl = slice(g * ctx, (g + 1) * ctx)
        khat = O.dequant_keys(_gpu_fields(To, kp, sl), To)
        vc = _np(vp["codes"][sl])
        venc = dict(codes=O.unpack_fields(vc, O.index_width(2), D), scale16=_np(vp["scale"][sl]).view(np.float16),
                    zero16=_np(vp["zero"][sl]).view(np.float16))
        vhat = O.dequant_values(venc)
        heads = slice(h * G, (h + 1) * G)
        s_ref, o_ref, lse_ref = O.decode_attention(qv[b, heads].astype(np.float64), khat, vhat, ctx)
        worst = max(worst, P.check_scores(_np(scores[b, heads]), s_ref))
        P.check_out(out[b, heads], o_ref)
        assert np.all(np.abs(lse[b, heads] - lse_ref) <= 5e-3 * np.maximum(1.0, np.abs(lse_ref)))
    print("gqa-decode-32k append step: worst relative score error %.3g" % worst, flush=True)


def test_needle_decode_128k_full_size():
    """1 sequence x 8 KV heads x 32 query heads, context 131072, prod 4-bit
    keys (3-bit index in nibbles + QJL), 4-bit values, five planted needles
    per KV head; parity on sampled heads, plus top-5 recall of the GPU scores
    against exact float32 attention scores over the original keys."""
    B, Hkv, Hq, ctx = 1, 8, 32, 131072
    G = Hq // Hkv
    n = B * Hkv * ctx
    kv, kb = W.kv_rows(4, W.T_KEYS, n)
    qv, qb = W.queries(4, B, Hq)
    nv, nb = W.w4_needles(qv, Hkv, Hq)
    pos = W.needle_positions(ctx)
    for h in range(Hkv):
        for i, p in enumerate(pos):
            kv[h * ctx + p] = nv[h, i]
            kb[h * ctx + p] = nb[h, i]
    _, vb = W.kv_rows(4, W.T_VALUES, n)
    keys = torch.from_numpy(kb.view(np.int16)).view(torch.bfloat16).to(DEV)
    vals = torch.from_numpy(vb.view(np.int16)).view(torch.bfloat16).to(DEV)
    q = torch.from_numpy(qb.view(np.int16)).view(torch.bfloat16).to(DEV)
    scores, oracle_scores = _full_decode_case(dict(mode="prod", bits=4), 4, B, Hkv, Hq, ctx, keys, vals, q, qv,
                                              [(0, 0), (0, 3), (0, 5), (0, 7)], "needle-decode-128k")
    s_gpu = _np(scores)[0]
    recalls, ranks = [], []
    for hq in range(Hq):
        h = hq // G
        exact = kv[h * ctx:(h + 1) * ctx] @ qv[0, hq]            # float32 exact q.k
        top_exact = set(np.argsort(-exact, kind="stable")[:5].tolist())
        top_gpu = set(np.argsort(-s_gpu[hq], kind="stable")[:5].tolist())
        recalls.append(len(top_exact & top_gpu) / 5.0)
        if hq % G == 0:   # the query head the needles point at
            order = np.argsort(-s_gpu[hq], kind="stable")
            rank = np.empty(ctx, dtype=np.int64)
            rank[order] = np.arange(ctx)
            ranks.append([int(rank[p]) for p in pos])
    recall = float(np.mean(recalls))
    print("needle-decode-128k: top-5 recall vs exact fp32 %.3f; needle ranks per KV head %s" % (recall, ranks),
          flush=True)
    # Head by head on the sampled KV heads: the GPU's recall equals the
    # oracle's (the same estimator on the CPU, from its own encode of these
    # keys), except where the oracle's 5th and 6th scores are within 2 % of
    # their RMS, where either may make the top 5 (then they may differ by one).
    compared = 0
    for (b, h), s_or in oracle_scores.items():
        for i in range(G):
            hq = h * G + i
            exact = kv[h * ctx:(h + 1) * ctx] @ qv[0, hq]
            te = set(np.argsort(-exact, kind="stable")[:5].tolist())
            to = np.argsort(-s_or[i], kind="stable")
            r_or = len(te & set(to[:5].tolist())) / 5.0
            srt = s_or[i][to[:6]]
            tied = srt[4] - srt[5] < 2e-2 * math.sqrt(float(np.mean(s_or[i] ** 2)))
            assert abs(recalls[hq] - r_or) <= (0.2 if tied else 1e-9), (hq, recalls[hq], r_or)
            compared += 1
    assert compared == len(oracle_scores) * G
    # and the needles themselves stay at the top (the pages' needle retrieval)
    assert max(max(r) for r in ranks) < ctx // 1000, ranks


def test_outlier_grouped_16k_full_size():
    """8 sequences x 8 KV heads x 32 query heads, context 16384; key channels
    0..63 ~ N(0, 10^2) and 64..127 ~ N(0, 1); grouped keys (4-bit outlier
    half, 2-bit normal half), 4-bit values: encode + one decode step."""
    B, Hkv, Hq, ctx = 8, 8, 32, 16384
    n = B * Hkv * ctx
    keys = W.normal_bf16_device(5, 1, (n, D), DEV, scale_cols=W.w5_col_scale())
    vals = W.normal_bf16_device(5, 2, (n, D), DEV)
    q = W.normal_bf16_device(5, 3, (1, B, Hq, D), DEV)[0].contiguous()
    _full_decode_case(dict(mode="grouped", bits_outlier=4, bits_normal=2), 4, B, Hkv, Hq, ctx, keys, vals, q,
                      _np(q.float()), [(0, 0), (1, 2), (3, 6), (5, 4), (7, 7)], "outlier-grouped-16k")


@pytest.mark.parametrize("bits", [4, 8])
def test_mse_prefill_encode_full_size(bits):
    """28 layers x 2 KV heads x 32768 bf16 keys (norms log-uniform in [2, 20]),
    MSE mode at 4 and 8 bits, one seed per layer: all layers are encoded in
    one batched launch (as the benchmark times them); sampled rows of five
    layers are checked against the oracle."""
    n_layer = 2 * 32768
    rng = np.random.default_rng(2024)
    xs = [W.w2_layer_keys_device(layer, DEV) for layer in range(28)]
    tabs = [tq.Tables(L.key_config(mode="mse", bits=bits, seed=42 + layer), DEV) for layer in range(28)]
    kps = tq.encode_keys_batched(tabs, xs)
    torch.cuda.synchronize()
    for layer in (0, 6, 13, 20, 27):
        x, kp = xs[layer], kps[layer]
        To = O.build_tables(O.KeyConfig(d=D, mode="mse", bits=bits, seed=42 + layer))
        rows = np.concatenate([np.arange(1024), n_layer - 1024 + np.arange(1024),
                               rng.choice(n_layer, 2048, replace=False)])
        rows_t = torch.from_numpy(rows).to(DEV)
        kx = x[rows_t].float().cpu().numpy().astype(np.float64)
        rep = {}
        P.check_keys(kx, To, _gpu_fields(To, kp, rows_t), rep)
        assert math.isfinite(float(_np(kp["norm"].float()).max()))
        print("mse%d layer %d: band cases %s" % (bits, layer, rep), flush=True)
