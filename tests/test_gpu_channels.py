"""Outlier-channel selection for GROUPED mode on the GPU.

The selection equals the oracle's variance ranking.  Keys whose 64
high-variance channels sit at scattered positions: the per-channel moments
match float64 sums on the host, the selection recovers exactly the planted
channels, and grouped encode + decode on the reordered
keys and queries (a common channel permutation leaves q.k unchanged) agrees
with the oracle and beats the fixed split that ignores the variances."""
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


def _planted(n=8192):
    rng = np.random.default_rng(51)
    outl = np.sort(rng.choice(128, 64, replace=False))
    scale = np.ones(128, dtype=np.float32)
    scale[outl] = 10.0
    kv, kb = W.kv_rows(51, 1, n, scale_cols=scale)
    return outl, kv, torch.from_numpy(kb.view(np.int16)).view(torch.bfloat16).to(DEV)


def test_channel_moments_match_float64_sums():
    _, kv, x = _planted(5000)   # ragged: 4 full 1024-row blocks and a partial one
    m = tq.channel_moments(x).cpu().numpy()
    k = kv.astype(np.float64)
    assert np.allclose(m[0], k.sum(0), rtol=0, atol=1e-12 * np.abs(k).sum(0).max())
    assert np.allclose(m[1], (k * k).sum(0), rtol=1e-12, atol=0)


def test_selection_matches_oracle():
    """tq_select_outlier_channels against the oracle's variance ranking,
    element for element: channel scales spread over two decades (ranks are
    far apart at this sample size), a copy of a channel (an exact tie: the
    lower channel wins on both sides), a constant channel, a ragged row count,
    and the degenerate splits 0 and 128 and an empty key set (identity)."""
    rng = np.random.default_rng(52)
    n = 3001
    scale = np.exp(rng.uniform(np.log(0.1), np.log(10.0), 128)).astype(np.float32)
    kv, kb = W.kv_rows(52, 1, n, scale_cols=scale)
    kv = kv.copy()
    kv[:, 90] = kv[:, 17]                         # exact tie with channel 17
    kv[:, 5] = 2.5                                # constant channel: variance 0
    kv, kb = W.to_bf16(kv)                        # (both edits are bf16 values already)
    x = torch.from_numpy(kb.view(np.int16)).view(torch.bfloat16).to(DEV)
    for n_out in (64, 1, 0, 128, 37):
        got = tq.select_outlier_channels(x, n_out).cpu().numpy()
        want = O.select_outlier_channels(kv.astype(np.float64), n_out)
        assert np.array_equal(got, want), (n_out, got[:8], want[:8])
    empty = tq.select_outlier_channels(x[:0], 64).cpu().numpy()
    assert np.array_equal(empty, np.arange(128))


def test_selection_recovers_planted_channels_and_grouped_parity():
    outl, kv, x = _planted()
    perm = tq.select_outlier_channels(x, 64).cpu().numpy()
    rest = np.setdiff1d(np.arange(128), outl)
    assert np.array_equal(perm, np.concatenate([outl, rest]))
    # grouped keys on the reordered channels (the planted order, now verified)
    kw = dict(mode="grouped", bits_outlier=4, bits_normal=2)
    Tg = tq.Tables(L.key_config(seed=9, **kw), DEV)
    To = O.build_tables(O.KeyConfig(mode="grouped", seed=9, bits_outlier=4, bits_normal=2))
    n, Hq = kv.shape[0], 4
    pt = torch.from_numpy(perm).to(DEV)
    xp = x[:, pt].contiguous()
    kp = tq.encode_keys(Tg, xp)
    vv, vb = W.kv_rows(51, 2, n)
    vp = tq.encode_values(torch.from_numpy(vb.view(np.int16)).view(torch.bfloat16).to(DEV), 4)
    qv, qb = W.queries(51, 1, Hq)
    q = torch.from_numpy(qb.view(np.int16)).view(torch.bfloat16).to(DEV)
    qp = q[..., pt].contiguous()
    ctx = torch.tensor([n], dtype=torch.int32, device=DEV)
    out, _, scores = tq.decode_attention(Tg, qp, ctx, kp, vp, 4, n, with_scores=True)
    torch.cuda.synchronize()
    kperm = kv[:, perm].astype(np.float64)
    enc = P.check_keys(kperm, To, P.unpack_gpu_keys(To, {k: v.cpu().numpy() for k, v in kp.items()}))
    khat = O.dequant_keys(enc, To)
    vhat = O.dequant_values(O.encode_values(vv, 4))
    s_ref, o_ref, _ = O.decode_attention(qv[0][:, perm].astype(np.float64), khat, vhat, n)
    P.check_out(out.cpu().numpy()[0], o_ref)
    # scores on keys whose bytes match the oracle's (band cases aside)
    same = np.all(kp["idx"].cpu().numpy() == O.pack_key_record(enc, To)["idx"], axis=1)
    P.check_scores(scores.cpu().numpy()[0][:, same], s_ref[:, same])
    # selection beats the fixed split (channels 0..63 as the outlier half)
    exact = kv.astype(np.float64) @ qv[0].astype(np.float64).T            # [n, Hq]
    kp_fixed = tq.encode_keys(Tg, x)
    _, _, s_fixed = tq.decode_attention(Tg, q, ctx, kp_fixed, vp, 4, n, with_scores=True)
    err_sel = np.sqrt(np.mean((scores.cpu().numpy()[0].T - exact) ** 2))
    err_fix = np.sqrt(np.mean((s_fixed.cpu().numpy()[0].T - exact) ** 2))
    print("grouped score RMS error: selected %.4f, fixed split %.4f" % (err_sel, err_fix))
    assert err_sel < 0.8 * err_fix
