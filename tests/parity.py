"""Comparison rules between the HIP path and the CPU oracle (test
infrastructure; imports the oracle).

Bytes: index and sign bytes equal the oracle's, except coordinates whose
oracle float64 value lies within 1e-6 of a decision boundary (index) or of
zero (sign), measured in the unit-norm domain (the sketch of the unit key's
residual, z / sqrt(d) for prod and z / ||k|| for grouped_prod); those are counted and must be
at most 1e-4 of all coordinates.  A key whose index legitimately differs at a
boundary gets its sign bits and residual norm checked against the oracle's
QJL stage rerun with the GPU's indices (both choices are correct there).
Norms: fp16 within one ulp.  Value codes, scales and zeros: exact (both sides
decide them with the same float32 operations).
Scores: |s - s_ref| <= 2e-3 * max(|s_ref|, rms(s_ref)); outputs 1e-2 absolute.
"""
from __future__ import annotations

import math

import numpy as np

import oracle.tq_oracle as O

BAND = 1e-6
BAND_FRACTION = 1e-4
SCORE_RTOL = 2e-3
OUT_ATOL = 1e-2


def fp16_ulps(a16, b16) -> np.ndarray:
    """Distance in ulps between fp16 arrays (same sign assumed for nonzero)."""
    a = np.asarray(a16, dtype=np.float16).view(np.uint16).astype(np.int64)
    b = np.asarray(b16, dtype=np.float16).view(np.uint16).astype(np.int64)
    # map sign-magnitude to a monotone integer line
    a = np.where(a & 0x8000, -(a & 0x7FFF), a)
    b = np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(a - b)


def _boundary_distance(y, boundaries):
    return np.min(np.abs(y[..., None] - boundaries[None, None, :]), axis=-1)


def check_keys(rows_keys, T, gpu: dict, report: dict | None = None):
    """rows_keys: [n, d] float64 inputs; gpu: unpacked planes for those rows
    (idx [n, d] int, norm16, and for the QJL modes bits [n, m], rnorm16)."""
    cfg = T.cfg
    d = cfg.d
    enc = O.encode_keys(rows_keys, T)
    n = rows_keys.shape[0]
    stats = dict(n=n, idx_band=0, sign_band=0)
    # ---- indices
    qjl = cfg.mode in ("prod", "grouped_prod")
    if cfg.mode in ("grouped", "grouped_prod"):
        h = d // 2
        dist = np.concatenate([_boundary_distance(enc["y"][:, :h], T.halves[0]["boundaries"]),
                               _boundary_distance(enc["y"][:, h:], T.halves[1]["boundaries"])], axis=1)
        dist = dist / math.sqrt(h)
    else:
        dist = _boundary_distance(enc["y"], T.boundaries) / math.sqrt(d)
    diff = gpu["idx"] != enc["idx"]
    bad = diff & (dist >= BAND)
    assert not bad.any(), "index mismatch outside the band at %s" % (np.argwhere(bad)[:5].tolist(),)
    stats["idx_band"] = int(diff.sum())
    # ---- norms
    ul = fp16_ulps(gpu["norm16"], enc["norm16"])
    assert ul.max(initial=0) <= 1, "norm differs by %d ulp" % ul.max()
    if qjl:
        keys_diff = diff.any(axis=1)
        z = enc["z"].copy()
        ref_bits = enc["bits"].copy()
        ref_rn = enc["rnorm16"].copy()
        if keys_diff.any():
            stage = O.prod_given_idx if cfg.mode == "prod" else O.grouped_prod_given_idx
            re = stage(enc["norm"][keys_diff], enc["y"][keys_diff], gpu["idx"][keys_diff], T)
            z[keys_diff] = re["z"]
            ref_bits[keys_diff] = re["bits"]
            ref_rn[keys_diff] = re["rnorm16"]
        if cfg.mode == "prod":
            zu = np.abs(z) / math.sqrt(d)
        else:
            kn = np.sqrt(np.sum(enc["norm"] ** 2, axis=1))
            zu = np.abs(z) / np.where(kn > 0, kn, 1.0)[:, None]
        sdiff = gpu["bits"] != ref_bits
        sbad = sdiff & (zu >= BAND)
        assert not sbad.any(), "sign mismatch outside the band at %s (|z|=%s)" % (
            np.argwhere(sbad)[:5].tolist(), np.abs(z[sbad])[:5])
        stats["sign_band"] = int(sdiff.sum())
        rul = fp16_ulps(gpu["rnorm16"], ref_rn)
        assert rul.max(initial=0) <= 1, "rnorm differs by %d ulp" % rul.max()
    total = n * d * (2 if qjl else 1)
    assert stats["idx_band"] + stats["sign_band"] <= max(1, BAND_FRACTION * total), stats
    if report is not None:
        report.update(stats)
    return enc


def unpack_gpu_keys(T, planes: dict) -> dict:
    """GPU planes (numpy) -> fields comparable with the oracle's."""
    rec = dict(idx=planes["idx"], norm=planes["norm"].view(np.float16))
    qjl = T.cfg.mode in ("prod", "grouped_prod")
    if qjl:
        rec["signs"] = planes["signs"]
        rec["rnorm"] = planes["rnorm"].view(np.float16)
    u = O.unpack_key_record(rec, T)
    out = dict(idx=u["idx"], norm16=u["norm16"])
    if qjl:
        out["bits"] = u["bits"]
        out["rnorm16"] = u["rnorm16"]
    return out


def check_values(values, bits, gpu_codes, gpu_scale, gpu_zero):
    enc = O.encode_values(values, bits)
    rec = O.pack_value_record(enc, bits)
    assert np.array_equal(gpu_codes, rec["codes"]), "value codes differ at %s" % (
        np.argwhere(gpu_codes != rec["codes"])[:5].tolist(),)
    assert np.array_equal(gpu_scale.view(np.uint16), rec["scale"].view(np.uint16))
    assert np.array_equal(gpu_zero.view(np.uint16), rec["zero"].view(np.uint16))
    return enc


def check_scores(s_gpu, s_ref):
    s_ref = np.asarray(s_ref, dtype=np.float64)
    rms = math.sqrt(float(np.mean(s_ref ** 2))) if s_ref.size else 0.0
    tol = SCORE_RTOL * np.maximum(np.abs(s_ref), rms)
    err = np.abs(np.asarray(s_gpu, dtype=np.float64) - s_ref)
    assert np.all(err <= tol), "score error %.3g > tol (worst at %s)" % (
        float(np.max(err - tol)), np.unravel_index(np.argmax(err - tol), err.shape))
    return float(np.max(err / np.maximum(np.abs(s_ref), rms))) if s_ref.size else 0.0


def check_out(o_gpu, o_ref):
    err = np.abs(np.asarray(o_gpu, dtype=np.float64) - o_ref)
    assert np.all(err <= OUT_ATOL), "output error %.3g" % float(err.max())
    return float(err.max(initial=0))
