"""Planted mistakes in the oracle (on the CPU, through monkeypatching) must
each be caught by at least one pin in test_oracle_pins."""
import math

import numpy as np
import pytest

import oracle.tq_oracle as O
import tests.test_oracle_pins as P


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def test_wrong_qjl_constant_is_caught(monkeypatch):
    orig = O.dequant_keys

    def mutant(enc, T):
        e = dict(enc)
        if "rnorm16" in e:
            e["rnorm16"] = (e["rnorm16"].astype(np.float64) * 1.1).astype(np.float16)
        return orig(e, T)
    monkeypatch.setattr(O, "dequant_keys", mutant)
    assert _fails(P.test_prod_unbiased_over_S_draws)


def test_transposed_rotation_is_caught(monkeypatch):
    orig = O.rotation_matrix
    calls = {"n": 0}

    def mutant(sigma):
        return orig(sigma).T
    monkeypatch.setattr(O, "rotation_matrix", mutant)
    assert _fails(P.test_key_built_from_centroids)


def test_ties_going_down_is_caught(monkeypatch):
    monkeypatch.setattr(O, "bucketize",
                        lambda y, t: np.sum(y[..., None] > t, axis=-1).astype(np.int64))
    assert _fails(P.test_bucketize_ties_go_up)


def test_msb_first_packing_is_caught(monkeypatch):
    orig = O.pack_fields

    def mutant(codes, width):
        per = 8 // width
        c = np.asarray(codes).reshape(codes.shape[0], -1, per)[:, :, ::-1].reshape(codes.shape)
        return orig(c, width)
    monkeypatch.setattr(O, "pack_fields", mutant)
    assert _fails(P.test_pack_golden_examples)


def test_dropped_sign_flip_sigma_is_caught(monkeypatch):
    """Rotating without the random signs still gives an orthogonal Pi; the
    all-plus reduction check catches a sigma applied on the wrong side."""
    orig = O.rotation_matrix
    monkeypatch.setattr(O, "rotation_matrix",
                        lambda sigma: sigma[:, None] * O.hadamard(sigma.shape[0]) / math.sqrt(sigma.shape[0]))
    assert _fails(P.test_key_built_from_centroids)


def test_value_rounding_half_up_is_caught(monkeypatch):
    """Rounding exact ties up instead of to even."""
    orig = O.encode_values

    def mutant(values, bits, group=32):
        e = orig(values, bits, group)
        code = np.clip(np.floor(e["ratio"] + 0.5), 0, (1 << bits) - 1)
        s16 = np.repeat(e["scale16"], group, axis=-1).reshape(code.shape)
        e["codes"] = np.where(s16 == 0, 0, code).astype(np.int64)
        return e
    monkeypatch.setattr(O, "encode_values", mutant)
    assert _fails(P.test_value_rounding_ties_to_even, 2)
    assert _fails(P.test_value_rounding_ties_to_even, 4)


def test_value_rounding_truncation_is_caught(monkeypatch):
    orig = O.encode_values

    def mutant(values, bits, group=32):
        e = orig(values, bits, group)
        e["codes"] = np.clip(np.floor(e["ratio"]), 0, (1 << bits) - 1).astype(np.int64)
        return e
    monkeypatch.setattr(O, "encode_values", mutant)
    assert _fails(P.test_value_quantisation_error_bound, 2)
    assert _fails(P.test_value_rounding_ties_to_even, 2)


def test_uncentred_spearman_is_caught(monkeypatch):
    def mutant(a, b):
        ra = np.argsort(np.argsort(a)).astype(np.float64)
        rb = np.argsort(np.argsort(b)).astype(np.float64)
        return float((ra * rb).sum() / math.sqrt((ra * ra).sum() * (rb * rb).sum()))
    monkeypatch.setattr(O, "spearman", mutant)
    assert _fails(P.test_spearman_matches_scipy)


def test_recall_of_bottom_k_is_caught(monkeypatch):
    def mutant(true_scores, est_scores, k):
        t = np.argsort(true_scores, axis=-1, kind="stable")[:, :k]
        e = np.argsort(est_scores, axis=-1, kind="stable")[:, :k]
        return float(np.mean([len(set(a) & set(b)) / k for a, b in zip(t, e)]))
    monkeypatch.setattr(O, "recall_at_k", mutant)
    assert _fails(P.test_recall_at_k_worked_example)


def test_grouped_shared_norm_is_caught(monkeypatch):
    """Normalising both halves by the whole key's norm."""
    orig = O._rotate_unit
    state = {}

    def mutant(keys, sigma):
        k = np.asarray(keys, dtype=np.float64)
        if k.shape[-1] == 64 and "full" in state:
            n = state["full"]
            u = k / np.where(n > 0, n, 1.0)[..., None]
            return n, u @ O.rotation_matrix(sigma).T * 8.0
        return orig(keys, sigma)
    enc_orig = O.encode_keys

    def enc_mutant(keys, T):
        state["full"] = np.sqrt(np.sum(np.asarray(keys, dtype=np.float64) ** 2, axis=-1))
        try:
            return enc_orig(keys, T)
        finally:
            state.pop("full", None)
    monkeypatch.setattr(O, "_rotate_unit", mutant)
    monkeypatch.setattr(O, "encode_keys", enc_mutant)
    assert _fails(P.test_grouped_key_built_from_centroids)


def test_grouped_swapped_rotations_are_caught(monkeypatch):
    """Encoding each half with the other half's random signs."""
    enc_orig = O.encode_keys

    def enc_mutant(keys, T):
        if T.cfg.mode == "grouped":
            T2 = O.KeyTables()
            T2.cfg = T.cfg
            T2.halves = [dict(h) for h in T.halves]
            T2.halves[0]["sigma"], T2.halves[1]["sigma"] = T.halves[1]["sigma"], T.halves[0]["sigma"]
            return enc_orig(keys, T2)
        return enc_orig(keys, T)
    monkeypatch.setattr(O, "encode_keys", enc_mutant)
    assert _fails(P.test_grouped_key_built_from_centroids)


def _grouped_prod_mutant(weight=True, rotate=True):
    """grouped_prod_given_idx with the norm weights dropped or the residual
    sketched in the original domain instead of the block-rotated frame."""
    def fn(norms, y, idx, T):
        d, h = T.cfg.d, T.cfg.d // 2
        parts = []
        for j, half in enumerate(T.halves):
            sl = slice(j * h, (j + 1) * h)
            r = y[:, sl] - half["centroids"][idx[:, sl]]
            r = r * (norms[:, j:j + 1] if weight else 1.0) / math.sqrt(h)
            parts.append(r if rotate else r @ O.rotation_matrix(half["sigma"]))
        w = np.concatenate(parts, axis=1)
        z = w @ T.S.T
        rho = np.sqrt(np.sum(w * w, axis=-1))
        return dict(w=w, z=z, bits=(z >= 0).astype(np.uint8), rnorm=rho, rnorm16=O.fp16_round(rho))
    return fn


def test_grouped_prod_unweighted_halves_are_caught(monkeypatch):
    monkeypatch.setattr(O, "grouped_prod_given_idx", _grouped_prod_mutant(weight=False))
    assert _fails(P.test_grouped_prod_sketch_is_the_block_rotated_residual)


def test_grouped_prod_unrotated_residual_is_caught(monkeypatch):
    monkeypatch.setattr(O, "grouped_prod_given_idx", _grouped_prod_mutant(rotate=False))
    assert _fails(P.test_grouped_prod_sketch_is_the_block_rotated_residual)


def test_grouped_prod_wrong_qjl_constant_is_caught(monkeypatch):
    orig = O.dequant_keys

    def mutant(enc, T):
        e = dict(enc)
        if "rnorm16" in e:
            e["rnorm16"] = (e["rnorm16"].astype(np.float64) * 1.15).astype(np.float16)
        return orig(e, T)
    monkeypatch.setattr(O, "dequant_keys", mutant)
    assert _fails(P.test_grouped_prod_bias_regression_slope_is_zero)


def test_outlier_ties_to_higher_channel_are_caught(monkeypatch):
    def mutant(keys, n_outlier):
        k = np.asarray(keys, dtype=np.float64)
        var = k.var(axis=0)
        ranked = sorted(range(k.shape[1]), key=lambda c: (-var[c], -c))
        return np.array(sorted(ranked[:n_outlier]) + sorted(ranked[n_outlier:]))
    monkeypatch.setattr(O, "select_outlier_channels", mutant)
    assert _fails(P.test_select_outlier_channels_worked_example)


def test_outlier_by_mean_square_is_caught(monkeypatch):
    """Ranking by the uncentred second moment instead of the variance."""
    def mutant(keys, n_outlier):
        k = np.asarray(keys, dtype=np.float64)
        ms = (k * k).mean(axis=0)
        ranked = sorted(range(k.shape[1]), key=lambda c: (-ms[c], c))
        return np.array(sorted(ranked[:n_outlier]) + sorted(ranked[n_outlier:]))
    monkeypatch.setattr(O, "select_outlier_channels", mutant)
    assert _fails(P.test_select_outlier_channels_worked_example)


def test_reversed_kl_is_caught(monkeypatch):
    orig = O.attention_quality

    def mutant(q, k, v, khat, vhat, sm_scale=None, topk=5):
        r = orig(q, khat, vhat, k, v, sm_scale, topk)     # KL(p_hat || p), cosines symmetric
        return r
    monkeypatch.setattr(O, "attention_quality", mutant)
    assert _fails(P.test_attention_quality_against_scipy)


def test_output_cosine_with_exact_weights_is_caught(monkeypatch):
    orig = O.attention_quality

    def mutant(q, k, v, khat, vhat, sm_scale=None, topk=5):
        r = orig(q, k, v, khat, vhat, sm_scale, topk)
        r2 = orig(q, k, v, k, vhat, sm_scale, topk)       # p v against p v_hat
        r["out_cosine"] = r2["out_cosine"]
        return r
    monkeypatch.setattr(O, "attention_quality", mutant)
    assert _fails(P.test_attention_quality_against_scipy)
