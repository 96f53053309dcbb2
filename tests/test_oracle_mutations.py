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
    orig = O.encode_values

    def mutant(values, bits, group=32):
        e = orig(values, bits, group)
        e["codes"] = np.clip(np.floor(e["ratio"] + 0.5), 0, (1 << bits) - 1).astype(np.int64) * 0 + \
            np.clip(np.floor(e["ratio"]), 0, (1 << bits) - 1).astype(np.int64)
        return e
    monkeypatch.setattr(O, "encode_values", mutant)
    assert _fails(P.test_value_quantisation_error_bound, 2)
