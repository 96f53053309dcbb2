"""Pins for the CPU oracle: each checks it against something other than itself
(printed values, closed forms, textbook tables, library routines, invariants,
exact expectations).  No GPU needed."""
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg
import scipy.stats
from scipy.integrate import quad

import oracle.tq_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- generator

def test_splitmix64_published_vector():
    g = _gold("lloyd_max_textbook.json")["splitmix64"]
    assert O.splitmix64_stream(g["seed"], 0, 5) == [int(x) for x in g["outputs"]]


def test_rademacher_signs_are_pm1_and_balanced():
    s = O.rademacher_signs(42, O.TAG_SIGMA, 8192)
    assert set(np.unique(s)) <= {-1.0, 1.0}
    assert abs(s.mean()) < 4.0 / math.sqrt(8192)
    # different tags give different streams
    assert not np.array_equal(O.rademacher_signs(42, 1, 128), O.rademacher_signs(42, 3, 128))


def test_gaussian_matrix_is_standard_normal():
    S = O.gaussian_matrix(42, O.TAG_S, 128, 128)
    x = S.ravel()
    assert np.all(x.astype(np.float16) == x)          # fp16 values
    assert scipy.stats.kstest(x, "norm").pvalue > 1e-3
    assert abs(x.mean()) < 4 / math.sqrt(x.size)
    assert abs(x.var() - 1) < 4 * math.sqrt(2 / x.size)
    # Box-Muller pairs are uncorrelated
    assert abs(np.corrcoef(x[0::2], x[1::2])[0, 1]) < 4 / math.sqrt(x.size / 2)


# ---------------------------------------------------------------- codebook

def test_codebook_two_levels_closed_form():
    c, t, D = O.lloyd_max_gaussian(2)
    assert np.allclose(c, [-math.sqrt(2 / math.pi), math.sqrt(2 / math.pi)], atol=1e-14)
    assert t[0] == 0.0
    assert abs(D - (1 - 2 / math.pi)) < 1e-14


@pytest.mark.parametrize("L", [4, 8])
def test_codebook_matches_max_1960(L):
    g = _gold("lloyd_max_textbook.json")["levels_%d" % L]
    c, t, D = O.lloyd_max_gaussian(L)
    assert np.allclose(c[L // 2:], g["centroids_pos"], atol=g["tol"])
    assert np.allclose(t[L // 2:], g["boundary_pos"], atol=g["tol"])
    assert abs(D - g["D"]) < g["tol"]


def test_codebook_16_levels_D():
    g = _gold("lloyd_max_textbook.json")["levels_16"]
    assert abs(O.lloyd_max_gaussian(16)[2] - g["D"]) < g["tol"]


def test_codebook_table1_band():
    g = _gold("lloyd_max_textbook.json")["table1_pages"]
    lo, hi = g["ratio_band"]
    for b, expected in g["values"].items():
        _, _, D = O.codebook(int(b))
        assert lo <= D / expected <= hi, (b, D)


@pytest.mark.parametrize("b", [1, 2, 3, 4, 5, 6, 7, 8])
def test_codebook_fixed_point_and_symmetry(b):
    """Lloyd-Max conditions checked by numerical integration (scipy.quad), an
    independent route from the erf-based update the solver iterates."""
    L = 1 << b
    c, t, D = O.lloyd_max_gaussian(L)
    assert np.array_equal(c, -c[::-1])
    assert np.all(np.diff(c) > 0)
    assert np.allclose(t, 0.5 * (c[:-1] + c[1:]), atol=1e-15, rtol=0)
    assert t[L // 2 - 1] == 0.0
    lo = np.concatenate(([-np.inf], t))
    hi = np.concatenate((t, [np.inf]))
    pdf = lambda x: math.exp(-0.5 * x * x) / math.sqrt(2 * math.pi)
    ks = range(L) if L <= 16 else list(range(0, L, 17)) + [L - 1]
    for k in ks:
        m0 = quad(pdf, lo[k], hi[k], epsabs=0, epsrel=1e-12)[0]
        m1 = quad(lambda x: x * pdf(x), lo[k], hi[k], epsabs=0, epsrel=1e-12)[0]
        assert abs(m1 / m0 - c[k]) < 1e-9 * max(1.0, abs(c[k])), (b, k)
    # D by the identity D = 1 - sum c_k^2 P_k at the fixed point
    P = np.array([quad(pdf, lo[k], hi[k], epsabs=0, epsrel=1e-12)[0] for k in range(L)])
    assert abs(D - (1 - np.sum(c * c * P))) < 1e-9


def test_codebook_b8_below_theorem1_bound():
    coef = _gold("lloyd_max_textbook.json")["theorem1_pages"]["coef"]
    for b in range(1, 9):
        _, _, D = O.codebook(b)
        assert D <= coef * 4.0 ** (-b)
    assert abs(O.codebook(8)[2] - 4.1185e-5) < 1e-8


def test_codebook_independent_of_start():
    """The fixed point does not depend on the start: plain Lloyd iteration from
    uniform quantiles reaches the same centroids (8 levels)."""
    from scipy.special import ndtri
    L = 8
    c = ndtri((np.arange(L) + 0.5) / L) * 1.7
    for _ in range(3000):
        c, _, _, _ = O._lloyd_map(c)
    ref, _, _ = O.lloyd_max_gaussian(L)
    assert np.allclose(c, ref, atol=1e-10)


# ---------------------------------------------------------------- rotation

@pytest.mark.parametrize("d", [2, 8, 64, 128])
def test_hadamard_is_sylvester(d):
    assert np.array_equal(O.hadamard(d), scipy.linalg.hadamard(d).astype(np.float64))


@pytest.mark.parametrize("d", [64, 128])
def test_rotation_orthogonal(d):
    Pi = O.rotation_matrix(O.rademacher_signs(7, O.TAG_SIGMA, d))
    assert np.abs(Pi @ Pi.T - np.eye(d)).max() < 1e-12
    # all-plus signs reduce to the normalised Hadamard matrix
    assert np.allclose(O.rotation_matrix(np.ones(d)), scipy.linalg.hadamard(d) / math.sqrt(d))


def test_rotated_unit_vector_has_norm_sqrt_d():
    T = O.build_tables(O.KeyConfig(mode="mse", bits=4))
    k = np.random.default_rng(0).standard_normal((10, 128)) * 7
    enc = O.encode_keys(k, T)
    assert np.allclose(np.linalg.norm(enc["y"], axis=1), math.sqrt(128), rtol=1e-12)
    assert np.allclose(enc["norm"], np.linalg.norm(k, axis=1), rtol=1e-14)


# ---------------------------------------------------------------- bucketize

@pytest.mark.parametrize("b", [1, 2, 3, 4, 8])
def test_bucketize_equals_nearest_centroid(b):
    c, t, _ = O.codebook(b)
    rng = np.random.default_rng(b)
    y = np.concatenate([rng.standard_normal(4000) * 1.5, t, np.nextafter(t, -np.inf),
                        np.nextafter(t, np.inf), [0.0, -0.0, 9.0, -9.0]])
    # The fp32 boundary and the midpoint of the fp32 centroids differ by up to
    # an ulp, and |y - c| rounds in float64: points within 1e-9 of a boundary
    # are left to test_bucketize_ties_go_up.
    idx = O.bucketize(y, t)
    nn = O.nearest_centroid(y, c)
    near = np.min(np.abs(y[:, None] - t[None, :]), axis=1) < 1e-9
    assert np.array_equal(idx[~near], nn[~near])
    assert near.sum() <= 3 * len(t) + 2
    if b == 1:
        assert np.array_equal(idx, (y >= 0).astype(np.int64))


def test_bucketize_ties_go_up():
    _, t, _ = O.codebook(2)
    assert np.array_equal(O.bucketize(t, t), np.arange(1, 4))


# ---------------------------------------------------------------- packing

def test_pack_golden_examples():
    g = _gold("pack_examples.json")
    for ex in g["two_bit"]:
        want = ex["bytes"] if "bytes" in ex else [ex["byte"]]
        got = O.pack_fields(np.array([ex["codes"]]), 2)[0]
        assert list(got) == want
    for ex in g["four_bit"] + g["three_bit_as_four"]:
        assert list(O.pack_fields(np.array([ex["codes"]]), 4)[0]) == [ex["byte"]]
    for ex in g["signs"]:
        bits = (np.array(ex["signs"]) > 0).astype(np.uint8)
        assert list(O.pack_signs(bits[None, :])[0]) == [ex["byte"]]


@pytest.mark.parametrize("w", [1, 2, 4, 8])
def test_pack_round_trip(w):
    rng = np.random.default_rng(w)
    codes = rng.integers(0, 1 << w, size=(37, 128))
    assert np.array_equal(O.unpack_fields(O.pack_fields(codes, w), w, 128), codes)
    bits = rng.integers(0, 2, size=(37, 128)).astype(np.uint8)
    assert np.array_equal(O.unpack_signs(O.pack_signs(bits), 128), bits)


def test_record_bytes():
    g = _gold("pack_examples.json")["record_bytes"]
    assert O.record_bytes(O.KeyConfig(mode="prod", bits=3)) == g["prod3_d128"]
    assert O.record_bytes(O.KeyConfig(mode="prod", bits=4)) == 84
    assert O.record_bytes(O.KeyConfig(mode="mse", bits=4)) == 66
    assert O.record_bytes(O.KeyConfig(mode="mse", bits=8)) == 130
    assert O.record_bytes(O.KeyConfig(mode="grouped", bits_outlier=4, bits_normal=2)) == 52
    # the grouped quantiser's 52 bytes plus m = 128 sign bits and one fp16 norm
    # ("tqlite" README mode table: the QJL stage adds d + 32 bits, the norm here fp16)
    assert O.record_bytes(O.KeyConfig(mode="grouped_prod", bits_outlier=4, bits_normal=2)) == 52 + 16 + 2


# ---------------------------------------------------------------- MSE encode

def _sphere_marginal_mse(b, d=128):
    """Exact E[(y - Q(y))^2] when y = sqrt(d) * (a coordinate of a uniform
    point on the unit sphere in R^d): density of x = y/sqrt(d) is
    proportional to (1 - x^2)^((d-3)/2) on [-1, 1]."""
    c, t, _ = O.codebook(b)
    lo = np.concatenate(([-math.sqrt(d)], t))
    hi = np.concatenate((t, [math.sqrt(d)]))
    logC = math.lgamma(d / 2) - math.lgamma((d - 1) / 2) - 0.5 * math.log(math.pi)
    f = lambda y: math.exp(logC + 0.5 * (d - 3) * math.log1p(-y * y / d)) / math.sqrt(d)
    tot = 0.0
    for k in range(len(c)):
        tot += quad(lambda y: (y - c[k]) ** 2 * f(y), lo[k], hi[k], epsabs=1e-13, epsrel=1e-11)[0]
    return tot


@pytest.mark.parametrize("b", [1, 2, 3, 4, 8])
def test_mse_distortion_theorem1_and_exact_expectation(b):
    coef = _gold("lloyd_max_textbook.json")["theorem1_pages"]["coef"]
    T = O.build_tables(O.KeyConfig(mode="mse", bits=b, seed=42))
    u = np.random.default_rng(100 + b).standard_normal((3000, 128))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    enc = O.encode_keys(u, T)
    uh = O.dequant_keys(enc, T)
    err = np.sum((u - uh) ** 2, axis=1)
    assert err.mean() <= coef * 4.0 ** (-b)
    exact = _sphere_marginal_mse(b)
    se = err.std() / math.sqrt(err.size)
    assert abs(err.mean() - exact) < 4 * se + 1e-6 * exact, (err.mean(), exact, se)
    # the sphere marginal is close to N(0,1): within 2% of D_b
    assert abs(exact / O.codebook(b)[2] - 1) < 0.02


def test_key_built_from_centroids():
    """k = Pi^T c[idx] / ||c[idx]|| (unit norm).  Then y = sqrt(d) Pi k =
    lam * c[idx] with lam = sqrt(d) / ||c[idx]|| (close to 1 for the chosen
    index mix), so: the indices come back, the MSE reconstruction is k / lam,
    and rho = ||k - k_mse|| = (lam - 1) / lam.  A transposed or unsigned
    rotation, or a wrong scale, breaks one of these."""
    T = O.build_tables(O.KeyConfig(mode="prod", bits=3, seed=5))
    rng = np.random.default_rng(1)
    rows = []
    for _ in range(3):
        inner = rng.permutation(np.r_[np.ones(79, int), np.zeros(49, int)])  # 79 small, 49 large levels
        sign = rng.integers(0, 2, 128)
        rows.append(np.where(sign == 1, 2 + (1 - inner), 1 - (1 - inner)))   # 2/3 positive, 1/0 negative
    idx = np.array(rows)
    c = T.centroids[idx]
    cn = np.linalg.norm(c, axis=1, keepdims=True)
    # Pi = H diag(sigma) / sqrt(d), written here from scipy's Hadamard matrix
    Pi = scipy.linalg.hadamard(128) * T.sigma[None, :] / math.sqrt(128)
    k = (c / cn) @ Pi
    lam = math.sqrt(128) / cn[:, 0]
    enc = O.encode_keys(k, T)
    assert np.array_equal(enc["idx"], idx)
    assert np.allclose(enc["rnorm"], np.abs(lam - 1) / lam, rtol=1e-9, atol=1e-15)
    mse_only = dict(enc)
    mse_only["rnorm16"] = np.zeros(3, dtype=np.float16)
    assert np.all(enc["norm16"] == 1.0)
    assert np.allclose(O.dequant_keys(mse_only, T), k / lam[:, None], atol=1e-12)


def test_zero_key_scores_zero():
    T = O.build_tables(O.KeyConfig(mode="prod", bits=3))
    enc = O.encode_keys(np.zeros((1, 128)), T)
    assert enc["norm16"][0] == 0 and enc["rnorm16"][0] == 0
    assert np.all(enc["idx"] == 2)                 # y = 0 sits on the middle boundary, goes up
    q = np.random.default_rng(0).standard_normal((2, 128))
    assert np.all(O.key_scores(q, enc, T) == 0)


# ---------------------------------------------------------------- QJL / prod

def _prod_setup(bits, seed=42):
    return O.build_tables(O.KeyConfig(mode="prod", bits=bits, seed=seed))


def test_prod_unbiased_over_S_draws():
    """For fixed unit keys, queries, Pi and indices, the mean of q.k_hat over
    independent Gaussian S is q.k (Theorem 2); the variance matches the
    closed form ((pi/2)||r||^2||a||^2 - <a,r>^2)/m of the sign estimator,
    a = Pi q scaled into the residual's units."""
    T = _prod_setup(3)
    rng = np.random.default_rng(2)
    k = rng.standard_normal((4, 128))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    q = rng.standard_normal((4, 128))
    base = O.encode_keys(k, T)
    Pi = O.rotation_matrix(T.sigma)
    true = np.sum(q * k, axis=1)
    ests = []
    draws = 3000
    g = np.random.default_rng(3)
    for _ in range(draws):
        T.S = g.standard_normal((128, 128)).astype(np.float16).astype(np.float64)
        enc = dict(base)
        enc.update(O.prod_given_idx(base["norm"], base["y"], base["idx"], T))
        ests.append(np.sum(q * O.dequant_keys(enc, T), axis=1))
    ests = np.array(ests)
    mean, sd = ests.mean(0), ests.std(0)
    assert np.all(np.abs(mean - true) < 4 * sd / math.sqrt(draws)), (mean, true)
    # variance of the estimate: only the QJL term varies
    r = base["y"] - T.centroids[base["idx"]]                   # rotated residual, sqrt(d) units
    a = (q @ Pi.T)                                             # Pi q
    rn = np.linalg.norm(r, axis=1)
    an = np.linalg.norm(a, axis=1)
    ar = np.sum(a * r, axis=1)
    # estimate of <a, r>/sqrt(d): rho/m sqrt(pi/2) <S a, sign(S r)>, rho = ||r||/sqrt(d)
    var_theory = ((math.pi / 2) * rn ** 2 * an ** 2 - ar ** 2) / 128 / 128
    assert np.all(np.abs(sd ** 2 / var_theory - 1) < 0.12), sd ** 2 / var_theory


def test_sign_estimator_with_fp16_entries():
    """S is stored in fp16 (each N(0,1) draw rounded to nearest even).  The
    sign estimator's constant sqrt(pi/2) holds exactly for Gaussian rows:
    E[sign(s.r)(s.a)] = sqrt(2/pi) <a,r>/||r|| (difai.kr tutorial, the QJL
    correction).  A paired experiment over 2^20 rows (the same Gaussian draw
    with and without the fp16 rounding) bounds how far the rounding moves that
    expectation: below 1e-4 of its value, against a sampling spread of about
    10% for one key's 128-row estimate.  The unrounded mean is also checked
    against the closed form."""
    rng = np.random.default_rng(31)
    d = 128
    r = rng.standard_normal(d)
    a = r / np.linalg.norm(r) + 0.8 * rng.standard_normal(d) / math.sqrt(d)
    a /= np.linalg.norm(a)
    exact = math.sqrt(2 / math.pi) * (a @ r) / np.linalg.norm(r)
    n, chunk = 1 << 20, 1 << 16
    diff_sum = diff_sq = e64_sum = e64_sq = 0.0
    for _ in range(n // chunk):
        S = rng.standard_normal((chunk, d))
        S16 = O.fp16_round(S).astype(np.float64)
        e64 = np.where(S @ r >= 0, 1.0, -1.0) * (S @ a)
        e16 = np.where(S16 @ r >= 0, 1.0, -1.0) * (S16 @ a)
        dd = e16 - e64
        diff_sum += dd.sum()
        diff_sq += (dd * dd).sum()
        e64_sum += e64.sum()
        e64_sq += (e64 * e64).sum()
    dm = diff_sum / n
    dse = math.sqrt(max(diff_sq / n - dm * dm, 0.0) / n)
    em = e64_sum / n
    ese = math.sqrt((e64_sq / n - em * em) / n)
    assert abs(em - exact) < 4 * ese, (em, exact, ese)
    assert (abs(dm) + 4 * dse) / exact < 1e-4, (dm, dse, exact)


def test_prod_bias_regression_slope_is_zero():
    """Regress (estimate - truth) on <q, k - k_mse_hat> over many pairs: a
    wrong QJL constant alpha shows as slope alpha - 1."""
    T = _prod_setup(3)
    rng = np.random.default_rng(4)
    k = rng.standard_normal((3000, 128))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    q = rng.standard_normal((3000, 128))
    enc = O.encode_keys(k, T)
    est = np.sum(q * O.dequant_keys(enc, T), axis=1)
    mse_only = dict(enc)
    mse_only["rnorm16"] = np.zeros_like(enc["rnorm16"])
    kmse = O.dequant_keys(mse_only, T)
    a = np.sum(q * (k - kmse), axis=1)
    e = est - np.sum(q * k, axis=1)
    slope = np.sum(e * a) / np.sum(a * a)
    resid = e - slope * a
    se = math.sqrt(np.sum(resid ** 2) / (len(a) - 1) / np.sum(a * a))
    assert abs(slope) < 4 * se + 0.02, (slope, se)
    # and the QJL term recovers most of the residual's projection
    qjl = est - np.sum(q * kmse, axis=1)
    assert np.corrcoef(qjl, a)[0, 1] > 0.5


def test_prod_distortion_theorem3_and_scaling():
    """D_prod = E[(<y,x_hat> - <y,x>)^2] <= sqrt(3) pi^2 ||y||^2 / d * 4^-b
    for unit x; each extra bit cuts it by more than 2x (about 4x)."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2000, 128))
    x /= np.linalg.norm(x, axis=1, keepdims=True)
    y = rng.standard_normal(128)
    D = {}
    for b in (2, 3, 4):
        T = _prod_setup(b)
        enc = O.encode_keys(x, T)
        est = O.dequant_keys(enc, T) @ y
        D[b] = float(np.mean((est - x @ y) ** 2))
        bound = math.sqrt(3) * math.pi ** 2 * (y @ y) / 128 * 4.0 ** (-b)
        assert D[b] <= bound, (b, D[b], bound)
    assert D[2] / D[3] > 2.0 and D[3] / D[4] > 2.0


def test_grouped_key_built_from_centroids():
    """Each half of the key is (n_j / lam_j) Pi_j^T c_j[idx_j] with its own
    64-point rotation and codebook ("tqlite" README mode table: outlier and
    normal channels quantised separately), written here from scipy's Hadamard
    matrix rather than through the MSE path.  The encoder must return both
    index halves, both norms and, dequantised, each half scaled by 1/lam_j.  A
    norm shared by the halves, swapped rotations or codebooks, or one
    128-point rotation over both halves breaks one of these."""
    cfg = O.KeyConfig(mode="grouped", bits_outlier=4, bits_normal=2, seed=17)
    T = O.build_tables(cfg)
    rng = np.random.default_rng(21)
    H64 = scipy.linalg.hadamard(64)
    rows, idxs, lams = [], [], []
    for n_out, n_norm in ((10.0, 1.0), (0.5, 3.0), (64.0, 0.25)):
        halves, ih, lh = [], [], []
        for half, n in zip(T.halves, (n_out, n_norm)):
            c_all, t = half["centroids"], half["boundaries"]
            L = len(c_all)
            while True:
                idx = rng.integers(0, L, 64)
                c = c_all[idx]
                lam = 8.0 / np.linalg.norm(c)             # sqrt(64) / ||c||
                y = lam * c                               # the rotated, sqrt(h)-scaled half
                if np.array_equal(np.sum(y[:, None] >= t[None, :], axis=1), idx) and \
                        np.min(np.abs(y[:, None] - t[None, :])) > 1e-3:
                    break
            Pi = H64 * half["sigma"][None, :] / 8.0
            halves.append(n * (c / np.linalg.norm(c)) @ Pi)
            ih.append(idx)
            lh.append(lam)
        rows.append(np.concatenate(halves))
        idxs.append(np.concatenate(ih))
        lams.append(lh)
    k = np.array(rows)
    enc = O.encode_keys(k, T)
    assert np.array_equal(enc["idx"], np.array(idxs))
    norms = np.array([[10.0, 1.0], [0.5, 3.0], [64.0, 0.25]])
    assert np.allclose(enc["norm"], norms, rtol=1e-12)
    assert np.array_equal(enc["norm16"].astype(np.float64), norms)   # exact in fp16
    kh = O.dequant_keys(enc, T)
    lam = np.array(lams)
    assert np.allclose(kh[:, :64], k[:, :64] / lam[:, :1], atol=1e-12)
    assert np.allclose(kh[:, 64:], k[:, 64:] / lam[:, 1:], atol=1e-12)


def test_grouped_halves_are_independent_mse():
    cfg = O.KeyConfig(mode="grouped", bits_outlier=4, bits_normal=2, seed=9)
    T = O.build_tables(cfg)
    rng = np.random.default_rng(6)
    k = rng.standard_normal((500, 128)) * np.r_[np.full(64, 10.0), np.ones(64)]
    enc = O.encode_keys(k, T)
    kh = O.dequant_keys(enc, T)
    for j, b in ((0, 4), (1, 2)):
        sl = slice(64 * j, 64 * (j + 1))
        half = O.KeyConfig(d=64, mode="mse", bits=b)
        Th = O.build_tables(half)
        Th.sigma = T.halves[j]["sigma"]
        ench = O.encode_keys(k[:, sl], Th)
        assert np.array_equal(ench["idx"], enc["idx"][:, sl])
        assert np.allclose(O.dequant_keys(ench, Th), kh[:, sl], atol=1e-12)
    rel = np.sum((k - kh) ** 2, axis=1) / np.sum(k * k, axis=1)
    assert rel.mean() < 0.02


# ---------------------------------------------------------------- grouped + QJL

def _grouped_prod_setup(seed=42, bo=4, bn=2):
    return O.build_tables(O.KeyConfig(mode="grouped_prod", bits_outlier=bo, bits_normal=bn, seed=seed))


def _dense_grouped_hat(k, enc, T, norms):
    """k_hat of the grouped stage written out with scipy's Hadamard matrix:
    half j is (n_j / 8) c_j[idx_j] Pi_j with Pi_j = H_64 diag(sigma_j) / 8."""
    H64 = scipy.linalg.hadamard(64)
    parts, rots = [], []
    for j, half in enumerate(T.halves):
        Pi = H64 * half["sigma"][None, :] / 8.0
        c = half["centroids"][enc["idx"][:, 64 * j:64 * (j + 1)]]
        parts.append((norms[:, j] / 8.0)[:, None] * (c @ Pi))
        rots.append(Pi)
    return np.concatenate(parts, axis=1), rots


def test_grouped_prod_sketch_is_the_block_rotated_residual():
    """The sign bits sketch the whole key's residual k - k_grouped_hat (float64
    norms) after rotating each half by its own Pi_j: z = S blockdiag(Pi_o,
    Pi_n) (k - k_grouped_hat), and rho = ||k - k_grouped_hat||.  The residual
    is formed here in the original domain from a dense Hadamard matrix, not
    through the encoder's rotated coordinates, so a dropped norm weight, a
    missing 1/sqrt(h), one norm for both halves or an unrotated residual
    fails."""
    T = _grouped_prod_setup()
    rng = np.random.default_rng(61)
    k = rng.standard_normal((40, 128)) * np.r_[np.full(64, 6.0), np.full(64, 0.5)]
    k[:10, 64:] *= 30.0                          # some keys with the larger normal half
    enc = O.encode_keys(k, T)
    norms = np.stack([np.linalg.norm(k[:, :64], axis=1), np.linalg.norm(k[:, 64:], axis=1)], axis=1)
    kg, rots = _dense_grouped_hat(k, enc, T, norms)
    e = k - kg
    w = np.concatenate([e[:, :64] @ rots[0].T, e[:, 64:] @ rots[1].T], axis=1)
    z = w @ T.S.T
    scale = np.linalg.norm(k, axis=1, keepdims=True)
    assert np.allclose(enc["z"], z, rtol=0, atol=1e-11 * scale.max())
    clear = np.abs(z) > 1e-9 * scale
    assert np.array_equal(enc["bits"][clear], (z[clear] >= 0).astype(np.uint8))
    assert np.allclose(enc["rnorm"], np.linalg.norm(e, axis=1), rtol=1e-12)
    assert np.array_equal(enc["rnorm16"], np.linalg.norm(e, axis=1).astype(np.float16))


def test_grouped_prod_keys_along_centroids_closed_form():
    """A half built along a centroid row, y_j = lam_j c_j[idx_j] with
    lam_j = 8 / ||c_j[idx_j]|| (the rotated half then has norm sqrt(64) and
    keeps its indices), has residual r_j = (lam_j - 1) c_j[idx_j], so
    rho = sqrt(sum_j n_j^2 (1 - 1/lam_j)^2) and the grouped stage returns
    k_j / lam_j."""
    T = _grouped_prod_setup(seed=17)
    rng = np.random.default_rng(62)
    H64 = scipy.linalg.hadamard(64)
    for n_out, n_norm in ((8.0, 0.5), (0.25, 3.0)):
        halves, lams = [], []
        for half, n in zip(T.halves, (n_out, n_norm)):
            c_all, t = half["centroids"], half["boundaries"]
            while True:
                idx = rng.integers(0, len(c_all), 64)
                c = c_all[idx]
                lam = 8.0 / np.linalg.norm(c)
                y = lam * c
                if np.array_equal(np.sum(y[:, None] >= t[None, :], axis=1), idx) and \
                        np.min(np.abs(y[:, None] - t[None, :])) > 1e-3:
                    break
            Pi = H64 * half["sigma"][None, :] / 8.0
            halves.append(n * (c / np.linalg.norm(c)) @ Pi)
            lams.append(lam)
        k = np.concatenate(halves)[None, :]
        enc = O.encode_keys(k, T)
        rho = math.sqrt(n_out ** 2 * (1 - 1 / lams[0]) ** 2 + n_norm ** 2 * (1 - 1 / lams[1]) ** 2)
        assert math.isclose(enc["rnorm"][0], rho, rel_tol=1e-12)
        g_only = dict(enc)
        g_only["rnorm16"] = np.zeros(1, dtype=np.float16)
        kh = O.dequant_keys(g_only, T)
        assert np.allclose(kh[0, :64], k[0, :64] / lams[0], atol=1e-12)
        assert np.allclose(kh[0, 64:], k[0, 64:] / lams[1], atol=1e-12)


def test_grouped_prod_unbiased_over_S_draws():
    """Theorem 2 for the grouped sketch: with the indices and fp16-exact half
    norms fixed, the mean of q.k_hat over independent Gaussian S (fp16
    entries) is q.k, and its variance is ((pi/2)||w||^2||a||^2 - <a,w>^2)/m
    with a = blockdiag(Pi) q the query in the sketch's frame."""
    T = _grouped_prod_setup(seed=5)
    rng = np.random.default_rng(63)
    k = rng.standard_normal((4, 128))
    k[:, :64] *= 4.0 / np.linalg.norm(k[:, :64], axis=1, keepdims=True)    # half norms 4 and 0.75,
    k[:, 64:] *= 0.75 / np.linalg.norm(k[:, 64:], axis=1, keepdims=True)   # exact in fp16
    q = rng.standard_normal((4, 128))
    base = O.encode_keys(k, T)
    assert np.array_equal(base["norm16"].astype(np.float64), np.tile([4.0, 0.75], (4, 1)))
    true = np.sum(q * k, axis=1)
    ests = []
    draws = 3000
    g = np.random.default_rng(64)
    for _ in range(draws):
        T.S = g.standard_normal((128, 128)).astype(np.float16).astype(np.float64)
        enc = dict(base)
        enc.update(O.grouped_prod_given_idx(base["norm"], base["y"], base["idx"], T))
        ests.append(np.sum(q * O.dequant_keys(enc, T), axis=1))
    ests = np.array(ests)
    mean, sd = ests.mean(0), ests.std(0)
    assert np.all(np.abs(mean - true) < 4 * sd / math.sqrt(draws)), (mean, true)
    H64 = scipy.linalg.hadamard(64)
    a = np.concatenate([q[:, 64 * j:64 * (j + 1)] @ (H64 * T.halves[j]["sigma"][None, :] / 8.0).T
                        for j in (0, 1)], axis=1)
    w = base["w"]
    var_theory = ((math.pi / 2) * np.sum(w * w, 1) * np.sum(a * a, 1) - np.sum(a * w, 1) ** 2) / 128
    assert np.all(np.abs(sd ** 2 / var_theory - 1) < 0.12), sd ** 2 / var_theory


def test_grouped_prod_bias_regression_slope_is_zero():
    """As for prod: the estimate's error has no component along the grouped
    stage's residual term <q, k - k_grouped_hat>."""
    T = _grouped_prod_setup(seed=7)
    rng = np.random.default_rng(65)
    k = rng.standard_normal((3000, 128)) * np.r_[np.full(64, 5.0), np.ones(64)]
    q = rng.standard_normal((3000, 128))
    enc = O.encode_keys(k, T)
    est = np.sum(q * O.dequant_keys(enc, T), axis=1)
    g_only = dict(enc)
    g_only["rnorm16"] = np.zeros_like(enc["rnorm16"])
    kg = O.dequant_keys(g_only, T)
    a = np.sum(q * (k - kg), axis=1)
    e = est - np.sum(q * k, axis=1)
    slope = np.sum(e * a) / np.sum(a * a)
    resid = e - slope * a
    se = math.sqrt(np.sum(resid ** 2) / (len(a) - 1) / np.sum(a * a))
    assert abs(slope) < 4 * se + 0.02, (slope, se)
    # with q isotropic and independent of the residual w, E<a, w>^2 = ||w||^2 ||a||^2 / d,
    # so the unbiased estimate's mean squared error is (pi/2 - 1/d) times that of the
    # grouped stage alone (whose error is -<a, w>); a QJL constant alpha scales it by alpha^2
    ratio = np.mean(e ** 2) / np.mean(a ** 2)
    assert abs(ratio / (math.pi / 2 - 1 / 128) - 1) < 0.1, ratio
    qjl = est - np.sum(q * kg, axis=1)
    assert np.corrcoef(qjl, a)[0, 1] > 0.5


# ---------------------------------------------------------------- outlier channels

def test_select_outlier_channels_worked_example():
    """Six channels over four rows with variances 1, 9, 4, 9, 0, 2.25 (channel
    2 shifted by 5 and channel 4 constant, which leave variance as it is)."""
    alt = np.array([1.0, -1.0, 1.0, -1.0])
    k = np.stack([alt, 3 * alt, 2 * alt + 5, -3 * alt, np.full(4, 7.0), 1.5 * alt], axis=1)
    assert np.array_equal(O.select_outlier_channels(k, 3), [1, 2, 3, 0, 4, 5])
    assert np.array_equal(O.select_outlier_channels(k, 1), [1, 0, 2, 3, 4, 5])   # tie 1/3: lower first
    assert np.array_equal(O.select_outlier_channels(k, 2), [1, 3, 0, 2, 4, 5])
    assert np.array_equal(O.select_outlier_channels(k, 5), [0, 1, 2, 3, 5, 4])
    assert np.array_equal(O.select_outlier_channels(k, 0), np.arange(6))
    assert np.array_equal(O.select_outlier_channels(k, 6), np.arange(6))


def test_select_outlier_channels_brute_force():
    """Over all 70 four-channel subsets of an 8-channel key set, the chosen
    outlier channels have the largest total variance."""
    import itertools
    rng = np.random.default_rng(66)
    k = rng.standard_normal((200, 8)) * rng.uniform(0.1, 5.0, 8) + rng.uniform(-3, 3, 8)
    var = np.var(k, axis=0)
    best = max(itertools.combinations(range(8), 4), key=lambda c: sum(var[list(c)]))
    perm = O.select_outlier_channels(k, 4)
    assert sorted(perm.tolist()) == list(range(8))
    assert tuple(perm[:4]) == best and list(perm[4:]) == sorted(set(range(8)) - set(best))


# ---------------------------------------------------------------- attention quality

def test_attention_quality_against_scipy():
    """KL of the exact softmax weights to the compressed ones against
    scipy.stats.entropy(p, p_hat); score and output cosines against
    scipy.spatial.distance.cosine."""
    import scipy.spatial.distance as SD
    import scipy.special as SS
    rng = np.random.default_rng(67)
    G, N, d = 3, 300, 16
    q, k, v = rng.standard_normal((G, d)) * 2, rng.standard_normal((N, d)), rng.standard_normal((N, d))
    kh = k + 0.3 * rng.standard_normal((N, d))
    vh = v + 0.1 * rng.standard_normal((N, d))
    r = O.attention_quality(q, k, v, kh, vh, sm_scale=0.4)
    for g in range(G):
        s, sh = k @ q[g], kh @ q[g]
        p, ph = SS.softmax(0.4 * s), SS.softmax(0.4 * sh)
        assert math.isclose(r["kl"][g], scipy.stats.entropy(p, ph), rel_tol=1e-9)
        assert math.isclose(r["score_cosine"][g], 1 - SD.cosine(s, sh), rel_tol=1e-12)
        assert math.isclose(r["out_cosine"][g], 1 - SD.cosine(p @ v, ph @ vh), rel_tol=1e-12)
        assert math.isclose(r["err2"][g], np.sum((sh - s) ** 2), rel_tol=1e-12)
        assert math.isclose(r["ref2"][g], np.sum(s * s), rel_tol=1e-12)
    assert r["kl"].min() > 0


def test_attention_quality_identical_cache_and_worked_topk():
    rng = np.random.default_rng(68)
    q, k, v = rng.standard_normal((2, 8)), rng.standard_normal((50, 8)), rng.standard_normal((50, 8))
    r = O.attention_quality(q, k, v, k, v)
    assert np.all(np.abs(r["kl"]) < 1e-14) and np.allclose(r["score_cosine"], 1, atol=1e-14)
    assert np.all(r["top1"] == 1) and np.all(r["topk_overlap"] == 1) and np.allclose(r["out_cosine"], 1)
    # scores 5, 4, 3, 2, 1, 0 against 5, 3, 4, 0, 1, 2: the same top token; top-5 sets
    # {0, 1, 2, 3, 4} and {0, 2, 1, 5, 4} share four; top-3 sets are equal
    q1 = np.array([[1.0, 0.0]])
    ka = np.array([[5, 0], [4, 0], [3, 0], [2, 0], [1, 0], [0, 0]], dtype=float)
    kb = np.array([[5, 0], [3, 0], [4, 0], [0, 0], [1, 0], [2, 0]], dtype=float)
    r5 = O.attention_quality(q1, ka, ka, kb, ka, topk=5)
    r3 = O.attention_quality(q1, ka, ka, kb, ka, topk=3)
    assert r5["top1"][0] == 1 and r5["topk_overlap"][0] == 0.8 and r3["topk_overlap"][0] == 1.0
    kc = np.array([[4, 0], [5, 0], [3, 0], [2, 0], [1, 0], [0, 0]], dtype=float)   # top token 1, not 0
    r1 = O.attention_quality(q1, ka, ka, kc, ka, topk=1)
    assert r1["top1"][0] == 0 and r1["topk_overlap"][0] == 0


def test_attention_quality_two_token_kl_closed_form():
    """Two tokens with logits (0, a) and (0, b): KL = sum_i p_i log(p_i / p_hat_i)
    with p_1 = 1 / (1 + e^-a)."""
    for a, b in ((1.0, 0.5), (3.0, -2.0), (0.25, 4.0)):
        q = np.array([[1.0]])
        r = O.attention_quality(q, np.array([[0.0], [a]]), np.ones((2, 1)), np.array([[0.0], [b]]),
                                np.ones((2, 1)), sm_scale=1.0)
        p1, h1 = 1 / (1 + math.exp(-a)), 1 / (1 + math.exp(-b))
        kl = (1 - p1) * math.log((1 - p1) / (1 - h1)) + p1 * math.log(p1 / h1)
        assert math.isclose(r["kl"][0], kl, rel_tol=1e-12, abs_tol=1e-15)


def test_packed_record_round_trip_all_modes():
    rng = np.random.default_rng(8)
    k = rng.standard_normal((64, 128))
    for cfg in (O.KeyConfig(mode="prod", bits=3), O.KeyConfig(mode="prod", bits=4),
                O.KeyConfig(mode="mse", bits=8), O.KeyConfig(mode="grouped"),
                O.KeyConfig(mode="grouped_prod", bits_outlier=3, bits_normal=2)):
        T = O.build_tables(cfg)
        enc = O.encode_keys(k, T)
        rec = O.pack_key_record(enc, T)
        back = O.unpack_key_record(rec, T)
        assert np.array_equal(back["idx"], enc["idx"])
        assert np.allclose(O.dequant_keys(back, T), O.dequant_keys(enc, T))
        nbytes = sum(v.shape[1] if v.ndim == 2 and v.dtype == np.uint8 else
                     v.dtype.itemsize * (v.shape[1] if v.ndim == 2 else 1) for v in rec.values())
        assert nbytes == O.record_bytes(cfg)


# ---------------------------------------------------------------- values

@pytest.mark.parametrize("bits", [2, 4])
def test_value_quantisation_error_bound(bits):
    rng = np.random.default_rng(bits)
    v = rng.standard_normal((2000, 128)).astype(np.float32)
    enc = O.encode_values(v, bits)
    vh = O.dequant_values(enc)
    s = enc["scale16"].astype(np.float64)
    z = enc["zero16"].astype(np.float64)
    vg = v.reshape(2000, 4, 32).astype(np.float64)
    err = np.abs(vg - vh.reshape(2000, 4, 32))
    # rounding error is at most s/2; clamping at the ends adds the fp16
    # rounding of min (z) and of the scale times the top level
    slack = np.abs(vg.min(-1) - z) + np.abs(vg.max(-1) - (z + ((1 << bits) - 1) * s))
    assert np.all(err <= (s / 2 + slack)[..., None] + 1e-6)
    codes = enc["codes"].reshape(2000, 4, 32)
    am = vg.argmin(-1)
    ax = vg.argmax(-1)
    assert np.all(np.take_along_axis(codes, am[..., None], -1) == 0)
    assert np.all(np.take_along_axis(codes, ax[..., None], -1) == (1 << bits) - 1)


@pytest.mark.parametrize("bits", [2, 4])
def test_value_rounding_ties_to_even(bits):
    """A group with min 0 and max 2^b - 1 has s = 1 and z = 0 exactly, so
    every value k + 1/2 is an exact rounding tie: ties go to the even code
    (0.5 -> 0, 1.5 -> 2, 2.5 -> 2, ...), the reading taken for the value
    quantiser.  Half-up would give 1, 2, 3, ...; truncation 0, 1, 2, ..."""
    top = (1 << bits) - 1
    ties = np.arange(top, dtype=np.float64) + 0.5            # 0.5 .. top - 0.5
    row = np.zeros(32)
    row[0], row[1] = 0.0, float(top)
    row[2:2 + len(ties)] = ties
    row[2 + len(ties):] = 1.0
    v = np.tile(row, 4)[None, :].astype(np.float32)
    enc = O.encode_values(v, bits)
    assert np.all(enc["scale16"] == 1.0) and np.all(enc["zero16"] == 0.0)
    want = np.array([int(t - 0.5) if int(t - 0.5) % 2 == 0 else int(t + 0.5) for t in ties])
    got = enc["codes"][0, 2:2 + len(ties)]
    assert np.array_equal(got, want), (got, want)
    assert enc["codes"][0, 0] == 0 and enc["codes"][0, 1] == top


def test_value_cosine_at_4_bits_matches_pack_article():
    """[pack] sec 三: 4-bit values reach cos_sim 0.997."""
    rng = np.random.default_rng(11)
    v = rng.standard_normal((4000, 128)).astype(np.float32)
    vh = O.dequant_values(O.encode_values(v, 4))
    cos = np.sum(v * vh, 1) / np.linalg.norm(v, axis=1) / np.linalg.norm(vh, axis=1)
    assert abs(cos.mean() - 0.997) < 0.0006
    vh2 = O.dequant_values(O.encode_values(v, 2))
    cos2 = np.sum(v * vh2, 1) / np.linalg.norm(v, axis=1) / np.linalg.norm(vh2, axis=1)
    assert 0.90 < cos2.mean() < 0.96


def test_value_constant_group():
    v = np.ones((2, 128), dtype=np.float32) * 3.25
    enc = O.encode_values(v, 2)
    assert np.all(enc["codes"] == 0) and np.all(enc["scale16"] == 0)
    assert np.array_equal(O.dequant_values(enc), v.astype(np.float64))


# ---------------------------------------------------------------- decode

def test_decode_attention_definitions():
    import torch
    rng = np.random.default_rng(12)
    q = rng.standard_normal((4, 128))
    k = rng.standard_normal((50, 128))
    v = rng.standard_normal((50, 128))
    s, o, lse = O.decode_attention(q, k, v, 37)
    assert s.shape == (4, 37)
    p = torch.softmax(torch.from_numpy(q @ k[:37].T / math.sqrt(128)), dim=-1).numpy()
    assert np.allclose(o, p @ v[:37], atol=1e-12)
    assert np.allclose(lse, np.log(np.exp(q @ k[:37].T / math.sqrt(128)).sum(-1)))
    # one token: output is that value
    _, o1, _ = O.decode_attention(q, k, v, 1)
    assert np.allclose(o1, np.broadcast_to(v[0], (4, 128)))
    # equal scores: plain mean
    _, o2, _ = O.decode_attention(np.zeros((1, 128)), k, v, 50)
    assert np.allclose(o2[0], v.mean(0))
    # tokens past ctx_len never matter
    v2 = v.copy()
    v2[37:] = 1e6
    assert np.allclose(O.decode_attention(q, k, v2, 37)[1], o)


# ---------------------------------------------------------------- quality

def test_recall_and_rank_correlation_thresholds():
    """validate_paper.py test_recall_at_scale: recall@8 >= 0.40 (3-bit),
    >= 0.55 (4-bit), 4-bit better; rank correlation > 0.75 / 0.90."""
    rng = np.random.default_rng(13)
    keys = rng.standard_normal((4096, 128)) * 0.1
    qs = rng.standard_normal((32, 128)) * 0.1
    true = qs @ keys.T
    rec, rho = {}, {}
    for b in (3, 4):
        T = _prod_setup(b)
        est = O.key_scores(qs, O.encode_keys(keys, T), T)
        rec[b] = O.recall_at_k(true, est, 8)
        rho[b] = np.mean([O.spearman(true[i], est[i]) for i in range(32)])
    assert rec[3] >= 0.40 and rec[4] >= 0.55 and rec[4] > rec[3], rec
    assert rho[3] > 0.75 and rho[4] > 0.90, rho


def test_spearman_matches_scipy():
    """The rank correlation is Spearman's rho: on tie-free data it equals
    scipy.stats.spearmanr, and it is invariant under monotone maps."""
    rng = np.random.default_rng(15)
    for n in (5, 64, 2048):
        a = rng.standard_normal(n)
        b = 0.6 * a + rng.standard_normal(n)
        ref = scipy.stats.spearmanr(a, b).statistic
        assert abs(O.spearman(a, b) - ref) < 1e-12, (n, O.spearman(a, b), ref)
        assert abs(O.spearman(np.exp(a), b ** 3) - ref) < 1e-12
    # worked example: ranks (0,1,2,3,4) against (0,2,1,4,3): d^2 = 4, rho = 1 - 6*4/(5*24) = 0.8
    assert abs(O.spearman(np.array([1., 2, 3, 4, 5]), np.array([10., 30, 20, 50, 40])) - 0.8) < 1e-12
    assert abs(O.spearman(np.arange(6.0), -np.arange(6.0)) + 1.0) < 1e-12


def test_recall_at_k_worked_example():
    """recall@k = |top-k(true) & top-k(est)| / k, averaged over queries."""
    true = np.array([[5., 4, 3, 2, 1], [1., 2, 3, 4, 5]])
    est = np.array([[5., 3, 4, 1, 2], [5., 4, 3, 2, 1]])
    # query 0: true top-2 {0,1}, est top-2 {0,2} -> 1/2; query 1: {4,3} vs {0,1} -> 0
    assert O.recall_at_k(true, est, 2) == 0.25
    # top-3: {0,1,2} vs {0,2,1} -> 1; {4,3,2} vs {0,1,2} -> 1/3
    assert abs(O.recall_at_k(true, est, 3) - (1 + 1 / 3) / 2) < 1e-15
    assert O.recall_at_k(true, true, 4) == 1.0
    assert O.recall_at_k(true, est, 5) == 1.0


def test_needle_argmax_over_dequantised_keys():
    """validate_paper.py test_needle_retrieval_depths, one KV head."""
    rng = np.random.default_rng(14)
    N = 4096
    for b in (3, 4):
        T = _prod_setup(b)
        for depth in (0.1, 0.5, 0.9):
            keys = rng.standard_normal((N, 128)) * 0.02
            needle = rng.standard_normal(128) * 3.0
            pos = int(N * depth)
            keys[pos] = needle
            s = O.key_scores(needle[None, :], O.encode_keys(keys, T), T)[0]
            assert int(np.argmax(s)) == pos
