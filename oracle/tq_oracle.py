"""CPU oracle for the TurboQuant KV-cache path: plain, slow, float64 NumPy.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and its
Python binding) may import or call this module; only the tests, the package's
smoke check and the CPU-baseline leg of the benchmark do.  It shares no code,
table or constant generator with the HIP implementation: every number it uses
is derived here from the definitions below.

Sources (the web pages this method is described on), cited by page and section:
  [tqlite]   "tqlite" README (gh.p.csz.net/YChange01/tqlite): sections
             "三种量化模式" (mode table: mse / prod / grouped and their bit costs),
             "设计要点" (per-row L2 normalisation to sqrt(d), per-layer seeds),
             "已知限制" (dense rotation, no packing).
  [difai]    "实现 TurboQuant (第5部分)" (difai.kr tutorial), section "算法概述"
             (residual = k - decompress, QJL sign(S @ residual), estimator
             <q,k_hat> + sqrt(pi/2)*(S@q)^T*sign_bits).
  [pack]     m.lqnn.cn article on TurboQuant's bit-packing layout, sections
             二 (2-bit: four per byte from the low bits), 三 (4-bit: two per
             byte; "3 比特怎么办": 3-bit stored as 4-bit), 四 (QJL signs eight
             per byte, weights 1..128; 52-byte key record).
  [validate] electron-rare/turboquant "validate_paper.py": test_mse_distortion_bounds
             (Theorem-1 bound), test_mse_codebook_table1 (Table 1 totals),
             test_prod_unbiased (Theorem 2), test_prod_distortion_scaling
             (Theorem 3), test_recall_at_scale, test_needle_retrieval_depths.

Readings of points the pages leave open are marked "Reading:" below.

Functions and their pins (what each is checked against, outside itself):
  lloyd_max_gaussian     closed form at 2 levels; textbook Gaussian Lloyd-Max
                         values (Max, 1960); Table 1 band; symmetry; the
                         centroid/midpoint conditions at the fixed point.
  splitmix64 / streams   published SplitMix64 test vector (seed 1234567).
  rademacher_signs       +-1 only; balanced on large draws.
  gaussian_matrix        moments of a large draw; Box-Muller identity.
  hadamard / rotation    scipy.linalg.hadamard; Pi Pi^T = I.
  bucketize              brute-force nearest centroid (ties upward) on tiny inputs.
  encode_* / dequant_*   Theorem-1 bound and D_b sampling band; QJL unbiasedness
                         over seeds and the regression slope; Theorem-3 bound;
                         exact k_hat for a key that sits on a centroid.
  pack / unpack          worked examples built from the pack article's rules
                         (tests/golden/pack_examples.json); round trips.
  encode_values          |v - v_hat| <= s/2 + fp16 error; min -> 0, max -> 2^b-1;
                         mean cosine at 4 bits (0.997 on the pack article, sec 三).
  decode_attention       one token -> o = v_hat; equal scores -> mean; masking;
                         torch.softmax on the CPU as a second opinion.
  grouped_prod           the sketch equals S applied to the block-rotated
                         original-domain residual built densely from scipy's
                         Hadamard matrix; rho = ||k - k_grouped_hat||; keys on
                         centroids give rho = 0 and exact k_hat; unbiasedness
                         over S draws and the regression slope.
  select_outlier_channels  hand-worked variances (ties to the lower channel);
                         brute force over all channel subsets of a small key.
  attention_quality      scipy's entropy (KL) and cosine distance; identical
                         caches give KL 0, cosine 1, full top-k agreement; a
                         worked top-k example; the two-token KL closed form.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import ndtr

__all__ = [
    "SPLITMIX_GAMMA", "TAG_SIGMA", "TAG_S", "TAG_SIGMA_OUT", "TAG_SIGMA_NORMAL",
    "splitmix64_stream", "rademacher_signs", "gaussian_matrix",
    "lloyd_max_gaussian", "codebook", "index_width",
    "hadamard", "rotation_matrix", "bucketize", "nearest_centroid",
    "KeyConfig", "KeyTables", "build_tables",
    "encode_keys", "dequant_keys", "key_scores", "prod_given_idx",
    "pack_fields", "unpack_fields", "pack_signs", "unpack_signs",
    "fp16_round", "encode_values", "dequant_values",
    "decode_attention", "record_bytes",
    "recall_at_k", "spearman",
    "grouped_prod_given_idx", "select_outlier_channels", "attention_quality",
]

# ---------------------------------------------------------------------------
# Random draws: SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
# number generators", OOPSLA 2014) with Box-Muller for Gaussians.
# Reading: the pages seed torch's generator (validate_paper.py sets
# torch.manual_seed(42) and builds quantisers with seed=42), which cannot be
# reproduced without torch; the method only needs i.i.d. signs and an i.i.d.
# N(0,1) matrix from a seed, so both sides use this published generator.
# ---------------------------------------------------------------------------
_MASK64 = (1 << 64) - 1
SPLITMIX_GAMMA = 0x9E3779B97F4A7C15
TAG_SIGMA = 1          # sigma of a full-width rotation
TAG_S = 2              # QJL matrix S
TAG_SIGMA_OUT = 3      # sigma of the outlier half (grouped mode)
TAG_SIGMA_NORMAL = 4   # sigma of the normal half (grouped mode)


def _mix64(z: int) -> int:
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def splitmix64_stream(seed: int, tag: int, count: int) -> list[int]:
    """Outputs 0..count-1 of SplitMix64 started at state seed XOR tag*gamma.

    Output i is mix64(state0 + (i+1)*gamma), the generator's published form."""
    s0 = (int(seed) ^ ((int(tag) * SPLITMIX_GAMMA) & _MASK64)) & _MASK64
    return [_mix64((s0 + (i + 1) * SPLITMIX_GAMMA) & _MASK64) for i in range(count)]


def rademacher_signs(seed: int, tag: int, d: int) -> np.ndarray:
    """sigma_j = +1 if the top bit of output j is 0, else -1 (float64, shape [d])."""
    out = splitmix64_stream(seed, tag, d)
    return np.array([1.0 - 2.0 * (x >> 63) for x in out], dtype=np.float64)


def gaussian_matrix(seed: int, tag: int, m: int, d: int) -> np.ndarray:
    """m x d i.i.d. N(0,1), row-major, Box-Muller on consecutive output pairs.

    u1 = (top 53 bits + 1) * 2^-53 in (0,1], u2 = top 53 bits * 2^-53 in [0,1);
    r = sqrt(-2 ln u1); element 2i = r cos(2 pi u2), element 2i+1 = r sin(2 pi u2).
    Each element is then rounded to float16 (round to nearest even) and
    returned as float64 holding that value.
    Reading: the pages fix no precision for S.  Rounding each N(0,1) draw to
    fp16 keeps the entries i.i.d. and symmetric but not exactly Gaussian, and
    the sign estimator's constant sqrt(pi/2) is exact only for Gaussian rows.
    The rounding (relative error <= 2^-11 per entry) moves E[sign(s.r)(s.a)]
    by less than 1e-4 of its value, bounded by a paired experiment in the pins
    (test_sign_estimator_with_fp16_entries); one key's 128-row estimate has a
    sampling spread near 10%."""
    n = m * d
    raw = splitmix64_stream(seed, tag, n + (n & 1))
    vals = []
    two_pi = 6.283185307179586
    for i in range(0, len(raw), 2):
        u1 = ((raw[i] >> 11) + 1) * (2.0 ** -53)
        u2 = (raw[i + 1] >> 11) * (2.0 ** -53)
        r = math.sqrt(-2.0 * math.log(u1))
        vals.append(r * math.cos(two_pi * u2))
        vals.append(r * math.sin(two_pi * u2))
    a = np.array(vals[:n], dtype=np.float64).astype(np.float16).astype(np.float64)
    return a.reshape(m, d)


# ---------------------------------------------------------------------------
# Lloyd-Max codebook for N(0,1)  ([tqlite] "三种量化模式": mse = rotation +
# Lloyd-Max codebook; [validate] test_mse_codebook_table1: get_codebook(d, b)
# with a "mse_total" field).
# Reading: the codebook is the MSE-optimal scalar quantiser of N(0,1), applied
# to the coordinates of sqrt(d) * Pi * u, which are close to N(0,1) for a unit
# vector u.  Its fixed point is unique (log-concave density).
# ---------------------------------------------------------------------------

def _phi(x):
    return np.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def _cell_prob(a, b):
    """P(a <= X < b) for X ~ N(0,1), computed on the tail that avoids cancellation."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    lower = ndtr(b) - ndtr(a)          # accurate when the cell sits below 0
    upper = ndtr(-a) - ndtr(-b)        # accurate when the cell sits above 0
    return np.where(a >= 0, upper, lower)


def _lloyd_map(c):
    """One Lloyd step: boundaries at midpoints, centroids at conditional means."""
    t = 0.5 * (c[:-1] + c[1:])
    lo = np.concatenate(([-np.inf], t))
    hi = np.concatenate((t, [np.inf]))
    p = _cell_prob(lo, hi)
    return (_phi(lo) - _phi(hi)) / p, lo, hi, p


def lloyd_max_gaussian(levels: int, tol: float = 1e-15, max_newton: int = 60):
    """Lloyd-Max quantiser of N(0,1) with `levels` cells.

    Returns (centroids[L], boundaries[L-1], D) in float64, D = E[(X - Q(X))^2].

    The fixed point of the Lloyd map is found in two stages: plain Lloyd steps
    from the high-resolution start c_k = sqrt(3) * Phi^-1((k + 1/2) / L), then
    Newton steps on c - lloyd(c) = 0 (Jacobian of the Lloyd map written out
    below), keeping the solution exactly antisymmetric.  Stops when a step
    changes no centroid by more than `tol`."""
    from scipy.special import ndtri
    L = int(levels)
    if L < 2:
        raise ValueError("need at least 2 levels")
    k = np.arange(L, dtype=np.float64)
    c = math.sqrt(3.0) * ndtri((k + 0.5) / L)
    for _ in range(200):
        c_new, _, _, _ = _lloyd_map(c)
        c = 0.5 * (c_new - c_new[::-1])
    for _ in range(max_newton):
        g, lo, hi, p = _lloyd_map(c)
        # d g_k / d lo_k = phi(lo)(g_k - lo)/p ; d g_k / d hi_k = phi(hi)(hi - g_k)/p
        dlo = np.where(np.isfinite(lo), _phi(lo) * (g - np.where(np.isfinite(lo), lo, 0.0)) / p, 0.0)
        dhi = np.where(np.isfinite(hi), _phi(hi) * (np.where(np.isfinite(hi), hi, 0.0) - g) / p, 0.0)
        J = np.zeros((L, L))
        for i in range(L):
            # lo_i = (c_{i-1} + c_i)/2, hi_i = (c_i + c_{i+1})/2
            if i > 0:
                J[i, i - 1] += 0.5 * dlo[i]
                J[i, i] += 0.5 * dlo[i]
            if i < L - 1:
                J[i, i + 1] += 0.5 * dhi[i]
                J[i, i] += 0.5 * dhi[i]
        F = c - g
        step = np.linalg.solve(np.eye(L) - J, F)
        c = c - step
        c = 0.5 * (c - c[::-1])
        if np.max(np.abs(step)) <= tol:
            break
    t = 0.5 * (c[:-1] + c[1:])
    t[(L - 1) // 2] = 0.0 if L % 2 == 0 else t[(L - 1) // 2]
    D = distortion(c, t)
    return c, t, D


def distortion(c, t) -> float:
    """E[(X - c_k)^2 ; X in cell k] summed over cells, by the cell integrals
    int x^2 phi = P - [x phi]_a^b, int x phi = phi(a) - phi(b)."""
    lo = np.concatenate(([-np.inf], t))
    hi = np.concatenate((t, [np.inf]))
    p = _cell_prob(lo, hi)
    xphi_lo = np.where(np.isfinite(lo), np.where(np.isfinite(lo), lo, 0.0) * _phi(lo), 0.0)
    xphi_hi = np.where(np.isfinite(hi), np.where(np.isfinite(hi), hi, 0.0) * _phi(hi), 0.0)
    m2 = p - (xphi_hi - xphi_lo)
    m1 = _phi(lo) - _phi(hi)
    return float(np.sum(m2 - 2.0 * c * m1 + c * c * p))


def index_width(bits: int) -> int:
    """Storage width of a b-bit index ([pack] sec 二/三: 2-bit four per byte,
    4-bit two per byte, 3-bit stored as 4-bit).  Reading: 1-bit indices eight
    per byte, 5..8-bit indices one byte each."""
    return {1: 1, 2: 2, 3: 4, 4: 4, 5: 8, 6: 8, 7: 8, 8: 8}[int(bits)]


_CODEBOOK_CACHE: dict = {}


def codebook(bits: int):
    """(centroids fp32-valued, boundaries fp32-valued, mse_total float64).

    Reading: each float64 value is rounded to float32 independently (the tables
    live in float32); mse_total is D of the float64 quantiser, which for unit
    vectors at any d equals the expected total squared error (d coordinates of
    variance 1/d each)."""
    b = int(bits)
    if b not in _CODEBOOK_CACHE:
        c, t, D = lloyd_max_gaussian(1 << b)
        _CODEBOOK_CACHE[b] = (c.astype(np.float32).astype(np.float64),
                              t.astype(np.float32).astype(np.float64), D)
    return _CODEBOOK_CACHE[b]


# ---------------------------------------------------------------------------
# Rotation Pi = Hadamard x random signs ([tqlite] directory listing:
# rotation.py "随机旋转 Π (Hadamard × 随机符号)"; "已知限制": dense O(d^2)).
# Reading: Pi = H diag(sigma) / sqrt(d) with Sylvester-ordered H
# (H[i, j] = (-1)^popcount(i & j)): the signs act first.
# ---------------------------------------------------------------------------

def hadamard(d: int) -> np.ndarray:
    i = np.arange(d)
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1.0, -1.0)


def rotation_matrix(sigma: np.ndarray) -> np.ndarray:
    d = sigma.shape[0]
    return hadamard(d) * sigma[None, :] / math.sqrt(d)


def bucketize(y: np.ndarray, boundaries: np.ndarray) -> np.ndarray:
    """idx = #{k : y >= t_k} (ties go to the upper cell)."""
    return np.sum(y[..., None] >= boundaries, axis=-1).astype(np.int64)


def nearest_centroid(y: np.ndarray, centroids: np.ndarray) -> np.ndarray:
    """Brute-force argmin_k |y - c_k|; on an exact tie the larger index wins."""
    dist = np.abs(y[..., None] - centroids)
    best = dist.min(axis=-1, keepdims=True)
    L = centroids.shape[0]
    cand = np.where(dist == best, np.arange(L), -1)
    return cand.max(axis=-1).astype(np.int64)


# ---------------------------------------------------------------------------
# Key configuration and seed-derived tables.
# ---------------------------------------------------------------------------

class KeyConfig:
    """mode: "mse" | "prod" | "grouped" | "grouped_prod".

    mse:     index bits = bits ([tqlite] mode table: d*bits).
    prod:    bits = total bits per coordinate; index bits = bits - 1, plus one
             QJL sign per row of S.  Reading: the pages disagree ([tqlite]
             charges d*bits + d + 32, [difai] "PolarQuant (b-1 bit) + QJL
             (1 bit)", [pack] sec 四 3-bit = 2-bit index + 1 sign); the
             (b-1)+1 split is taken.  m = d rows of S.
    grouped: channels [0, d/2) take bits_outlier, [d/2, d) bits_normal, each
             half its own norm, rotation and codebook, no QJL ([tqlite] mode
             table: d_out*b_out + d_n*b_n).
    grouped_prod: the grouped quantiser as above, then one QJL stage over the
             whole key's residual: m = d sign bits and one fp16 residual norm.
             Reading: the pages describe grouped mode without a residual stage
             and the QJL stage on a single-rotation MSE quantiser; [tqlite]'s
             mode table charges the QJL stage d + 32 bits on top of the MSE
             stage's own bits, so here bits_outlier / bits_normal stay the
             halves' index bits and the signs come on top.  The residual is
             sketched as one d-vector (see grouped_prod_given_idx)."""

    def __init__(self, d=128, mode="prod", bits=3, seed=42, bits_outlier=4, bits_normal=2):
        self.d = int(d)
        self.mode = mode
        self.bits = int(bits)
        self.seed = int(seed)
        self.bits_outlier = int(bits_outlier)
        self.bits_normal = int(bits_normal)
        if self.d & (self.d - 1) or self.d < 2:
            raise ValueError("d must be a power of two")
        if mode not in ("mse", "prod", "grouped", "grouped_prod"):
            raise ValueError(mode)

    @property
    def idx_bits(self):
        return self.bits - 1 if self.mode == "prod" else self.bits

    @property
    def m(self):
        return self.d


class KeyTables:
    pass


def build_tables(cfg: KeyConfig) -> KeyTables:
    T = KeyTables()
    T.cfg = cfg
    if cfg.mode in ("grouped", "grouped_prod"):
        h = cfg.d // 2
        T.halves = []
        for tag, b in ((TAG_SIGMA_OUT, cfg.bits_outlier), (TAG_SIGMA_NORMAL, cfg.bits_normal)):
            c, t, D = codebook(b)
            T.halves.append(dict(d=h, bits=b, sigma=rademacher_signs(cfg.seed, tag, h),
                                 centroids=c, boundaries=t, mse=D))
        if cfg.mode == "grouped_prod":
            T.S = gaussian_matrix(cfg.seed, TAG_S, cfg.m, cfg.d)
        return T
    c, t, D = codebook(cfg.idx_bits)
    T.centroids, T.boundaries, T.mse = c, t, D
    T.sigma = rademacher_signs(cfg.seed, TAG_SIGMA, cfg.d)
    if cfg.mode == "prod":
        T.S = gaussian_matrix(cfg.seed, TAG_S, cfg.m, cfg.d)
    return T


# ---------------------------------------------------------------------------
# fp16 storage ([pack] sec 四: norms stored as float16).
# ---------------------------------------------------------------------------

def fp16_round(x) -> np.ndarray:
    """IEEE binary16, round to nearest even, from the float64 value."""
    return np.asarray(x, dtype=np.float64).astype(np.float16)


# ---------------------------------------------------------------------------
# Key encoding.
# ---------------------------------------------------------------------------

def _rotate_unit(keys: np.ndarray, sigma: np.ndarray):
    """n = ||k||, u = k / n (u = 0 when n = 0), y = sqrt(d) Pi u = H (sigma * u).

    [tqlite] "设计要点": keys are scaled to ||.|| = sqrt(d) before quantising and
    the norm is restored afterwards; sqrt(d) Pi u is exactly that rescaling."""
    k = np.asarray(keys, dtype=np.float64)
    d = k.shape[-1]
    n = np.sqrt(np.sum(k * k, axis=-1))
    safe = np.where(n > 0, n, 1.0)
    u = np.where(n[..., None] > 0, k / safe[..., None], 0.0)
    y = u @ rotation_matrix(sigma).T * math.sqrt(d)
    return n, y


def encode_keys(keys: np.ndarray, T: KeyTables) -> dict:
    """Encode keys [n, d] (any float dtype, taken exactly as float64).

    Returns a dict with
      idx    int64 [n, d]   centroid indices (grouped: halves concatenated)
      norm16 float16 [n] (grouped: [n, 2])
      prod:  bits uint8 [n, m] (1 iff z >= 0), rnorm16 float16 [n]
      and the float64 intermediates y (rotated coordinates, sqrt(d)-scaled)
      and z (S r, prod) used to locate decision-boundary cases.

    prod ([difai] "算法概述"; [tqlite] mode table "MSE + QJL 1-bit 残差"):
      r = y - c[idx] in the rotated domain; z = S r; bit_i = [z_i >= 0];
      rho = n ||r|| / sqrt(d) = ||k - k_mse_hat||.
    Reading: the pages take the residual in the original domain
    (k - decompress(codes)) and project it with S; taking it in the rotated
    domain is the same estimator with S' = S Pi, whose rows are again i.i.d.
    N(0, I), and rho is exactly the original-domain residual norm."""
    cfg = T.cfg
    keys = np.asarray(keys, dtype=np.float64)
    out = {}
    if cfg.mode in ("grouped", "grouped_prod"):
        h = cfg.d // 2
        idxs, norms, ys = [], [], []
        for half, sl in zip(T.halves, (slice(0, h), slice(h, cfg.d))):
            n, y = _rotate_unit(keys[:, sl], half["sigma"])
            idxs.append(bucketize(y, half["boundaries"]))
            norms.append(n)
            ys.append(y)
        out["idx"] = np.concatenate(idxs, axis=1)
        out["norm"] = np.stack(norms, axis=1)
        out["norm16"] = fp16_round(out["norm"])
        out["y"] = np.concatenate(ys, axis=1)
        if cfg.mode == "grouped_prod":
            out.update(grouped_prod_given_idx(out["norm"], out["y"], out["idx"], T))
        return out
    n, y = _rotate_unit(keys, T.sigma)
    idx = bucketize(y, T.boundaries)
    out.update(idx=idx, norm=n, norm16=fp16_round(n), y=y)
    if cfg.mode == "prod":
        out.update(prod_given_idx(n, y, idx, T))
    return out


def prod_given_idx(n: np.ndarray, y: np.ndarray, idx: np.ndarray, T: KeyTables) -> dict:
    """QJL stage for a given index choice (also used when a coordinate on a
    decision boundary may legitimately go either way)."""
    d = T.cfg.d
    r = y - T.centroids[idx]
    z = r @ T.S.T
    bits = (z >= 0).astype(np.uint8)
    rho = n * np.sqrt(np.sum(r * r, axis=-1)) / math.sqrt(d)
    return dict(r=r, z=z, bits=bits, rnorm=rho, rnorm16=fp16_round(rho))


def grouped_prod_given_idx(norms: np.ndarray, y: np.ndarray, idx: np.ndarray, T: KeyTables) -> dict:
    """QJL stage of grouped_prod for given half indices.

    Half j (h = d/2 channels) has the rotated, sqrt(h)-scaled coordinates y_j,
    the residual r_j = y_j - c_j[idx_j] and, in the original domain, the
    residual e_j = (n_j / sqrt(h)) Pi_j^T r_j.  The sketch takes
    w = concat_j (n_j / sqrt(h)) r_j = blockdiag(Pi_o, Pi_n) e: the whole
    key's residual in the block-rotated frame, where the queries are rotated
    too.  z = S w, bit_i = [z_i >= 0], rho = ||w|| = ||k - k_grouped_hat||.
    Reading: [difai] "算法概述" sketches the residual k - decompress(codes)
    with one Gaussian S; blockdiag(Pi) is orthogonal, so S blockdiag(Pi) again
    has i.i.d. N(0, 1) entries and the estimator is unchanged."""
    d = T.cfg.d
    h = d // 2
    parts = []
    for j, half in enumerate(T.halves):
        sl = slice(j * h, (j + 1) * h)
        r = y[:, sl] - half["centroids"][idx[:, sl]]
        parts.append((norms[:, j] / math.sqrt(h))[:, None] * r)
    w = np.concatenate(parts, axis=1)
    z = w @ T.S.T
    bits = (z >= 0).astype(np.uint8)
    rho = np.sqrt(np.sum(w * w, axis=-1))
    return dict(w=w, z=z, bits=bits, rnorm=rho, rnorm16=fp16_round(rho))


def dequant_keys(enc: dict, T: KeyTables) -> np.ndarray:
    """Dense k_hat [n, d] from the stored fields (fp16 norms as stored).

    mse:  k_hat = (n16 / sqrt(d)) Pi^T c[idx]
    prod: + rho16 * sqrt(pi/2) / m * Pi^T S^T (2 bit - 1)
    grouped: each half (n16_j / sqrt(h)) Pi_j^T c_j[idx_j]
    grouped_prod: + rho16 * sqrt(pi/2) / m * blockdiag(Pi_o, Pi_n)^T S^T (2 bit - 1)
    Reading: [difai] prints the QJL term as sqrt(pi/2) * (S@q)^T * sign_bits,
    without ||r|| and 1/m; both are required for E[<q, k_hat>] = <q, k>
    (E[sign(s.r)(s.a)] = sqrt(2/pi) <a, r>/||r|| for s ~ N(0, I))."""
    cfg = T.cfg
    if cfg.mode in ("grouped", "grouped_prod"):
        h = cfg.d // 2
        parts = []
        if cfg.mode == "grouped_prod":
            sgn = 2.0 * enc["bits"].astype(np.float64) - 1.0
            rho16 = enc["rnorm16"].astype(np.float64)
            t = (rho16 * math.sqrt(math.pi / 2.0) / cfg.m)[:, None] * (sgn @ T.S)   # block-rotated frame
        for j, half in enumerate(T.halves):
            Pi = rotation_matrix(half["sigma"])
            c = half["centroids"][enc["idx"][:, j * h:(j + 1) * h]]
            n16 = enc["norm16"][:, j].astype(np.float64)
            part = (n16 / math.sqrt(h))[:, None] * (c @ Pi)
            if cfg.mode == "grouped_prod":
                part = part + t[:, j * h:(j + 1) * h] @ Pi
            parts.append(part)
        return np.concatenate(parts, axis=1)
    d = cfg.d
    Pi = rotation_matrix(T.sigma)
    n16 = enc["norm16"].astype(np.float64)
    k = (n16 / math.sqrt(d))[:, None] * (T.centroids[enc["idx"]] @ Pi)
    if cfg.mode == "prod":
        sgn = 2.0 * enc["bits"].astype(np.float64) - 1.0
        rho16 = enc["rnorm16"].astype(np.float64)
        k = k + (rho16 * math.sqrt(math.pi / 2.0) / cfg.m)[:, None] * ((sgn @ T.S) @ Pi)
    return k


def key_scores(q: np.ndarray, enc: dict, T: KeyTables) -> np.ndarray:
    """Estimated q . k for every (query, key): q [nq, d] against the dense
    k_hat.  This is the plain definition; the packed-domain estimator computes
    the same quantity without forming k_hat."""
    return np.asarray(q, dtype=np.float64) @ dequant_keys(enc, T).T


# ---------------------------------------------------------------------------
# Bit packing ([pack] sec 二, 三, "3 比特怎么办", 四).
# Element j of a row of w-bit fields goes to byte floor(j*w/8), starting at bit
# (j mod (8/w)) * w: the first element takes the lowest bits.  Sign bit i goes
# to byte floor(i/8) with weight 2^(i mod 8).
# ---------------------------------------------------------------------------

def pack_fields(codes: np.ndarray, width: int) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.int64)
    n, d = codes.shape
    per = 8 // width
    if d % per:
        raise ValueError("row length must fill whole bytes")
    if codes.min(initial=0) < 0 or codes.max(initial=0) >= (1 << width):
        raise ValueError("code does not fit its field")
    out = np.zeros((n, d // per), dtype=np.int64)
    for j in range(d):
        out[:, j // per] |= codes[:, j] << ((j % per) * width)
    return out.astype(np.uint8)


def unpack_fields(packed: np.ndarray, width: int, d: int) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.int64)
    per = 8 // width
    mask = (1 << width) - 1
    out = np.zeros((packed.shape[0], d), dtype=np.int64)
    for j in range(d):
        out[:, j] = (packed[:, j // per] >> ((j % per) * width)) & mask
    return out


def pack_signs(bits: np.ndarray) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.int64)
    n, m = bits.shape
    weights = np.array([1, 2, 4, 8, 16, 32, 64, 128], dtype=np.int64)
    return (bits.reshape(n, m // 8, 8) * weights).sum(axis=-1).astype(np.uint8)


def unpack_signs(packed: np.ndarray, m: int) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.int64)
    out = np.zeros((packed.shape[0], m), dtype=np.uint8)
    for i in range(m):
        out[:, i] = (packed[:, i // 8] >> (i % 8)) & 1
    return out


def pack_key_record(enc: dict, T: KeyTables) -> dict:
    """Packed planes of an encoded key set: idx bytes, sign bytes, fp16 norms."""
    cfg = T.cfg
    if cfg.mode in ("grouped", "grouped_prod"):
        h = cfg.d // 2
        parts = [pack_fields(enc["idx"][:, j * h:(j + 1) * h], index_width(half["bits"]))
                 for j, half in enumerate(T.halves)]
        rec = dict(idx=np.concatenate(parts, axis=1), norm=enc["norm16"])
        if cfg.mode == "grouped_prod":
            rec["signs"] = pack_signs(enc["bits"])
            rec["rnorm"] = enc["rnorm16"]
        return rec
    rec = dict(idx=pack_fields(enc["idx"], index_width(cfg.idx_bits)), norm=enc["norm16"])
    if cfg.mode == "prod":
        rec["signs"] = pack_signs(enc["bits"])
        rec["rnorm"] = enc["rnorm16"]
    return rec


def unpack_key_record(rec: dict, T: KeyTables) -> dict:
    cfg = T.cfg
    if cfg.mode in ("grouped", "grouped_prod"):
        h = cfg.d // 2
        w0, w1 = (index_width(half["bits"]) for half in T.halves)
        nb0 = h * w0 // 8
        idx = np.concatenate([unpack_fields(rec["idx"][:, :nb0], w0, h),
                              unpack_fields(rec["idx"][:, nb0:], w1, h)], axis=1)
        enc = dict(idx=idx, norm16=np.asarray(rec["norm"], dtype=np.float16))
        if cfg.mode == "grouped_prod":
            enc["bits"] = unpack_signs(rec["signs"], cfg.m)
            enc["rnorm16"] = np.asarray(rec["rnorm"], dtype=np.float16)
        return enc
    enc = dict(idx=unpack_fields(rec["idx"], index_width(cfg.idx_bits), cfg.d),
               norm16=np.asarray(rec["norm"], dtype=np.float16))
    if cfg.mode == "prod":
        enc["bits"] = unpack_signs(rec["signs"], cfg.m)
        enc["rnorm16"] = np.asarray(rec["rnorm"], dtype=np.float16)
    return enc


def record_bytes(cfg: KeyConfig) -> int:
    """Bytes of one packed key record (planes summed)."""
    if cfg.mode in ("grouped", "grouped_prod"):
        h = cfg.d // 2
        b = (h * index_width(cfg.bits_outlier) + h * index_width(cfg.bits_normal)) // 8 + 4
        return b + (cfg.m // 8 + 2 if cfg.mode == "grouped_prod" else 0)
    b = cfg.d * index_width(cfg.idx_bits) // 8 + 2
    if cfg.mode == "prod":
        b += cfg.m // 8 + 2
    return b


# ---------------------------------------------------------------------------
# Values: per-token group quantisation ([pack] sec 二 value cache 2-bit by
# default, sec 三 4-bit values; group size 32 with fp16 scale and zero).
# Reading (the pages give no formula): groups of 32 consecutive channels of one
# token, asymmetric min-max, s = (max - min) / (2^b - 1) rounded to fp16,
# z = min rounded to fp16, code = clamp(rint((v - z) / s), 0, 2^b - 1) with
# ties to even, all in float32 (the pages' tensors are float32) using the
# fp16-rounded s and z; a constant group (s16 == 0) gets code 0.
# ---------------------------------------------------------------------------

def encode_values(values: np.ndarray, bits: int, group: int = 32) -> dict:
    v = np.asarray(values, dtype=np.float32)
    n, d = v.shape
    G = d // group
    vg = v.reshape(n, G, group)
    mn = vg.min(axis=-1)
    mx = vg.max(axis=-1)
    levels = np.float32((1 << bits) - 1)
    s32 = ((mx - mn).astype(np.float32) / levels).astype(np.float32)
    s16 = s32.astype(np.float16)
    z16 = mn.astype(np.float16)
    s = s16.astype(np.float32)
    z = z16.astype(np.float32)
    diff = (vg - z[..., None]).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = (diff / s[..., None]).astype(np.float32)
    code = np.clip(np.rint(ratio), 0, (1 << bits) - 1)
    code = np.where(s[..., None] == 0, 0, code).astype(np.int64)
    return dict(codes=code.reshape(n, d), scale16=s16, zero16=z16, ratio=ratio.reshape(n, d))


def dequant_values(enc: dict, group: int = 32) -> np.ndarray:
    code = enc["codes"].astype(np.float64)
    n, d = code.shape
    s = enc["scale16"].astype(np.float64)
    z = enc["zero16"].astype(np.float64)
    return (code.reshape(n, d // group, group) * s[..., None] + z[..., None]).reshape(n, d)


def pack_value_record(enc: dict, bits: int) -> dict:
    return dict(codes=pack_fields(enc["codes"], index_width(bits)),
                scale=enc["scale16"], zero=enc["zero16"])


def unpack_value_record(rec: dict, bits: int, d: int) -> dict:
    return dict(codes=unpack_fields(rec["codes"], index_width(bits), d),
                scale16=np.asarray(rec["scale"], dtype=np.float16),
                zero16=np.asarray(rec["zero"], dtype=np.float16))


# ---------------------------------------------------------------------------
# Decode attention over the dequantised cache (definition).
# Reading: softmax scale defaults to 1/sqrt(d) (the pages' attention_score
# returns raw inner products); query head h reads KV head h // (Hq / Hkv).
# ---------------------------------------------------------------------------

def decode_attention(q: np.ndarray, khat: np.ndarray, vhat: np.ndarray, ctx_len: int,
                     sm_scale: float | None = None):
    """One (sequence, KV head) group: q [G, d] query heads sharing khat/vhat
    [N, d].  Returns (scores [G, ctx_len] raw q.k_hat, out [G, d], lse [G])."""
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[-1]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    k = np.asarray(khat, dtype=np.float64)[:ctx_len]
    v = np.asarray(vhat, dtype=np.float64)[:ctx_len]
    s = q @ k.T
    if ctx_len == 0:
        return s, np.zeros_like(q), np.full(q.shape[0], -np.inf)
    x = sm_scale * s
    mx = x.max(axis=-1, keepdims=True)
    e = np.exp(x - mx)
    l = e.sum(axis=-1, keepdims=True)
    out = (e / l) @ v
    lse = (mx + np.log(l))[:, 0]
    return s, out, lse


# ---------------------------------------------------------------------------
# Quality metrics ([validate] test_recall_at_scale; rank correlation check).
# ---------------------------------------------------------------------------

def recall_at_k(true_scores: np.ndarray, est_scores: np.ndarray, k: int) -> float:
    t = np.argsort(-true_scores, axis=-1, kind="stable")[:, :k]
    e = np.argsort(-est_scores, axis=-1, kind="stable")[:, :k]
    return float(np.mean([len(set(a) & set(b)) / k for a, b in zip(t, e)]))


def spearman(a: np.ndarray, b: np.ndarray) -> float:
    ra = np.argsort(np.argsort(a)).astype(np.float64)
    rb = np.argsort(np.argsort(b)).astype(np.float64)
    ra -= ra.mean()
    rb -= rb.mean()
    return float((ra * rb).sum() / math.sqrt((ra * ra).sum() * (rb * rb).sum()))


# ---------------------------------------------------------------------------
# Outlier channels for grouped mode ([tqlite] mode table: "高方差通道分配更高
# bit", the high-variance channels get the higher bit width).
# Reading: the page names the criterion but not the estimator or tie rule:
# population variance of each channel over the given key rows, the n_outlier
# largest taken (equal variances: the lower channel first); the result lists
# the chosen channels in increasing order, then the others in increasing
# order.  Keys and queries are both reordered by it, which leaves q.k as it is.
# ---------------------------------------------------------------------------

def select_outlier_channels(keys: np.ndarray, n_outlier: int) -> np.ndarray:
    k = np.asarray(keys, dtype=np.float64)
    d = k.shape[1]
    if not 0 <= n_outlier <= d:
        raise ValueError("n_outlier out of range")
    if k.shape[0] == 0:
        var = np.zeros(d)
    else:
        mean = k.mean(axis=0)
        var = ((k - mean) ** 2).mean(axis=0)
    ranked = sorted(range(d), key=lambda c: (-var[c], c))
    chosen = sorted(ranked[:n_outlier])
    rest = sorted(ranked[n_outlier:])
    return np.array(chosen + rest, dtype=np.int64)


# ---------------------------------------------------------------------------
# Attention quality of a compressed cache against the exact one ([difai]
# compare.py output items 3 and 5: cosine similarity, Top-1/5 agreement and KL
# divergence of the attention scores at 2/3/4 bits).
# Reading: "attention score" comparisons are taken per query head over one
# KV head's tokens: cosine of the raw score vectors q.k vs q.k_hat; KL of the
# exact softmax weights to the compressed ones, KL(p || p_hat); Top-1 agreement
# of the highest-scoring token; Top-k overlap |top_k(s) & top_k(s_hat)| / k.
# The attention outputs' cosine (p v against p_hat v_hat) is added, since the
# value cache is compressed too.
# ---------------------------------------------------------------------------

def _cosine(a, b) -> float:
    """<a, b> / (||a|| ||b||); NaN when either vector is zero."""
    den = math.sqrt(float(a @ a) * float(b @ b))
    return float(a @ b) / den if den > 0 else float("nan")


def attention_quality(q: np.ndarray, k: np.ndarray, v: np.ndarray, khat: np.ndarray,
                      vhat: np.ndarray, sm_scale: float | None = None, topk: int = 5) -> dict:
    """q [G, d] query heads of one KV head, k/v the exact cache [N, d],
    khat/vhat the compressed one.  Returns per-query-head float64 arrays
    score_cosine, kl, top1 (0/1), topk_overlap, out_cosine, and the squared
    score error and squared exact score summed over tokens (err2, ref2)."""
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[-1]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    s = q @ np.asarray(k, dtype=np.float64).T
    sh = q @ np.asarray(khat, dtype=np.float64).T
    res = {key: [] for key in ("score_cosine", "kl", "top1", "topk_overlap", "out_cosine", "err2", "ref2")}
    for g in range(q.shape[0]):
        a, b = s[g], sh[g]
        res["score_cosine"].append(_cosine(a, b))
        xa, xb = sm_scale * a, sm_scale * b
        la = xa - xa.max() - math.log(float(np.sum(np.exp(xa - xa.max()))))
        lb = xb - xb.max() - math.log(float(np.sum(np.exp(xb - xb.max()))))
        p, ph = np.exp(la), np.exp(lb)
        res["kl"].append(float(np.sum(p * (la - lb))))
        order_a = sorted(range(len(a)), key=lambda t: (-a[t], t))
        order_b = sorted(range(len(b)), key=lambda t: (-b[t], t))
        res["top1"].append(1.0 if order_a[0] == order_b[0] else 0.0)
        res["topk_overlap"].append(len(set(order_a[:topk]) & set(order_b[:topk])) / topk)
        o = p @ np.asarray(v, dtype=np.float64)
        oh = ph @ np.asarray(vhat, dtype=np.float64)
        res["out_cosine"].append(_cosine(o, oh))
        res["err2"].append(float(np.sum((b - a) ** 2)))
        res["ref2"].append(float(np.sum(a * a)))
    return {key: np.array(val) for key, val in res.items()}
