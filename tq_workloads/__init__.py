"""Seeded synthetic inputs for the TurboQuant KV-cache path.

This module only draws random inputs and describes workload shapes; it holds
none of the method's arithmetic (no rotation, codebook, quantisation or
attention).  Both the CPU oracle's tests and the HIP path's tests, benchmark
and smoke check take their inputs from here, so the two sides see the same
numbers.

Every tensor is drawn from numpy.random.default_rng(SeedSequence([42, workload_id,
tensor_id])).  bf16 inputs are float32 draws rounded to bfloat16 with
round-to-nearest-even (returned as float32 arrays that hold bf16 values, and as
the raw uint16 bit pattern for upload).

Workloads (head_dim 128 throughout, the pages' shapes: GQA, 4k..128k context,
3-bit keys and 2-bit values by default):
  W1 tiny prod check   1 KV head x 4096 keys, unit-norm fp32 keys, 8 queries
  W2 MSE prefill encode 28 layers x 2 KV heads x 32768 bf16 keys, norms
                       log-uniform in [2, 20]
  W3 batched GQA decode 16 seqs x 8 KV heads x 32 query heads, ctx 32768
  W4 long-context needle 1 seq x 8 KV heads x 32 query heads, ctx 131072
  W5 outlier-grouped   8 seqs x 8 KV heads x 32 query heads, ctx 16384,
                       channels 0..63 ~ N(0, 10^2), 64..127 ~ N(0, 1)
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BASE_SEED = 42


def rng(workload_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([BASE_SEED, int(workload_id), int(tensor_id)]))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.
    NaN is not expected in these inputs."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> the float32 values they denote."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_bf16(x: np.ndarray):
    b = bf16_bits(x)
    return bf16_values(b), b


@dataclass
class Workload:
    wid: int
    name: str
    B: int
    Hkv: int
    Hq: int
    ctx: int
    d: int = 128
    key_mode: str = "prod"
    key_bits: int = 3
    bits_outlier: int = 4
    bits_normal: int = 2
    v_bits: int = 2
    v_group: int = 32
    dtype: str = "bf16"
    layers: int = 1
    extra: dict = field(default_factory=dict)

    @property
    def n_token_heads(self) -> int:
        return self.B * self.Hkv * self.ctx


WORKLOADS = {
    1: Workload(1, "tiny-prod-check", B=1, Hkv=1, Hq=8, ctx=4096, key_mode="prod", key_bits=3,
                v_bits=2, dtype="f32"),
    2: Workload(2, "mse-prefill-encode", B=1, Hkv=2, Hq=2, ctx=32768, key_mode="mse", key_bits=4,
                dtype="bf16", layers=28),
    3: Workload(3, "gqa-decode-32k", B=16, Hkv=8, Hq=32, ctx=32768, key_mode="prod", key_bits=3,
                v_bits=2),
    4: Workload(4, "needle-decode-128k", B=1, Hkv=8, Hq=32, ctx=131072, key_mode="prod", key_bits=4,
                v_bits=4),
    5: Workload(5, "outlier-grouped-16k", B=8, Hkv=8, Hq=32, ctx=16384, key_mode="grouped",
                key_bits=4, bits_outlier=4, bits_normal=2, v_bits=4),
}

# tensor ids
T_KEYS, T_VALUES, T_QUERIES, T_NORMS, T_NEEDLE_NOISE = 1, 2, 3, 4, 5
NEEDLE_DEPTHS = (0.1, 0.3, 0.5, 0.7, 0.9)


def gaussian(wid: int, tid: int, shape, scale=1.0) -> np.ndarray:
    return (rng(wid, tid).standard_normal(shape, dtype=np.float32) * np.float32(scale)).astype(np.float32)


# --- W1 ---------------------------------------------------------------------

def w1_inputs(n_keys: int = 4096, n_queries: int = 8, d: int = 128):
    """Keys N(0,1) scaled to unit L2 norm (float32), values N(0,1) float32,
    queries N(0,1) float32."""
    k = gaussian(1, T_KEYS, (n_keys, d)).astype(np.float64)
    k = (k / np.linalg.norm(k, axis=1, keepdims=True)).astype(np.float32)
    v = gaussian(1, T_VALUES, (n_keys, d))
    q = gaussian(1, T_QUERIES, (n_queries, d))
    return k, v, q


# --- W2 ---------------------------------------------------------------------

def w2_layer_keys(layer: int, heads: int = 2, n_tok: int = 32768, d: int = 128, row_slice=None):
    """Keys of one layer, [heads * n_tok, d] bf16 (as float32 values + bits):
    N(0, I) direction times a norm drawn log-uniform in [2, 20]."""
    g = rng(2, 100 + layer)
    dirs = g.standard_normal((heads * n_tok, d), dtype=np.float32).astype(np.float64)
    norms = np.exp(g.uniform(math.log(2.0), math.log(20.0), size=heads * n_tok))
    if row_slice is not None:
        dirs, norms = dirs[row_slice], norms[row_slice]
    k = dirs / np.linalg.norm(dirs, axis=1, keepdims=True) * norms[:, None]
    return to_bf16(k.astype(np.float32))


# --- W3 / W4 / W5 -------------------------------------------------------------

def kv_rows(wid: int, tid: int, n_rows: int, d: int = 128, row0: int = 0, scale_cols=None):
    """Rows row0 .. row0+n_rows of an N(0,1) [*, d] bf16 tensor, drawn in
    blocks of 65536 rows so that any row range can be regenerated alone."""
    BLK = 65536
    out = np.empty((n_rows, d), dtype=np.float32)
    r = row0
    while r < row0 + n_rows:
        blk = r // BLK
        g = np.random.default_rng(np.random.SeedSequence([BASE_SEED, wid, tid, blk]))
        block = g.standard_normal((BLK, d), dtype=np.float32)
        lo = r - blk * BLK
        hi = min(BLK, row0 + n_rows - blk * BLK)
        out[r - row0:r - row0 + (hi - lo)] = block[lo:hi]
        r += hi - lo
    if scale_cols is not None:
        out = out * np.asarray(scale_cols, dtype=np.float32)[None, :]
    return to_bf16(out)


def w5_col_scale(d: int = 128):
    """Outlier channels 0..63 have std 10, channels 64..127 std 1."""
    s = np.ones(d, dtype=np.float32)
    s[: d // 2] = 10.0
    return s


def queries(wid: int, B: int, Hq: int, d: int = 128):
    return to_bf16(gaussian(wid, T_QUERIES, (B, Hq, d)))


def needle_positions(ctx: int):
    return [int(math.floor(f * ctx)) for f in NEEDLE_DEPTHS]


def w4_needles(q_vals: np.ndarray, Hkv: int, Hq: int, d: int = 128):
    """Needle keys for each KV head: 4 x the unit direction of the first query
    head of its group plus N(0, 0.1^2) noise, one per depth; bf16."""
    G = Hq // Hkv
    noise = gaussian(4, T_NEEDLE_NOISE, (Hkv, len(NEEDLE_DEPTHS), d), scale=0.1)
    out = np.empty((Hkv, len(NEEDLE_DEPTHS), d), dtype=np.float32)
    for h in range(Hkv):
        qv = q_vals[0, h * G].astype(np.float64)
        qhat = qv / np.linalg.norm(qv)
        out[h] = (4.0 * qhat)[None, :] + noise[h]
    return to_bf16(out)


# --- device-side generation for full-size workloads --------------------------------

def torch_generator(wid: int, tid: int, device):
    """torch generator on `device` seeded from (42, workload, tensor)."""
    import torch
    seed = int(np.random.SeedSequence([BASE_SEED, int(wid), int(tid)]).generate_state(1, dtype=np.uint64)[0]
               & 0x7FFFFFFFFFFFFFFF)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal_bf16_device(wid: int, tid: int, shape, device, scale_cols=None, chunk_rows=1 << 20):
    """N(0,1) float32 draws on the device, optionally scaled per column,
    rounded to bfloat16 (torch's conversion is round-to-nearest-even).
    Generated in row chunks to bound the float32 temporary."""
    import torch
    g = torch_generator(wid, tid, device)
    rows, d = int(np.prod(shape[:-1])), shape[-1]
    out = torch.empty((rows, d), dtype=torch.bfloat16, device=device)
    sc = None if scale_cols is None else torch.as_tensor(scale_cols, dtype=torch.float32, device=device)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        x = torch.randn((r1 - r0, d), generator=g, device=device, dtype=torch.float32)
        if sc is not None:
            x *= sc
        out[r0:r1] = x.to(torch.bfloat16)
    return out.reshape(*shape)


def w2_layer_keys_device(layer: int, device, heads: int = 2, n_tok: int = 32768, d: int = 128):
    """Device version of w2_layer_keys' recipe: N(0, I) direction scaled to a
    norm drawn log-uniform in [2, 20], bf16."""
    import torch
    g = torch_generator(2, 100 + layer, device)
    x = torch.randn((heads * n_tok, d), generator=g, device=device, dtype=torch.float32)
    u = torch.rand((heads * n_tok, 1), generator=g, device=device, dtype=torch.float32)
    norms = torch.exp(math.log(2.0) + u * (math.log(20.0) - math.log(2.0)))
    x = x / torch.linalg.vector_norm(x, dim=1, keepdim=True) * norms
    return x.to(torch.bfloat16)
