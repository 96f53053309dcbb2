"""Attention-quality metrics and memory accounting for synthetic workloads.

The pages report compressed-cache quality as cosine similarity of attention
outputs, distribution distance of the attention weights, top-k agreement and
memory per token across bit widths (the difai.kr tutorial's comparison table;
validate_paper.py's test_recall_at_scale and rank-correlation checks; the
bit-packing article sec 四's 52-byte record against 256 bytes of fp16).  These
helpers measure the same quantities for the HIP path against exact attention
computed with plain float32 torch on the same device (the reference, not part
of the path).
"""
from __future__ import annotations

import math

import torch

from .api import Decoder, Tables, encode_keys, encode_values
from ._lib import key_config

FP16_BYTES_PER_TOKEN_HEAD = 2 * 128 * 2  # K and V, fp16, head dim 128


def key_record_bytes(mode: str, bits: int = 3, bits_outlier: int = 4, bits_normal: int = 2, d: int = 128) -> int:
    """Bytes of one packed key (index row, signs, fp16 norms)."""
    width = lambda b: 1 if b == 1 else 2 if b == 2 else 4 if b <= 4 else 8  # noqa: E731
    if mode in ("grouped", "grouped_prod"):
        b = d // 2 * width(bits_outlier) // 8 + d // 2 * width(bits_normal) // 8 + 4
        return b + (d // 8 + 2 if mode == "grouped_prod" else 0)
    if mode == "prod":
        return d * width(bits - 1) // 8 + d // 8 + 4
    return d * width(bits) // 8 + 2


def value_record_bytes(bits: int, d: int = 128, group: int = 32) -> int:
    return d * bits // 8 + 4 * (d // group)


def memory_table(contexts=(1024, 4096, 16384, 32768, 65536, 131072), kv_heads: int = 8, layers: int = 28,
                 configs=(("prod", 3, 2), ("prod", 4, 4), ("mse", 4, 4), ("grouped", None, 4))):
    """KV-cache bytes per sequence for each (key mode, key bits, value bits)
    configuration against fp16, over a range of context lengths."""
    rows = []
    for ctx in contexts:
        base = ctx * kv_heads * layers * FP16_BYTES_PER_TOKEN_HEAD
        for mode, kb, vb in configs:
            per = key_record_bytes(mode, kb or 3) + value_record_bytes(vb)
            total = ctx * kv_heads * layers * per
            rows.append(dict(context=ctx, key_mode=mode, key_bits=kb, value_bits=vb, bytes=total,
                             fp16_bytes=base, ratio=base / total))
    return rows


@torch.no_grad()
def attention_quality(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, key_cfg: dict, v_bits: int,
                      seed: int = 42, topk: int = 5, per_head: bool = False) -> dict:
    """q [B, Hq, d], k and v [B, Hkv, N, d] (any float dtype, on the GPU).
    Encodes k and v with the HIP path, runs one decode step returning scores,
    and compares with exact float32 attention:
      score_cosine mean cosine similarity of the score vectors q.k vs q.k_hat
      out_cosine   mean cosine similarity of attention outputs
      kl           mean KL(p_exact || p_quant) of the attention weights
      top1         fraction of heads whose highest-scoring token agrees
      topk_overlap mean |top-k exact & top-k quant| / k
      score_rel_rms  RMS of the score error over the RMS of the exact scores
    With per_head, also "heads": the per-head values ([B, Hq] arrays on the
    host), the quantised scores and the decoded outputs."""
    B, Hq, d = q.shape
    _, Hkv, N, _ = k.shape
    G = Hq // Hkv
    dev = q.device
    T = Tables(key_config(seed=seed, **key_cfg), dev)
    kp = encode_keys(T, k.reshape(-1, d).contiguous())
    vp = encode_values(v.reshape(-1, d).contiguous(), v_bits)
    dec = Decoder(T, B, Hq, Hkv, N, v_bits, q.dtype, dev)
    scores = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    out = dec(q.contiguous(), torch.full((B,), N, dtype=torch.int32, device=dev), kp, vp, scores=scores)
    # exact float32 attention (GQA: query head h reads KV head h // G)
    kf = k.float().repeat_interleave(G, dim=1)                      # [B, Hq, N, d]
    vf = v.float().repeat_interleave(G, dim=1)
    s_ex = torch.matmul(kf, q.float().unsqueeze(-1)).squeeze(-1)    # [B, Hq, N]
    scale = 1.0 / math.sqrt(d)
    p_ex = torch.softmax(s_ex * scale, dim=-1)
    o_ex = torch.matmul(p_ex.unsqueeze(-2), vf).squeeze(-2)
    logp_q = torch.log_softmax(scores * scale, dim=-1)
    kl = torch.sum(p_ex * (torch.log(p_ex.clamp_min(1e-30)) - logp_q), dim=-1)
    cos = torch.nn.functional.cosine_similarity(out, o_ex, dim=-1)
    scos = torch.nn.functional.cosine_similarity(scores, s_ex, dim=-1)
    top_ex = torch.topk(s_ex, topk, dim=-1).indices
    top_q = torch.topk(scores, topk, dim=-1).indices
    overlap = (top_ex.unsqueeze(-1) == top_q.unsqueeze(-2)).any(-1).float().sum(-1) / topk
    top1 = (top_ex[..., 0] == top_q[..., 0]).float()
    rel = torch.sqrt(torch.mean((scores - s_ex) ** 2) / torch.mean(s_ex ** 2))
    res = dict(score_cosine=float(scos.mean()), out_cosine=float(cos.mean()), kl=float(kl.mean()),
               top1=float(top1.mean()), topk_overlap=float(overlap.mean()), score_rel_rms=float(rel))
    if per_head:
        res["heads"] = dict(score_cosine=scos.cpu().numpy(), out_cosine=cos.cpu().numpy(), kl=kl.cpu().numpy(),
                            top1=top1.cpu().numpy(), topk_overlap=overlap.cpu().numpy(),
                            err2=torch.sum((scores - s_ex) ** 2, dim=-1).cpu().numpy(),
                            ref2=torch.sum(s_ex ** 2, dim=-1).cpu().numpy(), scores=scores.cpu().numpy(),
                            out=out.cpu().numpy())
    return res
