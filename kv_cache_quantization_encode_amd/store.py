"""Chunked compressed KV store on paged planes (plumbing only).

The store keeps one pool of pages per plane and a block table per sequence,
as the bit-packing article (section 五) describes for the compressed store:
new tokens are appended in chunks, already packed, and decode reads them in
place.  A page holds `page_size` consecutive tokens of every KV head; the
record of token t of (sequence b, KV head h) is

    (block_table[b][t // page_size] * Hkv + h) * page_size + t % page_size

This module only allocates pages, keeps the tables and computes those record
indices (slots); the quantisation and the attention run in libtq's kernels
(tq_append_kv, or tq_encode_keys / tq_encode_values, with slots;
tq_decode_attention_paged; tq_decode_attention_paged_append for a decode
step that appends its token in the same launch).
"""
from __future__ import annotations

import torch

from .api import Decoder, Tables, append_kv, encode_keys, encode_values, key_planes, value_planes


class PagedKVCache:
    """Compressed K/V for up to `max_seqs` sequences of at most
    `max_pages_per_seq * page_size` tokens, in a shared pool of `n_pages`."""

    def __init__(self, tables: Tables, Hkv: int, v_bits: int, n_pages: int, page_size: int = 256,
                 max_seqs: int = 1, max_pages_per_seq: int | None = None, device="cuda"):
        if page_size <= 0 or page_size % 64:
            raise ValueError("page_size must be a positive multiple of 64")
        self.tables, self.Hkv, self.v_bits = tables, Hkv, v_bits
        self.page_size, self.n_pages, self.max_seqs = page_size, n_pages, max_seqs
        self.max_pages_per_seq = max_pages_per_seq or n_pages
        self.device = device
        n_rec = n_pages * Hkv * page_size
        self.kp = key_planes(tables, n_rec, device)
        self.vp = value_planes(v_bits, n_rec, device=device)
        # unused entries point at page 0; the kernels never read past ctx_len
        self.block_table = torch.zeros((max_seqs, self.max_pages_per_seq), dtype=torch.int32, device=device)
        self._pages = [[] for _ in range(max_seqs)]      # host copy of each sequence's pages
        self._free = list(range(n_pages - 1, -1, -1))
        self.lengths = [0] * max_seqs

    @property
    def n_records(self) -> int:
        return self.n_pages * self.Hkv * self.page_size

    def memory_bytes(self) -> int:
        """Bytes of the packed planes (the whole pool)."""
        return sum(t.numel() * t.element_size() for t in list(self.kp.values()) + list(self.vp.values()))

    def _grow(self, seq: int, n_tokens: int):
        need = -(-n_tokens // self.page_size)
        if need > self.max_pages_per_seq:
            raise ValueError("sequence %d would exceed %d pages" % (seq, self.max_pages_per_seq))
        pages = self._pages[seq]
        new = []
        while len(pages) < need:
            if not self._free:
                raise RuntimeError("page pool exhausted")
            pages.append(self._free.pop())
            new.append(len(pages) - 1)
        if new:
            idx = torch.tensor(new, dtype=torch.long, device=self.device)
            self.block_table[seq, idx] = torch.tensor([pages[i] for i in new], dtype=torch.int32,
                                                      device=self.device)

    def slots(self, seq: int, t0: int, n: int) -> torch.Tensor:
        """Records of tokens t0 .. t0+n-1 of `seq`, rows ordered (token, KV head)."""
        P, H = self.page_size, self.Hkv
        t = torch.arange(t0, t0 + n, device=self.device, dtype=torch.long)
        page = self.block_table[seq].long()[t // P]
        h = torch.arange(H, device=self.device, dtype=torch.long)
        return ((page[:, None] * H + h[None, :]) * P + (t % P)[:, None]).reshape(-1).contiguous()

    def append(self, seq: int, k: torch.Tensor, v: torch.Tensor):
        """Encode a chunk of new tokens, k and v [n, Hkv, d] (float32 / bf16 /
        fp16), straight into the sequence's pages."""
        n = k.shape[0]
        if k.dim() != 3 or k.shape[1] != self.Hkv or v.shape != k.shape:
            raise ValueError("k and v must both be [n, Hkv=%d, d]" % self.Hkv)
        t0 = self.lengths[seq]
        self._grow(seq, t0 + n)
        sl = self.slots(seq, t0, n)
        kr, vr = k.reshape(n * self.Hkv, -1), v.reshape(n * self.Hkv, -1)
        if kr.dtype == vr.dtype:  # one launch for both
            append_kv(self.tables, kr, vr, self.v_bits, self.kp, self.vp, slots=sl, n_records=self.n_records)
        else:
            encode_keys(self.tables, kr, self.kp, slots=sl, n_records=self.n_records)
            encode_values(vr, self.v_bits, planes=self.vp, slots=sl, n_records=self.n_records)
        self.lengths[seq] = t0 + n

    def decoder(self, B: int, Hq: int, q_dtype=torch.bfloat16) -> Decoder:
        return Decoder(self.tables, B, Hq, self.Hkv, self.max_pages_per_seq * self.page_size, self.v_bits,
                       q_dtype, self.device, page_size=self.page_size)

    def decode(self, q: torch.Tensor, seqs=None, dec: Decoder | None = None, **kw):
        """One decode step for the sequences `seqs` (default 0 .. B-1): q is
        [B, Hq, d]; returns out [B, Hq, d] float32."""
        B, Hq, _ = q.shape
        seqs = list(range(B)) if seqs is None else list(seqs)
        dec = dec or self.decoder(B, Hq, q.dtype)
        ctx = torch.tensor([self.lengths[s] for s in seqs], dtype=torch.int32, device=self.device)
        bt = self.block_table[torch.tensor(seqs, dtype=torch.long, device=self.device)].contiguous()
        return dec(q, ctx, self.kp, self.vp, block_table=bt, **kw)

    def decode_step(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seqs=None, dec: Decoder | None = None,
                    **kw):
        """One decode step that appends one token per sequence: k and v are
        [B, Hkv, d] (one dtype of float32 / bf16 / fp16), q is [B, Hq, d].  The
        token is encoded into its page and attended in one launch
        (tq_decode_attention_paged_append); returns out [B, Hq, d] float32."""
        B, Hq, _ = q.shape
        seqs = list(range(B)) if seqs is None else list(seqs)
        if tuple(k.shape[:2]) != (B, self.Hkv) or v.shape != k.shape:
            raise ValueError("k and v must both be [B, Hkv=%d, d]" % self.Hkv)
        for s in seqs:
            self._grow(s, self.lengths[s] + 1)
        for s in seqs:
            self.lengths[s] += 1
        dec = dec or self.decoder(B, Hq, q.dtype)
        ctx = torch.tensor([self.lengths[s] for s in seqs], dtype=torch.int32, device=self.device)
        bt = self.block_table[torch.tensor(seqs, dtype=torch.long, device=self.device)].contiguous()
        return dec(q, ctx, self.kp, self.vp, block_table=bt, k_new=k, v_new=v, **kw)
