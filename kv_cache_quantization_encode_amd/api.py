"""Thin Python API over libtq's C ABI.  torch supplies device memory and the
current HIP stream; every computation happens in the library's kernels."""
from __future__ import annotations

import ctypes
import math
import struct

import numpy as np
import torch

from ._lib import (TQ_BF16, TQ_F16, TQ_F32, TQ_MODE_GROUPED, TQ_MODE_GROUPED_PROD, TQ_MODE_PROD,
                   TQ_STREAM_READ_SINK, KeyBatch, KeyConfig, check,
                   key_config, lib)

_DT = {torch.float32: TQ_F32, torch.bfloat16: TQ_BF16, torch.float16: TQ_F16}

# tq_blob_header (kv_cache_quantization_encode_amd/csrc/tq_tables.h)
_HDR = struct.Struct("<4I4i" + "2i2i2i" + "2I2I2I2I" + "2i2f2f" + "2I" + "2d")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


# ---- argument checks.  The C ABI checks pointers, alignment and sizes it is
# given, but it cannot see how large a tensor is: these checks keep every
# buffer the kernels touch inside the tensors passed in.

def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _on_device(t, name, dtypes=None, contiguous=False):
    if not isinstance(t, torch.Tensor):
        raise ValueError("%s must be a torch tensor" % name)
    dev = t.get_device()
    if dev < 0:
        raise ValueError("%s must be on the GPU" % name)
    if dev != torch.cuda.current_device():
        raise ValueError("%s is on cuda:%d but the current device is cuda:%d" % (name, dev,
                                                                              torch.cuda.current_device()))
    if dtypes is not None:
        dtypes = dtypes if isinstance(dtypes, (tuple, list)) else (dtypes,)
        if t.dtype not in dtypes:
            raise ValueError("%s has dtype %s, expected one of %s" % (name, t.dtype, list(dtypes)))
    if contiguous and not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _check_rows(x, name, d=128):
    _on_device(x, name, tuple(_DT))
    _need(x.dim() == 2 and x.shape[1] == d and x.stride(1) == 1,
          "%s must be [n, %d] with unit channel stride, got shape %s strides %s" % (name, d, tuple(x.shape),
                                                                                 x.stride()))


def _check_slots(slots, n, name="slots"):
    if slots is not None:
        _on_device(slots, name, torch.int64, contiguous=True)
        _need(slots.numel() == n, "%s has %d entries for %d rows" % (name, slots.numel(), n))


def _grouped(mode) -> bool:
    return mode in (TQ_MODE_GROUPED, TQ_MODE_GROUPED_PROD)


def _qjl(mode) -> bool:
    return mode in (TQ_MODE_PROD, TQ_MODE_GROUPED_PROD)


def _check_key_planes(tables, p, n_records):
    mode = tables.mode
    d = tables.cfg.d
    _on_device(p["idx"], "idx plane", torch.uint8, contiguous=True)
    _need(p["idx"].numel() >= n_records * tables.row_bytes,
          "idx plane holds %d bytes, %d records need %d" % (p["idx"].numel(), n_records,
                                                           n_records * tables.row_bytes))
    _on_device(p["norm"], "norm plane", torch.float16, contiguous=True)
    _need(p["norm"].numel() >= n_records * (2 if _grouped(mode) else 1), "norm plane too small")
    if _qjl(mode):
        _need(p.get("signs") is not None and p.get("rnorm") is not None, "QJL keys need signs and rnorm planes")
        _on_device(p["signs"], "signs plane", torch.uint8, contiguous=True)
        _need(p["signs"].numel() >= n_records * (d // 8), "signs plane too small")
        _on_device(p["rnorm"], "rnorm plane", torch.float16, contiguous=True)
        _need(p["rnorm"].numel() >= n_records, "rnorm plane too small")
    else:
        _need(p.get("signs") is None and p.get("rnorm") is None, "only QJL keys have signs and rnorm planes")


def _check_value_planes(p, bits, n_records, d=128, group=32):
    _on_device(p["codes"], "codes plane", torch.uint8, contiguous=True)
    _need(p["codes"].numel() >= n_records * d * bits // 8, "codes plane too small for %d records" % n_records)
    for k in ("scale", "zero"):
        _on_device(p[k], "%s plane" % k, torch.float16, contiguous=True)
        _need(p[k].numel() >= n_records * (d // group), "%s plane too small for %d records" % (k, n_records))


def _records(planes: dict, key: str, per_record: int) -> int:
    return planes[key].numel() // per_record


def idx_row_bytes(cfg: KeyConfig) -> int:
    return int(lib.tq_idx_row_bytes(ctypes.byref(cfg)))


def build_codebook(cfg: KeyConfig):
    """Host call: returns (blob as uint8 numpy array, list of mse_total)."""
    size = ctypes.c_size_t(0)
    mse = (ctypes.c_double * 2)()
    check("tq_build_codebook", lib.tq_build_codebook(ctypes.byref(cfg), None, ctypes.byref(size), mse))
    buf = np.zeros(size.value, dtype=np.uint8)
    check("tq_build_codebook", lib.tq_build_codebook(ctypes.byref(cfg), buf.ctypes.data_as(ctypes.c_void_p),
                                                      ctypes.byref(size), mse))
    n = 2 if _grouped(cfg.mode) else 1
    return buf, [mse[i] for i in range(n)]


def parse_tables(blob: np.ndarray) -> dict:
    """Decode the blob's header and arrays on the host (inspection and tests)."""
    f = _HDR.unpack_from(blob.tobytes(), 0)
    h = dict(magic=f[0], version=f[1], total_bytes=f[2], header_bytes=f[3], d=f[4], mode=f[5],
             m=f[6], n_parts=f[7], part_d=f[8:10], part_bits=f[10:12], part_levels=f[12:14],
             off_centroids=f[14:16], off_bounds=f[16:18], off_sigma=f[18:20], off_hint=f[20:22],
             hint_n=f[22:24], hint_lo=f[24:26], hint_scale=f[26:28], off_S=f[28], mse=f[30:32])
    parts = []
    for i in range(h["n_parts"]):
        L = h["part_levels"][i]
        c = blob[h["off_centroids"][i]:h["off_centroids"][i] + 4 * L].view(np.float32)
        t = blob[h["off_bounds"][i]:h["off_bounds"][i] + 4 * (L + 1)].view(np.float32)
        s = blob[h["off_sigma"][i]:h["off_sigma"][i] + 4 * h["part_d"][i]].view(np.float32)
        hint = blob[h["off_hint"][i]:h["off_hint"][i] + 16 * h["hint_n"][i]].view(np.int32).reshape(-1, 4)
        parts.append(dict(centroids=c.copy(), bounds=t.copy(), sigma=s.copy(), hint=hint.copy()))
    h["parts"] = parts
    if h["m"] > 0:
        n = h["m"] * h["d"]
        h["S"] = blob[h["off_S"]:h["off_S"] + 2 * n].view(np.float16).reshape(h["m"], h["d"]).copy()
    return h


class Tables:
    """Seed-derived tables of one key configuration, resident on a device."""

    def __init__(self, cfg: KeyConfig, device="cuda"):
        self.cfg = cfg
        blob, self.mse = build_codebook(cfg)
        self.blob = blob
        self.dev = torch.from_numpy(blob).to(device)
        self.row_bytes = idx_row_bytes(cfg)

    @property
    def mode(self):
        return self.cfg.mode


def key_planes(tables: Tables, n_records: int, device="cuda") -> dict:
    d = tables.cfg.d
    p = dict(idx=torch.empty((n_records, tables.row_bytes), dtype=torch.uint8, device=device))
    if _grouped(tables.mode):
        p["norm"] = torch.empty((n_records, 2), dtype=torch.float16, device=device)
    else:
        p["norm"] = torch.empty((n_records,), dtype=torch.float16, device=device)
    if _qjl(tables.mode):
        p["signs"] = torch.empty((n_records, d // 8), dtype=torch.uint8, device=device)
        p["rnorm"] = torch.empty((n_records,), dtype=torch.float16, device=device)
    return p


def value_planes(bits: int, n_records: int, d=128, group=32, device="cuda") -> dict:
    return dict(codes=torch.empty((n_records, d * bits // 8), dtype=torch.uint8, device=device),
                scale=torch.empty((n_records, d // group), dtype=torch.float16, device=device),
                zero=torch.empty((n_records, d // group), dtype=torch.float16, device=device))


def encode_keys(tables: Tables, keys: torch.Tensor, planes: dict | None = None, slots=None,
                n_records: int | None = None) -> dict:
    """keys: [n, d] float32/bfloat16/float16 CUDA tensor (rows may be strided)."""
    _check_rows(keys, "keys", tables.cfg.d)
    n = keys.shape[0]
    if n_records is None:
        n_records = n if planes is None else _records(planes, "idx", tables.row_bytes)
    if planes is None:
        planes = key_planes(tables, n_records, keys.device)
    _check_key_planes(tables, planes, n_records)
    _check_slots(slots, n)
    _need(slots is not None or n <= n_records, "%d rows do not fit in %d records" % (n, n_records))
    st = lib.tq_encode_keys(ctypes.byref(tables.cfg), _ptr(tables.dev), _ptr(keys), _DT[keys.dtype],
                            n, keys.stride(0), _ptr(slots), n_records, _ptr(planes["idx"]),
                            _ptr(planes.get("signs")), _ptr(planes["norm"]), _ptr(planes.get("rnorm")),
                            _stream())
    check("tq_encode_keys", st)
    return planes


def encode_values(values: torch.Tensor, bits: int, group: int = 32, planes: dict | None = None,
                  slots=None, n_records: int | None = None) -> dict:
    _check_rows(values, "values", values.shape[-1] if values.dim() == 2 else 128)
    n, d = values.shape
    _need(bits in (2, 4), "value bits must be 2 or 4")
    if n_records is None:
        n_records = n if planes is None else _records(planes, "codes", d * bits // 8)
    if planes is None:
        planes = value_planes(bits, n_records, d, group, values.device)
    _check_value_planes(planes, bits, n_records, d, group)
    _check_slots(slots, n)
    _need(slots is not None or n <= n_records, "%d rows do not fit in %d records" % (n, n_records))
    st = lib.tq_encode_values(bits, group, d, _ptr(values), _DT[values.dtype], n, values.stride(0),
                              _ptr(slots), n_records, _ptr(planes["codes"]), _ptr(planes["scale"]),
                              _ptr(planes["zero"]), _stream())
    check("tq_encode_values", st)
    return planes


class KeyBatchEncoder:
    """A prepared tq_encode_keys_batched launch: the key sets (e.g. the layers
    of a prefill, each with its own Tables of one config), their output planes
    and slot maps are checked once here; each call then only enqueues the
    launch on the current stream (the tensors must stay alive and unchanged
    in shape).  keys: list of [n, d] tensors of one shape, dtype and stride."""

    def __init__(self, tables: list, keys: list, planes: list | None = None, slots: list | None = None,
                 n_records: int | None = None):
        nb = len(tables)
        _need(nb == len(keys) and 0 < nb <= 32, "need 1..32 key sets, one Tables per set")
        k0 = keys[0]
        for i, k in enumerate(keys):
            _check_rows(k, "keys[%d]" % i, tables[0].cfg.d)
            _need(k.shape == k0.shape and k.dtype == k0.dtype and k.stride() == k0.stride(),
                  "every key set needs the shape, dtype and strides of the first")
            _need(tables[i].mode == tables[0].mode and tables[i].row_bytes == tables[0].row_bytes,
                  "every Tables must have the first one's mode and widths")
        n = k0.shape[0]
        if planes is None:
            rec = n if n_records is None else n_records
            planes = [key_planes(t, rec, k0.device) for t in tables]
        if n_records is None:
            n_records = min(_records(pl, "idx", tables[0].row_bytes) for pl in planes)
        slots = slots or [None] * nb
        _need(len(planes) == nb and len(slots) == nb, "one plane dict and one slot map (or None) per set")
        for t, pl, sl in zip(tables, planes, slots):
            _check_key_planes(t, pl, n_records)
            _check_slots(sl, n)
            _need(sl is not None or n <= n_records, "%d rows do not fit in %d records" % (n, n_records))
        self.planes = planes
        self._keep = (list(tables), list(keys), list(slots))
        self._arr = (KeyBatch * nb)(*[KeyBatch(_ptr(t.dev), _ptr(k), _ptr(sl), _ptr(p["idx"]),
                                               _ptr(p.get("signs")), _ptr(p["norm"]), _ptr(p.get("rnorm")))
                                      for t, k, p, sl in zip(tables, keys, planes, slots)])
        self._args = (ctypes.byref(tables[0].cfg), self._arr, nb, _DT[k0.dtype], n, k0.stride(0), n_records)

    def __call__(self) -> list:
        check("tq_encode_keys_batched", lib.tq_encode_keys_batched(*self._args, _stream()))
        return self.planes


def encode_keys_batched(tables: list, keys: list, planes: list | None = None, slots: list | None = None,
                        n_records: int | None = None) -> list:
    """tq_encode_keys for several key sets (e.g. the layers of a prefill, each
    with its own Tables of one config) in one launch; returns (or fills) one
    plane dict per set, equal to what encode_keys writes.  For repeated
    launches over the same tensors, KeyBatchEncoder checks them once."""
    return KeyBatchEncoder(tables, keys, planes, slots, n_records)()


def append_kv(tables: Tables, keys: torch.Tensor, values: torch.Tensor, v_bits: int, kp: dict, vp: dict,
              slots=None, n_records: int | None = None, group: int = 32):
    """Encode keys and values [n, d] (same dtype) of the same tokens into the
    key planes kp and value planes vp in one launch (tq_append_kv); the
    planes equal those of encode_keys + encode_values."""
    _check_rows(keys, "keys", tables.cfg.d)
    _check_rows(values, "values", tables.cfg.d)
    _need(keys.shape == values.shape and keys.dtype == values.dtype, "keys and values need one shape and dtype")
    _need(v_bits in (2, 4), "value bits must be 2 or 4")
    n = keys.shape[0]
    if n_records is None:
        n_records = min(_records(kp, "idx", tables.row_bytes), _records(vp, "codes", tables.cfg.d * v_bits // 8))
    _check_key_planes(tables, kp, n_records)
    _check_value_planes(vp, v_bits, n_records, tables.cfg.d, group)
    _check_slots(slots, n)
    _need(slots is not None or n <= n_records, "%d rows do not fit in %d records" % (n, n_records))
    st = lib.tq_append_kv(ctypes.byref(tables.cfg), _ptr(tables.dev), _ptr(keys), _ptr(values),
                          _DT[keys.dtype], n, keys.stride(0), values.stride(0), _ptr(slots), n_records,
                          _ptr(kp["idx"]), _ptr(kp.get("signs")), _ptr(kp["norm"]), _ptr(kp.get("rnorm")),
                          v_bits, group, _ptr(vp["codes"]), _ptr(vp["scale"]), _ptr(vp["zero"]), _stream())
    check("tq_append_kv", st)


def dequantize_keys(tables: Tables, planes: dict, n_vec: int | None = None, slots=None,
                    dtype=torch.float32, out=None):
    """Dense k_hat [n_vec, d] from the key planes (rows `slots`, or 0..n_vec-1)."""
    n_records = _records(planes, "idx", tables.row_bytes)
    _check_key_planes(tables, planes, n_records)
    if n_vec is None:
        n_vec = n_records if slots is None else slots.shape[0]
    _check_slots(slots, n_vec)
    _need(slots is not None or n_vec <= n_records, "%d rows exceed the %d records" % (n_vec, n_records))
    if out is None:
        out = torch.empty((n_vec, tables.cfg.d), dtype=dtype, device=planes["idx"].device)
    _check_rows(out, "out", tables.cfg.d)
    _need(out.shape[0] >= n_vec, "out has fewer than %d rows" % n_vec)
    st = lib.tq_dequantize_keys(ctypes.byref(tables.cfg), _ptr(tables.dev), n_vec, _ptr(slots), n_records,
                                _ptr(planes["idx"]), _ptr(planes.get("signs")), _ptr(planes["norm"]),
                                _ptr(planes.get("rnorm")), _ptr(out), _DT[out.dtype], out.stride(0), _stream())
    check("tq_dequantize_keys", st)
    return out


def dequantize_values(planes: dict, bits: int, n_vec: int | None = None, slots=None, dtype=torch.float32,
                      out=None, group: int = 32):
    """Dense v_hat [n_vec, d] from the value planes."""
    _need(bits in (2, 4), "value bits must be 2 or 4")
    d = planes["codes"].shape[1] * 8 // bits if planes["codes"].dim() == 2 else 128
    n_records = _records(planes, "codes", d * bits // 8)
    _check_value_planes(planes, bits, n_records, d, group)
    if n_vec is None:
        n_vec = n_records if slots is None else slots.shape[0]
    _check_slots(slots, n_vec)
    _need(slots is not None or n_vec <= n_records, "%d rows exceed the %d records" % (n_vec, n_records))
    if out is None:
        out = torch.empty((n_vec, d), dtype=dtype, device=planes["codes"].device)
    _check_rows(out, "out", d)
    _need(out.shape[0] >= n_vec, "out has fewer than %d rows" % n_vec)
    st = lib.tq_dequantize_values(bits, group, d, n_vec, _ptr(slots), n_records, _ptr(planes["codes"]),
                                  _ptr(planes["scale"]), _ptr(planes["zero"]), _ptr(out), _DT[out.dtype],
                                  out.stride(0), _stream())
    check("tq_dequantize_values", st)
    return out


def channel_moments(x: torch.Tensor) -> torch.Tensor:
    """float64 [2, d]: per-channel sum and sum of squares of the rows of x [n, d]."""
    _check_rows(x, "x", x.shape[-1] if x.dim() == 2 else 128)
    n, d = x.shape
    size = ctypes.c_size_t(0)
    check("tq_channel_moments", lib.tq_channel_moments(None, _DT[x.dtype], n, x.stride(0), d, None, None,
                                                       ctypes.byref(size), None))
    ws = torch.empty(max(size.value, 8), dtype=torch.uint8, device=x.device)
    out = torch.empty((2, d), dtype=torch.float64, device=x.device)
    size = ctypes.c_size_t(ws.numel())
    check("tq_channel_moments", lib.tq_channel_moments(_ptr(x), _DT[x.dtype], n, x.stride(0), d, _ptr(out),
                                                       _ptr(ws), ctypes.byref(size), _stream()))
    return out


def stream_read(src: torch.Tensor, sink: torch.Tensor) -> None:
    """One nontemporal streaming pass over src's bytes (tq_stream_read), the
    read-bandwidth reference the decode's roofline is set against; sink is a
    device int32/uint32 tensor of TQ_STREAM_READ_SINK elements."""
    if not src.is_cuda or not src.is_contiguous() or not sink.is_cuda or sink.numel() < TQ_STREAM_READ_SINK:
        raise ValueError("stream_read: contiguous device src and a device sink of %d words" % TQ_STREAM_READ_SINK)
    if sink.element_size() != 4:
        raise ValueError("stream_read: sink must hold 32-bit words")
    check("tq_stream_read", lib.tq_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream()))


def select_outlier_channels(x: torch.Tensor, n_outlier: int = 64) -> torch.Tensor:
    """Channel order for the grouped modes (tq_select_outlier_channels): the
    n_outlier highest-variance channels of the key rows x [n, d] first, then
    the rest (each in channel order), int64 on x's device.  Apply it to keys
    and queries alike: k[:, perm], q[..., perm]."""
    _check_rows(x, "x", x.shape[-1] if x.dim() == 2 else 128)
    n, d = x.shape
    size = ctypes.c_size_t(0)
    check("tq_select_outlier_channels", lib.tq_select_outlier_channels(None, _DT[x.dtype], n, x.stride(0), d,
                                                                       n_outlier, None, None, ctypes.byref(size),
                                                                       None))
    ws = torch.empty(max(size.value, 8), dtype=torch.uint8, device=x.device)
    perm = torch.empty(d, dtype=torch.int32, device=x.device)
    size = ctypes.c_size_t(ws.numel())
    check("tq_select_outlier_channels", lib.tq_select_outlier_channels(_ptr(x), _DT[x.dtype], n, x.stride(0), d,
                                                                       n_outlier, _ptr(perm), _ptr(ws),
                                                                       ctypes.byref(size), _stream()))
    return perm.long()


def decode_workspace_bytes(tables: Tables, B, Hq, Hkv, max_ctx, q_dtype=torch.bfloat16, v_bits=2,
                           page_size=None) -> int:
    """Workspace size of tq_decode_attention (or, with page_size, of
    tq_decode_attention_paged with max_ctx // page_size blocks per sequence)."""
    size = ctypes.c_size_t(0)
    keys = (None, None, None, None, v_bits, 32, None, None, None, ctypes.c_float(1.0), None, None, None,
            None, ctypes.byref(size), None)
    if page_size is None:
        st = lib.tq_decode_attention(ctypes.byref(tables.cfg), None, None, _DT[q_dtype], B, Hq, Hkv, None,
                                     max_ctx, *keys)
        check("tq_decode_attention", st)
    else:
        st = lib.tq_decode_attention_paged(ctypes.byref(tables.cfg), None, None, _DT[q_dtype], B, Hq, Hkv,
                                           None, None, max_ctx // page_size, page_size, 1, *keys)
        check("tq_decode_attention_paged", st)
    return size.value


class Decoder:
    """Holds the workspace for repeated decode steps of one shape.  With
    page_size set, the planes are a paged pool and each call passes the block
    table ([B, max_ctx // page_size] int32)."""

    def __init__(self, tables: Tables, B, Hq, Hkv, max_ctx, v_bits, q_dtype=torch.bfloat16,
                 device="cuda", page_size=None):
        self.tables, self.B, self.Hq, self.Hkv, self.max_ctx, self.v_bits = tables, B, Hq, Hkv, max_ctx, v_bits
        self.page_size = page_size
        if page_size is not None:
            _need(page_size > 0 and max_ctx % page_size == 0, "max_ctx must be a multiple of page_size")
        self.ws_bytes = decode_workspace_bytes(tables, B, Hq, Hkv, max_ctx, q_dtype, v_bits, page_size)
        self.ws = torch.empty(max(self.ws_bytes, 16), dtype=torch.uint8, device=device)

    def __call__(self, q, ctx_len, kp: dict, vp: dict, sm_scale=None, out=None, lse=None,
                 scores=None, block_table=None, k_new=None, v_new=None):
        """One decode step.  With k_new and v_new ([B, Hkv, d], one dtype of
        float32 / bfloat16 / float16) the step first appends them as token
        ctx_len[b] - 1 of each sequence (tq_decode_attention_append: encoded,
        stored into the planes and attended, in the same launch)."""
        return self.bind(q, ctx_len, kp, vp, sm_scale, out, lse, scores, block_table, k_new, v_new)()

    def bind(self, q, ctx_len, kp: dict, vp: dict, sm_scale=None, out=None, lse=None,
             scores=None, block_table=None, k_new=None, v_new=None):
        """Checks the arguments of one decode step (as __call__ takes them) once
        and returns a function of no arguments that enqueues that step on the
        stream current now, on the same tensors, and returns out: for loops
        that repeat a step without paying the checks each time.  The tensors
        must stay alive and in place while the function is used."""
        _on_device(q, "q", tuple(_DT), contiguous=True)
        _need(q.dim() == 3, "q must be [B, Hq, d]")
        B, Hq, d = q.shape
        _need((B, Hq, d) == (self.B, self.Hq, self.tables.cfg.d), "q shape %s does not match the decoder's"
              % (tuple(q.shape),))
        _on_device(ctx_len, "ctx_len", torch.int32, contiguous=True)
        _need(ctx_len.numel() == B, "ctx_len needs one entry per sequence")
        if sm_scale is None:
            sm_scale = 1.0 / math.sqrt(d)
        if out is None:
            out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
        _on_device(out, "out", torch.float32, contiguous=True)
        _need(out.numel() >= B * Hq * d, "out must hold [B, Hq, d]")
        if lse is not None:
            _on_device(lse, "lse", torch.float32, contiguous=True)
            _need(lse.numel() >= B * Hq, "lse must hold [B, Hq]")
        if scores is not None:
            _on_device(scores, "scores", torch.float32, contiguous=True)
            _need(scores.numel() >= B * Hq * self.max_ctx, "scores must hold [B, Hq, max_ctx]")
        n_rec = min(_records(kp, "idx", self.tables.row_bytes), _records(vp, "codes", d * self.v_bits // 8))
        if self.page_size is None:
            _need(n_rec >= B * self.Hkv * self.max_ctx, "the planes hold %d records, B * Hkv * max_ctx = %d"
                  % (n_rec, B * self.Hkv * self.max_ctx))
        _check_key_planes(self.tables, kp, n_rec)
        _check_value_planes(vp, self.v_bits, n_rec, d)
        size = ctypes.c_size_t(self.ws.numel())
        keys = (_ptr(kp["idx"]), _ptr(kp.get("signs")), _ptr(kp["norm"]), _ptr(kp.get("rnorm")))
        vals = (self.v_bits, 32, _ptr(vp["codes"]), _ptr(vp["scale"]), _ptr(vp["zero"]))
        tail = (ctypes.c_float(sm_scale), _ptr(out), _ptr(lse), _ptr(scores), _ptr(self.ws),
                ctypes.byref(size), _stream())
        appending = k_new is not None or v_new is not None
        if appending:
            for name, t in (("k_new", k_new), ("v_new", v_new)):
                _on_device(t, name, tuple(_DT), contiguous=True)
                _need(tuple(t.shape) == (B, self.Hkv, d), "%s must be [B, Hkv, d]" % name)
            _need(k_new.dtype == v_new.dtype, "k_new and v_new must have one dtype")
            new = (_ptr(k_new), _ptr(v_new), _DT[k_new.dtype])
        head = (ctypes.byref(self.tables.cfg), _ptr(self.tables.dev), _ptr(q), _DT[q.dtype], B, Hq, self.Hkv,
                _ptr(ctx_len))
        if self.page_size is None:
            _need(block_table is None, "a contiguous decoder takes no block table")
            if appending:
                name, fn = "tq_decode_attention_append", lib.tq_decode_attention_append
                args = head + (self.max_ctx,) + new + keys + vals + tail
            else:
                name, fn = "tq_decode_attention", lib.tq_decode_attention
                args = head + (self.max_ctx,) + keys + vals + tail
        else:
            nb = self.max_ctx // self.page_size
            _need(block_table is not None, "a paged decoder needs the block table")
            _on_device(block_table, "block_table", torch.int32, contiguous=True)
            _need(tuple(block_table.shape) == (B, nb), "block_table must be [B, max_ctx // page_size]")
            # pages of the pool: the planes' records over the records of one page
            n_pages = n_rec // (self.Hkv * self.page_size)
            _need(n_pages > 0, "the planes hold less than one page")
            paged = (_ptr(block_table), nb, self.page_size, n_pages)
            if appending:
                name, fn = "tq_decode_attention_paged_append", lib.tq_decode_attention_paged_append
                args = head + paged + new + keys + vals + tail
            else:
                name, fn = "tq_decode_attention_paged", lib.tq_decode_attention_paged
                args = head + paged + keys + vals + tail

        def run():
            check(name, fn(*args))
            return out
        return run


def decode_attention_noalloc(tables: Tables, q, ctx_len, kp: dict, vp: dict, v_bits: int, max_ctx: int,
                             Hkv: int, out, sm_scale=None, lse=None, scores=None):
    """tq_decode_attention_noalloc: the decode step without a workspace (the
    library's own per-GPU array holds the split-K partials), for callers that
    cannot allocate.  out [B, Hq, d] float32 (and lse / scores, if given) are
    the caller's; nothing is allocated here either."""
    _on_device(q, "q", tuple(_DT), contiguous=True)
    _need(q.dim() == 3, "q must be [B, Hq, d]")
    B, Hq, d = q.shape
    _need(d == tables.cfg.d, "q has head dim %d, the tables %d" % (d, tables.cfg.d))
    _on_device(ctx_len, "ctx_len", torch.int32, contiguous=True)
    _need(ctx_len.numel() == B, "ctx_len needs one entry per sequence")
    _on_device(out, "out", torch.float32, contiguous=True)
    _need(out.numel() >= B * Hq * d, "out must hold [B, Hq, d]")
    if lse is not None:
        _on_device(lse, "lse", torch.float32, contiguous=True)
        _need(lse.numel() >= B * Hq, "lse must hold [B, Hq]")
    if scores is not None:
        _on_device(scores, "scores", torch.float32, contiguous=True)
        _need(scores.numel() >= B * Hq * max_ctx, "scores must hold [B, Hq, max_ctx]")
    n_rec = min(_records(kp, "idx", tables.row_bytes), _records(vp, "codes", d * v_bits // 8))
    _need(n_rec >= B * Hkv * max_ctx, "the planes hold %d records, B * Hkv * max_ctx = %d"
          % (n_rec, B * Hkv * max_ctx))
    _check_key_planes(tables, kp, n_rec)
    _check_value_planes(vp, v_bits, n_rec, d)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    st = lib.tq_decode_attention_noalloc(ctypes.byref(tables.cfg), _ptr(tables.dev), _ptr(q), _DT[q.dtype],
                                         B, Hq, Hkv, _ptr(ctx_len), max_ctx, _ptr(kp["idx"]),
                                         _ptr(kp.get("signs")), _ptr(kp["norm"]), _ptr(kp.get("rnorm")),
                                         v_bits, 32, _ptr(vp["codes"]), _ptr(vp["scale"]), _ptr(vp["zero"]),
                                         ctypes.c_float(sm_scale), _ptr(out), _ptr(lse), _ptr(scores),
                                         _stream())
    check("tq_decode_attention_noalloc", st)
    return out


def decode_attention(tables: Tables, q, ctx_len, kp, vp, v_bits, max_ctx, sm_scale=None,
                     with_lse=False, with_scores=False, k_new=None, v_new=None):
    B, Hq, d = q.shape
    Hkv = kp["idx"].shape[0] // (B * max_ctx)
    dec = Decoder(tables, B, Hq, Hkv, max_ctx, v_bits, q.dtype, q.device)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if with_lse else None
    scores = torch.full((B, Hq, max_ctx), float("nan"), dtype=torch.float32, device=q.device) \
        if with_scores else None
    out = dec(q, ctx_len, kp, vp, sm_scale, lse=lse, scores=scores, k_new=k_new, v_new=v_new)
    return out, lse, scores
