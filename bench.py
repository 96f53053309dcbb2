#!/usr/bin/env python3
"""Benchmark of the TurboQuant KV-cache hot path on one MI355X.

Workload (printed as config.workload): batched GQA decode, 16 sequences x 8 KV
heads x 32 query heads, head dim 128, context 32768 per sequence; keys in prod
mode at 3 bits (2-bit Lloyd-Max index + 1-bit QJL signs + fp16 norm and
residual norm), values at 2 bits in groups of 32 with fp16 scale and zero;
bf16 queries, keys and values drawn N(0,1) (synthetic, seeded).

One step = one pass of the whole path for one decode step of the batch:
  encode the step's new key and value of every (sequence, KV head) into the
  packed cache in one launch (norm, rotation, bucketize, QJL signs, packing;
  value groups),
  then decode attention over the full 32768-token context (query rotation and
  projection, lookup-table scores from the packed bytes, online softmax,
  p.V, split-K merge).
`value` = KV tokens per second = 16 * 32768 / step time.  Inputs are resident
in HBM before timing starts.

Also reported (measured outside the timed steps): bulk encode throughput of
the same cache (4,194,304 keys and values) and of the 28-layer MSE prefill
workload (1,835,008 bf16 keys at 4 and 8 bits); the decode-call time of the
128k-context needle workload (prod 4-bit keys, 4-bit values) and of the 16k
grouped workload (4/2-bit grouped keys, 4-bit values), with the needle
workload's top-5 score recall against exact float32 attention and the ranks
of its planted needles; the bandwidth of a plain device copy (the practical
HBM ceiling); and the CPU oracle's decode throughput on a bounded sample on
the host cores.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
B, HKV, HQ, CTX, D = 16, 8, 32, 32768, 128
KEY_BYTES = 52      # 32 B index + 16 B signs + 2 B norm + 2 B residual norm
VAL_BYTES = 48      # 32 B codes + 4 groups x (2 B scale + 2 B zero)
DECODE_BYTES = B * HKV * CTX * (KEY_BYTES + VAL_BYTES)   # 419,430,400 B per decode
# the appending decode reads the cache without the new token's record, the new
# bf16 key and value rows, and writes that record: 65,536 B more per step
STEP_BYTES = DECODE_BYTES + B * HKV * 2 * D * 2


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-seconds", type=float, default=0.5,
                    help="untimed steps after the warm-up, until the GPU clocks have settled")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--two-launch-step", action="store_true",
                    help="append with tq_append_kv, then decode (two launches) instead of appending inside "
                         "the decode launch; the timed call is then the decode alone")
    ap.add_argument("--no-encode-bench", action="store_true")
    ap.add_argument("--no-other-decodes", action="store_true",
                    help="skip the decode timings of the 128k needle and 16k grouped workloads")
    ap.add_argument("--cpu-groups", type=int, default=128,
                    help="(sequence, KV head) groups the CPU oracle decodes for its baseline")
    ap.add_argument("--profile-decode", type=int, default=0,
                    help="only run this many decode calls after setup (for rocprofv3 runs)")
    ap.add_argument("--profile-encode", type=int, default=0,
                    help="only run this many bulk key and value encodes of the cache (rocprofv3 runs)")
    ap.add_argument("--profile-copy", type=int, default=0,
                    help="with --profile-decode or --profile-encode: also run five float32 negations of "
                         "this many MiB (a plain streaming kernel of known size that calibrates HBM counters)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: turn two rocprofv3 --pmc counter_collection.csv files "
                         "(FETCH_SIZE, WRITE_SIZE) of a --profile-decode (or --profile-encode) "
                         "--profile-copy run into profiles/decode_gqa32k_traffic.json (or "
                         "profiles/encode_gqa32k_traffic.json)")
    return ap.parse_args()


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profile():
    """HBM bytes per decode launch from the committed counter summary, if it
    was taken on the current decode source; else None."""
    p = os.path.join(ROOT, "profiles", "decode_gqa32k_traffic.json")
    src = os.path.join(ROOT, "kv_cache_quantization_encode_amd", "csrc", "tq_decode.hip")
    try:
        with open(p) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256_16") != source_hash(src):
        return None
    return t.get("traffic_bytes_per_launch")


def _pmc_means(path, counter):
    """Mean per-dispatch value of `counter` by kernel family (decode, merge,
    calibration copy) from a rocprofv3 counter_collection.csv."""
    import csv
    acc = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            fam = ("decode" if "decode_kernel" in name else "merge" if "merge_kernel" in name
                   else "copy" if "neg_kernel" in name else "encode_keys" if "encode_keys_kernel" in name
                   else "encode_values" if "encode_values_kernel" in name else None)
            if fam is None:
                continue
            key = (fam, r["Dispatch_Id"])
            acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (fam, _), v in acc.items():
        out.setdefault(fam, []).append(v)
    return {fam: sum(v) / len(v) for fam, v in out.items()}, {fam: len(v) for fam, v in out.items()}


def write_traffic(fetch_csv, write_csv, copy_mib):
    """HBM traffic of one tq_decode_attention_append call (decode_kernel +
    merge_kernel) from FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each scaled
    by the ratio of the true bytes of the calibration copy to what the same
    counter reports for it."""
    fetch, nf = _pmc_means(fetch_csv, "FETCH_SIZE")
    write, nw = _pmc_means(write_csv, "WRITE_SIZE")
    copy_bytes = copy_mib * 1024 * 1024
    f_scale = copy_bytes / (fetch["copy"] * 1024.0)
    w_scale = copy_bytes / (write["copy"] * 1024.0)
    if "decode" not in fetch:
        return write_encode_traffic(fetch, write, nf, nw, copy_bytes, f_scale, w_scale)
    rd = (fetch["decode"] + fetch.get("merge", 0.0)) * 1024.0 * f_scale
    wr = (write["decode"] + write.get("merge", 0.0)) * 1024.0 * w_scale
    src = os.path.join(ROOT, "kv_cache_quantization_encode_amd", "csrc", "tq_decode.hip")
    rec = {"source_sha256_16": source_hash(src),
           "workload": "gqa-decode-32k",
           "fetch_kib_per_dispatch": fetch, "write_kib_per_dispatch": write,
           "dispatches": {"fetch": nf, "write": nw},
           "copy_bytes": copy_bytes, "fetch_scale": f_scale, "write_scale": w_scale,
           "read_bytes_per_launch": rd, "write_bytes_per_launch": wr,
           "traffic_bytes_per_launch": rd + wr,
           "algorithmic_bytes": STEP_BYTES,
           "traffic_over_algorithmic": (rd + wr) / STEP_BYTES}
    p = os.path.join(ROOT, "profiles", "decode_gqa32k_traffic.json")
    with open(p, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


def write_encode_traffic(fetch, write, nf, nw, copy_bytes, f_scale, w_scale):
    """HBM traffic of the bulk encode of the 32k GQA cache (4,194,304 keys,
    then as many value rows) from a --profile-encode --profile-copy run."""
    n = B * HKV * CTX
    src = os.path.join(ROOT, "kv_cache_quantization_encode_amd", "csrc", "tq_encode.hip")
    rec = {"source_sha256_16": source_hash(src), "workload": "gqa-decode-32k cache encode",
           "copy_bytes": copy_bytes, "fetch_scale": f_scale, "write_scale": w_scale}
    for fam, algo in (("encode_keys", n * (2 * D + KEY_BYTES)), ("encode_values", n * (2 * D + VAL_BYTES))):
        rd = fetch[fam] * 1024.0 * f_scale
        wr = write[fam] * 1024.0 * w_scale
        rec[fam] = {"fetch_kib_per_dispatch": fetch[fam], "write_kib_per_dispatch": write[fam],
                    "dispatches": {"fetch": nf[fam], "write": nw[fam]},
                    "read_bytes_per_launch": rd, "write_bytes_per_launch": wr,
                    "traffic_bytes_per_launch": rd + wr, "algorithmic_bytes": algo,
                    "traffic_over_algorithmic": (rd + wr) / algo}
    p = os.path.join(ROOT, "profiles", "encode_gqa32k_traffic.json")
    with open(p, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


def cpu_baseline(n_groups):
    """The oracle (float64 NumPy) decoding one step for `n_groups` (sequence,
    KV head) groups of the same workload shape: unpack the packed cache,
    dequantise keys and values, softmax attention for the group's 4 query
    heads.  Cache contents come from the oracle's own encode (not timed)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle.tq_oracle as O
    import tq_workloads as W

    To = O.build_tables(O.KeyConfig(mode="prod", bits=3, seed=42))
    G = HQ // HKV
    qv, _ = W.queries(3, 1, G * n_groups)
    caches = []
    for gi in range(n_groups):
        kv, _ = W.kv_rows(3, 1, CTX, row0=gi * CTX)
        vv, _ = W.kv_rows(3, 2, CTX, row0=gi * CTX)
        rec = O.pack_key_record(O.encode_keys(kv.astype(np.float64), To), To)
        vrec = O.pack_value_record(O.encode_values(vv, 2), 2)
        caches.append((rec, vrec))
    t0 = time.perf_counter()
    for gi, (rec, vrec) in enumerate(caches):
        enc = O.unpack_key_record(rec, To)
        khat = O.dequant_keys(enc, To)
        vhat = O.dequant_values(O.unpack_value_record(vrec, 2, D))
        O.decode_attention(qv[0, gi * G:(gi + 1) * G].astype(np.float64), khat, vhat, CTX)
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    tokens_per_s = n_groups * CTX / HKV / dt   # KV tokens/s in the same unit as value
    return {"value": tokens_per_s, "unit": "KV tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d of %d (sequence, KV head) groups x %d tokens, one decode step each "
                      "(unpack, dequantise, float64 softmax attention); %.1f s; scaled as "
                      "groups/%d sequences" % (n_groups, B * HKV, CTX, dt, HKV),
            "seconds": dt, "cpu_count": os.cpu_count()}


def main():
    args = parse()
    if args.traffic_from:
        write_traffic(args.traffic_from[0], args.traffic_from[1], args.profile_copy or 1024)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only (this path has no multi-GPU mode); got --gpus %d" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    import torch

    import kv_cache_quantization_encode_amd as tq
    import tq_workloads as W

    dev = "cuda:0"
    torch.cuda.set_device(0)
    cfg = tq.key_config(mode="prod", bits=3, seed=42)
    T = tq.Tables(cfg, dev)
    n_rec = B * HKV * CTX
    # ---- resident inputs: the cache's keys and values, then the packed cache
    keys = W.normal_bf16_device(3, 1, (n_rec, D), dev)
    vals = W.normal_bf16_device(3, 2, (n_rec, D), dev)
    kp = tq.key_planes(T, n_rec, dev)
    vp = tq.value_planes(2, n_rec, device=dev)
    tq.encode_keys(T, keys, kp)
    tq.encode_values(vals, 2, planes=vp)
    # per-step new tokens and queries (resident)
    n_steps_total = args.warmup + max(args.steps, 1)
    new_k = W.normal_bf16_device(3, 6, (n_steps_total, B * HKV, D), dev)
    new_v = W.normal_bf16_device(3, 7, (n_steps_total, B * HKV, D), dev)
    qs = W.normal_bf16_device(3, 3, (n_steps_total, B, HQ, D), dev)
    slots = (torch.arange(B * HKV, device=dev, dtype=torch.int64) * CTX + (CTX - 1)).contiguous()
    ctx_len = torch.full((B,), CTX, dtype=torch.int32, device=dev)
    dec = tq.Decoder(T, B, HQ, HKV, CTX, 2, torch.bfloat16, dev)
    out = torch.empty((B, HQ, D), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    # one decode call per step's inputs, its arguments checked once here
    # (Decoder.bind), so that each step only enqueues the launch
    if args.two_launch_step:
        calls = [dec.bind(qs[i], ctx_len, kp, vp, out=out) for i in range(n_steps_total)]
    else:
        calls = [dec.bind(qs[i], ctx_len, kp, vp, out=out, k_new=new_k[i].view(B, HKV, D),
                          v_new=new_v[i].view(B, HKV, D)) for i in range(n_steps_total)]

    def call(i):
        calls[i]()

    if args.profile_decode:
        for i in range(args.profile_decode):
            call(i % n_steps_total)
        torch.cuda.synchronize()
        print("profiled %d decode calls" % args.profile_decode, flush=True)
        if args.profile_copy:
            del keys, vals
            profile_copies(args.profile_copy, dev)
        return
    if args.profile_encode:
        for _ in range(args.profile_encode):
            tq.encode_keys(T, keys, kp)
            tq.encode_values(vals, 2, planes=vp)
        torch.cuda.synchronize()
        print("profiled %d bulk encodes of %d keys and values" % (args.profile_encode, n_rec), flush=True)
        if args.profile_copy:
            profile_copies(args.profile_copy, dev)
        return

    def step(i, ev=None):
        if args.two_launch_step:
            tq.append_kv(T, new_k[i], new_v[i], 2, kp, vp, slots=slots, n_records=n_rec)
        if ev is not None:
            ev[0].record()
        call(i)
        if ev is not None:
            ev[1].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # The GPU's clocks take tens of milliseconds of sustained load to settle;
    # keep stepping (untimed, on the warm-up inputs) until settle_seconds have
    # passed so that the timed steps measure the steady state.
    def settle(seconds):
        t_settle = time.perf_counter()
        i = 0
        while time.perf_counter() - t_settle < seconds:
            step(i % max(args.warmup, 1))
            i += 1
            if i % 50 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()

    settle(args.settle_seconds)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(args.warmup + k)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    # The decode call's own time: the same K steps again, with a pair of HIP
    # events around each call (kept out of the timed steps above, where their
    # records would sit between the launches).
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    settle(0.2 * args.settle_seconds)  # clocks back at steady load after the pause above
    for k in range(args.steps):
        step(args.warmup + k, evs[k])
    torch.cuda.synchronize()
    dec_ms = sorted(a.elapsed_time(b) for a, b in evs)
    dec_ms_mean = sum(dec_ms) / len(dec_ms)
    dec_ms_median = dec_ms[len(dec_ms) // 2]
    value = B * CTX / (ms_per_step * 1e-3)
    call_bytes = DECODE_BYTES if args.two_launch_step else STEP_BYTES
    achieved = call_bytes / (dec_ms_mean * 1e-3) / 1e9

    extra = {}
    if not args.no_encode_bench:
        extra.update(encode_bench(tq, W, T, keys, vals, dev))
    del keys, vals, kp, vp
    if not args.no_other_decodes:
        extra.update(other_decodes(tq, W, dev))
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.cpu_groups)
    traffic = traffic_from_profile()
    copy_gbps = copy_bandwidth()
    read_gbps = read_bandwidth(tq)
    line = {
        "metric": "decode-attn KV tokens/s & HBM GB/s (% of peak); encode keys/s",
        "value": value,
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u16 lookup tables + fp16 softmax weights, f32 accumulate",
        "data": "synthetic",
        "config": {"workload": "gqa-decode-32k", "sequences": B, "kv_heads": HKV, "q_heads": HQ,
                   "head_dim": D, "context": CTX, "keys": "prod 3-bit (2-bit index + QJL)",
                   "values": "2-bit group 32",
                   "step": ("append-encode 128 K/V rows (tq_append_kv), then decode" if args.two_launch_step else
                            "one launch: append-encode 128 K/V rows and decode (tq_decode_attention_append)")},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic,
                     "kernel": ("tq_decode_attention" if args.two_launch_step else "tq_decode_attention_append")
                     + " (decode_kernel + merge_kernel)",
                     "algorithmic_bytes": call_bytes, "ms_mean": dec_ms_mean,
                     "ms_median": dec_ms_median,
                     "achievable_copy_gbps": copy_gbps, "frac_of_copy": achieved / copy_gbps,
                     "achievable_read_gbps": read_gbps, "frac_of_read": achieved / read_gbps},
        "cpu_baseline": cpu,
    }
    line.update(extra)
    print(json.dumps(line))


def profile_copies(mib, dev):
    """Five float32 negations of `mib` MiB: the counter calibration kernel."""
    import torch
    n = mib * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print("profiled 5 copies of %d MiB" % mib, flush=True)


def copy_bandwidth(mib=2048, reps=20):
    """HBM bandwidth a plain device-to-device copy reaches (read + write
    bytes over time; torch's copy kernel, 2 GiB, settled clocks): the
    practical ceiling next to the 8 TB/s specification."""
    import torch
    n = mib * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.2:
        dst.copy_(src)
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return 2.0 * n * 4 / (ms * 1e-3) / 1e9


def read_bandwidth(tq, mib=2048, reps=20):
    """Read bandwidth of one streaming pass with 16-byte nontemporal loads
    (tq_stream_read over 2 GiB, settled clocks): the access pattern of the
    decode's reads of the packed cache, so the ceiling its achieved bytes per
    second compare against on this GPU."""
    import torch
    src = torch.ones(mib * 1024 * 1024 // 4, dtype=torch.int32, device="cuda:0")
    sink = torch.empty(65536, dtype=torch.int32, device="cuda:0")
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.2:
        tq.stream_read(src, sink)
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        tq.stream_read(src, sink)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nbytes = src.numel() * 4
    del src, sink
    return nbytes / (ms * 1e-3) / 1e9


def encode_bench(tq, W, T, keys, vals, dev, reps=10):
    """Bulk encode throughput (not part of the timed steps)."""
    import torch

    def timed(fn):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.1:   # settle the clocks
            fn()
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    n = keys.shape[0]
    kp = tq.key_planes(T, n, dev)
    vp = tq.value_planes(2, n, device=dev)
    ms_k = timed(lambda: tq.encode_keys(T, keys, kp))
    ms_v = timed(lambda: tq.encode_values(vals, 2, planes=vp))
    kbytes = n * (2 * D + KEY_BYTES)
    vbytes = n * (2 * D + VAL_BYTES)
    res = {"encode_prod3": {"keys": n, "ms": ms_k, "keys_per_s": n / (ms_k * 1e-3),
                            "gbps": kbytes / (ms_k * 1e-3) / 1e9,
                            "gflops_qjl": 2.0 * D * D * n / (ms_k * 1e-3) / 1e9},
           "encode_values2": {"rows": n, "ms": ms_v, "rows_per_s": n / (ms_v * 1e-3),
                              "gbps": vbytes / (ms_v * 1e-3) / 1e9}}
    del kp, vp
    # 28-layer MSE prefill encode, 4 and 8 bits, one seed per layer
    layers = [W.w2_layer_keys_device(l, dev) for l in range(28)]
    n2 = sum(x.shape[0] for x in layers)
    for bits in (4, 8):
        tabs = [tq.Tables(tq.key_config(mode="mse", bits=bits, seed=42 + l), dev) for l in range(28)]
        planes = [tq.key_planes(tabs[0], layers[0].shape[0], dev) for _ in range(28)]

        run = tq.KeyBatchEncoder(tabs, layers, planes)   # all 28 layers in one launch, checked once
        ms = timed(run)
        row = tabs[0].row_bytes + 2
        res["encode_mse%d_prefill" % bits] = {"keys": n2, "ms": ms, "keys_per_s": n2 / (ms * 1e-3),
                                             "gbps": n2 * (2 * D + row) / (ms * 1e-3) / 1e9}
        del planes
    return res


def other_decodes(tq, W, dev, reps=50):
    """Decode-call time of the two other decode workloads (not part of the
    timed steps; settled clocks, HIP events over `reps` back-to-back calls):
    1 x 8 x 32 heads at context 131072 with prod 4-bit keys and 4-bit values
    (164 B per token-head), and 8 x 8 x 32 heads at context 16384 with grouped
    (4-bit outlier half, 2-bit normal half) keys and 4-bit values (132 B)."""
    import torch

    res = {}
    G = HQ // HKV
    cases = [("decode_needle128k", dict(mode="prod", bits=4), 1, 131072, 4, None, 4, 164),
             ("decode_grouped16k", dict(mode="grouped", bits_outlier=4, bits_normal=2), 8, 16384, 4,
              W.w5_col_scale(), 5, 132)]
    for name, kw, b, ctx, vbits, scale, wid, per in cases:
        T = tq.Tables(tq.key_config(seed=42, **kw), dev)
        n = b * HKV * ctx
        keys = W.normal_bf16_device(wid, 1, (n, D), dev, scale_cols=scale)
        q = W.normal_bf16_device(wid, 3, (1, b, HQ, D), dev)[0].contiguous()
        needles = name == "decode_needle128k"
        if needles:
            # five needles per KV head at the pages' depths, along the first
            # query head of the group (4 x its unit direction + N(0, 0.1^2))
            nv, _ = W.w4_needles(q.float().cpu().numpy(), HKV, HQ)
            pos = W.needle_positions(ctx)
            for h in range(HKV):
                for i, p in enumerate(pos):
                    keys[h * ctx + p] = torch.from_numpy(nv[h, i]).to(dev).to(torch.bfloat16)
        kp = tq.encode_keys(T, keys)
        vals = W.normal_bf16_device(wid, 2, (n, D), dev)
        vp = tq.encode_values(vals, vbits)
        del vals
        ctx_len = torch.full((b,), ctx, dtype=torch.int32, device=dev)
        dec = tq.Decoder(T, b, HQ, HKV, ctx, vbits, torch.bfloat16, dev)
        out = torch.empty((b, HQ, D), dtype=torch.float32, device=dev)
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.2:   # settle the clocks
            for _ in range(20):
                dec(q, ctx_len, kp, vp, out=out)
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            dec(q, ctx_len, kp, vp, out=out)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        nbytes = n * per
        res[name] = {"token_heads": n, "algorithmic_bytes": nbytes, "ms": ms,
                     "kv_tokens_per_s": b * ctx / (ms * 1e-3), "gbps": nbytes / (ms * 1e-3) / 1e9,
                     "frac_of_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS}
        if needles:
            # top-5 recall of the decoded scores against exact float32 q.k over
            # the original keys, and the needles' ranks (one decode call with
            # scores, outside the timing)
            scores = torch.empty((b, HQ, ctx), dtype=torch.float32, device=dev)
            dec(q, ctx_len, kp, vp, out=out, scores=scores)
            kf = keys.view(HKV, ctx, D).float()
            rec, ranks = [], []
            for hq in range(HQ):
                h = hq // G
                exact = kf[h] @ q[0, hq].float()
                te = set(torch.topk(exact, 5).indices.tolist())
                tg = set(torch.topk(scores[0, hq], 5).indices.tolist())
                rec.append(len(te & tg) / 5.0)
                if hq % G == 0:
                    order = torch.argsort(scores[0, hq], descending=True)
                    rank = torch.empty_like(order)
                    rank[order] = torch.arange(ctx, device=dev)
                    ranks.append([int(rank[p]) for p in pos])
            res[name].update(recall_at_5=sum(rec) / len(rec), needle_ranks=ranks, needles_per_kv_head=len(pos))
            del kf, scores
        del kp, vp, dec, keys
    return res


if __name__ == "__main__":
    main()
