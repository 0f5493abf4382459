"""Benchmark: MLA decode step (absorb -> decode -> combine -> up-projection) on
one MI355X, synthetic inputs, printed as one JSON line.

Timed workload (default): the paged ragged batch, the largest configuration
that fits one GPU -- DeepSeek-V2 geometry (128 heads, d_nope 128, d_rope 64,
d_c 512, d_v 128), bf16 cache and weights with fp32 accumulation, 64
sequences with lengths drawn uniformly in [512, 16384], the cache in 64-token
pages in a shuffled block table, 8 split ranges per sequence.  A "step" is one
decode step of one layer for the whole batch; tokens/s = batch / step time.

The inputs of R independent replicas (cache rows, queries, weights; >= 1.25
GiB in total) are resident in HBM before timing starts and the steps rotate
over them, so the 256 MB Infinity Cache cannot serve the cache stream.  HIP
events recorded between the step's launches, on the launch stream, give each
kernel's per-launch duration over the timed steps (median, p10, p90, mean).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD's published peak
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "decode_traffic.json")
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}  # dense matrix-core peaks at 2.4 GHz
CLOCK_HZ = 2.4e9  # rated engine clock (the matrix-core peaks are quoted at it)
N_SIMD = 256 * 4
# the sources of the decode kernels (a traffic record is valid for these bytes only)
KERNEL_SOURCES = [os.path.join(ROOT, "mla_latent_kv_15_amd", "csrc", f)
                  for f in ("mla_kernels.hip", "mla_decode_fp8.hip", "mla_decode_tile.h",
                            "mla_device.h")]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the board settles at its power limit within a few hundred launches of
    # the step (clock ramp, then a dip): the warm-up covers that, so the timed
    # steps see the sustained clock
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--workload", default="paged_b64_ragged")
    ap.add_argument("--events-every", type=int, default=4, metavar="N",
                    help="per-launch HIP events around the launches of every N-th timed step "
                         "(the event markers lengthen the steps they bracket by ~9 us; 1 = all)")
    ap.add_argument("--splits", type=int, default=0, help="0: the workload's own split count")
    ap.add_argument("--part-dtype", default="bf16", choices=["bf16", "f32"])
    ap.add_argument("--decode-kernel", default=None,
                    choices=["auto", "h64", "balanced"],
                    help="decode work decomposition (mla_decode_ex); auto = mla_decode's choice; "
                         "default: the workload's (balanced for a balanced-partition workload, "
                         "else auto)")
    ap.add_argument("--query-dtype", default="auto", choices=["auto", "bf16", "fp8"],
                    help="absorbed-query format: fp8 (E4M3 + one factor per sequence and head; "
                         "the decode then runs on the fp8 matrix cores) needs an fp8 cache; "
                         "auto = fp8 for an fp8 cache, else the activation dtype")
    ap.add_argument("--replica-bytes", type=float, default=1.25 * 2**30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--two-call-tail", action="store_true",
                    help="merge and up-project with mla_combine + mla_up_proj")
    ap.add_argument("--q-len", type=int, default=1,
                    help="query tokens per sequence (> 1: multi-token decode with "
                         "mla_decode_multi; tokens/s counts every query token)")
    ap.add_argument("--mha", action="store_true",
                    help="the MHA baseline instead: per-head bf16 K/V cache at the geometry of "
                         "--workload (batch, heads, lengths; head dim 128), mla_mha_decode")
    ap.add_argument("--prefill", type=int, default=0, metavar="CHUNK",
                    help="chunked prefill in the naive form instead: the last CHUNK cached "
                         "tokens of every sequence of --workload are the queries; keys and values "
                         "rebuilt for the whole context (mla_prefill_rebuild_kv), then causal "
                         "attention (mla_prefill_attn); query tokens/s, matrix-core roofline")
    ap.add_argument("--gqa", type=int, default=0, metavar="KV_HEADS",
                    help="with --mha: grouped-query attention with this many key/value heads "
                         "(mla_gqa_decode); 0 = one per query head")
    ap.add_argument("--stream-ceiling", action="store_true",
                    help="time the decode's tile stream without its arithmetic (mla_stream_probe: "
                         "256 workgroups x 100 tiles of 36 KB, paired and private) and a torch "
                         "reduction over 1 GiB; print one JSON line")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a device copy of known size (counter calibration)")
    ap.add_argument("--record-traffic", metavar="DIR",
                    help="no GPU work: read the rocprofv3 --pmc CSVs under DIR/{fetch,write,"
                         "cfetch,cwrite} and store the decode kernel's HBM bytes per launch in "
                         "profiles/decode_traffic.json")
    return ap.parse_args()


def source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def query_dtype(args, wl) -> str:
    """the absorbed query's format for this run"""
    if args.query_dtype == "auto":
        return "fp8" if wl.cache_dtype == "fp8" else ("f32" if wl.cache_dtype == "f32" else "bf16")
    if args.query_dtype == "fp8" and wl.cache_dtype != "fp8":
        raise SystemExit("an fp8 query needs an fp8 cache")
    return args.query_dtype


def traffic_key(workload, splits, partials, decode_kernel, query="bf16"):
    """the launch configuration a traffic record belongs to (an fp8 query,
    which runs another kernel, is part of it)"""
    key = {"workload": workload, "splits": splits, "partials": partials,
           "decode_kernel": decode_kernel}
    if query == "fp8":
        key["query"] = "fp8"
    return key


def _records():
    try:
        rec = json.load(open(PROFILE_TRAFFIC))
    except (OSError, ValueError):
        return []
    return rec.get("records", []) if isinstance(rec, dict) else []


def stored_counters(key):
    """The counter record of the decode kernel (HBM bytes per launch from
    FETCH_SIZE / WRITE_SIZE, matrix-core busy cycles), if it was taken on the
    current kernel source and on the launch configuration `key`; else None."""
    for rec in _records():
        if rec.get("kernel_source_sha256_16") == source_hash() and rec.get("config") == key:
            return rec
    return None


def _counter_means(path, counter):
    """mean value of `counter` per kernel name in a rocprofv3 counter CSV"""
    import csv
    acc = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        name = r["Kernel_Name"]
        v = acc.setdefault(name, [0.0, 0])
        v[0] += float(r["Counter_Value"])
        v[1] += 1
    return {k: v[0] / v[1] for k, v in acc.items()}


def decode_kernel_of(args, wl) -> str:
    """--decode-kernel, else the workload's own: balanced or mla_decode's choice"""
    if args.decode_kernel:
        return args.decode_kernel
    return "balanced" if wl.partition == "balanced" else "auto"


def record_traffic(d, args):
    """HBM bytes per mla_decode launch from FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), each scaled by the factor that maps the same counter onto the
    known bytes of a 1 GiB device copy, and (if DIR/sq exists) the decode's
    SQ_VALU_MFMA_BUSY_CYCLES per launch.  The counter runs used the launch
    configuration given by the other options (the defaults unless stated);
    the record replaces any earlier one for the same configuration."""
    import synth
    wl = synth.workload(args.workload)
    args.decode_kernel = decode_kernel_of(args, wl)
    key = traffic_key(args.workload, args.splits or wl.num_splits, args.part_dtype,
                      args.decode_kernel, query_dtype(args, wl))
    f = _counter_means(os.path.join(d, "fetch", "run_counter_collection.csv"), "FETCH_SIZE")
    w = _counter_means(os.path.join(d, "write", "run_counter_collection.csv"), "WRITE_SIZE")
    cf = _counter_means(os.path.join(d, "cfetch", "run_counter_collection.csv"), "FETCH_SIZE")
    cw = _counter_means(os.path.join(d, "cwrite", "run_counter_collection.csv"), "WRITE_SIZE")
    copy_kib = (1 << 30) / 1024.0
    kf = copy_kib / max(v for k, v in cf.items() if "copyBuffer" in k)
    kw = copy_kib / max(v for k, v in cw.items() if "copyBuffer" in k)
    name = next(k for k in f if "decode_" in k and "kernel" in k)
    short = name.replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]
    rec = {"kernel": short, "kernel_source_sha256_16": source_hash(), "config": key,
           "fetch_kib_per_launch": f[name], "write_kib_per_launch": w[name],
           "fetch_scale": kf, "write_scale": kw,
           "hbm_bytes_per_launch": (f[name] * kf + w[name] * kw) * 1024.0,
           "counters_from": os.path.relpath(os.path.abspath(d), ROOT)}
    sq = os.path.join(d, "sq", "run_counter_collection.csv")
    if os.path.exists(sq):
        busy = _counter_means(sq, "SQ_VALU_MFMA_BUSY_CYCLES")
        if name in busy:
            rec["mfma_busy_cycles_per_launch"] = busy[name]
    recs = [r for r in _records() if r.get("config") != key]
    recs.append(rec)
    json.dump({"records": recs}, open(PROFILE_TRAFFIC, "w"), indent=1)
    print(json.dumps(rec))


def pct(xs, q):
    """q-th percentile (0..100) of the samples xs, linear between order statistics"""
    import numpy as np
    return float(np.percentile(np.asarray(xs, np.float64), q))


def launch_stats(us):
    """per-launch durations (us) -> {median, p10, p90, mean, n}"""
    return {"median": pct(us, 50), "p10": pct(us, 10), "p90": pct(us, 90),
            "mean": float(sum(us) / len(us)), "n": len(us)}


def multi_token_bench(args, wl, dev, reps, R, S, act, part, out, cache_bytes):
    """Multi-token decode step: mla_absorb_q over B*q_len query tokens ->
    mla_decode_multi -> mla_combine_up_proj over B*q_len rows.  Synthetic
    queries (seeded); the cache replicas of the plain bench."""
    import numpy as np
    import torch

    import mla_latent_kv_15_amd as mla

    B, QL, H = wl.batch, args.q_len, wl.heads
    g = torch.Generator(device="cuda").manual_seed(wl.seed + QL)
    qn = torch.randn(B * QL, H, wl.d_nope, device="cuda", generator=g).to(act)
    qr = torch.randn(B * QL, H, wl.d_rope, device="cuda", generator=g).to(act)
    q_abs = torch.empty(B, QL, H, 576, dtype=act, device="cuda")
    u_part = torch.empty(B, QL, S, H, wl.d_latent, dtype=part, device="cuda")
    lse_part = torch.empty(B, QL, S, H, dtype=torch.float32, device="cuda")
    o = torch.empty(B * QL, H, wl.d_v, dtype=out, device="cuda")
    stream = torch.cuda.current_stream()
    geo = dev.geo

    stages = [
        ("mla_absorb_q", lambda rp: mla.mla_absorb_q(geo, qn, qr, rp["w_uk"], q_abs.view(B * QL, H, 576),
                                                     stream=stream)),
        ("mla_decode_multi", lambda rp: mla.mla_decode_multi(geo, q_abs, rp["cache"], S, u_part,
                                                             lse_part, stream=stream)),
        ("mla_combine_up_proj", lambda rp: mla.mla_combine_up_proj(
            geo, u_part.view(B * QL, S, H, wl.d_latent), lse_part.view(B * QL, S, H), rp["w_uv"], o,
            stream=stream)),
    ]

    def one(i):
        for _, fn in stages:
            fn(reps[i % R])

    for i in range(args.warmup):
        one(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        one(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    kernel_us = {}
    for name, fn in stages:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            fn(reps[i % R])
        e1.record(stream)
        torch.cuda.synchronize()
        kernel_us[name] = e0.elapsed_time(e1) / args.steps * 1e3
    t_dec = kernel_us["mla_decode_multi"] * 1e-6
    flops = float(np.sum(np.asarray(dev.inp.seq_lens, np.float64))) * QL * 2 * H * 1088
    rec = {
        "metric": "MLA multi-token decode query tokens/s (q_len per sequence), 1 GPU",
        "value": B * QL / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if wl.cache_dtype == "bf16" else wl.cache_dtype,
        "data": "synthetic (seeded N(0,1) activations/cache, N(0,1/512) weights)",
        "config": {"workload": wl.name, "batch": B, "q_len": QL, "heads": H, "splits": S,
                   "seq_len": int(dev.inp.max_seq_len), "parallelism": "none (1 GPU)"},
        "cache_GBps": cache_bytes / t_dec / 1e9,
        "kernel_us_mean": kernel_us,
        "roofline": {"kernel": "mla_decode_multi", "bound": "mfma", "achieved": flops / t_dec / 1e12,
                     "peak": 2500.0, "unit": "TFLOP/s", "frac": flops / t_dec / 1e12 / 2500.0,
                     "traffic": None, "algorithmic_flops_per_launch": flops},
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)


def mha_baseline(args):
    """Multi-head (or, with --gqa N, grouped-query with N key/value heads)
    attention decode over a per-head K/V cache -- what MLA's latent cache
    replaces -- at the batch, heads and lengths of --workload: one launch of
    mla_mha_decode / mla_gqa_decode per step.  The cache (2 x h_kv x 128 bf16
    per token) is streamed from HBM (replicas rotated when one copy would fit
    the 256 MB Infinity Cache)."""
    import torch

    import mla_latent_kv_15_amd as mla
    import synth

    wl = synth.workload(args.workload)
    lens = synth.workloads.sequence_lengths(wl)
    B, H, D = wl.batch, wl.heads, 128
    Hkv = args.gqa or H
    if H % Hkv:
        sys.exit(f"--gqa {Hkv} does not divide {H} heads")
    L = int(lens.max())
    kind = "MHA" if Hkv == H else f"GQA ({Hkv} key/value heads)"
    print(f"[bench] {kind} baseline at {wl.name}: B={B} h={H} L<={L}", file=sys.stderr, flush=True)
    g = torch.Generator(device="cuda").manual_seed(wl.seed)
    q = torch.randn(B, H, D, device="cuda", generator=g).to(torch.bfloat16)
    kv_bytes = int(lens.astype("int64").sum()) * Hkv * D * 2 * 2
    R = max(1, math.ceil(args.replica_bytes / (B * Hkv * L * D * 2 * 2)))
    reps = []
    for _ in range(R):
        k = torch.empty(B, Hkv, L, D, dtype=torch.bfloat16, device="cuda")
        v = torch.empty_like(k)
        for b in range(B):  # per sequence, to bound the fp32 temporaries
            k[b] = torch.randn(Hkv, L, D, device="cuda", generator=g).to(torch.bfloat16)
            v[b] = torch.randn(Hkv, L, D, device="cuda", generator=g).to(torch.bfloat16)
        reps.append((k, v))
    seq = torch.from_numpy(lens.astype("int32")).cuda()
    o = torch.empty(B, H, D, dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    calls = [mla.mla_gqa_decode(q, k, v, seq, L, o, stream=stream, prepare=True)
             for k, v in reps]

    for i in range(args.warmup):
        calls[i % R]()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i].record(stream)
        calls[i % R]()
    ev[args.steps].record(stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    us = [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(args.steps)]
    st = launch_stats(us)
    t_k = st["mean"] * 1e-6
    mla_bytes = synth.cache_bytes(wl, lens)
    achieved = kv_bytes / t_k / 1e9
    name = "MHA" if Hkv == H else "GQA"
    rec = {
        "metric": f"{name} baseline decode tokens/s + K/V HBM GB/s (% of MI355X peak), 1 GPU",
        "value": B / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1) q, K, V)",
        "config": {"workload": f"{name.lower()}_baseline_{wl.name}", "batch": B, "heads": H,
                   "kv_heads": Hkv, "d_head": D, "seq_len": L, "replicas": R,
                   "cache": "bf16 per-head K and V, head-major", "parallelism": "none (1 GPU)"},
        "kv_cache_bytes": kv_bytes, "mla_cache_bytes_same_tokens": mla_bytes,
        "cache_ratio": kv_bytes / mla_bytes,
        "kernel_us": {"mla_gqa_decode": st},
        "roofline": {"kernel": "mla_gqa_decode", "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": None, "algorithmic_bytes_per_launch": kv_bytes},
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)


def prefill_bench(args):
    """Chunked prefill, naive (rebuild) form: each step rebuilds every head's
    keys and values for each sequence's whole context and runs the causal
    attention of its last CHUNK tokens.  Inputs of the workload (one copy: the
    rebuilt keys and values alone are larger than the Infinity Cache)."""
    import numpy as np
    import torch

    import mla_latent_kv_15_amd as mla
    import synth
    from tests.device_inputs import DeviceInputs

    wl = synth.workload(args.workload)
    inp = synth.make_inputs(wl)
    dev = DeviceInputs(inp)
    lens = np.asarray(inp.seq_lens, np.int64)
    B, H, QL = wl.batch, wl.heads, args.prefill
    S = int(-(-int(lens.max()) // 32) * 32)
    nq = np.minimum(lens, QL)
    print(f"[bench] prefill {wl.name}: B={B} h={H} chunk={QL} context<={int(lens.max())}",
          file=sys.stderr, flush=True)
    g = torch.Generator(device="cuda").manual_seed(wl.seed + 9)
    q = torch.randn(B, QL, H, wl.d_nope + wl.d_rope, device="cuda", generator=g).to(torch.bfloat16)
    q_lens = torch.from_numpy(nq.astype(np.int32)).cuda()
    k = torch.empty(B, H, S, wl.d_nope + wl.d_rope, dtype=torch.bfloat16, device="cuda")
    vt = torch.empty(B, H, wl.d_v, S, dtype=torch.bfloat16, device="cuda")
    o = torch.empty(B, QL, H, wl.d_v, dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    stages = [("mla_prefill_rebuild_kv", mla.mla_prefill_rebuild_kv(
                  dev.geo, dev.cache, dev.w_uk, dev.w_uv, k, vt, stream=stream, prepare=True)),
              ("mla_prefill_attn", mla.mla_prefill_attn(
                  dev.geo, q, q_lens, k, vt, dev.cache.seq_lens, int(lens.max()), o,
                  stream=stream, prepare=True))]
    for _ in range(args.warmup):
        for _, c in stages:
            c()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        for jj, (_, c) in enumerate(stages):
            c()
            ev[i][jj + 1].record(stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    st = {name: launch_stats([ev[i][jj].elapsed_time(ev[i][jj + 1]) * 1e3
                              for i in range(args.steps)])
          for jj, (name, _) in enumerate(stages)}
    # matrix-core work: rebuild 2 * 512 * (d_nope + d_v) per head and cached
    # token; attention 2 * (192 + 128) per head, query and attended key
    f_rebuild = float(lens.sum()) * H * 2 * wl.d_latent * (wl.d_nope + wl.d_v)
    att_keys = float(sum(int(n) * (int(L) - int(n)) + int(n) * (int(n) + 1) // 2
                         for L, n in zip(lens, nq)))
    f_attn = att_keys * H * 2 * (wl.d_nope + wl.d_rope + wl.d_v)
    t_r, t_a = st["mla_prefill_rebuild_kv"]["mean"] * 1e-6, st["mla_prefill_attn"]["mean"] * 1e-6
    rec = {
        "metric": "MLA chunked prefill (naive rebuild form) query tokens/s, 1 GPU",
        "value": float(nq.sum()) / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) queries/cache, N(0,1/512) weights)",
        "config": {"workload": f"prefill_{wl.name}_chunk{QL}", "batch": B, "heads": H,
                   "chunk": QL, "context_max": int(lens.max()), "query_tokens": int(nq.sum()),
                   "parallelism": "none (1 GPU)"},
        "kernel_us": st,
        "tflops": {"mla_prefill_rebuild_kv": f_rebuild / t_r / 1e12,
                   "mla_prefill_attn": f_attn / t_a / 1e12},
        "roofline": {"kernel": "mla_prefill_attn", "bound": "mfma",
                     "achieved": f_attn / t_a / 1e12, "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": f_attn / t_a / 1e12 / 2500.0, "traffic": None,
                     "algorithmic_flops_per_launch": f_attn},
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)


def stream_ceiling():
    """The read rate of the decode's tile stream alone (mla_stream_probe), the
    ceiling the decode's roofline fraction is read against, and a plain torch
    reduction's read rate.  Two 1 GiB sources alternate so that no launch
    reads what the previous one left in the 256 MB Infinity Cache; per-launch
    times from HIP events on the launch stream."""
    import torch

    import mla_latent_kv_15_amd as mla
    srcs = [torch.full((1 << 30,), i + 1, dtype=torch.uint8, device="cuda") for i in range(2)]
    sink = torch.empty(256, dtype=torch.int32, device="cuda")
    wg, tiles, tile_bytes, n = 256, 100, 36864, 40
    stream = torch.cuda.current_stream()
    out = {"metric": "decode tile stream without arithmetic (read ceiling), 1 GPU", "unit": "GB/s",
           "workgroups": wg, "tiles_per_workgroup": tiles, "tile_bytes": tile_bytes}

    def timed(fn):
        for i in range(4):
            fn(srcs[i & 1])
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        for i, (e0, e1) in enumerate(ev):
            e0.record(stream)
            fn(srcs[i & 1])
            e1.record(stream)
        torch.cuda.synchronize()
        us = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in ev)
        return us[n // 2], us[n // 10], us[(9 * n) // 10]

    for paired in (True, False):
        med, p10, p90 = timed(lambda s: mla.mla_stream_probe(s, wg, tiles, paired, sink, stream=stream))
        unique = (wg // 2 if paired else wg) * tiles * tile_bytes
        key = "paired" if paired else "private"
        out[key] = {"us_median": med, "us_p10": p10, "us_p90": p90, "bytes_unique": unique,
                    "GBps_unique": unique / med / 1e3, "frac_of_8TBps": unique / med / 8e6,
                    "GBps_into_CUs": wg * tiles * tile_bytes / med / 1e3}
    acc = torch.empty((), dtype=torch.float32, device="cuda")
    med, p10, p90 = timed(lambda s: torch.sum(s.view(torch.bfloat16), dim=0, dtype=torch.float32,
                                              out=acc))
    out["torch_sum_bf16_1GiB"] = {"us_median": med, "GBps": (1 << 30) / med / 1e3,
                                  "frac_of_8TBps": (1 << 30) / med / 8e6}
    print(json.dumps(out), flush=True)


def calibrate_copy():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read": n, "bytes_written": n,
                      "launches": 5}), flush=True)


def cpu_baseline(inp, target_s: float = 15.0):
    """The oracle timed on the host cores on whole sequences (all heads, all
    cached tokens) of the same workload, as many as fit in about target_s
    seconds (at least one).  The oracle's time is linear in the cached tokens,
    so the sample's time is scaled to the whole batch by cached tokens;
    tokens/s = sequences of the batch / that time."""
    import numpy as np

    import oracle
    wl = inp.wl
    t = time.perf_counter()
    oracle.decode_inputs(inp, sel=[(0, h) for h in range(wl.heads)])
    first = time.perf_counter() - t
    n_seq = int(max(1, min(wl.batch, round(target_s / max(first, 1e-3)))))
    if n_seq > 1:
        pairs = [(b, h) for b in range(1, n_seq) for h in range(wl.heads)]
        oracle.decode_inputs(inp, sel=pairs)
    dt = time.perf_counter() - t
    lens = np.asarray(inp.seq_lens, np.float64)
    sampled, total = float(lens[:n_seq].sum()), float(lens.sum())
    batch_s = dt * total / max(sampled, 1.0)
    return {"value": wl.batch / batch_s, "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{n_seq} of {wl.batch} sequences ({int(sampled)} of {int(total)} cached "
                      f"tokens), all {wl.heads} heads, naive float64 rebuild of K and V, "
                      f"{dt:.1f} s; scaled to the whole batch by cached tokens"}


# the oracle's one-thread run, in a child process (OpenMP reads its thread
# count when the library starts); no GPU is touched there
_ONE_CORE = r"""
import json, sys, time
sys.path.insert(0, sys.argv[1])
import numpy as np
import oracle, synth
inp = synth.make_inputs(synth.workload(sys.argv[2]))
target = float(sys.argv[3])
wl = inp.wl
t = time.perf_counter()
n = 0
while n < wl.batch and (n == 0 or time.perf_counter() - t < target):
    oracle.decode_inputs(inp, sel=[(n, h) for h in range(wl.heads)])
    n += 1
dt = time.perf_counter() - t
lens = np.asarray(inp.seq_lens, np.float64)
print(json.dumps({"seqs": n, "sampled": float(lens[:n].sum()), "total": float(lens.sum()),
                  "s": dt, "threads": oracle.num_threads()}))
"""


def cpu_baseline_one_core(name: str, target_s: float = 10.0):
    """The oracle on one host thread (whole sequences, all heads, about
    target_s seconds), scaled to the whole batch by cached tokens."""
    import subprocess
    env = dict(os.environ, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-c", _ONE_CORE, os.path.dirname(os.path.abspath(__file__)),
                        name, str(target_s)], env=env, capture_output=True, text=True, timeout=600)
    if r.returncode != 0:
        raise RuntimeError(r.stderr[-2000:])
    d = json.loads(r.stdout.strip().splitlines()[-1])
    batch_s = d["s"] * d["total"] / max(d["sampled"], 1.0)
    import synth
    wl = synth.workload(name)
    return {"value": wl.batch / batch_s, "unit": "tokens/s", "cores": d["threads"], "kind": "oracle",
            "sample": f"{d['seqs']} of {wl.batch} sequences ({int(d['sampled'])} of {int(d['total'])} "
                      f"cached tokens), all {wl.heads} heads, one host thread, {d['s']:.1f} s; "
                      f"scaled to the whole batch by cached tokens"}


# workloads whose oracle is also timed on one thread
ONE_CORE_WORKLOADS = ("tiny_f32", "dsv2_b32_l2k")


def main():
    args = parse()
    if args.record_traffic:
        record_traffic(args.record_traffic, args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU mode "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import mla_latent_kv_15_amd as mla
    import synth
    from tests.device_inputs import DeviceInputs

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    torch.cuda.set_device(0)
    if args.stream_ceiling:
        stream_ceiling()
        return
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.mha:
        mha_baseline(args)
        return
    if args.prefill:
        prefill_bench(args)
        return

    wl = synth.workload(args.workload)
    S = args.splits or wl.num_splits
    args.decode_kernel = decode_kernel_of(args, wl)
    print(f"[bench] generating {wl.name}", file=sys.stderr, flush=True)
    inp = synth.make_inputs(wl)
    dev = DeviceInputs(inp)
    cache_bytes = synth.cache_bytes(wl, inp.seq_lens)
    per_replica = (cache_bytes + dev.w_uk.numel() * dev.w_uk.element_size() * 2
                   + dev.q_nope.numel() * 2 * 2)
    R = max(1, math.ceil(args.replica_bytes / per_replica))

    # replicas: same values at different addresses
    reps = []
    for r in range(R):
        c = dev.cache
        reps.append(dict(
            q_nope=dev.q_nope.clone(), q_rope=dev.q_rope.clone(), w_uk=dev.w_uk.clone(),
            w_uv=dev.w_uv.clone(),
            cache=mla.Cache(rows=c.rows.clone(), seq_lens=c.seq_lens.clone(),
                            max_seq_len=c.max_seq_len,
                            row_scale=None if c.row_scale is None else c.row_scale.clone(),
                            block_table=None if c.block_table is None else c.block_table.clone(),
                            seq_stride=c.seq_stride, page_size=c.page_size)))
    act = torch.float32 if wl.cache_dtype == "f32" else torch.bfloat16
    part = torch.float32 if args.part_dtype == "f32" else act
    out = torch.float32 if wl.out_dtype == "f32" else torch.bfloat16
    QL = args.q_len
    if QL > 1:
        return multi_token_bench(args, wl, dev, reps, R, S, act, part, out, cache_bytes)
    fp8q = query_dtype(args, wl) == "fp8"
    if fp8q and args.decode_kernel != "auto":
        raise SystemExit("an fp8 query runs its own decode kernel: use --decode-kernel auto")
    step = mla.DecodeStep(dev.geo, wl.batch, S, act_dtype=act, part_dtype=part, out_dtype=out,
                          fp8_query=fp8q)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    # tail of the step: with several splits and bf16 W_UV the merge and the
    # W_UV product run as one launch (mla_combine_up_proj; u is not stored)
    fused = step.fused_tail(dev.w_uv) and not args.two_call_tail

    kernel = {"auto": mla.KERNEL_AUTO, "h64": mla.KERNEL_H64,
              "balanced": mla.KERNEL_H64_BALANCED}[args.decode_kernel]

    def decode(rp, prepare=False):
        if fp8q:
            return mla.mla_decode(step.geo, step.q_abs, rp["cache"], S, step.u_part, step.lse_part,
                                  q_abs_scale=step.q_abs_scale, stream=stream, prepare=prepare)
        return mla.mla_decode_ex(step.geo, step.q_abs, rp["cache"], S, step.u_part, step.lse_part,
                                 kernel=kernel, stream=stream, prepare=prepare)

    # the step's launches in order: (name, fn(replica, prepare))
    stages = [("mla_absorb_q", lambda rp, prepare=False: mla.mla_absorb_q(
                  step.geo, rp["q_nope"], rp["q_rope"], rp["w_uk"], step.q_abs, step.q_abs_scale,
                  stream=stream, prepare=prepare)),
              ("mla_decode", decode)]
    if fused:
        stages.append(("mla_combine_up_proj", lambda rp, prepare=False: mla.mla_combine_up_proj(
            step.geo, step.u_part, step.lse_part, rp["w_uv"], step.o, stream=stream,
            prepare=prepare)))
    else:
        if S > 1:
            stages.append(("mla_combine", lambda rp, prepare=False: mla.mla_combine(
                step.geo, step.u_part, step.lse_part, step.u, step.lse, stream=stream,
                prepare=prepare)))
        stages.append(("mla_up_proj", lambda rp, prepare=False: mla.mla_up_proj(
            step.geo, step.u, rp["w_uv"], step.o, stream=stream, prepare=prepare)))
    # every launch validated and marshalled once per replica (mla.Call), so the
    # timed loop issues launches without the binding's per-call checks
    prepared = [[fn(rp, prepare=True) for _, fn in stages] for rp in reps]

    print(f"[bench] warmup {args.warmup}, R={R} replicas", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        for call in prepared[i % R]:
            call()
    torch.cuda.synchronize()

    # the timed region: K steps between two synchronisations; in every N-th
    # step an event on the launch stream before its first launch and after
    # each launch gives each kernel's per-launch duration (a sample of K / N
    # launches per kernel; the markers are left out of the other steps, which
    # a serving loop would run without them)
    every = max(1, args.events_every)
    n_inst = (args.steps + every - 1) // every
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
          for _ in range(n_inst)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        if i % every == 0:
            e = ev[i // every]
            e[0].record(stream)
            for j, call in enumerate(prepared[i % R]):
                call()
                e[j + 1].record(stream)
        else:
            for call in prepared[i % R]:
                call()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    per_launch = {name: [ev[i][j].elapsed_time(ev[i][j + 1]) * 1e3 for i in range(n_inst)]
                  for j, (name, _) in enumerate(stages)}
    kernel_stats = {name: launch_stats(us) for name, us in per_launch.items()}
    kernel_us = {name: st["mean"] for name, st in kernel_stats.items()}
    t_decode = kernel_us["mla_decode"] * 1e-6
    t_tail = sum(v for k, v in kernel_us.items() if k not in ("mla_absorb_q", "mla_decode")) * 1e-6

    # outside the step: the cache append that precedes it (each sequence's
    # last row is rewritten with a fresh bf16 row), timed the same way
    def loop_ms(fn):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            fn(reps[i % R])
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    g = torch.Generator(device="cuda").manual_seed(7)
    new_c = torch.randn(wl.batch, wl.d_latent, device="cuda", generator=g).to(act)
    new_r = torch.randn(wl.batch, wl.d_rope, device="cuda", generator=g).to(act)
    last = (dev.cache.seq_lens - 1).to(torch.int32)
    # a launch this small is shorter than the binding's per-call marshalling,
    # so the loop calls the C entry point with its arguments built once
    import ctypes
    L = mla.lib()
    geo_c = step.geo.c()
    cache_cs = [rp["cache"].c() for rp in reps]
    a_args = (wl.batch, new_c.data_ptr(), new_r.data_ptr(), mla.dtype_code(new_c), last.data_ptr())
    s_ptr = stream.cuda_stream
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        st = L.mla_cache_append(ctypes.byref(geo_c), *a_args, ctypes.byref(cache_cs[i % R]), s_ptr)
        assert st == 0, st
    e1.record(stream)
    torch.cuda.synchronize()
    outside_us = {"mla_cache_append": e0.elapsed_time(e1) / args.steps * 1e3}
    # and the absorb with the decoupled RoPE of q_R (the step's absorb variant
    # for callers whose q_R is not rotated yet)
    q_rope_out = (torch.empty(wl.batch, wl.heads, 576, dtype=act, device="cuda") if fp8q
                  else step.q_abs)  # the RoPE variant writes a bf16 / fp32 query
    # (calls prepared once per replica: the loop then measures the launches,
    # not the binding's argument checks)
    rope_calls = [mla.mla_absorb_q_rope(step.geo, rp["q_nope"], rp["q_rope"], rp["w_uk"], last,
                                        q_rope_out, stream=stream, prepare=True) for rp in reps]
    for c in rope_calls:
        c()
    rope_idx = {id(rp): i for i, rp in enumerate(reps)}
    outside_us["mla_absorb_q_rope"] = loop_ms(lambda rp: rope_calls[rope_idx[id(rp)]]()) * 1e3

    # roofline of the decode: algorithmic bytes of one launch (the cache rows
    # it attends) over its mean launch duration
    launch_bytes = cache_bytes
    achieved = launch_bytes / t_decode / 1e9
    key = traffic_key(wl.name, S, args.part_dtype, args.decode_kernel, "fp8" if fp8q else "bf16")
    counters = stored_counters(key)
    traffic = None if counters is None else counters.get("hbm_bytes_per_launch")
    # matrix-core work of the decode: 2 h (576 + 512) FLOP per attended token
    n_tok = float(np.sum(np.asarray(inp.seq_lens, np.float64)))
    dec_flops = n_tok * 2 * wl.heads * (576 + wl.d_latent)
    mfma_dt = "fp8" if step.q_abs.dtype == torch.uint8 else "bf16"  # the QK operand type
    mfma = {"algorithmic_flops_per_launch": dec_flops,
            "achieved_tflops": dec_flops / t_decode / 1e12,
            "peak_tflops": MFMA_PEAK_TFLOPS[mfma_dt],
            "frac_of_peak": dec_flops / t_decode / 1e12 / MFMA_PEAK_TFLOPS[mfma_dt],
            "busy_frac_from_counters": None}
    if counters is not None and "mfma_busy_cycles_per_launch" in counters:
        mfma["busy_frac_from_counters"] = (counters["mfma_busy_cycles_per_launch"] / N_SIMD
                                           / (t_decode * CLOCK_HZ))
    tokens_per_s = wl.batch / (ms_per_step * 1e-3)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(inp)
    cpu1 = None
    if not args.no_cpu_baseline and wl.name in ONE_CORE_WORKLOADS:
        print("[bench] cpu baseline on one thread (oracle)", file=sys.stderr, flush=True)
        cpu1 = cpu_baseline_one_core(wl.name)

    rec = {
        "metric": "MLA decode tokens/s + latent-KV HBM GB/s (% of MI355X peak), 1 GPU",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.cache_dtype == "bf16" else wl.cache_dtype,
        "data": "synthetic (seeded N(0,1) activations/cache, N(0,1/512) weights)",
        "config": {"workload": wl.name, "batch": wl.batch, "heads": wl.heads,
                   "d_nope": wl.d_nope, "d_rope": wl.d_rope, "d_latent": wl.d_latent,
                   "d_v": wl.d_v, "seq_len": int(inp.max_seq_len),
                   "tokens_attended": int(n_tok), "splits": S,
                   "cache": f"{wl.cache_dtype} {'paged' if wl.page_size else 'contiguous'}",
                   "partials": args.part_dtype, "decode_kernel": args.decode_kernel,
                   "query": "fp8" if fp8q else str(act).replace("torch.", ""),
                   "replicas": R, "parallelism": "none (1 GPU)"},
        # cache bytes over the time of the launches that handle the cache
        # stream: the decode and the merge of its partials (the fused tail
        # also applies W_UV)
        "cache_bytes": cache_bytes,
        "cache_GBps": cache_bytes / (t_decode + t_tail) / 1e9,
        "cache_pct_hbm_peak": 100.0 * cache_bytes / (t_decode + t_tail) / 1e9 / HBM_PEAK_GBPS,
        "cache_GBps_decode_only": achieved,
        "kernel_us": kernel_stats,
        # per-launch durations: events around the launches of every N-th timed step
        "launch_events": {"every_nth_step": every, "samples_per_kernel": n_inst},
        "outside_step_us_mean": outside_us,
        "mfma": mfma,
        "roofline": {"kernel": "mla_decode", "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": traffic, "algorithmic_bytes_per_launch": launch_bytes},
        "cpu_baseline": cpu,
        "cpu_baseline_one_thread": cpu1,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
