"""Benchmark of the Flint MoE block decode on one MI355X.

Workload: the full 47-layer stack at batch 1 (hidden 2048, 256 experts of 512,
top-6, shared expert 1024, int4 group 128, distinct seeded weights per layer,
the last ten layers with routed up-projection scales x 4096).  One step = one
token through all 47 layers (one forward call): RMSNorm, router, top-6,
gate/up + SwiGLU, down + combine, residual, per layer.  Tokens come from a pool
of 64 distinct seeded vectors already resident in HBM.

Prints one JSON line.  Use --gpus 1 (this build runs on one GPU).
"""
import argparse
import hashlib
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-block decode tokens/s and achieved HBM GB/s (47-layer int4, batch 1)"
N_LAYERS = 47
H, E, I, IS, K, G = 2048, 256, 512, 1024, 6, 128
PEAK_HBM_GBPS = 8000.0


def q4_bytes(rows, k):
    return rows * k // 2 + rows * (k // G) * 2


# Algorithmic bytes one token reads in one layer (what the hot path must read
# from HBM at least once): bf16 router + fp32 bias, and for each of the six
# routed experts plus the shared expert their int4 codes and bf16 scales.
EXPERT_BYTES = 2 * q4_bytes(I, H) + q4_bytes(H, I)            # 1,622,016
SHARED_BYTES = 2 * q4_bytes(IS, H) + q4_bytes(H, IS)          # 3,244,032
ROUTER_BYTES = E * H * 2 + E * 4                               # 1,049,600
LAYER_BYTES = ROUTER_BYTES + K * EXPERT_BYTES + SHARED_BYTES   # 14,025,728
TOKEN_BYTES = N_LAYERS * LAYER_BYTES                           # 659,209,216


# Sources each profiled kernel is compiled from: a counter summary holds only
# while these are unchanged.
KERNEL_SOURCES = {
    "decode": ("decode_persistent.hip", "decode_persistent.h", "decode_common.h", "decode.h", "flint_device.h"),
    "head": ("dense.hip", "dense.h", "flint_device.h"),
    "attn": ("attn.hip", "attn.h", "flint_device.h"),
}


def kernel_source_hash(which="decode"):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "int4_expert_ffn_amd", "csrc")
    for f in sorted(KERNEL_SOURCES[which]):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_stack47_traffic.txt")
DECODE_KERNEL = "k_decode_persistent"


def traffic_from_profiles(path=None, which="decode"):
    """HBM bytes per launch of a kernel from a committed rocprofv3 counter
    summary (the decode kernel by default), if it was taken on the current
    kernel sources; else None."""
    path = path or TRAFFIC_FILE
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_hash") != kernel_source_hash(which):
        return None
    return int(vals["hbm_bytes_per_launch"])


def _counter_values(run_dir, counter, name_pattern=None):
    """Per-dispatch values of one counter from a rocprofv3 --pmc csv output,
    keyed by kernel name (optionally only names containing name_pattern)."""
    import csv
    import glob
    out = {}
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                name = row.get("Kernel_Name", "")
                if name_pattern and name_pattern not in name:
                    continue
                out.setdefault(name, []).append(float(row["Counter_Value"]))
    return out


HEAD_KERNEL = "k_rows_mfma"
HEAD_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "head_kernel_traffic.txt")
HEAD_BYTES = 150144 * (H // 2) + 150144 * (H // G) * 2                # 158,552,064
ATT_KERNEL = "k_attn_chunk"
ATT_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_chunk_traffic.txt")
ATT_POSITIONS = 100000
ATT_BYTES_PER_POS = 2 * 4 * 128 * 2        # k and v rows of the 4 KV heads, bf16
# one batch-1 full-layer call: the cache, q, out and the sinks
ATT_CALL_BYTES = ATT_POSITIONS * ATT_BYTES_PER_POS + 2 * 32 * 128 * 4 + 32 * 4   # 204,832,896


def summarize_counters(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, commands, which="decode"):
    """Write the traffic summary from four rocprofv3 --pmc runs: the benchmark
    (FETCH_SIZE, WRITE_SIZE, KiB per dispatch of its dominant kernel) and a
    plain 1 GiB device copy (the same two counters) that calibrates them.
    which: "decode" (47-layer decode launch), "head" (output head launch) or
    "attn" (the chunk kernel of a batch-1 full attention layer)."""
    kernel, out_file, algo, title = {
        "decode": (DECODE_KERNEL, TRAFFIC_FILE, TOKEN_BYTES,
                   "# HBM traffic of one decode launch (47-layer Flint MoE stack, batch 1, the bench workload)"),
        "head": (HEAD_KERNEL, HEAD_TRAFFIC_FILE, HEAD_BYTES,
                 "# HBM traffic of one output-head launch (150,144 x 2,048 int4, bench.py --head-dense workload)"),
        "attn": (ATT_KERNEL, ATT_TRAFFIC_FILE, ATT_CALL_BYTES,
                 "# HBM traffic of one attention chunk launch (full layer, 100,000 positions, 1 token; "
                 "bench.py --attn --attn-batch1 workload; the algorithmic bytes are the whole call's)"),
    }[which]
    def one(d, counter, pattern):
        vals = _counter_values(d, counter, pattern)
        if not vals:
            raise SystemExit(f"no {counter} rows for {pattern or 'any kernel'} under {d}")
        name = max(vals, key=lambda k: len(vals[k]))
        return name, vals[name]
    copy_bytes = 1 << 30
    kname, f = one(fetch_dir, "FETCH_SIZE", kernel)
    _, w = one(write_dir, "WRITE_SIZE", kernel)
    cf = max(max(v) for v in _counter_values(copy_fetch_dir, "FETCH_SIZE").values())
    cw_all = _counter_values(copy_write_dir, "WRITE_SIZE")
    cw = max(max(v) for v in cw_all.values())
    f_factor = copy_bytes / (cf * 1024.0)
    w_factor = copy_bytes / (cw * 1024.0)
    f_kib, w_kib = float(np.median(f)), float(np.median(w))
    total = f_kib * 1024.0 * f_factor + w_kib * 1024.0 * w_factor
    lines = [
        title,
        "# from rocprofv3 --pmc, one counter per run, calibrated with a plain 1 GiB device copy",
        f"kernel: {kname}",
        f"kernel_source_hash: {kernel_source_hash(which)}",
        f"kernel_sources: {' '.join(KERNEL_SOURCES[which])}",
        f"dispatches_fetch: {len(f)}",
        f"fetch_kib_per_dispatch_median: {f_kib:.1f}",
        f"write_kib_per_dispatch_median: {w_kib:.1f}",
        f"copy_fetch_kib: {cf:.1f}",
        f"copy_write_kib: {cw:.1f}",
        f"fetch_factor: {f_factor:.4f}",
        f"write_factor: {w_factor:.4f}",
        f"hbm_bytes_per_launch: {int(round(total))}",
        f"algorithmic_bytes_per_launch: {algo}",
        f"traffic_over_algorithmic: {total / algo:.3f}",
    ] + [f"command: {c}" for c in commands]
    os.makedirs(os.path.dirname(out_file), exist_ok=True)
    with open(out_file, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


PEAK_BF16_TFLOPS = 2500.0
PF_TOKENS = 2048


def prefill_flops(n):
    """Algorithmic flops of one layer for n tokens: router GEMM, routed gate/up
    and down for the n x 6 (token, expert) pairs, shared gate/up and down."""
    return {"router": 2 * n * E * H, "routed_gate_up": 2 * 2 * n * K * I * H, "routed_down": 2 * n * K * H * I,
            "shared_gate_up": 2 * 2 * n * IS * H, "shared_down": 2 * n * H * IS}


def prefill_roofline(flops, bytes_moved, layer_s):
    """The layer against both roofs: at 48 (token, slot) pairs per expert a
    weight byte carries about 190 flops, under the chip's 312 (2.5 PFLOP/s over
    8 TB/s), so the weight stream, not the matrix cores, bounds the layer.  The
    binding roof is the one whose time at peak is longer; the other is reported
    beside it."""
    t_hbm = bytes_moved / (PEAK_HBM_GBPS * 1e9)
    t_mfma = flops / (PEAK_BF16_TFLOPS * 1e12)
    gbps = bytes_moved / layer_s / 1e9
    tflops = flops / layer_s / 1e12
    hbm = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
           "frac": round(gbps / PEAK_HBM_GBPS, 4)}
    mfma = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4)}
    main, other = (hbm, mfma) if t_hbm >= t_mfma else (mfma, hbm)
    return dict(main, traffic=None, kernel="whole layer (9 launches)", layer_us_median=round(layer_s * 1e6, 2),
                us_at_peak={"hbm": round(t_hbm * 1e6, 2), "mfma": round(t_mfma * 1e6, 2)}, other_roof=other,
                bytes_per_layer=int(bytes_moved))


def bench_prefill(args):
    """One real-shape layer, 2,048 tokens, Zipf-skewed router bias."""
    import torch
    import flintgen as fg
    import int4_expert_ffn_amd as F
    synth = fg.Synth(fg.FLINT, seed=0, n_layers=1, bias_kind="zipf")
    model = _track(F.FlintMoE([synth.layer(0, "cuda")]))
    torch.cuda.empty_cache()
    n = PF_TOKENS
    ids = torch.full((1, n, K), -1, dtype=torch.int32, device="cuda")
    wts = torch.zeros((1, n, K), dtype=torch.float32, device="cuda")
    model.set_trace(ids, wts, n)
    x = torch.from_numpy(fg.tokens(0, range(2000, 2000 + n))).cuda()
    out = torch.empty_like(x)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        F.flint_moe_forward(model.h, x, n, 0, 1, out, stream)
    torch.cuda.synchronize()
    model.status()
    used = int((torch.bincount(ids[0].flatten().long(), minlength=E) > 0).sum().item())
    model.set_trace(None, None, 0)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        F.flint_moe_forward(model.h, x, n, 0, 1, out, stream)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    model.status()
    durs = np.array([a.elapsed_time(b) for a, b in ev]) * 1e-3
    layer_s = float(np.median(durs))
    flops = prefill_flops(n)
    total = sum(flops.values())
    weight_bytes = ROUTER_BYTES + used * EXPERT_BYTES + SHARED_BYTES
    act_bytes = 2 * n * H * 4
    res = {
        "metric": "MoE-block prefill tokens/s (one layer, 2048-token chunk)",
        "value": round(n / layer_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int4xbf16->fp32 (MFMA bf16)",
        "data": "synthetic (seeded int4 weights, bf16 scales, Zipf-skewed router bias, N(0,1) tokens)",
        "config": {"workload": "one Flint MoE layer, 2048-token prefill chunk", "tokens": n, "experts_used": used,
                   "algorithmic_flops": total, "flops_by_part": flops},
        "roofline": prefill_roofline(total, weight_bytes + act_bytes, layer_s),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_prefill(args.cpu_seconds)
    print(json.dumps(res), flush=True)


_OPEN_MODELS = []


def _track(model):
    """Remember a library handle so that main() closes it before returning:
    released at interpreter exit instead, its device memory would be freed
    while the HIP runtime (and a profiler's hooks) are shutting down."""
    _OPEN_MODELS.append(model)
    return model


def _close_models():
    """Close the library handles and hand PyTorch's cached device blocks back
    to the runtime while the process is still running."""
    import gc
    import torch
    if not torch.cuda.is_available():
        return
    torch.cuda.synchronize()
    while _OPEN_MODELS:
        _OPEN_MODELS.pop().close()
    gc.collect()
    torch.cuda.empty_cache()
    torch.cuda.synchronize()


def build_stack_model(dev, interm_div=0):
    """The 47-layer stack on ``dev``; interm_div > 0 gives the fp16-intermediate
    pack form of the same weights (routed up scales divided by it)."""
    import torch
    import flintgen as fg
    import int4_expert_ffn_amd as F
    synth = fg.flint_stack(0, N_LAYERS, up_div=interm_div or 1)
    layers = [synth.layer(l, dev) for l in range(N_LAYERS)]
    torch.cuda.synchronize()
    model = _track(F.FlintMoE(layers, interm_div=interm_div))
    del layers
    torch.cuda.empty_cache()
    return model


COST_TABLE_FILE = os.path.join(ROOT, "profiles", "decode_cost_table_stack47.txt")


def bench_cost_table(args):
    """Verify-block cost table: one forward call of n = 1..16 independent tokens
    through the 47 layers (the decode path), median time per call.  Algorithmic
    bytes per call count each layer's router, shared expert and the distinct
    routed experts the call's tokens picked (from the trace).  --interm-div
    gives the fp16-intermediate pack form of the same weights."""
    import torch
    import flintgen as fg
    import int4_expert_ffn_amd as F
    dev = torch.device("cuda:0")
    model = build_stack_model(dev, args.interm_div)
    cap = 16
    pool = torch.from_numpy(fg.tokens(0, range(64))).to(dev)
    ids = torch.full((N_LAYERS, cap, K), -1, dtype=torch.int32, device=dev)
    wts = torch.zeros((N_LAYERS, cap, K), dtype=torch.float32, device=dev)
    out = torch.empty((cap, H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    batches = 4                         # distinct token batches per n, used in turn
    rows = []
    ns = [int(v) for v in args.cost_table_tokens.split(",")] if args.cost_table_tokens else range(1, cap + 1)
    for n in ns:
        xs = [pool[b * 16:b * 16 + n] for b in range(batches)]
        # distinct experts per layer of each batch, from one traced call
        model.set_trace(ids, wts, cap)
        call_bytes = []
        for x in xs:
            F.flint_moe_forward(model.h, x, n, 0, N_LAYERS, out, stream)
            torch.cuda.synchronize()
            tr = ids[:, :n].cpu().numpy()
            distinct = [len(np.unique(tr[l])) for l in range(N_LAYERS)]
            call_bytes.append(sum(ROUTER_BYTES + SHARED_BYTES + d * EXPERT_BYTES for d in distinct))
        model.set_trace(None, None, 0)
        for i in range(args.warmup):
            F.flint_moe_forward(model.h, xs[i % batches], n, 0, N_LAYERS, out, stream)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            ev[i][0].record(stream)
            F.flint_moe_forward(model.h, xs[i % batches], n, 0, N_LAYERS, out, stream)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        model.status()
        durs = np.array([a.elapsed_time(b) for a, b in ev]) * 1e-3
        med = float(np.median(durs))
        mean_bytes = float(np.mean([call_bytes[i % batches] for i in range(args.steps)]))
        rows.append({"n": n, "us_median": round(med * 1e6, 1),
                     "us_p10": round(float(np.percentile(durs, 10)) * 1e6, 1),
                     "us_p90": round(float(np.percentile(durs, 90)) * 1e6, 1),
                     "tokens_per_s": round(n / med, 1),
                     "distinct_experts_per_layer": round((mean_bytes / N_LAYERS - ROUTER_BYTES - SHARED_BYTES)
                                                         / EXPERT_BYTES, 2),
                     "algorithmic_bytes": int(mean_bytes),
                     "gbps": round(mean_bytes / med / 1e9, 1)})
        print(f"n={n}: {rows[-1]}", file=sys.stderr, flush=True)
    if args.cost_table_out:
        with open(args.cost_table_out, "w") as f:
            form = (f"fp16-intermediate form (routed up projections / {args.interm_div})" if args.interm_div
                    else "fp32 intermediates")
            f.write("# Verify-block cost table: one flint_moe_forward call of n independent tokens through the\n"
                    f"# 47-layer stack (decode path, {form}), hip events on the launch stream, "
                    f"{args.steps} timed calls per n after {args.warmup} warm-up, 4 token batches per n in turn.\n"
                    "# bytes: router + shared + distinct routed experts per layer (from the trace), summed over layers.\n"
                    "# command: python bench.py --cost-table --steps "
                    f"{args.steps} --warmup {args.warmup}"
                    + (f" --interm-div {args.interm_div}" if args.interm_div else "") + " --cost-table-out <file>\n")
            f.write("n,us_median,us_p10,us_p90,tokens_per_s,distinct_experts_per_layer,algorithmic_bytes,gbps,frac_of_8tbs\n")
            for r in rows:
                f.write(f"{r['n']},{r['us_median']},{r['us_p10']},{r['us_p90']},{r['tokens_per_s']},"
                        f"{r['distinct_experts_per_layer']},{r['algorithmic_bytes']},{r['gbps']},"
                        f"{r['gbps'] / PEAK_HBM_GBPS:.4f}\n")
    print(json.dumps({"metric": "verify-block cost table (47-layer decode call time for n = 1..16 tokens)",
                      "unit": "us per call", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                      "data": "synthetic (seeded int4 weights, bf16 scales, N(0,1) tokens)",
                      "config": {"workload": "47-layer Flint MoE block stack, n independent tokens per call",
                                 "interm_div": args.interm_div},
                      "table": rows}), flush=True)


def q4_matrix_bytes(rows, k):
    return rows * (k // 2) + rows * (k // G) * 2


def bench_head_dense(args):
    """The model's other int4 GEMVs at batch 1: the output head (150,144 x 2,048)
    and the dense SwiGLU MLP of layers 0 and 1 (width 6,144).  Timed launches
    rotate through enough copies of the weights that the 256 MB last-level
    cache cannot hold them, so every launch streams its weights from HBM."""
    import torch
    import flintgen as fg
    import int4_expert_ffn_amd as F
    dev = torch.device("cuda:0")
    rows, inter = fg.VOCAB, fg.DENSE_MLP_SIZE
    heads = [fg.head(0, device=dev) for _ in range(3)]                     # 3 x 158.5 MB
    denses = [fg.dense_layer(0, i % 2, device=dev) for i in range(16)]     # 16 x 19.5 MB
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    pool = torch.from_numpy(fg.tokens(0, range(64))).to(dev)
    logits = torch.empty((16, rows), dtype=torch.float32, device=dev)
    hbuf = torch.empty((16, inter), dtype=torch.float32, device=dev)
    xo = torch.empty((16, H), dtype=torch.float32, device=dev)

    def head_call(i, n):
        c, sc = heads[i % len(heads)]
        F.flint_head_forward(F.q4(c, sc), rows, pool[i % 48:i % 48 + n], n, logits, stream)

    def dense_call(i, n):
        w = denses[i % len(denses)]
        F.flint_dense_mlp_forward(F.q4(w["gate"], w["gate_s"]), F.q4(w["up"], w["up_s"]), F.q4(w["down"], w["down_s"]),
                                  inter, pool[i % 48:i % 48 + n], n, hbuf, xo, stream)

    def timed(fn, n):
        for i in range(args.warmup):
            fn(i, n)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            ev[i][0].record(stream)
            fn(i, n)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        d = np.array([a.elapsed_time(b) for a, b in ev]) * 1e-3
        return float(np.median(d)), float(np.percentile(d, 10)), float(np.percentile(d, 90))

    head_bytes = q4_matrix_bytes(rows, H)
    dense_bytes = 2 * q4_matrix_bytes(inter, H) + q4_matrix_bytes(H, inter)
    res_head = {n: timed(head_call, n) for n in (1, 4, 16)}
    res_dense = {n: timed(dense_call, n) for n in (1, 4, 16)}
    med = res_head[1][0]
    achieved = (head_bytes + rows * 4 + H * 4) / med / 1e9
    out = {
        "metric": "output-head int4 GEMV achieved HBM GB/s (150,144 x 2,048, batch 1)",
        "value": round(achieved, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(med * 1e3, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int4xbf16->fp32", "data": "synthetic (seeded int4 weights, bf16 scales, N(0,1) tokens)",
        "config": {"workload": "output head 150,144 x 2,048 int4 and dense SwiGLU MLP 2,048 -> 6,144 -> 2,048, "
                               "decode", "head_bytes": head_bytes, "dense_mlp_bytes": dense_bytes},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic_from_profiles(HEAD_TRAFFIC_FILE, "head"),
                     "kernel": "k_rows_mfma (head, one launch)"},
        "head_us": {str(n): [round(v * 1e6, 2) for v in r] for n, r in res_head.items()},
        "dense_mlp_us": {str(n): [round(v * 1e6, 2) for v in r] for n, r in res_dense.items()},
        "dense_mlp_gbps_batch1": round(dense_bytes / res_dense[1][0] / 1e9, 1),
        "timing_note": "median, p10, p90 of hip-event launch durations; the head and MLP weights rotate over "
                       "3 and 16 copies so the working set exceeds the last-level cache",
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_head(args.cpu_seconds)
    print(json.dumps(out), flush=True)


def bench_attn(args):
    """Decode attention with learned sinks: a full layer at 100,000 positions
    (the recipe's 100K decode context) for 1, 4 and 16 query tokens at
    consecutive positions, and a window layer (513 positions in the 640-row
    ring).  Two full-layer caches rotate so that the 256 MB last-level cache
    cannot hold the 205 MB being read."""
    import torch
    import flintgen as fg
    import int4_expert_ffn_amd as F
    dev = torch.device("cuda:0")
    n_pos = ATT_POSITIONS
    caches = []
    for i in range(2):
        kb, vb = fg.attn_cache(0, 10 + i, n_pos)
        caches.append((torch.from_numpy(kb).to(dev), torch.from_numpy(vb).to(dev)))
    wk, wv = (torch.from_numpy(x).to(dev) for x in fg.attn_cache(0, 20, fg.ATT_RING))
    sinks = torch.from_numpy(fg.attn_sinks(0, 10)).to(dev)
    q = torch.from_numpy(fg.attn_queries(0, 10, 16)).to(dev)
    out = torch.empty((16, 32, 128), dtype=torch.float32, device=dev)
    wsb = F.flint_attn_workspace_bytes(16, n_pos)
    ws = torch.empty(wsb // 4 + 4, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def timed(call):
        for i in range(args.warmup):
            call(i)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            ev[i][0].record(stream)
            call(i)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        d = np.array([a.elapsed_time(b) for a, b in ev]) * 1e-3
        return float(np.median(d)), float(np.mean(d)), float(np.percentile(d, 10)), float(np.percentile(d, 90))

    def full(n):
        pos = [n_pos - n + i for i in range(n)]
        def call(i):
            k, v = caches[i % 2]
            F.flint_attn_decode(q, k, v, n_pos, sinks, pos, n, 0, out, ws, wsb, stream)
        return call

    def window(n):
        pos = [5000 + i for i in range(n)]
        return lambda i: F.flint_attn_decode(q, wk, wv, fg.ATT_RING, sinks, pos, n, fg.ATT_WINDOW, out, ws, wsb, stream)

    res_full = {n: timed(full(n)) for n in ((1,) if args.attn_batch1 else (1, 4, 16))}
    res_win = {} if args.attn_batch1 else {n: timed(window(n)) for n in (1, 16)}
    med, mean = res_full[1][0], res_full[1][1]
    algo = ATT_CALL_BYTES
    achieved = algo / mean / 1e9
    outj = {
        "metric": "decode attention with sinks, achieved HBM GB/s (full layer, 100,000 positions, batch 1)",
        "value": round(algo / med / 1e9, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(med * 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 KV x fp32 q (MFMA bf16, q in three parts) -> fp32",
        "data": "synthetic (seeded N(0,1) q, k, v; sink logits U(-9, 12.4))",
        "config": {"workload": "one full attention layer at 100,000 positions and one window layer (513 of a "
                               "640-row ring), 32 query / 4 KV heads of 128", "positions": n_pos,
                   "algorithmic_bytes_batch1": algo},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": traffic_from_profiles(ATT_TRAFFIC_FILE, "attn"),
                     "traffic_note": "HBM bytes of the chunk kernel alone (rocprofv3 counters); the combine adds the "
                                     "partials' read",
                     "kernel": "k_attn_chunk + k_attn_combine (one call, hip events; mean duration)"},
        "full_layer_us": {str(n): [round(v * 1e6, 2) for v in (r[0], r[2], r[3])] for n, r in res_full.items()},
        "window_layer_us": {str(n): [round(v * 1e6, 2) for v in (r[0], r[2], r[3])] for n, r in res_win.items()},
        "timing_note": "median, p10, p90 of hip-event call durations; n tokens at consecutive positions share the "
                       "cache, which each call reads once per token",
    }
    if not args.no_cpu_baseline:
        outj["cpu_baseline"] = cpu_baseline_attn(args.cpu_seconds)
    print(json.dumps(outj), flush=True)


def cpu_baseline_attn(seconds_budget=20.0):
    """The CPU oracle on a bounded sample: one token of a full layer at 100,000
    positions (all 32 query heads, one oracle call, repeated while the budget
    allows); scaled to GB/s of cache read."""
    import flintgen as fg
    import torch
    from oracle import flint_oracle as O
    n_pos = 100000
    kb, vb = fg.attn_cache(0, 10, n_pos)
    k = torch.from_numpy(kb).view(torch.bfloat16).double().numpy()
    v = torch.from_numpy(vb).view(torch.bfloat16).double().numpy()
    q = fg.attn_queries(0, 10, 1)[0].astype(np.float64)
    sinks = fg.attn_sinks(0, 10)
    t0 = time.perf_counter()
    calls = 0
    while True:
        O.attention_decode(q, k, v, sinks, n_pos - 1, 0)
        calls += 1
        if time.perf_counter() - t0 > min(seconds_budget, 5.0) or calls >= 20:
            break
    dt = (time.perf_counter() - t0) / calls
    return {"value": round(n_pos * ATT_BYTES_PER_POS / dt / 1e9, 4), "unit": "GB/s", "cores": _oracle_threads(),
            "kind": "oracle", "sample": f"one token, 32 query heads, 100,000 positions; {calls} oracle calls, "
                                        f"{dt:.2f} s each"}


def measure_copy_gbps(torch, dev, n_bytes=1 << 30, reps=10):
    """Bandwidth of a plain device-to-device copy of 1 GiB (read + write bytes
    per second, hip events): the attainable HBM rate the roofline fraction can
    also be read against."""
    a = torch.empty(n_bytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3 / reps
    del a, b
    torch.cuda.empty_cache()
    return 2 * n_bytes / sec / 1e9


def _oracle_threads():
    try:
        import threadpoolctl
        return int(max((p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()), default=1))
    except Exception:
        return 1


def cpu_baseline_prefill(seconds_budget=20.0):
    """The CPU oracle on a bounded sample of the prefill workload: tokens of the
    2,048-token Zipf chunk through the layer, one at a time (the oracle has no
    batched path), scaled to tokens/s through one layer."""
    import flintgen as fg
    from oracle import flint_oracle as O
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from oracle_sources import SynthSource
    synth = fg.Synth(fg.FLINT, seed=0, n_layers=1, bias_kind="zipf")
    src = SynthSource(synth)
    t0 = time.perf_counter()
    done = 0
    for t in range(PF_TOKENS):
        x = fg.token(0, 2000 + t)
        O.moe_block(O.block_input(x, fg.FLINT), src, 0, fg.FLINT)
        done += 1
        if time.perf_counter() - t0 > seconds_budget:
            break
    dt = time.perf_counter() - t0
    return {"value": round(done / dt, 4), "unit": "tokens/s", "cores": _oracle_threads(), "kind": "oracle",
            "sample": f"the first {done} tokens of the 2,048-token chunk through layer 0 ({dt:.1f} s, weights "
                      f"regenerated per token included)"}


def cpu_baseline_head(seconds_budget=20.0):
    """The CPU oracle on a bounded sample of the head: logits of one token for
    blocks of 4,096 rows, timing the oracle call only; scaled to GB/s of int4
    weights processed."""
    import flintgen as fg
    from oracle import flint_oracle as O
    x = fg.token(0, 40)
    spent, rows = 0.0, 0
    while spent < seconds_budget and rows < fg.VOCAB:
        r1 = min(rows + 4096, fg.VOCAB)
        c, sc = fg.head(0, row_ids=range(rows, r1))
        t0 = time.perf_counter()
        O.head_logits(x, c.numpy(), sc.numpy(), fg.FLINT)
        spent += time.perf_counter() - t0
        rows = r1
    gbps = rows * (H // 2 + (H // G) * 2) / spent / 1e9
    return {"value": round(gbps, 4), "unit": "GB/s", "cores": _oracle_threads(), "kind": "oracle",
            "sample": f"one token, head rows 0..{rows - 1} in blocks of 4,096 ({spent:.1f} s of oracle time)"}


class _CachedLayers:
    """Oracle source over tensors generated before the clock starts: the
    router, bias, shared expert and the experts a token selects, per layer."""

    def __init__(self, synth, picks):
        self.router_ = {l: synth.router(l).numpy() for l in picks}
        self.bias_ = {l: synth.bias(l).numpy() for l in picks}
        self.shared_ = {l: {k: v.numpy() for k, v in synth.shared(l).items()} for l in picks}
        self.ex_ = {l: (list(ids), {k: v.numpy() for k, v in synth.experts(l, list(ids)).items()})
                    for l, ids in picks.items()}

    def router(self, l):
        return self.router_[l]

    def bias(self, l):
        return self.bias_[l]

    def shared(self, l):
        return self.shared_[l]

    def experts(self, l, ids):
        have, d = self.ex_[l]
        idx = [have.index(int(e)) for e in ids]
        return {k: v[idx] for k, v in d.items()}


def cpu_baseline(seconds_budget=20.0, interm_div=0):
    """The CPU oracle (fp64 NumPy, explicit dequantisation, full sort) timed
    alone: one token through the 47-layer stack, with every tensor the token
    touches generated before the clock starts (a first, untimed pass finds
    the experts it selects).  Reported: tokens/s through the 47 layers with
    the BLAS library's threads, the one-layer rate (the single-layer
    workload), and the same with one thread.  Each timed pass stops early
    past its share of the budget and is scaled to the 47 layers.
    interm_div > 0: the oracle's fp16-intermediate form on the pack weights."""
    import flintgen as fg
    from oracle import flint_oracle as O
    import threadpoolctl
    synth = fg.flint_stack(0, N_LAYERS, up_div=interm_div or 1)

    def block(a, src, l):
        return (O.moe_block_fp16_interm(a, src, l, fg.FLINT, interm_div) if interm_div
                else O.moe_block(a, src, l, fg.FLINT))

    class _Lazy:   # the untimed pass: generates on demand, records the picks
        def __init__(self):
            self.picks = {}

        def router(self, l):
            return synth.router(l).numpy()

        def bias(self, l):
            return synth.bias(l).numpy()

        def shared(self, l):
            return {k: v.numpy() for k, v in synth.shared(l).items()}

        def experts(self, l, ids):
            self.picks[l] = [int(e) for e in ids]
            return {k: v.numpy() for k, v in synth.experts(l, ids).items()}

    x0 = fg.token(0, 0)
    lazy = _Lazy()
    x = x0
    for l in range(N_LAYERS):
        x = (x.astype(np.float64) + block(O.block_input(x, fg.FLINT), lazy, l).delta).astype(np.float32)
    src = _CachedLayers(synth, lazy.picks)

    def timed(budget):
        x, per_layer = x0, []
        t_start = time.perf_counter()
        for l in range(N_LAYERS):
            t0 = time.perf_counter()
            res = block(O.block_input(x, fg.FLINT), src, l)
            per_layer.append(time.perf_counter() - t0)
            x = (x.astype(np.float64) + res.delta).astype(np.float32)
            if time.perf_counter() - t_start > budget:
                break
        return per_layer

    threads = _oracle_threads()
    all_t = timed(seconds_budget * 0.6)
    with threadpoolctl.threadpool_limits(1):
        one_t = timed(seconds_budget * 0.4)
    per_token = float(np.mean(all_t)) * N_LAYERS
    per_token_1 = float(np.mean(one_t)) * N_LAYERS
    return {"value": round(1.0 / per_token, 6), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"1 token through layers 0..{len(all_t) - 1} of the 47-layer stack, oracle calls only "
                      f"(tensors generated before timing), scaled to 47 layers",
            "cpu_count": os.cpu_count(),
            "one_layer_tokens_per_s": round(1.0 / float(np.mean(all_t)), 4),
            "one_thread_tokens_per_s": round(1.0 / per_token_1, 6),
            "one_thread_sample_layers": len(one_t)}


# Phase markers of the decode kernel's profiling build (thread 0 of each
# workgroup records the wall clock at marker k of layer l): the phases are the
# intervals between consecutive markers of one workgroup.
PHASES = (("x gather", 0, 1), ("norm (block input)", 1, 2), ("router (and the shared rows' wait)", 2, 4),
          ("(c, s) gather", 4, 5), ("routing (top-6, weights)", 5, 7), ("gate/up", 7, 8),
          ("h gather", 8, 9), ("down and combine", 9, 10))


def bench_exchange_probe(args):
    """XCD placement of a 256-workgroup launch and the round trip of one value
    between two workgroups with the exchanges' store and load policies
    (profiling build libflint_moe_phase.so, flint_moe_debug_exchange_probe)."""
    import int4_expert_ffn_amd as F
    F.LIB_PATH = os.path.join(F.HERE, "libflint_moe_phase.so")
    if not os.path.exists(F.LIB_PATH):
        raise FileNotFoundError(f"{F.LIB_PATH} is missing: python -m int4_expert_ffn_amd.build --phase-ts")
    L = F.lib()
    L.flint_moe_debug_exchange_probe.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    L.flint_moe_debug_exchange_probe.restype = ctypes.c_int
    xcc = np.zeros(256, dtype=np.int32)
    rt = np.zeros(3, dtype=np.float64)
    rc = L.flint_moe_debug_exchange_probe(xcc.ctypes.data, rt.ctypes.data)
    assert rc == 0, rc
    round_robin = int(np.sum(xcc == np.arange(256) % 8))
    lines = ["# exchange probe: XCD of each workgroup of a 256-workgroup launch (XCC_ID register) and the round trip",
             "# of one 32-bit value between workgroup 0 and another (stored by one, polled by the other, back), 2,000 rounds",
             "# command: python -m int4_expert_ffn_amd.build --phase-ts && python bench.py --exchange-probe",
             f"workgroups on XCD w % 8: {round_robin} of 256",
             f"xcd of workgroups 0..15: {' '.join(str(int(v)) for v in xcc[:16])}",
             f"round trip, agent-scope store / sc1 poll, same XCD: {rt[0]:.3f} us",
             f"round trip, agent-scope store / sc1 poll, other XCD: {rt[1]:.3f} us",
             f"round trip, sc0 store / sc1 poll, same XCD: {rt[2]:.3f} us"]
    print("\n".join(lines))
    if args.exchange_probe_out:
        with open(args.exchange_probe_out, "w") as f:
            f.write("\n".join(lines) + "\n")


def bench_phase_table(args):
    """Phase durations of the single-token decode kernel (profiling build
    libflint_moe_phase.so): median over workgroups and over layers 1..46 of
    10 calls of the bench workload (47 layers, 1 token)."""
    import torch
    import flintgen as fg
    import int4_expert_ffn_amd as F
    F.LIB_PATH = os.path.join(F.HERE, "libflint_moe_phase.so")
    if not os.path.exists(F.LIB_PATH):
        raise FileNotFoundError(f"{F.LIB_PATH} is missing: python -m int4_expert_ffn_amd.build --phase-ts")
    L = F.lib()
    L.flint_moe_debug_phase_ts.argtypes = [ctypes.c_void_p]
    L.flint_moe_debug_phase_ts.restype = ctypes.c_int
    dev = torch.device("cuda", 0)
    model = build_stack_model(dev, args.interm_div)
    pool = torch.from_numpy(fg.tokens(0, range(64))).to(dev)
    out = torch.empty((1, H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    nl, nm, nwg = 48, 16, 256
    buf = np.zeros((nl, nm, nwg), dtype=np.uint64)
    for i in range(args.warmup):
        F.flint_moe_forward(model.h, pool[i % 64:i % 64 + 1], 1, 0, N_LAYERS, out, stream)
    torch.cuda.synchronize()
    per_phase = [[] for _ in PHASES]
    layer_us = []
    for i in range(10):
        F.flint_moe_forward(model.h, pool[i % 64:i % 64 + 1], 1, 0, N_LAYERS, out, stream)
        torch.cuda.synchronize()
        rc = L.flint_moe_debug_phase_ts(buf.ctypes.data)
        assert rc == 0, rc
        ts = buf.astype(np.float64) * 0.01   # 100 MHz ticks -> us
        for l in range(1, N_LAYERS):
            for p, (_, a, b) in enumerate(PHASES):
                per_phase[p].extend((ts[l][b] - ts[l][a]).tolist())
            layer_us.extend((ts[l][10] - ts[l - 1][10]).tolist())
    model.status()
    if args.phase_raw_out:   # raw per-workgroup timestamps of the last call, for inspection
        np.save(args.phase_raw_out, buf)
    lines = ["# decode phase table: 47-layer stack, 1 token; per-workgroup phase durations, median over"
             " the 256 workgroups and layers 1..46 of 10 calls",
             "# command: python -m int4_expert_ffn_amd.build --phase-ts && python bench.py --phase-table"
             + (f" --interm-div {args.interm_div}" if args.interm_div else ""),
             f"# kernel_sources_sha16: {kernel_source_hash('decode')}",
             f"# layer time (marker to marker): {np.median(layer_us):.2f} us",
             "phase, us"]
    for p, (name, _, _) in enumerate(PHASES):
        lines.append(f"{name:40s} {np.median(per_phase[p]):7.2f}")
    text = "\n".join(lines)
    print(text, flush=True)
    if args.phase_table_out:
        with open(args.phase_table_out, "w") as f:
            f.write(text + "\n")


def main():
    try:
        return _main()
    finally:
        _close_models()


def _main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for counter calibration)")
    ap.add_argument("--counters-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="write the traffic summary under profiles/ from four rocprofv3 --pmc output folders")
    ap.add_argument("--command", action="append", default=[], help="command lines recorded in the summary")
    ap.add_argument("--counters-kernel", choices=("decode", "head", "attn"), default="decode",
                    help="which kernel --counters-summary summarises")
    ap.add_argument("--prefill", action="store_true",
                    help="time the prefill path instead: one layer, a 2048-token chunk")
    ap.add_argument("--head-dense", action="store_true",
                    help="time the output head and the dense MLP int4 GEMVs instead (batch 1, 4, 16)")
    ap.add_argument("--cost-table", action="store_true",
                    help="time one 47-layer call for n = 1..16 tokens (verify-block cost table)")
    ap.add_argument("--cost-table-out", default=None, help="write the cost table (CSV with a header) to this file")
    ap.add_argument("--attn", action="store_true",
                    help="time the decode attention with sinks instead (full layer at 100,000 positions, window layer)")
    ap.add_argument("--attn-batch1", action="store_true",
                    help="with --attn: only the batch-1 full layer (for a kernel trace of that one shape)")
    ap.add_argument("--cost-table-tokens", default=None,
                    help="comma-separated token counts for --cost-table (default 1..16)")
    ap.add_argument("--exchange-probe", action="store_true",
                    help="XCD placement and workgroup-to-workgroup round trips (profiling build)")
    ap.add_argument("--exchange-probe-out", default=None, help="write the probe's summary to this file")
    ap.add_argument("--phase-table", action="store_true",
                    help="decode phase timestamps (needs the --phase-ts build of the library)")
    ap.add_argument("--phase-table-out", default=None, help="write the phase table to this file")
    ap.add_argument("--phase-raw-out", default=None, help="save the raw timestamps of the last call (.npy)")
    ap.add_argument("--interm-div", type=int, default=0,
                    help="time the fp16-intermediate form instead: the same stack with routed up projections "
                         "divided by this power of two (128 in the published packs)")
    args = ap.parse_args()
    if args.counters_summary:
        summarize_counters(*args.counters_summary, commands=args.command, which=args.counters_kernel)
        return
    if args.exchange_probe:
        return bench_exchange_probe(args)
    if args.phase_table:
        return bench_phase_table(args)
    if args.prefill:
        bench_prefill(args)
        return
    if args.cost_table:
        bench_cost_table(args)
        return
    if args.head_dense:
        bench_head_dense(args)
        return
    if args.attn:
        bench_attn(args)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the per-GPU shard is the whole block, see the sharding note of the design", file=sys.stderr)
        sys.exit(2)

    import torch
    import flintgen as fg
    import int4_expert_ffn_amd as F

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": a.numel() * 4}))
        return

    t_setup = time.perf_counter()
    model = build_stack_model(dev, args.interm_div)
    pool = torch.from_numpy(fg.tokens(0, range(64))).to(dev)
    out = torch.empty((1, H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    setup_s = time.perf_counter() - t_setup

    def step(i):
        F.flint_moe_forward(model.h, pool[i % 64:i % 64 + 1], 1, 0, N_LAYERS, out, stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    model.status()
    # the timed region: K launches back to back, two events on the launch
    # stream around them (events between the launches would add their own
    # time to every step)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    model.status()
    ms_per_step = wall / args.steps * 1e3
    value = args.steps / wall
    launch_s = e0.elapsed_time(e1) * 1e-3 / args.steps   # mean launch duration, launch gaps included
    # the spread of single launches, from a separate pass with an event pair per launch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    model.status()
    durs = np.array([a.elapsed_time(b) for a, b in ev]) * 1e-3   # seconds
    achieved = TOKEN_BYTES / launch_s / 1e9
    traffic = traffic_from_profiles()
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4xbf16->fp32" + (", fp16 SwiGLU outputs" if args.interm_div else ""),
        "data": "synthetic (seeded int4 weights, bf16 scales, N(0,1) tokens)",
        "config": {"workload": "47-layer Flint MoE block stack, batch 1 decode"
                               + (f", fp16 intermediates (routed up / {args.interm_div})" if args.interm_div else ""),
                   "layers": N_LAYERS,
                   "hidden": H, "experts": E, "top_k": K, "expert_size": I, "shared_size": IS,
                   "group": G, "tokens_per_step": 1, "token_pool": 64,
                   "algorithmic_bytes_per_token": TOKEN_BYTES},
        "hbm_gbps": round(TOKEN_BYTES * value / 1e9, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic,
                     "kernel": "one forward launch sequence (47 layers, 1 token)",
                     "launch_us_mean": round(launch_s * 1e6, 2),
                     "launch_us_p10": round(float(np.percentile(durs, 10)) * 1e6, 2),
                     "launch_us_p90": round(float(np.percentile(durs, 90)) * 1e6, 2),
                     "launch_us_note": "mean: events around the timed region / steps; p10, p90: per-launch "
                                       "events of a separate pass"},
        "setup_s": round(setup_s, 1),
    }
    copy_gbps = measure_copy_gbps(torch, dev)
    res["roofline"]["copy_gbps"] = round(copy_gbps, 1)
    res["roofline"]["frac_of_copy"] = round(achieved / copy_gbps, 4)
    if args.interm_div:
        res["config"]["interm_div"] = args.interm_div
        res["roofline"]["traffic"] = None   # the counters were taken on the fp32 form
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(args.cpu_seconds, args.interm_div)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
