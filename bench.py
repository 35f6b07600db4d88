#!/usr/bin/env python3
"""Throughput and latency of the BF16 encoder pass on one MI355X.

One step = one laya_encoder_run over one batch of the workload (embedding,
28 encoder layers, 2 decision layers, final LayerNorm).  Timed region: K
graph replays on indices already resident in device memory
(LAYA_RUN_RESIDENT), back to back, bracketed by device synchronisation.
Reported next to it: per-call p50/p95 (device-resident inputs, synchronised
per call), the pages' host boundary (pack + upload + replay + sync) p50, the
first-shape capture cost, the same figures for the 1x48 call, the dominant
kernel's roofline fraction measured with HIP events on its launch stream
(back to back, and inside the pass), and the CPU oracle timed on the whole
benchmarked batch (one warm call, then three timed).

Prints ONE JSON line.  Defaults finish in a few minutes (the oracle's three
full passes take about 30 s of that).  Other modes: --protocol (every
workload, the pages' recipe), --plan-check and --tile-sweep (GEMM plans),
--summarize-counters (rocprofv3 --pmc output), --copy-calibration-mib,
--chip-peaks (the chip probe).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "encoder calls/s + p50 ms (28+2 layers, BF16) at 1×48 and 16×512, 1 GPU"
# The pages' H800 figure for the same call shape (native eager, host timer,
# run 1), quoted for context: 38.7 req/s at 16x512, 358.9 req/s at 1x48.
PAGES_CALLS_PER_S = {"mixed_16": 38.7, "short_1": 358.9, "short_3": 311.0, "long_3": 132.9}

# kernel that runs each op class (prefix of its symbol in rocprofv3 summaries;
# the GEMM tile configuration and K split follow the plan for the batch shape)
DOMINANT_KERNEL_SYMBOL = {
    "up_geglu_gemm": "gemm_kernel<Cfg<...>, 1, ...> (GeGLU epilogue)",
    "qkv_gemm": "gemm_kernel<Cfg<...>, 2, ...> (QKV epilogue)",
    "up_gelu_gemm": "gemm_kernel<Cfg<...>, 3, ...> (bias + GELU epilogue)",
    "down_gemm": "gemm_kernel<Cfg<...>, 0, ...>",
    "out_proj_gemm": "gemm_kernel<Cfg<...>, 0, ...>", "attention": "attention_kernel",
    "layernorm": "layernorm_kernel", "rope": "rope_kernel",
}

# HBM traffic of the dominant kernel, measured: per-launch FETCH_SIZE and
# WRITE_SIZE (KiB) of the GeGLU up projection at mixed_16 from two
# rocprofv3 --pmc runs of this script, each divided by what the same counter
# reads per byte moved by a plain 1 GiB device copy (this script's
# --copy-calibration-mib mode).  Commands and figures:
# profiles/pass_traffic_mixed_16.md.  The figure holds only for the
# GEMM sources it was taken with (SHA-256 over k_gemm.hip, common.h,
# kernels.h); after any change to them the traffic is reported as null.
TRAFFIC = {"op": "up_geglu_gemm", "workload": "mixed_16", "fetch_kib": 48664.8,
           "write_kib": 20756.2, "fetch_per_byte": 0.5000, "write_per_byte": 1.0000,
           "sources_sha256": "f8a31ce1aad8fd313d88549071213fb7c8f463ebb155a6d892b129079c95ef75"}
TRAFFIC_SOURCES = ("k_gemm.hip", "common.h", "kernels.h")

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense BF16 MFMA
PEAK_HBM_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="mixed_16")
    p.add_argument("--latency-calls", type=int, default=50)
    p.add_argument("--profile-passes", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--rope", choices=("fused", "standalone", "original"), default="fused",
                   help="RoPE variant of the measured pass: in the QKV epilogue (default), by its "
                        "own kernel, or by its own kernel in the original launch geometry")
    p.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                   help="only print a per-kernel markdown table of the rocprofv3 counter runs "
                        "written to these directories (counter_collection.csv), then exit")
    p.add_argument("--copy-fetch-per-byte", type=float, default=None,
                   help="FETCH_SIZE KiB per KiB of a plain device copy (scales HBM reads)")
    p.add_argument("--copy-write-per-byte", type=float, default=None,
                   help="WRITE_SIZE KiB per KiB of a plain device copy (scales HBM writes)")
    p.add_argument("--dec-head", action="store_true",
                   help="decision layers as the biased head variant (biased projections, "
                        "4*hidden GELU FFN)")
    p.add_argument("--cpu-calls", type=int, default=3,
                   help="timed oracle calls on the whole batch after one warm call")
    p.add_argument("--short-workload", default="short_1",
                   help="the second shape the metric is quoted on, measured in the same run "
                        "(graph replays); 'none' to skip")
    p.add_argument("--protocol", action="store_true",
                   help="the full measurement protocol over every workload (ABBA rounds of "
                        "eager and graph calls, device timer, capture cost, per-op shares, "
                        "roofline time, RoPE variant A/B, oracle timing); writes a results "
                        "JSON to --protocol-out and prints a summary")
    p.add_argument("--protocol-out", default="protocol_results.json")
    p.add_argument("--protocol-warmup", type=int, default=20)
    p.add_argument("--protocol-calls", type=int, default=100)
    p.add_argument("--protocol-oracle-calls", type=int, default=3,
                   help="oracle calls per workload in --protocol (0: skip the oracle)")
    p.add_argument("--plan-check", action="store_true",
                   help="time each projection at the first token count of every plan range, "
                        "with the range's plan and with the plan for exactly that count")
    p.add_argument("--tile-sweep", action="store_true",
                   help="time every whole-K tile shape for each projection over a range of "
                        "token counts (markdown table)")
    p.add_argument("--gemm-phases", action="store_true",
                   help="per-workgroup phases (prologue, main loop, epilogue) of the pass's four "
                        "projections at the workload's token count, from the library's "
                        "diagnostic build (markdown table)")
    p.add_argument("--chip-peaks", action="store_true",
                   help="run the chip probe (matrix-core issue rate, LDS read bandwidth, one "
                        "workgroup's HBM stream) and print its figures")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="only run a plain device-to-device copy of this many MiB three times "
                        "(the reference for scaling HBM byte counters), then exit")
    args = p.parse_args()
    if args.profile_passes < 1:
        p.error("--profile-passes must be at least 1: the roofline figure comes from the per-op table")
    return args


def copy_calibration(mib):
    """A plain copy of known size: reads and writes mib MiB per launch."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": 3}), flush=True)


def op_table(enc, batch, mk, repeats, flags=0):
    """Per-op-class average of `repeats` event-bracketed eager passes."""
    acc, tot = {}, 0.0
    for _ in range(repeats):
        ops, t = enc.profile(batch.ids, batch.lengths, markers=mk, flags=flags)
        tot += t
        for k, v in ops.items():
            a = acc.setdefault(k, {"calls": 0, "ms": 0.0, "flops": 0.0, "bytes": 0.0})
            for f in a:
                a[f] += v[f]
    table = {}
    for k, v in acc.items():
        sec = v["ms"] / 1e3
        per_launch_us = v["ms"] / v["calls"] * 1e3
        row = {"launches_per_pass": v["calls"] // repeats,
               "ms_per_pass": round(v["ms"] / repeats, 4),
               "share": round(v["ms"] / sum(x["ms"] for x in acc.values()), 4),
               "avg_launch_us": round(per_launch_us, 2)}
        if v["flops"] > 0:
            row["tflops"] = round(v["flops"] / sec / 1e12, 1)
            row["mfma_frac"] = round(v["flops"] / sec / 1e12 / PEAK_BF16_TFLOPS, 4)
        row["hbm_gbs"] = round(v["bytes"] / sec / 1e9, 1)
        row["hbm_frac"] = round(v["bytes"] / sec / 1e9 / PEAK_HBM_GBS, 4)
        row["_flops"], row["_bytes"], row["_calls"], row["_sec"] = (v["flops"], v["bytes"],
                                                                    v["calls"], sec)
        table[k] = row
    return table, tot / repeats


def back_to_back_gemm(op, cfg, T, n=30):
    """Average duration (us) and FLOP per launch of the dominant GEMM's kernel,
    timed over `n` back-to-back launches through laya_op_gemm at the pass's
    shape and plan, with HIP events on the launch stream around the whole
    run (events around single launches add their own overhead).  The weights
    rotate through copies larger than the MALL, so each launch streams them
    from HBM as in the pass.  None for ops without a plain GEMM entry."""
    import torch
    from transformer_encoder_bf16_amd import binding
    H, F = cfg["hidden"], cfg["ffn"]
    shapes = {"up_geglu_gemm": (F, H, 1, 2 * F), "down_gemm": (H, F, 0, H),
              "out_proj_gemm": (H, H, 0, H), "up_gelu_gemm": (4 * H, H, 3, 4 * H)}
    if op not in shapes or T <= 0:
        return None
    N, K, epi, rows = shapes[op]
    g = torch.Generator(device="cuda").manual_seed(0)
    a = (torch.randn(T, K, device="cuda", generator=g)).to(torch.bfloat16)
    w0 = (0.02 * torch.randn(rows, K, device="cuda", generator=g)).to(torch.bfloat16)
    ws = [w0.clone() for _ in range(int(600e6 // (w0.numel() * 2)) + 1)]
    bias = torch.zeros(N, dtype=torch.bfloat16, device="cuda") if epi == 3 else None
    c = torch.empty(T, N, dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    for i in range(5):
        binding.op_gemm(a, ws[i % len(ws)], c, T, N, K, epi, bias=bias)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n):
        binding.op_gemm(a, ws[i % len(ws)], c, T, N, K, epi, bias=bias)
    e1.record(stream)
    e1.synchronize()
    us = e0.elapsed_time(e1) / n * 1e3
    del ws
    return us, 2.0 * T * rows * K


def measured_traffic(op, workload):
    """HBM bytes per launch of `op` from the recorded counters, or None."""
    import hashlib
    if op != TRAFFIC["op"] or workload != TRAFFIC["workload"]:
        return None
    h = hashlib.sha256()
    for name in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "transformer_encoder_bf16_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != TRAFFIC["sources_sha256"]:
        return None
    return round(TRAFFIC["fetch_kib"] * 1024 / TRAFFIC["fetch_per_byte"] +
                 TRAFFIC["write_kib"] * 1024 / TRAFFIC["write_per_byte"])


def cpu_baseline(cfg, batch, calls):
    """The CPU oracle on the whole benchmarked batch: one warm call, then
    `calls` timed calls; calls/s = calls / their total time, with the p50."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=os.cpu_count())
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    w = oracle.Weights(cfg, 1)
    o = oracle.Oracle(cfg, w)
    o.forward(batch.ids, batch.lengths, markers=batch.markers)  # warm (weights widened)
    ts = []
    for _ in range(calls):
        t0 = time.perf_counter()
        o.forward(batch.ids, batch.lengths, markers=batch.markers)
        ts.append(time.perf_counter() - t0)
    cpu = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        pass
    return {"value": round(calls / sum(ts), 4), "unit": "calls/s", "cores": int(cores),
            "kind": "oracle", "p50_ms": round(float(np.percentile(ts, 50)) * 1e3, 1),
            "host_cpu": cpu,
            "sample": f"the whole {batch.B}x{batch.S} batch ({batch.T} tokens), one warm call "
                      f"then {calls} timed full 30-layer passes"}


def _host_calls(enc, batch, flags, n, sync):
    out = []
    for _ in range(n):
        t = time.perf_counter()
        enc.run(batch.ids, batch.lengths, markers=batch.markers, flags=flags)
        sync()
        out.append((time.perf_counter() - t) * 1e3)
    return out


def _summ(samples):
    a = np.asarray(samples)
    return {"p50_ms": round(float(np.percentile(a, 50)), 4),
            "p95_ms": round(float(np.percentile(a, 95)), 4),
            "calls_per_s": round(len(a) / (a.sum() / 1e3), 3)}


def _metadata(enc, cfg):
    import hashlib
    import subprocess
    import torch
    from transformer_encoder_bf16_amd import binding
    with open(binding.LIB_PATH, "rb") as f:
        lib_sha = hashlib.sha256(f.read()).hexdigest()
    try:
        sha = subprocess.run(["git", "rev-parse", "HEAD"], cwd=ROOT, capture_output=True,
                             text=True, timeout=10).stdout.strip() or None
    except Exception:
        sha = None
    cpu = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        pass
    smt = None
    try:
        with open("/sys/devices/system/cpu/smt/active") as f:
            smt = f.read().strip() == "1"
    except OSError:
        pass
    n_tensors = 1 + 4 * (cfg["n_enc_layers"] + cfg["n_dec_layers"])
    if cfg.get("dec_head", 0):
        n_tensors += 4 * cfg["n_dec_layers"]
    digests = [format(enc.weight_digest(t), "016x") for t in range(n_tensors)]
    props = torch.cuda.get_device_properties(0)
    return {"git_sha": sha, "library_sha256": lib_sha, "gpu": props.name,
            "gpu_arch": getattr(props, "gcnArchName", None), "host_cpu": cpu,
            "host_cores": os.cpu_count(), "smt": smt, "weight_fnv1a64": digests}


def protocol(args):
    """The measurement protocol over every workload.  Per workload: one
    feasibility call (excluded, also the first graph capture), then rounds in
    ABBA order (eager, graph, graph, eager), each with warmups and measured
    calls timed on the host from the call to the completion sync (packing,
    upload and sync included); a device timer (HIP events around resident
    graph replays on the stream); the per-op table of one event-profiled
    eager pass and the roofline time sum over op classes of max(FLOP/peak,
    bytes/peak); the RoPE variants (fused into the QKV epilogue against the
    standalone kernel) in ABBA order; and the CPU oracle."""
    import torch
    from transformer_encoder_bf16_amd import binding
    from transformer_encoder_bf16_amd.inputs import ALL_WORKLOADS, WEIGHT_SEED, make_batch

    if not os.path.exists(binding.LIB_PATH):
        from transformer_encoder_bf16_amd import build_lib
        build_lib.build()
    torch.cuda.set_device(0)
    sync = torch.cuda.synchronize
    MODEL = model_config(args)
    enc = binding.Encoder(MODEL, seed=WEIGHT_SEED, device=0)
    meta = _metadata(enc, MODEL)
    meta["decision_layers"] = "head" if args.dec_head else "encoder-shaped"
    meta["create_ms"] = round(enc.stats()["create_ms"], 1)
    results = {"metric": METRIC, "protocol": {"warmup": args.protocol_warmup,
                                              "calls": args.protocol_calls,
                                              "order": ["eager", "graph", "graph", "eager"]},
               "meta": meta, "workloads": {}}
    stream = torch.cuda.current_stream()
    for name, wl in ALL_WORKLOADS.items():
        batch = make_batch(MODEL, wl)
        res = {"B": batch.B, "S": batch.S, "T": batch.T,
               "R": 0 if batch.markers is None else int(len(batch.markers)), "seed": wl.seed}
        t = time.perf_counter()
        enc.run(batch.ids, batch.lengths, markers=batch.markers)  # feasibility + capture
        sync()
        res["first_graph_call_ms"] = round((time.perf_counter() - t) * 1e3, 3)
        res["capture_ms"] = round(enc.stats()["last_capture_ms"], 3)
        rounds = []
        for mode in ("eager", "graph", "graph", "eager"):
            flags = binding.RUN_EAGER if mode == "eager" else 0
            _host_calls(enc, batch, flags, args.protocol_warmup, sync)
            samples = _host_calls(enc, batch, flags, args.protocol_calls, sync)
            rounds.append({"mode": mode, **_summ(samples),
                           "samples_ms": [round(x, 4) for x in samples]})
        res["rounds"] = rounds
        for mode in ("eager", "graph"):
            all_s = [x for r in rounds if r["mode"] == mode for x in r["samples_ms"]]
            res[f"{mode}_host"] = _summ(all_s)
        # device timer: HIP events on the stream around resident graph replays
        enc.run(batch.ids, batch.lengths, markers=batch.markers)
        dev = []
        for _ in range(args.protocol_calls):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            enc.run(batch.ids, batch.lengths, markers=batch.markers, flags=binding.RUN_RESIDENT)
            e1.record(stream)
            e1.synchronize()
            dev.append(e0.elapsed_time(e1))
        res["device_graph"] = {"p50_ms": round(float(np.percentile(dev, 50)), 4),
                               "p95_ms": round(float(np.percentile(dev, 95)), 4)}
        # per-op shares and the roofline time
        table, pass_ms = op_table(enc, batch, batch.markers, 1)
        t_roof = sum(max(v["_flops"] / (PEAK_BF16_TFLOPS * 1e12), v["_bytes"] / (PEAK_HBM_GBS * 1e9))
                     for v in table.values())
        res["profiled_eager_pass_ms"] = round(pass_ms, 4)
        res["roofline_time_ms"] = round(t_roof * 1e3, 4)
        res["graph_p50_over_roofline"] = round(res["graph_host"]["p50_ms"] / (t_roof * 1e3), 2)
        res["ops"] = {k: {f: v for f, v in row.items() if not f.startswith("_")}
                      for k, row in table.items()}
        # RoPE variants in mirrored order (original, standalone, fused, fused,
        # standalone, original), graph replays
        ab = []
        rope_flags = {"original": binding.RUN_ROPE_ORIGINAL,
                      "standalone": binding.RUN_ROPE_STANDALONE, "fused": 0}
        for variant in ("original", "standalone", "fused", "fused", "standalone", "original"):
            flags = rope_flags[variant]
            enc.run(batch.ids, batch.lengths, markers=batch.markers, flags=flags)
            sync()
            _host_calls(enc, batch, flags | binding.RUN_RESIDENT, args.protocol_warmup, sync)
            samples = _host_calls(enc, batch, flags | binding.RUN_RESIDENT,
                                  args.protocol_calls, sync)
            ab.append({"variant": variant, **_summ(samples)})
        bits = {}
        for variant, flags in rope_flags.items():
            out = enc.run(batch.ids, batch.lengths, markers=batch.markers,
                          flags=flags | binding.RUN_EAGER)
            sync()
            bits[variant] = enc.hidden_bits(out)
        res["rope_ab"] = {"rounds": ab,
                          "bitwise_equal": bool(np.array_equal(bits["fused"], bits["standalone"]) and
                                                np.array_equal(bits["fused"], bits["original"]))}
        # the standalone kernels' own time, from one event-profiled eager pass each
        for variant in ("original", "standalone"):
            t_ops, _ = op_table(enc, batch, batch.markers, 1, flags=rope_flags[variant])
            key = "rope_original" if variant == "original" else "rope"
            if key in t_ops:
                res["rope_ab"][f"{variant}_kernel_us"] = t_ops[key]["avg_launch_us"]
                res["rope_ab"][f"{variant}_kernel_gbs"] = t_ops[key]["hbm_gbs"]
        if args.protocol_oracle_calls > 0:
            res["oracle"] = oracle_timing(MODEL, batch, args.protocol_oracle_calls)
        results["workloads"][name] = res
        print(f"{name:14s} T={res['T']:5d} graph p50 {res['graph_host']['p50_ms']:8.3f} ms "
              f"({res['graph_host']['calls_per_s']:8.1f} calls/s)  eager p50 "
              f"{res['eager_host']['p50_ms']:8.3f}  device p50 {res['device_graph']['p50_ms']:8.3f}  "
              f"roofline {res['roofline_time_ms']:7.3f} ms  capture {res['capture_ms']:7.1f} ms  "
              f"rope original/standalone/fused p50 {ab[0]['p50_ms']:.3f}/{ab[1]['p50_ms']:.3f}/"
              f"{ab[2]['p50_ms']:.3f}", flush=True)
    enc.close()
    with open(args.protocol_out, "w") as f:
        json.dump(results, f)
    print(json.dumps({"protocol_out": args.protocol_out,
                      "workloads": {k: {"graph_p50_ms": v["graph_host"]["p50_ms"],
                                        "calls_per_s": v["graph_host"]["calls_per_s"],
                                        "roofline_ms": v["roofline_time_ms"]}
                                    for k, v in results["workloads"].items()}}), flush=True)


def chip_peaks():
    """Run the chip probe built next to the library (a child process: this
    process touches no GPU first) and print its figures as markdown."""
    import subprocess
    from transformer_encoder_bf16_amd import build_lib
    if not os.path.exists(build_lib.PROBE):
        build_lib.build()
    r = subprocess.run([build_lib.PROBE], capture_output=True, text=True, timeout=300)
    if r.returncode != 0:
        print(r.stdout, r.stderr, file=sys.stderr)
        sys.exit(r.returncode)
    recs = [json.loads(line) for line in r.stdout.splitlines() if line.startswith("{")]
    dev = next(x for x in recs if x["probe"] == "device")
    print(f"Device: {dev['name']} ({dev['arch']}), {dev['cus']} CUs.\n")
    print("| Matrix cores (4 independent 32x32x16 BF16 chains per wave) | µs | TFLOP/s | of 2500 |")
    print("|---|---|---|---|")
    for x in recs:
        if x["probe"] == "mfma_bf16_32x32x16":
            print(f"| {x['workgroups_per_cu']} four-wave workgroups per CU | {x['us']} | {x['tflops']} | "
                  f"{x['tflops'] / PEAK_BF16_TFLOPS:.2f} |")
    print("\n| LDS reads (ds_read_b128, no bank conflicts) | µs | TB/s (chip) | B/clk per CU at 2.1 GHz |")
    print("|---|---|---|---|")
    for x in recs:
        if x["probe"] == "lds_read_b128":
            print(f"| {x['workgroups_per_cu']} workgroups of 512 threads per CU | {x['us']} | {x['tb_per_s']} | "
                  f"{x['bytes_per_clk_per_cu_at_2.1ghz']} |")
    print("\n| One workgroup streaming HBM -> LDS (16 workgroups) | KB per workgroup | empty launch µs | µs, 8 waves "
          "| µs, 16 waves | GB/s per workgroup above the empty launch, 8 / 16 waves |")
    print("|---|---|---|---|---|---|")
    for x in recs:
        if x["probe"] == "one_workgroup_stream":
            print(f"| | {x['kb_per_workgroup']} | {x['empty_launch_us']} | {x['us_8_waves']} | {x['us_16_waves']} | "
                  f"{x['gb_per_s_per_workgroup_8_waves']} / {x['gb_per_s_per_workgroup_16_waves']} |")


CONFIG_NAMES = ["XS", "XSG", "S", "M", "L", "XL", "M2", "XS2", "XSG2", "PP", "Q3", "W2"]


def plan_check():
    """A captured graph serves the run of live token counts whose GEMM plans
    agree (laya_pass_plans).  For the first count of every such run, each
    projection is timed with the pass's plan and with the planner evaluated
    at exactly that count (laya_plan_gemm; the two agree when the pass plans
    per count), as back-to-back launches in a captured graph with the weights
    rotated through copies larger than the MALL.  Split plans run with their
    own reduce launch here (laya_op_gemm_noalloc; the pass fuses that reduce
    with the LayerNorm).  Prints a markdown table."""
    import torch
    from transformer_encoder_bf16_amd import binding as B
    from transformer_encoder_bf16_amd.inputs import MODEL
    torch.cuda.set_device(0)
    dev = "cuda"
    H, F = MODEL["hidden"], MODEL["ffn"]
    gemms = [("qkv", 3 * H, H, 2), ("out", H, H, 0), ("up", F, H, 1), ("down", H, F, 0)]
    cb, sb = B.rope_table(160000.0, 512, 64)
    ct = torch.from_numpy(cb.view(np.int16)).to(dev)
    st = torch.from_numpy(sb.view(np.int16)).to(dev)

    def graph_us(fn, n_inner, reps=5):
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            fn()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                fn()
            g.replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(s)
            for _ in range(reps):
                g.replay()
            e1.record(s)
            torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * n_inner)

    ranges = []
    T = 1
    while T <= MODEL["max_batch"] * MODEL["max_seq"]:
        lo, hi, plans = B.pass_plans(MODEL, T)
        ranges.append((max(lo, 48), lo, hi, plans))
        T = hi + 1
    print("| T | Range | GEMM | Range plan (tile, K ranges) | µs | Plan at T | µs | Range / at-T |")
    print("|---|---|---|---|---|---|---|---|")
    for T, lo, hi, plans in ranges:
        pos = torch.from_numpy((np.arange(T) % 512).astype(np.int32)).to(dev)
        vtok = torch.arange(T, dtype=torch.int32, device=dev)
        vt = torch.empty(H, T + 64, dtype=torch.bfloat16, device=dev)
        for (name, N, K, epi), pl in zip(gemms, plans[:4]):
            wr = 2 * N if epi == 1 else N
            A = (torch.randn(T, K, device=dev) * 0.5).bfloat16()
            W = (torch.randn(wr, K, device=dev) * 0.03).bfloat16()
            C = torch.empty(T, N, device=dev, dtype=torch.bfloat16)
            ncopy = max(8, int(600e6 // (wr * K * 2)))
            Ws = [W.clone() for _ in range(ncopy)]
            del W

            def timed(cfg, sp):
                def fn():
                    for w in Ws:
                        if epi == 2:
                            B.op_gemm_qkv(A, w, C, T, N, K, pos, ct, st, 2 * H, vt, vtok, 2 * H,
                                          config=cfg, splits=sp)
                        else:
                            B.op_gemm_noalloc(A, w, C, T, N, K, epi, cfg, sp)
                return graph_us(fn, ncopy)

            at = B.plan_gemm(T, N, K, epi)
            rng = (pl[0], pl[1])
            us_r = timed(*rng)
            us_t = us_r if at == rng else timed(*at)
            print(f"| {T} | {lo}–{hi} | {name} | {CONFIG_NAMES[rng[0]]}, {rng[1]} | {us_r:.2f} | "
                  f"{'same' if at == rng else f'{CONFIG_NAMES[at[0]]}, {at[1]}'} | {us_t:.2f} | "
                  f"{us_r / us_t:.3f} |", flush=True)
            del Ws


SWEEP_T = [257, 320, 384, 448, 512, 640, 768, 896, 1024, 1152, 1280, 1344, 1536, 1715, 2048,
           2400, 2688, 3072, 3500, 4050, 4500, 5000, 5400, 5800, 6144, 7000, 8192]
SWEEP_CONFIGS = [2, 3, 4, 5, 6, 9, 10, 11]


def tile_sweep():
    """Every whole-K tile shape for each projection of the pass at a range of
    token counts, timed as back-to-back launches in a captured graph with the
    weights rotated through copies larger than the MALL.  The shapes give
    bitwise equal outputs, so the planner may take the fastest; this is the
    measurement it is checked against.  Prints a markdown table (µs)."""
    import torch
    from transformer_encoder_bf16_amd import binding as B
    from transformer_encoder_bf16_amd.inputs import MODEL
    torch.cuda.set_device(0)
    dev = "cuda"
    H, F = MODEL["hidden"], MODEL["ffn"]
    gemms = [("qkv", 3 * H, H, 2), ("out", H, H, 0), ("up", F, H, 1), ("down", H, F, 0)]
    cb, sb = B.rope_table(160000.0, 512, 64)
    ct = torch.from_numpy(cb.view(np.int16)).to(dev)
    st = torch.from_numpy(sb.view(np.int16)).to(dev)
    tmax = max(SWEEP_T)
    pos = torch.from_numpy((np.arange(tmax) % 512).astype(np.int32)).to(dev)
    vtok = torch.arange(tmax, dtype=torch.int32, device=dev)
    vt = torch.empty(H, tmax + 64, dtype=torch.bfloat16, device=dev)
    names = [CONFIG_NAMES[c] for c in SWEEP_CONFIGS]
    print("| GEMM | T | " + " | ".join(names) + " | fastest | planner |")
    print("|---|---|" + "---|" * (len(names) + 2))
    for name, N, K, epi in gemms:
        wr = 2 * N if epi == 1 else N
        A = (torch.randn(tmax, K, device=dev) * 0.5).bfloat16()
        W = (torch.randn(wr, K, device=dev) * 0.03).bfloat16()
        C = torch.empty(tmax, N, device=dev, dtype=torch.bfloat16)
        ncopy = max(8, int(600e6 // (wr * K * 2)))
        Ws = [W.clone() for _ in range(ncopy)]
        del W
        for T in SWEEP_T:
            us = []
            for cfg in SWEEP_CONFIGS:
                def fn():
                    for w in Ws:
                        if epi == 2:
                            B.op_gemm_qkv(A, w, C, T, N, K, pos, ct, st, 2 * H, vt, vtok, 2 * H,
                                          config=cfg, splits=1)
                        else:
                            B.op_gemm_noalloc(A, w, C, T, N, K, epi, cfg, 1)
                us.append(_graph_launch_us(fn, ncopy))
            best = SWEEP_CONFIGS[int(np.argmin(us))]
            plan = B.plan_gemm(T, N, K, epi)
            print(f"| {name} | {T} | " + " | ".join(f"{u:.2f}" for u in us) +
                  f" | {CONFIG_NAMES[best]} | {CONFIG_NAMES[plan[0]]}, {plan[1]} |", flush=True)
        del Ws


# whole-K tile shapes: weight rows, tokens, workgroups one CU holds
PHASE_TILES = {2: (128, 64, 1), 3: (128, 128, 1), 4: (256, 128, 1), 5: (256, 256, 1),
               6: (128, 128, 2), 10: (192, 256, 1), 11: (256, 192, 1)}


def gemm_phases(workload):
    """The pass's four projections at the workload's token count, with the
    planner's whole-K tile shapes, run through the library's diagnostic build,
    whose GEMM workgroups record the shader clock at their start, when their
    ring is first full, at the end of their main loop, before and after the
    barrier ahead of their stores, and at their end (plus the 100 MHz clock at
    start and end, from which the shader clock's rate is fitted).  One launch
    per projection after three warm ones, weights rotated beyond the MALL.
    Prints the medians over the workgroups as markdown."""
    import ctypes
    import torch
    from transformer_encoder_bf16_amd import binding as B
    from transformer_encoder_bf16_amd import build_lib
    from transformer_encoder_bf16_amd.inputs import ALL_WORKLOADS, MODEL, make_batch
    if not os.path.exists(build_lib.PHASES_LIB):
        build_lib.build()
    B.LIB_PATH = build_lib.PHASES_LIB
    lib = B.load()
    lib.laya_gemm_phases_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    torch.cuda.set_device(0)
    dev = "cuda"
    T = make_batch(MODEL, ALL_WORKLOADS[workload]).T
    H, F = MODEL["hidden"], MODEL["ffn"]
    cb, sb = B.rope_table(160000.0, 512, 64)
    ct = torch.from_numpy(cb.view(np.int16)).to(dev)
    st = torch.from_numpy(sb.view(np.int16)).to(dev)
    pos = torch.from_numpy((np.arange(T) % 512).astype(np.int32)).to(dev)
    vtok = torch.arange(T, dtype=torch.int32, device=dev)
    vt = torch.empty(H, T + 64, dtype=torch.bfloat16, device=dev)
    print(f"Workload {workload}: T = {T} tokens.\n")
    print("| GEMM | Tile | Workgroups | Clock GHz | Span µs | Prologue µs | Main loop µs "
          "| µs per 64-wide K step | Loop at MFMA rate | Epilogue: compute + staging µs "
          "| barrier µs | stores µs |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|")
    for name, N, K, epi in [("qkv", 3 * H, H, 2), ("out", H, H, 0), ("up", F, H, 1),
                            ("down", H, F, 0)]:
        cfg, splits = B.plan_gemm(T, N, K, epi)
        if splits != 1 or cfg not in PHASE_TILES:
            print(f"| {name} | {CONFIG_NAMES[cfg]}, {splits} K ranges | (split K: not recorded) "
                  "| | | | | | | | | |")
            continue
        wr = 2 * N if epi == 1 else N
        A = (torch.randn(T, K, device=dev) * 0.5).bfloat16()
        W = (torch.randn(wr, K, device=dev) * 0.03).bfloat16()
        C = torch.empty(T, N, device=dev, dtype=torch.bfloat16)
        Ws = [W.clone() for _ in range(max(8, int(600e6 // (wr * K * 2))))]
        del W

        def one(w):
            if epi == 2:
                B.op_gemm_qkv(A, w, C, T, N, K, pos, ct, st, 2 * H, vt, vtok, 2 * H,
                              config=cfg, splits=1)
            else:
                B.op_gemm_noalloc(A, w, C, T, N, K, epi, cfg, 1)
        for i in range(3):
            one(Ws[i])
        torch.cuda.synchronize()
        if lib.laya_gemm_phases_clear() != 0:
            raise RuntimeError("laya_gemm_phases_clear failed")
        one(Ws[3])
        torch.cuda.synchronize()
        buf = np.zeros(65536 * 10, dtype=np.uint64)
        if lib.laya_gemm_phases_read(buf.ctypes.data, buf.nbytes) != 0:
            raise RuntimeError("laya_gemm_phases_read failed")
        rec = buf.reshape(-1, 10)
        rec = rec[rec[:, 9] == 1].astype(np.int64)
        c, r0, r1 = rec[:, :6], rec[:, 6], rec[:, 7]
        clock = float(np.median((c[:, 5] - c[:, 0]) / np.maximum(r1 - r0, 1))) * 100e6
        us = lambda cyc: float(np.median(cyc)) / clock * 1e6
        bw, bt, occ = PHASE_TILES[cfg]
        steps = K // 64
        # one MFMA-bound K step: the tile's 2*bw*bt*64 FLOP at 4 SIMDs x 1024 FLOP
        # per clock, shared with the other workgroups the CU holds
        conc = min(occ, -(-len(rec) // 256))
        ideal = 2.0 * bw * bt * 64 * conc / (4 * 1024) / clock * 1e6
        step = us(c[:, 2] - c[:, 1]) / steps
        print(f"| {name} | {CONFIG_NAMES[cfg]} {bw}x{bt} | {len(rec)} | {clock / 1e9:.2f} | "
              f"{(r1.max() - r0.min()) / 100.0:.1f} | {us(c[:, 1] - c[:, 0]):.2f} | "
              f"{us(c[:, 2] - c[:, 1]):.2f} | {step:.3f} | {ideal / step:.2f} | "
              f"{us(c[:, 3] - c[:, 2]):.2f} | {us(c[:, 4] - c[:, 3]):.2f} | "
              f"{us(c[:, 5] - c[:, 4]):.2f} |", flush=True)
        del Ws


def _graph_launch_us(fn, n_inner, reps=5):
    """µs per launch of `fn`'s n_inner launches, captured in one graph."""
    import torch
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            fn()
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(reps):
            g.replay()
        e1.record(s)
        torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * n_inner)


def model_config(args) -> dict:
    """The model, or with --dec-head its biased decision-head variant."""
    from transformer_encoder_bf16_amd.inputs import MODEL
    return dict(MODEL, dec_head=1) if args.dec_head else dict(MODEL)


def oracle_timing(cfg, batch, calls):
    """The CPU oracle on the whole batch: one warm call, then `calls` timed."""
    import oracle
    w = oracle.Weights(cfg, 1)
    o = oracle.Oracle(cfg, w)
    o.forward(batch.ids[:1, :4], np.array([4], np.int32))  # widen weights (untimed)
    o.forward(batch.ids, batch.lengths, markers=batch.markers)
    ts = []
    for _ in range(calls):
        t = time.perf_counter()
        o.forward(batch.ids, batch.lengths, markers=batch.markers)
        ts.append((time.perf_counter() - t) * 1e3)
    return {"calls": calls, "p50_ms": round(float(np.percentile(ts, 50)), 1),
            "calls_per_s": round(calls / (sum(ts) / 1e3), 4), "cores": os.cpu_count()}


def summarize_counters(dirs, fetch_per_byte=None, write_per_byte=None):
    """Per-kernel averages of rocprofv3 --pmc runs, as a markdown table.

    Each dispatch's duration comes from its timestamps.  GRBM_GUI_ACTIVE is
    summed over the 8 XCDs and carries a fixed overhead per dispatch, so the
    clock and that overhead are fitted over every dispatch of a run
    (GRBM/8 = clock * duration + overhead); busy fractions are then per SIMD
    (1024) or per CU (256) over duration x fitted clock.  MFMA TFLOP/s comes
    from SQ_INSTS_VALU_MFMA_MOPS_BF16 (512 FLOP each).  HBM bytes: FETCH_SIZE
    and WRITE_SIZE (KiB) divided by what they read per byte of a plain copy."""
    import csv
    import re
    import collections
    kern = collections.defaultdict(lambda: collections.defaultdict(list))
    durs = collections.defaultdict(dict)
    fits = []
    for d in dirs:
        path = None
        for root, _, files in os.walk(d):
            for f in files:
                if f.endswith("counter_collection.csv"):
                    path = os.path.join(root, f)
        if path is None:
            continue
        per_dispatch = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                name = r["Kernel_Name"]
                m = re.search(r"gemm_kernel<laya::\(anonymous namespace\)::Cfg<([^>]*)>, (\d+), (\d+)>", name)
                if m:
                    short = f"gemm_kernel<Cfg<{m.group(1)}>, {m.group(2)}, {m.group(3)}>"
                else:
                    short = re.sub(r"\(.*", "", name.replace("laya::(anonymous namespace)::", "")
                                   .replace("void ", "").replace("laya::", ""))
                key = (short, int(r["Grid_Size"]))
                us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                kern[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
                durs[key][(d, r["Dispatch_Id"])] = us
                if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                    per_dispatch[r["Dispatch_Id"]] = (us, float(r["Counter_Value"]) / 8)
        if len(per_dispatch) >= 2:
            x = np.array([v[0] for v in per_dispatch.values()])
            y = np.array([v[1] for v in per_dispatch.values()])
            fits.append(np.polyfit(x, y, 1))
    clock_mhz, overhead = (np.mean([f[0] for f in fits]), np.mean([f[1] for f in fits])) if fits \
        else (2100.0, 0.0)
    print(f"Fitted over every dispatch: clock {clock_mhz / 1e3:.2f} GHz, GRBM overhead "
          f"{overhead:.0f} cycles per dispatch.\n")
    cols = ["Kernel", "Grid", "Dispatches", "Avg µs"]
    rows = []
    for key, cs in kern.items():
        a = {c: sum(v) / len(v) for c, v in cs.items()}
        us = sum(durs[key].values()) / len(durs[key])
        cyc = us * clock_mhz
        row = {"Kernel": f"`{key[0]}`", "Grid": key[1], "Dispatches": len(durs[key]),
               "Avg µs": f"{us:.2f}"}
        if "SQ_VALU_MFMA_BUSY_CYCLES" in a:
            row["MFMA busy %"] = f"{100 * a['SQ_VALU_MFMA_BUSY_CYCLES'] / 1024 / cyc:.1f}"
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in a:
            row["MFMA TFLOP/s"] = f"{a['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512 / us / 1e6:.0f}"
        if "SQ_ACTIVE_INST_VALU" in a:
            row["VALU busy %"] = f"{100 * a['SQ_ACTIVE_INST_VALU'] * 4 / 1024 / cyc:.1f}"
        if "SQ_INSTS_MFMA" in a and a["SQ_INSTS_MFMA"] and "SQ_INSTS_VALU" in a:
            row["VALU instr / MFMA"] = f"{(a['SQ_INSTS_VALU'] - a['SQ_INSTS_MFMA']) / a['SQ_INSTS_MFMA']:.2f}"
        if "SQ_LDS_BANK_CONFLICT" in a:
            row["LDS bank-conflict %"] = f"{100 * a['SQ_LDS_BANK_CONFLICT'] / 256 / cyc:.2f}"
        if "SQ_WAVE_CYCLES" in a and a["SQ_WAVE_CYCLES"]:
            for c in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY"):
                if c in a:
                    row[c[3:] + " % of wave cycles"] = f"{100 * a[c] / a['SQ_WAVE_CYCLES']:.1f}"
        if "FETCH_SIZE" in a:
            b = a["FETCH_SIZE"] * 1024 / (fetch_per_byte or 1.0)
            row["HBM read MB"] = f"{b / 1e6:.2f}"
            row["read GB/s"] = f"{b / us / 1e3:.0f}"
        if "WRITE_SIZE" in a:
            b = a["WRITE_SIZE"] * 1024 / (write_per_byte or 1.0)
            row["HBM write MB"] = f"{b / 1e6:.2f}"
            row["write GB/s"] = f"{b / us / 1e3:.0f}"
        rows.append((us * len(durs[key]), row))
        for k in row:
            if k not in cols:
                cols.append(k)
    rows.sort(key=lambda t: -t[0])
    print("| " + " | ".join(cols) + " |")
    print("|" + "---|" * len(cols))
    for _, row in rows:
        print("| " + " | ".join(str(row.get(c, "")) for c in cols) + " |")


def graph_replays(enc, batch, steps, warmup, latency_calls, sync, vflags=0):
    """First call (upload + graph capture), then `warmup` and `steps` timed
    back-to-back graph replays on device-resident indices, then per-call
    latencies (synchronised per call), the pages' host boundary (pack + upload
    + replay + sync) and eager calls."""
    from transformer_encoder_bf16_amd import binding
    mk = batch.markers
    t = time.perf_counter()
    enc.run(batch.ids, batch.lengths, markers=mk, flags=vflags)
    sync()
    first_ms = (time.perf_counter() - t) * 1e3
    capture_ms = enc.stats()["last_capture_ms"]
    flags = binding.RUN_RESIDENT | vflags
    for _ in range(warmup):
        enc.run(batch.ids, batch.lengths, markers=mk, flags=flags)
    sync()
    t0 = time.perf_counter()
    for _ in range(steps):
        enc.run(batch.ids, batch.lengths, markers=mk, flags=flags)
    sync()
    elapsed = time.perf_counter() - t0
    lat, host, eager = [], [], []
    for _ in range(latency_calls):
        t = time.perf_counter()
        enc.run(batch.ids, batch.lengths, markers=mk, flags=flags)
        sync()
        lat.append((time.perf_counter() - t) * 1e3)
    for _ in range(latency_calls):
        t = time.perf_counter()
        enc.run(batch.ids, batch.lengths, markers=mk, flags=vflags)
        sync()
        host.append((time.perf_counter() - t) * 1e3)
    for _ in range(max(5, latency_calls // 5)):
        t = time.perf_counter()
        enc.run(batch.ids, batch.lengths, markers=mk, flags=binding.RUN_EAGER | vflags)
        sync()
        eager.append((time.perf_counter() - t) * 1e3)
    launches = enc.stats()["launches_last_run"]
    return {"calls_per_s": steps / elapsed, "ms_per_call": elapsed / steps * 1e3,
            "p50_ms": round(float(np.percentile(lat, 50)), 4),
            "p95_ms": round(float(np.percentile(lat, 95)), 4),
            "host_boundary_p50_ms": round(float(np.percentile(host, 50)), 4),
            "eager_host_boundary_p50_ms": round(float(np.percentile(eager, 50)), 4),
            "first_call_ms": round(first_ms, 2), "capture_ms": round(capture_ms, 2),
            "launches_per_call": launches}


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.copy_fetch_per_byte,
                           args.copy_write_per_byte)
        return
    if args.chip_peaks:
        chip_peaks()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the pass has no "
              f"multi-GPU sharding", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration_mib:
        torch.cuda.set_device(0)
        copy_calibration(args.copy_calibration_mib)
        return
    if args.protocol:
        protocol(args)
        return
    if args.plan_check:
        plan_check()
        return
    if args.tile_sweep:
        tile_sweep()
        return
    if args.gemm_phases:
        gemm_phases(args.workload)
        return
    from transformer_encoder_bf16_amd import binding
    from transformer_encoder_bf16_amd.inputs import ALL_WORKLOADS, WEIGHT_SEED, make_batch

    if not os.path.exists(binding.LIB_PATH):
        from transformer_encoder_bf16_amd import build_lib
        build_lib.build()
    torch.cuda.set_device(0)
    MODEL = model_config(args)
    wl = ALL_WORKLOADS[args.workload]
    batch = make_batch(MODEL, wl)
    enc = binding.Encoder(MODEL, seed=WEIGHT_SEED, device=0)
    st0 = enc.stats()
    mk = batch.markers
    sync = torch.cuda.synchronize

    vflags = {"fused": 0, "standalone": binding.RUN_ROPE_STANDALONE,
              "original": binding.RUN_ROPE_ORIGINAL}[args.rope]
    main_run = graph_replays(enc, batch, args.steps, args.warmup, args.latency_calls, sync,
                             vflags)
    calls_per_s = main_run["calls_per_s"]

    # the second shape the metric is quoted on, the same way
    short = None
    if args.short_workload != "none" and args.short_workload != args.workload:
        sb = make_batch(MODEL, ALL_WORKLOADS[args.short_workload])
        r = graph_replays(enc, sb, max(args.steps, 200), args.warmup, args.latency_calls, sync)
        short = {"workload": args.short_workload, "B": sb.B, "S": sb.S, "T": sb.T,
                 "calls_per_s": round(r["calls_per_s"], 3),
                 "ms_per_call": round(r["ms_per_call"], 4),
                 **{k: r[k] for k in ("p50_ms", "p95_ms", "host_boundary_p50_ms",
                                      "eager_host_boundary_p50_ms", "capture_ms",
                                      "launches_per_call")}}

    # per-op table from event-bracketed eager passes (HIP events on the launch stream)
    table, pass_ms = op_table(enc, batch, mk, args.profile_passes, flags=vflags)
    enc.close()
    dom = max(table, key=lambda k: table[k]["ms_per_pass"])
    d = table[dom]
    # the dominant op's bound: its algorithmic FLOP per byte against the
    # ridge of the two peaks (312.5 FLOP/B); a short call's GEMMs stream their
    # weights at about 2T FLOP/B and are HBM-bound
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    hbm_bound = d["_flops"] <= 0 or d["_flops"] / d["_bytes"] < ridge
    b2b = None if hbm_bound else back_to_back_gemm(dom, MODEL, batch.T)
    if b2b is not None:
        b2b_us, b2b_flops = b2b
        roof = {"bound": "mfma", "achieved": round(b2b_flops / (b2b_us * 1e-6) / 1e12, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    elif not hbm_bound:
        roof = {"bound": "mfma", "achieved": round(d["_flops"] / d["_sec"] / 1e12, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(d["_bytes"] / d["_sec"] / 1e9, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    # the counters were taken on the default model
    roof["traffic"] = None if args.dec_head else measured_traffic(dom, args.workload)
    roof["op"] = dom
    roof["kernel"] = DOMINANT_KERNEL_SYMBOL.get(dom, dom)
    if b2b is not None:
        roof["avg_launch_us"] = round(b2b_us, 2)
        roof["timing"] = ("back-to-back launches of the kernel at the pass's shape and plan, "
                          "weights rotated beyond the MALL, HIP events on the launch stream")
        roof["per_launch_algorithmic"] = b2b_flops
    else:
        roof["avg_launch_us"] = d["avg_launch_us"]
        roof["timing"] = "HIP events around each launch of an eager pass"
        roof["per_launch_algorithmic"] = (d["_bytes"] if hbm_bound else d["_flops"]) / d["_calls"]
    # the same kernel inside the pass: HIP events around each of its launches
    roof["avg_launch_us_in_pass_events"] = d["avg_launch_us"]
    in_pass = (d["_bytes"] / d["_sec"] / 1e9) if hbm_bound else (d["_flops"] / d["_sec"] / 1e12)
    roof["achieved_in_pass"] = round(in_pass, 2)
    roof["frac_in_pass"] = round(in_pass / roof["peak"], 4)
    gemm_ops = [k for k in table if "_gemm" in k]
    gemm_frac = (sum(table[k]["_flops"] for k in gemm_ops) /
                 sum(table[k]["_sec"] for k in gemm_ops) / 1e12 / PEAK_BF16_TFLOPS)
    ops_out = {k: {f: v for f, v in row.items() if not f.startswith("_")}
               for k, row in sorted(table.items(), key=lambda kv: -kv[1]["ms_per_pass"])}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(MODEL, batch, args.cpu_calls)

    pages = None if args.dec_head else PAGES_CALLS_PER_S.get(args.workload)
    line = {
        "metric": METRIC,
        "value": round(calls_per_s, 3),
        "unit": "calls/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_run["ms_per_call"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(calls_per_s / pages, 3) if pages else None,
        "vs_baseline_note": "pages' H800 native eager host-timed calls/s on real requests of the "
                            "same B x S; context only (other GPU, other lengths)",
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "B": batch.B, "S": batch.S, "T": batch.T,
                   "R": 0 if mk is None else int(len(mk)), "input_seed": wl.seed,
                   "weight_seed": WEIGHT_SEED, "layers": "28+2", "mode": "hipGraph replay",
                   "inputs": "device-resident",
                   "decision_layers": "head" if args.dec_head else "encoder-shaped",
                   "rope": args.rope},
        **{k: main_run[k] for k in ("p50_ms", "p95_ms", "host_boundary_p50_ms",
                                    "eager_host_boundary_p50_ms", "first_call_ms", "capture_ms",
                                    "launches_per_call")},
        "create_ms": round(st0["create_ms"], 1),
        "short_call": short,
        "roofline": roof,
        "gemm_mfma_frac": round(gemm_frac, 4),
        "profiled_pass_ms": round(pass_ms, 4),
        "ops": ops_out,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
