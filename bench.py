#!/usr/bin/env python3
"""Benchmark one absorbed-MLA decode step on one MI355X.

A step is the whole path for one batch: mla_absorb_q and mla_cache_append (in
one call, mla_absorb_q_append) -> mla_decode (split-KV + log-sum-exp merge) ->
mla_out_proj, on the DeepSeek-V3
shape workload (16 sequences x 4,096 cached rows, 128 heads, d_c = 512,
d_rope = 64, bf16).  Inputs are seeded synthetic draws, resident in HBM before
timing starts.  To measure HBM rather than the 256 MB last-level cache, the
timed loop rotates over several independent copies of the cache pool and
weights (--rotate, default 8 x 109 MB).

Prints one JSON line: whole-step tokens/s, the roofline of the dominant launch
(mla_decode, timed with HIP events on the stream it runs on), and the CPU
oracle timed on a bounded sample of the same workload on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16

# Kernel sources of one mla_decode launch; the committed HBM byte counts are
# used only while these files are unchanged.
DECODE_SOURCES = ("mla_latent_kv_36_amd/csrc/decode_mfma.hip",
                  "mla_latent_kv_36_amd/csrc/decode_generic.hip",
                  "mla_latent_kv_36_amd/csrc/common.h",
                  "mla_latent_kv_36_amd/csrc/launch.h",
                  "mla_latent_kv_36_amd/csrc/abi.hip")
TRAFFIC_FILE = "profiles/mla_decode_v3_traffic.json"


def decode_sources_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in DECODE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read() + b"\0")
    return h.hexdigest()


def measured_traffic(workload: str, splits: int):
    """HBM bytes per mla_decode launch from the committed rocprofv3 counter
    passes (FETCH_SIZE, WRITE_SIZE, each scaled by a known-size copy), or None
    if they were taken on other kernel sources or another launch shape."""
    path = os.path.join(ROOT, TRAFFIC_FILE)
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if (rec.get("sources_sha256") != decode_sources_sha256() or rec.get("workload") != workload
            or rec.get("num_splits") != splits):
        return None
    return rec


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [d.get("num_threads", 0) for d in threadpool_info()
             if d.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


def cpu_baseline(w, budget_s: float) -> dict:
    """The fp64 oracle, as it stands, on a sub-batch of the same workload
    (k sequences of the same shape and distributions), timed on this host."""
    import oracle
    from workloads import make_inputs

    def run(k):
        bt = make_inputs(w.scaled(B=k), seed=w.seed + 1000)
        t0 = time.perf_counter()
        oracle.step_ref(bt.q_nope, bt.q_rope, bt.w_uk, bt.w_uv, bt.pool, bt.block_table,
                        bt.lengths, bt.new_rows, w.d_c, w.scale, w.causal, w.block_size)
        return time.perf_counter() - t0

    # one sequence first, to size the sample: whole batches of the workload's
    # shape, repeated until about budget_s of CPU work
    t1 = run(1)
    k = int(max(1, min(w.B, budget_s / max(t1, 1e-3))))
    reps = int(max(1, round(budget_s / max(t1 * k, 1e-3))))
    dt = sum(run(k) for _ in range(reps))
    return {"value": reps * k * w.T / dt, "unit": "tokens/s", "cores": _blas_threads(),
            "kind": "oracle",
            "sample": f"fp64 numpy oracle, whole step (absorb, append, decode, out-proj), "
                      f"{reps} x {k} sequences of the workload's shape (fresh seeded draws), "
                      f"{dt:.1f} s",
            "host_cpus": os.cpu_count(), "cpu_model": _cpu_model()}


def producer_phase(w, bt, steps, torch, mla) -> dict:
    """mla_kv_produce for the step's new tokens (W^DKV / W^KR down-projection,
    RoPE on k^R, written into the cache), replayed over enough copies of the
    hidden vectors and weights (>= 512 MiB in all) that the 256 MB MALL cannot
    serve them: the weights are the bytes that bound this call."""
    from workloads import make_producer_inputs
    from workloads.device import to_dev
    pi = make_producer_inputs(w)
    cfg = mla.make_config(w.H, w.d_c, w.d_r, w.d_n, w.d_v, w.block_size, 0.0, w.dtype)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    elem = 2 if w.dtype == "bf16" else 4
    M, N, d = w.B * w.T, w.d_c + w.d_r, w.d_model
    read_bytes = (N * d + M * d) * elem
    copies = max(8, -(-(512 << 20) // read_bytes))
    base = [to_dev(a, dt, "cuda") for a in (pi.hidden, pi.w_dkv, pi.w_kr)]
    sets = [base] + [[t.clone() for t in base] for _ in range(copies - 1)]
    nbytes = mla.mla_kv_produce_workspace_size(cfg, M, d)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
    lengths = torch.from_numpy(bt.lengths.astype("int32")).cuda()
    cap = int(bt.seq_lens.max())

    def call(k):
        h, wd, wk = sets[k]
        st = steps[k % len(steps)]
        mla.mla_kv_produce(cfg, h, wd, wk, st.pool, st.block_table, lengths, cap, ws)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for k in range(copies):
            call(k)
    stream = torch.cuda.current_stream()
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * copies)
    algo = read_bytes + M * N * elem
    return {"call": "mla_kv_produce", "kernels": "kv_proj_mfma_kernel + kv_rope_append_kernel",
            "d_model": d, "tokens": M, "us": us, "bound": "hbm",
            "algorithmic_bytes": algo, "GBps": algo / (us * 1e-6) / 1e9,
            "frac": algo / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
            "k_split_workspace_bytes": nbytes, "rotated_copies": copies}


def output_side_phase(w, torch, mla) -> dict:
    """The output side after the step's W^UV up-projection: mla_o_proj (W^O over
    the concatenated heads) replayed over enough copies of W^O and the per-head
    outputs (>= 512 MiB in all) that the 256 MB MALL cannot serve them; the
    one-time fold of W^UV into W^O; and mla_o_proj_folded, the folded matrix
    (671 MB at the V2-scale widths, larger than the MALL) on the fp32 latent
    outputs."""
    from workloads import make_output_inputs
    from workloads.device import to_dev
    oi = make_output_inputs(w)
    cfg = mla.make_config(w.H, w.d_c, w.d_r, w.d_n, w.d_v, w.block_size, 0.0, w.dtype)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    elem = 2 if w.dtype == "bf16" else 4
    M, d = w.B * w.T, w.d_model
    K, Kf = w.H * w.d_v, w.H * w.d_c
    stream = torch.cuda.current_stream()

    def timed(fn, reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    def graph_of(calls):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for c in calls:
                c()
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        return g

    # W^O, rotated over copies
    wo_bytes = d * K * elem
    copies = max(8, -(-(512 << 20) // wo_bytes))
    base = [to_dev(oi.attn, dt, "cuda"), to_dev(oi.w_o, dt, "cuda")]
    sets = [base] + [[t.clone() for t in base] for _ in range(copies - 1)]
    y = torch.empty((M, d), dtype=dt, device="cuda")
    n_ws = mla.mla_o_proj_workspace_size(cfg, M, d, False)
    ws = torch.empty(max(n_ws, 256), dtype=torch.uint8, device="cuda")
    g = graph_of([lambda a=a, wo=wo: mla.mla_o_proj(cfg, a, wo, y, ws) for a, wo in sets])
    us = timed(g.replay, 5) / copies
    algo = wo_bytes + M * K * elem + M * d * elem
    out = {"o_proj": {"call": "mla_o_proj", "kernels": "wo_gemm_mfma_kernel + wo_finish_kernel",
                      "tokens": M, "k": K, "d_model": d, "us": us, "bound": "hbm",
                      "algorithmic_bytes": algo, "GBps": algo / (us * 1e-6) / 1e9,
                      "frac": algo / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                      "k_split_workspace_bytes": n_ws, "rotated_copies": copies}}
    del sets, base
    # the fold (once per model), then the folded product
    w_uv = to_dev(oi.w_uv, dt, "cuda")
    w_o = to_dev(oi.w_o, dt, "cuda")
    wf = torch.empty((d, Kf), dtype=dt, device="cuda")
    us_fold = timed(lambda: mla.mla_fold_uv_o(cfg, w_uv, w_o, wf), 3)
    fold_bytes = (d * Kf + d * K + w.H * w.d_v * w.d_c) * elem
    out["fold"] = {"call": "mla_fold_uv_o", "kernels": "fold_uv_o_kernel", "us": us_fold,
                   "algorithmic_bytes": fold_bytes, "GBps": fold_bytes / (us_fold * 1e-6) / 1e9}
    o_lat = torch.from_numpy(oi.o_lat).cuda()
    n_wsf = mla.mla_o_proj_workspace_size(cfg, M, d, True)
    wsf = torch.empty(max(n_wsf, 256), dtype=torch.uint8, device="cuda")
    g2 = graph_of([lambda: mla.mla_o_proj_folded(cfg, o_lat, wf, y, wsf)])
    us_f = timed(g2.replay, 5)
    algo_f = d * Kf * elem + M * Kf * 4 + M * d * elem
    out["o_proj_folded"] = {"call": "mla_o_proj_folded",
                            "kernels": "wo_gemm_mfma_kernel + wo_finish_kernel",
                            "us": us_f, "bound": "hbm", "algorithmic_bytes": algo_f,
                            "GBps": algo_f / (us_f * 1e-6) / 1e9,
                            "frac": algo_f / (us_f * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                            "k_split_workspace_bytes": n_wsf,
                            "weight_bytes_vs_w_o": d * Kf / (d * K)}
    del wf, g2
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="v3_decode")
    ap.add_argument("--rotate", type=int, default=8)
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB five times "
                         "(the known-size reference for HBM byte counters) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if args.copy_probe_mib > 0:
        # One elementwise kernel per call that reads n bytes and writes n bytes.
        n = args.copy_probe_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n,
                          "launches": 5}))
        return 0

    from mla_latent_kv_36_amd import binding as mla
    from mla_latent_kv_36_amd import build as mbuild
    from mla_latent_kv_36_amd.step import DecodeStep
    from workloads import BY_NAME, make_inputs
    from workloads.device import upload

    if not mbuild.built():
        mbuild.build()
    mla.load()
    w = BY_NAME[args.workload]
    torch.cuda.set_device(0)
    bt = make_inputs(w)
    cfg = mla.make_config(w.H, w.d_c, w.d_r, w.d_n, w.d_v, w.block_size, 0.0, w.dtype)
    total_tokens = int(bt.seq_lens.sum())

    steps = []
    base = upload(bt)
    for r in range(args.rotate):
        dev = dict(base)
        if r > 0:   # independent copies of everything large
            for k in ("pool", "w_uk", "w_uv"):
                dev[k] = base[k].clone()
        steps.append(DecodeStep(cfg, q_nope=dev["q_nope"], q_rope=dev["q_rope"],
                                w_uk=dev["w_uk"], w_uv=dev["w_uv"], pool=dev["pool"],
                                block_table=dev["block_table"], lengths=dev["lengths"],
                                new_rows=dev["new_rows"], max_len_after=bt.max_seq_len,
                                causal=w.causal, num_splits=args.num_splits,
                                total_tokens=total_tokens))
    splits = mla.mla_decode_num_splits(cfg, w.B, w.T, bt.max_seq_len, total_tokens) \
        if args.num_splits == 0 else args.num_splits

    # Each phase (and the whole step) over all rotated copies is captured once in
    # a HIP graph and replayed, so the timing sees GPU time, not Python launch cost.
    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for st in steps:
                fn(st)
        return g

    graphs = {
        "step": capture(lambda st: st.run()),
        "decode": capture(lambda st: st.decode()),
        "absorb_q": capture(lambda st: st.absorb()),
        "cache_append": capture(lambda st: st.append()),
        "absorb_q_append": capture(lambda st: st.absorb_append()),
        "out_proj": capture(lambda st: st.out_proj()),
    }
    stream = torch.cuda.current_stream()
    reps = max(1, -(-args.steps // args.rotate))
    wreps = max(1, -(-args.warmup // args.rotate))

    def timed(g):
        for _ in range(wreps):
            g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * args.rotate)   # ms per call

    ms_step = timed(graphs["step"])
    ms_decode = timed(graphs["decode"])
    ms_absorb = timed(graphs["absorb_q"])
    ms_append = timed(graphs["cache_append"])
    ms_absorb_append = timed(graphs["absorb_q_append"])
    ms_out = timed(graphs["out_proj"])

    W = w.d_c + w.d_r
    elem = 2 if w.dtype == "bf16" else 4
    cache_bytes = total_tokens * W * elem                       # per decode launch
    # (query, cached row) pairs: with the causal mask query t of a sequence of
    # n rows (after the append) sees n - T + t + 1 of them
    if w.causal:
        pairs = sum(int(n) * w.T - w.T * (w.T - 1) // 2 for n in bt.seq_lens)
    else:
        pairs = sum(int(n) * w.T for n in bt.seq_lens)
    decode_flops = pairs * w.H * (2 * W + 2 * w.d_c)
    gbps = cache_bytes / (ms_decode * 1e-3) / 1e9
    tflops = decode_flops / (ms_decode * 1e-3) / 1e12
    # the bound is the one the workload's arithmetic intensity puts it under
    # (T = 1 decode sits below the ridge, many queries per row above it)
    mfma_bound = decode_flops / cache_bytes > MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    tokens = w.B * w.T
    traffic = measured_traffic(w.name, splits)
    line = {
        "metric": "MLA decode tokens/s & latent-cache GB/s (% HBM peak, % MFMA) on 1 MI355X",
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": reps * args.rotate,
        "warmup": wreps * args.rotate,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) draws, bf16; no model weights)",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "H": w.H, "d_c": w.d_c,
                   "d_rope": w.d_r, "d_nope": w.d_n, "d_v": w.d_v,
                   "cached_rows_before_step": w.N, "rows_attended": int(bt.seq_lens.max()),
                   "block_size": w.block_size, "num_splits": splits,
                   "rotated_copies": args.rotate, "timing": "HIP graph replay"},
        "roofline": {"kernel": "mla_decode launch = decode_mfma_kernel + combine_kernel",
                     "bound": "mfma" if mfma_bound else "hbm",
                     "achieved": tflops if mfma_bound else gbps,
                     "peak": MFMA_BF16_PEAK_TFLOPS if mfma_bound else HBM_PEAK_GBPS,
                     "unit": "TFLOP/s" if mfma_bound else "GB/s",
                     "frac": (tflops / MFMA_BF16_PEAK_TFLOPS) if mfma_bound
                     else (gbps / HBM_PEAK_GBPS),
                     "traffic": traffic["hbm_bytes_per_launch"] if traffic else None,
                     "traffic_detail": ({k: traffic[k] for k in
                                         ("fetch_bytes_per_launch", "write_bytes_per_launch",
                                          "per_kernel", "calibration")}
                                        if traffic else None),
                     "algorithmic_bytes_per_launch": cache_bytes,
                     "avg_launch_us": ms_decode * 1e3,
                     "algorithmic_flops_per_launch": decode_flops,
                     "cache_GBps": gbps, "hbm_frac": gbps / HBM_PEAK_GBPS,
                     "mfma_tflops": tflops, "mfma_frac": tflops / MFMA_BF16_PEAK_TFLOPS},
        "latent_cache_GBps_step": cache_bytes / (ms_step * 1e-3) / 1e9,
        "decode_tokens_per_s": tokens / (ms_decode * 1e-3),
        "phases_us": {"absorb_q": ms_absorb * 1e3, "cache_append": ms_append * 1e3,
                      "absorb_q_append": ms_absorb_append * 1e3,
                      "decode": ms_decode * 1e3, "out_proj": ms_out * 1e3},
    }
    if w.d_model > 0:
        line["producer"] = producer_phase(w, bt, steps, torch, mla)
        line["output_side"] = output_side_phase(w, torch, mla)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
