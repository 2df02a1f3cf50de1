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
                  "mla_latent_kv_36_amd/csrc/merge.h",
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


def _affinity_cpus() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def cpu_baseline(w, budget_s: float) -> dict:
    """The oracle, as it stands, on a sub-batch of the same workload (k
    sequences of the same shape and distributions, fresh seeded draws), timed
    on this host: the whole step (absorb, append, decode, out-projection) in
    float32, whose per-sequence decode is the BLAS products [H x W].[W x n]
    per new token, as the median of 3 runs; the same in float64 beside it."""
    import numpy as np
    import oracle
    from workloads import make_inputs

    def run(k, dtype):
        bt = make_inputs(w.scaled(B=k), seed=w.seed + 1000)
        t0 = time.perf_counter()
        oracle.step_ref(bt.q_nope, bt.q_rope, bt.w_uk, bt.w_uv, bt.pool, bt.block_table,
                        bt.lengths, bt.new_rows, w.d_c, w.scale, w.causal, w.block_size,
                        dtype=dtype)
        return time.perf_counter() - t0

    # one sequence of each precision first, to size the sample so that three
    # runs of each take about budget_s in all
    t32, t64 = run(1, np.float32), run(1, np.float64)
    k = int(max(1, min(w.B, budget_s / max(3 * (t32 + t64), 1e-3))))
    d32 = sorted(run(k, np.float32) for _ in range(3))
    d64 = sorted(run(k, np.float64) for _ in range(3))
    threads = _blas_threads()
    return {"value": k * w.T / d32[1], "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"float32 oracle, whole step (absorb, append, decode, out-proj) on "
                      f"{k} of the workload's {w.B} sequences (same shapes and "
                      f"distributions, fresh seeded draws); median of 3 runs "
                      f"({', '.join(f'{d:.2f}' for d in d32)} s)",
            "fp64": {"value": k * w.T / d64[1], "unit": "tokens/s",
                     "runs_s": [round(d, 3) for d in d64]},
            "blas_threads": threads, "host_cpus": os.cpu_count(),
            "affinity_cpus": _affinity_cpus(), "cpu_model": _cpu_model()}


def _stats_us(samples_ms):
    import numpy as np
    a = np.asarray(samples_ms, dtype=np.float64) * 1e3
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "reps": int(a.size)}


def replay_stats(torch, g, per_replay: int, reps: int, warm: int = 5) -> dict:
    """Per-call time of a captured graph holding `per_replay` calls (one per
    rotated copy): `warm` untimed replays, then `reps` replays each between
    its own pair of HIP events on the replay stream, all enqueued before one
    synchronisation.  Returns the median, p10 and p90 per call, in us."""
    stream = torch.cuda.current_stream()
    for _ in range(warm):
        g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(stream)
    for i in range(reps):
        g.replay()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return _stats_us([ev[i].elapsed_time(ev[i + 1]) / per_replay for i in range(reps)])


def streaming_read(torch, mla, mib: int = 2048, reps: int = 20) -> dict:
    """The box's achievable HBM rate for a plain streaming read of a buffer of
    `mib` MiB (8x the 256 MB MALL): the library's mla_stream_read (16-byte
    non-temporal loads over the whole chip, the rate the decode roofline is
    set beside), and torch's sum and copy for comparison."""
    n = (mib << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record(stream)
        for i in range(reps):
            fn()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        return sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(reps))[reps // 2]

    ms_hip = timed(lambda: mla.mla_stream_read(x, sink, 0))
    ms_lds = timed(lambda: mla.mla_stream_read(x, sink, 1))
    ms_read = timed(lambda: x.sum())
    ms_copy = timed(lambda: y.copy_(x))
    del x, y, sink
    return {"read_GBps": (mib << 20) / (ms_hip * 1e-3) / 1e9,
            "read_kernel": "mla_stream_read mode 0 (16-byte non-temporal loads, 256 x 256 threads)",
            "read_direct_to_lds_GBps": (mib << 20) / (ms_lds * 1e-3) / 1e9,
            "torch_sum_GBps": (mib << 20) / (ms_read * 1e-3) / 1e9,
            "copy_GBps": 2 * (mib << 20) / (ms_copy * 1e-3) / 1e9,
            "bytes": mib << 20, "copy_kernel": "torch copy_ (fp32), read + written bytes",
            "median_of": reps}


def producer_phase(w, bt, steps, torch, mla, reps) -> dict:
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
    st_us = replay_stats(torch, g, copies, reps)
    us = st_us["median"]
    algo = read_bytes + M * N * elem
    return {"call": "mla_kv_produce", "kernels": "kv_proj_mfma_kernel + kv_rope_append_kernel",
            "d_model": d, "tokens": M, "us": us, "bound": "hbm",
            "algorithmic_bytes": algo, "GBps": algo / (us * 1e-6) / 1e9,
            "frac": algo / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, "us_stats": st_us,
            "k_split_workspace_bytes": nbytes, "rotated_copies": copies}


def output_side_phase(w, torch, mla, reps) -> dict:
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

    def timed(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

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
    st_o = replay_stats(torch, g, copies, reps)
    us = st_o["median"]
    algo = wo_bytes + M * K * elem + M * d * elem
    # the library's kernel for these token rows: up to 16 the register-streaming
    # kernel, up to 128 bf16 rows the LDS-streaming kernel, more the tiled GEMM
    o_kernel = ("wo_stream_direct_kernel" if M <= 16 else
                "wo_stream_lds_kernel" if M <= 128 and w.dtype == "bf16" else "wo_gemm_mfma_kernel")
    out = {"o_proj": {"call": "mla_o_proj", "kernels": o_kernel + " + wo_finish_kernel",
                      "tokens": M, "k": K, "d_model": d, "us": us, "bound": "hbm",
                      "algorithmic_bytes": algo, "GBps": algo / (us * 1e-6) / 1e9,
                      "frac": algo / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, "us_stats": st_o,
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
    st_f = replay_stats(torch, g2, 1, reps)
    us_f = st_f["median"]
    algo_f = d * Kf * elem + M * Kf * 4 + M * d * elem
    out["o_proj_folded"] = {"call": "mla_o_proj_folded",
                            "kernels": "wo_gemm_mfma_kernel + wo_finish_kernel",
                            "us": us_f, "bound": "hbm", "algorithmic_bytes": algo_f,
                            "GBps": algo_f / (us_f * 1e-6) / 1e9,
                            "frac": algo_f / (us_f * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                            "us_stats": st_f, "k_split_workspace_bytes": n_wsf,
                            "weight_bytes_vs_w_o": d * Kf / (d * K)}
    del wf, g2
    return out


def log(msg: str) -> None:
    """A progress line on stderr (the JSON line alone goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def decode_work(w, bt):
    """Algorithmic bytes (the cache rows read, once per sequence) and flops of
    one mla_decode call on batch bt."""
    W = w.d_c + w.d_r
    elem = 2 if w.dtype == "bf16" else 4
    cache_bytes = int(bt.seq_lens.sum()) * W * elem
    # (query, cached row) pairs: with the causal mask query t of a sequence of
    # n rows (after the append) sees n - T + t + 1 of them
    if w.causal:
        pairs = sum(int(n) * w.T - w.T * (w.T - 1) // 2 for n in bt.seq_lens)
    else:
        pairs = sum(int(n) * w.T for n in bt.seq_lens)
    return cache_bytes, pairs * w.H * (2 * W + 2 * w.d_c)


def roofline(cache_bytes, flops, us):
    """The bound the workload's arithmetic intensity puts it under (T = 1
    decode sits below the ridge, many queries per row above it) and the
    fractions of both peaks."""
    gbps = cache_bytes / (us * 1e-6) / 1e9
    tflops = flops / (us * 1e-6) / 1e12
    mfma_bound = flops / cache_bytes > MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    return {"bound": "mfma" if mfma_bound else "hbm",
            "achieved": tflops if mfma_bound else gbps,
            "peak": MFMA_BF16_PEAK_TFLOPS if mfma_bound else HBM_PEAK_GBPS,
            "unit": "TFLOP/s" if mfma_bound else "GB/s",
            "frac": (tflops / MFMA_BF16_PEAK_TFLOPS) if mfma_bound else (gbps / HBM_PEAK_GBPS),
            "cache_GBps": gbps, "hbm_frac": gbps / HBM_PEAK_GBPS,
            "mfma_tflops": tflops, "mfma_frac": tflops / MFMA_BF16_PEAK_TFLOPS}


def make_steps(w, bt, rotate, num_splits, mla, DecodeStep, copy_weights=True):
    """One DecodeStep per rotated copy: independent copies of the cache pool
    (and of the weights, when copy_weights) so that no call of a replay reads
    what the previous one left in the 256 MB MALL."""
    from workloads.device import upload
    cfg = mla.make_config(w.H, w.d_c, w.d_r, w.d_n, w.d_v, w.block_size, 0.0, w.dtype)
    total_tokens = int(bt.seq_lens.sum())
    base = upload(bt)
    steps = []
    for r in range(rotate):
        dev = dict(base)
        if r > 0:
            for k in (("pool", "w_uk", "w_uv") if copy_weights else ("pool",)):
                dev[k] = base[k].clone()
        steps.append(DecodeStep(cfg, q_nope=dev["q_nope"], q_rope=dev["q_rope"],
                                w_uk=dev["w_uk"], w_uv=dev["w_uv"], pool=dev["pool"],
                                block_table=dev["block_table"], lengths=dev["lengths"],
                                new_rows=dev["new_rows"], max_len_after=bt.max_seq_len,
                                causal=w.causal, num_splits=num_splits,
                                total_tokens=total_tokens))
    return cfg, steps


def capture(torch, steps, fn):
    """One graph holding fn(step) for every rotated copy, in order."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for st in steps:
            fn(st)
    return g


def fused_phase(torch, mla, steps, reps, us_two_kernel, cache_bytes, flops) -> dict:
    """mla_decode_fused (split-KV attention and merge in one launch) on the
    same rotated copies: per-call time, its roofline, and whether it left the
    same o_lat / lse bits as mla_decode (it does whenever the plan is plain;
    a balanced plan writes its one-split sequences directly, without the
    bf16 partial round trip)."""
    st0 = steps[0]
    try:
        mla.mla_decode_fused_workspace_size(st0.cfg, st0.B, st0.T, st0.max_len_after,
                                            st0.total_tokens, st0.num_splits)
    except RuntimeError as e:  # a shape the one-launch decode does not take
        return {"supported": False, "reason": str(e)}
    st0.decode()
    torch.cuda.synchronize()
    o_ref, lse_ref = st0.o_lat.clone(), st0.lse.clone()
    for st in steps:              # workspaces allocated (zeroed) outside the graph
        st.decode_fused()
    torch.cuda.synchronize()
    same = bool(torch.equal(st0.o_lat.view(torch.int32), o_ref.view(torch.int32)) and
                torch.equal(st0.lse.view(torch.int32), lse_ref.view(torch.int32)))
    rel = float((st0.o_lat - o_ref).abs().max() / o_ref.abs().max().clamp_min(1e-30))
    g = capture(torch, steps, lambda st: st.decode_fused())
    dec = replay_stats(torch, g, len(steps), reps)
    del g
    ctr = mla.mla_decode_fused_counter_bytes()
    zero = all(int(torch.count_nonzero(st.fused_workspace[:ctr])) == 0 for st in steps)
    rl = roofline(cache_bytes, flops, dec["median"])
    return {"call_us": dec, "vs_two_kernel": us_two_kernel / dec["median"],
            "roofline": {k: rl[k] for k in ("bound", "achieved", "peak", "unit", "frac")},
            "bitwise_equal_to_mla_decode": same, "max_rel_diff_to_mla_decode": rel,
            "counters_left_zero": zero}


def extra_workload(name, args, torch, mla, DecodeStep, reps) -> dict:
    """mla_decode of another workload, timed the same way as the main one
    (rotated copies, per-replay events), with its own roofline; the
    multi-token workload also reports its whole step."""
    from workloads import BY_NAME, make_inputs
    w = BY_NAME[name]
    log(f"{name}: drawing inputs")
    bt = make_inputs(w)
    cfg, steps = make_steps(w, bt, args.rotate, 0, mla, DecodeStep, copy_weights=False)
    log(f"{name}: timing")
    for st in steps:            # the appended rows and absorbed queries decode reads
        st.absorb_append()
    torch.cuda.synchronize()
    g = capture(torch, steps, lambda st: st.decode())
    dec = replay_stats(torch, g, len(steps), reps)
    del g
    cache_bytes, flops = decode_work(w, bt)
    tokens = w.B * w.T
    out = {"workload": name, "B": w.B, "T": w.T, "H": w.H, "rows_attended_max": int(bt.seq_lens.max()),
           "total_rows": int(bt.seq_lens.sum()),
           "num_splits": mla.mla_decode_num_splits(cfg, w.B, w.T, bt.max_seq_len,
                                                   int(bt.seq_lens.sum())),
           "decode_us": dec, "decode_tokens_per_s": tokens / (dec["median"] * 1e-6),
           "algorithmic_bytes_per_launch": cache_bytes,
           "algorithmic_flops_per_launch": flops,
           "roofline": roofline(cache_bytes, flops, dec["median"]),
           "rotated_copies": len(steps)}
    log(f"{name}: one-launch decode")
    out["decode_fused"] = fused_phase(torch, mla, steps, reps, dec["median"], cache_bytes, flops)
    if w.T > 1:
        gs = capture(torch, steps, lambda st: st.run())
        stp = replay_stats(torch, gs, len(steps), reps)
        out["step_us"] = stp
        out["step_tokens_per_s"] = tokens / (stp["median"] * 1e-6)
        del gs
    del steps
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


EXTRA_WORKLOADS = ("varlen_serving", "long_128k", "v2_multi_token")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="v3_decode")
    ap.add_argument("--rotate", type=int, default=8)
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--phase-reps", type=int, default=50,
                    help="graph replays per timed phase (each replay: one call per copy)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other workloads' mla_decode timings")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB and the "
                         "library's streaming read of it in both modes, five times "
                         "each (known-size references for HBM byte counters), and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0 or args.rotate < 1 or args.phase_reps < 1:
        print("--steps, --rotate and --phase-reps must be >= 1, --warmup >= 0",
              file=sys.stderr)
        return 2

    import torch

    if args.copy_probe_mib > 0:
        # Kernels of known bytes for the HBM byte counters: one elementwise
        # kernel per call that reads n bytes and writes n bytes, then the
        # library's streaming read of n bytes through registers (mode 0) and
        # through direct-to-LDS copies (mode 1, the decode kernel's path).
        n = args.copy_probe_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.mul(src, 1.0, out=dst)
        from mla_latent_kv_36_amd import binding as mla
        sink = torch.zeros(4, dtype=torch.int32, device="cuda")
        for mode in (0, 1):
            for _ in range(5):
                mla.mla_stream_read(src, sink, mode)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n,
                          "stream_read_bytes": n, "launches": 5}))
        return 0

    from mla_latent_kv_36_amd import binding as mla
    from mla_latent_kv_36_amd import build as mbuild
    from mla_latent_kv_36_amd.step import DecodeStep
    from workloads import BY_NAME, make_inputs

    if not mbuild.built():
        mbuild.build()
    mla.load()
    w = BY_NAME[args.workload]
    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)
    log(f"{w.name}: drawing inputs")
    bt = make_inputs(w)
    cfg, steps = make_steps(w, bt, args.rotate, args.num_splits, mla, DecodeStep)
    total_tokens = int(bt.seq_lens.sum())
    splits = mla.mla_decode_num_splits(cfg, w.B, w.T, bt.max_seq_len, total_tokens) \
        if args.num_splits == 0 else args.num_splits
    stream = torch.cuda.current_stream()

    # The step: one graph per rotated copy (absorb + append, then decode +
    # out-projection: mla_absorb_q_append and mla_decode_out_proj), replayed
    # in turn: `warmup` untimed steps, then exactly `steps` timed ones between
    # two synchronisations.
    step_graphs = [capture(torch, [st], lambda x: x.run()) for st in steps]
    for i in range(args.warmup):
        step_graphs[i % len(step_graphs)].replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step_graphs[(args.warmup + i) % len(step_graphs)].replay()
    e1.record(stream)
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / args.steps
    log(f"{args.steps} steps timed: {ms_step * 1e3:.1f} us per step")

    # Each phase over all rotated copies in one graph, timed per replay.
    phase_fns = {"decode": lambda st: st.decode(), "absorb_q": lambda st: st.absorb(),
                 "cache_append": lambda st: st.append(),
                 "absorb_q_append": lambda st: st.absorb_append(),
                 "out_proj": lambda st: st.out_proj(),
                 "decode_out_proj": lambda st: st.decode_out_proj()}
    phases = {}
    for name, fn in phase_fns.items():
        g = capture(torch, steps, fn)
        phases[name] = replay_stats(torch, g, len(steps), args.phase_reps)
        del g
        log(f"phase {name}: median {phases[name]['median']:.2f} us per call")
    us_decode = phases["decode"]["median"]

    cache_bytes, decode_flops = decode_work(w, bt)
    tokens = w.B * w.T
    traffic = measured_traffic(w.name, splits)
    rl = roofline(cache_bytes, decode_flops, us_decode)
    line = {
        "metric": "MLA decode tokens/s & latent-cache GB/s (% HBM peak, % MFMA) on 1 MI355X",
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
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
                   "rotated_copies": args.rotate,
                   "timing": "HIP graph replay; step: one graph per rotated copy, "
                             "replayed in turn; phases: per-replay HIP events"},
        "roofline": dict(
            {"kernel": "mla_decode call (split kernel + log-sum-exp merge), median of "
                       f"{args.phase_reps} replays x {args.rotate} calls"},
            **{k: rl[k] for k in ("bound", "achieved", "peak", "unit", "frac")},
            traffic=traffic["hbm_bytes_per_launch"] if traffic else None,
            traffic_detail=({k: traffic[k] for k in
                             ("fetch_bytes_per_launch", "write_bytes_per_launch",
                              "per_kernel", "calibration")} if traffic else None),
            algorithmic_bytes_per_launch=cache_bytes,
            algorithmic_flops_per_launch=decode_flops,
            launch_us=phases["decode"],
            **{k: rl[k] for k in ("cache_GBps", "hbm_frac", "mfma_tflops", "mfma_frac")}),
        "wall_s_timed_steps": wall_s,
        "latent_cache_GBps_step": cache_bytes / (ms_step * 1e-3) / 1e9,
        "decode_tokens_per_s": tokens / (us_decode * 1e-6),
        "phases_us": phases,
        "device": {"name": props.name, "compute_units": props.multi_processor_count,
                   "gcn_arch": getattr(props, "gcnArchName", "")},
    }
    del step_graphs
    log("one-launch decode")
    line["decode_fused"] = fused_phase(torch, mla, steps, args.phase_reps, us_decode,
                                       cache_bytes, decode_flops)
    line["achievable_hbm"] = streaming_read(torch, mla)
    if line["roofline"]["unit"] == "GB/s":  # the measured read rate beside the published peak
        ach = line["achievable_hbm"]["read_GBps"]
        line["roofline"]["achievable_read_GBps"] = ach
        line["roofline"]["frac_of_achievable"] = line["roofline"]["achieved"] / ach
    if w.d_model > 0:
        line["producer"] = producer_phase(w, bt, steps, torch, mla, args.phase_reps)
        line["output_side"] = output_side_phase(w, torch, mla, args.phase_reps)
    del steps
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_extra:
        line["workloads"] = {name: extra_workload(name, args, torch, mla, DecodeStep,
                                                  args.phase_reps)
                             for name in EXTRA_WORKLOADS if name != w.name}
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
