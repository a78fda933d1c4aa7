"""Benchmark of one absorbed-MLA decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload v3_b32_s4096] [--only]

A step is the whole decode path of one layer for one batch: mla_absorb_q,
mla_decode_latent (split-KV; variable-length batches through the
length-aware plan of mla_plan_decode_splits) and the merge + W_UV
(mla_combine_expand_v), on seeded synthetic inputs already resident in HBM,
rotated over enough replicas that every step streams its latent cache from
HBM (the working set exceeds the 256 MB Infinity Cache).

Prints one JSON line:
  value           latent-KV GB/s of the headline workload (V3, B=32, 4096
                  tokens) over the whole step: W untimed steps, then the K
                  steps as one HIP graph replay between two synchronisations,
                  its GPU time from HIP events at the replay's ends, with a
                  spin kernel ahead of the first event so that the host's
                  submission of the graph is not timed (the host clock around
                  another replay: ms_per_step_host_clock)
  step_us_stats   per-step time over 7 more replays, each timed the same
                  way: median / p10 / p90
  roofline        the dominant kernel (mla_decode_latent): algorithmic cache
                  bytes per launch / its mean launch duration (HIP events at the
                  ends of graph replays of 16 back-to-back launches on the
                  launch stream), against 8 TB/s; traffic from the committed
                  rocprofv3 byte counters
  sclk            the shader clock sampled while the step runs
  configs         every workload (the 26-token V2-Lite step, V2-Lite B=64,
                  V3 B=32, paged V3 B=128 with varied lengths, E4M3 V3 B=64
                  at 32,768 tokens): step and decode-kernel time statistics,
                  and GB/s, TFLOP/s and tokens/s each with its fraction of the
                  roofline (max of cache bytes / 8 TB/s and core FLOPs /
                  2.5 PFLOP/s bf16, or 5.0 PFLOP/s fp8 for the 128-head
                  E4M3 workload, whose products run on fp8 MFMAs)
  fused_step      (contexts up to 2048) mla_decode_step_fused, the same step
                  in one launch, GPU time per step from graph replays
  prefill         mla_prefill_latent on prompt / chunk shapes, TFLOP/s against
                  the bf16 MFMA peak
  naive           mla_naive_decode (expand every step) on the same inputs,
                  and the absorbed step's speedup over it
  crossover_v2lite_b1   naive vs absorbed vs fused against context length
                  (H=16, one sequence)
  append          mla_cache_append on the same shape (timed apart from the
                  step): one token per sequence, and the whole history in one
                  call against the HBM roofline (input read + cache write bytes)
  cpu_baseline    the float64 oracle on all host cores, on a bounded sample of
                  the same workload, in the same unit (cpu_baseline_1core: one
                  core)
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
FP8_MFMA_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 MFMA (the 128-head E4M3 kernel)
METRIC = "MLA decode latent-KV GB/s + TFLOP/s (% roofline), V3 H=128 B=32 S=4096"
METRIC_OTHER = "MLA decode latent-KV GB/s + TFLOP/s (% roofline), {}"
COUNTERS_FILE = os.path.join(ROOT, "profiles", "decode_latent_v3_b32_s4096_hbm_counters.json")
KERNEL_SOURCES = ["mla_absorbed_latent_absorb_amd/csrc/decode_latent.hip",
                  "mla_absorbed_latent_absorb_amd/csrc/decode_latent_wide.hip",
                  "mla_absorbed_latent_absorb_amd/csrc/tile_layout.hpp",
                  "mla_absorbed_latent_absorb_amd/csrc/device_common.hpp"]


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def core_flops(B, H, lens_sum):
    """Score (2*H*576) + latent P.V (2*H*512) multiply-adds per cached token."""
    return 2 * H * (576 + 512) * lens_sum


def proj_flops(B, H):
    """absorb_q + expand_v: 2 * B * H * 128 * 512 each."""
    return 2 * 2 * B * H * 128 * 512


def traffic_from_counters(workload):
    """HBM bytes per decode launch from the committed rocprofv3 counter runs,
    or None when they are missing, were taken on another workload, or the
    kernel source changed since."""
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_hash") != kernel_source_hash() or c.get("workload") != workload:
        return None
    return c.get("hbm_bytes_per_launch")


def cpu_baseline(x, target_s=10.0):
    """Time the float64 oracle (as it stands) on the host cores: absorbed
    decode of the workload's sequences one at a time, cycling over the batch
    until about target_s seconds of CPU work."""
    import oracle
    from tests.gpu_helpers import cache_args, f64
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover - informational only
        threads = os.cpu_count()
    args = cache_args(x)
    qn, qp, wuk, wuv = f64(x.q_nope), f64(x.q_pe), f64(x.w_uk), f64(x.w_uv)
    lens = x.seq_lens.cpu().numpy()
    per_tok = 1152 if x.workload.dtype == "bf16" else 580
    n_seq, nbytes, t_total = 0, 0, 0.0
    while t_total < target_s:
        b = n_seq % x.batch
        t0 = time.perf_counter()
        oracle.absorbed_decode(qn, qp, wuk, wuv, seq_lens=lens, scale=x.scale, batch_indices=[b], **args)
        t_total += time.perf_counter() - t0
        n_seq += 1
        nbytes += int(lens[b]) * per_tok
    return {"value": round(nbytes / t_total / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n_seq} sequence decodes cycling over the {x.batch} sequences of {x.workload.name} "
                      f"(absorbed form, float64 NumPy; {nbytes} cache bytes in {t_total:.2f} s; "
                      f"{os.cpu_count()} host CPUs visible)"}


COPY_ELEMS = 1 << 28          # float32 elements of the calibration copy (1 GiB each way)
PMC_COMMANDS = [
    "export TMPDIR=/tmp",
    "timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE -d $PWD/gpurun_out/pmc_fetch -o run --output-format csv "
    "-- python -u $PWD/bench.py --copy-calibration --steps 10 --warmup 2 --only --no-cpu-baseline --no-append --no-naive --no-prefill",
    "timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE -d $PWD/gpurun_out/pmc_write -o run --output-format csv "
    "-- python -u $PWD/bench.py --copy-calibration --steps 10 --warmup 2 --only --no-cpu-baseline --no-append --no-naive --no-prefill",
    "python bench.py --summarize-counters gpurun_out/pmc_fetch/run_counter_collection.csv "
    "gpurun_out/pmc_write/run_counter_collection.csv",
]


def _counter_means(path, counter):
    """Mean counter value per dispatch, by kernel name, from a rocprofv3
    counter_collection.csv (FETCH_SIZE / WRITE_SIZE are KiB per dispatch)."""
    import csv
    acc = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            k = row["Kernel_Name"]
            n, t = acc.get(k, (0, 0.0))
            acc[k] = (n + 1, t + float(row["Counter_Value"]))
    return {k: (t / n, n) for k, (n, t) in acc.items()}


def _pick(means, pattern):
    hits = [(k, v) for k, v in means.items() if pattern in k]
    if len(hits) != 1:
        raise SystemExit(f"expected one kernel matching {pattern!r} in the counter file, found {len(hits)}")
    return hits[0]


def summarize_trace(trace_csv):
    """Print a markdown table of this library's kernels from a rocprofv3
    --kernel-trace CSV, one line per (kernel, launch grid): calls and
    average / min / max duration in microseconds."""
    import csv
    groups = {}
    with open(trace_csv) as f:
        for row in csv.DictReader(f):
            name = row["Kernel_Name"]
            if "mla::" not in name:
                continue
            short = name.replace("(anonymous namespace)::", "").split("(")[0]
            short = short.replace("void ", "").replace("mla::", "")
            grid = "x".join(str(int(row[k]) // (int(row[w]) if k == "Grid_Size_X" else 1))
                            for k, w in (("Grid_Size_X", "Workgroup_Size_X"), ("Grid_Size_Y", ""),
                                         ("Grid_Size_Z", "")))
            d = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) * 1e-3
            groups.setdefault((short, grid), []).append(d)
    print("| kernel | workgroups (x*y*z) | calls | average (us) | min (us) | max (us) |")
    print("|---|---|---|---|---|---|")
    for (k, g), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        print(f"| `{k}` | {g} | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} |")


def summarize_counters(args, fetch_csv, write_csv):
    """HBM bytes per decode launch = counter KiB x 1024, each counter scaled by
    (known bytes / counter reading) of the calibration copy kernel."""
    fetch = _counter_means(fetch_csv, "FETCH_SIZE")
    write = _counter_means(write_csv, "WRITE_SIZE")
    name, (dec_f, n_f) = _pick(fetch, "decode_latent")
    _, (dec_w, n_w) = _pick(write, "decode_latent")
    _, (cp_f, _) = _pick(fetch, "neg_kernel")
    _, (cp_w, _) = _pick(write, "neg_kernel")
    copy_kib = COPY_ELEMS * 4 / 1024
    rs, ws = copy_kib / cp_f, copy_kib / cp_w
    rd, wr = dec_f * rs * 1024, dec_w * ws * 1024
    out = {
        "kernel": name,
        "workload": args.workload,
        "kernel_source_hash": kernel_source_hash(),
        "decode_fetch_kib_per_launch": round(dec_f, 1),
        "decode_write_kib_per_launch": round(dec_w, 1),
        "launches": [n_f, n_w],
        "copy_fetch_kib": round(cp_f, 1),
        "copy_write_kib": round(cp_w, 1),
        "copy_known_kib": copy_kib,
        "read_scale": round(rs, 4),
        "write_scale": round(ws, 4),
        "hbm_read_bytes_per_launch": int(rd),
        "hbm_write_bytes_per_launch": int(wr),
        "hbm_bytes_per_launch": int(rd + wr),
        "commands": PMC_COMMANDS,
    }
    with open(COUNTERS_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def graph_time_per_call(fn, n_cap, reps):
    """GPU time per call of fn: n_cap calls captured in one HIP graph, replayed
    `reps` times between two events (one untimed replay first)."""
    import torch

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(n_cap):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    del graph
    return e0.elapsed_time(e1) * 1e-3 / (reps * n_cap)


NAIVE_MAX_WORKSPACE = 16 << 30   # expanded rows the naive baseline may hold
CROSSOVER_CONTEXTS = [64, 256, 1024, 4096, 16384]


def bench_naive(x0, d, dev, absorbed_step_s):
    """The naive (expand every step) decode on the workload, against the
    absorbed step; None when its expanded rows would exceed 16 GiB."""
    import torch
    from mla_absorbed_latent_absorb_amd import binding

    need = binding.mla_naive_workspace_bytes(d, x0.max_seq_len)
    if need > NAIVE_MAX_WORKSPACE:
        return None
    cache = binding.make_cache(x0.kv_rows, x0.pe_rows, seq_stride=x0.seq_stride, block_table=x0.block_table,
                               block_size=x0.block_size, token_scale=x0.token_scale)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    out = torch.empty((x0.batch, x0.heads, 128), dtype=torch.bfloat16, device=dev)

    def call():
        binding.mla_naive_decode(d, cache, x0.q_nope, x0.q_pe, x0.w_uk, x0.w_uv, x0.seq_lens, x0.max_seq_len,
                                 workspace=ws, out=out)

    call()
    torch.cuda.synchronize()
    t = graph_time_per_call(call, 4, 3)
    flops = 2 * 2 * x0.heads * 128 * 512 * int(x0.seq_lens.to(torch.int64).sum().item())
    del ws
    torch.cuda.empty_cache()
    return {"kernel": "mla_naive_decode", "step_us": round(t * 1e6, 2),
            "absorbed_speedup": round(t / absorbed_step_s, 2),
            "expand_tflops": round(flops / t / 1e12, 1), "workspace_bytes": need}


def bench_crossover(dev):
    """Naive vs absorbed (three launches) vs fused one-launch step against context
    length at the V2-Lite shape with one sequence (H=16), the setting of the
    pages' naive-vs-absorbed latency comparison; GPU time per step from graph
    replays."""
    import torch
    from mla_absorbed_latent_absorb_amd import binding, datagen

    rows = []
    ncu = torch.cuda.get_device_properties(dev).multi_processor_count
    for T in CROSSOVER_CONTEXTS:
        x = datagen.make_inputs(datagen.WORKLOADS["v2lite_b64_s4096"], device=dev, batch=1, seq_len=T)
        d = binding.dims(1, x.heads, x.scale)
        cache = binding.make_cache(x.kv_rows, x.pe_rows, seq_stride=x.seq_stride)
        P = binding.mla_recommended_splits(d, T, ncu)
        step = binding.DecodeStep(d, cache, x.seq_lens, T, P, dev)
        ws = torch.empty(binding.mla_naive_workspace_bytes(d, T), dtype=torch.uint8, device=dev)
        out = torch.empty((1, x.heads, 128), dtype=torch.bfloat16, device=dev)
        absorbed = lambda: step(x.q_nope, x.q_pe, x.w_uk, x.w_uv)
        naive = lambda: binding.mla_naive_decode(d, cache, x.q_nope, x.q_pe, x.w_uk, x.w_uv, x.seq_lens, T,
                                                 workspace=ws, out=out)
        fused = lambda: binding.mla_decode_step_fused(d, cache, x.q_nope, x.q_pe, x.w_uk, x.w_uv, x.seq_lens, T,
                                                      out=out)
        for f in (absorbed, naive, fused):
            f()
        torch.cuda.synchronize()
        row = {"context": T, "splits": P,
               "absorbed_us": round(graph_time_per_call(absorbed, 16, 4) * 1e6, 2),
               "naive_us": round(graph_time_per_call(naive, 16, 4) * 1e6, 2)}
        if T <= FUSED_MAX_CONTEXT:
            row["fused_us"] = round(graph_time_per_call(fused, 16, 4) * 1e6, 2)
        rows.append(row)
        del ws, step
    torch.cuda.empty_cache()
    return rows


PREFILL_CASES = [  # (name, workload, heads, batch, context, chunk)
    ("v3_last_chunk", "v3_b32_s4096", 128, 2, 4096, 512),
    ("v3_prompt_4096", "v3_b32_s4096", 128, 1, 4096, 4096),
    ("v2lite_prompt_4096", "v2lite_b64_s4096", 16, 1, 4096, 4096),
]


def bench_prefill(dev):
    """mla_prefill_latent (causal latent attention of a prefill chunk whose rows
    are already cached) against the bf16 MFMA peak: FLOPs = sum over query
    rows of 2 * H * (576 + 512) * (causal prefix length)."""
    import torch
    from mla_absorbed_latent_absorb_amd import binding, datagen

    res = {}
    for name, wl, H, B, S, L in PREFILL_CASES:
        x = datagen.make_inputs(datagen.WORKLOADS[wl], device=dev, batch=B, seq_len=S, heads=H)
        d = binding.dims(B, H, x.scale)
        cache = binding.make_cache(x.kv_rows, x.pe_rows, seq_stride=x.seq_stride)
        q_lat = datagen.random_latent_queries(B * L, H, 5, device=dev).view(B, L, H, 512)
        q_pe = datagen.random_latent_queries(B * L, H, 6, device=dev)[..., :64].contiguous().view(B, L, H, 64)
        q_start = torch.full((B,), S - L, dtype=torch.int32, device=dev)
        o_lat = torch.empty((B, L, H, 512), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((B, L, H), dtype=torch.float32, device=dev)
        call = lambda: binding.mla_prefill_latent(d, cache, q_lat, q_pe, q_start, S, o_lat=o_lat, lse=lse)
        call()
        torch.cuda.synchronize()
        t = graph_time_per_call(call, 2, 3)
        rows_tokens = B * sum(S - L + i + 1 for i in range(L))
        flops = 2 * H * (576 + 512) * rows_tokens
        tf = flops / t / 1e12
        res[name] = {"heads": H, "batch": B, "context": S, "chunk": L, "us": round(t * 1e6, 1),
                     "tflops": round(tf, 1), "mfma_frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4)}
        del x, q_lat, q_pe, o_lat
    torch.cuda.empty_cache()
    return res


FUSED_MAX_CONTEXT = 2048   # the fused one-launch step is timed on short contexts only


def bench_fused_step(x0, d, dev, steps):
    """mla_decode_step_fused (absorb + attention + expand in one launch) on the
    same inputs: 32 launches captured in a HIP graph and replayed, so the
    figure is GPU time per step."""
    import torch
    from mla_absorbed_latent_absorb_amd import binding

    cache = binding.make_cache(x0.kv_rows, x0.pe_rows, seq_stride=x0.seq_stride, block_table=x0.block_table,
                               block_size=x0.block_size, token_scale=x0.token_scale)
    out = torch.empty((x0.batch, x0.heads, 128), dtype=torch.bfloat16, device=dev)

    def call():
        binding.mla_decode_step_fused(d, cache, x0.q_nope, x0.q_pe, x0.w_uk, x0.w_uv, x0.seq_lens, x0.max_seq_len,
                                      out=out)

    for _ in range(5):
        call()
    torch.cuda.synchronize()
    n_cap = 32
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(n_cap):
            call()
    graph.replay()
    torch.cuda.synchronize()
    reps = max(2, steps // 10)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / (reps * n_cap)
    del graph
    return {"kernel": "mla_decode_step_fused", "step_us": round(t * 1e6, 3),
            "timing": "HIP graph of 32 launches, replayed"}


def bench_append(x0, d, dev, steps):
    """Time mla_cache_append on the workload's shape: one new token per
    sequence (a decode step's write, launch-bound) and the whole history in one
    call (a prefill's write, HBM-bound: reads 1152 B of bf16 input and writes
    one cache row per token).  Writes go to buffers of their own, so the
    decode inputs stay untouched."""
    import torch
    from mla_absorbed_latent_absorb_amd import binding, datagen

    B, T = x0.batch, x0.max_seq_len
    fp8 = x0.workload.dtype == "fp8_e4m3"
    row_bytes = 576 + 4 if fp8 else 1152
    ad = binding.dims(B, x0.heads, x0.scale)

    def new_cache(seq_stride):
        store = torch.empty((B * seq_stride, 576), dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev)
        scale = torch.empty((B * seq_stride,), dtype=torch.float32, device=dev) if fp8 else None
        return binding.make_cache(store[:, :512], store[:, 512:], seq_stride=seq_stride, token_scale=scale)

    def timed(calls, n):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i in range(n):
            ev[i][0].record()
            calls[i % len(calls)]()
            ev[i][1].record()
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in ev) / n * 1e-3

    # decode step: one token per sequence at position T - 1.  The launch is
    # shorter than its host-side enqueue, so the calls are captured in a HIP
    # graph and timed over graph replays (the GPU's own time per launch).
    one = [datagen.random_projection_rows(B, 1, 900 + i, device=dev) for i in range(4)]
    pos_last = torch.full((B,), T - 1, dtype=torch.int32, device=dev)
    c_dec = new_cache(T)
    n_cap = 32
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for k in range(n_cap):
            binding.mla_cache_append(ad, c_dec, one[k % len(one)], pos_last)
    graph.replay()
    torch.cuda.synchronize()
    reps = max(2, steps // 10)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    t_one = e0.elapsed_time(e1) * 1e-3 / (reps * n_cap)
    del graph

    # prefill: the whole history in one call, two input and two output buffers in turn
    ins = [datagen.random_projection_rows(B, T, 910 + i, device=dev) for i in range(2)]
    outs = [new_cache(T) for _ in range(2)]
    zero = torch.zeros((B,), dtype=torch.int32, device=dev)
    pre_calls = [lambda k=k: binding.mla_cache_append(ad, outs[k % 2], ins[(k // 2) % 2], zero) for k in range(4)]
    n_pre = max(4, min(steps, 40))
    timed(pre_calls, 4)
    t_all = timed(pre_calls, n_pre)
    moved = B * T * (1152 + row_bytes)
    del ins, outs, c_dec
    torch.cuda.empty_cache()
    return {
        "kernel": "mla_cache_append",
        "one_token_per_seq_us": round(t_one * 1e6, 3),
        "one_token_per_seq_timing": "HIP graph of 32 launches, replayed",
        "whole_history_us": round(t_all * 1e6, 3),
        "whole_history_tokens": B * T,
        "whole_history_bytes": moved,
        "roofline": {"bound": "hbm", "achieved": round(moved / t_all / 1e9, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(moved / t_all / 1e9 / HBM_PEAK_GBS, 4)},
    }


def _stats(xs):
    """median / p10 / p90 / mean of a list of durations (seconds) in us."""
    import numpy as np
    v = np.asarray(xs, dtype=np.float64) * 1e6
    return {"median": round(float(np.median(v)), 3), "p10": round(float(np.percentile(v, 10)), 3),
            "p90": round(float(np.percentile(v, 90)), 3), "mean": round(float(v.mean()), 3), "n": int(v.size)}


class SclkSampler:
    """Samples the GPU's current shader clock (the level the driver marks in
    pp_dpm_sclk) in a thread while the timed work runs."""

    def __init__(self):
        import glob
        self.path = next(iter(sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))), None)
        self.samples = []
        self._stop = False

    def _read(self):
        try:
            with open(self.path) as f:
                for line in f:
                    if line.strip().endswith("*"):
                        return int(line.split(":")[1].strip().lower().split("mhz")[0])
        except (OSError, ValueError, IndexError):
            return None
        return None

    def __enter__(self):
        import threading
        if self.path is not None:
            def loop():
                while not self._stop:
                    v = self._read()
                    if v is not None:
                        self.samples.append(v)
                    time.sleep(0.002)
            self._t = threading.Thread(target=loop, daemon=True)
            self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop = True
        if self.path is not None:
            self._t.join()

    def summary(self):
        import numpy as np
        if not self.samples:
            return None
        v = np.asarray(self.samples)
        busy = v[v > 500]   # levels below 500 MHz are idle moments between replays
        if busy.size == 0:
            busy = v
        return {"median_mhz": int(np.median(busy)), "min_mhz": int(busy.min()), "max_mhz": int(busy.max()),
                "samples": int(v.size), "source": "pp_dpm_sclk (current level) sampled every 2 ms during graph "
                                                  "replays of the step"}


# the five workloads of the decode benchmark (headline: v3_b32_s4096)
CONFIGS = ["v2lite_b1_s26", "v2lite_b64_s4096", "v3_b32_s4096", "v3_b128_paged", "v3_b64_s32768_fp8"]


def measure_config(name, dev, steps, warmup, splits=0, replicas=0, sample_sclk=False):
    """Time the whole decode step of one workload on inputs resident in HBM.

    Step: mla_absorb_q, then the latent attention (split-KV with the library's
    recommended split count; variable-length batches through the length-aware
    plan, mla_plan_decode_splits, computed on the host from the host lengths
    as an input of the step like seq_lens), then the merge + W_UV
    (mla_combine_expand_v[_planned]) or W_UV alone (one split).  Input replicas
    rotate so the working set exceeds the 256 MB Infinity Cache.

      headline      `steps` steps as ONE HIP graph replay between two
                    synchronisations (HIP events at its ends, a spin kernel
                    ahead of them while the host submits the graph; the host
                    clock around another replay beside it)
      step_us       per-step time of 7 more replays timed the same way:
                    median / p10 / p90
      decode_us     mla_decode_latent[_planned] alone: 16 launches (inputs
                    rotating over the replicas) captured in a HIP graph, 9
                    replays each timed with HIP events at its ends on the
                    launch stream -> mean launch duration per replay
      merge_expand_us  the launch after it, timed the same way
    """
    import torch
    from mla_absorbed_latent_absorb_amd import binding, datagen

    props = torch.cuda.get_device_properties(dev)
    wl = datagen.WORKLOADS[name]
    x0 = datagen.make_inputs(wl, device=dev)
    cache_bytes = x0.cache_bytes()
    R = replicas or min(64, max(2, math.ceil(512e6 / cache_bytes) + 1))
    reps = [x0] + [datagen.make_inputs(wl, device=dev) for _ in range(R - 1)]
    d = binding.dims(x0.batch, x0.heads, x0.scale)
    lens_host = x0.seq_lens.cpu().tolist()
    planned = wl.len_range is not None and not splits
    P = splits or binding.mla_recommended_splits(d, x0.max_seq_len, props.multi_processor_count)
    plan = binding.mla_plan_decode_splits(d, lens_host, x0.max_seq_len, props.multi_processor_count,
                                          device=dev) if planned else None
    steps_objs = []
    for x in reps:
        cache = binding.make_cache(x.kv_rows, x.pe_rows, seq_stride=x.seq_stride, block_table=x.block_table,
                                   block_size=x.block_size, token_scale=x.token_scale)
        if planned:
            st = binding.PlannedDecodeStep(d, cache, x.seq_lens, x.max_seq_len, plan, dev, keep_latent=False)
        else:
            st = binding.DecodeStep(d, cache, x.seq_lens, x.max_seq_len, P, dev, keep_latent=False)
        steps_objs.append((x, st))

    def run(i, ev=None):
        x, st = steps_objs[i % R]
        binding.mla_absorb_q(d, x.q_nope, x.w_uk, q_lat=st.q_lat)
        if ev is not None:
            ev[0].record()
        st.decode(x.q_pe)
        if ev is not None:
            ev[1].record()
        st.finish(x.w_uv)
        if ev is not None:
            ev[2].record()

    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()

    # eager step: every call launched from Python
    t0 = time.perf_counter()
    for i in range(steps):
        run(i)
    torch.cuda.synchronize()
    t_eager = (time.perf_counter() - t0) / steps

    # headline: the K steps as one graph replay between two synchronisations
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(steps):
            run(i)
    graph.replay()  # untimed: the first replay uploads the graph
    torch.cuda.synchronize()
    # The host clock around one replay between two synchronisations (one
    # graph launch and one synchronisation included).
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    t_host = (time.perf_counter() - t0) / steps
    # The timed region: exactly the K steps, one graph replay between two
    # synchronisations, its GPU time from HIP events recorded at the replay's
    # two ends on the launch stream.  A spin kernel queued before the first
    # event keeps the GPU busy while the host submits the graph's launches
    # (~1 us each), so the events time the steps' execution, not the
    # submission lag that an idle GPU would wait through (at K = 20 that lag
    # adds ~3-6 us per V3 step; at K = 200 the figures agree).
    spin_cycles = int(2e6 + 4000 * 3 * steps)
    spin = getattr(torch.cuda, "_sleep", None)  # torch's bounded spin kernel

    def timed_replay():
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if spin is not None:
            spin(spin_cycles)
        e0.record()
        graph.replay()
        e1.record()
        return e0, e1

    e_start, e_end = timed_replay()
    torch.cuda.synchronize()
    t_step = e_start.elapsed_time(e_end) * 1e-3 / steps
    # repeated replays, each timed the same way
    n_rep = 7
    evs = [timed_replay() for _ in range(n_rep)]
    torch.cuda.synchronize()
    per_step = [e0.elapsed_time(e1) * 1e-3 / steps for e0, e1 in evs]
    sclk = None
    if sample_sclk:
        sampler = SclkSampler()
        with sampler:
            t_end = time.perf_counter() + 0.4
            while time.perf_counter() < t_end:
                graph.replay()
                torch.cuda.synchronize()
        sclk = sampler.summary()
    del graph

    # kernel launches: n_k launches of one kernel alone (inputs rotating over
    # the replicas) captured in a graph; each replay timed with HIP events at
    # its ends gives that replay's mean launch duration
    def kernel_replays(fn):
        n_k = 16
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n_k):
                fn(i)
        g.replay()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(9)]
        for e0, e1 in ev:
            e0.record()
            g.replay()
            e1.record()
        torch.cuda.synchronize()
        del g
        return [e0.elapsed_time(e1) * 1e-3 / n_k for e0, e1 in ev]

    def dec_only(i):
        x, st = steps_objs[i % R]
        st.decode(x.q_pe)

    def tail_only(i):
        x, st = steps_objs[i % R]
        st.finish(x.w_uv)

    dec = kernel_replays(dec_only)
    tail = kernel_replays(tail_only)

    lens_sum = sum(int(v) for v in lens_host)
    flops = core_flops(x0.batch, x0.heads, lens_sum)
    fp8 = wl.dtype == "fp8_e4m3"
    fp8_mfma = fp8 and x0.heads == 128
    mfma_peak = FP8_MFMA_PEAK_TFLOPS if fp8_mfma else BF16_MFMA_PEAK_TFLOPS
    t_med = float(sorted(per_step)[len(per_step) // 2])
    t_dec = sum(dec) / len(dec)
    t_roof = max(cache_bytes / (HBM_PEAK_GBS * 1e9), flops / (mfma_peak * 1e12))
    bound = "hbm" if cache_bytes / (HBM_PEAK_GBS * 1e9) >= flops / (mfma_peak * 1e12) else "mfma"

    def rates(t):
        return {"gbs": round(cache_bytes / t / 1e9, 2), "hbm_frac": round(cache_bytes / t / 1e9 / HBM_PEAK_GBS, 4),
                "tflops": round(flops / t / 1e12, 2), "mfma_frac": round(flops / t / 1e12 / mfma_peak, 4),
                "tokens_per_s": round(x0.batch / t, 1), "tokens_frac": round(t_roof / t, 4)}

    obj = {
        "workload": name, "description": wl.description, "batch": x0.batch, "heads": x0.heads,
        "seq_len": x0.max_seq_len, "cache_dtype": wl.dtype, "layout": wl.layout,
        "split": ({"kind": "plan", "items": plan.num_items,
                   "longest_item_tiles": int(plan.items_host[:, 2].max()),
                   "uniform_rule_splits": P} if planned else {"kind": "uniform", "splits": P}),
        "input_replicas": R, "cache_bytes": cache_bytes, "core_flops": flops,
        "roof": {"bound": bound, "time_us": round(t_roof * 1e6, 3),
                 "note": ("max(cache bytes / 8 TB/s, core FLOPs / 5.0 PFLOP/s fp8 MFMA); core FLOPs count each "
                          "product once (the kernel's split query runs the score products twice)" if fp8_mfma else
                          "max(cache bytes / 8 TB/s, core FLOPs / 2.5 PFLOP/s bf16 MFMA)" +
                          ("; E4M3 codes enter bf16 MFMAs exactly" if fp8 else ""))},
        "headline_step_us": round(t_step * 1e6, 3),
        "headline_step_us_host_clock": round(t_host * 1e6, 3),
        "step_us": _stats(per_step),
        "step_eager_us": round(t_eager * 1e6, 3),
        "decode_us": _stats(dec),
        "merge_expand_us": _stats(tail),
        "step": rates(t_med),
        "decode": rates(t_dec),
    }
    if sclk is not None:
        obj["sclk"] = sclk
    if x0.max_seq_len <= FUSED_MAX_CONTEXT:
        obj["fused_step"] = bench_fused_step(x0, d, dev, steps)
    out = dict(obj=obj, t_step=t_step, t_host=t_host, t_dec=t_dec, x0=x0, d=d, P=P, R=R, cache_bytes=cache_bytes, flops=flops,
               t_eager=t_eager, steps=steps_objs)
    return out


def cpu_baselines(x):
    """The oracle on all host cores, then on one core (BLAS threads limited)."""
    res = {"all": cpu_baseline(x)}
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            one = cpu_baseline(x, target_s=10.0)
        one["cores"] = 1
        res["one"] = one
    except Exception as e:  # pragma: no cover - informational only
        res["one"] = {"error": str(e)}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="v3_b32_s4096")
    ap.add_argument("--splits", type=int, default=0, help="0 = library recommendation (plan for variable lengths)")
    ap.add_argument("--replicas", type=int, default=0, help="input replicas (0 = enough for > 512 MB)")
    ap.add_argument("--only", action="store_true", help="measure the headline workload only (no other configs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-append", action="store_true", help="skip the cache-append measurement")
    ap.add_argument("--no-naive", action="store_true", help="skip the naive-decode baseline and context sweep")
    ap.add_argument("--no-prefill", action="store_true", help="skip the chunked-prefill measurement")
    ap.add_argument("--no-fp8", action="store_true", help="skip the E4M3 long-context workload")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 1 GiB elementwise copy (y = -x) 5 times: the reference kernel "
                         "for the HBM byte counters")
    ap.add_argument("--summarize-trace", metavar="TRACE_CSV",
                    help="print this library's kernel durations from a rocprofv3 --kernel-trace CSV, grouped by "
                         "kernel and launch grid, and exit")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the HBM byte counter file from two rocprofv3 --pmc runs of "
                         "'bench.py --copy-calibration' (FETCH_SIZE, then WRITE_SIZE) and exit")
    args = ap.parse_args()

    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_counters:
        summarize_counters(args, *args.summarize_counters)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}): this build has no "
              "multi-GPU path; batch sharding across GPUs needs no exchange and is described in DESIGN.md.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from mla_absorbed_latent_absorb_amd import binding

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    binding.load()

    if args.copy_calibration:
        src = torch.empty(COPY_ELEMS, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.neg(src, out=dst)  # one elementwise kernel: reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src, dst

    head = measure_config(args.workload, dev, args.steps, args.warmup, splits=args.splits, replicas=args.replicas,
                          sample_sclk=True)
    ho, x0, d = head["obj"], head["x0"], head["d"]
    t_step, t_dec = head["t_step"], head["t_dec"]
    cache_bytes = head["cache_bytes"]
    flops_core = head["flops"]
    flops_step = flops_core + proj_flops(x0.batch, x0.heads)
    gbs_step = cache_bytes / t_step / 1e9
    gbs_dec = cache_bytes / t_dec / 1e9
    wl = x0.workload
    traffic = traffic_from_counters(wl.name)

    result = {
        "metric": METRIC if wl.name == "v3_b32_s4096" else METRIC_OTHER.format(wl.description),
        "value": round(gbs_step, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 5),
        "ms_per_step_host_clock": round(head["t_host"] * 1e3, 5),
        "ms_per_step_eager": round(head["t_eager"] * 1e3, 5),
        "step_timing": "the K steps as one HIP graph replay between two synchronisations (three launches per "
                       "step: absorb_q, decode_latent, combine_expand_v or expand_v), GPU time from HIP events "
                       "at the replay's ends, a spin kernel queued before the first event so that the host's "
                       "submission of the graph's launches is not timed (ms_per_step_host_clock: the host clock "
                       "around another replay between two synchronisations, which adds one graph launch and the "
                       "GPU's wait for it); step_us: 7 more replays timed the same way",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else
                 "fp8_e4m3 cache / " + ("fp8 MFMA" if x0.heads == 128 else "bf16 MFMA"),
        "data": "synthetic (seeded N(0,1) cache and queries, N(0,1/512) weights; no checkpoint)",
        "config": {"workload": wl.name, "batch": x0.batch, "heads": x0.heads, "seq_len": x0.max_seq_len,
                   "kv_lora_rank": 512, "qk_rope_head_dim": 64, "layout": wl.layout, "cache_dtype": wl.dtype,
                   "split": ho["split"], "input_replicas": head["R"], "cache_bytes_per_step": cache_bytes},
        "roofline": {"bound": "hbm", "achieved": round(gbs_dec, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs_dec / HBM_PEAK_GBS, 4), "traffic": traffic},
        "kernel": "mla_decode_latent",
        "decode_us": ho["decode_us"]["mean"],
        "decode_us_stats": ho["decode_us"],
        "merge_expand_us": ho["merge_expand_us"]["mean"],
        "step_us_stats": ho["step_us"],
        "tflops_step": round(flops_step / t_step / 1e12, 3),
        "tflops_decode": round(flops_core / t_dec / 1e12, 3),
        "decode_mfma_frac": round(flops_core / t_dec / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
        "tokens_per_s": round(x0.batch / t_step, 1),
        "sclk": ho.get("sclk"),
        "device": props.name,
        "cus": props.multi_processor_count,
    }
    if "fused_step" in ho:
        result["fused_step"] = ho["fused_step"]
    configs = {wl.name: ho}
    if not args.only:
        for name in CONFIGS:
            if name == wl.name or (args.no_fp8 and name == "v3_b64_s32768_fp8"):
                continue
            steps_c = max(4, min(args.steps, 40)) if name in ("v3_b128_paged", "v3_b64_s32768_fp8") else args.steps
            c = measure_config(name, dev, steps_c, max(2, min(args.warmup, 5)))
            configs[name] = c["obj"]
            del c
            torch.cuda.empty_cache()
    result["configs"] = configs
    if not args.no_prefill:
        result["prefill"] = bench_prefill(dev)
    if not args.no_naive:
        result["naive"] = bench_naive(x0, d, dev, t_step)
        result["crossover_v2lite_b1"] = bench_crossover(dev)
    if not args.no_append:
        result["append"] = bench_append(x0, d, dev, args.steps)
    if not args.no_cpu_baseline:
        cb = cpu_baselines(x0)
        result["cpu_baseline"] = cb["all"]
        result["cpu_baseline_1core"] = cb["one"]
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
