"""Throughput of the causal prefill-attention kernel on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one ``attn_prefill`` call (one layer's causal prefill attention)
over the workload's seeded synthetic batch, inputs resident in HBM.  W
untimed warm-up steps, then exactly K timed steps bracketed by
``torch.cuda.synchronize()``.  Prints ONE JSON line:

* ``value``: causal TFLOP/s of the whole step (F / wall time per step),
  F = 4 * head_dim * n_q_heads * (visible query-key pairs);
* ``roofline``: the kernel's average launch duration from two HIP events
  on the launch stream around the K timed launches (their span / K: the
  launches run back to back), the algorithmic TFLOP/s it implies against
  the bf16 dense MFMA peak, and the HBM traffic measured by rocprofv3
  counters (from ``profiles/``, null when the kernel source changed since
  the counters were taken).  Per-launch durations (median, minimum, each
  launch in order) come from a second pass of K launches right after, each
  between its own pair of events: an event between launches adds a few µs
  of idle time per step, so that pass is not the timed one;
* ``cpu_baseline``: the FP64 CPU oracle timed on a bounded sample of the
  same workload (a subset of the query heads, all tokens), scaled to the
  same unit, with the number of threads it used.

After the timed region, from the same process and without touching
``value``: the other problem shapes of the metric (128 tokens, 2048 tokens,
the 4096-token window, the packed GQA batch) each timed on their own
(``other_configs``), a sustained run of the main workload for a few seconds
with the graphics clock read from sysfs while it runs (``sustained``), the
ROCm and HIP versions (``env``), and the oracle on one core for the two
smallest shapes (``cpu_baseline.single_core``).

``--mode copy`` instead runs a plain device-to-device copy of known size;
its rocprofv3 FETCH_SIZE / WRITE_SIZE readings calibrate the counters.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

KERNEL_SOURCES = [
    os.path.join(ROOT, "causal_prefill_attention_amd", "csrc", "prefill_fwd.hip"),
    os.path.join(ROOT, "causal_prefill_attention_amd", "csrc", "prefill_params.h"),
    os.path.join(ROOT, "causal_prefill_attention_amd", "csrc", "device_common.h"),
    os.path.join(ROOT, "causal_prefill_attention_amd", "csrc", "prefill_work.h"),
]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def _code_of(text: str) -> str:
    """Source text without // comments, trailing blanks and empty lines, so
    that an edit of the comments does not count as a change of the kernel."""
    out = []
    for line in text.splitlines():
        code = line.split("//", 1)[0].rstrip()
        if code:
            out.append(code)
    return "\n".join(out)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, encoding="utf-8") as f:
            h.update(_code_of(f.read()).encode())
    return h.hexdigest()


def load_traffic(workload: str):
    """HBM bytes per launch from committed rocprofv3 counters, if current."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(workload)
    if not entry or entry.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return entry.get("bytes_per_launch")


def host_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(w, inp, n_heads_sample: int):
    """Times the oracle on the first ``n_heads_sample`` query heads."""
    import oracle
    from causal_prefill_attention_amd import measure

    hs = max(1, min(n_heads_sample, w.n_q_heads))
    n_kv = 1
    if w.n_kv_heads > 1:
        # whole GQA groups, so that every sampled head keeps its kv head
        group = w.n_q_heads // w.n_kv_heads
        n_kv = (hs + group - 1) // group
        hs = n_kv * group
    q = inp["q"][:, :hs]
    k = inp["k"][:, :n_kv]
    v = inp["v"][:, :n_kv]
    threads = host_threads()
    kv_lengths = inp.get("kv_lengths")
    t0 = time.perf_counter()
    if kv_lengths is None:
        oracle.attention_varlen(q, k, v, inp["cu_seqlens"], hs, n_kv, w.attn_scale,
                                w.window, workers=threads)
    else:
        oracle.attention_chunked(q, k, v, inp["cu_seqlens"], inp["cu_seqlens_k"], hs,
                                 n_kv, w.attn_scale, w.window, workers=threads)
    dt = time.perf_counter() - t0
    flops = measure.causal_flops(inp["lengths"], hs, w.head_dim, w.window, kv_lengths,
                                 w.head_dim_v)
    jobs = hs * sum(1 for n in inp["lengths"] if n > 0)
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": min(threads, jobs),
        "kind": "oracle",
        "sample": (f"{w.name}: {hs} of {w.n_q_heads} query heads, all "
                   f"{sum(inp['lengths'])} tokens, numpy float64, {dt:.2f} s wall"),
        "seconds": dt,
    }


#: The other problem shapes of the metric, reported beside the main line.
OTHER_CONFIGS = ["causal_128tok_4q1kv", "mla_2048tok_32q1kv", "window1024_4096tok_32q1kv",
                 "varlen16_gqa32q8kv_fp32q_fp16kv"]


def rocm_version():
    try:
        with open("/opt/rocm/.info/version") as f:
            return f.read().strip()
    except OSError:
        return None


def make_step(w, binding, dev, stream):
    """Device inputs of workload ``w`` and a closure that runs one call."""
    from causal_prefill_attention_amd import workloads

    inp = workloads.make_inputs(w)
    q = inp["q"].to(dev)
    k = inp["k"].to(dev)
    v = inp["v"].to(dev)
    cu = inp["cu_seqlens"].to(dev)
    kv_lengths = inp.get("kv_lengths")
    cuk = inp["cu_seqlens_k"].to(dev) if kv_lengths is not None else None
    dv = w.head_dim_v or w.head_dim
    if w.head_dim_v is not None:
        v = k[:, :, :w.head_dim_v]  # the values are part of the cache rows
    import torch
    out = torch.empty(q.shape[0], w.n_q_heads, dv, dtype=torch.bfloat16, device=dev)
    lengths = inp["lengths"]
    # partial results of key ranges split across workgroups (decode batches
    # and prefill calls that would not fill the chip; allocated once, outside
    # the timed region)
    workspace = None
    if w.decode:
        workspace = binding.decode_workspace(q.shape[0], w.n_q_heads, w.n_kv_heads, w.head_dim,
                                             device=dev)
    elif binding.prefill_workspace_size(q.shape[0], k.shape[0], len(lengths), w.n_q_heads,
                                        w.n_kv_heads, w.head_dim, dv, w.window) > 0:
        workspace = binding.prefill_workspace(q.shape[0], k.shape[0], len(lengths), w.n_q_heads,
                                              w.n_kv_heads, w.head_dim, dv, w.window,
                                              device=dev)

    def step():
        if workspace is not None and not w.decode:
            binding.attn_prefill_ex(q, k, v, out, cu, w.n_q_heads, w.n_kv_heads, w.head_dim, dv,
                                    w.attn_scale, w.window, cu_seqlens_k=cuk, stream=stream,
                                    workspace=workspace)
        elif w.head_dim_v is not None:
            binding.attn_prefill_ex(q, k, v, out, cu, w.n_q_heads, w.n_kv_heads, w.head_dim,
                                    w.head_dim_v, w.attn_scale, w.window,
                                    cu_seqlens_k=cuk, stream=stream)
        elif w.decode:
            binding.attn_decode(q, k, v, out, cuk, w.n_q_heads, w.n_kv_heads, w.head_dim,
                                w.attn_scale, w.window, stream=stream, workspace=workspace)
        elif cuk is None:
            binding.attn_prefill(q, k, v, out, cu, w.n_q_heads, w.n_kv_heads,
                                 w.head_dim, w.attn_scale, w.window, stream=stream)
        else:
            binding.attn_prefill_chunked(q, k, v, out, cu, cuk, w.n_q_heads,
                                         w.n_kv_heads, w.head_dim, w.attn_scale,
                                         w.window, stream=stream)

    return inp, workspace, step


def time_launches(step, stream, n, warmup):
    """Per-launch durations (ms) from HIP events on the launch stream."""
    import torch

    for _ in range(warmup):
        step()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    torch.cuda.synchronize()
    for i in range(n):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    return [s.elapsed_time(e) for s, e in zip(starts, ends)]


def other_configs(binding, dev, stream):
    """Kernel time of the metric's other problem shapes, each on its own."""
    from causal_prefill_attention_amd import measure, workloads

    res = {}
    for name in OTHER_CONFIGS:
        w = workloads.WORKLOADS[name]
        inp, _, step = make_step(w, binding, dev, stream)
        n = 1000 if sum(inp["lengths"]) <= 128 else 50
        durs = time_launches(step, stream, n, warmup=10)
        med = statistics.median(durs)
        flops = measure.causal_flops(inp["lengths"], w.n_q_heads, w.head_dim, w.window,
                                     inp.get("kv_lengths"), w.head_dim_v)
        tf = flops / (med * 1e-3) / 1e12
        res[name] = {"kernel_median_us": round(med * 1e3, 2),
                     "kernel_avg_us": round(sum(durs) / len(durs) * 1e3, 2),
                     "kernel_min_us": round(min(durs) * 1e3, 2),
                     "launches": n, "causal_flops": flops,
                     "tflops_at_median": round(tf, 2),
                     "pct_of_peak": round(100.0 * tf / measure.PEAK_BF16_TFLOPS, 2)}
    return res


def sclk_path(dev):
    """The device's ``pp_dpm_sclk`` sysfs file (graphics clock levels, the
    current one starred), found through its PCI address."""
    import torch

    props = torch.cuda.get_device_properties(dev)
    bus = getattr(props, "pci_bus_id", None)
    if bus is None:
        return None
    dom = getattr(props, "pci_domain_id", 0) or 0
    devid = getattr(props, "pci_device_id", 0) or 0
    path = f"/sys/bus/pci/devices/{dom:04x}:{bus:02x}:{devid:02x}.0/pp_dpm_sclk"
    return path if os.path.exists(path) else None


def read_sclk_mhz(path):
    """Current graphics clock (MHz) from the starred ``pp_dpm_sclk`` line."""
    try:
        with open(path) as f:
            for line in f:
                if "*" in line:
                    num = "".join(ch for ch in line.split(":", 1)[-1] if ch.isdigit())
                    return int(num) if num else None
    except OSError:
        return None
    return None


def sustained_run(step, stream, seconds, dev):
    """Runs ``step`` back to back for about ``seconds`` while a thread reads
    the graphics clock from sysfs every 10 ms.  Returns the average launch
    time over the last third of the run and the clock readings."""
    import threading

    import torch

    path = sclk_path(dev)
    samples = []
    stop = threading.Event()

    def sampler():
        while not stop.is_set():
            mhz = read_sclk_mhz(path) if path else None
            if mhz is not None:
                samples.append((time.perf_counter(), mhz))
            stop.wait(0.01)

    batch = 50
    marks = []  # (start event, end event) per batch
    th = threading.Thread(target=sampler, daemon=True)
    t0 = time.perf_counter()
    th.start()
    while time.perf_counter() - t0 < seconds:
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(batch):
            step()
        b.record(stream)
        marks.append((a, b))
        if len(marks) >= 2:
            marks[-2][1].synchronize()  # keep at most two batches queued
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    stop.set()
    th.join()
    per_batch = [x.elapsed_time(y) / batch for x, y in marks]
    tail = per_batch[-max(1, len(per_batch) // 3):]
    load = [mhz for t, mhz in samples if t0 + 0.1 <= t <= t_end]
    last = [mhz for t, mhz in samples if t_end - (t_end - t0) / 3 <= t <= t_end]

    def mean(x):
        return round(sum(x) / len(x), 1) if x else None

    return {"seconds": round(t_end - t0, 2), "launches": batch * len(marks),
            "last_third_avg_us": round(1e3 * sum(tail) / len(tail), 2),
            "first_batch_avg_us": round(1e3 * per_batch[0], 2),
            "gpu_clock": {"source": path, "samples": len(load),
                          "mhz_mean_under_load": mean(load),
                          "mhz_mean_last_third": mean(last),
                          "mhz_min": min(load) if load else None,
                          "mhz_max": max(load) if load else None}}


def cpu_single_core(names):
    """The oracle on one thread for the smallest problem shapes (seconds)."""
    import oracle
    from causal_prefill_attention_amd import workloads

    res = {}
    for name in names:
        w = workloads.WORKLOADS[name]
        inp = workloads.make_inputs(w)
        t0 = time.perf_counter()
        oracle.attention_varlen(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"],
                                w.n_q_heads, w.n_kv_heads, w.attn_scale, w.window,
                                workers=1)
        res[name] = round(time.perf_counter() - t0, 3)
    return res


def run_copy(args):
    import torch

    n = args.copy_mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    print(json.dumps({"mode": "copy", "bytes_read": n, "bytes_written": n,
                      "ms_per_copy": dt * 1e3, "GB/s": 2 * n / dt / 1e9}))


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--cpu-heads", type=int, default=0,
                    help="query heads of the workload the CPU oracle times "
                         "(default: all of them)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the other shapes, the sustained run and the "
                         "single-core oracle times")
    ap.add_argument("--sustain-s", type=float, default=2.0)
    ap.add_argument("--mode", choices=["attn", "copy"], default="attn")
    ap.add_argument("--copy-mib", type=int, default=1024)
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(prefill attention would shard by query head or by sequence "
              "with no exchange); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.mode == "copy":
        run_copy(args)
        return

    from causal_prefill_attention_amd import binding, measure, workloads

    name = args.workload or workloads.HEADLINE
    w = workloads.WORKLOADS[name]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    inp, workspace, step = make_step(w, binding, dev, stream)
    lengths = inp["lengths"]
    kv_lengths = inp.get("kv_lengths")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K back-to-back steps between two events on the launch stream
    first = torch.cuda.Event(enable_timing=True)
    last = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    first.record(stream)
    for _ in range(args.steps):
        step()
    last.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg_ms = first.elapsed_time(last) / args.steps
    # per-launch durations: K more launches, each between its own events
    in_order = time_launches(step, stream, args.steps, warmup=0)  # ms
    durs = sorted(in_order)

    flops = measure.causal_flops(lengths, w.n_q_heads, w.head_dim, w.window, kv_lengths,
                                 w.head_dim_v)
    ms_per_step = wall * 1e3 / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (avg_ms * 1e-3) / 1e12
    peak = measure.PEAK_BF16_TFLOPS
    traffic = load_traffic(name)
    alg_bytes = measure.algorithmic_bytes(lengths, w.n_q_heads, w.n_kv_heads, w.head_dim,
                                          w.q_dtype, w.kv_dtype, kv_lengths, w.head_dim_v,
                                          v_in_k=w.head_dim_v is not None)
    if w.decode:  # one query per sequence: the step streams K/V from HBM
        roof = {"bound": "hbm", "achieved": round(alg_bytes / (avg_ms * 1e-3) / 1e9, 1),
                "peak": measure.PEAK_HBM_GBS, "unit": "GB/s"}
        roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    else:
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak, 1),
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4)}

    line = {
        "metric": "causal prefill attention TFLOP/s and % of bf16 MFMA peak "
                  "(hd=128, MQA)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "pct_of_peak": round(100.0 * value / peak, 2),
        "config": {
            "workload": name,
            "seq_lens": lengths if len(lengths) <= 16 else f"{len(lengths)} seqs",
            "tokens": int(sum(lengths)),
            **({"kv_history": list(w.history)} if w.history else {}),
            **({"key_split_workspace_bytes": int(workspace.numel())}
               if workspace is not None else {}),
            "n_q_heads": w.n_q_heads,
            "n_kv_heads": w.n_kv_heads,
            "head_dim": w.head_dim,
            "sliding_window": w.window,
            "q_dtype": w.q_dtype,
            "kv_dtype": w.kv_dtype,
            "k_outlier_frac": w.k_outlier_frac,
            "scale": w.attn_scale,
            "causal_flops": flops,
        },
        "roofline": {
            **roof,
            "traffic": traffic,
            "kernel_avg_us": round(avg_ms * 1e3, 2),
            "per_launch_pass": {
                "note": "K further launches right after the timed region, each between "
                        "its own events",
                "kernel_avg_us": round(sum(durs) / len(durs) * 1e3, 2),
                "kernel_median_us": round(statistics.median(durs) * 1e3, 2),
                "kernel_min_us": round(durs[0] * 1e3, 2),
                "kernel_us_in_order": [round(x * 1e3, 1) for x in in_order]},
            "algorithmic_bytes": alg_bytes,
        },
        "cpu_baseline": None,
    }
    line["env"] = {"rocm": rocm_version(), "hip_runtime": torch.version.hip,
                   "torch": torch.__version__,
                   "device": torch.cuda.get_device_name(dev),
                   "compute_units": torch.cuda.get_device_properties(dev).multi_processor_count}
    if not args.no_extras:
        line["sustained"] = sustained_run(step, stream, args.sustain_s, dev)
        line["other_configs"] = other_configs(binding, dev, stream)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_heads or w.n_q_heads)
        if not args.no_extras:
            line["cpu_baseline"]["single_core"] = {
                "seconds": cpu_single_core(OTHER_CONFIGS[:2]), "cores": 1, "kind": "oracle"}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
