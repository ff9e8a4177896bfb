"""Benchmark of the paged-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--headline-only]

Headline (the JSON line's ``value``): ``pa_decode`` on the batched GQA
decode workload -- 64 sequences, 32 query / 8 KV heads, d = 128, context
lengths uniform in [128, 4096], block size 16, fp16 -- as achieved HBM GB/s
of algorithmic bytes (every attended K/V row once per KV head, q, out, the
table entries used) per step.  One step = one ``pa_decode`` call, which is
one kernel (split units are merged by the wavefront that finishes their last
partition).  Inputs are resident in HBM; steps rotate over three copies of
the pools so that the 256 MB Infinity Cache cannot hold the 0.55 GB of K/V
between steps.

The same line carries:
* ``roofline``: the partition kernel's algorithmic bytes / its average
  duration, from HIP events the library records around each launch on the
  launch stream, over a second pass of the same K steps; ``traffic`` comes
  from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary when that
  summary was taken on the current kernel source, else null.
* ``step_us`` / ``kernel_us``: median, p10 and p90 of the per-step times
  (HIP events between steps, a pass of their own) and of the per-launch
  kernel times.
* ``cpu_baseline``: the fp64 CPU oracle on the same workload, with the
  host's CPU count, affinity set and BLAS threads.
* ``extra``: the long-context decode (4 x 100,000 keys, bf16), the GQA and
  long-context decodes again with pools head-major within blocks (the other
  pool layout the library reads), the prefix-shared decode sweep
  (B = 16/32/64/128), the causal prefill (8 prompts of 512..4096 tokens,
  bf16; TFLOP/s against the bf16 MFMA peak, and against the peak at the
  shader clock measured while it runs), the same prompts with group sizes
  1, 2 and 8 (kernel time only) and, as context for the HBM
  fractions, the rate of a plain 1 GiB device copy.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16/fp16 MFMA
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the extra workloads and the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (torch) 10 times, to scale "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--write-traffic", nargs=6, default=None,
                    metavar=("KERNEL", "WORKLOAD", "FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV",
                             "COPY_WRITE_CSV"),
                    help="turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE counter files of a "
                         "workload run and of a --copy-calibration run into "
                         "profiles/<KERNEL>_<WORKLOAD>_traffic.json (no GPU needed)")
    ap.add_argument("--rdreq-check", nargs=4, default=None,
                    metavar=("KERNEL", "WORKLOAD", "RDREQ_CSV", "COPY_RDREQ_CSV"),
                    help="add to profiles/<KERNEL>_<WORKLOAD>_traffic.json the read bytes "
                         "given by the TCC_EA0_RDREQ_{32B,64B,128B} request counts of a "
                         "workload run and of a --copy-calibration run: an independent "
                         "check of the FETCH_SIZE scale factor (no GPU needed)")
    ap.add_argument("--only", default="",
                    help="comma list of workloads to run (for profiling): "
                         "gqa,long,gqa-hm,long-hm,share,prefix,prefill,prefill-g,copy; "
                         "prefill-g: the prefill prompts with 32, 16 and 4 KV heads; prefix16 runs "
                         "the prefix-shared workload at B = 16 only; -hm: pools head-major "
                         "within blocks; share: one eighth of the long context and the "
                         "merge of eight partial states")
    return ap.parse_args()


# Headers every kernel source includes; a change in any of them can change
# the compiled kernels, so they enter every kernel's source hash.
SHARED_HEADERS = ("device_common.h", "kernels.h", "launch.h", "plan.h")
# The device code each kernel file compiles.
KERNEL_FILES = {"decode.hip": ("decode.hip", "decode_kernel.h"),
                "prefill.hip": ("prefill.hip", "prefill_kernel.h"),
                "shared_prefix.hip": ("shared_prefix.hip", "decode_kernel.h", "prefill_kernel.h")}


def source_hash(kernel_file):
    """Hash of the code a kernel file compiles, comments and blank space
    left out (a comment edit does not change the kernel)."""
    import re
    h = hashlib.sha256()
    for n in (*KERNEL_FILES[kernel_file], *SHARED_HEADERS):
        with open(os.path.join(ROOT, "paged_kv_cache_decode_amd", "csrc", n)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def load_traffic(kernel, workload, src_hash, bytes_per_launch):
    """HBM traffic measured by rocprofv3 counters, if taken on this source."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != src_hash:
        return None
    return {"fetch_bytes": rec["fetch_bytes"], "write_bytes": rec["write_bytes"],
            "ratio_to_algorithmic": round((rec["fetch_bytes"] + rec["write_bytes"]) /
                                          bytes_per_launch, 4),
            "scale_factor": rec.get("scale_factor"),
            "request_count_cross_check": (rec["rdreq_cross_check"]["over_scaled_fetch_bytes"]
                                          if "rdreq_cross_check" in rec else None),
            "source": os.path.basename(path)}


# Kernel record name -> (substring of its demangled symbol, source).  The
# last three tell apart the kernels of the prefix-shared workload: plain
# decode, and the shared-prefix call's two kernels (prefix and suffix steps
# in one kernel, then the join).
KERNEL_SOURCES = {"decode_partitions": ("decode_partitions_kernel", "decode.hip"),
                  "prefill": ("prefill_kernel", "prefill.hip"),
                  "decode_partitions_plain":
                      ("decode_partitions_kernel<pa::TBF16, 128, 4, false>", "decode.hip"),
                  "shared_prefix": ("shared_prefix_kernel", "shared_prefix.hip"),
                  "prefix_join": ("prefix_join_kernel", "decode.hip")}
COPY_CALIBRATION_BYTES = 1 << 30


def counter_mean(path, name_part, counter):
    """Mean per-dispatch value of `counter` over dispatches whose kernel
    symbol contains `name_part`, from a rocprofv3 counter_collection.csv
    (FETCH_SIZE / WRITE_SIZE are in KiB, request counters are counts)."""
    import csv
    vals = []
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] == counter and name_part in row["Kernel_Name"]:
                vals.append(float(row["Counter_Value"]))
    if not vals:
        raise SystemExit(f"{path}: no {counter} rows for kernels matching {name_part!r}")
    return sum(vals) / len(vals), len(vals)


def write_traffic(kernel, workload, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv):
    """FETCH_SIZE / WRITE_SIZE per launch, each scaled by what the same
    counter reports for a plain device copy of known size."""
    part, src_file = KERNEL_SOURCES[kernel]
    cf, _ = counter_mean(copy_fetch_csv, "copyBuffer", "FETCH_SIZE")
    cw, _ = counter_mean(copy_write_csv, "copyBuffer", "WRITE_SIZE")
    fetch_scale = COPY_CALIBRATION_BYTES / (cf * 1024.0)
    write_scale = COPY_CALIBRATION_BYTES / (cw * 1024.0)
    fk, nf = counter_mean(fetch_csv, part, "FETCH_SIZE")
    wk, nw = counter_mean(write_csv, part, "WRITE_SIZE")
    rec = {"kernel": kernel, "workload": workload, "source_hash": source_hash(src_file),
           "fetch_bytes": round(fk * 1024.0 * fetch_scale),
           "write_bytes": round(wk * 1024.0 * write_scale),
           "fetch_kib_raw": round(fk, 1), "write_kib_raw": round(wk, 1),
           "dispatches": [nf, nw],
           "scale_factor": {"fetch": round(fetch_scale, 4), "write": round(write_scale, 4)},
           "calibration": "1 GiB device-to-device copy (bench.py --copy-calibration)"}
    os.makedirs(PROFILES, exist_ok=True)
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def rdreq_bytes(path, name_part):
    """Mean per-dispatch read bytes from the memory-request counts of the
    dispatches whose kernel symbol contains `name_part`: 32, 64 and 128 B
    requests counted separately, plus their total as a consistency check."""
    sizes = {"TCC_EA0_RDREQ_32B": 32, "TCC_EA0_RDREQ_64B": 64, "TCC_EA0_RDREQ_128B": 128}
    got = {}
    for c in (*sizes, "TCC_EA0_RDREQ"):
        got[c], _ = counter_mean(path, name_part, c)
    nbytes = sum(got[c] * b for c, b in sizes.items())
    return nbytes, got


def rdreq_check(kernel, workload, rdreq_csv, copy_rdreq_csv):
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.json")
    with open(path) as f:
        rec = json.load(f)
    part, _ = KERNEL_SOURCES[kernel]
    kb, kc = rdreq_bytes(rdreq_csv, part)
    cb, cc = rdreq_bytes(copy_rdreq_csv, "copyBuffer")
    rec["rdreq_cross_check"] = {
        "read_bytes_from_request_counts": round(kb),
        "over_scaled_fetch_bytes": round(kb / rec["fetch_bytes"], 4),
        "over_raw_fetch_size": round(kb / (rec["fetch_kib_raw"] * 1024.0), 4),
        "copy_read_bytes_over_1GiB": round(cb / COPY_CALIBRATION_BYTES, 4),
        "request_counts": {k: round(v) for k, v in kc.items()},
        "copy_request_counts": {k: round(v) for k, v in cc.items()}}
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec["rdreq_cross_check"]))


def prefix_dram_measured(unique):
    """Measured DRAM bytes per call on the prefix-shared workload at B = 16
    (rocprofv3 counter records, if taken on the current sources), against
    the unique bytes the method must move."""
    wl = "prefix-shared-bf16-decode-B16"
    dec, sp = source_hash("decode.hip"), source_hash("shared_prefix.hip")
    plain = load_traffic("decode_partitions_plain", wl, dec, unique)
    comb = load_traffic("shared_prefix", wl, sp, unique)
    join = load_traffic("prefix_join", wl, dec, unique)
    out = {"plain_decode": None, "shared_prefix_call": None}
    if plain:
        out["plain_decode"] = {"fetch_bytes": plain["fetch_bytes"],
                               "write_bytes": plain["write_bytes"],
                               "over_unique": plain["ratio_to_algorithmic"]}
    if comb and join:
        tot = (comb["fetch_bytes"] + comb["write_bytes"] + join["fetch_bytes"] +
               join["write_bytes"])
        out["shared_prefix_call"] = {
            "prefix_and_suffix_kernel": {"fetch_bytes": comb["fetch_bytes"],
                                         "write_bytes": comb["write_bytes"]},
            "join_kernel": {"fetch_bytes": join["fetch_bytes"],
                            "write_bytes": join["write_bytes"]},
            "over_unique": round(tot / unique, 4)}
    return out


class Timer:
    """Wall clock over K steps, bracketed by device synchronisation."""

    def __init__(self, torch):
        self.torch = torch

    def run(self, fn, steps):
        self.torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            fn(i)
        self.torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps

    def step_times_ms(self, fn, steps):
        """Per-step durations from HIP events recorded between the steps on
        the stream the library launches on (a pass of its own, so the
        event packets stay out of the wall-clock pass)."""
        torch = self.torch
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        for i in range(steps):
            ev[i].record()
            fn(i)
        ev[steps].record()
        torch.cuda.synchronize()
        return [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]


def spread_us(ms):
    """Median, p10 and p90 of a list of millisecond timings, in us."""
    import numpy as np
    a = np.asarray(ms, dtype=np.float64) * 1e3
    if a.size == 0:
        return None
    p10, p50, p90 = np.percentile(a, [10, 50, 90])
    return {"median": round(float(p50), 2), "p10": round(float(p10), 2),
            "p90": round(float(p90), 2), "n": int(a.size)}


def shader_mhz_during(torch, binding, fn, steps, est_step_sec):
    """Shader clock (MHz) while `steps` steps run: pa_clock_probe's single
    wave on a side stream (default priority) counts shader-clock ticks over
    about 80 % of the steps' expected span of 100 MHz reference ticks.  A
    pass of its own, so the probe's wave slot stays out of the timed
    passes."""
    side = torch.cuda.Stream()
    out = torch.zeros(2, dtype=torch.int64, device="cuda")
    ticks = int(min(1e8, max(1e4, 0.8 * est_step_sec * steps * 1e8)))
    torch.cuda.synchronize()
    binding.clock_probe(out, ticks, stream=side)
    for i in range(steps):
        fn(i)
    torch.cuda.synchronize()
    c, r = (int(x) for x in out.tolist())
    mhz = 100.0 * c / r if r > 0 else float("nan")
    return mhz if 300.0 < mhz < 4000.0 else None


def host_info():
    """What the CPU baseline could use on this host."""
    import numpy  # noqa: F401  (loads the BLAS threadpoolctl reports)
    info = {"os_cpu_count": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS")}
    try:
        from threadpoolctl import threadpool_info
        info["blas"] = [{"library": p.get("internal_api"), "threads": p.get("num_threads")}
                        for p in threadpool_info() if p.get("user_api") == "blas"]
    except Exception as e:  # threadpoolctl missing or failing: say so
        info["blas"] = f"unavailable: {e}"
    return info


def blas_threads(info):
    blas = info.get("blas")
    if isinstance(blas, list) and blas:
        return max(int(b["threads"] or 1) for b in blas)
    return 1


def workload_meta(case):
    return {"seed": case.meta["seed"], "NB": int(case.meta["NB"]), "MB": int(case.meta["MB"])}


def kernel_avg_ms(binding, name):
    ms, n = binding.profiler_read(name)
    return (ms / n if n else float("nan")), n


def kernel_spread(binding, name):
    return spread_us(binding.profiler_samples(name))


def warm_up(torch, fn, steps, min_seconds):
    """Untimed calls: `steps` of them, then more (in groups of 10) until at
    least `min_seconds` have passed, so that the GPU's clocks have settled
    when a measurement starts after idle time (uploads, other workloads)."""
    t0 = time.perf_counter()
    for i in range(steps):
        fn(i)
    torch.cuda.synchronize()
    i = steps
    while time.perf_counter() - t0 < min_seconds:
        for _ in range(10):
            fn(i)
            i += 1
        torch.cuda.synchronize()


# Time-based warm-up of the `extra` entries (the headline keeps exactly the
# --warmup steps of the command line).
EXTRA_WARM_S = 0.1


def bench_decode_case(torch, binding, case, steps, warmup, copies, out_dtype,
                      prefix_len=None, head_major=False, warm_seconds=0.0):
    """Time pa_decode (or pa_decode_shared_prefix with ``prefix_len``) on a
    case, rotating over `copies` device copies of the pools (token-major, or
    head-major within blocks).  Returns a dict of timings."""
    devs = [binding.upload_case(case, head_major) for _ in range(copies)]
    out = torch.empty(case.q.shape, dtype=out_dtype, device="cuda")
    calls = [binding.PreparedDecode(d["q"], d["k_pool"], d["v_pool"], d["block_table"],
                                    d["context_lens"], case.scale, out, prefix_len)
             for d in devs]
    plan = binding.decode_plan(devs[0]["q"], devs[0]["k_pool"], devs[0]["v_pool"],
                               devs[0]["block_table"], devs[0]["context_lens"], out)
    step = lambda i: calls[i % copies]()  # noqa: E731
    timer = Timer(torch)
    warm_up(torch, step, warmup, warm_seconds)
    sec = timer.run(step, steps)
    # Second pass with the library's per-kernel event timer on.
    binding.profiler_reset()
    binding.profiler_enable(True)
    timer.run(step, steps)
    binding.profiler_enable(False)
    part_ms, part_n = kernel_avg_ms(binding, "decode_partitions")
    part_spread = kernel_spread(binding, "decode_partitions") if part_n else None
    comb_spread = kernel_spread(binding, "shared_prefix")
    join_spread = kernel_spread(binding, "prefix_join")
    binding.profiler_reset()
    step_spread = spread_us(timer.step_times_ms(step, steps))
    del calls, devs
    torch.cuda.synchronize()
    binding.workspace_release()
    torch.cuda.empty_cache()
    return dict(sec=sec, part_ms=part_ms, part_launches=part_n, plan=plan,
                part_spread=part_spread, comb_spread=comb_spread, join_spread=join_spread,
                step_spread=step_spread)


def bench_long_share(torch, binding, W, steps, warmup):
    """The long-context workload split eight ways by contiguous block ranges
    (the split across GPUs that pa_decode_lse + pa_merge_states serve): one
    range's pa_decode_lse and the merge of eight such partial states, timed
    by the library's kernel timer."""
    import numpy as np
    case = W.long_bf16_decode()
    B = case.block_size
    b1 = round(-(-int(case.context_lens.max()) // B) / 8)
    table = np.ascontiguousarray(case.block_table[:, :b1])
    lens = np.minimum(case.context_lens, b1 * B).astype(np.int32)
    share = W.PagedCase(case.dtype, case.q, case.k_pool, case.v_pool, table, lens, case.scale)
    nbytes = W.decode_bytes(share, out_bytes_per_elem=4)
    d = binding.upload_case(share)
    S, H, D = case.q.shape
    out = torch.empty((S, H, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((S, H), dtype=torch.float32, device="cuda")
    parts = torch.randn((8, S, H, D), dtype=torch.float32, device="cuda")
    part_lse = torch.randn((8, S, H), dtype=torch.float32, device="cuda")
    merged = torch.empty((S, H, D), dtype=torch.bfloat16, device="cuda")
    call = lambda: binding.decode_lse(d["q"], d["k_pool"], d["v_pool"], d["block_table"],  # noqa
                                      d["context_lens"], case.scale, out=out, lse=lse)
    def both(i):
        call()
        binding.merge_states(parts, part_lse, out=merged, want_lse=False)
    warm_up(torch, both, warmup, EXTRA_WARM_S)
    binding.profiler_reset()
    binding.profiler_enable(True)
    for _ in range(steps):
        call()
        binding.merge_states(parts, part_lse, out=merged, want_lse=False)
    torch.cuda.synchronize()
    binding.profiler_enable(False)
    dec_ms, _ = kernel_avg_ms(binding, "decode_partitions")
    mrg_ms, _ = kernel_avg_ms(binding, "merge_states")
    binding.profiler_reset()
    del d, out, lse, parts, part_lse, merged
    binding.workspace_release()
    torch.cuda.empty_cache()
    return {"keys_per_sequence": int(lens.max()),
            "share_decode_kernel_avg_us": round(dec_ms * 1e3, 2),
            "share_decode_kernel_GB/s": round(nbytes / (dec_ms * 1e-3) / 1e9, 1),
            "merge_8_parts_kernel_avg_us": round(mrg_ms * 1e3, 2),
            "algorithmic_bytes_share": nbytes}


def copy_bandwidth(torch, reps=10):
    """Attainable HBM rate for context: a 1 GiB device-to-device copy (1 GiB
    read + 1 GiB written per call), wall clock over `reps` calls."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * (1 << 30) / sec / 1e9


def cpu_oracle_decode(case, budget_s=10.0, max_passes=8):
    """The fp64 oracle on the whole workload, timed on the host: passes
    until about `budget_s` seconds of work (at most `max_passes`)."""
    import oracle
    t0 = time.perf_counter()
    c0 = time.process_time()
    passes = 0
    while True:
        oracle.decode(case.q, case.k_pool, case.v_pool, case.block_table, case.context_lens,
                      case.scale, case.dtype)
        passes += 1
        if time.perf_counter() - t0 > budget_s or passes >= max_passes:
            break
    wall = time.perf_counter() - t0
    cpu = time.process_time() - c0
    return wall / passes, cpu / wall, passes


def main():
    a = parse()
    if a.write_traffic:
        write_traffic(*a.write_traffic)
        return
    if a.rdreq_check:
        rdreq_check(*a.rdreq_check)
        return
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); the decode and "
              "prefill kernels shard by sequence or KV head with no exchange, and this build "
              "measures the one-GPU share.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from paged_kv_cache_decode_amd import binding
    from paged_kv_cache_decode_amd import workloads as W

    binding.lib()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if a.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 1 << 30, "launches": 10}))
        return
    only = set(x for x in a.only.split(",") if x)
    want = lambda k: not only or k in only  # noqa: E731
    result = {}
    extra = {}

    def headline():
        """The headline: batched GQA decode, fp16.  Measured after the extra
        entries, so that it starts on a GPU in the state of a serving loop
        rather than after process start-up; its warm-up is exactly the
        --warmup steps and its timed region exactly the --steps steps."""
        nonlocal result
        # ---------------- headline: batched GQA decode, fp16 -----------------
        if want("gqa"):
            case = W.gqa_f16_decode()
            nbytes = W.decode_bytes(case, out_bytes_per_elem=2)
            r = bench_decode_case(torch, binding, case, a.steps, a.warmup, 3, torch.float16)
            gbs = nbytes / r["sec"] / 1e9
            part_gbs = nbytes / (r["part_ms"] * 1e-3) / 1e9
            src = source_hash("decode.hip")
            roof = {"bound": "hbm", "achieved": round(part_gbs, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(part_gbs / HBM_PEAK_GBS, 4),
                    "traffic": load_traffic("decode_partitions", "gqa-f16-decode", src, nbytes),
                    "kernel": "decode_partitions_kernel<f16,128,4>",
                    "kernel_avg_us": round(r["part_ms"] * 1e3, 2),
                    "kernel_us": r["part_spread"],
                    "algorithmic_bytes_per_launch": nbytes}
            result = {
                "metric": "Paged attn: decode HBM GB/s (% of peak); causal prefill TFLOP/s "
                          "(% MFMA peak)",
                "value": round(gbs, 1),
                "unit": "GB/s",
                "n_gpus": 1,
                "steps": a.steps,
                "warmup": a.warmup,
                "ms_per_step": round(r["sec"] * 1e3, 4),
                "step_us": r["step_spread"],
                "higher_is_better": True,
                "scaling": "weak",
                "vs_baseline": None,
                "dtype": "f16",
                "data": "synthetic",
                "config": {"workload": "gqa-f16-decode", "seqs": 64, "heads": 32, "kv_heads": 8,
                           "head_dim": 128, "block_size": 16, "context": "uniform[128,4096]",
                           "total_keys": int(case.context_lens.sum()), "out": "f16",
                           "pool_copies_rotated": 3, "decode_workers": r["plan"]["workers"],
                           **workload_meta(case)},
                "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                "roofline": roof,
            }
            if not a.headline_only and not a.no_cpu_baseline:
                sec, busy, passes = cpu_oracle_decode(case)
                host = host_info()
                result["cpu_baseline"] = {
                    "value": round(nbytes / sec / 1e9, 4), "unit": "GB/s",
                    "cores": min(blas_threads(host), host["affinity_cpus"]),
                    "kind": "oracle",
                    "sample": f"the whole workload (64 sequences x 32 heads), {passes} pass(es), "
                              f"{sec:.2f} s per pass, fp64 numpy",
                    "host": host, "avg_busy_threads": round(busy, 2)}
            del case


    if not a.headline_only:
        # ---------------- long-context decode, bf16 ----------------------
        if want("long"):
            case = W.long_bf16_decode()
            nbytes = W.decode_bytes(case, out_bytes_per_elem=2)
            r = bench_decode_case(torch, binding, case, max(10, a.steps // 2), a.warmup, 1,
                                  torch.bfloat16, warm_seconds=EXTRA_WARM_S)
            lgbs = nbytes / (r["part_ms"] * 1e-3) / 1e9
            extra["long-bf16-decode"] = {
                "GB/s": round(nbytes / r["sec"] / 1e9, 1),
                "frac_of_hbm_peak": round(nbytes / r["sec"] / 1e9 / HBM_PEAK_GBS, 4),
                "ms_per_step": round(r["sec"] * 1e3, 4),
                "step_us": r["step_spread"],
                "roofline": {"bound": "hbm", "achieved": round(lgbs, 1), "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": round(lgbs / HBM_PEAK_GBS, 4),
                             "traffic": load_traffic("decode_partitions", "long-bf16-decode",
                                                     source_hash("decode.hip"), nbytes),
                             "kernel": "decode_partitions_kernel<bf16,128,4>",
                             "kernel_avg_us": round(r["part_ms"] * 1e3, 2),
                             "kernel_us": r["part_spread"],
                             "algorithmic_bytes_per_launch": nbytes},
                "decode_workers": r["plan"]["workers"],
                "config": {"seqs": 4, "heads": 32, "kv_heads": 8, "head_dim": 128,
                           "block_size": 16, "context": 100_000, "out": "bf16",
                           **workload_meta(case)},
                "algorithmic_bytes": nbytes}
            del case
        # ---- the same two workloads with head-major blocks (layout option) ----
        for key, name, make, steps, copies, odt in (
                ("gqa-hm", "gqa-f16-decode-head-major-blocks", W.gqa_f16_decode, a.steps, 3,
                 torch.float16),
                ("long-hm", "long-bf16-decode-head-major-blocks", W.long_bf16_decode,
                 max(10, a.steps // 2), 1, torch.bfloat16)):
            if not want(key):
                continue
            case = make()
            nbytes = W.decode_bytes(case, out_bytes_per_elem=2)
            rh = bench_decode_case(torch, binding, case, steps, a.warmup, copies, odt,
                                   warm_seconds=EXTRA_WARM_S,
                                   head_major=True)
            extra[name] = {
                "GB/s": round(nbytes / rh["sec"] / 1e9, 1),
                "frac_of_hbm_peak": round(nbytes / rh["sec"] / 1e9 / HBM_PEAK_GBS, 4),
                "ms_per_step": round(rh["sec"] * 1e3, 4),
                "partition_kernel_GB/s": round(nbytes / (rh["part_ms"] * 1e-3) / 1e9, 1),
                "partition_kernel_avg_us": round(rh["part_ms"] * 1e3, 2),
                "partition_kernel_us": rh["part_spread"],
                "step_us": rh["step_spread"],
                "pool_layout": "[NB, Hkv, B, d] memory, viewed as [NB, B, Hkv, d]",
                "config": workload_meta(case)}
            del case
        # ---- one GPU's share of the long context split eight ways ----------
        if want("share"):
            extra["long-bf16-decode-8way-share"] = bench_long_share(torch, binding, W,
                                                                    max(10, a.steps // 2),
                                                                    a.warmup)
        # ---------------- prefix-shared decode sweep ---------------------
        if want("prefix") or want("prefix16"):
            for B in ((16, 32, 64, 128) if want("prefix") else (16,)):
                case = W.prefix_shared_bf16_decode(B)
                logical = W.decode_bytes(case, out_bytes_per_elem=2)
                unique = (case.meta["unique_tokens"] * 8 * 128 * 2 * 2 +
                          logical - int(case.context_lens.sum()) * 8 * 128 * 2 * 2)
                r = bench_decode_case(torch, binding, case, max(10, a.steps // 2), a.warmup, 3,
                                      torch.bfloat16, warm_seconds=EXTRA_WARM_S)
                rc = bench_decode_case(torch, binding, case, max(10, a.steps), a.warmup, 3,
                                       torch.bfloat16, prefix_len=case.meta["prefix_len"],
                                       warm_seconds=EXTRA_WARM_S)
                med = rc["step_spread"]["median"] * 1e-6
                extra[f"prefix-shared-bf16-decode-B{B}"] = {
                    "unique_GB/s": round(unique / r["sec"] / 1e9, 1),
                    "frac_of_hbm_peak_unique": round(unique / r["sec"] / 1e9 / HBM_PEAK_GBS, 4),
                    "logical_GB/s": round(logical / r["sec"] / 1e9, 1),
                    "ms_per_step": round(r["sec"] * 1e3, 4),
                    "step_us": r["step_spread"],
                    "partition_kernel_avg_us": round(r["part_ms"] * 1e3, 2),
                    "partition_kernel_us": r["part_spread"],
                    "shared_prefix_call": {
                        "unique_GB/s": round(unique / rc["sec"] / 1e9, 1),
                        "frac_of_hbm_peak_unique": round(unique / rc["sec"] / 1e9 /
                                                         HBM_PEAK_GBS, 4),
                        "ms_per_step": round(rc["sec"] * 1e3, 4),
                        "step_us": rc["step_spread"],
                        "frac_of_hbm_peak_unique_at_median_step": round(
                            unique / med / 1e9 / HBM_PEAK_GBS, 4),
                        "prefix_and_suffix_kernel_us": rc["comb_spread"],
                        "join_kernel_us": rc["join_spread"]},
                    "unique_bytes": unique, "logical_bytes": logical,
                    "config": {**workload_meta(case), "prefix_len": case.meta["prefix_len"]}}
                if B == 16:
                    extra["prefix-shared-bf16-decode-B16"]["dram_measured"] = \
                        prefix_dram_measured(unique)
                del case
        # ---------------- causal prefill, bf16 ---------------------------
        if want("prefill"):
            case = W.causal_bf16_prefill()
            flops = W.prefill_flops(case)
            d = binding.upload_case(case)
            out = torch.empty(case.q.shape, dtype=torch.bfloat16, device="cuda")
            call = binding.PreparedPrefill(d["q"], d["k_pool"], d["v_pool"], d["block_table"],
                                           d["context_lens"], d["query_start_loc"],
                                           case.max_query_len, case.scale, True, out)
            timer = Timer(torch)
            warm_up(torch, lambda i: call(), a.warmup, EXTRA_WARM_S)
            steps = max(10, a.steps // 2)
            sec = timer.run(lambda i: call(), steps)
            binding.profiler_reset()
            binding.profiler_enable(True)
            timer.run(lambda i: call(), steps)
            binding.profiler_enable(False)
            k_ms, _ = kernel_avg_ms(binding, "prefill")
            k_spread = kernel_spread(binding, "prefill")
            binding.profiler_reset()
            step_spread = spread_us(timer.step_times_ms(lambda i: call(), steps))
            mhz = shader_mhz_during(torch, binding, lambda i: call(), steps, sec)
            cus = torch.cuda.get_device_properties(0).multi_processor_count
            tf = flops / sec / 1e12
            ktf = flops / (k_ms * 1e-3) / 1e12
            roof = {"bound": "mfma", "achieved": round(ktf, 1), "peak": BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(ktf / BF16_PEAK_TFLOPS, 4),
                    "kernel": "prefill_kernel<bf16,4,4>",
                    "kernel_avg_us": round(k_ms * 1e3, 2), "kernel_us": k_spread,
                    "traffic": load_traffic("prefill", "causal-bf16-prefill",
                                            source_hash("prefill.hip"),
                                            W.prefill_bytes(case))}
            if mhz:
                # 4096 dense bf16 FLOPs per clock per CU (2.5 PFLOP/s nominal
                # is 256 CUs x 2.4 GHz x 4096).
                measured_peak = cus * mhz * 1e6 * 4096 / 1e12
                roof["clock_measured"] = {
                    "shader_MHz": round(mhz, 1), "compute_units": cus,
                    "peak_at_measured_clock": round(measured_peak, 1),
                    "frac_at_measured_clock": round(ktf / measured_peak, 4),
                    "how": "pa_clock_probe wave on a side stream during a separate pass "
                           "of the same steps"}
            entry = {"TFLOP/s": round(tf, 1),
                     "frac_of_bf16_mfma_peak": round(tf / BF16_PEAK_TFLOPS, 4),
                     "ms_per_step": round(sec * 1e3, 4), "step_us": step_spread,
                     "flops": flops, "prompt_lens": case.meta["lens"],
                     "config": workload_meta(case), "roofline": roof}
            if not a.no_cpu_baseline:
                import oracle
                # The prompts one by one, all 32 heads, until all are done or
                # about 25 s of host work has been spent.
                qsl = case.query_start_loc
                t0 = time.perf_counter()
                c0 = time.process_time()
                sub_flops, done = 0, []
                for s0 in range(case.num_seqs):
                    L = int(qsl[s0 + 1] - qsl[s0])
                    oracle.prefill(case.q[qsl[s0]:qsl[s0 + 1]], case.k_pool, case.v_pool,
                                   case.block_table[s0:s0 + 1], case.context_lens[s0:s0 + 1],
                                   np.array([0, L], dtype=np.int32), case.scale, True,
                                   case.dtype)
                    sub_flops += 2 * 32 * 128 * L * (L + 1)
                    done.append(L)
                    if time.perf_counter() - t0 > 25.0:
                        break
                wall = time.perf_counter() - t0
                cpu = time.process_time() - c0
                what = ("the whole workload" if len(done) == case.num_seqs else
                        f"the first {len(done)} of {case.num_seqs} prompts")
                host = host_info()
                entry["cpu_baseline"] = {
                    "value": round(sub_flops / wall / 1e12, 6), "unit": "TFLOP/s",
                    "cores": min(blas_threads(host), host["affinity_cpus"]), "kind": "oracle",
                    "host": host, "avg_busy_threads": round(cpu / wall, 2),
                    "sample": f"{what} ({sum(done)} query rows), all 32 heads, fp64 numpy, "
                              f"{wall:.1f} s"}
            extra["causal-bf16-prefill"] = entry
            del d, call
        # ------- the same prompts with other group sizes (G = 1, 2, 8) -------
        if want("prefill-g"):
            for hkv in (32, 16, 4):
                case = W.causal_bf16_prefill(num_kv_heads=hkv)
                flops = W.prefill_flops(case)
                d = binding.upload_case(case)
                out = torch.empty(case.q.shape, dtype=torch.bfloat16, device="cuda")
                call = binding.PreparedPrefill(d["q"], d["k_pool"], d["v_pool"],
                                               d["block_table"], d["context_lens"],
                                               d["query_start_loc"], case.max_query_len,
                                               case.scale, True, out)
                warm_up(torch, lambda i: call(), a.warmup, EXTRA_WARM_S)
                binding.profiler_reset()
                binding.profiler_enable(True)
                Timer(torch).run(lambda i: call(), max(10, a.steps // 2))
                binding.profiler_enable(False)
                k_ms, _ = kernel_avg_ms(binding, "prefill")
                k_spread = kernel_spread(binding, "prefill")
                binding.profiler_reset()
                G = 32 // hkv
                extra[f"causal-bf16-prefill-G{G}"] = {
                    "kv_heads": hkv, "kernel_TFLOP/s": round(flops / (k_ms * 1e-3) / 1e12, 1),
                    "frac_of_bf16_mfma_peak": round(flops / (k_ms * 1e-3) / 1e12 /
                                                    BF16_PEAK_TFLOPS, 4),
                    "kernel_us": k_spread, "flops": flops}
                del d, call, case
    headline()
    if not a.headline_only and (not only or "copy" in only):
        gbs = copy_bandwidth(torch)
        extra["device_copy"] = {
            "GB/s": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "what": "attainable-rate context: torch copy of 1 GiB (1 GiB read + 1 GiB "
                    "written per call)"}
    if extra:
        result["extra"] = extra
    if not result:
        result = {"extra": extra}
    print(json.dumps(result))


if __name__ == "__main__":
    main()
