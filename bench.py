#!/usr/bin/env python3
"""Decode-step benchmark for paged attention on one MI355X.

One step = the whole hot path over one batch:
  host allocator bookkeeping for one new token per sequence (slots, copy-on-write
  pairs, block tables), the upload of the step's index data (pa_upload),
  pa_copy_blocks (when pairs exist), pa_reshape_and_cache of the new K/V, and the
  decode over every cached token (pa_decode_auto: single pass, or split partials +
  LSE merge).  --fused-write runs the write inside the decode launch instead
  (pa_decode_append).  Workloads 6 and 7 keep the pools as 8-bit codes (FP8 E4M3 /
  int8 with per-pool scales): pa_reshape_and_cache_quant quantises the new K/V and
  pa_decode_quant decodes.  Workload 8 appends 4 tokens per sequence and verifies them
  in one pa_decode_multi launch (4 causal query tokens per sequence).  Workload 9 keeps
  int8 codes with one scale per (token, KV head) in each block's tiles: the write
  quantises every new row with its own scale.

Default workload: 64 sequences, 32 query / 32 KV heads of dimension 128, fp16,
block size 16, contexts uniform in [256, 2048] (a LLaMA-7B-like layer), pool of
8192 blocks in shuffled order.  Inputs are synthetic (seeded normals) and
resident in HBM before the timed region.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload 1..9] [--path single|split]
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

PEAK_HBM_GBS = 8000.0


def steps_that_fit(context_lens, block_size, num_blocks, tokens_per_step, max_steps):
    """The most steps (up to max_steps) in which every sequence can grow by tokens_per_step
    tokens without its blocks outgrowing a pool of num_blocks (no block is shared)."""
    def blocks(k):
        return sum(-(-(n + k * tokens_per_step) // block_size) for n in context_lens)
    return max(k for k in range(max_steps + 1) if k == 0 or blocks(k) <= num_blocks)
DECODE_SRC = os.path.join(ROOT, "paged_kv_cache_333_amd", "csrc", "decode.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")


STAGING_BUFFERS = 16  # rotating pinned staging buffers of the step's index data
EVENT_EVERY = 8       # a stream event after the decode of every 8th step (see Bench.__init__)
TIMING_SETS = 4     # event sets reused round robin by the steps that time the decode
# the window [k - STAGING_BUFFERS, k - 2] holds STAGING_BUFFERS - 1 consecutive steps, so it holds
# an event step whenever EVENT_EVERY <= STAGING_BUFFERS - 1
assert EVENT_EVERY <= STAGING_BUFFERS - 1


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5, 6, 7, 8, 9])
    ap.add_argument("--path", choices=["auto", "single", "split", "shared"], default=None,
                    help="decode path: pa_decode_auto (the library picks), pa_decode, pa_decode_split, or "
                         "pa_decode_shared (groups of sequences sharing leading blocks, from "
                         "pa_shared_prefix_groups each step); default: shared for the parallel-sampling "
                         "workload (5), auto otherwise")
    ap.add_argument("--partition", type=int, default=512)
    ap.add_argument("--block-size", type=int, default=None,
                    help="run the workload with this block size instead (8, 16, 32 or 64): same contexts, a "
                         "pool of the same token capacity, its free order drawn again")
    ap.add_argument("--fused-write", action="store_true",
                    help="write the new K/V inside the decode launch (pa_decode_append, auto path) instead of "
                         "pa_upload_and_cache before it: a step 1-2 %% shorter, but the decode kernel then "
                         "carries the write (its time by events 5 us longer), so off by default")
    ap.add_argument("--separate-upload", action="store_true",
                    help="upload the index data and write the new K/V in two launches (pa_upload, then "
                         "pa_reshape_and_cache) instead of one (pa_upload_and_cache)")
    ap.add_argument("--order", choices=["longest", "index"], default=None,
                    help="launch order of the sequences (default: index for workload 5, whose forked branches "
                         "share blocks and should run side by side; longest-first otherwise)")
    ap.add_argument("--cache", choices=["stream", "cached"], default=None,
                    help="K/V cache policy (default: cached for workload 5, streaming otherwise)")
    ap.add_argument("--time-every", type=int, default=8,
                    help="time the decode on every k-th timed step (the first one included), by events "
                         "attached to the kernels (pa_set_launch_events)")
    ap.add_argument("--decode-reps", type=int, default=50,
                    help="after the timed steps, time this many decodes of the last step's inputs each way: "
                         "after an untimed scratch copy that flushes the caches, and back to back (median, p10, "
                         "p90; the flushed median sets the roofline figure)")
    ap.add_argument("--flush-mib", type=int, default=1024,
                    help="HBM traffic of the untimed cache flush before each flushed decode, in MiB (half read, "
                         "half written by one pa_copy_blocks launch over a scratch pool; at least 512 MiB written "
                         "is twice the 256 MB MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--json-out", metavar="PATH", help="also write the result line to PATH")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum oracle time for the CPU baseline")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="time a plain copy of known size instead (pa_copy_blocks, 1 GiB read + 1 GiB written "
                         "per launch), to scale HBM counters and give a measured copy bandwidth")
    ap.add_argument("--measure-swap", action="store_true",
                    help="time pa_swap_blocks between the device pool and a pinned host pool instead "
                         "(1024 blocks of 256 KiB each way)")
    ap.add_argument("--profile-commands", metavar="OUTDIR",
                    help="print the rocprofv3 commands that profile this workload into OUTDIR (no GPU needed)")
    ap.add_argument("--summarize-profile", metavar="OUTDIR",
                    help="read the rocprofv3 CSVs those commands wrote, print a markdown summary and record the "
                         "decode kernel's HBM bytes per launch in profiles/decode_traffic.json (no GPU needed)")
    args = ap.parse_args(argv)
    if args.decode_reps < 1:
        ap.error("--decode-reps must be at least 1")
    if args.flush_mib < 2:
        ap.error("--flush-mib must be at least 2")
    return args


def percentiles(values):
    """Median, 10th and 90th percentile (linear interpolation) and the sample count."""
    import numpy as np
    v = np.asarray(values, dtype=np.float64)
    return {"median": float(np.median(v)), "p10": float(np.percentile(v, 10)),
            "p90": float(np.percentile(v, 90)), "n": int(v.size)}


def calibrate_copy(launches: int = 10):
    import torch

    import paged_kv_cache_333_amd as pa
    NB, Hkv, bs, D = 8192, 32, 16, 128          # 128 KiB per block and pool, 1 GiB per pool
    kc = torch.zeros((NB, Hkv, bs, D), dtype=torch.float16, device="cuda")
    vc = torch.zeros((NB, Hkv, D, bs), dtype=torch.float16, device="cuda")
    half = NB // 2
    pairs = torch.stack([torch.arange(half), torch.arange(half, NB)], dim=1).to(torch.int32).cuda()
    per_launch = half * Hkv * bs * D * 2 * 2     # bytes read (= bytes written), both pools
    pa.pa_copy_blocks(kc, vc, pairs)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
    for a, b in ev:
        a.record()
        pa.pa_copy_blocks(kc, vc, pairs)
        b.record()
    torch.cuda.synchronize()
    us = sum(a.elapsed_time(b) for a, b in ev) / launches * 1e3
    print(json.dumps({"calibration": "pa_copy_blocks", "launches": launches + 1,
                      "bytes_read_per_launch": per_launch, "bytes_written_per_launch": per_launch,
                      "kernel_us": us, "copy_gbps_read_plus_write": 2 * per_launch / us / 1e3}), flush=True)


def measure_swap(launches: int = 10):
    """Swap bandwidth over the host link: pa_swap_blocks moving 1024 LLaMA-7B-like blocks
    (128 KiB per block and pool, 256 MiB in all) from the device pool to a pinned host pool
    and back, timed with HIP events on the stream."""
    import torch

    import paged_kv_cache_333_amd as pa
    NB, NH, Hkv, bs, D = 4096, 1024, 32, 16, 128
    kc = torch.zeros((NB, Hkv, bs, D), dtype=torch.float16, device="cuda")
    vc = torch.zeros((NB, Hkv, D, bs), dtype=torch.float16, device="cuda")
    hk = torch.zeros((NH, Hkv, bs, D), dtype=torch.float16).pin_memory()
    hv = torch.zeros((NH, Hkv, D, bs), dtype=torch.float16).pin_memory()
    dev_ids = torch.randperm(NB, generator=torch.Generator().manual_seed(7))[:NH].to(torch.int32)
    out_pairs = torch.stack([dev_ids, torch.arange(NH, dtype=torch.int32)], dim=1).contiguous().cuda()
    in_pairs = torch.stack([torch.arange(NH, dtype=torch.int32), dev_ids], dim=1).contiguous().cuda()
    nbytes = NH * Hkv * bs * D * 2 * 2
    res = {"measurement": "pa_swap_blocks", "blocks": NH, "bytes_per_launch": nbytes}
    for name, args in (("swap_out", (hk, hv, kc, vc, out_pairs)), ("swap_in", (kc, vc, hk, hv, in_pairs))):
        pa.pa_swap_blocks(*args)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
        for a, b in ev:
            a.record()
            pa.pa_swap_blocks(*args)
            b.record()
        torch.cuda.synchronize()
        us = sum(a.elapsed_time(b) for a, b in ev) / launches * 1e3
        res[name + "_us"] = us
        res[name + "_gbps"] = nbytes / us / 1e3
    print(json.dumps(res), flush=True)


# ---------------------------------------------------------------------------
# rocprofv3: kernel trace + HBM counters of the decode kernel, scaled by the same
# counters read on a plain copy of known size (pa_copy_blocks moving 1 GiB).

# (steps, warmup, decode reps): the bench's defaults, so that the repetitions decode the same
# inputs as a default bench run's (the last step's); the counter runs take fewer repetitions
PROFILE_STEPS = {"trace": (50, 10, 50), "counters": (50, 10, 10)}
REP_WARM = 5  # untimed repetitions before each timed set in Bench.kernel_timing


def default_path(workload: int, path: str | None) -> str:
    """The decode path a bench run takes: the one asked for, else pa_decode_shared for the
    parallel-sampling workload (its branches share their prefix blocks) and pa_decode_auto
    for the others."""
    return path or ("shared" if workload == 5 else "auto")


def profile_commands(workload: int, outdir: str, path: str | None) -> list[str]:
    bench = f"python3 {os.path.join(ROOT, 'bench.py')}"
    sel = f" --workload {workload}" + (f" --path {path}" if path else "") + " --no-cpu-baseline"
    ts, tw, tr = PROFILE_STEPS["trace"]
    cs, cw, cr = PROFILE_STEPS["counters"]
    cmds = [f"rocprofv3 --kernel-trace --stats -f csv -d {outdir}/trace -o run -- "
            f"{bench}{sel} --steps {ts} --warmup {tw} --decode-reps {tr} --json-out {outdir}/trace/bench.json"]
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        cmds.append(f"rocprofv3 --pmc {ctr} -f csv -d {outdir}/{ctr.lower()} -o run -- "
                    f"{bench}{sel} --steps {cs} --warmup {cw} --decode-reps {cr}")
        cmds.append(f"rocprofv3 --pmc {ctr} -f csv -d {outdir}/copy_{ctr.lower()} -o run -- "
                    f"{bench} --calibrate-copy")
    return cmds


def _csv_rows(folder: str, suffix: str):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(folder, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {folder}")
    rows = []
    for fn in files:
        with open(fn, newline="", encoding="utf-8") as f:
            rows.extend({k.strip().lower(): v for k, v in r.items()} for r in csv.DictReader(f))
    return rows


def _counter_per_dispatch(folder: str, counter: str, kernel_substr: str,
                          pick: tuple[int, int] | None = None) -> tuple[float, int]:
    """Mean over dispatches of `counter` (summed over its rows per dispatch) for kernels whose
    name contains kernel_substr; with pick = (first, count), over those dispatches only, counted
    in dispatch order among the matching ones."""
    per = {}
    for r in _csv_rows(folder, "counter_collection.csv"):
        if r.get("counter_name") != counter or kernel_substr not in r.get("kernel_name", ""):
            continue
        d = int(r.get("dispatch_id") or r.get("correlation_id"))
        per[d] = per.get(d, 0.0) + float(r["counter_value"])
    if not per:
        raise SystemExit(f"no {counter} rows for *{kernel_substr}* under {folder}")
    vals = [per[d] for d in sorted(per)]
    if pick is not None:
        if len(vals) < pick[0] + pick[1]:
            raise SystemExit(f"{len(vals)} *{kernel_substr}* dispatches under {folder}, expected at least "
                             f"{pick[0] + pick[1]}")
        vals = vals[pick[0]:pick[0] + pick[1]]
    return sum(vals) / len(vals), len(vals)


def summarize_profile(workload: int, outdir: str, path: str | None) -> None:
    # the path that ran (pa_decode_auto takes split on the long-context workload only); the bench
    # line looks its traffic up under the same name.  The commands are listed as they were run.
    asked = path
    path = default_path(workload, path)
    w_path = ("split" if workload == 4 else "single") if path == "auto" else path
    decode = "decode_kernel"
    stats = _csv_rows(os.path.join(outdir, "trace"), "kernel_stats.csv")
    stats.sort(key=lambda r: -float(r["totaldurationns"]))
    dec = [r for r in stats if decode in r["name"]]
    if not dec:
        raise SystemExit("decode kernel missing from the kernel trace")
    # one decode launch per call on every path (the split and shared-prefix paths merge in a
    # second kernel, listed on its own in the trace)
    if len(dec) != 1:
        raise SystemExit(f"{len(dec)} decode kernel instances in the trace, expected one")
    dec_avg_ns = float(dec[0]["averagens"])
    # per-dispatch durations of the decode kernel, in dispatch order: the step loop's decodes,
    # then the flushed repetitions, then the back-to-back ones (each set after REP_WARM untimed)
    trace = [r for r in _csv_rows(os.path.join(outdir, "trace"), "kernel_trace.csv") if decode in r["kernel_name"]]
    trace.sort(key=lambda r: int(r["dispatch_id"]))
    durs = [(int(r["end_timestamp"]) - int(r["start_timestamp"])) / 1e3 for r in trace]
    calls = durs
    ts, tw, tr = PROFILE_STEPS["trace"]
    if len(calls) != ts + tw + 2 * (tr + REP_WARM):
        raise SystemExit(f"{len(calls)} decode calls in the trace, expected {ts + tw + 2 * (tr + REP_WARM)}")
    a = ts + tw
    phases = {"pipelined (timed steps)": calls[tw:a],
              "flushed": calls[a + REP_WARM:a + REP_WARM + tr],
              "back to back": calls[a + 2 * REP_WARM + tr:]}
    copy_bytes = 8192 // 2 * 32 * 16 * 128 * 2 * 2   # calibrate_copy: read (= written) per launch
    cs, cw, cr = PROFILE_STEPS["counters"]
    flushed_reps = (cs + cw + REP_WARM, cr)  # the counter runs' flushed repetitions
    scale, meas = {}, {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        ck, cn = _counter_per_dispatch(os.path.join(outdir, f"copy_{ctr.lower()}"), ctr, "copy_blocks_kernel")
        scale[ctr] = copy_bytes / (ck * 1024.0)
        meas[ctr] = _counter_per_dispatch(os.path.join(outdir, ctr.lower()), ctr, decode, flushed_reps)
        meas[ctr] = (meas[ctr][0], meas[ctr][1], ck, cn)
    traffic = sum(meas[c][0] * 1024.0 * scale[c] for c in meas)
    # the traced bench run's own line: the same decodes timed by its HIP events, and their bytes
    with open(os.path.join(outdir, "trace", "bench.json"), encoding="utf-8") as f:
        line = json.loads(f.read().strip().splitlines()[-1])
    alg = line["decode_alg_bytes"]
    ev_med = line["decode_us"]["flushed"]["median"]
    rp_med = percentiles(phases["flushed"])["median"]
    key = f"workload{workload}-{w_path}"
    try:
        with open(TRAFFIC_FILE, encoding="utf-8") as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    rec[key] = {"bytes_per_launch": traffic, "source_digest": source_digest(),
                "fetch_kib_per_dispatch": meas["FETCH_SIZE"][0], "write_kib_per_dispatch": meas["WRITE_SIZE"][0],
                "fetch_scale": scale["FETCH_SIZE"], "write_scale": scale["WRITE_SIZE"],
                "rocprof_decode_avg_us": dec_avg_ns / 1e3,
                "rocprof_decode_flushed_median_us": rp_med, "events_call_flushed_median_us": ev_med,
                "alg_bytes_per_launch": alg}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w", encoding="utf-8") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")
    out = [f"# rocprofv3: decode kernel, workload {workload} ({w_path} path)", "",
           f"Decode kernel source digest (decode.hip + decode_kernel.hpp + device_common.hpp): "
           f"`{source_digest()}`", "",
           "Commands (run from /tmp with TMPDIR=/tmp; REPO is the repository root, OUTDIR a scratch folder):", "",
           "```"]
    out += [c.replace(ROOT, "$REPO") for c in profile_commands(workload, "OUTDIR", asked)]
    out += ["```", "", "## Kernel trace (--kernel-trace --stats)", "",
                                                        "| kernel | calls | avg us | min us | max us | % time |",
                                                        "|---|---|---|---|---|---|"]
    for r in stats[:8]:
        name = r["name"] if len(r["name"]) < 90 else r["name"][:87] + "..."
        out.append(f"| `{name}` | {r['calls']} | {float(r['averagens']) / 1e3:.2f} | "
                   f"{float(r['minns']) / 1e3:.2f} | {float(r['maxns']) / 1e3:.2f} | {float(r['percentage']):.1f} |")
    out += ["", "Decode kernel duration per dispatch in the trace, by phase of the run:", "",
            "| phase | dispatches | median us | p10 us | p90 us |", "|---|---|---|---|---|"]
    for name, v in phases.items():
        st = percentiles(v)
        out.append(f"| {name} | {st['n']} | {st['median']:.2f} | {st['p10']:.2f} | {st['p90']:.2f} |")
    merge = [r for r in stats if "lse_" in r["name"]]
    merge_us = float(merge[0]["averagens"]) / 1e3 if merge else 0.0
    out += ["", f"The traced run's own bench line times the same flushed decode calls by HIP events at a median "
                f"of {ev_med:.2f} us (decode kernel"
                + (f" and merge, {merge_us:.2f} us average in the trace" if merge else "") + f"). Algorithmic bytes "
                f"of one call on these inputs: {alg / 1e6:.2f} MB, so {alg / ev_med / 1e3:.0f} GB/s by the events "
                f"and {alg / (rp_med + merge_us) / 1e3:.0f} GB/s by the trace.", ""]
    out += ["## HBM counters (--pmc, one counter per run, KiB per dispatch)", "",
            f"Averaged over the {cr} flushed repetitions of each counter run (the last step's inputs, as above).", "",
            "| counter | decode kernel | dispatches | copy kernel (1 GiB each way) | dispatches | scale |",
            "|---|---|---|---|---|---|"]
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        v, n, ck, cn = meas[c]
        out.append(f"| {c} | {v:.1f} | {n} | {ck:.1f} | {cn} | {scale[c]:.4f} |")
    out += ["", f"Scaled HBM traffic per decode launch: **{traffic / 1e6:.2f} MB**, {traffic / alg:.3f} of the "
                f"algorithmic bytes "
                f"(fetch {meas['FETCH_SIZE'][0] * 1024 * scale['FETCH_SIZE'] / 1e6:.2f} MB + write "
                f"{meas['WRITE_SIZE'][0] * 1024 * scale['WRITE_SIZE'] / 1e6:.2f} MB); "
                f"average decode duration in the trace {dec_avg_ns / 1e3:.2f} us."]
    print("\n".join(out))


def source_digest() -> str:
    h = hashlib.sha256()
    for name in ("decode.hip", "decode_kernel.hpp", "device_common.hpp"):
        with open(os.path.join(ROOT, "paged_kv_cache_333_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: int, path: str):
    """HBM bytes per decode launch from the committed rocprofv3 counter summary, if it was taken
    on the current decode kernel source for this workload and path; else None."""
    try:
        with open(TRAFFIC_FILE, encoding="utf-8") as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(f"workload{workload}-{path}")
    if not entry or entry.get("source_digest") != source_digest():
        return None
    return entry.get("bytes_per_launch")


class Bench:
    def __init__(self, args):
        import numpy as np
        import torch

        import paged_kv_cache_333_amd as pa
        import synth

        self.np, self.torch, self.pa, self.synth = np, torch, pa, synth
        self.args = args
        self.w = w = synth.workload(args.workload)
        if args.block_size and args.block_size != w.block_size:
            if args.workload in (1, 5):
                raise SystemExit("--block-size applies to the growing workloads (2-4, 6-9)")
            self.w = w = synth.with_block_size(w, args.block_size)
        self.path = args.path = default_path(args.workload, args.path)
        self.path_ran = set()
        shared = args.workload == 5
        # the branches of a fork stay next to each other (the shared-prefix groups need it);
        # plain decode over shared blocks reads them through the caches
        self.order = args.order or ("index" if shared else "longest")
        self.cached = (args.cache or ("cached" if shared and self.path != "shared" else "stream")) == "cached"
        self.dev = torch.device("cuda:0")
        self.stream = torch.cuda.current_stream()
        seeds = synth.tensor_seeds(args.workload)
        S, H, Hkv, D, bs = w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, w.block_size
        total_steps = args.warmup + args.steps

        # host allocator state (product path: the C++ allocator)
        self.alloc = pa.Allocator(w.num_blocks, bs, w.free_order)
        # Workloads 1 and 5 time one step from a fixed state: workload 1's 16-block pool
        # holds a single step's growth, and workload 5's copies happen on the first append.
        if args.workload == 5:
            for g in range(w.groups):
                parent = 10_000 + g
                self.alloc.seq_create(parent, w.parent_len)
                for b in range(w.branches):
                    s = g * w.branches + b
                    self.alloc.seq_fork(parent, s, w.context_lens[s])
                self.alloc.seq_free(parent)
            self.base = self.alloc.clone()  # every step starts from the post-fork state
            growth = 1
        else:
            for s, n in enumerate(w.context_lens):
                self.alloc.seq_create(s, n)
            self.base = self.alloc.clone() if args.workload == 1 else None
            growth = 1 if args.workload == 1 else total_steps * w.query_len
            # the pool is a shape of the workload, sized for its initial contexts: say up front
            # when the run's growth would not fit instead of failing in the middle of it
            fit = steps_that_fit(w.context_lens, bs, w.num_blocks, w.query_len, total_steps)
            if self.base is None and fit < total_steps:  # workload 1 restarts from its base state
                raise SystemExit(f"workload {args.workload}'s pool of {w.num_blocks} blocks holds "
                                 f"{fit} steps of growth; --warmup {args.warmup} --steps {args.steps} "
                                 f"asks for {total_steps}")
        self.max_blocks = -(-(max(w.context_lens) + growth) // bs) + 1
        self.max_ctx = self.max_blocks * bs

        # device data, resident before timing
        k_shape, v_shape = synth.pool_shapes(w)
        self.quant = bool(w.kv_format)
        if self.quant and args.fused_write:
            raise SystemExit("--fused-write has no 8-bit form: 8-bit pools are written by "
                             "pa_reshape_and_cache_quant")
        # int8 pools with a scale per (token, KV head): each tile holds its codes, then its
        # rows' scales (pa.token_pool); written in two launches (pa_upload, then the write)
        self.rows = w.kv_format == "int8_token"
        if self.quant:
            self.kc = synth.normal_codes_device(k_shape, seeds["key_cache"], w.kv_format)
            self.vc = synth.normal_codes_device(v_shape, seeds["value_cache"], w.kv_format)
            if self.rows:
                sc_shape = (w.num_blocks, Hkv, bs)
                self.kc, self.vc = pa.pack_token_pools(self.kc, synth.row_scales_device(sc_shape, seeds["key_scales"]),
                                                       self.vc, synth.row_scales_device(sc_shape, seeds["value_scales"]))
        else:
            self.kc = synth.normal_device(k_shape, seeds["key_cache"], w.dtype)
            self.vc = synth.normal_device(v_shape, seeds["value_cache"], w.dtype)
        L = self.L = w.query_len  # query tokens (new tokens) per sequence and step
        NS = L * S
        if L > 1 and (self.quant or args.fused_write):
            raise SystemExit("the multi-token workload has model-type pools and a separate write")
        self.q = synth.normal_device((NS, H, D), seeds["query"], w.dtype)
        R = 8  # distinct new-token K/V batches, cycled
        self.newk = synth.normal_device((R, NS, Hkv, D), seeds["new_key"], w.dtype)
        self.newv = synth.normal_device((R, NS, Hkv, D), seeds["new_value"], w.dtype)
        self.out = torch.empty_like(self.q)
        # query rows of sequence s: s L .. s L + L - 1 (constant, resident)
        self.qstart = torch.arange(0, NS + 1, L, dtype=torch.int32, device=self.dev)
        self.ws = None
        if self.path == "shared":
            if L > 1 or self.quant:
                raise SystemExit("--path shared runs on workloads with model-type pools and one query token")
            nbytes = pa.pa_decode_shared_workspace_bytes(S, H, D, self.max_ctx)
            self.ws = torch.empty(nbytes, dtype=torch.uint8, device=self.dev)
        elif self.path != "single":
            nbytes = (pa.pa_decode_multi_workspace_bytes(NS, H, D, self.max_ctx, args.partition) if L > 1 else
                      pa.pa_decode_split_workspace_bytes(S, H, D, self.max_ctx, args.partition))
            self.ws = torch.empty(nbytes, dtype=torch.uint8, device=self.dev)

        # index data in STAGING_BUFFERS rotating pinned staging buffers, one upload (a kernel on the
        # compute stream) per step:
        # [slots LS | lens S | order S | pairs 2LS | tables S*MB | group_start S+1 | prefix_len S]
        # int32 (L new tokens per sequence; the last two for the shared-prefix path)
        self.ids = torch.arange(S, dtype=torch.int64).repeat(L).pin_memory()
        self.bufs = []
        tab_end = 3 * NS + 2 * S + S * self.max_blocks
        total = tab_end + 2 * S + 1
        # A step reusing a buffer must know that the step which last used it has finished.  Every
        # event recorded on the stream as a marker leaves the GPU idle for a few microseconds, so
        # one is recorded after the decode of every EVENT_EVERY-th step only, and step k waits on
        # the host for the latest one recorded at a step in [k - STAGING_BUFFERS, k - 2]: one
        # exists, every step before it has finished, and the GPU still has step k - 1 queued
        # while the host prepares step k.
        self.events = {}
        for _ in range(STAGING_BUFFERS):
            hb = torch.empty(total, dtype=torch.int32).pin_memory()
            db = torch.empty(total, dtype=torch.int32, device=self.dev)
            b = {"idx_h": hb, "idx_d": db}
            for side, t in (("h", hb), ("d", db)):
                b["slots_" + side] = t[0:NS]
                b["len_" + side] = t[NS:NS + S]
                b["order_" + side] = t[NS + S:NS + 2 * S]
                b["pairs_" + side] = t[NS + 2 * S:3 * NS + 2 * S].view(NS, 2)
                b["tab_" + side] = t[3 * NS + 2 * S:tab_end].view(S, self.max_blocks)
                b["gs_" + side] = t[tab_end:tab_end + S + 1]
                b["pl_" + side] = t[tab_end + S + 1:]
            self.bufs.append(b)
        # a few event sets for the steps that time the decode, recorded once here so that they
        # exist (pa_set_launch_events hands them to the kernels) and reused round robin: an
        # event's first use in a launch costs the host far more than later ones.  A set's result
        # is read before its next use, many steps later, when that step has long finished.
        self.timing_pool = []
        for _ in range(TIMING_SETS):
            trio = tuple(torch.cuda.Event(enable_timing=True) for _ in range(3))
            for ev in trio:
                ev.record(self.stream)
            self.timing_pool.append(trio)
        self.pool_next = 0
        self.pool_owner = [None] * TIMING_SETS  # the timing entry each set's pending result goes to
        self.elem = synth.ELEM_BYTES[w.dtype]
        self.kv_elem = 1 if self.quant else self.elem
        # KV bytes per token: every element once, plus (row scales) one fp32 scale per K and V row
        self.kv_bytes_token = 2 * Hkv * (D * self.kv_elem + (4 if self.rows else 0))
        torch.cuda.synchronize()

    def step(self, k: int, timing: list | None, instrument: bool = False):
        pa, w = self.pa, self.w
        b = self.bufs[k % STAGING_BUFFERS]
        if k >= STAGING_BUFFERS:  # the step that last used this buffer is done, its upload included
            last = max(j for j in self.events if k - STAGING_BUFFERS <= j <= k - 2)
            self.events[last].synchronize()
        alloc = self.alloc
        if self.base is not None:
            alloc = self.alloc = self.base.clone()
        S = w.num_seqs
        npairs = alloc.seq_append_slots_into(self.ids.data_ptr(), self.L * S, b["slots_h"].data_ptr(),
                                             b["pairs_h"].data_ptr())
        alloc.build_block_tables_into(self.ids.data_ptr(), S, self.max_blocks, b["tab_h"].data_ptr(),
                                      b["len_h"].data_ptr())
        groups = None
        if self.path == "shared":
            groups = pa.pa_shared_prefix_groups_into(b["tab_h"].data_ptr(), b["len_h"].data_ptr(), S,
                                                     self.max_blocks, w.block_size, b["gs_h"].data_ptr(),
                                                     b["pl_h"].data_ptr())
        order = None
        if self.order == "longest" and self.path != "shared":
            pa.pa_order_longest_first_into(b["len_h"].data_ptr(), S, b["order_h"].data_ptr())
            order = b["order_d"]
        r = k % self.newk.shape[0]
        if instrument:
            # The decode's time, by events attached to the kernels (pa_set_launch_events), which
            # bound them more tightly than marker events recorded around the call: the end of the
            # decode's last kernel (e_end) minus the later of two starts, the end of the last kernel
            # before it (each call below records e_prev at its end; the last one stays) and the
            # processing of the decode's own first dispatch (e_start).  Both precede the decode's
            # first wave, e_prev by stream order.  When the decode was queued behind the previous
            # kernel, e_start comes early and e_prev is the closer bound; when the host enqueued it
            # late (a host-bound step), e_start is.
            slot = self.pool_next % TIMING_SETS
            self.pool_next += 1
            self._resolve(slot)
            e_prev, e_start, e_end = self.timing_pool[slot]
        mark = (lambda: pa.pa_set_launch_events(None, e_prev)) if instrument else (lambda: None)
        fused = self.path == "auto" and self.args.fused_write
        # One launch for the upload and the K/V write when no copy-on-write pair must come
        # between them (the write may land in a block the copy fills).
        one_launch = not npairs and not fused and not self.args.separate_upload and not self.rows
        if one_launch:
            mark()
            pa.pa_upload_and_cache(b["idx_d"], b["idx_h"], self.newk[r], self.newv[r], self.kc, self.vc,
                                   b["slots_h"], w.k_scale, w.v_scale, kv_format=w.kv_format or None)
        else:
            mark()
            pa.pa_upload(b["idx_d"], b["idx_h"])
        if npairs:
            mark()
            pa.pa_copy_blocks(self.kc, self.vc, b["pairs_d"], num_pairs=npairs)
        if one_launch:
            pass
        elif self.quant:
            mark()
            pa.pa_reshape_and_cache_quant(self.newk[r], self.newv[r], self.kc, self.vc, b["slots_d"], w.k_scale,
                                          w.v_scale, kv_format=w.kv_format)
        elif not fused:
            mark()
            pa.pa_reshape_and_cache(self.newk[r], self.newv[r], self.kc, self.vc, b["slots_d"])
        if instrument:
            pa.pa_set_launch_events(e_start, e_end)
        self.last = (b, groups, order, r)
        self.decode(b, groups, order, r)
        if k % EVENT_EVERY == 0:
            self.events[k] = self.torch.cuda.Event()
            self.events[k].record(self.stream)
        for j in [j for j in self.events if j < k - STAGING_BUFFERS]:
            del self.events[j]
        entry = None
        if timing is not None:
            lens = b["len_h"].numpy()
            entry = [None, int(lens.sum()), int(((lens + w.block_size - 1) // w.block_size).sum()), npairs]
            timing.append(entry)
        if instrument:
            self.pool_owner[slot] = entry  # None for a warm-up step: its result is dropped

    def decode(self, b, groups, order, r):
        """The step's decode call over the index data in staging buffer b."""
        pa, w = self.pa, self.w
        fused = self.path == "auto" and self.args.fused_write
        if self.L > 1:
            self.path_ran.add(pa.pa_decode_multi(self.out, self.q, self.kc, self.vc, b["tab_d"], b["len_d"],
                                                 self.qstart, self.L, self.max_ctx, w.scale,
                                                 partition_size=self.args.partition, workspace=self.ws,
                                                 split=self.path == "split", seq_order=order,
                                                 cached_kv=self.cached))
        elif self.quant:
            self.path_ran.add(pa.pa_decode_quant(self.out, self.q, self.kc, self.vc, b["tab_d"], b["len_d"],
                                                 self.max_ctx, w.scale, w.k_scale, w.v_scale,
                                                 kv_format=w.kv_format, partition_size=self.args.partition,
                                                 workspace=self.ws, split=self.path == "split", seq_order=order,
                                                 cached_kv=self.cached))
        elif self.path == "single":
            pa.pa_decode(self.out, self.q, self.kc, self.vc, b["tab_d"], b["len_d"], self.max_ctx, w.scale,
                         seq_order=order, cached_kv=self.cached)
            self.path_ran.add("single")
        elif self.path == "shared":
            pa.pa_decode_shared(self.out, self.q, self.kc, self.vc, b["tab_d"], b["len_d"], b["gs_d"], b["pl_d"],
                                groups[0], groups[1], self.max_ctx, w.scale, self.ws, cached_kv=self.cached)
            self.path_ran.add("shared")
        elif self.path == "split":
            pa.pa_decode_split(self.out, self.q, self.kc, self.vc, b["tab_d"], b["len_d"], self.max_ctx, w.scale,
                               self.args.partition, self.ws, seq_order=order, cached_kv=self.cached)
            self.path_ran.add("split")
        elif fused:
            self.path_ran.add(pa.pa_decode_append(self.out, self.q, self.newk[r], self.newv[r], b["slots_d"],
                                                  self.kc, self.vc, b["tab_d"], b["len_d"], self.max_ctx, w.scale,
                                                  self.args.partition, self.ws, seq_order=order,
                                                  cached_kv=self.cached))
        else:
            self.path_ran.add(pa.pa_decode_auto(self.out, self.q, self.kc, self.vc, b["tab_d"], b["len_d"],
                                                self.max_ctx, w.scale, self.args.partition, self.ws,
                                                seq_order=order, cached_kv=self.cached))

    def kernel_timing(self, reps: int, flush_mib: int, warm: int = 5):
        """Decode time of the last step's inputs, repeated: `reps` decodes each preceded by an
        untimed cache flush (one pa_copy_blocks launch over a scratch pool, flush_mib MiB of
        HBM traffic, half read and half written), then `reps` back to back.  Each decode is
        timed by events attached to its own kernels, as in the step loop (the tighter of the
        end of the kernel before it and the decode's first dispatch, to its last kernel's end).
        The pools hold no more writes than the last step made (its new tokens are rewritten
        only by a step), so every repetition computes the same output.  Returns
        {"flushed": [ms...], "unflushed": [ms...]}."""
        torch, pa = self.torch, self.pa
        blk = 32 * 16 * 128  # elements of one scratch block: 128 KiB in fp16
        half = max(1, flush_mib * 1024 * 1024 // 2 // (blk * 2 * 2))   # read = written = flush_mib / 2
        sk = torch.zeros((2 * half, 32, 16, 128), dtype=torch.float16, device=self.dev)
        sv = torch.zeros((2 * half, 32, 128, 16), dtype=torch.float16, device=self.dev)
        pairs = torch.stack([torch.arange(half), torch.arange(half, 2 * half)], dim=1).to(torch.int32).to(self.dev)
        res = {}
        for mode in ("flushed", "unflushed"):
            trios = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(reps + warm)]
            for trio in trios:
                for ev in trio:
                    ev.record(self.stream)
            torch.cuda.synchronize()
            for e_prev, e_start, e_end in trios:
                if mode == "flushed":
                    pa.pa_set_launch_events(None, e_prev)
                    pa.pa_copy_blocks(sk, sv, pairs)
                else:
                    e_prev.record(self.stream)
                pa.pa_set_launch_events(e_start, e_end)
                self.decode(*self.last)
            torch.cuda.synchronize()
            res[mode] = [min(p.elapsed_time(e), s.elapsed_time(e)) for p, s, e in trios[warm:]]
        del sk, sv
        return res

    def _resolve(self, slot: int):
        """Store the decode time (ms) of the step that last used event set `slot`."""
        entry = self.pool_owner[slot]
        if entry is not None:
            prev_end, start, end = self.timing_pool[slot]
            end.synchronize()
            # two windows that each hold the whole decode; the smaller is the closer bound
            entry[0] = min(prev_end.elapsed_time(end), start.elapsed_time(end))
        self.pool_owner[slot] = None

    def run(self):
        torch = self.torch
        a = self.args
        every = max(1, a.time_every)
        for k in range(a.warmup):  # the warm-up steps take every event set into use
            self.step(k, None, instrument=True)
        torch.cuda.synchronize()
        timing = []
        t0 = time.perf_counter()
        for k in range(a.warmup, a.warmup + a.steps):
            self.step(k, timing, instrument=(k - a.warmup) % every == 0)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        for slot in range(TIMING_SETS):
            self._resolve(slot)
        return wall, timing

    def cpu_baseline(self, min_seconds: float):
        """The float64 oracle on the final step's inputs (all sequences, all heads), repeated
        whole until min_seconds have passed; single-threaded BLAS."""
        import numpy as np
        from threadpoolctl import threadpool_limits

        from oracle import attention as A
        torch, synth, w = self.torch, self.synth, self.w
        b = self.bufs[(self.args.warmup + self.args.steps - 1) % STAGING_BUFFERS]
        lens = b["len_h"].numpy().copy()
        tabs = b["tab_h"].numpy().copy()
        # copy just the used blocks back, renumbered 0..n-1 (a plain re-indexing of the inputs)
        used = np.unique(tabs[tabs >= 0])
        remap = -np.ones(w.num_blocks, dtype=np.int32)
        remap[used] = np.arange(len(used), dtype=np.int32)
        idx = torch.from_numpy(used.astype(np.int64)).to(self.dev)
        if self.rows:
            kc, ks, vc, vs = (t.cpu().numpy() for t in self.pa.unpack_token_pools(
                self.kc.index_select(0, idx), self.vc.index_select(0, idx), w.block_size, w.head_dim))
        elif self.quant:
            kc = self.kc.index_select(0, idx).cpu().numpy()
            vc = self.vc.index_select(0, idx).cpu().numpy()
        else:
            kc = synth.to_numpy(self.kc.index_select(0, idx), w.dtype)
            vc = synth.to_numpy(self.vc.index_select(0, idx), w.dtype)
        q = synth.to_numpy(self.q, w.dtype)
        quant = ((w.kv_format, ks, vs) if self.rows else (w.kv_format, w.k_scale, w.v_scale)) if self.quant else None
        qstart = self.qstart.cpu().numpy()
        t2 = np.where(tabs >= 0, remap[np.maximum(tabs, 0)], -1)
        passes, tokens = 0, 0
        with threadpool_limits(1):
            t0 = time.perf_counter()
            while True:
                if self.L > 1:
                    A.paged_decode_multi(q, kc, vc, t2, lens, qstart, w.scale, w.dtype)
                else:
                    A.paged_decode(q, kc, vc, t2, lens, w.scale, w.dtype, quant=quant)
                passes += 1
                tokens += int(lens.sum())
                el = time.perf_counter() - t0
                if el >= min_seconds:
                    break
        return {"value": tokens / el, "unit": "KV tokens/s", "cores": 1, "host_cores": len(os.sched_getaffinity(0)),
                "kind": "oracle",
                "sample": f"float64 NumPy oracle, whole decode step ({w.num_seqs} seqs x {w.num_heads} heads, "
                          f"{int(lens.sum())} KV tokens) repeated {passes}x in {el:.1f} s on one thread (1 BLAS "
                          f"thread) of the {len(os.sched_getaffinity(0))} host cores this process may use"}


def main():
    args = parse()
    if args.profile_commands:
        print("\n".join(profile_commands(args.workload, args.profile_commands, args.path)))
        return
    if args.summarize_profile:
        summarize_profile(args.workload, args.summarize_profile, args.path)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (the decode shards by "
              "sequence or KV head with no exchange between GPUs, so one GPU's share is the measured unit)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.measure_swap:
        measure_swap()
        return
    bench = Bench(args)
    wall, timing = bench.run()
    reps = bench.kernel_timing(args.decode_reps, args.flush_mib)
    w = bench.w
    e = bench.elem
    timed = [t for t in timing if t[0] is not None]  # the steps whose decode was timed
    kv_tokens = sum(t[1] for t in timing)
    kv_bytes_token = bench.kv_bytes_token
    qo_bytes = 2 * w.num_seqs * w.query_len * w.num_heads * w.head_dim * e

    def alg_bytes(t):
        """Algorithmic bytes of one decode: every valid KV element once, q and out, the table
        entries read and the context lengths."""
        return t[1] * kv_bytes_token + qo_bytes + 4 * t[2] + 4 * w.num_seqs

    # the repetitions run the last step's decode: its bytes over the flushed median
    last_bytes = alg_bytes(timing[-1])
    stats = {"flushed": percentiles(reps["flushed"]), "unflushed": percentiles(reps["unflushed"]),
             "pipelined": percentiles([t[0] for t in timed])}
    med_s = stats["flushed"]["median"] * 1e-3
    achieved = last_bytes / med_s / 1e9
    traffic = measured_traffic(args.workload, "+".join(sorted(bench.path_ran)))
    res = {
        "metric": "paged decode attention: KV GB/s achieved (% of HBM peak) and KV tokens/s",
        "value": kv_tokens / wall,
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": w.num_seqs, "num_heads": w.num_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block_size": w.block_size,
                   "kv_cache_dtype": w.kv_format or w.dtype,
                   "query_tokens_per_seq": w.query_len,
                   "context_lens": "per workload definition, +1 token per step",
                   "mean_kv_tokens_per_step": kv_tokens / len(timing),
                   "decode_path": ("auto: " if bench.path == "auto" else "") + "+".join(sorted(bench.path_ran)),
                   "kv_write": "fused into the decode (pa_decode_append)" if args.fused_write
                   else ("upload and write in one launch (pa_upload_and_cache) when the step has no "
                         "copy-on-write pair, else pa_upload, pa_copy_blocks, write"
                         if not (args.separate_upload or bench.rows) else "pa_upload, then the write (two launches)"),
                   "partition_size": args.partition if "split" in bench.path_ran else None,
                   "launch_order": bench.order, "kv_cache_policy": "cached" if bench.cached else "stream",
                   "cow_pairs_per_step": sum(t[3] for t in timing) / len(timing),
                   # KV slots holding a token, over the slots of the blocks the tables hold (last step)
                   "kv_slot_utilization": timing[-1][1] / max(1, timing[-1][2] * w.block_size)},
        "decode_kernel_us": stats["flushed"]["median"] * 1e3,
        "decode_us": {k: {q: (v * 1e3 if q != "n" else v) for q, v in st.items()} for k, st in stats.items()},
        "decode_timing": (f"median, p10, p90 of HIP events attached to the decode's kernels: 'flushed' = "
                          f"{args.decode_reps} decodes of the last step's inputs, each after an untimed "
                          f"{args.flush_mib} MiB scratch copy (half read, half written); 'unflushed' = the same "
                          f"decodes back to back; 'pipelined' = the decodes timed inside the step loop (every "
                          f"{max(1, args.time_every)}th step)"),
        "decode_alg_bytes": last_bytes,
        "kv_gbps_step": kv_tokens * kv_bytes_token / wall / 1e9,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS,
                     "traffic": traffic},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = bench.cpu_baseline(args.cpu_seconds)
    print(json.dumps(res), flush=True)
    if args.json_out:
        os.makedirs(os.path.dirname(os.path.abspath(args.json_out)), exist_ok=True)
        with open(args.json_out, "w", encoding="utf-8") as f:
            f.write(json.dumps(res) + "\n")


if __name__ == "__main__":
    main()
