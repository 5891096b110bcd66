#!/usr/bin/env python3
"""Benchmark of the paged latent-KV MLA decode hot path on one MI355X.

One step is one full decode call over one batch: the split-KV attention pass plus
the log-sum-exp combine pass, with every input already resident in HBM.  The
default workload is speculative-verify decode at B=4, Sq=4 draft tokens, H=16
heads (one GPU's share of a 64-head model at attention TP4) over a 65,536-token
cached prefix per request ("spec4").  Inputs are seeded synthetic tensors shaped
like the pages' coding-agent workloads.

Prints one JSON line.  `value` is KV-read throughput: the latent bytes a step must
read (every visible row once, 576 bf16) divided by the measured time per step.
`step_us_percentiles` come from HIP events recorded between consecutive steps, over
at least 100 steps and at least a second of them.
`roofline` rates the dominant kernel (the split-KV pass) against its MI355X peak:
its duration is the average of per-launch HIP event pairs recorded around each
split launch on the stream the kernels run on, in a second run of the same steps
(the timed steps themselves carry no event markers); like rocprofv3's kernel
durations, they include each launch's dispatch and end-of-kernel release.  Its
`traffic` is the HBM bytes per launch measured by rocprofv3 counters (stored under
profiles/ and used only while the kernel sources are unchanged).  `measured_peaks`
are same-run HIP microbenchmarks (libmla_peaks.so): a 4 GiB streaming read, the
split kernel's own global->LDS load path, and a bf16 MFMA loop; they run before the
warm-up, which also brings the clocks up.  With the default workload, the other
decode configurations of the metric (B=8 and B=16 spec-decode, the H=128 sweep)
and the prefix prefill are timed too, each as a sub-record with its own roofline.
`cpu_baseline` times the fp64 CPU oracle on a bounded sample of the main workload.

Step counts: --steps K and --warmup W are taken exactly when given.  By default a
workload first runs 20 probe steps to estimate its step time, then warms up for at
least 50 ms of steps (the GPU's clocks climb for tens of ms after any idle time,
the host-side set-up included) and times at least 0.2 s of steps (200 steps at the
least; 100 for a sub-record), so that the window's first launch and final
synchronisation are amortised.  The JSON line reports the counts actually run;
`warmup` includes the probe steps.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
METRIC = "MLA decode µs/step + KV-read HBM GB/s (% peak), B=4/8/16, Sq=4–16, 64K ctx"
SUB_RECORDS = ["spec8", "spec16", "sweep", "prefill"]
PERCENTILE_STEPS = 100
PERCENTILE_SECONDS = 1.0
PERCENTILE_MAX_STEPS = 20000
WARMUP_SECONDS = 0.05  # default least span of untimed steps before the timed window
TIMED_SECONDS = 0.2    # default least span of the timed window
PROBE_STEPS = 20       # untimed steps that estimate the step time for the defaults


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def algorithmic_work(w):
    """Bytes a step must move and flops it must do (split partials not counted).

    Bytes: every visible latent row once (576 values: bf16, or E4M3 for an E4M3
    pool), the queries (576 bf16 per folded row), the outputs (512 fp32 + 1 fp32 LSE
    per folded row) and the block table entries of the visible pages.  Flops:
    2 (576 + 512) per visible (query row, key) pair."""
    import numpy as np
    L = w.seq_lens.astype(np.int64)
    M = w.Sq * w.H
    pages = int(((L + 63) // 64).sum())
    kv = w.kv_bytes()
    q = w.B * M * (512 + w.rope_width) * 2
    out = w.B * M * (512 * 4 + 4)
    bt = pages * 4
    t = np.arange(w.Sq, dtype=np.int64)
    if w.causal:
        n_vis = (L[:, None] - w.Sq + t[None, :] + 1).sum()
    else:
        n_vis = L.sum() * w.Sq
    flops = int(n_vis) * w.H * 2 * (512 + w.rope_width + 512)
    return dict(kv_bytes=kv, bytes=kv + q + out + bt, flops=flops, pages=pages)


def host_cpu_model():
    """The host CPU's model name, from /proc/cpuinfo (None where unreadable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def blas_name():
    """The BLAS numpy was built against (name and version), or None."""
    import numpy as np
    try:
        blas = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        return f"{blas.get('name')} {blas.get('version')}"
    except Exception:
        return None


def cpu_baseline(w, budget_s=12.0):
    """fp64 oracle on whole requests (cycling through the batch) until ~budget_s has
    passed; KV bytes of the requests done over the wall time, in GB/s."""
    from oracle import E4M3Pool, mla_attention_folded, mla_attention_nope
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    pool = E4M3Pool(w.kv_pool, w.kv_scale) if w.kv_format == "e4m3" else w.kv_pool
    done, kv, t0 = 0, 0, time.perf_counter()
    while True:
        b = done % w.B
        sl = slice(b, b + 1)
        if w.kv_pool.shape[2] == 512:  # NoPE rows
            mla_attention_nope(w.q_nope[sl], pool, w.block_table[sl], w.seq_lens[sl], w.scale,
                               w.causal)
        else:
            mla_attention_folded(w.q_nope[sl], w.q_rope[sl], pool, w.block_table[sl],
                                 w.seq_lens[sl], w.scale, w.causal)
        done += 1
        kv += int(w.seq_lens[b]) * w.row_bytes
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": kv / dt / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": host_cpu_model(), "blas": blas_name(),
            "sample": f"{done} request passes (cycling over the {w.B} requests of the same "
                      f"workload), fp64 numpy, {dt:.1f} s wall",
            "seconds_per_step_extrapolated": dt * w.B / done}


def stored_traffic(config, kv):
    """HBM bytes per split-KV launch from profiles/traffic_<config>[_e4m3|_nope].json,
    if the counters were taken on the current kernel sources (kv: bf16, e4m3 or nope,
    the pool format they were taken with)."""
    from mla_latent_kv_16_amd.profiling import kernel_hash
    tag = config if kv == "bf16" else f"{config}_{kv}"
    path = os.path.join(ROOT, "profiles", f"traffic_{tag}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_hash") != kernel_hash():
        return None
    fb, wb = rec.get("split_fetch_bytes"), rec.get("split_write_bytes")
    if fb is None or wb is None:
        return None
    return int(fb + wb)


def scale_later_pages(w, first, factor):
    """Multiplies the bf16 latent rows of logical pages >= `first` of every request by
    `factor` (a power of two, so exactly), in place."""
    import numpy as np
    from mla_latent_kv_16_amd.workloads import f32_to_bf16_bits
    pages = np.unique(w.block_table[:, first:][w.block_table[:, first:] >= 0])
    for chunk in np.array_split(pages, max(1, len(pages) // 256)):
        f = (w.kv_pool[chunk].astype(np.uint32) << 16).view(np.float32) * np.float32(factor)
        w.kv_pool[chunk] = f32_to_bf16_bits(f)


class HostWorkload:
    """A numpy workload (mla_latent_kv_16_amd.workloads) moved to the device."""

    def __init__(self, w, torch, dev, copies, nope):
        import numpy as np
        self.w, self.name = w, w.spec.name
        self.B, self.Sq, self.H, self.causal = w.B, w.Sq, w.H, w.causal
        self.seq_lens, self.max_pages, self.scale = w.seq_lens, w.max_pages, float(w.scale)
        self.rope_width = w.q_rope.shape[3]
        self.kv_scale = w.kv_scale if w.kv_format == "e4m3" else None
        self.nope = nope
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
        self.q_nope, self.q_rope = t(w.q_nope), t(w.q_rope)
        if w.kv_format == "e4m3":
            self.pools = [torch.from_numpy(w.kv_pool).to(dev) for _ in range(copies)]
        else:
            self.pools = [t(w.kv_pool) for _ in range(copies)]
        self.bt = torch.from_numpy(w.block_table).to(dev)
        self.sl = torch.from_numpy(w.seq_lens).to(dev)

    def kv_bytes(self):
        return self.w.kv_bytes()


class DeviceWorkload:
    """A workload whose lengths and block table follow the numpy recipe (steps 1 and 2,
    same seed) and whose latent rows and queries are drawn on the device: N(0,1)
    from torch's seeded device generator, rounded to bf16 (nearest even).  Used for
    the sub-records, whose multi-GB pools would take tens of seconds to draw on the
    host.  Every pool page holds finite values (no NaN poison; nothing here checks
    results)."""

    def __init__(self, name, torch, dev):
        from mla_latent_kv_16_amd.workloads import DEFAULT_SCALE, draw_layout
        spec, L, bt, pool_pages = draw_layout(name)
        self.name, self.B, self.Sq, self.H, self.causal = name, spec.B, spec.Sq, spec.H, spec.causal
        self.seq_lens, self.max_pages = L.astype("int32"), bt.shape[1]
        self.scale, self.rope_width, self.kv_scale, self.nope = float(DEFAULT_SCALE), 64, None, False
        g = torch.Generator(device=dev)
        g.manual_seed(1000 + spec.seed)
        pool = torch.empty((pool_pages, 64, 576), dtype=torch.bfloat16, device=dev)
        chunk = 2048  # pages per draw: 302 MB of fp32
        for p0 in range(0, pool_pages, chunk):
            n = min(chunk, pool_pages - p0)
            pool[p0:p0 + n] = torch.randn((n, 64, 576), generator=g, device=dev).to(torch.bfloat16)
        self.pools = [pool.view(torch.int16)]
        rnd = lambda *shape: torch.randn(shape, generator=g, device=dev).to(
            torch.bfloat16).view(torch.int16)
        self.q_nope = rnd(spec.B, spec.Sq, spec.H, 512)
        self.q_rope = rnd(spec.B, spec.Sq, spec.H, 64)
        self.bt = torch.from_numpy(bt).to(dev)
        self.sl = torch.from_numpy(self.seq_lens).to(dev)

    def kv_bytes(self):
        return int(self.seq_lens.astype("int64").sum()) * 1152


def timeline_summary(torch, np, mla, hw, G, reps):
    """Per-workgroup timelines of the split pass (mla_decode_splitkv_timeline) over
    `reps` launches, each on the next pool copy: medians of the start-up phases, and per
    XCD (the hardware XCC id each workgroup ran on) the median and latest end of the
    walk and the latest completed stores, in us from the launch's first start."""
    per_xcd = {x: {"walk_end_med": [], "walk_end_max": [], "stores_done_max": []} for x in range(8)}
    phases = {"start_to_prefix": [], "prefix_to_first_block": [], "first_block_to_walk_end": [],
              "walk_end_to_stores_done": []}
    spans = []
    for r in range(reps):
        pool = hw.pools[r % len(hw.pools)]
        _, _, trace, ticks = mla.decode_splitkv_timeline(
            hw.q_nope, hw.q_rope, pool, hw.bt, hw.sl, hw.scale, causal=hw.causal,
            num_partitions=G)
        torch.cuda.synchronize()
        tr, tk = trace.cpu().numpy(), ticks.cpu().numpy().astype(np.float64)
        tk = tk[(tk > 0).all(axis=1)]
        xcc = tr[(ticks.cpu().numpy() > 0).all(axis=1), 0]
        us = (tk - tk[:, 0].min()) / 100.0
        spans.append(float(us[:, 4].max()))
        d = np.diff(us, axis=1)
        for k, name in enumerate(phases):
            phases[name].append(float(np.median(d[:, k])))
        for x in range(8):
            m = xcc == x
            if m.any():
                per_xcd[x]["walk_end_med"].append(float(np.median(us[m, 3])))
                per_xcd[x]["walk_end_max"].append(float(us[m, 3].max()))
                per_xcd[x]["stores_done_max"].append(float(us[m, 4].max()))
    med = lambda v: round(float(np.median(v)), 2) if v else None
    return {"launches": reps, "span_us_median": med(spans),
            "phase_us_median": {k: med(v) for k, v in phases.items()},
            "per_xcd": [{"xcc": x, **{k: [round(a, 2) for a in v] for k, v in per_xcd[x].items()}}
                        for x in range(8)],
            "how": "mla_decode_splitkv_timeline: 100 MHz clock stamps per workgroup (start, "
                   "page prefix, first block in LDS, walk over, stores complete) and its XCC id"}


def roofline(work, kernel_s, traffic):
    """The dominant kernel against the roof the step's arithmetic intensity meets first."""
    hbm = work["bytes"] / kernel_s / 1e9
    tf = work["flops"] / kernel_s / 1e12
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    if work["flops"] / work["bytes"] > ridge:
        return {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": traffic}, hbm, tf
    return {"bound": "hbm", "achieved": round(hbm, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(hbm / HBM_PEAK_GBPS, 4), "traffic": traffic}, hbm, tf


def default_counts(step_s, steps=None, warmup=None, min_steps=200, min_warmup=20):
    """(timed steps, untimed steps) for a step time of step_s seconds: an explicit count
    is kept; otherwise at least WARMUP_SECONDS of untimed and TIMED_SECONDS of timed
    steps, and never fewer than min_warmup / min_steps."""
    step_s = max(step_s, 1e-7)
    if warmup is None:
        warmup = max(min_warmup, math.ceil(WARMUP_SECONDS / step_s))
    if steps is None:
        steps = max(min_steps, math.ceil(TIMED_SECONDS / step_s))
    return steps, warmup


def time_workload(torch, np, mla, dw, G, steps, warmup, traffic, peaks,
                  percentile_seconds=PERCENTILE_SECONDS, min_steps=200, min_warmup=20):
    """Times one workload: steps (two launches each: split-KV + combine), per-step event
    percentiles, per-launch split events, and back-to-back split launches.  steps or
    warmup None: chosen from the step time (module docstring)."""
    dev = dw.q_nope.device
    ws = mla.new_workspace(dw.B, dw.Sq, dw.H, dw.max_pages, G, device=dev)
    O = torch.empty((dw.B, dw.Sq, dw.H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((dw.B, dw.Sq, dw.H), dtype=torch.float32, device=dev)
    calls = [mla.BoundDecode(dw.q_nope, dw.q_rope, pool, dw.bt, dw.sl, dw.scale, dw.causal, G, O,
                             lse, ws, kv_scale=dw.kv_scale, nope=dw.nope) for pool in dw.pools]
    n = len(calls)

    def step(i):
        c = calls[i % n]
        c.splitkv()
        c.combine()

    probe = 0
    if steps is None or warmup is None:
        probe = PROBE_STEPS
        torch.cuda.synchronize()
        t_probe = time.perf_counter()
        for i in range(probe):
            step(i)
        torch.cuda.synchronize()
        steps, warmup = default_counts((time.perf_counter() - t_probe) / probe, steps, warmup,
                                       min_steps, min_warmup)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # the timed steps: nothing but the decode calls between the two synchronisations
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    us_step = (time.perf_counter() - t0) * 1e6 / steps
    if mla.read_error_flags(ws):
        raise SystemExit(f"{dw.name}: kernel reported a data fault flag")

    ev = lambda: torch.cuda.Event(enable_timing=True)
    # step durations between consecutive events (one event per step boundary) over at
    # least PERCENTILE_STEPS steps and at least percentile_seconds of steps
    np_steps = int(max(PERCENTILE_STEPS, steps,
                       min(PERCENTILE_MAX_STEPS, percentile_seconds / (us_step * 1e-6))))
    marks = [ev() for _ in range(np_steps + 1)]
    torch.cuda.synchronize()
    marks[0].record()
    for i in range(np_steps):
        step(i)
        marks[i + 1].record()
    torch.cuda.synchronize()
    step_us = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(np_steps)]) * 1e3
    # per-launch events around each split launch (the dominant kernel), on its stream
    kev = [(ev(), ev()) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        c = calls[i % n]
        kev[i][0].record()
        c.splitkv()
        kev[i][1].record()
        c.combine()
    torch.cuda.synchronize()
    split_us = np.array([a.elapsed_time(b) for a, b in kev]) * 1e3
    # the split pass alone, back to back
    b2b = (ev(), ev())
    torch.cuda.synchronize()
    b2b[0].record()
    for i in range(steps):
        calls[i % n].splitkv()
    b2b[1].record()
    torch.cuda.synchronize()
    split_b2b = b2b[0].elapsed_time(b2b[1]) * 1e3 / steps

    work = algorithmic_work(dw)
    split_avg = float(split_us.mean())
    roof, hbm, tf = roofline(work, split_avg * 1e-6, traffic)
    if peaks:
        key = "mfma_bf16_TFLOPs" if roof["bound"] == "mfma" else "lds_dma_stream_GBps"
        roof["frac_of_measured_peak"] = round(roof["achieved"] / peaks[key], 4)
        roof["measured_peak_used"] = key
    rec = {
        "steps": int(steps),
        "warmup": int(warmup + probe),
        "us_per_step": round(us_step, 2),
        "kv_GBps_per_step": round(work["kv_bytes"] / (us_step * 1e-6) / 1e9, 1),
        "kv_frac_of_hbm_peak": round(work["kv_bytes"] / (us_step * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "step_us_percentiles": {"steps": int(np_steps),
                                "median": round(float(np.median(step_us)), 2),
                                "p10": round(float(np.percentile(step_us, 10)), 2),
                                "p90": round(float(np.percentile(step_us, 90)), 2)},
        "split_pass_us": round(split_avg, 2),
        "split_pass_us_median": round(float(np.median(split_us)), 2),
        "split_pass_us_p10_p90": [round(float(np.percentile(split_us, 10)), 2),
                                  round(float(np.percentile(split_us, 90)), 2)],
        "split_kernel_us_back_to_back": round(split_b2b, 2),
        "split_pass_hbm_frac": round(hbm / HBM_PEAK_GBPS, 4),
        "split_pass_mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
        "roofline": roof,
    }
    log(f"{dw.name}: step {us_step:.1f} us (median {rec['step_us_percentiles']['median']:.1f}, "
        f"p10 {rec['step_us_percentiles']['p10']:.1f}, p90 {rec['step_us_percentiles']['p90']:.1f}"
        f" over {np_steps}); split pass {split_avg:.1f} us per launch, {split_b2b:.1f} us back to "
        f"back; split kernel {hbm:.0f} GB/s, {tf:.1f} TFLOP/s ({roof['bound']} frac "
        f"{roof['frac']})")
    return rec, calls, ws, work


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: at least 0.2 s of steps, 200 at the least)")
    ap.add_argument("--percentile-seconds", type=float, default=PERCENTILE_SECONDS,
                    help="least span of steps behind the step percentiles (at least 100 "
                         "steps are always timed); a profiled run passes 0 to keep its "
                         "traces short")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default: at least 50 ms of steps, 20 at the "
                         "least, after 20 probe steps)")
    ap.add_argument("--config", default="spec4",
                    help="tiny | spec4 | spec8 | spec16 | sweep | prefill")
    ap.add_argument("--kv", default="bf16", choices=["bf16", "e4m3"],
                    help="latent pool format: bf16, or E4M3 codes with a per-tensor scale")
    ap.add_argument("--nope", action="store_true",
                    help="NoPE-MLA rows (the 512-wide latent alone, no RoPE part; bf16)")
    ap.add_argument("--partitions", type=int, default=0, help="0 = library default")
    ap.add_argument("--rotate", type=int, default=0,
                    help="input copies cycled per step (0 = enough to exceed 2x MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-measured-peaks", action="store_true",
                    help="skip the same-run peak microbenchmarks")
    ap.add_argument("--no-sub-records", action="store_true",
                    help="time only --config (no spec8 / spec16 / sweep / prefill sub-records)")
    ap.add_argument("--no-single-pass", action="store_true",
                    help="skip the one-launch comparison (profiler runs: every split-KV kernel "
                         "launch is then a split pass alone)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the cache-write and absorb/project timings")
    ap.add_argument("--rescale", action="store_true",
                    help="worst case of the exp2 reference: keys of every page from the seventh "
                         "on scaled by 8 and queries drawn N(0, 4^2), so that later scores pass "
                         "the first block's reference by far more than 32 (log2) and each piece is "
                         "walked three times (bf16 pools)")
    ap.add_argument("--timeline", type=int, default=0, metavar="LAUNCHES",
                    help="after timing, record per-workgroup timelines of this many split "
                         "passes (bf16 pools) and add their per-XCD summary to the line")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after timing, launch a plain 256 MiB device copy 3 times (counter "
                         "calibration for rocprofv3 --pmc runs)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this hot path runs on a single MI355X with no "
              "inter-GPU collectives (each GPU would serve its own head share, requests or KV "
              "range); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import mla_latent_kv_16_amd as mla
    from mla_latent_kv_16_amd.workloads import f32_to_bf16_bits, make_workload

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.init()

    t_gen = time.perf_counter()
    if args.nope and args.kv != "bf16":
        raise SystemExit("--nope pools are bf16")
    w = make_workload(args.config, kv_format=args.kv, rope=not args.nope,
                      q_sigma=4.0 if args.rescale else None)
    if args.rescale:
        if args.kv != "bf16":
            raise SystemExit("--rescale takes bf16 pools")
        scale_later_pages(w, first=6, factor=8.0)
    kv_main = w.kv_bytes()
    # Cycle over independent copies of the pool so that consecutive steps cannot be
    # served from the 256 MB MALL left warm by the previous step.
    n_copies = args.rotate or max(1, min(4, int(np.ceil(2 * 256e6 / max(kv_main, 1))) + 1))
    hw = HostWorkload(w, torch, dev, n_copies, args.nope)
    log(f"{args.config} ({args.kv} pool): B={w.B} Sq={w.Sq} H={w.H} "
        f"kv={kv_main / 1e6:.1f} MB, generated in {time.perf_counter() - t_gen:.1f}s, "
        f"{n_copies} pool copies")
    G = args.partitions or mla.auto_partitions(w.B, w.Sq, w.H, w.max_pages)
    traffic = stored_traffic(args.config, "nope" if args.nope else args.kv)
    # same-run peaks right before the timed work: about a second of sustained load,
    # which also settles the clocks that the host-side input generation let drop
    peaks = None
    if not args.no_measured_peaks:
        from mla_latent_kv_16_amd import peaks as peaks_mod
        peaks = peaks_mod.measure(torch, dev)
        log(f"measured peaks: {peaks}")
    main_rec, calls, ws, work = time_workload(torch, np, mla, hw, G, args.steps, args.warmup,
                                              traffic, peaks, args.percentile_seconds)
    O = calls[0].out

    # the same steps in one launch each (mla_decode_single_pass), for comparison
    single_pass_us = None
    if G > 1 and not args.no_single_pass and not args.nope:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(main_rec["steps"]):
            calls[i % n_copies].single_pass()
        torch.cuda.synchronize()
        single_pass_us = (time.perf_counter() - t0) * 1e6 / main_rec["steps"]
        if mla.read_error_flags(ws):
            raise SystemExit("kernel reported a data fault flag")

    timeline = None
    if args.timeline:
        if args.kv != "bf16" or args.nope:
            raise SystemExit("--timeline takes bf16 pools")
        timeline = timeline_summary(torch, np, mla, hw, G, args.timeline)
        log(f"timeline: {json.dumps(timeline)}")

    if args.copy_probe:
        from mla_latent_kv_16_amd.profiling import COPY_PROBE_BYTES
        src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    append_us = append_bytes = None
    gemm = {}
    if not args.nope and not args.no_extras:
        # the cache write of a step's new rows (mla_kv_append[_e4m3]), back to back after
        # every decode timing (it rewrites the draft rows of the pools)
        kv_new = torch.from_numpy(f32_to_bf16_bits(np.random.default_rng(1).standard_normal(
            (w.B, w.Sq, 576)).astype(np.float32)).view(np.int16)).to(dev)
        app_ws = torch.zeros(256, dtype=torch.uint8, device=dev)
        appends = [mla.bound_kv_append(kv_new, p, hw.bt, hw.sl, app_ws, hw.kv_scale)
                   for p in hw.pools]
        for i in range(3):
            appends[i % n_copies]()
        aev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        torch.cuda.synchronize()
        aev[0].record()
        for i in range(50):
            appends[i % n_copies]()
        aev[1].record()
        torch.cuda.synchronize()
        append_us = aev[0].elapsed_time(aev[1]) / 50 * 1e3
        if mla.read_error_flags(app_ws):
            raise SystemExit("kv append reported a data fault flag")
        append_bytes = w.B * w.Sq * 576 * (2 + w.row_bytes // 576)
        # the GEMMs around the attention for this batch's shape (absorb before, project
        # after), with seeded random weights, timed back to back
        g_rng = np.random.default_rng(2)
        bfw = lambda shape, sc: torch.from_numpy(f32_to_bf16_bits(
            (g_rng.standard_normal(shape) * sc).astype(np.float32)).view(np.int16)).to(dev)
        q_heads = bfw((w.B, w.Sq, w.H, 128), 1.0)
        w_uk_t, w_uv = bfw((w.H, 512, 128), 128 ** -0.5), bfw((w.H, 128, 512), 512 ** -0.5)
        q_lat = torch.empty((w.B, w.Sq, w.H, 512), dtype=torch.int16, device=dev)
        o_proj = torch.empty((w.B, w.Sq, w.H, 128), dtype=torch.float32, device=dev)
        rows_h = w.B * w.Sq * w.H
        for tag, (fn, _) in (("absorb", mla.bound_absorb_q(q_heads, w_uk_t, q_lat)),
                             ("project", mla.bound_project_o(O, w_uv, o_proj))):
            fn()
            gev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            torch.cuda.synchronize()
            gev[0].record()
            for _ in range(20):
                fn()
            gev[1].record()
            torch.cuda.synchronize()
            us = gev[0].elapsed_time(gev[1]) / 20 * 1e3
            gemm[f"{tag}_us"] = round(us, 2)
            gemm[f"{tag}_TFLOPs"] = round(2 * rows_h * 128 * 512 / (us * 1e-6) / 1e12, 2)
    del calls, hw
    torch.cuda.empty_cache()

    # the metric's other configurations, timed in the same run
    subs = {}
    if (args.config == "spec4" and args.kv == "bf16" and not args.nope
            and not args.no_sub_records):
        for name in SUB_RECORDS:
            t_gen = time.perf_counter()
            dw = DeviceWorkload(name, torch, dev)
            Gs = mla.auto_partitions(dw.B, dw.Sq, dw.H, dw.max_pages)
            log(f"{name}: B={dw.B} Sq={dw.Sq} H={dw.H} kv={dw.kv_bytes() / 1e6:.1f} MB, drawn "
                f"on the device in {time.perf_counter() - t_gen:.1f}s, partitions={Gs}")
            rec, c2, _, wk = time_workload(torch, np, mla, dw, Gs, None, None,
                                           stored_traffic(name, "bf16"), peaks,
                                           args.percentile_seconds, min_steps=100,
                                           min_warmup=50)
            rec = {"config": {"workload": name, "B": dw.B, "Sq": dw.Sq, "H": dw.H,
                              "context": [int(dw.seq_lens.min()), int(dw.seq_lens.max())],
                              "partitions": Gs, "kv_bytes": wk["kv_bytes"],
                              "tflops_per_step": wk["flops"] / 1e12},
                   **rec}
            subs[name] = rec
            del c2, dw
            torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w)
        log(f"cpu oracle: {cpu['value']:.4f} GB/s on {cpu['cores']} threads ({cpu['sample']})")

    us_step = main_rec["us_per_step"]
    value = work["kv_bytes"] / (us_step * 1e-6) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": main_rec["steps"],
        "warmup": main_rec["warmup"],
        "ms_per_step": round(us_step * 1e-3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": ("synthetic (seeded N(0,1) latents and queries; pages scattered in a 2x pool"
                 + (f"; latents stored as E4M3 codes of value / {w.kv_scale})" if args.kv == "e4m3"
                    else ")")),
        "config": {"workload": args.config, "B": w.B, "Sq": w.Sq, "H": w.H,
                   "context": [int(w.seq_lens.min()), int(w.seq_lens.max())],
                   "page_size": 64,
                   "latent": ("512 bf16 (NoPE)" if args.nope else
                              "512+64 " + ("e4m3, per-tensor scale" if args.kv == "e4m3"
                                           else "bf16")),
                   "partitions": G,
                   "kv_bytes": work["kv_bytes"], "tflops_per_step": work["flops"] / 1e12,
                   **({"values": "worst case of the exp2 reference: keys of pages 7 on x8, "
                                 "queries N(0, 4^2)"} if args.rescale else {})},
        **main_rec,
        "single_pass_us_per_step": None if single_pass_us is None else round(single_pass_us, 2),
        "kv_append_us": None if append_us is None else round(append_us, 2),
        "kv_append_GBps": (None if append_us is None
                           else round(append_bytes / (append_us * 1e-6) / 1e9, 2)),
        "absorb_project": gemm or None,
        "measured_peaks": peaks,
        **({"timeline": timeline} if timeline else {}),
        "sub_records": subs or None,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
