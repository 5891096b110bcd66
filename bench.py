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
`roofline` rates the dominant kernel (the split-KV pass) against its MI355X peak.
Its duration is the average of per-launch HIP event pairs recorded around each
split launch on the stream the kernels run on, in a second run of the same steps
(the timed steps themselves carry no event markers); like rocprofv3's kernel
durations, they include each launch's dispatch and end-of-kernel release.  A run of
back-to-back split launches, where those overlap the neighbouring launches, is
reported too.  Its `traffic` is the HBM bytes per
launch measured by rocprofv3 counters (stored under profiles/ and used only while
the kernel sources are unchanged).  `cpu_baseline`
times the fp64 CPU oracle on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
METRIC = "MLA decode µs/step + KV-read HBM GB/s (% peak), B=4/8/16, Sq=4–16, 64K ctx"


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
    q = w.B * M * (512 + w.q_rope.shape[3]) * 2
    out = w.B * M * (512 * 4 + 4)
    bt = pages * 4
    t = np.arange(w.Sq, dtype=np.int64)
    if w.causal:
        n_vis = (L[:, None] - w.Sq + t[None, :] + 1).sum()
    else:
        n_vis = L.sum() * w.Sq
    flops = int(n_vis) * w.H * 2 * (w.kv_pool.shape[2] + 512)
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


def measured_peaks(torch, dev):
    """Achievable peaks on this device, for context beside the spec-sheet ones: a plain
    2 GiB device-to-device copy (bytes read + written per second) and a 8192^3 bf16
    matmul through torch (hipBLASLt), each timed with events over back-to-back runs."""
    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e-3
    n = 2 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    t_copy = timed(lambda: dst.copy_(src), 10)
    del src, dst
    k = 8192
    x = torch.randn(k, k, device=dev, dtype=torch.bfloat16)
    y = torch.randn(k, k, device=dev, dtype=torch.bfloat16)
    t_mm = timed(lambda: torch.matmul(x, y), 10)
    del x, y
    torch.cuda.empty_cache()
    return {"hbm_copy_GBps": round(2 * n / t_copy / 1e9, 1),
            "mfma_bf16_matmul_TFLOPs": round(2 * k ** 3 / t_mm / 1e12, 1)}


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=400,
                    help="untimed steps first: the clocks take about 25 ms of load to settle")
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
                    help="skip the copy / matmul measurement of achievable peaks")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the graph-replayed steps")
    ap.add_argument("--no-single-pass", action="store_true",
                    help="skip the one-launch comparison (profiler runs: every split-KV kernel "
                         "launch is then a split pass alone)")
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
    t_gen = time.perf_counter()
    if args.nope and args.kv != "bf16":
        raise SystemExit("--nope pools are bf16")
    w = make_workload(args.config, kv_format=args.kv, rope=not args.nope)
    work = algorithmic_work(w)
    log(f"{args.config} ({args.kv} pool): B={w.B} Sq={w.Sq} H={w.H} pages={work['pages']} "
        f"kv={work['kv_bytes'] / 1e6:.1f} MB, generated in {time.perf_counter() - t_gen:.1f}s")

    # Cycle over independent copies of the pool so that consecutive steps cannot be
    # served from the 256 MB MALL left warm by the previous step.
    pool_bytes = w.kv_pool.nbytes
    n_copies = args.rotate or max(1, min(4, int(np.ceil(2 * 256e6 / max(work["kv_bytes"], 1))) + 1))
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    q_nope, q_rope = t(w.q_nope), t(w.q_rope)
    if args.kv == "e4m3":
        pools = [torch.from_numpy(w.kv_pool).to(dev) for _ in range(n_copies)]
        kv_scale = w.kv_scale
    else:
        pools = [t(w.kv_pool) for _ in range(n_copies)]
        kv_scale = None
    bt = torch.from_numpy(w.block_table).to(dev)
    sl = torch.from_numpy(w.seq_lens).to(dev)
    G = args.partitions or mla.auto_partitions(w.B, w.Sq, w.H, w.max_pages)
    ws = mla.new_workspace(w.B, w.Sq, w.H, w.max_pages, G, device=dev)
    O = torch.empty((w.B, w.Sq, w.H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((w.B, w.Sq, w.H), dtype=torch.float32, device=dev)
    scale = float(w.scale)
    log(f"partitions={G} pool copies={n_copies} ({pool_bytes / 1e9:.2f} GB each)")

    calls = [mla.BoundDecode(q_nope, q_rope, pool, bt, sl, scale, w.causal, G, O, lse, ws,
                             kv_scale=kv_scale, nope=args.nope) for pool in pools]

    def step(i, ev=None):
        c = calls[i % n_copies]
        if ev is not None:
            ev[0].record()
        c.splitkv()
        if ev is not None:
            ev[1].record()
        c.combine()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # The timed steps: nothing but the decode calls between the two synchronisations.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    if mla.read_error_flags(ws):
        raise SystemExit("kernel reported a data fault flag")

    # Per-launch split durations, from a second run of the same steps with events
    # around each split launch.  The library launches on torch's current stream, where
    # these events are recorded.  An event adds a marker to the stream, so this run is
    # kept out of the timed steps.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    split_ms = [a.elapsed_time(b) for a, b in evs]
    split_avg = float(np.mean(split_ms))

    # The dominant kernel alone: the split pass launched back to back over the same
    # rotation of pools, two events around the whole run.  Per-launch events around
    # each split inside the steps also count the dispatch of the launch and the
    # release at its end; back to back, those overlap the neighbouring launches.
    kev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    torch.cuda.synchronize()
    kev[0].record()
    for i in range(args.steps):
        calls[i % n_copies].splitkv()
    kev[1].record()
    torch.cuda.synchronize()
    split_b2b = kev[0].elapsed_time(kev[1]) / args.steps

    # The same steps replayed from HIP graphs (one captured step per pool copy), as a
    # serving loop that captures its decode step would run them.
    graph_us = None
    if not args.no_graph:
        gs = torch.cuda.Stream()
        gcalls = [mla.BoundDecode(q_nope, q_rope, pool, bt, sl, scale, w.causal, G, O, lse, ws,
                                  stream=gs, kv_scale=kv_scale, nope=args.nope) for pool in pools]
        graphs = []
        with torch.cuda.stream(gs):
            for c in gcalls:
                c()
        torch.cuda.synchronize()
        for c in gcalls:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=gs):
                c()
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % n_copies].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            graphs[i % n_copies].replay()
        torch.cuda.synchronize()
        graph_us = (time.perf_counter() - t0) * 1e6 / args.steps
        del graphs, gcalls

    # The same steps in one launch each (mla_decode_single_pass), for comparison.
    single_pass_us = None
    if G > 1 and not args.no_single_pass and not args.nope:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            calls[i % n_copies].single_pass()
        torch.cuda.synchronize()
        single_pass_us = (time.perf_counter() - t0) * 1e6 / args.steps
        if mla.read_error_flags(ws):
            raise SystemExit("kernel reported a data fault flag")

    if args.copy_probe:
        from mla_latent_kv_16_amd.profiling import COPY_PROBE_BYTES
        src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # The cache write of a step's new rows (mla_kv_append[_e4m3]), timed back to back
    # after every decode timing (it rewrites the draft rows of the pools); the write
    # takes 576-wide rows, so NoPE pools skip it.
    append_us = append_bytes = None
    if not args.nope:
        kv_new = torch.from_numpy(f32_to_bf16_bits(np.random.default_rng(1).standard_normal(
            (w.B, w.Sq, 576)).astype(np.float32)).view(np.int16)).to(dev)
        app_ws = torch.zeros(256, dtype=torch.uint8, device=dev)
        appends = [mla.bound_kv_append(kv_new, p, bt, sl, app_ws, kv_scale) for p in pools]
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

    # The GEMMs around the attention for this batch's shape (absorb before, project
    # after), with seeded random weights, timed back to back.
    gemm = {}
    if not args.nope:
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

    peaks = None if args.no_measured_peaks else measured_peaks(torch, dev)

    value = work["kv_bytes"] / (ms_step * 1e-3) / 1e9
    # the dominant kernel's average launch duration: per-launch events on its stream
    hbm_achieved = work["bytes"] / (split_avg * 1e-3) / 1e9
    mfma_achieved = work["flops"] / (split_avg * 1e-3) / 1e12
    traffic = stored_traffic(args.config, "nope" if args.nope else args.kv)
    # the bound is the roof the step's arithmetic intensity meets first
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    mfma_bound = work["flops"] / work["bytes"] > ridge
    if mfma_bound:
        roof = {"bound": "mfma", "achieved": round(mfma_achieved, 2),
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(mfma_achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic}
    else:
        roof = {"bound": "hbm", "achieved": round(hbm_achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(hbm_achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic}
    if peaks:
        key = "mfma_bf16_matmul_TFLOPs" if mfma_bound else "hbm_copy_GBps"
        roof["frac_of_measured_peak"] = round(roof["achieved"] / peaks[key], 4)
    log(f"step {ms_step * 1e3:.1f} us (split pass {split_avg * 1e3:.1f} us with per-launch events, "
        f"median {np.median(split_ms) * 1e3:.1f} p10 {np.percentile(split_ms, 10) * 1e3:.1f} "
        f"p90 {np.percentile(split_ms, 90) * 1e3:.1f}; "
        f"{split_b2b * 1e3:.1f} us back to back); {value:.0f} GB/s of KV; split kernel "
        f"{hbm_achieved:.0f} GB/s, {mfma_achieved:.1f} TFLOP/s")

    cpu = None
    if not args.no_cpu_baseline:
        del pools, calls
        torch.cuda.empty_cache()
        cpu = cpu_baseline(w)
        log(f"cpu oracle: {cpu['value']:.4f} GB/s on {cpu['cores']} threads ({cpu['sample']})")

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "us_per_step": round(ms_step * 1e3, 2),
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
                   "kv_bytes": work["kv_bytes"], "tflops_per_step": work["flops"] / 1e12},
        "kv_frac_of_hbm_peak": round(value / HBM_PEAK_GBPS, 4),
        "split_pass_us": round(split_avg * 1e3, 2),
        "split_pass_us_median": round(float(np.median(split_ms)) * 1e3, 2),
        "split_pass_us_p10_p90": [round(float(np.percentile(split_ms, 10)) * 1e3, 2),
                                  round(float(np.percentile(split_ms, 90)) * 1e3, 2)],
        "split_kernel_us_back_to_back": round(split_b2b * 1e3, 2),
        "us_per_step_graph_replay": None if graph_us is None else round(graph_us, 2),
        "single_pass_us_per_step": None if single_pass_us is None else round(single_pass_us, 2),
        "split_pass_hbm_frac": round(hbm_achieved / HBM_PEAK_GBPS, 4),
        "split_pass_mfma_frac": round(mfma_achieved / MFMA_BF16_PEAK_TFLOPS, 4),
        "kv_append_us": None if append_us is None else round(append_us, 2),
        "kv_append_GBps": (None if append_us is None
                           else round(append_bytes / (append_us * 1e-6) / 1e9, 2)),
        "absorb_project": gemm or None,
        "roofline": roof,
        "measured_peaks": peaks,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
