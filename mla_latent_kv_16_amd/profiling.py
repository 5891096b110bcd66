"""Summaries of rocprofv3 output for the profiles/ folder.

    python -m mla_latent_kv_16_amd.profiling stats   <kernel_stats.csv> <out.md> "<command>"
    python -m mla_latent_kv_16_amd.profiling traffic <fetch_counter.csv> <write_counter.csv>
                                                     <workload> <out.json> "<commands>"
    python -m mla_latent_kv_16_amd.profiling counters <out.md> "<commands>" <counter.csv>...
    python -m mla_latent_kv_16_amd.profiling table    <bench.jsonl> <out.md> "<commands>"
    python -m mla_latent_kv_16_amd.profiling timeline <bench.jsonl> <out.md> "<command>"

`stats` keeps the per-kernel table of a `--kernel-trace --stats` run.  `traffic`
turns two `--pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs of `bench.py --copy-probe`
into HBM bytes per launch of the split-KV kernel: each counter is scaled by what the
same counter reads for the plain device copy of known size that `--copy-probe`
launches, and the result is stamped with a hash of the kernel sources so that
bench.py reports it only while the kernel is unchanged.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ["csrc/mla_kernels.hip", "csrc/mla_device.h", "csrc/mla_internal.h",
                  "csrc/mla_api.hip"]
SPLIT_KERNEL = "splitkv_kernel"
COMBINE_KERNEL = "combine"  # combine_kernel and combine_rows_kernel
# bench.py --copy-probe copies this many bytes per launch (a plain device-to-device copy)
COPY_PROBE_BYTES = 256 << 20


def kernel_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(PKG, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def stats_table(path: str) -> str:
    rows = _rows(path)
    out = ["| kernel | calls | total (us) | average (us) | min (us) | max (us) | share |",
           "|---|---|---|---|---|---|---|"]
    for r in rows:
        name = r.get("Name") or r.get("KERNEL_NAME") or r.get("Kernel_Name")
        calls = int(float(r.get("Calls", 0)))
        tot = float(r.get("TotalDurationNs", 0)) / 1e3
        avg = float(r.get("AverageNs", 0)) / 1e3
        mn = float(r.get("MinNs", 0)) / 1e3
        mx = float(r.get("MaxNs", 0)) / 1e3
        pct = float(r.get("Percentage", 0))
        out.append(f"| `{name[:90]}` | {calls} | {tot:.1f} | {avg:.2f} | {mn:.2f} | {mx:.2f} | "
                   f"{pct:.1f}% |")
    return "\n".join(out)


def counter_per_kernel(path: str, counter: str):
    """{kernel name: [per-dispatch values]} for one counter of a --pmc CSV."""
    acc = defaultdict(list)
    for r in _rows(path):
        if r["Counter_Name"] != counter:
            continue
        acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return acc


def _pick(acc, needle):
    vals = [v for k, vs in acc.items() if needle in k for v in vs]
    return sum(vals) / len(vals) if vals else None


def _copy_value(acc):
    """Per-dispatch counter value of the copy probe: the copy kernels that moved
    COPY_PROBE_BYTES (the largest dispatches of any copy-like kernel)."""
    cands = []
    for k, vs in acc.items():
        low = k.lower()
        if "copy" in low or "elementwise" in low:
            cands.extend(vs)
    if not cands:
        return None
    top = max(cands)
    big = [v for v in cands if v > 0.5 * top]
    return sum(big) / len(big)


def traffic(fetch_csv: str, write_csv: str, workload: str, commands: str) -> dict:
    f_acc = counter_per_kernel(fetch_csv, "FETCH_SIZE")
    w_acc = counter_per_kernel(write_csv, "WRITE_SIZE")
    kib_copy = COPY_PROBE_BYTES / 1024.0
    f_copy = _copy_value(f_acc)
    w_copy = _copy_value(w_acc)
    f_scale = kib_copy / f_copy if f_copy else None
    w_scale = kib_copy / w_copy if w_copy else None
    res = {"workload": workload, "kernel_hash": kernel_hash(), "commands": commands,
           "copy_probe_bytes": COPY_PROBE_BYTES,
           "fetch_kib_copy_probe": f_copy, "write_kib_copy_probe": w_copy,
           "fetch_scale": f_scale, "write_scale": w_scale}
    for tag, needle in (("split", SPLIT_KERNEL), ("combine", COMBINE_KERNEL)):
        fk = _pick(f_acc, needle)
        wk = _pick(w_acc, needle)
        res[f"{tag}_fetch_kib_raw"] = fk
        res[f"{tag}_write_kib_raw"] = wk
        res[f"{tag}_fetch_bytes"] = fk * 1024 * f_scale if fk is not None and f_scale else None
        res[f"{tag}_write_bytes"] = wk * 1024 * w_scale if wk is not None and w_scale else None
    return res


def counters_table(paths) -> str:
    """Per-dispatch averages of every counter in the given --pmc CSVs, per kernel."""
    per = defaultdict(lambda: defaultdict(list))
    for path in paths:
        for r in _rows(path):
            per[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    out = ["| kernel | counter | dispatches | average per dispatch |", "|---|---|---|---|"]
    for k in sorted(per):
        if "copy" in k.lower() or "elementwise" in k.lower():
            continue
        for c in sorted(per[k]):
            v = per[k][c]
            out.append(f"| `{k[:60]}` | {c} | {len(v)} | {sum(v) / len(v):.4g} |")
    return "\n".join(out)


# Normalisation of the SQ/GRBM counters on this chip (8 XCDs, 32 CUs and 128 SIMDs
# each), checked against the split kernel's own algorithmic flops at prefill, where
# SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 equals them:
#   GRBM_GUI_ACTIVE            GPU-busy cycles summed over the 8 XCDs
#   SQ_VALU_MFMA_BUSY_CYCLES   matrix-core busy cycles summed over all 1,024 SIMDs
#   SQ_WAVE_CYCLES, SQ_BUSY_CU_CYCLES, SQ_WAIT_*, SQ_ACTIVE_INST_*
#                              wave-resident cycles summed over waves, in units of 4
XCDS = 8
SIMDS = 1024


def derived_table(paths) -> str:
    """Per-kernel figures derived from the averaged counters, with the normalisation
    above: clock cycles per XCD, matrix-core busy share of SIMD cycles, instructions
    per MFMA, and shares of wave-resident time."""
    per = defaultdict(lambda: defaultdict(list))
    for path in paths:
        for r in _rows(path):
            per[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    out = ["| kernel | figure | value | from |", "|---|---|---|---|"]
    for k in sorted(per):
        if "copy" in k.lower() or "elementwise" in k.lower():
            continue
        c = {n: sum(v) / len(v) for n, v in per[k].items()}
        name = f"`{k[:60]}`"
        cyc = c.get("GRBM_GUI_ACTIVE")
        if cyc:
            out.append(f"| {name} | GPU-busy cycles per XCD | {cyc / XCDS:.4g} | GRBM_GUI_ACTIVE / 8 |")
            if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
                out.append(f"| {name} | matrix cores busy, share of SIMD cycles | "
                           f"{c['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc / XCDS * SIMDS):.1%} | "
                           f"SQ_VALU_MFMA_BUSY_CYCLES / (1024 x GRBM_GUI_ACTIVE / 8) |")
            if "SQ_WAVE_CYCLES" in c:
                out.append(f"| {name} | waves resident per SIMD (average) | "
                           f"{4 * c['SQ_WAVE_CYCLES'] / (cyc / XCDS * SIMDS):.3g} | "
                           f"4 x SQ_WAVE_CYCLES / (1024 x GRBM_GUI_ACTIVE / 8) |")
        mf = c.get("SQ_INSTS_MFMA")
        if mf:
            for n in ("SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_INSTS_VMEM"):
                if n in c:
                    out.append(f"| {name} | {n} per MFMA | {c[n] / mf:.3g} | {n} / SQ_INSTS_MFMA |")
            if all(n in c for n in ("SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS")):
                tot = (c["SQ_INSTS_VALU"] - mf + c["SQ_INSTS_SALU"] + c["SQ_INSTS_LDS"]) / mf
                out.append(f"| {name} | non-MFMA VALU + SALU + LDS per MFMA | {tot:.3g} | "
                           f"(SQ_INSTS_VALU - SQ_INSTS_MFMA + SALU + LDS) / SQ_INSTS_MFMA |")
        wc = c.get("SQ_WAVE_CYCLES")
        if wc:
            for n in ("SQ_WAIT_ANY", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS"):
                if n in c:
                    out.append(f"| {name} | {n}, share of wave time | {c[n] / wc:.1%} | "
                               f"{n} / SQ_WAVE_CYCLES |")
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in c:
            out.append(f"| {name} | bf16 MFMA flops | {c['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512:.4g} | "
                       f"SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 |")
    return "\n".join(out)


def bench_table(jsonl: str) -> str:
    """One markdown row per bench.py JSON line (as printed by bench.py)."""
    out = ["| workload | KV | µs/step | step median (p10-p90) µs | KV-read rate per step "
           "| split (events) µs | split b2b µs | single pass µs/step | bound "
           "| split kernel achieved | of measured | CPU oracle |",
           "|" + "---|" * 12]
    with open(jsonl) as f:
        recs = [json.loads(ln) for ln in f if ln.startswith("{")]
    for r in recs:
        c, rf, cpu = r["config"], r["roofline"], r.get("cpu_baseline")
        kv = "e4m3" if "e4m3" in c["latent"] else ("nope" if "NoPE" in c["latent"] else "bf16")
        if "values" in c:
            kv += " (exp2-reference worst case)"
        pc = r.get("step_us_percentiles") or {}
        med = f"{pc['median']} ({pc['p10']}-{pc['p90']})" if pc else "—"
        fmt = lambda v: "—" if v is None else f"{v}"
        unit = rf["unit"]
        ach = f"{rf['achieved']} {unit} ({rf['frac']:.1%})"
        cpu_s = f"{cpu['value']:.4g} {cpu['unit']} on {cpu['cores']} threads" if cpu else "—"
        out.append(
            f"| {c['workload']} | {kv} | {r['us_per_step']} | {med} "
            f"| {r['value']} GB/s ({r['kv_frac_of_hbm_peak']:.1%} of 8 TB/s) | {r['split_pass_us']} "
            f"| {r['split_kernel_us_back_to_back']} | {fmt(r.get('single_pass_us_per_step'))} "
            f"| {rf['bound']} | {ach} | {rf.get('frac_of_measured_peak', 0):.0%} | {cpu_s} |")
    return "\n".join(out)


def timeline_table(jsonl: str) -> str:
    """Markdown of the `timeline` object of each bench.py JSON line that has one."""
    out = []
    with open(jsonl) as f:
        recs = [json.loads(ln) for ln in f if ln.startswith("{")]
    for r in recs:
        t = r.get("timeline")
        if not t:
            continue
        c = r["config"]
        out.append(f"## {c['workload']} (B={c['B']}, Sq={c['Sq']}, H={c['H']}, "
                   f"partitions={c['partitions']}), {t['launches']} launches\n")
        out.append(f"Median span of a launch (first start to last stores): {t['span_us_median']} us\n")
        out.append("| phase (median over workgroups, then over launches) | us |\n|---|---|")
        for k, v in t["phase_us_median"].items():
            out.append(f"| {k.replace('_', ' ')} | {v} |")
        out.append("\n| XCC | walk end, median (per launch) | walk end, latest | stores done, "
                   "latest |\n|---|---|---|---|")
        for x in t["per_xcd"]:
            fmt = lambda v: ", ".join(f"{a:.1f}" for a in v)
            out.append(f"| {x['xcc']} | {fmt(x['walk_end_med'])} | {fmt(x['walk_end_max'])} | "
                       f"{fmt(x['stores_done_max'])} |")
        out.append("")
    return "\n".join(out)


def main(argv):
    if len(argv) >= 4 and argv[0] == "stats":
        src, dst, cmd = argv[1], argv[2], argv[3]
        with open(dst, "w") as f:
            f.write(f"# Kernel trace summary\n\nCommand:\n\n```\n{cmd}\n```\n\n")
            f.write(f"Kernel sources hash: `{kernel_hash()}`\n\n")
            f.write(stats_table(src) + "\n")
        print(dst)
    elif len(argv) >= 6 and argv[0] == "traffic":
        res = traffic(argv[1], argv[2], argv[3], argv[5])
        with open(argv[4], "w") as f:
            json.dump(res, f, indent=1)
        print(json.dumps(res, indent=1))
    elif len(argv) >= 4 and argv[0] == "counters":
        dst, cmd = argv[1], argv[2]
        with open(dst, "w") as f:
            f.write(f"# Hardware counters\n\nCommands:\n\n```\n{cmd}\n```\n\n")
            f.write(f"Kernel sources hash: `{kernel_hash()}`\n\n")
            f.write(counters_table(argv[3:]) + "\n\n")
            f.write("Derived figures.  Normalisation: GRBM_GUI_ACTIVE sums the 8 XCDs; "
                    "SQ_VALU_MFMA_BUSY_CYCLES sums the 1,024 SIMDs, in cycles; SQ_WAVE_CYCLES, "
                    "SQ_WAIT_* and SQ_ACTIVE_INST_* sum the resident waves, in units of 4 "
                    "cycles; SQ_INSTS_VALU counts the MFMA instructions too.\n\n")
            f.write(derived_table(argv[3:]) + "\n")
        print(dst)
    elif len(argv) >= 4 and argv[0] == "timeline":
        src, dst, cmd = argv[1], argv[2], argv[3]
        with open(dst, "w") as f:
            f.write(f"# Split-pass timelines per workgroup and XCD\n\nCommand:\n\n```\n{cmd}\n```\n\n"
                    f"Kernel sources hash: `{kernel_hash()}`\n\nTimes in us from the "
                    f"launch's first workgroup start (100 MHz constant clock).\n\n")
            f.write(timeline_table(src) + "\n")
        print(dst)
    elif len(argv) >= 4 and argv[0] == "table":
        src, dst, cmd = argv[1], argv[2], argv[3]
        with open(dst, "w") as f:
            f.write(f"# bench.py on every workload\n\nCommand (one per line of the table):\n\n"
                    f"```\n{cmd}\n```\n\nKernel sources hash: `{kernel_hash()}`\n\n")
            f.write(bench_table(src) + "\n\nRaw JSON lines:\n\n```\n")
            with open(src) as g:
                f.write("".join(ln for ln in g if ln.startswith("{")))
            f.write("```\n")
        print(dst)
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
