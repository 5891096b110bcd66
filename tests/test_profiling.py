"""Host logic of the measurement tooling (no GPU): rocprofv3 CSV summaries, the
counter-calibrated traffic per launch, the bench table, bench.py's lookup of stored
traffic by workload and pool format, and its default step counts."""
import csv
import importlib.util
import json
import os

import pytest

from mla_latent_kv_16_amd import profiling as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _write_counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for k, c, v in rows:
            w.writerow({"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_kernel_hash_is_stable_hex():
    h = P.kernel_hash()
    assert len(h) == 16 and int(h, 16) >= 0
    assert P.kernel_hash() == h


def test_traffic_scales_each_counter_by_the_copy_probe(tmp_path):
    kib = P.COPY_PROBE_BYTES / 1024
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    # the copy probe reads half its bytes on FETCH_SIZE and all of them on WRITE_SIZE;
    # a small copy kernel of the same name is ignored (only the largest dispatches count)
    _write_counters(fetch, [("__amd_rocclr_copyBuffer", "FETCH_SIZE", kib / 2),
                            ("__amd_rocclr_copyBuffer", "FETCH_SIZE", kib / 2),
                            ("__amd_rocclr_copyBuffer", "FETCH_SIZE", 3.0),
                            ("void mla::splitkv_kernel<mla::Bf16Kv>(mla::SplitArgs)",
                             "FETCH_SIZE", 1000.0),
                            ("void mla::splitkv_kernel<mla::Bf16Kv>(mla::SplitArgs)",
                             "FETCH_SIZE", 3000.0),
                            ("mla::combine_kernel(mla::CombineArgs)", "FETCH_SIZE", 50.0)])
    _write_counters(write, [("__amd_rocclr_copyBuffer", "WRITE_SIZE", kib),
                            ("void mla::splitkv_kernel<mla::Bf16Kv>(mla::SplitArgs)",
                             "WRITE_SIZE", 400.0),
                            ("mla::combine_kernel(mla::CombineArgs)", "WRITE_SIZE", 8.0)])
    r = P.traffic(str(fetch), str(write), "spec4", "cmd")
    assert r["fetch_scale"] == pytest.approx(2.0) and r["write_scale"] == pytest.approx(1.0)
    assert r["split_fetch_bytes"] == pytest.approx(2000.0 * 1024 * 2.0)
    assert r["split_write_bytes"] == pytest.approx(400.0 * 1024)
    assert r["combine_fetch_bytes"] == pytest.approx(50.0 * 1024 * 2.0)
    assert r["kernel_hash"] == P.kernel_hash()


def test_bench_table_renders_a_row(tmp_path):
    rec = {"value": 3853.5, "us_per_step": 78.4, "us_per_step_graph_replay": 83.1,
           "kv_frac_of_hbm_peak": 0.4817, "split_pass_us": 69.3,
           "split_kernel_us_back_to_back": 66.1, "single_pass_us_per_step": None,
           "config": {"workload": "spec4", "latent": "512+64 e4m3, per-tensor scale"},
           "roofline": {"bound": "hbm", "achieved": 4369.2, "unit": "GB/s", "frac": 0.5462,
                        "frac_of_measured_peak": 0.88},
           "cpu_baseline": None}
    src = tmp_path / "b.jsonl"
    src.write_text("noise\n" + json.dumps(rec) + "\n")
    table = P.bench_table(str(src))
    rows = table.splitlines()
    assert len(rows) == 3
    cells = [c.strip() for c in rows[2].strip("|").split("|")]
    assert cells[:3] == ["spec4", "e4m3", "78.4"]
    assert cells[7] == "—" and cells[-1] == "—"
    assert "4369.2 GB/s (54.6%)" in rows[2]


def test_stored_traffic_follows_the_pool_format():
    """bench.py reports stored HBM traffic only for the pool format and kernel sources
    the counters were taken on: a NoPE pool reads its own file (never the bf16 pool's),
    and a format without counters gets none."""
    b = _bench()

    def expect(tag):
        path = os.path.join(ROOT, "profiles", f"traffic_{tag}.json")
        if not os.path.exists(path):
            return None
        with open(path) as f:
            rec = json.load(f)
        if rec["kernel_hash"] != P.kernel_hash():
            return None
        return int(rec["split_fetch_bytes"] + rec["split_write_bytes"])

    assert b.stored_traffic("spec4", "bf16") == expect("spec4")
    assert b.stored_traffic("spec4", "nope") == expect("spec4_nope")
    if expect("spec4") is not None and expect("spec4_nope") is not None:
        assert expect("spec4_nope") < expect("spec4")  # 1,024- against 1,152-byte rows
    assert b.stored_traffic("spec4", "e4m3") == expect("spec4_e4m3")
    assert b.stored_traffic("spec8", "e4m3") is None  # no counters taken for it
    assert b.stored_traffic("no-such-workload", "bf16") is None


def test_cpu_baseline_names_its_host():
    b = _bench()
    model, blas = b.host_cpu_model(), b.blas_name()
    assert model is None or (isinstance(model, str) and model)
    assert blas is None or (isinstance(blas, str) and blas)


def test_default_step_counts_follow_the_step_time():
    """Without --steps/--warmup the bench warms up for at least 50 ms and times at least
    0.2 s of steps, never fewer than the floors; explicit counts are kept exactly."""
    b = _bench()
    steps, warmup = b.default_counts(76e-6)  # a spec4 step
    assert steps == 2632 and warmup == 658
    assert steps * 76e-6 >= b.TIMED_SECONDS and warmup * 76e-6 >= b.WARMUP_SECONDS
    assert b.default_counts(10e-3) == (200, 20)  # a prefill step: the floors
    assert b.default_counts(1.15e-3, min_steps=100, min_warmup=50) == (174, 50)
    assert b.default_counts(76e-6, steps=50, warmup=5) == (50, 5)
    assert b.default_counts(76e-6, steps=7) == (7, 658)
    assert b.default_counts(0.0)[0] >= 200  # a zero estimate cannot divide by zero
