"""Host-side logic of bench.py: the HBM-traffic summary of rocprofv3 counter
files (no GPU; synthetic counter CSVs)."""
import csv
import importlib.util
import json
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _counters(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_summary_scales_by_the_copy_probe(tmp_path):
    b = _bench()
    kib = b.COPY_PROBE_BYTES / 1024.0
    # the fetch counter reads half the bytes on this part: the probe's sum shows
    # kib / 2, a kernel that truly reads 3 x 1 GiB shows 1.5 GiB; the write
    # counter reads true bytes: the probe's fill shows kib, and neither the
    # 1 GiB cache flush (twice the probe) nor the clock-ramp fills (192 MiB)
    # nor a half-size fill next to the full-size probe may be taken as it;
    # the rope instantiation of the kernel is not the one summarized
    fetch = tmp_path / "fetch.csv"
    _counters(fetch, "FETCH_SIZE", [
        ("void at::native::reduce_kernel<512, 1>", kib / 2),
        ("csa2::attend_mq_kernel<false>(MqArgs)", 1.5 * 1024 * 1024),
        ("csa2::attend_mq_kernel<false>(MqArgs)", 1.5 * 1024 * 1024),
        ("csa2::attend_mq_kernel<true>(MqArgs)", 9.0 * 1024 * 1024),
        ("void at::native::vectorized_elementwise_kernel<FillFunctor>", 10.0),
    ])
    write = tmp_path / "write.csv"
    _counters(write, "WRITE_SIZE", [
        ("void at::native::vectorized_elementwise_kernel<FillFunctor>", kib),
        ("void at::native::vectorized_elementwise_kernel<FillFunctor>", kib / 2),
        ("void at::native::vectorized_elementwise_kernel<FillFunctor>", 192.0 * 1024),
        ("void at::native::vectorized_elementwise_kernel<FillFunctor>", 2 * kib),
        ("csa2::attend_mq_kernel<false>(MqArgs)", 512.0 * 1024),
        ("csa2::attend_mq_kernel<false>(MqArgs)", 512.0 * 1024),
    ])
    out = tmp_path / "rec.json"
    name, _, src, workload, args = b.TRAFFIC_KERNELS["attend"]
    b.TRAFFIC_KERNELS["attend"] = (name, str(out), src, workload, args)
    b.summarize_traffic(str(fetch), str(write), which="attend")
    rec = json.load(open(out))
    assert rec["kernel"] == "attend_mq_kernel<false>"
    assert abs(rec["fetch"]["scale"] - 2.0) < 1e-12 and rec["write"]["scale"] == 1.0
    assert rec["hbm_bytes_per_launch"] == 3 * (1 << 30) + (512 << 20)
    assert rec["kernel_source_sha256_16"] == b.source_digest(src)
    # a record taken on the current source is used, a stale one is not
    assert b.traffic_from_profile("attend") == rec["hbm_bytes_per_launch"]
    rec["kernel_source_sha256_16"] = "0" * 16
    json.dump(rec, open(out, "w"))
    assert b.traffic_from_profile("attend") is None


def test_cpu_baseline_reports_cores_model_and_one_thread():
    b = _bench()
    calls = []

    def run(i):
        calls.append(i)
        sum(range(20000))

    rec = b.cpu_baseline(run, 8, "a test sample", min_seconds=0.05, single_seconds=0.02)
    assert rec["kind"] == "oracle" and rec["unit"] == "queries/s" and rec["value"] > 0
    assert rec["cores"] >= 1 and rec["cpu_model"]
    assert rec["single_thread"]["value"] > 0
