"""bench.py's host-side record keeping (no GPU): traffic records from
rocprofv3 counter files, the request-count cross-check, source hashes."""

import csv
import json
import os
import sys
import time

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def write_counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for k, c, v in rows:
            w.writerow({"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


@pytest.fixture
def profiles_dir(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    return tmp_path


def test_traffic_record_scales_by_the_copy_calibration(tmp_path, profiles_dir):
    kern = "void pa::decode_partitions_kernel<pa::TF16, 128, 4, false>(DecodeArgs)"
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    cfetch, cwrite = tmp_path / "cf.csv", tmp_path / "cw.csv"
    write_counters(fetch, [(kern, "FETCH_SIZE", 1000.0), (kern, "FETCH_SIZE", 1200.0),
                           ("other", "FETCH_SIZE", 9e9)])
    write_counters(write, [(kern, "WRITE_SIZE", 10.0)])
    # The copy reads 1 GiB but FETCH_SIZE reports half of it: factor 2.
    write_counters(cfetch, [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 524288.0)])
    write_counters(cwrite, [("__amd_rocclr_copyBuffer", "WRITE_SIZE", 1048576.0)])
    bench.write_traffic("decode_partitions", "wl", str(fetch), str(write), str(cfetch),
                        str(cwrite))
    rec = json.load(open(profiles_dir / "decode_partitions_wl_traffic.json"))
    assert rec["fetch_bytes"] == round(1100.0 * 1024 * 2)
    assert rec["write_bytes"] == round(10.0 * 1024)
    assert rec["scale_factor"] == {"fetch": 2.0, "write": 1.0}
    assert rec["dispatches"] == [2, 1]
    # bench.py reports the record only while the kernel's code is unchanged.
    alg = 2_000_000
    got = bench.load_traffic("decode_partitions", "wl", rec["source_hash"], alg)
    assert got["ratio_to_algorithmic"] == round((rec["fetch_bytes"] + rec["write_bytes"]) / alg, 4)
    assert bench.load_traffic("decode_partitions", "wl", "0" * 16, alg) is None

    # Request-count cross-check: 128/64/32-byte read requests give bytes
    # without the FETCH_SIZE factor.
    rq, crq = tmp_path / "rq.csv", tmp_path / "crq.csv"
    write_counters(rq, [(kern, "TCC_EA0_RDREQ_32B", 0), (kern, "TCC_EA0_RDREQ_64B", 100),
                        (kern, "TCC_EA0_RDREQ_128B", 17550), (kern, "TCC_EA0_RDREQ", 17650)])
    write_counters(crq, [("__amd_rocclr_copyBuffer", "TCC_EA0_RDREQ_32B", 0),
                         ("__amd_rocclr_copyBuffer", "TCC_EA0_RDREQ_64B", 0),
                         ("__amd_rocclr_copyBuffer", "TCC_EA0_RDREQ_128B", 8388608),
                         ("__amd_rocclr_copyBuffer", "TCC_EA0_RDREQ", 8388608)])
    bench.rdreq_check("decode_partitions", "wl", str(rq), str(crq))
    x = json.load(open(profiles_dir / "decode_partitions_wl_traffic.json"))["rdreq_cross_check"]
    assert x["read_bytes_from_request_counts"] == 100 * 64 + 17550 * 128
    assert x["copy_read_bytes_over_1GiB"] == 1.0
    assert x["over_scaled_fetch_bytes"] == round((100 * 64 + 17550 * 128) / rec["fetch_bytes"], 4)


def test_source_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    csrc = tmp_path / "paged_kv_cache_decode_amd" / "csrc"
    csrc.mkdir(parents=True)
    files = ("decode.hip", "decode_kernel.h", *bench.SHARED_HEADERS)
    for n in files:
        (csrc / n).write_text("int x = 1;  // a comment\n/* block\ncomment */ int y = 2;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.source_hash("decode.hip")
    (csrc / "decode.hip").write_text("int x = 1;  // another comment\n\n/* other */ int y = 2;\n")
    assert bench.source_hash("decode.hip") == h0
    (csrc / "decode.hip").write_text("int x = 1;\nint y = 3;\n")
    assert bench.source_hash("decode.hip") != h0


def test_spread_reports_median_and_deciles():
    s = bench.spread_us([i / 1000.0 for i in range(1, 102)])  # 1 .. 101 us
    assert s == {"median": 51.0, "p10": 11.0, "p90": 91.0, "n": 101}
    assert bench.spread_us([]) is None


def test_blas_threads_from_host_info():
    assert bench.blas_threads({"blas": [{"library": "openblas", "threads": 16}]}) == 16
    assert bench.blas_threads({"blas": "unavailable: x"}) == 1
    info = bench.host_info()
    assert info["os_cpu_count"] >= 1 and info["affinity_cpus"] >= 1


def test_more_than_one_gpu_is_refused(monkeypatch, capsys):
    monkeypatch.setattr(sys, "argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().err


def test_warm_up_counts_and_time():
    """Exactly `steps` calls without a time floor; with one, more calls in
    groups of 10 until the floor has passed (each group synchronised)."""
    class FakeCuda:
        syncs = 0

        @classmethod
        def synchronize(cls):
            cls.syncs += 1

    class FakeTorch:
        cuda = FakeCuda

    calls = []
    bench.warm_up(FakeTorch, calls.append, 7, 0.0)
    assert calls == list(range(7)) and FakeCuda.syncs == 1
    calls.clear()
    FakeCuda.syncs = 0
    t0 = time.perf_counter()
    bench.warm_up(FakeTorch, lambda i: (calls.append(i), time.sleep(0.001)), 3, 0.05)
    assert time.perf_counter() - t0 >= 0.05
    assert calls == list(range(len(calls))) and len(calls) >= 13 and (len(calls) - 3) % 10 == 0
    assert FakeCuda.syncs == 1 + (len(calls) - 3) // 10
