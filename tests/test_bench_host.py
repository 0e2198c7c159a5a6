"""Host-side logic of bench.py (no GPU): the one-GPU guard, the rocprofv3 counter summary and
the rule that recorded counters count only for the kernel sources they were taken on."""
from __future__ import annotations

import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr


def test_source_hash_is_stable_and_short():
    h = bench.kernel_source_hash()
    assert h == bench.kernel_source_hash()
    assert len(h) == 16 and int(h, 16) >= 0


def _write_counter_csv(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "b_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for r in rows:
            w.writerow(r)


def test_pmc_summary_scales_by_the_copy_calibration(tmp_path, capsys):
    """A kernel that fetched 3 GiB-as-counted and wrote 1.5 GiB-as-counted per dispatch, with a
    calibration copy whose FETCH_SIZE reads half of its 2 GiB: bytes are scaled accordingly."""
    kib = 1024.0
    gib = 1 << 30
    name = "void psgd::(anonymous namespace)::k_decomp<1>(psgd::DevMat const*)"
    copy = "void at::native::vectorized_elementwise_kernel<4, neg>(int)"
    d = tmp_path
    _write_counter_csv(d / "pmc_FETCH_SIZE" / "x", [(1, name, "FETCH_SIZE", 3 * gib / kib),
                                                   (2, name, "FETCH_SIZE", 3 * gib / kib)])
    _write_counter_csv(d / "pmc_WRITE_SIZE" / "x", [(1, name, "WRITE_SIZE", 1.5 * gib / kib)])
    _write_counter_csv(d / "pmccopy_FETCH_SIZE" / "x", [(i, copy, "FETCH_SIZE", 1 * gib / kib) for i in range(3)])
    _write_counter_csv(d / "pmccopy_WRITE_SIZE" / "x", [(i, copy, "WRITE_SIZE", 2 * gib / kib) for i in range(3)])
    assert bench.pmc_summary(str(d)) == 0
    out = capsys.readouterr().out
    line = next(l for l in out.splitlines() if l.startswith("TRAFFIC decompress"))
    f = line.split()
    assert int(f[4]) == 6 * gib           # fetch: 3 GiB counted x 2 (the copy's scale)
    assert int(f[6]) == int(1.5 * gib)    # write: scale 1
    assert int(f[2]) == 6 * gib + int(1.5 * gib)
    assert f[8] == bench.kernel_source_hash()


def test_recorded_figures_need_matching_sources(tmp_path, monkeypatch):
    f = tmp_path / "traffic.txt"
    f.write_text("TRAFFIC decompress 123 fetch 100 write 23 source 0000000000000000\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.recorded_traffic("decompress") is None
    f.write_text(f"TRAFFIC decompress 123 fetch 100 write 23 source {bench.kernel_source_hash()}\n")
    assert bench.recorded_traffic("decompress") == 123


@pytest.mark.parametrize("mode", ["default", "block"])
def test_parse_defaults(mode):
    a = bench.parse([] if mode == "default" else ["--block-scaling"])
    assert a.gpus == 1 and a.workload == 3 and a.steps > 0 and a.warmup >= 3
    assert a.block_scaling == (mode == "block")


def test_lds_summary_ratio(tmp_path, capsys):
    """The LDS table divides conflict cycles by indexed-access cycles, per kernel, over the
    launches that used the LDS."""
    name = "void psgd::(anonymous namespace)::k_ef_mq<1, 7>(psgd::DevMat const*)"
    _write_counter_csv(tmp_path / "pmc_LDS" / "x", [
        (1, name, "SQ_LDS_BANK_CONFLICT", 30.0), (1, name, "SQ_LDS_IDX_ACTIVE", 100.0),
        (1, name, "SQ_INSTS_LDS", 2e6),
        (2, name, "SQ_LDS_BANK_CONFLICT", 10.0), (2, name, "SQ_LDS_IDX_ACTIVE", 100.0),
        (2, name, "SQ_INSTS_LDS", 4e6)])
    assert bench.pmc_summary(str(tmp_path)) == 0
    row = next(l for l in capsys.readouterr().out.splitlines() if l.startswith("k_ef_mq<1, 7>"))
    f = row.split()
    assert f[2] == "2" and float(f[3]) == pytest.approx(0.2) and float(f[5]) == pytest.approx(3.0)


def test_pmc_summary_needs_some_counter_run(tmp_path):
    assert bench.pmc_summary(str(tmp_path)) == 1


def test_trace_summary_counts_steps_and_splits_the_two_gemms(tmp_path, capsys):
    """Steps are counted by the finite check; k_gemm_nt launches alternate between M q and
    M^T P_hat; per-step times are totals over the steps."""
    p = tmp_path / "b_kernel_trace.csv"
    ns = 0
    rows = []
    def add(kernel, us):
        nonlocal ns
        rows.append({"Kernel_Name": f"void psgd::(anonymous namespace)::{kernel}(int)",
                     "Start_Timestamp": ns, "End_Timestamp": ns + int(us * 1000)})
        ns += int(us * 1000) + 10
    for _ in range(3):
        add("k_gemm_nt", 100.0)
        add("k_gemm_nt", 50.0)
        add("k_check_finite", 2.0)
        rows.append({"Kernel_Name": "void at::native::other(int)", "Start_Timestamp": ns,
                     "End_Timestamp": ns + 5})
    with open(p, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        w.writerows(rows)
    assert bench.trace_summary(str(p)) == 0
    out = capsys.readouterr().out
    assert out.startswith("3 steps")
    mq = next(l for l in out.splitlines() if l.startswith("| k_gemm_nt (M q)"))
    mtp = next(l for l in out.splitlines() if l.startswith("| k_gemm_nt (M^T P_hat)"))
    assert mq.split("|")[2].strip() == "3" and float(mq.split("|")[3]) == pytest.approx(100.0)
    assert float(mtp.split("|")[4]) == pytest.approx(0.05)
