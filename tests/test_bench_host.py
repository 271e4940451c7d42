"""Host-side arithmetic of bench.py, on the CPU: the algorithmic byte counts
every roofline fraction divides by, the scaling of the traffic counters, the
lower bounds per launch, and the refusal of more than one GPU."""
import csv
import os
import subprocess
import sys
import types

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _count_fused_bytes(keep, H, es):
    """Byte count of one fused launch, tallied tensor by tensor over a keep
    mask: the mask itself, each kept position's q, k and v rows read once,
    every padded output row written once, and one CLS row per image."""
    row = H * 64 * es
    total = 0
    for image in keep:
        total += len(image)                       # mask bytes
        for flag in image:
            if flag:
                total += 3 * row                  # q, k, v rows of a kept token
            total += row                          # output row, kept or zero
        total += row                              # CLS row
    return total


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_fused_bytes_matches_a_tally_over_the_mask(dtype):
    keep = [[1, 0, 1], [0, 0, 1], [1, 1, 1]]
    T = sum(map(sum, keep))
    got = bench.fused_bytes(T, len(keep), len(keep[0]), 2, dtype)
    assert got == _count_fused_bytes(keep, 2, bench.ES[dtype])


def test_fused_bytes_of_a_small_case_by_hand():
    # B=2, N=3, H=1, bf16 (row = 128 B), 4 kept tokens:
    # 6 mask bytes + 3*4*128 + 6*128 + 2*128 = 6 + 1536 + 768 + 256
    assert bench.fused_bytes(4, 2, 3, 1, "bf16") == 2566


def test_attention_bytes():
    # q, k, v read and o written once: 4 tensors of T rows
    assert bench.attention_bytes(10, 12, "bf16") == 4 * 10 * 12 * 64 * 2


def _write_counter_csv(path, counter, copy_kib, fused_kib):
    cols = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        d = 1
        for v in copy_kib:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": "__amd_rocclr_copyBuffer",
                        "Grid_Size": 1 << 20, "Counter_Name": counter, "Counter_Value": v})
            d += 1
        for v in fused_kib:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": "rattn::fused16<__bf16, 4, 2>",
                        "Grid_Size": 196608, "Counter_Name": counter, "Counter_Value": v})
            d += 1


def test_pmc_summary_scales_by_the_copy(tmp_path, monkeypatch):
    # stand-in workloads, so the summary needs no real tensors
    fake = {n: types.SimpleNamespace(name=f"wl_{n}", B=2, N=3, H=1, dtype="bf16", total_kept=4)
            for n in bench.PMC_WORKLOADS}
    monkeypatch.setattr(bench.workloads, "by_name", lambda n: fake[n])
    copy_kib = 64 * 1024 * 1024 * 4 / 1024
    n = len(bench.PMC_WORKLOADS)
    # FETCH_SIZE reads half of the copy's bytes (scale 2), WRITE_SIZE all of them
    fetch = [float(10 * (i + 1)) for i in range(3 * n)]
    write = [float(5 * (i + 1)) for i in range(3 * n)]
    fp, wp = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _write_counter_csv(fp, "FETCH_SIZE", [copy_kib / 2] * 3, fetch)
    _write_counter_csv(wp, "WRITE_SIZE", [copy_kib] * 3, write)
    lines = bench.summarize_pmc(str(fp), str(wp)).splitlines()
    assert lines[0] == f"kernel_source_sha256 {bench.kernel_source_hash()}"
    assert lines[1] == "fetch_scale 2.0000" and lines[2] == "write_scale 1.0000"
    alg = bench.fused_bytes(4, 2, 3, 1, "bf16")
    for i, name in enumerate(bench.PMC_WORKLOADS):
        fk = sum(fetch[3 * i:3 * i + 3]) / 3
        wk = sum(write[3 * i:3 * i + 3]) / 3
        traffic = int(round((2 * fk + wk) * 1024))
        assert lines[3 + i] == (f"wl_{name} fetch_kib {fk:.2f} write_kib {wk:.2f} traffic_bytes "
                                f"{traffic} algorithmic_bytes {alg} ratio {traffic / alg:.3f}")


def test_pmc_summary_rejects_missing_dispatches(tmp_path):
    fp, wp = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _write_counter_csv(fp, "FETCH_SIZE", [131072.0], [1.0, 2.0])
    _write_counter_csv(wp, "WRITE_SIZE", [262144.0], [1.0, 2.0])
    with pytest.raises(RuntimeError):
        bench.summarize_pmc(str(fp), str(wp))


def test_roofs_us():
    # 8 GB at 8 TB/s is 1000 us; 2.5 GFLOP at 2.5 PFLOP/s is 1 us
    r = bench.roofs_us(8_000_000_000, 2_500_000_000, None, None)
    assert r == {"hbm": 1000.0, "mfma": 1.0}
    peaks = {"mfma_bf16_TFLOPs": 1250.0, "fma_exp2_per_s": 1e13}
    r = bench.roofs_us(8_000_000_000, 2_560_000_000, 4000.0, peaks)
    assert r["hbm_box"] == 2000.0
    assert r["mfma_box"] == pytest.approx(2.05, abs=0.01)
    # one fma + exp2 per score; 4 * 64 flops per score
    assert r["fma_exp2_box"] == pytest.approx(2_560_000_000 / 256 / 1e13 * 1e6, abs=0.01)


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
