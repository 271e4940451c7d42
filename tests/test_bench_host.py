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


def _write_counter_csv(path, counter, copy_kib, fused_kib, fwd_kib=()):
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
        for v in fwd_kib:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": "rattn::attn_fwd16<__bf16, 4, 2>",
                        "Grid_Size": 589824, "Counter_Name": counter, "Counter_Value": v})
            d += 1


def test_pmc_summary_scales_by_the_copy(tmp_path, monkeypatch):
    # stand-in workloads, so the summary needs no real tensors
    fake = {n: types.SimpleNamespace(name=f"wl_{n}", B=2, N=3, H=1, dtype="bf16", total_kept=4)
            for n in bench.PMC_WORKLOADS}
    monkeypatch.setattr(bench.workloads, "by_name", lambda n: fake[n])
    copy_kib = 64 * 1024 * 1024 * 4 / 1024
    n = len(bench.PMC_WORKLOADS)
    # FETCH_SIZE reads half of the copy's bytes (scale 2), WRITE_SIZE all of them
    nf = len(bench.PMC_FORWARD_WORKLOADS)
    fetch = [float(10 * (i + 1)) for i in range(3 * n)]
    write = [float(5 * (i + 1)) for i in range(3 * n)]
    ffetch = [float(7 * (i + 1)) for i in range(3 * nf)]
    fwrite = [float(3 * (i + 1)) for i in range(3 * nf)]
    fp, wp = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _write_counter_csv(fp, "FETCH_SIZE", [copy_kib / 2] * 3, fetch, ffetch)
    _write_counter_csv(wp, "WRITE_SIZE", [copy_kib] * 3, write, fwrite)
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
    alg = bench.attention_bytes(4, 1, "bf16")
    for i, name in enumerate(bench.PMC_FORWARD_WORKLOADS):
        fk = sum(ffetch[3 * i:3 * i + 3]) / 3
        wk = sum(fwrite[3 * i:3 * i + 3]) / 3
        traffic = int(round((2 * fk + wk) * 1024))
        assert lines[3 + n + i] == (f"forward_wl_{name} fetch_kib {fk:.2f} write_kib {wk:.2f} "
                                    f"traffic_bytes {traffic} algorithmic_bytes {alg} "
                                    f"ratio {traffic / alg:.3f}")


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


# ---------------------------------------------------------------------------
# the other byte counts and the flop count, tallied item by item; the pages'
# FLOP figure at 80 % pruning
# ---------------------------------------------------------------------------
def _count_three_call_bytes(keep, H, es):
    """rattn_pack: the mask, and every kept q, k, v row read and written;
    rattn_forward: every kept q, k, v row read and o row written; rattn_unpack:
    the mask, every kept o row read, every padded output row and one CLS row
    per image written."""
    row = H * 64 * es
    total = 0
    for image in keep:
        total += len(image)                   # pack reads the mask
        total += len(image)                   # unpack reads it again
        for flag in image:
            if flag:
                total += 3 * 2 * row          # pack: q, k, v read and written
                total += 4 * row              # forward: q, k, v read, o written
                total += row                  # unpack: o row read
            total += row                      # unpack: padded row written
        total += row                          # unpack: CLS row written
    return total


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_three_call_bytes_matches_a_tally_over_the_mask(dtype):
    keep = [[1, 0, 1, 1], [0, 0, 0, 0], [1, 1, 0, 1]]
    T = sum(map(sum, keep))
    got = bench.three_call_bytes(T, len(keep), len(keep[0]), 3, dtype)
    assert got == _count_three_call_bytes(keep, 3, bench.ES[dtype])


def _count_repack_bytes(keep2_per_image, H, es):
    """rattn_repack of q, k and v: the second flag of every flat row read,
    every row kept again read and written in each tensor, the input
    cu_seqlens read and the output cu_seqlens written (int32, B + 1 each)."""
    row = H * 64 * es
    total = 0
    for flags in keep2_per_image:
        for f in flags:
            total += 1
            if f:
                total += 3 * 2 * row
    B = len(keep2_per_image)
    total += 4 * (B + 1) + 4 * (B + 1)
    return total


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_repack_bytes_matches_a_tally(dtype):
    flags = [[1, 0, 1], [0], [], [1, 1, 1, 0, 1]]
    T = sum(len(f) for f in flags)
    T2 = sum(map(sum, flags))
    got = bench.repack_bytes(T, T2, len(flags), 2, dtype)
    assert got == _count_repack_bytes(flags, 2, bench.ES[dtype])


def test_attention_flops_matches_a_tally_over_pairs():
    # per head, every (query, key) pair of the same image costs one 64-term dot
    # product (64 multiplies, 64 adds) and one 64-wide p * v accumulation
    # (64 multiplies, 64 adds)
    lengths, H = [3, 0, 1, 5], 2
    tally = 0
    for L in lengths:
        for _h in range(H):
            for _i in range(L):
                for _j in range(L):
                    tally += 2 * 64 + 2 * 64
    assert bench.attention_flops(lengths, H) == tally


def test_attention_flops_reproduce_the_pages_reduction_at_80pct_pruning():
    """The write-up's lead paragraph: 80 % token pruning cuts attention FLOPs
    by 96 %; its section on FlashAttention-2's dispatch ceiling: DeiT-Base goes
    from 197 to about 39 tokens per image.  The count here gives that figure
    for the pages' token counts and for the serving sweep's nominal 80 % count
    (round(0.2 * 196) patches plus CLS)."""
    import json
    import workloads
    with open(os.path.join(ROOT, "tests", "golden", "pages_numbers.json")) as f:
        items = json.load(f)["items"]
    tokens = next(i for i in items if "tokens_after_about" in i)
    flops = next(i for i in items if "attention_flop_reduction" in i)
    assert tokens["prune_rate"] == flops["prune_rate"] == 0.8
    B, H = 32, 12  # the write-up's DeiT-Base batch of 32
    full = bench.attention_flops([tokens["tokens_before"]] * B, H)
    for after in (tokens["tokens_after_about"], workloads.sweep_kept_count(0.8)):
        reduction = 1.0 - bench.attention_flops([after] * B, H) / full
        assert round(reduction, 2) == flops["attention_flop_reduction"], (after, reduction)
    # and the closed form (1 - p)^2 of the kept fraction
    assert round(1.0 - (1.0 - flops["prune_rate"]) ** 2, 2) == flops["attention_flop_reduction"]


def test_config_workload_names():
    """bench.py --config: every configuration by name, sweep points with their
    parameters, an explicit seed, and clear errors for malformed names."""
    cases = {"tiny": ("tiny", 4, 197, 3, "f32"), "deit_s": ("deit_s_80pct", 32, 197, 6, "f16"),
             "deit_b_384": ("deit_b_384_50pct", 64, 577, 12, "bf16"),
             "large_batch": ("large_batch_threshold_l2", 512, 197, 6, "bf16"),
             "deit_b_sweep:4:0.8": ("deit_b_sweep_B4_p80", 4, 197, 12, "bf16"),
             "deit_b_sweep:1:exact": ("deit_b_sweep_B1_unpruned_exact", 1, 197, 12, "bf16")}
    for spec, (name, B, N, H, dt) in cases.items():
        w = bench.config_workload(spec, None)
        assert (w.name, w.B, w.N, w.H, w.dtype) == (name, B, N, H, dt), spec
    a = bench.config_workload("deit_s", 123)
    b = bench.config_workload("deit_s", 124)
    assert a.seed == 123 and a.kept_counts != b.kept_counts
    for bad in ("nope", "deit_s:3", "deit_b_sweep:4"):
        with pytest.raises(SystemExit):
            bench.config_workload(bad, None)


def test_cold_trace_summary_takes_the_launches_after_the_eviction(tmp_path):
    """Attention launches that directly follow the eviction's reduction
    kernel count as cold, those that follow a launch of the same kernel as
    warm, the rest (after another kernel) as neither; each kernel gets its own
    medians."""
    fused = "void rattn::(anonymous namespace)::fused16<__bf16, 4, 2>(...)"
    fwd = "void rattn::(anonymous namespace)::attn_fwd16<__bf16, 4, 2>(...)"
    red = "void at::native::reduce_kernel<512, 1>(...)"
    fill = "void at::native::vectorized_elementwise_kernel<4, FillFunctor>(...)"
    seq = [(fused, 40), (fill, 9), (red, 30), (fused, 50), (fill, 9), (red, 30), (fused, 52),
           (fill, 9), (red, 30), (fused, 54), (fused, 41), (fwd, 35), (fill, 9), (red, 30),
           (fwd, 44)]
    path = tmp_path / "trace.csv"
    t = 1000
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, ["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        wr.writeheader()
        # rows out of start order, as a trace may list them
        rows = []
        for name, us in seq:
            rows.append({"Kernel_Name": name, "Start_Timestamp": t,
                         "End_Timestamp": t + us * 1000})
            t += us * 1000 + 500
        for r in reversed(rows):
            wr.writerow(r)
    out = bench.summarize_cold_trace(str(path)).splitlines()
    assert len(out) == 3
    by = {(ln.split()[0], ln.split(" kernel ")[1]): ln.split() for ln in out}
    f = by[("cold", fused)]
    assert f[2] == "3" and f[4] == "52.00" and f[6] == "50.00" and f[8] == "54.00"
    assert by[("warm", fused)][2:5] == ["1", "median_us", "41.00"]
    w = by[("cold", fwd)]
    assert w[2] == "1" and w[4] == "44.00"
