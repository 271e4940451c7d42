"""Benchmark of the ragged pack -> attend -> unpack path on one MI355X.

One step = one pass of the whole hot path over one batch: the per-image kept
token ranks (the cu_seqlens scan), the gather of the kept q/k/v rows, the
bidirectional ragged attention, and the scatter to the padded output plus the
CLS rows -- all in ONE launch, `rattn_fused`, called through the Python
binding.  The default workload is the DeiT-S shape at 80 % token pruning (B=32,
N=197, H=6, head_dim 64, fp16), the setting the metric "ragged attn seqs/s +
us/call at 80% pruning" is quoted on.  Inputs are seeded synthetic tensors
already resident in HBM when the timed region starts.

Printed: ONE JSON line with the throughput (images/s), the fused kernel's
HIP-event duration and roofline, the CPU oracle timed on this host, and
(unless --quick) the per-call dispatch floors at batch 1-4 measured from C++
and the large-configuration kernels against the HBM roof.

Pages on "Dispatch-Aware Ragged Attention for Pruned Vision Transformers"
(arXiv 2604.15408): the paper abstract (dispatch floor, kernel latency at 80 %
pruning, serving batch sizes 1-4) and the radpulse.milrad-way.com write-up
(sections on FlashAttention-2's dispatch ceiling, the Triton kernel and the
integrated packing pipeline).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402
from ragged_variable_length_amd import (FusedPlan, RaggedPipeline, rattn_forward,  # noqa: E402
                                        rattn_fused, rattn_init)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, datasheet
# HBM traffic of the fused kernel measured with rocprofv3 counters (FETCH_SIZE,
# WRITE_SIZE); valid only for the kernel sources it was taken on
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "rattn_fused_hbm_traffic.txt")
KERNEL_SOURCES = ("ragged_variable_length_amd/csrc/attention.hip",
                  "ragged_variable_length_amd/csrc/internal.h")
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "f32": 157.3}  # dense
ES = {"f32": 4, "f16": 2, "bf16": 2}
METRIC = "ragged attn seqs/s + us/call at 80% pruning; % of MFMA/HBM roofline"


# ---------------------------------------------------------------------------
# algorithmic work of one launch: what the method must move / compute
# ---------------------------------------------------------------------------
def fused_bytes(T: int, B: int, N: int, H: int, dtype: str) -> int:
    """keep mask read; kept q, k, v rows read once; the padded output (kept
    rows and zero rows) and the CLS rows written once."""
    row = H * 64 * ES[dtype]
    return B * N + 3 * T * row + B * N * row + B * row


def attention_bytes(T: int, H: int, dtype: str) -> int:
    """the attention alone on a flat buffer: q, k, v read and o written once."""
    return 4 * T * H * 64 * ES[dtype]


def three_call_bytes(T: int, B: int, N: int, H: int, dtype: str) -> int:
    """rattn_pack (mask read, 3 kept rows read and written), rattn_forward
    (attention_bytes) and rattn_unpack (mask read, T rows read, the padded
    output and the CLS rows written)."""
    row = H * 64 * ES[dtype]
    pack = B * N + 2 * 3 * T * row
    unpack = B * N + T * row + B * N * row + B * row
    return pack + attention_bytes(T, H, dtype) + unpack


def repack_bytes(T: int, T2: int, B: int, H: int, dtype: str) -> int:
    """rattn_repack of q, k, v: the second keep flag of every row read, the
    kept rows read and written once, both cu_seqlens."""
    row = H * 64 * ES[dtype]
    return T + 2 * 3 * T2 * row + 2 * 4 * (B + 1)


def attention_flops(lengths, H: int) -> int:
    """QK^T and PV: 2 * 2 * 64 flops per (query, key) pair per head."""
    return 4 * 64 * H * sum(L * L for L in lengths)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """Bytes per launch from the committed counter summary, or None when the
    kernel sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            lines = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    except OSError:
        return None
    rec = {ln[0]: ln[1:] for ln in lines}
    if rec.get("kernel_source_sha256", [None])[0] != kernel_source_hash():
        return None
    row = rec.get(workload)
    if row is None or "traffic_bytes" not in row:
        return None
    return int(row[row.index("traffic_bytes") + 1])


PMC_WORKLOADS = ("deit_s", "deit_b_384", "large_batch")
# workloads whose rattn_forward launches are counted too (the attention alone
# on flat buffers, against attention_bytes)
PMC_FORWARD_WORKLOADS = ("deit_b_384", "large_batch")


def summarize_pmc(fetch_csv: str, write_csv: str) -> str:
    """Summary text of two rocprofv3 --pmc runs of `bench.py --pmc-target`
    (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch).  Each counter is scaled
    by what it reads for the 256 MiB copy, and the three launches of each
    workload are averaged."""
    import csv

    def per_kernel(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        copies = [float(r["Counter_Value"]) for r in rows
                  if "copyBuffer" in r["Kernel_Name"] and int(r["Grid_Size"]) > 100000]
        fused = [float(r["Counter_Value"]) for r in rows if "fused16" in r["Kernel_Name"]]
        fwd = [float(r["Counter_Value"]) for r in rows if "attn_fwd16" in r["Kernel_Name"]]
        return copies, fused, fwd

    copy_bytes = 64 * 1024 * 1024 * 4
    fc, ff, fwf = per_kernel(fetch_csv, "FETCH_SIZE")
    wc, wf, fww = per_kernel(write_csv, "WRITE_SIZE")
    if (len(ff) != 3 * len(PMC_WORKLOADS) or len(wf) != len(ff) or not fc or not wc
            or len(fwf) != 3 * len(PMC_FORWARD_WORKLOADS) or len(fww) != len(fwf)):
        raise RuntimeError("unexpected dispatches in the counter files")
    f_scale = copy_bytes / 1024.0 / (sum(fc) / len(fc))
    w_scale = copy_bytes / 1024.0 / (sum(wc) / len(wc))
    out = [f"kernel_source_sha256 {kernel_source_hash()}",
           f"fetch_scale {f_scale:.4f}",
           f"write_scale {w_scale:.4f}"]
    for i, name in enumerate(PMC_WORKLOADS):
        w = workloads.by_name(name)
        T = w.total_kept
        alg = fused_bytes(T, w.B, w.N, w.H, w.dtype)
        fk = sum(ff[3 * i:3 * i + 3]) / 3.0
        wk = sum(wf[3 * i:3 * i + 3]) / 3.0
        traffic = int(round((fk * f_scale + wk * w_scale) * 1024.0))
        out.append(f"{w.name} fetch_kib {fk:.2f} write_kib {wk:.2f} traffic_bytes {traffic} "
                   f"algorithmic_bytes {alg} ratio {traffic / alg:.3f}")
    for i, name in enumerate(PMC_FORWARD_WORKLOADS):
        w = workloads.by_name(name)
        alg = attention_bytes(w.total_kept, w.H, w.dtype)
        fk = sum(fwf[3 * i:3 * i + 3]) / 3.0
        wk = sum(fww[3 * i:3 * i + 3]) / 3.0
        traffic = int(round((fk * f_scale + wk * w_scale) * 1024.0))
        out.append(f"forward_{w.name} fetch_kib {fk:.2f} write_kib {wk:.2f} traffic_bytes "
                   f"{traffic} algorithmic_bytes {alg} ratio {traffic / alg:.3f}")
    return "\n".join(out) + "\n"


def pmc_target() -> None:
    """Launches for the traffic counters (run under rocprofv3 --pmc): a plain
    256 MiB device copy for calibration, then three rattn_fused launches on
    each of the DeiT-S 80 %, DeiT-B 384 px and batch-512 workloads, and three
    rattn_forward launches on the flat buffers of the last two."""
    rattn_init()
    stream = torch.cuda.current_stream()
    src = torch.randn(64 * 1024 * 1024, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[pmc] copy of {src.numel() * 4} bytes x3", flush=True)
    del src, dst
    for name in PMC_WORKLOADS:
        r = Resident(workloads.by_name(name), stream)
        for _ in range(3):
            r.step()
        torch.cuda.synchronize()
        print(f"[pmc] {r.w.name}: rattn_fused x3, algorithmic bytes "
              f"{fused_bytes(r.T, r.w.B, r.w.N, r.w.H, r.w.dtype)}", flush=True)
        del r
    for name in PMC_FORWARD_WORKLOADS:
        f = FlatResident(workloads.by_name(name), stream)
        step = f.c_step()
        if timing_lib().bench_loop(ctypes.byref(step), WHAT_FORWARD, 3) != 0:
            raise RuntimeError("bench_loop(rattn_forward) failed")
        torch.cuda.synchronize()
        print(f"[pmc] {f.w.name}: rattn_forward x3, algorithmic bytes "
              f"{attention_bytes(f.w.total_kept, f.w.H, f.w.dtype)}", flush=True)
        del f


def pmc_forward(name: str) -> None:
    """Five rattn_forward launches on one workload's flat buffers, prepared on
    the host (run under rocprofv3 --pmc for the SQ counters of the attention
    loop)."""
    rattn_init()
    stream = torch.cuda.current_stream()
    f = FlatResident(workloads.by_name(name), stream)
    step = f.c_step()
    if timing_lib().bench_loop(ctypes.byref(step), WHAT_FORWARD, 5) != 0:
        raise RuntimeError("bench_loop(rattn_forward) failed")
    torch.cuda.synchronize()
    print(f"[pmc] {f.w.name}: rattn_forward x5", flush=True)


# ---------------------------------------------------------------------------
# C++ timing helper (host clock around call + sync; no interpreter in the loop)
# ---------------------------------------------------------------------------
class BenchStats(ctypes.Structure):
    _fields_ = [("median_us", ctypes.c_double), ("p5_us", ctypes.c_double),
                ("p95_us", ctypes.c_double), ("mean_us", ctypes.c_double),
                ("min_us", ctypes.c_double)]

    def as_dict(self):
        return {k: round(getattr(self, k), 2) for k, _ in self._fields_}


class BenchPeaks(ctypes.Structure):
    """bench_peaks_result of bench_peaks.hip."""
    _fields_ = [("mfma_bf16_tflops", ctypes.c_double), ("fma_exp_per_s", ctypes.c_double),
                ("exp_per_s", ctypes.c_double), ("fma_f32_tflops", ctypes.c_double),
                ("mfma_ns", ctypes.c_double), ("mfma_exp_ns", ctypes.c_double),
                ("split_mixed_s", ctypes.c_double), ("split_mfma_s", ctypes.c_double),
                ("split_valu_s", ctypes.c_double)]


class BenchStep(ctypes.Structure):
    _fields_ = [("src", ctypes.c_void_p * 3), ("packed", ctypes.c_void_p * 3),
                ("o", ctypes.c_void_p), ("out_padded", ctypes.c_void_p),
                ("cls", ctypes.c_void_p), ("keep", ctypes.c_void_p), ("cu", ctypes.c_void_p),
                ("max_dev", ctypes.c_void_p), ("total_dev", ctypes.c_void_p),
                ("B", ctypes.c_int), ("N", ctypes.c_int), ("H", ctypes.c_int),
                ("max_seqlen", ctypes.c_int), ("dtype", ctypes.c_int), ("scale", ctypes.c_float),
                ("stream", ctypes.c_void_p), ("layers", ctypes.c_int),
                ("out_padded2", ctypes.c_void_p), ("keep2", ctypes.c_void_p),
                ("cu2", ctypes.c_void_p), ("repacked", ctypes.c_void_p * 3)]


WHAT_FORWARD = 0
WHAT_THREE_CALL = 1
WHAT_FUSED = 2
WHAT_LAYERS_PACKED = 3
WHAT_LAYERS_FUSED = 4
WHAT_REPACK = 5
REPACK_KEEP = 0.5   # fraction of the packed rows a second pruning stage keeps
STACK_LAYERS = 12   # DeiT-S / DeiT-B depth
_DT_CODE = {"f32": 0, "f16": 1, "bf16": 2}
_timing = None


def timing_lib():
    global _timing
    if _timing is None:
        path = os.path.join(ROOT, "ragged_variable_length_amd", "librattn_bench.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built (run __graft_entry__.build())")
        lib = ctypes.CDLL(path)
        P, i32 = ctypes.c_void_p, ctypes.c_int
        step, stats = ctypes.POINTER(BenchStep), ctypes.POINTER(BenchStats)
        lib.bench_empty_floor.argtypes = [i32, i32, P, stats]
        lib.bench_call_floor.argtypes = [step, i32, i32, i32, stats]
        lib.bench_enqueue_cost.argtypes = [step, i32, i32, stats]
        lib.bench_graph_floor.argtypes = [step, i32, i32, i32, stats]
        lib.bench_graph_enqueue_cost.argtypes = [step, i32, i32, stats]
        lib.bench_loop.argtypes = [step, i32, i32]
        lib.bench_peaks.argtypes = [i32, i32, P, ctypes.POINTER(BenchPeaks)]
        for f in (lib.bench_empty_floor, lib.bench_call_floor, lib.bench_enqueue_cost,
                  lib.bench_graph_floor, lib.bench_graph_enqueue_cost, lib.bench_loop,
                  lib.bench_peaks):
            f.restype = i32
        _timing = lib
    return _timing


class Resident:
    """A workload moved to the GPU plus its output buffers."""

    def __init__(self, w, stream):
        self.w = w
        dev = torch.device("cuda")
        self.q, self.k, self.v = (t.to(dev) for t in (w.q, w.k, w.v))
        self.keep = w.keep.to(dev)
        self.out = torch.empty_like(self.q)
        self.cls = torch.empty((w.B, w.H, w.D), dtype=self.q.dtype, device=dev)
        self.stream = stream
        self.lengths = w.kept_counts
        self.T = sum(self.lengths)
        torch.cuda.synchronize()  # inputs resident before any stream uses them
        self.plan = FusedPlan(self.q, self.k, self.v, self.keep, w.scale, out_padded=self.out,
                              cls=self.cls, stream=stream)
        self.step = self.plan.run

    def c_step(self) -> BenchStep:
        s = BenchStep()
        for i, t in enumerate((self.q, self.k, self.v)):
            s.src[i] = t.data_ptr()
        s.out_padded, s.cls = self.out.data_ptr(), self.cls.data_ptr()
        s.keep = self.keep.data_ptr()
        s.B, s.N, s.H, s.max_seqlen = self.w.B, self.w.N, self.w.H, self.w.N
        s.dtype, s.scale = _DT_CODE[self.w.dtype], self.w.scale
        s.stream = self.stream.cuda_stream
        return s


class FlatResident:
    """The flat ragged buffers of a workload (kept rows in order, prepared on
    the host) and cu_seqlens, resident on the GPU, for rattn_forward alone."""

    def __init__(self, w, stream):
        self.w = w
        dev = torch.device("cuda")
        keep = w.keep != 0
        self.flat = [t[keep].contiguous().to(dev) for t in (w.q, w.k, w.v)]
        self.o = torch.empty_like(self.flat[0])
        cu = torch.zeros(w.B + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(keep.sum(dim=1), 0).to(torch.int32)
        self.cu = cu.to(dev)
        self.stream = stream
        torch.cuda.synchronize()

    def c_step(self) -> BenchStep:
        s = BenchStep()
        for i, t in enumerate(self.flat):
            s.packed[i] = t.data_ptr()
        s.o, s.cu = self.o.data_ptr(), self.cu.data_ptr()
        s.B, s.N, s.H, s.max_seqlen = self.w.B, self.w.N, self.w.H, self.w.N
        s.dtype, s.scale = _DT_CODE[self.w.dtype], self.w.scale
        s.stream = self.stream.cuda_stream
        return s


class StackResident:
    """A Resident plus the flat buffers of the three-call form (RaggedPipeline)
    and a second padded buffer, for the three-call step and the layer stacks."""

    def __init__(self, r: Resident, layers: int = STACK_LAYERS):
        self.r = r
        w = r.w
        self.pipe = RaggedPipeline(w.B, w.N, w.H, r.q.dtype)
        self.out2 = torch.empty_like(r.out)
        self.layers = layers
        g = torch.Generator().manual_seed(11)
        cap = self.pipe.pq.shape[0]
        self.keep2 = (torch.rand(cap, generator=g) < REPACK_KEEP).to(torch.uint8).to("cuda")
        self.T2 = int(self.keep2[:r.T].sum().item())
        self.cu2 = torch.empty_like(self.pipe.cu)
        self.repacked = [torch.empty_like(self.pipe.pq) for _ in range(3)]
        torch.cuda.synchronize()

    def c_step(self) -> BenchStep:
        s = self.r.c_step()
        p = self.pipe
        for i, t in enumerate((p.pq, p.pk, p.pv)):
            s.packed[i] = t.data_ptr()
        s.o, s.cu = p.po.data_ptr(), p.cu.data_ptr()
        s.max_dev, s.total_dev = p.max_seqlen_dev.data_ptr(), p.total_dev.data_ptr()
        s.layers, s.out_padded2 = self.layers, self.out2.data_ptr()
        s.keep2, s.cu2 = self.keep2.data_ptr(), self.cu2.data_ptr()
        for i, t in enumerate(self.repacked):
            s.repacked[i] = t.data_ptr()
        return s


def settled_region_us(enqueue, stream, reps: int, rounds: int = 3) -> float:
    """Average device time of one step, `enqueue(n)` putting n steps on
    `stream` back to back: an untimed warm-up of 2*reps steps (at least 200),
    then `rounds` regions of `reps` steps with HIP events on the launch stream
    at their two ends only, and the median region.  The GPU takes a few tens
    of ms under load to settle: after a three-step warm-up the first
    300-launch region of rattn_forward at 384 px ran 44.2 us, the next ones
    41.0 and 38.9-39.2."""
    enqueue(max(2 * reps, 200))
    torch.cuda.synchronize()
    times = []
    for _ in range(rounds):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        enqueue(reps)
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1) * 1000.0 / reps)
    return statistics.median(times)


def c_region_us(step: BenchStep, what: int, reps: int, stream) -> float:
    """Average device time of one `what` step, enqueued back to back from C++
    (settled_region_us)."""
    lib = timing_lib()

    def enqueue(n):
        if lib.bench_loop(ctypes.byref(step), what, n) != 0:
            raise RuntimeError(f"bench_loop({what}) failed")
    return settled_region_us(enqueue, stream, reps)


def three_call_and_stacks(r: Resident, reps: int) -> dict:
    """The pages' three-call form (rattn_pack -> rattn_forward -> rattn_unpack)
    against the one launch, and a stack of STACK_LAYERS attention layers on one
    mask: packed once, attended per layer, unpacked once, against rattn_fused
    per layer (integrated packing pipeline: the packed buffer is kept across
    blocks).  Device time per step, warm, from back-to-back C++ enqueues."""
    w = r.w
    sr = StackResident(r)
    cs = sr.c_step()
    L = sr.layers
    one = {w_: c_region_us(cs, w_, reps, r.stream) for w_ in (WHAT_THREE_CALL, WHAT_FUSED)}
    stack_reps = max(1, reps // L)
    packed = c_region_us(cs, WHAT_LAYERS_PACKED, stack_reps, r.stream)
    fused = c_region_us(cs, WHAT_LAYERS_FUSED, stack_reps, r.stream)
    tc_bytes = three_call_bytes(r.T, w.B, w.N, w.H, w.dtype)
    c_region_us(cs, WHAT_THREE_CALL, 1, r.stream)  # the packed q, k, v the re-pack reads
    rp = c_region_us(cs, WHAT_REPACK, reps, r.stream)
    rp_bytes = repack_bytes(r.T, sr.T2, w.B, w.H, w.dtype)
    return {
        "three_call_us": round(one[WHAT_THREE_CALL], 2),
        "three_call_bytes": tc_bytes,
        "three_call_hbm_frac": round(tc_bytes / (one[WHAT_THREE_CALL] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "fused_us": round(one[WHAT_FUSED], 2),
        "fused_speedup_vs_three_call": round(one[WHAT_THREE_CALL] / one[WHAT_FUSED], 3),
        "stack": {
            "layers": L,
            "packed_once_us": round(packed, 2),
            "packed_once_us_per_layer": round(packed / L, 2),
            "fused_per_layer_us": round(fused, 2),
            "fused_per_layer_us_per_layer": round(fused / L, 2),
            "packed_speedup_vs_fused_per_layer": round(fused / packed, 3),
            "packed_once_bytes": (three_call_bytes(r.T, w.B, w.N, w.H, w.dtype)
                                  + (L - 1) * attention_bytes(r.T, w.H, w.dtype)),
            "fused_per_layer_bytes": L * fused_bytes(r.T, w.B, w.N, w.H, w.dtype),
        },
        "repack": {"keep_fraction": REPACK_KEEP, "T": r.T, "T2": sr.T2, "tensors": 3,
                   "us": round(rp, 2), "bytes": rp_bytes,
                   "hbm_frac": round(rp_bytes / (rp * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
    }


def python_call_floor(call, stream, iters: int, warmup: int) -> dict:
    """Host call -> completion through Python: `call()` then a stream
    synchronisation, timed with time.perf_counter_ns around both."""
    ts = []
    for i in range(warmup + iters):
        t0 = time.perf_counter_ns()
        call()
        stream.synchronize()
        t1 = time.perf_counter_ns()
        if i >= warmup:
            ts.append((t1 - t0) / 1000.0)
    ts.sort()
    n = len(ts)
    at = lambda f: ts[min(n - 1, int(f * (n - 1) + 0.5))]
    return {"median_us": round(at(0.5), 2), "p5_us": round(at(0.05), 2),
            "p95_us": round(at(0.95), 2), "mean_us": round(sum(ts) / n, 2),
            "min_us": round(ts[0], 2)}


def python_floors(r: Resident, stream, iters: int, warmup: int) -> dict:
    """The product's own Python path, call -> completion: FusedPlan.run()
    (checked and marshalled once), rattn_fused() with its per-call checks and
    marshalling, and rattn_forward() on flat buffers; next to a one-element
    torch in-place add on the same stream, the framework's own floor."""
    w = r.w
    f = FlatResident(w, stream)
    one = torch.zeros(1, device="cuda")
    calls = {
        "fused_plan_run": r.plan.run,
        "fused_call": lambda: rattn_fused(r.q, r.k, r.v, r.keep, w.scale, out_padded=r.out,
                                          cls=r.cls, stream=stream),
        "forward_call": lambda: rattn_forward(f.flat[0], f.flat[1], f.flat[2], f.o, f.cu, w.N,
                                              w.scale, stream=stream),
        "torch_add_one_element": lambda: one.add_(1.0),
    }
    with torch.cuda.stream(stream):
        return {name: python_call_floor(c, stream, iters, warmup) for name, c in calls.items()}


def dispatch_floors(stream, iters: int, warmup: int) -> dict:
    """Host call -> completion (C++ steady_clock) at serving batch sizes 1-4,
    80 % pruning, DeiT-B shape: the one-launch rattn_fused (also enqueue-only
    and replayed from a hipGraph) and rattn_forward alone on flat buffers,
    plus the platform's empty-kernel floor."""
    lib = timing_lib()
    st = BenchStats()
    res = {}
    if lib.bench_empty_floor(iters, warmup, stream.cuda_stream, ctypes.byref(st)) != 0:
        raise RuntimeError("bench_empty_floor failed")
    res["empty_kernel_launch_sync_us"] = st.as_dict()
    print(f"[bench] empty kernel launch+sync {st.median_us:.2f} us", flush=True)
    for B in workloads.SWEEP_B:
        r = Resident(workloads.deit_b_sweep(B, 0.8), stream)
        cs = r.c_step()
        row = {"T": r.T}
        if lib.bench_call_floor(ctypes.byref(cs), WHAT_FUSED, iters, warmup, ctypes.byref(st)):
            raise RuntimeError("bench_call_floor failed")
        row["fused_call_sync_us"] = st.as_dict()
        if lib.bench_enqueue_cost(ctypes.byref(cs), WHAT_FUSED, iters, ctypes.byref(st)):
            raise RuntimeError("bench_enqueue_cost failed")
        row["fused_enqueue_us"] = st.as_dict()
        if lib.bench_graph_floor(ctypes.byref(cs), WHAT_FUSED, iters, warmup, ctypes.byref(st)) == 0:
            row["fused_graph_replay_sync_us"] = st.as_dict()
        if lib.bench_graph_enqueue_cost(ctypes.byref(cs), WHAT_FUSED, iters, ctypes.byref(st)) == 0:
            row["fused_graph_launch_enqueue_us"] = st.as_dict()
        sr = StackResident(r)  # owns the flat buffers tc points into
        tc = sr.c_step()
        if lib.bench_call_floor(ctypes.byref(tc), WHAT_THREE_CALL, iters, warmup, ctypes.byref(st)):
            raise RuntimeError("bench_call_floor (three-call) failed")
        row["three_call_call_sync_us"] = st.as_dict()
        if lib.bench_graph_floor(ctypes.byref(tc), WHAT_THREE_CALL, iters, warmup,
                                 ctypes.byref(st)) == 0:
            row["three_call_graph_replay_sync_us"] = st.as_dict()
        f = FlatResident(r.w, stream)
        if lib.bench_call_floor(ctypes.byref(f.c_step()), WHAT_FORWARD, iters, warmup,
                                ctypes.byref(st)):
            raise RuntimeError("bench_call_floor (forward) failed")
        row["forward_call_sync_us"] = st.as_dict()
        row["python_call_sync_us"] = python_floors(r, stream, iters, warmup)
        res[f"deit_b_B{B}_p80"] = row
        print(f"[bench] dispatch floor B={B}: fused call+sync {row['fused_call_sync_us']['median_us']} us,"
              f" enqueue {row['fused_enqueue_us']['median_us']} us, rattn_forward alone call+sync "
              f"{row['forward_call_sync_us']['median_us']} us, three calls + sync "
              f"{row['three_call_call_sync_us']['median_us']} us", flush=True)
        py = row["python_call_sync_us"]
        print(f"[bench] Python path B={B}: FusedPlan.run+sync {py['fused_plan_run']['median_us']} us,"
              f" rattn_fused()+sync {py['fused_call']['median_us']} us, rattn_forward()+sync "
              f"{py['forward_call']['median_us']} us, torch one-element add+sync "
              f"{py['torch_add_one_element']['median_us']} us", flush=True)
    # every point of the serving sweep: the one launch, host call + sync and
    # device time back to back
    sweep = {}
    for B, p, exact in workloads.sweep_points():
        r = Resident(workloads.deit_b_sweep(B, p, exact_unpruned=exact), stream)
        cs = r.c_step()
        if lib.bench_call_floor(ctypes.byref(cs), WHAT_FUSED, iters, warmup, ctypes.byref(st)):
            raise RuntimeError("bench_call_floor failed")
        sweep[r.w.name] = {"B": B, "prune": p, "T": r.T, "fused_call_sync_us": st.median_us,
                           "fused_device_us": round(c_region_us(cs, WHAT_FUSED, iters, stream), 2)}
    res["sweep"] = sweep
    print("[bench] serving sweep, rattn_fused call+sync (device) us: " + ", ".join(
        f"B{v['B']} p{int(round(v['prune'] * 100))}{'x' if 'exact' in k else ''} "
        f"{v['fused_call_sync_us']:.1f} ({v['fused_device_us']:.1f})" for k, v in sweep.items()),
        flush=True)
    return res


def region_time_us(r: Resident, launches: int) -> float:
    """Average rattn_fused duration over back-to-back launches through the
    Python binding (settled_region_us: HIP events at the two ends of each
    region only; an event between launches adds a few microseconds of its
    own to each)."""
    def enqueue(n):
        for _ in range(n):
            r.step()
    return settled_region_us(enqueue, r.stream, launches)


def evict_caches(flush_buf) -> None:
    """Evict the L2s and the 256 MB MALL before a cold launch: a 512 MB write,
    then a read of the same buffer.  The read writes the dirty lines of the
    write back to HBM before the measured launch starts; after a write alone,
    that write-back lands inside the next launch and adds 12-16 us at 384 px,
    while a read alone, or the write and the read, give the same times."""
    flush_buf.zero_()
    flush_buf.view(torch.float32).sum()


def kernel_time_us(r: Resident, launches: int, cold: bool, flush_buf=None,
                   cold_launches: int = 50) -> float:
    """Warm: region average of back-to-back launches.  Cold: median of single
    launches between HIP events, each after `evict_caches` (the events add
    about 2 us to each)."""
    if not cold:
        return region_time_us(r, launches)
    r.step()
    torch.cuda.synchronize()
    times = []
    for _ in range(cold_launches):
        if cold:
            evict_caches(flush_buf)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(r.stream)
        r.step()
        e1.record(r.stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1) * 1000.0)
    times.sort()
    return times[len(times) // 2]


def forward_alone(w, stream, launches: int, flush_buf, cold_launches: int) -> dict:
    """rattn_forward alone on the flat buffers of a workload (prepared on the
    host, resident in HBM), against its own algorithmic bytes (q, k, v read and
    o written once): warm, back-to-back region average from C++; cold, median
    of single launches between HIP events, each after `evict_caches`."""
    f = FlatResident(w, stream)
    step = f.c_step()
    lib = timing_lib()
    warm = c_region_us(step, WHAT_FORWARD, launches, stream)
    times = []
    for _ in range(cold_launches):
        evict_caches(flush_buf)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        if lib.bench_loop(ctypes.byref(step), WHAT_FORWARD, 1) != 0:
            raise RuntimeError("bench_loop(forward) failed")
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1) * 1000.0)
    times.sort()
    cold = times[len(times) // 2]
    T = int(f.cu[-1].item())
    nbytes = attention_bytes(T, w.H, w.dtype)
    out = {"bytes": nbytes, "traffic_bytes": measured_traffic("forward_" + w.name)}
    for name, us in (("warm", warm), ("cold", cold)):
        gbs = nbytes / (us * 1e-6) / 1e9
        out[name] = {"us": round(us, 2), "GBps": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    return out


def padded_comparison(r: Resident, launches: int, rounds: int = 3) -> dict:
    """The ragged kernel against its dense comparator (rattn_fused_padded,
    same outputs): every image padded to the longest survivor, and to N (no
    pruning gain at all).  Warm back-to-back averages; the three are measured
    in turn, `rounds` times, and each reports its median, so that the first
    one measured does not absorb the GPU's ramp-up."""
    plans = {"ragged": r.plan.run}
    for name, pad in (("padded_longest", max(r.lengths)), ("padded_n", r.w.N)):
        plans[name] = FusedPlan(r.q, r.k, r.v, r.keep, r.w.scale, out_padded=r.out, cls=r.cls,
                                stream=r.stream, pad_len=max(pad, 1)).run
    times = {name: [] for name in plans}
    saved = r.step
    for _ in range(rounds):
        for name, run in plans.items():
            r.step = run
            times[name].append(region_time_us(r, launches))
    r.step = saved
    med = {name: sorted(t)[len(t) // 2] for name, t in times.items()}
    out = {"ragged_us": round(med["ragged"], 2)}
    for name in ("padded_longest", "padded_n"):
        out[f"{name}_us"] = round(med[name], 2)
        out[f"ragged_speedup_vs_{name}"] = round(med[name] / med["ragged"], 3)
    return out


def config_report(w, stream, launches: int, cold_launches: int, flush, box_gbs=None,
                  peaks=None) -> dict:
    """One workload on its own: rattn_fused warm and cold with its bytes,
    flops, measured traffic (when the counter profile covers it) and lower
    bounds; the dense comparator; the three-call step and the layer stacks;
    rattn_forward alone."""
    r = Resident(w, stream)
    nbytes = fused_bytes(r.T, w.B, w.N, w.H, w.dtype)
    flops = attention_flops(r.lengths, w.H)
    row = {"B": w.B, "N": w.N, "H": w.H, "dtype": w.dtype, "T": r.T,
           "fused_bytes": nbytes, "attn_flops": flops,
           "traffic_bytes": measured_traffic(w.name),
           "roofs_us": roofs_us(nbytes, flops, box_gbs, peaks)}
    row["padded_comparator"] = padded_comparison(r, launches)
    row["three_call_and_stacks"] = three_call_and_stacks(r, launches)
    row["forward_alone"] = forward_alone(w, stream, launches, flush, cold_launches)
    for cold in (False, True):
        us = kernel_time_us(r, launches, cold, flush, cold_launches)
        gbs = nbytes / (us * 1e-6) / 1e9
        tfl = flops / (us * 1e-6) / 1e12
        row["cold" if cold else "warm"] = {
            "us": round(us, 2), "seqs_per_s": round(w.B / (us * 1e-6), 1),
            "GBps": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "TFLOPs": round(tfl, 2), "mfma_frac": round(tfl / MFMA_PEAK_TFLOPS[w.dtype], 4)}
    pc = row["padded_comparator"]
    print(f"[bench] {w.name}: warm {row['warm']['us']} us ({row['warm']['hbm_frac']:.3f} of HBM),"
          f" cold {row['cold']['us']} us ({row['cold']['hbm_frac']:.3f}); padded comparator "
          f"{pc['padded_longest_us']} us (longest survivor) / {pc['padded_n_us']} us (N)",
          flush=True)
    _print_stacks(w.name, row["three_call_and_stacks"])
    fa = row["forward_alone"]
    print(f"[bench] {w.name}: rattn_forward alone warm {fa['warm']['us']} us "
          f"({fa['warm']['hbm_frac']:.3f} of HBM), cold {fa['cold']['us']} us "
          f"({fa['cold']['hbm_frac']:.3f})", flush=True)
    del r
    return row


def large_configs(stream, launches: int, cold_launches: int, box_gbs=None, peaks=None) -> dict:
    out = {}
    flush = torch.empty(512 * 1024 * 1024, dtype=torch.uint8, device="cuda")
    for name, maker in (("deit_b_384_50pct", workloads.deit_b_384),
                        ("large_batch_threshold_l2", workloads.large_batch)):
        out[name] = config_report(maker(), stream, launches, cold_launches, flush, box_gbs, peaks)
    del flush
    return out


def config_workload(spec: str, seed):
    """--config: tiny, deit_s, deit_b_384, large_batch, or deit_b_sweep:B:p
    (B images, pruning fraction p; p = exact for the unpruned point)."""
    name, *rest = spec.split(":")
    if name == "deit_b_sweep":
        if len(rest) != 2:
            raise SystemExit("--config deit_b_sweep:B:p, e.g. deit_b_sweep:4:0.8")
        exact = rest[1] == "exact"
        return workloads.deit_b_sweep(int(rest[0]), 0.0 if exact else float(rest[1]), seed=seed,
                                      exact_unpruned=exact)
    if rest:
        raise SystemExit(f"--config {name} takes no parameters")
    try:
        return workloads.by_name(name, seed=seed)
    except KeyError:
        raise SystemExit(f"unknown --config {name}") from None


COLD_TRACE_LAUNCHES = 20


def cold_trace_target(spec: str) -> None:
    """Launches for a kernel trace of cold single launches (run under
    rocprofv3 --kernel-trace): on one workload, COLD_TRACE_LAUNCHES launches of
    rattn_fused, each right after `evict_caches` on the same stream with no
    events around them, then as many back to back; then the same for
    rattn_forward on its flat buffers.  The trace gives each launch's own
    duration, measured without host events."""
    w = config_workload(spec, None)
    rattn_init()
    stream = torch.cuda.current_stream()
    flush = torch.empty(512 * 1024 * 1024, dtype=torch.uint8, device="cuda")
    r = Resident(w, stream)
    f = FlatResident(w, stream)
    step = f.c_step()
    lib = timing_lib()

    def forward():
        if lib.bench_loop(ctypes.byref(step), WHAT_FORWARD, 1) != 0:
            raise RuntimeError("bench_loop(forward) failed")

    for launch in (r.step, forward):
        launch()
        torch.cuda.synchronize()
        for _ in range(COLD_TRACE_LAUNCHES):
            evict_caches(flush)
            launch()
        torch.cuda.synchronize()
        # the same kernel back to back, for the trace's own warm figure
        for _ in range(COLD_TRACE_LAUNCHES + 1):
            launch()
        torch.cuda.synchronize()
    print(f"[bench] cold trace target {w.name}: {COLD_TRACE_LAUNCHES} cold and "
          f"{COLD_TRACE_LAUNCHES} back-to-back launches each of rattn_fused and rattn_forward",
          flush=True)


def summarize_cold_trace(trace_csv: str) -> str:
    """Summary text of a rocprofv3 kernel trace of `bench.py --cold-trace`,
    per attention kernel: the durations of the launches that directly follow
    the cache eviction's reduction kernel (cold), and of those that directly
    follow a launch of the same kernel (warm, back to back)."""
    import csv
    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Start_Timestamp"]))
    runs = {}
    for prev, row in zip(rows, rows[1:]):
        name = row["Kernel_Name"]
        if "fused16" not in name and "attn_fwd16" not in name:
            continue
        kind = ("cold" if "reduce" in prev["Kernel_Name"]
                else "warm" if prev["Kernel_Name"] == name else None)
        if kind:
            us = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1000.0
            runs.setdefault((kind, name), []).append(us)
    if not any(kind == "cold" for kind, _ in runs):
        raise RuntimeError("no cold attention launches in the trace")
    out = []
    for (kind, name), us in runs.items():
        us.sort()
        out.append(f"{kind} launches {len(us)} median_us {us[len(us) // 2]:.2f} "
                   f"min_us {us[0]:.2f} max_us {us[-1]:.2f} kernel {name}")
    return "\n".join(out) + "\n"


STACK_WORKLOADS = {"deit_s_80pct": workloads.deit_s, "deit_b_384_50pct": workloads.deit_b_384,
                   "large_batch_threshold_l2": workloads.large_batch}


def _print_stacks(name: str, t: dict) -> None:
    st = t["stack"]
    print(f"[bench] {name}: three calls {t['three_call_us']} us vs one launch {t['fused_us']} us;"
          f" {st['layers']} layers packed once {st['packed_once_us']} us vs rattn_fused per layer "
          f"{st['fused_per_layer_us']} us ({st['packed_speedup_vs_fused_per_layer']}x); re-pack "
          f"{t['repack']['us']} us ({t['repack']['hbm_frac']:.3f} of HBM)", flush=True)


def box_copy_bandwidth(stream, nbytes: int = 1 << 30, reps: int = 10) -> float:
    """Device-to-device copy of a 1 GiB buffer (the runtime's copy kernel):
    bytes read plus bytes written per second, GB/s -- the box's own measure
    of the HBM roof, next to the 8 TB/s datasheet figure."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        b.copy_(a)
    e1.record(stream)
    e1.synchronize()
    sec = e0.elapsed_time(e1) / 1000.0 / reps
    del a, b
    return round(2 * nbytes / sec / 1e9, 1)


def box_peaks(stream, grid: int = 1024, iters: int = 2048) -> dict:
    """Box-measured compute ceilings (bench_peaks.hip, 1024 workgroups of 256
    threads, eight independent chains per lane): dense bf16 MFMA, the
    softmax's per-score pair (one fma feeding one exp2), exp2 alone and float32
    fma -- next to the datasheet peaks the roofline fractions use."""
    res = BenchPeaks()
    if timing_lib().bench_peaks(grid, iters, stream.cuda_stream, ctypes.byref(res)) != 0:
        raise RuntimeError("bench_peaks failed")
    # co-issue: half the wavefronts of each launch alone are half its time
    mf, va, mix = res.split_mfma_s / 2, res.split_valu_s / 2, res.split_mixed_s
    return {"mfma_bf16_TFLOPs": round(res.mfma_bf16_tflops, 1),
            "fma_exp2_per_s": float(f"{res.fma_exp_per_s:.4g}"),
            "exp2_per_s": float(f"{res.exp_per_s:.4g}"),
            "fma_f32_TFLOPs": round(res.fma_f32_tflops, 1),
            "mfma_ns_per_simd": round(res.mfma_ns, 2),
            "mfma_plus_exp2_same_wave_ns_per_simd": round(res.mfma_exp_ns, 2),
            "mfma_beside_valu_waves": {"mixed_ms": round(mix * 1e3, 3), "mfma_half_ms": round(mf * 1e3, 3),
                                       "valu_half_ms": round(va * 1e3, 3),
                                       "hidden_frac_of_smaller": round((mf + va - mix) / min(mf, va), 3)},
            "from": "bench_peaks.hip: 1024 workgroups x 256 threads (split probes: 512 x 512), "
                    "2048 iterations of eight independent chains per lane, HIP events around one "
                    "launch after a warm-up"}


def roofs_us(nbytes: int, flops: int, box_gbs, peaks) -> dict:
    """Lower bounds on one launch of the attention path, us: its algorithmic
    bytes at the HBM peak, its contraction flops at the dense MFMA peak, and
    its H * sum(L^2) scores at the box's rate for one fma + one exp2 each (the
    vector work every score needs at least; the kernel spends about four more
    VALU instructions per score).  Datasheet peaks, and box-measured ones when
    given."""
    scores = flops // (4 * 64)
    out = {"hbm": round(nbytes / (HBM_PEAK_GBS * 1e9) * 1e6, 2),
           "mfma": round(flops / (MFMA_PEAK_TFLOPS["bf16"] * 1e12) * 1e6, 2)}
    if box_gbs:
        out["hbm_box"] = round(nbytes / (box_gbs * 1e9) * 1e6, 2)
    if peaks:
        out["mfma_box"] = round(flops / (peaks["mfma_bf16_TFLOPs"] * 1e12) * 1e6, 2)
        out["fma_exp2_box"] = round(scores / peaks["fma_exp2_per_s"] * 1e6, 2)
    return out


def tiny_fp32(stream, launches: int) -> dict:
    """The tiny float32 workload (B=4, N=197, H=3): rattn_fused warm, back to
    back, against both roofs -- float32 matrix/vector arithmetic binds here,
    not HBM, and at this size the launch itself is most of the time."""
    w = workloads.tiny()
    r = Resident(w, stream)
    us = region_time_us(r, launches)
    flops = attention_flops(r.lengths, w.H)
    nbytes = fused_bytes(r.T, w.B, w.N, w.H, w.dtype)
    out = {"B": w.B, "N": w.N, "H": w.H, "dtype": w.dtype, "T": r.T, "us": round(us, 2),
           "attn_flops": flops, "fused_bytes": nbytes,
           "fp32_frac": round(flops / (us * 1e-6) / 1e12 / MFMA_PEAK_TFLOPS["f32"], 5),
           "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 5)}
    print(f"[bench] {w.name}: rattn_fused {us:.2f} us (fp32 {out['fp32_frac']:.4f} of the "
          f"157.3 TFLOP/s roof, HBM {out['hbm_frac']:.4f})", flush=True)
    return out


def cpu_model() -> dict:
    """The host CPU: model name (from /proc/cpuinfo), logical CPUs, and the
    CPUs this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    return {"model": model, "logical_cpus": os.cpu_count() or 1, "usable_cpus": usable}


def _sub_workload(w, n_images: int):
    """The first n_images images of a workload (a bounded sample of it)."""
    if n_images >= w.B:
        return w
    import copy
    s = copy.copy(w)
    s.B = n_images
    s.keep = w.keep[:n_images].contiguous()
    s.q, s.k, s.v = (t[:n_images].contiguous() for t in (w.q, w.k, w.v))
    return s


def _oracle_loop(w, budget_s: float) -> tuple:
    """Whole batches of the fp64 oracle's scan, pack, attention and unpack on
    w until the budget is used; returns (batches, seconds)."""
    import oracle  # test infrastructure; used only for this reported baseline
    t0 = time.perf_counter()
    reps = 0
    while True:
        res = oracle.pipeline(w)
        oracle.unpack(res["o64"], w.keep, res["cu"])
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    return reps, time.perf_counter() - t0


def cpu_baseline(w, budget_s: float, sample_images: int | None = None) -> dict:
    """The CPU oracle (plain C, fp64, one thread) on the same workload, or on
    its first `sample_images` images: whole batches until the budget is used,
    images per second."""
    s = _sub_workload(w, sample_images) if sample_images else w
    reps, dt = _oracle_loop(s, budget_s)
    what = (f"the first {s.B} of the {w.B} images" if s.B < w.B else f"all {w.B} images")
    return {"value": round(reps * s.B / dt, 2), "unit": "seqs/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} pass(es) over {what} of the {w.name} workload through the fp64 "
                      f"oracle's scan, pack, attention and unpack, {dt:.1f} s on 1 host thread",
            "cpu": cpu_model()}


def cpu_baselines_per_config(budget_s: float) -> dict:
    """The one-thread oracle on every workload the GPU path is measured on;
    the two large ones on a bounded sample of their images."""
    out = {}
    for name, maker, sample in (("tiny_fp32", workloads.tiny, None),
                                ("deit_s_80pct", workloads.deit_s, None),
                                ("deit_b_sweep_B4_p80", lambda: workloads.deit_b_sweep(4, 0.8), None),
                                ("deit_b_384_50pct", workloads.deit_b_384, 2),
                                ("large_batch_threshold_l2", workloads.large_batch, 16)):
        out[name] = cpu_baseline(maker(), budget_s, sample)
        print(f"[bench] CPU oracle {name}: {out[name]['value']} images/s on 1 thread", flush=True)
    return out


def _oracle_worker_main(maker: str, budget_s: float) -> None:
    """Entry of one all-cores worker process: prints 'reps seconds'."""
    reps, dt = _oracle_loop(workloads.by_name(maker), budget_s)
    print(f"{reps} {dt}", flush=True)


def cpu_baseline_all_cores(w, maker: str, budget_s: float, max_procs: int = 16) -> dict:
    """The CPU oracle on every usable host core at once: one plain child
    process per core (at most max_procs, the host share of one GPU), each
    running the one-thread loop of cpu_baseline for the budget; images per
    second summed over the workers.  The children are started as fresh
    interpreters that never touch the GPU, and all of them are waited for, so
    none outlives the run."""
    import subprocess
    procs = max(1, min(max_procs, cpu_model()["usable_cpus"]))
    code = ("import sys; sys.path.insert(0, %r); import bench; "
            "bench._oracle_worker_main(%r, %r)" % (ROOT, maker, float(budget_s)))
    env = {**os.environ, "OMP_NUM_THREADS": "1"}
    children = [subprocess.Popen([sys.executable, "-c", code], stdout=subprocess.PIPE, text=True,
                                 env=env, cwd=ROOT) for _ in range(procs)]
    runs = []
    for c in children:
        out, _ = c.communicate()
        if c.returncode != 0:
            raise RuntimeError(f"oracle worker failed with status {c.returncode}")
        reps, dt = out.split()[-2:]
        runs.append((int(reps), float(dt)))
    rate = sum(reps * w.B / dt for reps, dt in runs)
    batches = sum(reps for reps, _ in runs)
    return {"value": round(rate, 2), "unit": "seqs/s", "cores": procs, "kind": "oracle",
            "sample": f"{batches} full batch(es) of the {w.name} workload (B={w.B}) through the "
                      f"fp64 oracle's scan, pack, attention and unpack, {procs} worker "
                      f"process(es) of one thread for {budget_s:.0f} s each",
            "cpu": cpu_model()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--quick", action="store_true",
                    help="main metric only: no dispatch floors, no large configs, no CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-trace", metavar="NAME",
                    help="only cold single launches of rattn_fused and rattn_forward on one "
                         "workload (for rocprofv3 --kernel-trace), then exit")
    ap.add_argument("--cold-summary", metavar="KERNEL_TRACE_CSV",
                    help="summarize the cold launches in a kernel trace of --cold-trace")
    ap.add_argument("--pmc-target", action="store_true",
                    help="only the launches the traffic counters are read on, then exit")
    ap.add_argument("--pmc-forward", choices=["deit_s", "deit_b_384", "large_batch"],
                    help="only five rattn_forward launches on one workload (for the SQ "
                         "counters of the attention loop), then exit")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the traffic summary of two counter runs, then exit")
    ap.add_argument("--config", metavar="NAME",
                    help="time one workload on its own (tiny, deit_s, deit_b_384, large_batch, "
                         "deit_b_sweep:B:p) and print its report as one JSON line, then exit")
    ap.add_argument("--seed", type=int, default=None,
                    help="with --config: the workload's seed (default: its fixed seed)")
    ap.add_argument("--peaks-only", action="store_true",
                    help="only the box-peak probes (MFMA, exp2, fma), printed as JSON, then exit")
    ap.add_argument("--stack-only", choices=sorted(STACK_WORKLOADS),
                    help="only the three-call step, the layer stacks and the re-pack of one "
                         "workload (for a kernel trace of those kernels), then exit")
    args = ap.parse_args()
    if args.pmc_summary:
        sys.stdout.write(summarize_pmc(*args.pmc_summary))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the path has no "
              "cross-GPU step and the library runs on a single MI355X; use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.cold_summary:
        sys.stdout.write(summarize_cold_trace(args.cold_summary))
        return
    if args.cold_trace:
        cold_trace_target(args.cold_trace)
        return
    if args.pmc_target:
        pmc_target()
        return
    if args.pmc_forward:
        pmc_forward(args.pmc_forward)
        return
    if args.peaks_only:
        print(json.dumps({"box_peaks": box_peaks(torch.cuda.current_stream())}), flush=True)
        return
    if args.stack_only:
        rattn_init()
        stream = torch.cuda.current_stream()
        w = STACK_WORKLOADS[args.stack_only]()
        t = three_call_and_stacks(Resident(w, stream), 200)
        _print_stacks(w.name, t)
        print(json.dumps({"workload": w.name, "three_call_and_stacks": t}), flush=True)
        return
    if args.config:
        w = config_workload(args.config, args.seed)
        rattn_init()
        stream = torch.cuda.current_stream()
        flush = torch.empty(512 * 1024 * 1024, dtype=torch.uint8, device="cuda")
        row = config_report(w, stream, 300, 50, flush)
        print(json.dumps({"config": args.config, "workload": w.name, "seed": w.seed,
                          "data": "synthetic", **row}), flush=True)
        return
    rattn_init()
    stream = torch.cuda.current_stream()

    w = workloads.deit_s()
    r = Resident(w, stream)
    print(f"[bench] workload {w.name}: B={w.B} N={w.N} H={w.H} {w.dtype} T={r.T}", flush=True)
    box = peaks = None
    if not args.quick:
        # the box's copy rate and compute ceilings, measured first: their
        # second of full-chip work also brings the GPU out of idle, so that
        # the timed steps below run at the clocks of a busy GPU and not at
        # those of a fresh process
        box = box_copy_bandwidth(stream)
        print(f"[bench] box-measured copy bandwidth {box} GB/s", flush=True)
        peaks = box_peaks(stream)
        print(f"[bench] box-measured peaks: bf16 MFMA {peaks['mfma_bf16_TFLOPs']} TFLOP/s, "
              f"fma+exp2 {peaks['fma_exp2_per_s']:.3g}/s, exp2 {peaks['exp2_per_s']:.3g}/s, "
              f"fp32 fma {peaks['fma_f32_TFLOPs']} TFLOP/s", flush=True)
    for _ in range(args.warmup):
        r.step()
    torch.cuda.synchronize()

    # timed region: K steps back to back, HIP events on the launch stream at its
    # two ends (events between steps would add their own time to each step)
    K = args.steps
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(K):
        r.step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1000.0 / K
    kern_us = e0.elapsed_time(e1) * 1000.0 / K
    nbytes = fused_bytes(r.T, w.B, w.N, w.H, w.dtype)
    achieved = nbytes / (kern_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "kernel": "rattn_fused", "achieved": round(achieved, 2),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 5),
                "traffic": measured_traffic(w.name), "bytes_per_launch": nbytes,
                "avg_launch_us": round(kern_us, 3),
                "avg_launch_us_from": "HIP events at the ends of the timed region / K "
                                      "(includes the gap between back-to-back dispatches)"}

    line = {
        "metric": METRIC, "value": round(w.B / (ms_per_step / 1000.0), 1), "unit": "seqs/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": "deit_s_80pct", "B": w.B, "N": w.N, "H": w.H, "head_dim": 64,
                   "total_tokens": r.T, "max_seqlen_arg": w.N,
                   "step": "rattn_fused (scan + pack + attention + unpack/CLS, one launch) "
                           "via the Python binding (FusedPlan.run)"},
        "us_per_step": round(ms_per_step * 1000.0, 2),
        "kernel_avg_us": {"rattn_fused": round(kern_us, 3)},
        "attn_flops": attention_flops(r.lengths, w.H),
        "roofline": roofline,
    }
    if not args.quick:
        roofline["box_peak_GBps"] = box
        roofline["box_peak_from"] = "1 GiB device-to-device copy, read + written bytes / time"
        roofline["box_frac"] = round(achieved / box, 5)
        line["box_peaks"] = peaks
        line["roofs_us"] = roofs_us(nbytes, line["attn_flops"], box, peaks)
        flush = torch.empty(512 * 1024 * 1024, dtype=torch.uint8, device="cuda")
        cold = kernel_time_us(r, K, True, flush, cold_launches=200)
        del flush
        line["cold"] = {"us": round(cold, 2), "hbm_frac": round(nbytes / (cold * 1e-6) / 1e9 / HBM_PEAK_GBS, 5),
                        "from": "median of single launches between HIP events, each after a 512 MB write "
                                "and a read of it that evict the L2s and the 256 MB MALL"}
        print(f"[bench] {w.name}: cold {cold:.2f} us per launch", flush=True)
        line["padded_comparator"] = padded_comparison(r, max(K, 500))
        pc = line["padded_comparator"]
        print(f"[bench] {w.name}: ragged {pc['ragged_us']} us, padded to longest survivor "
              f"{pc['padded_longest_us']} us, padded to N {pc['padded_n_us']} us", flush=True)
        line["three_call_and_stacks"] = three_call_and_stacks(r, 500)
        _print_stacks(w.name, line["three_call_and_stacks"])
        side = torch.cuda.Stream()  # graph capture needs a non-default stream
        line["dispatch_floor"] = dispatch_floors(side, iters=1000, warmup=100)
        line["large_configs"] = large_configs(stream, launches=300, cold_launches=50,
                                              box_gbs=box, peaks=peaks)
        line["tiny_fp32"] = tiny_fp32(stream, launches=2000)
    if not args.quick and not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
        line["cpu_baseline_all_cores"] = cpu_baseline_all_cores(w, "deit_s", args.cpu_budget)
        line["cpu_baseline_per_config"] = cpu_baselines_per_config(args.cpu_budget / 3)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
