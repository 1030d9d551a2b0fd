"""Benchmark of the ternary hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--G 128] [--rows all]
    python bench.py --trace-summary <rocprofv3 kernel_stats.csv> [<kernel_trace.csv>]

Workload of the step (`value`, `roofline`): the 24-layer Qwen-like FFN stack
(hidden 1024, intermediate 3584: gate and up W[3584,1024], down
W[1024,3584]; 72 matrices, 264,241,152 bf16 weights ~ N(0, 0.02)), G = 128.
One step is one pass of every step of the hot path over that stack, in the
path's own order (pack the weights, validate them, prefill, decode):
  quantize + pack all 72 bf16 matrices                 (tq_quantize_pack_batched:
      two launches, one per shape)
  unpack + validate all 72 packed matrices             (tq_unpack_batched: two)
  prefill GEMM, M = 512 tokens, through all 72 matrices (tq_gemm_grouped:
      one persistent launch over both shapes; each matrix has its own output)
  decode GEMV, M = 1, through all 72 matrices          (tq_gemv_grouped:
      one launch for the 48 K=1024 and the 24 K=3584 matrices together)
The packed weights live in a ring of eight slots (480 MB, more than the
256 MB memory-side cache).  Step t packs into slot (t+2)%8 and unpacks it,
runs the GEMM on slot (t+4)%8 and the GEMV on slot t%8: the bytes the GEMV
reads were packed and unpacked two steps (several GB of traffic) earlier and
come from HBM, and no row reads bytes the row before it read.  Every row is
direct launches (pointer arrays built once per ring slot); HIP events
recorded between the rows on the stream the kernels run on time each row,
dispatch included.  The events are created with hipEventDisableSystemFence
(--torch-events: torch's events, whose recording writes back and invalidates
the caches), so an interval holds its kernels and not the fences.

The GEMV kernel alone (`roofline`): after the steps, the decode pass runs
over all eight slots back to back (eight launches, each launch's dispatch
overlapping the previous kernel) between two HIP events; the average launch
is the median of three such chains / 8.

Rows outside the step (each selectable with --rows; every one times chains
of launches between HIP events on the same stream, median of three):
  gemv_g64     the decode pass of the stack at G = 64 (its own 8-slot ring)
  gemm_m2048   the prefill GEMM of the stack at M = 2048 (the grouped
               launch; each shape's batched launch also timed on its own)
  dense8b      8B-class FFN matrices W[14336,4096] and W[4096,14336], G = 128,
               decode at M = 1, 4, 16 over a ring of copies (>= 1 GiB)
  dequant      decode to bf16 of every matrix of a slot (two launches per slot)
  gemv2        the decode pass over the 2-bit format (one grouped launch), and the
               2-bit prefill matmul at --prefill-m rows (one launch per shape)
  w4a16        the decode pass over seeded W4A16 parameters (one grouped launch), and
               the W4A16 prefill matmul at --prefill-m rows (one launch per shape)
  qat          the QAT forward of the stack from bf16 and from fp32 latent
               weights (two launches a pass each)
  ceilings     plain HBM read streams over the decode pass's bytes (eight
               57.8 MB buffers) and over 1 GiB, a bf16 MFMA-only loop, LDS
               table reads and VALU issue of v_dot2_f32_bf16 and v_perm_b32
  cpu          the CPU oracle on bounded samples of the same workloads, at
               one thread and at the host's cores; it also checks the GPU
               outputs captured above against its own results

`value` is the decode GEMV's packed-weight bandwidth: (packed code bytes +
fp16 scale bytes of the 72 matrices) / GEMV time per step.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
METRIC = "ternary GEMV packed-weight GB/s (% HBM peak); prefill GEMM TFLOP/s (% MFMA)"
RING = 8
# bytes one 8B-class matrix launch reads: packed bytes + fp16 scales at G = 128
D8_LAUNCH_BYTES = 12845056
ALL_ROWS = ("step", "gemv_g64", "gemm_m2048", "dense8b", "dequant", "gemv2", "w4a16", "qat",
            "ceilings", "cpu")
# HBM bytes per GEMV launch from rocprofv3 FETCH_SIZE and WRITE_SIZE runs of this bench, each
# scaled by the same counter on a 256 MiB copy (profiles/gemv_m1_hbm_traffic.md); valid only
# for the kernel source they were taken on (sha256 prefix of csrc/tq_gemv_m1.hip).
GEMV_TRAFFIC = {"88cc61fdaeb49a3a": 61250201}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--G", type=int, default=128)
    ap.add_argument("--prefill-m", type=int, default=512)
    ap.add_argument("--rows", default="all",
                    help="comma-separated rows to run (%s), or all" % ",".join(ALL_ROWS))
    ap.add_argument("--no-cpu-baseline", action="store_true", help="same as leaving out row cpu")
    ap.add_argument("--torch-events", action="store_true",
                    help="time with torch.cuda.Event (system-scope fences) instead of HIP "
                         "events created with hipEventDisableSystemFence")
    ap.add_argument("--cpu-seconds", type=float, default=4.0,
                    help="minimum time of each timed oracle sample")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the rows, copy 256 MiB device to device three times "
                         "(a kernel of known traffic for scaling hardware byte counters)")
    ap.add_argument("--trace-summary", nargs="+", metavar="CSV",
                    help="print a markdown summary of a rocprofv3 kernel_stats.csv (and, if "
                         "given, its kernel_trace.csv) and exit")
    ap.add_argument("--pmc-summary", nargs="+", metavar="CSV",
                    help="print a markdown summary of rocprofv3 counter_collection.csv files "
                         "(per kernel and grid: dispatches, mean of each counter) and exit")
    ap.add_argument("--kernels", metavar="REGEX",
                    help="with --pmc-summary: only kernels whose name matches")
    return ap.parse_args()


def source_hash(name):
    import hashlib
    path = os.path.join(ROOT, "ternary_weight_only_amd", "csrc", name)
    try:
        with open(path, "rb") as f:
            return hashlib.sha256(f.read()).hexdigest()[:16]
    except OSError:
        return None


# ---------------------------------------------------------------------------
# rocprofv3 summaries
# ---------------------------------------------------------------------------

def short_kernel_name(name):
    """A kernel's name without namespaces' noise, argument list or 'void'."""
    name = name.replace("(anonymous namespace)::", "").split("(")[0].strip()
    return name[len("void "):] if name.startswith("void ") else name


def trace_summary(paths):
    """Markdown tables of a rocprofv3 run: per kernel (stats CSV) and per
    kernel and grid (trace CSV)."""
    import csv
    import statistics
    rows = list(csv.DictReader(open(paths[0])))
    tot = sum(float(r["TotalDurationNs"]) for r in rows) or 1.0
    print("| kernel | calls | avg us | min us | max us | share |")
    print("|---|---|---|---|---|---|")
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        print("| %s | %s | %.2f | %.2f | %.2f | %.1f%% |" % (
            short_kernel_name(r["Name"])[:90], r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, 100.0 * float(r["TotalDurationNs"]) / tot))
    if len(paths) > 1:
        tr = list(csv.DictReader(open(paths[1])))
        groups = {}
        for r in tr:
            key = (short_kernel_name(r["Kernel_Name"])[:70],
                   r.get("Grid_Size_X", r.get("Grid_Size", "?")),
                   r.get("Grid_Size_Y", ""), r.get("Workgroup_Size_X", r.get("Workgroup_Size", "")))
            groups.setdefault(key, []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        print()
        print("| kernel | grid x | grid y | block | calls | median us | min us | max us |")
        print("|---|---|---|---|---|---|---|---|")
        for key, d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
            print("| %s | %s | %s | %s | %d | %.2f | %.2f | %.2f |" % (
                key[0], key[1], key[2], key[3], len(d), statistics.median(d), min(d), max(d)))


def pmc_summary(paths, pattern=None):
    """Markdown tables of rocprofv3 counter runs: per kernel and grid, the mean
    of each counter over the dispatches (counters are summed over the chip;
    GRBM_GUI_ACTIVE over the 8 XCDs), and the figures derived from them:
    MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8),
    bf16 MFMA flop = 512 x SQ_INSTS_VALU_MFMA_MOPS_BF16, and HBM bytes =
    1024 x FETCH_SIZE or WRITE_SIZE (KiB), before any scaling."""
    import csv
    import statistics
    # dispatches are grouped by kernel, grid and block, and, where the run has
    # an instruction counter (exact for a given launch shape), by its value,
    # which tells apart launches of one kernel on different problems
    per_disp = {}  # (path, dispatch) -> (kernel, grid, block), {counter: value}, ns
    for path in paths:
        for r in csv.DictReader(open(path)):
            short = short_kernel_name(r["Kernel_Name"])
            disp = (path, r["Dispatch_Id"])
            if disp not in per_disp:
                per_disp[disp] = ((short[-70:], r["Grid_Size"], r["Workgroup_Size"]), {},
                                  int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
            per_disp[disp][1][r["Counter_Name"]] = float(r["Counter_Value"])
    data = {}   # key -> counter -> dispatch -> value
    durs = {}   # key -> dispatch -> ns
    for disp, (k3, ctr, ns) in per_disp.items():
        insts = sorted(c for c in ctr if c.startswith("SQ_INSTS_"))
        key = k3 + ((insts[0], ctr[insts[0]]) if insts else ("", 0.0),)
        for c, v in ctr.items():
            data.setdefault(key, {}).setdefault(c, {})[disp] = v
        durs.setdefault(key, {})[disp] = ns
    import re
    for key in sorted(data, key=lambda k: -sum(durs[k].values())):
        if pattern and not re.search(pattern, key[0]):
            continue
        ctr = data[key]
        n = max(len(v) for v in ctr.values())
        tag = ", %s = %.0f" % key[3] if key[3][0] else ""
        print("### %s (grid %s, block %s%s): %d dispatches, median %.2f us under counters" % (
            key[0], key[1], key[2], tag, n, statistics.median(durs[key].values()) / 1e3))
        print()
        print("| counter | mean per dispatch | min | max |")
        print("|---|---|---|---|")
        mean = {}
        for c in sorted(ctr):
            v = list(ctr[c].values())
            mean[c] = statistics.fmean(v)
            print("| %s | %.6g | %.6g | %.6g |" % (c, mean[c], min(v), max(v)))
        derived = []
        if "GRBM_GUI_ACTIVE" in mean:
            derived.append(("active cycles per XCD (GRBM_GUI_ACTIVE / 8)",
                            "%.0f" % (mean["GRBM_GUI_ACTIVE"] / 8)))
            if mean.get("SQ_VALU_MFMA_BUSY_CYCLES"):
                derived.append(("MFMA busy (of 1024 SIMDs x active cycles)", "%.3f" % (
                    mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * mean["GRBM_GUI_ACTIVE"] / 8))))
            if "SQ_INSTS_VALU" in mean:
                derived.append(("VALU instructions per CU per active cycle", "%.3f" % (
                    mean["SQ_INSTS_VALU"] / (256 * mean["GRBM_GUI_ACTIVE"] / 8))))
        if mean.get("SQ_INSTS_VALU_MFMA_MOPS_BF16"):
            derived.append(("bf16 MFMA flop (512 x MOPS)",
                            "%.6g" % (512 * mean["SQ_INSTS_VALU_MFMA_MOPS_BF16"])))
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            if c in mean:
                derived.append(("%s bytes (1024 x KiB, unscaled)" % c, "%.0f" % (1024 * mean[c])))
        if derived:
            print()
            for name, val in derived:
                print("- %s: %s" % (name, val))
        print()


# ---------------------------------------------------------------------------
# the GPU rows
# ---------------------------------------------------------------------------

class HipEvent:
    """A HIP timing event created with hipEventDisableSystemFence: recording it
    does not write back and invalidate the caches, so the interval between two
    such events holds the kernels between them and not the fences' cost (HIP
    documents the flag for events used only to measure time).  Read only
    after a device synchronisation."""
    DISABLE_SYSTEM_FENCE = 0x20000000
    _hip = None

    def __init__(self):
        if HipEvent._hip is None:
            # the HIP runtime the process already has (torch's), by its soname
            h = ctypes.CDLL("libamdhip64.so.7")
            vp = ctypes.c_void_p
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
            h.hipEventRecord.argtypes = [vp, vp]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
            h.hipEventDestroy.argtypes = [vp]
            HipEvent._hip = h
        self.ev = ctypes.c_void_p()
        rc = self._hip.hipEventCreateWithFlags(ctypes.byref(self.ev), self.DISABLE_SYSTEM_FENCE)
        assert rc == 0, "hipEventCreateWithFlags failed (%d)" % rc

    def record(self, stream):
        rc = self._hip.hipEventRecord(self.ev, stream.cuda_stream)
        assert rc == 0, "hipEventRecord failed (%d)" % rc

    def elapsed_time(self, end):
        ms = ctypes.c_float()
        rc = self._hip.hipEventElapsedTime(ctypes.byref(ms), self.ev, end.ev)
        assert rc == 0, "hipEventElapsedTime failed (%d)" % rc
        return ms.value

    def __del__(self):
        if self.ev and HipEvent._hip is not None:
            HipEvent._hip.hipEventDestroy(self.ev)


class Bench:
    def __init__(self, args):
        import numpy as np
        import torch

        import ternary_weight_only_amd as tq
        from ternary_weight_only_amd import inputs
        from ternary_weight_only_amd.binding import lib

        self.np, self.torch, self.tq, self.inputs = np, torch, tq, inputs
        self.args = args
        self.G = args.G
        self.dev = torch.device("cuda:0")
        torch.cuda.set_device(self.dev)
        self.L = lib()
        self.stream = torch.cuda.Stream()
        self.sp = self.stream.cuda_stream
        self.status = tq.new_status(self.dev)
        self.stp = self.status.data_ptr()
        self.mats = inputs.stack_weights(threads=16)
        self.shapes = inputs.stack_shapes()
        self.groups = {}
        for i, NK in enumerate(self.shapes):
            self.groups.setdefault(NK, []).append(i)
        self.w_dev = [self.bf16(w) for w in self.mats]
        self.x_dec_host = [inputs.stack_decode_activation(i, K)
                           for i, (N, K) in enumerate(self.shapes)]
        self.x_dec = [self.bf16(x) for x in self.x_dec_host]
        self.i64s = ctypes.c_int64 * len(self.shapes)
        self.g_ns = self.i64s(*[N for N, K in self.shapes])
        self.g_ks = self.i64s(*[K for N, K in self.shapes])
        self.weights = sum(N * K for N, K in self.shapes)
        self.captured = {}  # GPU results the cpu row checks against the oracle
        self.rows = {}

    # helpers
    def bf16(self, a):
        np, torch = self.np, self.torch
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(self.dev).view(
            torch.bfloat16)

    @staticmethod
    def ptrs(ts):
        return (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])

    def ok(self, rc):
        assert rc == 0, "library call failed: %s" % self.L.tq_status_string(rc).decode()

    def check_status(self):
        self.torch.cuda.synchronize()
        st = int(self.status.item())
        assert st == 0, "device status %d" % st

    def event(self):
        """A timing event (HipEvent, or torch's with --torch-events)."""
        if self.args.torch_events:
            return self.torch.cuda.Event(enable_timing=True)
        return HipEvent()

    def chain(self, body, inner, reps=4):
        """Median time (ms) of one body(i) call over `reps` chains of `inner`
        calls between HIP events on the bench stream (the first chain is a
        warm-up)."""
        torch = self.torch
        res = []
        with torch.cuda.stream(self.stream):
            for _ in range(reps):
                e0 = self.event()
                e1 = self.event()
                e0.record(self.stream)
                for i in range(inner):
                    body(i)
                e1.record(self.stream)
                res.append((e0, e1))
        self.check_status()
        t = sorted(a.elapsed_time(b) for a, b in res[1:])
        return t[len(t) // 2] / inner

    def quantize_ring(self, G, slots=RING):
        """`slots` copies of the stack packed at G (one batched launch per shape)."""
        torch, tq = self.torch, self.tq
        P = [[torch.empty(tq.packed_bytes(N, K, G), dtype=torch.uint8, device=self.dev)
              for N, K in self.shapes] for _ in range(slots)]
        S = [[torch.empty(N * (K // G), dtype=torch.float16, device=self.dev)
              for N, K in self.shapes] for _ in range(slots)]
        for slot in range(slots):
            for (N, K), idx in self.groups.items():
                self.ok(self.L.tq_quantize_pack_batched(
                    len(idx), self.ptrs([self.w_dev[i] for i in idx]), N, K, G,
                    self.ptrs([P[slot][i] for i in idx]), self.ptrs([S[slot][i] for i in idx]),
                    self.stp, self.sp))
        self.check_status()
        return P, S

    def packed_bytes(self, G):
        return sum(self.tq.packed_bytes(N, K, G) + 2 * N * (K // G) for N, K in self.shapes)

    # ---- the step ----
    def row_step(self):
        args, torch, tq, L = self.args, self.torch, self.tq, self.L
        G, MP = self.G, args.prefill_m
        P, S = self.quantize_ring(G)
        self.captured["step_packed"] = [p.cpu().numpy() for p in P[0]]
        self.captured["step_scales"] = [s.cpu().view(torch.int16).numpy() for s in S[0]]
        y_dec = [torch.empty(1, N, dtype=torch.float32, device=self.dev) for N, K in self.shapes]
        codes = [torch.empty(N, K, dtype=torch.int8, device=self.dev) for N, K in self.shapes]
        x_pre = {K: self.bf16(self.inputs.prefill_activation(MP, K))
                 for K in sorted({k for _, k in self.shapes})}
        y_pre = [torch.empty(MP, N, dtype=torch.float32, device=self.dev) for N, K in self.shapes]
        ptrs = self.ptrs
        grouped = {slot: (ptrs(self.x_dec), ptrs(P[slot]), ptrs(S[slot]), ptrs(y_dec))
                   for slot in range(RING)}
        gcalls = {slot: (ptrs([x_pre[K] for N, K in self.shapes]), ptrs(P[slot]), ptrs(S[slot]),
                         ptrs(y_pre)) for slot in range(RING)}
        qcalls = {slot: [(N, K, len(idx), ptrs([self.w_dev[i] for i in idx]),
                          ptrs([P[slot][i] for i in idx]), ptrs([S[slot][i] for i in idx]),
                          ptrs([codes[i] for i in idx]))
                         for (N, K), idx in self.groups.items()] for slot in range(RING)}
        stp, sp = self.stp, self.sp

        def run_gemv(slot):
            ax, ap, asc, ay = grouped[slot]
            self.ok(L.tq_gemv_grouped(len(self.shapes), ax, ap, asc, ay, self.g_ns, self.g_ks,
                                      G, stp, sp))

        def run_gemm(slot):
            ax, ap, asc, ay = gcalls[slot]
            self.ok(L.tq_gemm_grouped(len(self.shapes), ax, ap, asc, ay, MP, self.g_ns,
                                      self.g_ks, G, stp, sp))

        def run_quant(slot):
            for N, K, n, aw, ap, asc, _ in qcalls[slot]:
                self.ok(L.tq_quantize_pack_batched(n, aw, N, K, G, ap, asc, stp, sp))

        def run_unpack(slot):
            for N, K, n, _, ap, _, ac in qcalls[slot]:
                self.ok(L.tq_unpack_batched(n, ap, N, K, G, ac, stp, sp))

        run = {"gemv": run_gemv, "gemm": run_gemm, "quant": run_quant, "unpack": run_unpack}
        order = ("quant", "unpack", "gemm", "gemv")

        def step(t, evs=None):
            wr = (t + 2) % RING
            slots = {"quant": wr, "unpack": wr, "gemm": (t + 4) % RING, "gemv": t % RING}
            with torch.cuda.stream(self.stream):
                if evs is not None:
                    evs[0].record(self.stream)
                for j, name in enumerate(order):
                    run[name](slots[name])
                    if evs is not None:
                        evs[j + 1].record(self.stream)

        for t in range(args.warmup):
            step(t)
        torch.cuda.synchronize()
        evs = [[self.event() for _ in range(len(order) + 1)]
               for _ in range(args.steps)]
        t0 = time.perf_counter()
        for t in range(args.steps):
            step(args.warmup + t, evs[t])
        torch.cuda.synchronize()
        self.wall = time.perf_counter() - t0
        self.check_status()
        # outputs of the last step for the oracle check (every slot holds the same bytes)
        self.captured["step_y_dec"] = [y.cpu().numpy() for y in y_dec]
        self.captured["step_y_pre"] = {i: y_pre[i].cpu().numpy() for i in (0, 2)}
        self.captured["step_codes"] = {i: codes[i].cpu().numpy() for i in (0, 71)}
        # the GEMV kernel alone: the decode pass over all slots back to back
        launch_ms = self.chain(run_gemv, RING)

        per = {name: 0.0 for name in order}
        total = 0.0
        for t in range(args.steps):
            for j, name in enumerate(order):
                per[name] += evs[t][j].elapsed_time(evs[t][j + 1])
            total += evs[t][0].elapsed_time(evs[t][-1])
        per = {k: v / args.steps for k, v in per.items()}
        self.ms_per_step = total / args.steps
        pb = self.packed_bytes(G)
        gemm_flops = sum(2.0 * MP * N * K for N, K in self.shapes)
        gemv_gbs = pb / (per["gemv"] * 1e-3) / 1e9
        gemm_tf = gemm_flops / (per["gemm"] * 1e-3) / 1e12
        quant_bytes = self.weights * 2 + pb
        unpack_bytes = pb + self.weights
        self.value = gemv_gbs
        self.rows["decode_gemv"] = {
            "config": "72-matrix FFN stack, G=%d, M=1, one grouped launch" % G,
            "ms": per["gemv"], "GB/s": gemv_gbs, "frac_hbm": gemv_gbs / HBM_PEAK_GBS,
            "kernel_us": launch_ms * 1e3,
            "kernel_GB/s": pb / (launch_ms * 1e-3) / 1e9,
            "kernel_frac_hbm": pb / (launch_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "launches": 1, "bytes_per_step": pb}
        self.rows["prefill_gemm"] = {
            "config": "72-matrix FFN stack, G=%d, M=%d, one grouped launch" % (G, MP),
            "ms": per["gemm"], "TFLOP/s": gemm_tf, "frac_mfma": gemm_tf / MFMA_BF16_PEAK_TFLOPS,
            "M": MP, "flop_per_step": gemm_flops}
        self.rows["quantize_pack"] = {
            "ms": per["quant"], "GB/s": quant_bytes / (per["quant"] * 1e-3) / 1e9,
            "bytes_per_step": quant_bytes}
        self.rows["unpack"] = {
            "ms": per["unpack"], "GB/s": unpack_bytes / (per["unpack"] * 1e-3) / 1e9,
            "bytes_per_step": unpack_bytes}
        achieved = pb / (launch_ms * 1e-3) / 1e9
        h = source_hash("tq_gemv_m1.hip")
        self.roofline = {
            "kernel": "gemv_m1_kernel (tq_gemv_grouped)", "bound": "hbm",
            "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": GEMV_TRAFFIC.get(h),
            "algorithmic_bytes_per_launch": pb,
            "avg_launch_us": round(launch_ms * 1e3, 3),
            "timing": "median of 3 chains of the decode pass over all %d slots "
                      "(%d back-to-back launches) between HIP events" % (RING, RING)}
        self.P128, self.S128 = P, S
        del y_pre, codes

    # ---- the stack decode at G = 64 ----
    def row_gemv_g64(self):
        torch, L = self.torch, self.L
        G = 64
        P, S = self.quantize_ring(G)
        self.captured["g64_packed"] = [p.cpu().numpy() for p in P[0]]
        y = [torch.empty(1, N, dtype=torch.float32, device=self.dev) for N, K in self.shapes]
        calls = {slot: (self.ptrs(self.x_dec), self.ptrs(P[slot]), self.ptrs(S[slot]),
                        self.ptrs(y)) for slot in range(RING)}

        def run(slot):
            ax, ap, asc, ay = calls[slot]
            self.ok(L.tq_gemv_grouped(len(self.shapes), ax, ap, asc, ay, self.g_ns, self.g_ks,
                                      G, self.stp, self.sp))

        ms = self.chain(run, RING)
        self.captured["g64_y"] = [t.cpu().numpy() for t in y]
        self.captured["g64_scales"] = [s.cpu().view(torch.int16).numpy() for s in S[0]]
        pb = self.packed_bytes(G)
        gbs = pb / (ms * 1e-3) / 1e9
        self.rows["decode_gemv_g64"] = {
            "config": "72-matrix FFN stack, G=64, M=1, one grouped launch per pass",
            "kernel_us": ms * 1e3, "GB/s": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
            "bytes_per_pass": pb, "in_step": False,
            "timing": "median of 3 chains over %d ring slots" % RING}
        del P, S

    # ---- the stack GEMM at M = 2048 ----
    def row_gemm_m2048(self):
        torch, L = self.torch, self.L
        G, M = self.G, 2048
        if not hasattr(self, "P128"):
            self.P128, self.S128 = self.quantize_ring(G, slots=1)
        P, S = self.P128[0], self.S128[0]
        x = {K: self.bf16(self.inputs.prefill_activation(M, K)) for K in (1024, 3584)}
        y = [torch.empty(M, N, dtype=torch.float32, device=self.dev) for N, K in self.shapes]
        calls = {(N, K): (len(idx), self.ptrs([x[K]] * len(idx)), self.ptrs([P[i] for i in idx]),
                          self.ptrs([S[i] for i in idx]), self.ptrs([y[i] for i in idx]))
                 for (N, K), idx in self.groups.items()}
        out = {}
        batched_ms = 0.0
        for (N, K), (n, ax, ap, asc, ay) in calls.items():
            def run(_):
                self.ok(L.tq_gemm_batched(n, ax, ap, asc, ay, M, N, K, G, self.stp, self.sp))
            ms = self.chain(run, 2)
            flops = 2.0 * M * N * K * n
            tf = flops / (ms * 1e-3) / 1e12
            out["%dx W[%d,%d]" % (n, N, K)] = {"ms": ms, "TFLOP/s": tf,
                                               "frac_mfma": tf / MFMA_BF16_PEAK_TFLOPS}
            batched_ms += ms
        g = (self.ptrs([x[K] for N, K in self.shapes]), self.ptrs(P), self.ptrs(S), self.ptrs(y))

        def run_grouped(_):
            self.ok(L.tq_gemm_grouped(len(self.shapes), *g, M, self.g_ns, self.g_ks, G,
                                      self.stp, self.sp))
        total_ms = self.chain(run_grouped, 2)
        flops = sum(2.0 * M * N * K for N, K in self.shapes)
        tf = flops / (total_ms * 1e-3) / 1e12
        self.captured["m2048_y"] = {i: y[i][:64].cpu().numpy() for i in (0, 2)}
        self.rows["prefill_gemm_m2048"] = {
            "config": "72-matrix FFN stack, G=%d, M=2048, one grouped launch" % G,
            "ms": total_ms, "TFLOP/s": tf, "frac_mfma": tf / MFMA_BF16_PEAK_TFLOPS,
            "batched_per_shape": out,
            "batched_TFLOP/s": flops / (batched_ms * 1e-3) / 1e12, "in_step": False,
            "timing": "median of 3 chains of 2 launches (the grouped launch, and each "
                      "shape's batched launch)"}
        del y

    # ---- the 8B-class FFN matrices ----
    def row_dense8b(self):
        torch, tq, L, inputs = self.torch, self.tq, self.L, self.inputs
        G = 128
        res = {}
        for name, N, K in inputs.dense8b_shapes():
            w = inputs.dense8b_weight(N, K)
            wd = self.bf16(w)
            packed, scales = tq.quantize_pack(wd, G, status=self.status)
            self.check_status()
            del wd
            self.captured["d8_packed_%d" % N] = packed.cpu().numpy()
            self.captured["d8_scales_%d" % N] = scales.cpu().view(torch.int16).numpy()
            nbytes = packed.numel() + 2 * scales.numel()
            copies = max(2, -(-(1 << 30) // nbytes))
            ring = [(packed.clone(), scales.clone()) for _ in range(copies)]
            for M in (1, 4, 16):
                xh = inputs.dense8b_activation(M, N, K)
                x = self.bf16(xh)
                y = torch.empty(M, N, dtype=torch.float32, device=self.dev)

                def run(i):
                    p, s = ring[i]
                    self.ok(L.tq_gemv(x.data_ptr(), p.data_ptr(), s.data_ptr(), M, N, K, G,
                                      y.data_ptr(), self.stp, self.sp))

                ms = self.chain(run, copies)
                self.captured["d8_y_%d_%d" % (N, M)] = y.cpu().numpy()
                gbs = nbytes / (ms * 1e-3) / 1e9
                res["W[%d,%d] M=%d" % (N, K, M)] = {
                    "kernel_us": ms * 1e3, "GB/s": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
                    "TFLOP/s": 2.0 * M * N * K / (ms * 1e-3) / 1e12}
            del ring
        self.rows["dense8b_gemv"] = {
            "config": "W[14336,4096] and W[4096,14336], G=128, tq_gemv at M=1,4,16",
            "cases": res, "bytes_per_launch": nbytes, "in_step": False,
            "timing": "median of 3 chains over a ring of copies (>= 1 GiB)"}

    # ---- decode to bf16 ----
    def row_dequant(self):
        torch, L = self.torch, self.L
        G = self.G
        if not hasattr(self, "P128"):
            self.P128, self.S128 = self.quantize_ring(G)
        P, S = self.P128, self.S128
        w_hat = [torch.empty(N, K, dtype=torch.bfloat16, device=self.dev) for N, K in self.shapes]
        calls = {slot: [(N, K, len(idx), self.ptrs([P[slot][i] for i in idx]),
                         self.ptrs([S[slot][i] for i in idx]), self.ptrs([w_hat[i] for i in idx]))
                        for (N, K), idx in self.groups.items()] for slot in range(len(P))}

        def run(slot):
            for N, K, n, ap, asc, aw in calls[slot % len(P)]:
                self.ok(L.tq_dequantize_batched(n, ap, asc, aw, N, K, G, self.stp, self.sp))

        ms = self.chain(run, RING)
        self.captured["dequant_w_hat"] = {i: w_hat[i].cpu().view(torch.int16).numpy()
                                          for i in (0, 71)}
        b = self.packed_bytes(G) + 2 * self.weights
        self.rows["decode_bf16"] = {"ms": ms, "GB/s": b / (ms * 1e-3) / 1e9,
                                    "frac_hbm": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                    "bytes_per_pass": b, "launches": len(self.groups),
                                    "in_step": False}
        del w_hat

    # ---- 2-bit format ----
    def row_gemv2(self):
        torch, L = self.torch, self.L
        G = self.G
        P2 = {}
        for (N, K), idx in self.groups.items():
            out2 = [(torch.empty(N, K // 4, dtype=torch.uint8, device=self.dev),
                     torch.empty(N, K // G, dtype=torch.float16, device=self.dev)) for _ in idx]
            self.ok(L.tq_quantize_pack2_batched(len(idx), self.ptrs([self.w_dev[i] for i in idx]),
                                                N, K, G, self.ptrs([p for p, _ in out2]),
                                                self.ptrs([s for _, s in out2]), self.stp,
                                                self.sp))
            P2.update(zip(idx, out2))
        self.check_status()
        self.captured["gemv2_packed"] = {i: P2[i][0].cpu().numpy() for i in (0, 71)}
        nm = range(len(self.shapes))
        slots = [{i: (P2[i][0].clone(), P2[i][1].clone()) for i in nm} for _ in range(RING)]
        y2 = [torch.empty(1, N, dtype=torch.float32, device=self.dev) for N, K in self.shapes]
        calls = [(self.ptrs(self.x_dec), self.ptrs([sl[i][0] for i in nm]),
                  self.ptrs([sl[i][1] for i in nm]), self.ptrs(y2)) for sl in slots]

        def run(slot):
            ax, ap, asc, ay = calls[slot]
            self.ok(L.tq_gemv2_grouped(len(self.shapes), ax, ap, asc, ay, self.g_ns, self.g_ks,
                                       G, self.stp, self.sp))

        ms = self.chain(run, RING)
        self.captured["gemv2_y"] = {i: y2[i].cpu().numpy() for i in (0, 71)}
        b = sum(N * K // 4 + 2 * N * (K // G) for N, K in self.shapes)
        self.rows["decode_gemv_2bit"] = {
            "ms": ms, "GB/s": b / (ms * 1e-3) / 1e9, "frac_hbm": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "Tweights/s": self.weights / (ms * 1e-3) / 1e12, "bytes_per_pass": b, "launches": 1,
            "in_step": False}
        # the 2-bit prefill matmul on the matrix cores: one tq_gemm2_batched launch per shape
        MP = self.args.prefill_m
        xs = {K: self.bf16(self.inputs.prefill_activation(MP, K))
              for K in sorted({k for _, k in self.shapes})}
        yp = [torch.empty(MP, N, dtype=torch.float32, device=self.dev) for N, K in self.shapes]
        pcalls = [(N, K, len(idx), self.ptrs([xs[K]] * len(idx)),
                   self.ptrs([slots[0][i][0] for i in idx]), self.ptrs([slots[0][i][1] for i in idx]),
                   self.ptrs([yp[i] for i in idx])) for (N, K), idx in self.groups.items()]

        def run_mm(_):
            for N, K, n, ax, ap, asc, ay in pcalls:
                self.ok(L.tq_gemm2_batched(n, ax, ap, asc, ay, MP, N, K, G, self.stp, self.sp))

        ms2 = self.chain(run_mm, 2)
        self.captured["gemm2_y"] = {i: yp[i][:8].cpu().numpy() for i in (0, 71)}
        flops = sum(2.0 * MP * N * K for N, K in self.shapes)
        tf = flops / (ms2 * 1e-3) / 1e12
        self.rows["prefill_gemm_2bit"] = {
            "config": "72-matrix FFN stack, 2-bit G=%d, M=%d, one tq_gemm2_batched launch per shape"
                      % (G, MP),
            "ms": ms2, "TFLOP/s": tf, "frac_mfma": tf / MFMA_BF16_PEAK_TFLOPS, "launches": 2,
            "in_step": False, "timing": "median of 3 chains of 2 passes"}

    # ---- W4A16 ----
    def row_w4a16(self):
        np, torch, L, inputs = self.np, self.torch, self.L, self.inputs
        G = self.G
        W4 = {}
        host = {}
        for i, (N, K) in enumerate(self.shapes):
            pk, sc, bi = inputs.w4a16_problem(5000 + i, N, K, G)
            if i in (0, 71):
                host[i] = (pk, sc, bi)
            W4[i] = tuple(torch.from_numpy(a.view(np.int32 if a.dtype == np.uint32 else np.int16))
                          .to(self.dev) for a in (pk, sc, bi))
        nm = range(len(self.shapes))
        y4 = [torch.empty(1, N, dtype=torch.bfloat16, device=self.dev) for N, K in self.shapes]
        slots = [{i: tuple(t.clone() for t in W4[i]) for i in nm} for _ in range(RING)]
        calls = [(self.ptrs(self.x_dec), self.ptrs([sl[i][0] for i in nm]),
                  self.ptrs([sl[i][1] for i in nm]), self.ptrs([sl[i][2] for i in nm]),
                  self.ptrs(y4)) for sl in slots]

        def run(slot):
            ax, ap, asc, abi, ay = calls[slot]
            self.ok(L.tq_w4a16_gemv_grouped(len(self.shapes), ax, ap, asc, abi, ay, self.g_ns,
                                            self.g_ks, G, self.sp))

        ms = self.chain(run, RING)
        self.captured["w4a16"] = {i: host[i] + (y4[i].float().cpu().numpy(),) for i in (0, 71)}
        b = sum(N * K // 2 + 4 * N * (K // G) for N, K in self.shapes)
        self.rows["decode_gemv_w4a16"] = {
            "ms": ms, "GB/s": b / (ms * 1e-3) / 1e9, "frac_hbm": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "Tweights/s": self.weights / (ms * 1e-3) / 1e12, "bytes_per_pass": b, "launches": 1,
            "in_step": False}
        # the W4A16 prefill matmul on the matrix cores: one tq_w4a16_gemm launch per matrix
        MP = self.args.prefill_m
        xs = {K: self.bf16(self.inputs.prefill_activation(MP, K))
              for K in sorted({k for _, k in self.shapes})}
        yp = [torch.empty(MP, N, dtype=torch.bfloat16, device=self.dev) for N, K in self.shapes]
        sl = slots[0]

        gcalls = [(N, K, len(idx), self.ptrs([xs[K]] * len(idx)), self.ptrs([sl[i][0] for i in idx]),
                   self.ptrs([sl[i][1] for i in idx]), self.ptrs([sl[i][2] for i in idx]),
                   self.ptrs([yp[i] for i in idx])) for (N, K), idx in self.groups.items()]

        def run_gemm(_):
            for N, K, n, ax, ap, asc, abi, ay in gcalls:
                self.ok(L.tq_w4a16_gemm_batched(n, ax, ap, asc, abi, MP, N, K, G, ay, self.sp))

        ms = self.chain(run_gemm, 2)
        flops = sum(2.0 * MP * N * K for N, K in self.shapes)
        self.captured["w4a16_gemm"] = {i: host[i] + (yp[i][:8].float().cpu().numpy(),)
                                       for i in (0, 71)}
        self.rows["prefill_gemm_w4a16"] = {
            "config": "72-matrix FFN stack, W4A16 G=%d, M=%d, one tq_w4a16_gemm_batched launch "
                      "per shape" % (G, MP),
            "ms": ms, "TFLOP/s": flops / (ms * 1e-3) / 1e12,
            "frac_mfma": flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, "launches": 2,
            "in_step": False, "timing": "median of 3 chains of 2 passes"}
        del yp, xs

    # ---- QAT forward ----
    def row_qat(self):
        torch, L = self.torch, self.L
        G = self.G
        w_hat = [torch.empty(N, K, dtype=torch.bfloat16, device=self.dev) for N, K in self.shapes]
        calls = [(N, K, len(idx), self.ptrs([self.w_dev[i] for i in idx]),
                  self.ptrs([w_hat[i] for i in idx])) for (N, K), idx in self.groups.items()]

        def run(_):
            for N, K, n, aw, awh in calls:
                self.ok(L.tq_fake_quantize_batched(n, aw, N, K, G, awh, None, self.stp, self.sp))

        ms = self.chain(run, RING)
        self.captured["qat_w_hat"] = {i: w_hat[i].cpu().view(torch.int16).numpy() for i in (0, 71)}
        b = 4 * self.weights
        self.rows["qat_forward"] = {"ms": ms, "GB/s": b / (ms * 1e-3) / 1e9,
                                    "frac_hbm": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                    "bytes_per_pass": b, "launches": len(self.groups),
                                    "in_step": False}
        del w_hat
        # the same forward from fp32 latent weights (the bf16 weights widened)
        w32 = [w.float() for w in self.w_dev]
        h32 = [torch.empty_like(w) for w in w32]
        calls32 = [(N, K, len(idx), self.ptrs([w32[i] for i in idx]),
                    self.ptrs([h32[i] for i in idx])) for (N, K), idx in self.groups.items()]

        def run32(_):
            for N, K, n, aw, awh in calls32:
                self.ok(L.tq_fake_quantize_f32_batched(n, aw, N, K, G, awh, None, self.stp,
                                                       self.sp))

        ms = self.chain(run32, 4)
        self.captured["qat32_w_hat"] = {i: h32[i].cpu().numpy() for i in (0, 71)}
        b = 8 * self.weights
        self.rows["qat_forward_f32"] = {"ms": ms, "GB/s": b / (ms * 1e-3) / 1e9,
                                        "frac_hbm": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                        "bytes_per_pass": b, "launches": len(self.groups),
                                        "in_step": False}
        del w32, h32

    # ---- ceilings ----
    def row_ceilings(self):
        torch, L = self.torch, self.L
        sink = torch.zeros(65535 * 512, dtype=torch.int32, device=self.dev)
        pass_bytes = self.packed_bytes(128) // 16 * 16
        bufs = [torch.empty(pass_bytes, dtype=torch.uint8, device=self.dev) for _ in range(RING)]
        for b in bufs:
            b.fill_(1)
        big = torch.empty(1 << 30, dtype=torch.uint8, device=self.dev)
        big.fill_(1)
        out = {}
        for grid in (512, 1024):
            def run(i, grid=grid):
                self.ok(L.tq_probe_read_stream(bufs[i].data_ptr(), pass_bytes, grid,
                                               sink.data_ptr(), self.sp))
            ms = self.chain(run, RING)
            out["read_stream_57.8MB_grid%d" % grid] = {
                "us": ms * 1e3, "GB/s": pass_bytes / (ms * 1e-3) / 1e9}

            def run_big(i, grid=grid):
                self.ok(L.tq_probe_read_stream(big.data_ptr(), big.numel(), grid,
                                               sink.data_ptr(), self.sp))
            ms = self.chain(run_big, 2)
            out["read_stream_1GiB_grid%d" % grid] = {
                "us": ms * 1e3, "GB/s": big.numel() / (ms * 1e-3) / 1e9}

            # one 8B-class matrix's bytes (packed + scales) per launch, each
            # launch on the next stretch of the 1 GiB buffer
            nbytes8 = D8_LAUNCH_BYTES // 16 * 16
            stretches = big.numel() // nbytes8

            def run_d8(i, grid=grid):
                self.ok(L.tq_probe_read_stream(big.data_ptr() + i * nbytes8, nbytes8, grid,
                                               sink.data_ptr(), self.sp))
            ms = self.chain(run_d8, stretches)
            out["read_stream_12.8MB_grid%d" % grid] = {
                "us": ms * 1e3, "GB/s": nbytes8 / (ms * 1e-3) / 1e9}
        grid, iters = 512, 4096
        fs = sink.view(torch.float32)

        def run_mfma(_):
            self.ok(L.tq_probe_mfma_bf16(iters, grid, fs.data_ptr(), self.sp))
        ms = self.chain(run_mfma, 2)
        flops = grid * 8 * iters * 8 * 16384.0
        out["mfma_bf16_16x16x32"] = {"us": ms * 1e3, "TFLOP/s": flops / (ms * 1e-3) / 1e12}
        # LDS table reads and VALU issue, per CU and core cycle (the probe reports
        # the core clock of its own loop)
        clocks = torch.zeros(2, dtype=torch.int64, device=self.dev)
        sk = sink.data_ptr()

        def per_cycle(count, ms):
            c = clocks.cpu().tolist()
            ghz = c[0] / (c[1] * 10.0) if c[1] > 0 else float("nan")
            return ghz, count / (ms * 1e-3) / 256 / (ghz * 1e9)
        lds_iters = 4096

        def run_lds(_):
            self.ok(L.tq_probe_lds_table(lds_iters, grid, sk, clocks.data_ptr(), self.sp))
        ms = self.chain(run_lds, 2)
        lds_bytes = grid * 512 * lds_iters * 128.0
        ghz, bpc = per_cycle(lds_bytes, ms)
        out["lds_table_ds_read_b128"] = {"us": ms * 1e3, "GB/s": lds_bytes / (ms * 1e-3) / 1e9,
                                         "core_GHz": ghz, "bytes_per_CU_per_cycle": bpc}
        valu_iters = 2048
        for kind, name in ((0, "valu_v_dot2_f32_bf16"), (1, "valu_v_perm_b32")):
            def run_valu(_, kind=kind):
                self.ok(L.tq_probe_valu(kind, valu_iters, grid, sk, clocks.data_ptr(), self.sp))
            ms = self.chain(run_valu, 2)
            ghz, ipc = per_cycle(grid * 8 * valu_iters * 128.0, ms)
            out[name] = {"us": ms * 1e3, "core_GHz": ghz, "wave_instr_per_CU_per_cycle": ipc}
        best_read = max(v["GB/s"] for k, v in out.items() if k.startswith("read_stream_57"))
        out["spec_hbm_GB/s"] = HBM_PEAK_GBS
        out["spec_mfma_bf16_TFLOP/s"] = MFMA_BF16_PEAK_TFLOPS
        self.ceilings = out
        if "decode_gemv" in self.rows:
            r = self.rows["decode_gemv"]
            r["kernel_frac_of_read_stream"] = r["kernel_GB/s"] / best_read
        best_d8 = max(v["GB/s"] for k, v in out.items() if k.startswith("read_stream_12.8"))
        if "dense8b_gemv" in self.rows:
            for case in self.rows["dense8b_gemv"]["cases"].values():
                case["frac_of_read_stream"] = case["GB/s"] / best_d8
        del bufs, big, sink

    # ---- the oracle on the host ----
    def row_cpu(self):
        self.cpu = cpu_baseline(self, self.args.cpu_seconds)


def _timed(fn, min_s):
    """Run fn() until min_s seconds have passed; returns (calls, seconds, last result)."""
    t0 = time.perf_counter()
    n, r = 0, None
    while True:
        r = fn()
        n += 1
        el = time.perf_counter() - t0
        if el >= min_s:
            return n, el, r


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(b, min_s):
    """The CPU oracle (unchanged) on bounded samples of the bench's workloads:
    quantize + pack, the M = 1 GEMV pass and the M = 512 prefill GEMM, at one
    thread and at the host's cores (rows split over threads).  Its results
    are then compared with the GPU outputs the rows captured: packed bytes,
    scales and codes bit-exact, matmul outputs within 1e-3 * sum |x w_hat|."""
    import numpy as np
    import oracle
    inputs = b.inputs
    G = b.G
    nt = oracle.default_threads()
    shapes, mats = b.shapes, b.mats
    out = {"cpu_model": cpu_model(), "threads_available": nt}
    checks = []

    # quantize + pack: 8 matrices at one thread, all 72 at nt threads
    def quant(idx, th):
        return [oracle.quantize_pack(mats[i], G, threads=th) for i in idx]
    n1, t1, _ = _timed(lambda: quant(range(8), 1), min_s / 2)
    ntc, tnt, qres = _timed(lambda: quant(range(72), nt), min_s / 2)
    qb8 = sum(mats[i].nbytes + b.tq.packed_bytes(*shapes[i], G) + 2 * shapes[i][0] *
              (shapes[i][1] // G) for i in range(8))
    qb72 = sum(w.nbytes + b.tq.packed_bytes(N, K, G) + 2 * N * (K // G)
               for w, (N, K) in zip(mats, shapes))
    out["quantize_pack"] = {"GB/s_1_thread": qb8 * n1 / t1 / 1e9,
                            "GB/s_threads": qb72 * ntc / tnt / 1e9, "threads": nt}
    packs = [(p, s) for p, s, _ in qres]

    # GEMV pass over the 72 matrices (M = 1, fp64)
    def gemv_pass(th):
        return [oracle.matmul(x, p, s, N, K, G, threads=th)
                for (p, s), x, (N, K) in zip(packs, b.x_dec_host, shapes)]
    nb = sum(p.nbytes + s.nbytes for p, s in packs)
    n1, t1, _ = _timed(lambda: gemv_pass(1), min_s)
    ntc, tnt, gres = _timed(lambda: gemv_pass(nt), min_s)
    gemv_1 = nb * n1 / t1 / 1e9
    gemv_nt = nb * ntc / tnt / 1e9

    # prefill GEMM, M = 512, on gate (matrix 0) and down (matrix 2) of layer 0
    M = 512
    xs = {K: inputs.prefill_activation(M, K) for K in (1024, 3584)}

    def gemm(idx, th):
        return {i: oracle.matmul(xs[shapes[i][1]], packs[i][0], packs[i][1], *shapes[i], G,
                                 threads=th) for i in idx}
    n1, t1, _ = _timed(lambda: gemm((0,), 1), min_s / 2)
    ntc, tnt, mres = _timed(lambda: gemm((0, 2), nt), min_s / 2)
    f0 = 2.0 * M * shapes[0][0] * shapes[0][1]
    f02 = f0 + 2.0 * M * shapes[2][0] * shapes[2][1]
    out["prefill_gemm_m512"] = {"GFLOP/s_1_thread": f0 * n1 / t1 / 1e9,
                                "GFLOP/s_threads": f02 * ntc / tnt / 1e9, "threads": nt}

    # ---- checks of the GPU outputs (untimed) ----
    def within(y, ref, bound, what):
        err = np.abs(np.asarray(y, np.float64) - ref)
        ok = bool((err <= 1e-3 * bound).all() and np.isfinite(y).all())
        checks.append({"what": what, "ok": ok})
        assert ok, "bench check failed: " + what

    def exact(a, bref, what):
        ok = bool(np.array_equal(a, bref))
        checks.append({"what": what, "ok": ok})
        assert ok, "bench check failed: " + what

    cap = b.captured
    if "step_packed" in cap:
        ok = all(np.array_equal(g.reshape(-1), p.reshape(-1))
                 for g, (p, _) in zip(cap["step_packed"], packs))
        ok = ok and all(np.array_equal(g.view(np.uint16).reshape(-1), s.reshape(-1))
                        for g, (_, s) in zip(cap["step_scales"], packs))
        exact(ok, True, "G=%d packed bytes and scales of all 72 matrices" % G)
        ok = all(bool((np.abs(cap["step_y_dec"][i].astype(np.float64) - gres[i][0])
                       <= 1e-3 * gres[i][1]).all()) for i in range(72))
        exact(ok, True, "decode GEMV outputs of all 72 matrices within the bound")
        for i in (0, 2):
            y_ref, bound, _ = mres[i]
            within(cap["step_y_pre"][i], y_ref, bound, "prefill GEMM M=512 matrix %d" % i)
        for i in (0, 71):
            codes, _ = oracle.unpack(packs[i][0], *shapes[i], G)
            exact(cap["step_codes"][i], codes, "unpacked codes, matrix %d" % i)
    if "g64_packed" in cap:
        q64 = [oracle.quantize_pack(w, 64, threads=nt) for w in mats]
        ok = all(np.array_equal(g.reshape(-1), p.reshape(-1)) and
                 np.array_equal(gs.view(np.uint16).reshape(-1), s.reshape(-1))
                 for g, gs, (p, s, _) in zip(cap["g64_packed"], cap["g64_scales"], q64))
        exact(ok, True, "G=64 packed bytes and scales of all 72 matrices")
        ok = True
        for i, ((p, s, _), x, (N, K)) in enumerate(zip(q64, b.x_dec_host, shapes)):
            y_ref, bound, _ = oracle.matmul(x, p, s, N, K, 64, threads=nt)
            ok = ok and bool((np.abs(cap["g64_y"][i].astype(np.float64) - y_ref)
                              <= 1e-3 * bound).all())
        exact(ok, True, "G=64 decode GEMV outputs of all 72 matrices within the bound")
    if "m2048_y" in cap:
        for i in (0, 2):
            N, K = shapes[i]
            x = inputs.prefill_activation(2048, K)[:64]
            y_ref, bound, _ = oracle.matmul(x, packs[i][0], packs[i][1], N, K, G, threads=nt)
            within(cap["m2048_y"][i], y_ref, bound, "prefill GEMM M=2048 rows 0-63, matrix %d" % i)
    for name, N, K in inputs.dense8b_shapes():
        key = "d8_packed_%d" % N
        if key not in cap:
            continue
        w = inputs.dense8b_weight(N, K)
        p, s, _ = oracle.quantize_pack(w, 128, threads=nt)
        exact(cap[key], p, "8B-class W[%d,%d] packed bytes" % (N, K))
        exact(cap["d8_scales_%d" % N].view(np.uint16), s, "8B-class W[%d,%d] scales" % (N, K))
        for M in (1, 4, 16):
            x = inputs.dense8b_activation(M, N, K)
            y_ref, bound, _ = oracle.matmul(x, p, s, N, K, 128, threads=nt)
            within(cap["d8_y_%d_%d" % (N, M)], y_ref, bound, "8B-class W[%d,%d] M=%d" % (N, K, M))
    if "dequant_w_hat" in cap:
        for i in (0, 71):
            d, _ = oracle.dequantize(packs[i][0], packs[i][1], *shapes[i], G)
            exact(cap["dequant_w_hat"][i].view(np.uint16), d, "decode to bf16, matrix %d" % i)
    if "gemv2_packed" in cap:
        for i in (0, 71):
            N, K = shapes[i]
            p2, s2, _ = oracle.quantize_pack2(mats[i], G)
            exact(cap["gemv2_packed"][i], p2, "2-bit packed bytes, matrix %d" % i)
            y_ref, bound, _ = oracle.matmul2(b.x_dec_host[i], p2, s2, N, K, G, threads=nt)
            within(cap["gemv2_y"][i], y_ref, bound, "2-bit decode GEMV, matrix %d" % i)
            if "gemm2_y" in cap:
                xp = b.inputs.prefill_activation(b.args.prefill_m, K)[:8]
                y_ref, bound, _ = oracle.matmul2(xp, p2, s2, N, K, G, threads=nt)
                within(cap["gemm2_y"][i], y_ref, bound,
                       "2-bit prefill GEMM M=%d rows 0-7, matrix %d" % (b.args.prefill_m, i))
    if "w4a16" in cap:
        for i in (0, 71):
            N, K = shapes[i]
            pk, sc, bi, yg = cap["w4a16"][i]
            y_ref, bd = oracle.w4a16_matmul(b.x_dec_host[i], pk, sc, bi, N, K, G, threads=nt)
            tol = 1e-3 * bd * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(y_ref)
            ok = bool((np.abs(yg.astype(np.float64) - y_ref) <= tol).all())
            exact(ok, True, "W4A16 decode GEMV, matrix %d" % i)
    if "w4a16_gemm" in cap:
        for i in (0, 71):
            N, K = shapes[i]
            pk, sc, bi, yg = cap["w4a16_gemm"][i]
            xp = b.inputs.prefill_activation(b.args.prefill_m, K)[:8]
            y_ref, bd = oracle.w4a16_matmul(xp, pk, sc, bi, N, K, G, threads=nt)
            tol = 1e-3 * bd * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(y_ref)
            ok = bool((np.abs(yg.astype(np.float64) - y_ref) <= tol).all())
            exact(ok, True, "W4A16 prefill GEMM M=%d rows 0-7, matrix %d" % (b.args.prefill_m, i))
    if "qat_w_hat" in cap:
        for i in (0, 71):
            f, _, _ = oracle.fake_quantize(mats[i], G)
            exact(cap["qat_w_hat"][i].view(np.uint16), f, "QAT forward, matrix %d" % i)
    if "qat32_w_hat" in cap:
        for i in (0, 71):
            w32 = inputs.bf16_bits_to_f32(mats[i]).astype(np.float32)
            f, _, _ = oracle.fake_quantize_f32(w32, G)
            exact(cap["qat32_w_hat"][i].view(np.uint32), f.view(np.uint32),
                  "QAT forward from fp32, matrix %d" % i)

    return {"value": gemv_nt, "unit": "GB/s", "cores": nt, "kind": "oracle",
            "sample": "fp64 GEMV passes (M=1) through the 72-matrix FFN stack (G=%d) on %d "
                      "threads, %d passes in %.1f s; the same at 1 thread: %.4f GB/s; "
                      "quantize+pack and the M=512 GEMM in 'detail'" % (G, nt, ntc, tnt, gemv_1),
            "single_thread_GB/s": gemv_1, "detail": out,
            "checks": {"passed": all(c["ok"] for c in checks), "count": len(checks),
                       "items": [c["what"] for c in checks]}}


def main():
    args = parse()
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.pmc_summary:
        pmc_summary(args.pmc_summary, args.kernels)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only; --gpus %d is not supported (no multi-GPU path is "
              "built)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    rows = ALL_ROWS if args.rows == "all" else tuple(r for r in args.rows.split(",") if r)
    bad = [r for r in rows if r not in ALL_ROWS]
    if bad:
        print("unknown rows %s (rows: %s)" % (bad, ",".join(ALL_ROWS)), file=sys.stderr)
        sys.exit(2)
    if args.no_cpu_baseline:
        rows = tuple(r for r in rows if r != "cpu")

    b = Bench(args)
    for r in rows:
        t0 = time.perf_counter()
        getattr(b, "row_" + r)()
        print("# row %s done in %.1f s" % (r, time.perf_counter() - t0), file=sys.stderr,
              flush=True)
    if args.calibrate_copy:
        torch = b.torch
        src = torch.empty(256 << 20, dtype=torch.uint8, device=b.dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    out = {
        "metric": METRIC,
        "value": round(b.value, 2) if hasattr(b, "value") else None,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(b.ms_per_step, 4) if hasattr(b, "ms_per_step") else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "qwen-like FFN stack: 24 layers x {gate,up W[3584,1024], down "
                               "W[1024,3584]}, G=%d; decode GEMV M=1 + prefill GEMM M=%d + "
                               "quantize/pack + unpack per step" % (args.G, args.prefill_m),
                   "G": args.G, "matrices": len(b.shapes), "weights": b.weights, "decode_M": 1,
                   "prefill_M": args.prefill_m, "parallelism": "single GPU"},
        "rows": b.rows,
    }
    if hasattr(b, "roofline"):
        out["roofline"] = b.roofline
    if hasattr(b, "ceilings"):
        out["ceilings"] = b.ceilings
    if hasattr(b, "wall"):
        out["wall_s_timed"] = round(b.wall, 4)
    if hasattr(b, "cpu"):
        out["cpu_baseline"] = b.cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
