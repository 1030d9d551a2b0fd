"""Benchmark of the ternary hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--G 128] [--prefill-m 512]

Workload: the 24-layer Qwen-like FFN stack (hidden 1024, intermediate 3584:
gate and up W[3584,1024], down W[1024,3584]; 72 matrices, 264,241,152 bf16
weights ~ N(0, 0.02)), G = 128.  One step is one pass of every step of the
hot path over that stack, in this order:
  decode GEMV, M = 1, through all 72 matrices          (tq_gemv_grouped:
      one launch for the 48 K=1024 and the 24 K=3584 matrices together)
  prefill GEMM, M = 512 tokens, through all 72 matrices (tq_gemm_batched:
      two launches, one per shape; each matrix has its own activations and output)
  quantize + pack all 72 bf16 matrices                 (tq_quantize_pack_batched:
      two launches, one per shape)
  unpack + validate all 72 packed matrices             (tq_unpack_batched: two)
The packed weights live in a ring of eight slots (480 MB, more than the
256 MB memory-side cache); step t reads slot t%8 and packs into slot
(t+2)%8, so the weights a GEMV reads were written six steps (several GB of
traffic) earlier and come from HBM, not from the caches.
Every row is direct launches (pointer arrays built once per ring slot).  HIP
events between the rows time each row on the stream the kernels run on, so
a row's time includes its launches' dispatch.

Outside the step, the decode to bf16 of every matrix of a slot (two
tq_dequantize_batched calls, one per shape) runs over all eight slots back to
back between two HIP events (median of three such chains, per pass); each
chain writes 4.2 GB, so the 256 MB memory-side cache holds at most 6% of the
writes back.  The row counts packed + scale bytes read and bf16 bytes
written.

Also outside the step, the QAT forward (tq_fake_quantize_batched: bf16
weights to their bf16 ternarized values, two launches a pass) runs eight passes
back to back between two HIP events (median of three chains); its row counts
2 bytes read and 2 written per weight.

Also outside the step, two other weight formats run the decode GEMV through
the same 72 shapes, each over eight ring-slot copies back to back between two
HIP events (median of three chains): the 2-bit ternary format (the same
scales and codes, four codes a byte; tq_gemv2_grouped, one launch a pass)
and W4A16 (seeded stored 4-bit affine codes with bf16 scales and biases;
tq_w4a16_gemv_grouped, one launch a pass).  Their rows count code plus
scale (and bias) bytes.

The roofline entry times the GEMV kernel itself: after the timed steps, the
decode pass runs over all eight slots back to back (8 launches, so each
launch's dispatch overlaps the previous kernel) between two HIP events, and
the average launch is the elapsed time / 8; every slot is read once per
chain, after 7 others (405 MB), so the weights again come from HBM.

`value` is the decode GEMV's packed-weight bandwidth: (packed code bytes +
fp16 scale bytes of the 72 matrices) / GEMV time per step.  The JSON line
also carries every row's throughput, the roofline entry of the GEMV kernel
and the CPU oracle's rate on a bounded sample of the same GEMV workload.
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
# HBM bytes per GEMV launch from rocprofv3 FETCH_SIZE and WRITE_SIZE runs of this bench, each
# scaled by the same counter on a 256 MiB copy (profiles/gemv_m1_hbm_traffic.md); valid only
# for the kernel source they were taken on (sha256 prefix of csrc/tq_gemv_m1.hip).
GEMV_TRAFFIC = {"1cfc50b97901eb3f": 60691548}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--G", type=int, default=128)
    ap.add_argument("--prefill-m", type=int, default=512)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed steps, copy 256 MiB device to device three times "
                         "(a kernel of known traffic for scaling hardware byte counters)")
    return ap.parse_args()


def gen_weights():
    """The 72 bf16 weight matrices (seeded; generated in parallel processes)."""
    from concurrent.futures import ProcessPoolExecutor
    from ternary_weight_only_amd import inputs
    jobs = [(l, p) for l in range(24) for p in range(3)]
    workers = min(16, os.cpu_count() or 1)
    with ProcessPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(_gen_one, jobs))


def _gen_one(job):
    from ternary_weight_only_amd import inputs
    return inputs.ffn_weight(job[0], job[1])


def cpu_baseline(mats, x_dec, G, seconds):
    """The CPU oracle (unchanged) on a bounded sample of the GEMV workload:
    whole passes of fp64 GEMV through the 72 packed matrices, on one core."""
    import oracle
    packed = [oracle.quantize_pack(w, G)[:2] for w in mats]
    nbytes = sum(p.nbytes + s.nbytes for p, s in packed)
    t0 = time.perf_counter()
    passes = 0
    while True:
        for (p, s), w, x in zip(packed, mats, x_dec):
            N, K = w.shape
            oracle.matmul(x, p, s, N, K, G)
        passes += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": nbytes * passes / el / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "%d full passes of M=1 fp64 GEMV through the 72-matrix FFN stack (G=%d), "
                      "single thread, %.1f s" % (passes, G, el)}


def gemv_traffic():
    import hashlib
    path = os.path.join(ROOT, "ternary_weight_only_amd", "csrc", "tq_gemv_m1.hip")
    try:
        with open(path, "rb") as f:
            h = hashlib.sha256(f.read()).hexdigest()[:16]
    except OSError:
        return None
    return GEMV_TRAFFIC.get(h)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only; --gpus %d is not supported (no multi-GPU path is "
              "built)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import ternary_weight_only_amd as tq
    from ternary_weight_only_amd import inputs
    from ternary_weight_only_amd.binding import lib

    G, MP = args.G, args.prefill_m
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = lib()

    mats = gen_weights()
    shapes = [w.shape for w in mats]
    x_dec_host = [inputs.activation(5000 + i, 1, K) for i, (N, K) in enumerate(shapes)]

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    w_dev = [bf16(w) for w in mats]
    x_dec = [bf16(x) for x in x_dec_host]
    x_pre = {K: bf16(inputs.activation(30 + K, MP, K)) for K in sorted({k for _, k in shapes})}
    RING = 8
    P = [[torch.empty(tq.packed_bytes(N, K, G), dtype=torch.uint8, device=dev) for N, K in shapes]
         for _ in range(RING)]
    S = [[torch.empty(N * (K // G), dtype=torch.float16, device=dev) for N, K in shapes]
         for _ in range(RING)]
    y_dec = [torch.empty(1, N, dtype=torch.float32, device=dev) for N, K in shapes]
    codes = [torch.empty(N, K, dtype=torch.int8, device=dev) for N, K in shapes]
    status = tq.new_status(dev)
    stp = status.data_ptr()


    # the decode pass: one grouped call over all 72 matrices (one launch);
    # the prefill pass: two batched calls (gate+up of all layers share
    # K=1024, the downs K=3584); the pointer arrays of every slot are built
    # once
    groups = {}
    for i, (N, K) in enumerate(shapes):
        groups.setdefault((N, K), []).append(i)
    arr = ctypes.c_void_p

    def ptrs(ts):
        return (arr * len(ts))(*[t.data_ptr() for t in ts])

    y_pre = [torch.empty(MP, N, dtype=torch.float32, device=dev) for N, K in shapes]
    calls = {}  # (slot, (N, K)) -> pointer arrays of the GEMV and GEMM calls
    for slot in range(RING):
        for key, idx in groups.items():
            calls[(slot, key)] = (
                len(idx), ptrs([x_dec[i] for i in idx]), ptrs([P[slot][i] for i in idx]),
                ptrs([S[slot][i] for i in idx]), ptrs([y_dec[i] for i in idx]),
                ptrs([x_pre[key[1]] for i in idx]), ptrs([y_pre[i] for i in idx]))

    # quantize/pack and unpack: one batched call per shape (48 and 24 matrices)
    qcalls = {slot: [(N, K, len(idx), ptrs([w_dev[i] for i in idx]), ptrs([P[slot][i] for i in idx]),
                      ptrs([S[slot][i] for i in idx]), ptrs([codes[i] for i in idx]))
                     for (N, K), idx in groups.items()] for slot in range(RING)}

    def run_quant(slot, stream):
        for N, K, n, aw, ap, asc, _ in qcalls[slot]:
            rc = L.tq_quantize_pack_batched(n, aw, N, K, G, ap, asc, stp, stream)
            assert rc == 0, rc

    def run_unpack(slot, stream):
        for N, K, n, _, ap, _, ac in qcalls[slot]:
            rc = L.tq_unpack_batched(n, ap, N, K, G, ac, stp, stream)
            assert rc == 0, rc

    i64s = ctypes.c_int64 * len(shapes)
    g_ns = i64s(*[N for N, K in shapes])
    g_ks = i64s(*[K for N, K in shapes])
    grouped = {slot: (ptrs(x_dec), ptrs(P[slot]), ptrs(S[slot]), ptrs(y_dec))
               for slot in range(RING)}

    def run_gemv(slot, stream):
        ax, ap, asc, ay = grouped[slot]
        rc = L.tq_gemv_grouped(len(shapes), ax, ap, asc, ay, g_ns, g_ks, G, stp, stream)
        assert rc == 0, rc

    # the prefill pass: likewise two batched calls, each problem with its own
    # output (the activations of a K are shared)
    def run_gemm(slot, stream):
        for (N, K) in groups:
            n, _, ap, asc, _, axp, ayp = calls[(slot, (N, K))]
            rc = L.tq_gemm_batched(n, axp, ap, asc, ayp, MP, N, K, G, stp, stream)
            assert rc == 0, rc

    # fill every ring slot, then check slot 0 against the oracle on sampled rows
    s0 = torch.cuda.current_stream().cuda_stream
    for slot in range(RING):
        run_quant(slot, s0)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    import oracle
    for i in (0, 2, 71):
        N, K = shapes[i]
        rows = np.array([0, 1, N // 2, N - 1])
        p_ref, s_ref, _ = oracle.quantize_pack(mats[i][rows], G)
        p = P[0][i].view(N, -1)[torch.from_numpy(rows).to(dev)].cpu().numpy()
        assert np.array_equal(p, p_ref), "bench inputs: packed bytes differ from the oracle"

    # all rows run on one side stream, every launch a direct one
    stream = torch.cuda.Stream()
    sp = stream.cuda_stream
    run = {"gemv": run_gemv, "gemm": run_gemm, "quant": run_quant, "unpack": run_unpack}

    order = ("gemv", "gemm", "quant", "unpack")

    def step(t, evs=None):
        rd, wr = t % RING, (t + 2) % RING
        slots = {"gemv": rd, "gemm": rd, "quant": wr, "unpack": wr}
        with torch.cuda.stream(stream):
            if evs is not None:
                evs[0].record(stream)
            for j, name in enumerate(order):
                run[name](slots[name], sp)
                if evs is not None:
                    evs[j + 1].record(stream)

    for t in range(args.warmup):
        step(t)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(order) + 1)]
           for _ in range(args.steps)]
    t_start = time.perf_counter()
    for t in range(args.steps):
        step(args.warmup + t, evs[t])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    assert int(status.item()) == 0, "device status %d" % int(status.item())

    # the GEMV kernel on its own: the decode pass over all slots back to back
    chain = []
    with torch.cuda.stream(stream):
        for rep in range(4):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for slot in range(RING):
                run_gemv(slot, sp)
            e1.record(stream)
            chain.append((e0, e1))
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "device status %d" % int(status.item())
    chain_ms = sorted(a.elapsed_time(b) for a, b in chain[1:])
    gemv_launches = 1
    launch_ms = chain_ms[len(chain_ms) // 2] / (RING * gemv_launches)

    # decode to bf16, outside the step: every matrix of a slot into its own
    # bf16 output, one batched call per shape (2 launches), median of 3 passes
    w_hat = [torch.empty(N, K, dtype=torch.bfloat16, device=dev) for N, K in shapes]
    dq_calls = {slot: [(N, K, len(idx), ptrs([P[slot][i] for i in idx]),
                        ptrs([S[slot][i] for i in idx]), ptrs([w_hat[i] for i in idx]))
                       for (N, K), idx in groups.items()] for slot in range(RING)}

    def run_dequant(slot, stream):
        for N, K, n, ap, asc, aw in dq_calls[slot]:
            rc = L.tq_dequantize_batched(n, ap, asc, aw, N, K, G, stp, stream)
            assert rc == 0, rc

    dq = []
    with torch.cuda.stream(stream):
        for rep in range(4):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for slot in range(RING):
                run_dequant(slot, sp)
            e1.record(stream)
            dq.append((e0, e1))
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "device status %d" % int(status.item())
    dq_ms = sorted(a.elapsed_time(b) for a, b in dq[1:])[1] / RING

    # decode GEMV over the 2-bit format, outside the step: the same matrices
    # packed four codes a byte (same scales and codes), one batched call per
    # shape over each ring slot, all slots back to back
    P2 = {}
    for (N, K), idx in groups.items():
        out2 = [(torch.empty(N, K // 4, dtype=torch.uint8, device=dev),
                 torch.empty(N, K // G, dtype=torch.float16, device=dev)) for _ in idx]
        rc = L.tq_quantize_pack2_batched(len(idx), ptrs([w_dev[i] for i in idx]), N, K, G,
                                         ptrs([p for p, _ in out2]), ptrs([s for _, s in out2]),
                                         stp, s0)
        assert rc == 0, rc
        P2.update(zip(idx, out2))
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for i in (0, 71):
        N, K = shapes[i]
        rows = np.array([0, N // 2, N - 1])
        p_ref, _, _ = oracle.quantize_pack2(mats[i][rows], G)
        p = P2[i][0][torch.from_numpy(rows).to(dev)].cpu().numpy()
        assert np.array_equal(p, p_ref), "bench inputs: 2-bit packed bytes differ from the oracle"
    P2s = {slot: {i: (P2[i][0].clone(), P2[i][1].clone()) for i in P2} for slot in range(RING)}
    del P2
    y2 = [torch.empty(1, N, dtype=torch.float32, device=dev) for N, K in shapes]
    g2_calls = {slot: (ptrs(x_dec), ptrs([P2s[slot][i][0] for i in range(len(shapes))]),
                       ptrs([P2s[slot][i][1] for i in range(len(shapes))]), ptrs(y2))
                for slot in range(RING)}

    def run_gemv2(slot, stream):
        ax, ap, asc, ay = g2_calls[slot]
        rc = L.tq_gemv2_grouped(len(shapes), ax, ap, asc, ay, g_ns, g_ks, G, stp, stream)
        assert rc == 0, rc

    g2 = []
    with torch.cuda.stream(stream):
        for rep in range(4):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for slot in range(RING):
                run_gemv2(slot, sp)
            e1.record(stream)
            g2.append((e0, e1))
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "device status %d" % int(status.item())
    g2_ms = sorted(a.elapsed_time(b) for a, b in g2[1:])[1] / RING
    packed2_bytes = sum(N * K // 4 + 2 * N * (K // G) for N, K in shapes)
    del P2s, g2_calls

    # W4A16 decode GEMV, outside the step: stored 4-bit affine parameters of
    # the same 72 shapes (seeded, both scale orientations), each ring slot a
    # copy, one batched call per shape and slot, all slots back to back
    W4 = {}
    for i, (N, K) in enumerate(shapes):
        pk, sc, bi = inputs.w4a16_problem(5000 + i, N, K, G)
        W4[i] = tuple(torch.from_numpy(a.view(np.int32 if a.dtype == np.uint32 else np.int16))
                      .to(dev) for a in (pk, sc, bi))
    y4 = [torch.empty(1, N, dtype=torch.bfloat16, device=dev) for N, K in shapes]
    W4s = {slot: {i: tuple(t.clone() for t in W4[i]) for i in W4} for slot in range(RING)}
    nm = range(len(shapes))
    w4_calls = {slot: (ptrs(x_dec), ptrs([W4s[slot][i][0] for i in nm]),
                       ptrs([W4s[slot][i][1] for i in nm]), ptrs([W4s[slot][i][2] for i in nm]),
                       ptrs(y4))
                for slot in range(RING)}

    def run_w4(slot, stream):
        ax, ap, asc, abi, ay = w4_calls[slot]
        rc = L.tq_w4a16_gemv_grouped(len(shapes), ax, ap, asc, abi, ay, g_ns, g_ks, G, stream)
        assert rc == 0, rc

    with torch.cuda.stream(stream):
        run_w4(0, sp)
    torch.cuda.synchronize()
    # sampled rows of two matrices against the oracle, to the W4A16 bar
    for i in (0, 71):
        N, K = shapes[i]
        rows = np.array([0, N // 2, N - 1])
        pk, sc, bi = (t.cpu().numpy() for t in W4[i])
        xb = x_dec[i].cpu().view(torch.int16).numpy().view(np.uint16)
        y_ref, bd = oracle.w4a16_matmul(xb, pk.view(np.uint32)[rows], sc.view(np.uint16)[rows],
                                        bi.view(np.uint16)[rows], len(rows), K, G)
        yg = y4[i].float().cpu().numpy()[0, rows].astype(np.float64)
        tol = 1e-3 * bd[0] * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(y_ref[0])
        assert (np.abs(yg - y_ref[0]) <= tol).all(), "W4A16 GEMV differs from the oracle"
    w4 = []
    with torch.cuda.stream(stream):
        for rep in range(4):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for slot in range(RING):
                run_w4(slot, sp)
            e1.record(stream)
            w4.append((e0, e1))
    torch.cuda.synchronize()
    w4_ms = sorted(a.elapsed_time(b) for a, b in w4[1:])[1] / RING
    w4_bytes = sum(N * K // 2 + 4 * N * (K // G) for N, K in shapes)
    del W4, W4s, w4_calls

    # QAT forward (fake quantization), outside the step: every bf16 matrix to
    # its bf16 w_hat (72 direct launches a pass), eight passes per chain
    fq_calls = [(N, K, len(idx), ptrs([w_dev[i] for i in idx]), ptrs([w_hat[i] for i in idx]))
                for (N, K), idx in groups.items()]

    def run_fake(stream):
        for N, K, n, aw, awh in fq_calls:
            rc = L.tq_fake_quantize_batched(n, aw, N, K, G, awh, None, stp, stream)
            assert rc == 0, rc

    fq = []
    with torch.cuda.stream(stream):
        for rep in range(4):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(RING):
                run_fake(sp)
            e1.record(stream)
            fq.append((e0, e1))
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "device status %d" % int(status.item())
    fq_ms = sorted(a.elapsed_time(b) for a, b in fq[1:])[1] / RING
    del w_hat

    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    per = {name: 0.0 for name in order}
    total_ms = 0.0
    for t in range(args.steps):
        for j, name in enumerate(order):
            per[name] += evs[t][j].elapsed_time(evs[t][j + 1])
        total_ms += evs[t][0].elapsed_time(evs[t][-1])
    per = {k: v / args.steps for k, v in per.items()}
    ms_per_step = total_ms / args.steps

    packed_bytes = sum(P[0][i].numel() + 2 * S[0][i].numel() for i in range(len(shapes)))
    weights = sum(N * K for N, K in shapes)
    gemm_flops = sum(2.0 * MP * N * K for N, K in shapes)
    gemv_gbs = packed_bytes / (per["gemv"] * 1e-3) / 1e9
    gemm_tflops = gemm_flops / (per["gemm"] * 1e-3) / 1e12
    quant_bytes = weights * 2 + packed_bytes
    unpack_bytes = packed_bytes + weights
    dequant_bytes = packed_bytes + 2 * weights
    rows = {
        "decode_gemv": {"ms": per["gemv"], "GB/s": gemv_gbs, "frac_hbm": gemv_gbs / HBM_PEAK_GBS,
                    "launches": gemv_launches, "bytes_per_step": packed_bytes},
        "prefill_gemm": {"ms": per["gemm"], "TFLOP/s": gemm_tflops,
                    "frac_mfma": gemm_tflops / MFMA_BF16_PEAK_TFLOPS, "M": MP,
                    "flop_per_step": gemm_flops},
        "quantize_pack": {"ms": per["quant"],
                                "GB/s": quant_bytes / (per["quant"] * 1e-3) / 1e9,
                                "bytes_per_step": quant_bytes},
        "decode_bf16": {"ms": dq_ms, "GB/s": dequant_bytes / (dq_ms * 1e-3) / 1e9,
                        "frac_hbm": dequant_bytes / (dq_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                        "bytes_per_pass": dequant_bytes, "launches": len(groups),
                        "in_step": False},
        "decode_gemv_2bit": {"ms": g2_ms, "GB/s": packed2_bytes / (g2_ms * 1e-3) / 1e9,
                             "frac_hbm": packed2_bytes / (g2_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                             "Tweights/s": weights / (g2_ms * 1e-3) / 1e12,
                             "bytes_per_pass": packed2_bytes, "launches": 1,
                             "in_step": False},
        "decode_gemv_w4a16": {"ms": w4_ms, "GB/s": w4_bytes / (w4_ms * 1e-3) / 1e9,
                              "frac_hbm": w4_bytes / (w4_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                              "Tweights/s": weights / (w4_ms * 1e-3) / 1e12,
                              "bytes_per_pass": w4_bytes, "launches": 1,
                              "in_step": False},
        "qat_forward": {"ms": fq_ms, "GB/s": 4 * weights / (fq_ms * 1e-3) / 1e9,
                        "frac_hbm": 4 * weights / (fq_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                        "bytes_per_pass": 4 * weights, "launches": len(groups),
                        "in_step": False},
        "unpack": {"ms": per["unpack"], "GB/s": unpack_bytes / (per["unpack"] * 1e-3) / 1e9,
                      "bytes_per_step": unpack_bytes},
    }
    out = {
        "metric": METRIC,
        "value": round(gemv_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "qwen-like FFN stack: 24 layers x {gate,up W[3584,1024], down "
                               "W[1024,3584]}, G=%d; decode GEMV M=1 + prefill GEMM M=%d + "
                               "quantize/pack + unpack per step" % (G, MP),
                   "G": G, "matrices": len(shapes), "weights": weights, "decode_M": 1,
                   "prefill_M": MP, "parallelism": "single GPU"},
        "roofline": {"kernel": "gemv_m1_kernel (tq_gemv_grouped)", "bound": "hbm",
                     "achieved": round(packed_bytes / gemv_launches / (launch_ms * 1e-3) / 1e9, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(packed_bytes / gemv_launches / (launch_ms * 1e-3) / 1e9
                                   / HBM_PEAK_GBS, 4),
                     "traffic": gemv_traffic(),
                     "avg_launch_us": round(launch_ms * 1e3, 3),
                     "timing": "median of 3 chains of the decode pass over all %d slots "
                               "(%d back-to-back launches) between HIP events"
                               % (RING, RING * gemv_launches)},
        "rows": rows,
        "wall_s_timed": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(mats, x_dec_host, G, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
