"""Benchmark of the packed low-bit decode GEMV and prefill GEMM on one MI355X.

One step = the whole hot path over one batch of synthetic input:
  1. the 27B-class decode weight sweep (64 blocks of q/k/v/o 5120x5120,
     gate/up 17408x5120, down 5120x17408, plus the LM head 151936x5120),
     dependency-ordered GEMV launches on one stream, captured in a HIP graph,
     once with Binary g128 (q1) weights and once with Ternary g128 2-bit-slot
     (tq2) weights, each at batch M = 1 and M = 16 (x bf16, y fp32); the
     matrices that share an input run as one fused launch (q/k/v, gate/up),
     so a block is 4 launches and the sweep 257;
  2. the two prefill GEMMs at M = 512 tokens (x bf16, y fp32): q1 weights
     17408x5120 and tq5 (5 trits/byte) weights 5120x17408.
Weights are packed once before timing (the packer is off the timed path).

value = HBM GB/s of the decode GEMVs: algorithmic bytes (packed weights +
scales + x + y of every launch) / GPU time of the sweeps (HIP events on the
launch stream).  Prefill TFLOP/s = 2*M*N*K / GPU time of each GEMM.

Outside the timed step the same line also reports: single-launch timings of
every workload shape and sweep launch over a >= 1 GiB rotation pool, each next
to a plain streaming read of the same bytes (`shapes`); platform probes
(`platform_probes`); what each part multiplies (`arithmetic`); and the CPU
oracle on the host cores (`cpu_baseline`).

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--no-shapes] [--only PART]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
# Plain copy run once before timing so that a hardware-counter pass over this
# same command can scale FETCH_SIZE / WRITE_SIZE by a kernel of known traffic.
CALIB_COPY_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemv_sweep.txt")
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s

BLOCK = [(5120, 5120)] * 4 + [(17408, 5120), (17408, 5120), (5120, 17408)]
N_BLOCKS = 64
HEAD = (151936, 5120)
SWEEP = [(f, m) for f in ("q1", "tq2") for m in (1, 16)]
GEMMS = [("q1", 512, 17408, 5120, None), ("tq5", 512, 5120, 17408, 1.0 / 3.0)]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=1.0,
                    help="seconds of oracle time per (workload shape, thread setting) of the CPU baseline")
    ap.add_argument("--no-shapes", action="store_true", help="skip the per-shape launch timings")
    ap.add_argument("--print-source-digest", action="store_true")
    ap.add_argument("--only", default=None,
                    help="run one part only, for counter passes: a sweep (q1_M1, q1_M16, tq2_M1, tq2_M16) "
                         "or a GEMM (gemm_q1, gemm_tq5); the JSON line then covers that part")
    return ap.parse_args()


def sweep_layers():
    layers = []
    for _ in range(N_BLOCKS):
        layers.extend(BLOCK)
    layers.append(HEAD)
    return layers


def gen_weights_gpu(torch, lb, fmt, layers, seed):
    """Packed blobs for every layer, drawn directly on the GPU.

    Plane A: q1 signs are i.i.d. Bernoulli(0.5), so the plane is i.i.d.
    uniform bytes (the layout only permutes bits); tq2 codes are i.i.d. with
    P(t=0) = 0.3, P(t=+-1) = 0.35 each, four whole 2-bit codes per byte; tq5
    bytes are uniform below 243 (five uniform trits each; the padding digits
    of a row's last byte are never read).
    Plane B: FP16 scales |N(0, 0.02)| + 1e-3.
    """
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1_000_003 * seed + (7 if fmt == "q1" else 11))
    offs, total = [], 0
    for (N, K) in layers:
        offs.append(total)
        total += (lb.packed_bytes(fmt, N, K) + 255) // 256 * 256
    buf = torch.empty(total, dtype=torch.uint8, device="cuda")
    for (N, K), off in zip(layers, offs):
        a = lb.packed_bytes(fmt, N, K) - N * (K // 128) * 2
        if fmt == "q1":
            plane = torch.randint(0, 256, (a,), dtype=torch.uint8, device="cuda", generator=gen)
        elif fmt == "tq5":  # five uniform trits per byte: a uniform byte below 3^5
            plane = torch.randint(0, 243, (a,), dtype=torch.uint8, device="cuda", generator=gen)
        else:
            r = torch.randint(0, 20, (a, 4), dtype=torch.uint8, device="cuda", generator=gen)
            c = (r >= 7).to(torch.uint8) + (r >= 13).to(torch.uint8)  # 0:-1 (0.35), 1:0 (0.3), 2:+1 (0.35)
            plane = c[:, 0] | (c[:, 1] << 2) | (c[:, 2] << 4) | (c[:, 3] << 6)
            del r, c
        s = (torch.randn(N * (K // 128), device="cuda", generator=gen).abs() * 0.02 + 1e-3).half()
        buf[off:off + a].copy_(plane)
        buf[off + a:off + a + 2 * s.numel()].copy_(s.view(torch.uint8))
    torch.cuda.synchronize()
    return buf, offs


def progress(msg):
    """One line per set-up phase on stderr (the result line stays alone on stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.print_source_digest:
        print(_source_digest())
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the low-bit GEMV/GEMM path runs on a single MI355X "
              "and has no multi-GPU mode; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    sweeps = [k for k in SWEEP if args.only in (None, f"{k[0]}_M{k[1]}")]
    gemm_ids = [i for i, g in enumerate(GEMMS) if args.only in (None, f"gemm_{g[0]}")]
    if not sweeps and not gemm_ids:
        print(f"--only {args.only}: no such part", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import ternary_group_scaled_q1_amd as lb

    lb.load()
    progress("library loaded")
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream
    BF = lb.DT_BF16
    F32 = lb.DT_F32

    # ---------------------------------------------------------- decode sweep
    layers = sweep_layers()
    weights = {f: gen_weights_gpu(torch, lb, f, layers, args.seed)
               for f in ("q1", "tq2") if args.only in (None, f"{f}_M1", f"{f}_M16")}
    progress(f"weights packed on the GPU: {', '.join(weights) or 'none'}")
    gx = torch.Generator(device="cuda")
    gx.manual_seed(args.seed + 99)
    xs = {(m, K): torch.randn((m, K), device=dev, generator=gx).to(torch.bfloat16)
          for m in (1, 16) for K in (5120, 17408)}
    # Launches: lists of layer indices that share one input (fused).
    launches = []
    for b in range(N_BLOCKS):
        i = len(BLOCK) * b
        launches += [[i, i + 1, i + 2], [i + 3], [i + 4, i + 5], [i + 6]]
    launches.append([len(BLOCK) * N_BLOCKS])
    # Output buffers per (M, N, slot in its launch).
    ys = {(m, N, j): torch.empty((m, N), device=dev, dtype=torch.float32)
          for m in (1, 16) for N in (5120, 17408, 151936) for j in range(3)}
    # One caller-owned GEMV workspace, reused by every launch of a sweep.
    ws_bytes = max([lb.gemv_multi_workspace_bytes(f, [layers[i][0] for i in L], m, layers[L[0]][1])
                    for f in weights for m in (1, 16) for L in launches] + [0])
    ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device=dev)

    def sweep(fmt, m):
        buf, offs = weights[fmt]
        base = buf.data_ptr()
        f = lb.FORMATS[fmt]
        s = torch.cuda.current_stream(dev).cuda_stream
        for L in launches:
            K = layers[L[0]][1]
            Ns = [layers[i][0] for i in L]
            yp = [ys[(m, N, j)].data_ptr() for j, N in enumerate(Ns)]
            if len(L) == 1:
                lb.gemv_raw(f, base + offs[L[0]], xs[(m, K)].data_ptr(), BF, yp[0], F32, m, Ns[0], K, s,
                            ws.data_ptr(), ws_bytes)
            else:
                lb.gemv_multi_raw(f, [base + offs[i] for i in L], Ns, xs[(m, K)].data_ptr(), BF, yp, F32, m, K, s,
                                  ws.data_ptr(), ws_bytes)

    sweep_bytes = {}
    for fmt, m in SWEEP:
        if fmt not in weights:
            continue
        sweep_bytes[(fmt, m)] = sum(lb.packed_bytes(fmt, N, K) + m * K * 2 + m * N * 4 for (N, K) in layers)

    graphs = {}
    for fmt, m in sweeps:
        sweep(fmt, m)  # eager warm-up (first launches initialise the code objects)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            sweep(fmt, m)
        graphs[(fmt, m)] = g
    torch.cuda.synchronize()
    progress(f"sweep graphs captured: {len(graphs)}")

    # ------------------------------------------------------- prefill GEMMs
    gemm_data = {}
    for i, (fmt, M, N, K, p0) in enumerate(GEMMS):
        if i not in gemm_ids:
            continue
        codes, sc = synth.draw_matrix(args.seed, synth.WORKLOADS["prefill_gemm_512"]["stream"], i, N, K, p0)
        w = torch.from_numpy(lb.pack(fmt, codes, sc)).to(dev)
        x = torch.from_numpy(synth.draw_x(args.seed, synth.WORKLOADS["prefill_gemm_512"]["stream"], i, M, K, "bf16").view(np.int16)).view(torch.bfloat16).to(dev)
        y = torch.empty((M, N), device=dev, dtype=torch.float32)
        gemm_data[i] = (lb.FORMATS[fmt], w, x, y, M, N, K)
        del codes, sc

    gws_bytes = max(lb.gemm_workspace_bytes(fmt, M, N, K) for (fmt, M, N, K, _) in GEMMS)
    gws = torch.zeros(max(gws_bytes, 16), dtype=torch.uint8, device=dev)

    def run_gemm(i):
        f, w, x, y, M, N, K = gemm_data[i]
        lb.gemm_raw(f, w.data_ptr(), x.data_ptr(), BF, y.data_ptr(), F32, M, N, K, sptr, gws.data_ptr(), gws_bytes)

    # Counter calibration: one plain device copy of CALIB_COPY_BYTES (untimed).
    cal_src = torch.ones(CALIB_COPY_BYTES // 4, device=dev, dtype=torch.float32)
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    torch.cuda.synchronize()
    del cal_src, cal_dst

    # ------------------------------------------------------------- timing
    parts = [("sweep", k) for k in sweeps] + [("gemm", i) for i in gemm_ids]
    ev = {p: [] for p in parts}

    def step(record):
        for p in parts:
            if record:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            if p[0] == "sweep":
                graphs[p[1]].replay()
            else:
                run_gemm(p[1])
            if record:
                e1.record(stream)
                ev[p].append((e0, e1))

    progress("timing")
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    ms = {p: sum(a.elapsed_time(b) for a, b in ev[p]) / args.steps for p in parts}
    sweep_ms = sum(ms[("sweep", k)] for k in sweeps)
    total_sweep_bytes = sum(sweep_bytes[k] for k in sweeps)
    value = total_sweep_bytes / (sweep_ms * 1e-3) / 1e9 if sweeps else None

    per_sweep = {}
    for k in sweeps:
        t = ms[("sweep", k)]
        per_sweep[f"{k[0]}_M{k[1]}"] = {
            "ms": round(t, 4), "GB_s": round(sweep_bytes[k] / (t * 1e-3) / 1e9, 1),
            "tok_s": round(k[1] / (t * 1e-3), 1), "launches": len(launches),
            "gbytes": round(sweep_bytes[k] / 1e9, 4)}
    gemm_out = {}
    for i in gemm_ids:
        fmt, M, N, K, _ = GEMMS[i]
        t = ms[("gemm", i)]
        gemm_out[f"{fmt}_{M}x{N}x{K}"] = {"ms": round(t, 4), "TFLOP_s": round(2 * M * N * K / (t * 1e-3) / 1e12, 1)}

    # Dominant kernel: the GEMV sweep with the most GPU time (its launches
    # run the GEMV kernels of that format and batch); average launch
    # duration = the sweep's event time / its launches.
    roofline = None
    if sweeps:
        dom = max(sweeps, key=lambda k: ms[("sweep", k)])
        dom_ms = ms[("sweep", dom)]
        achieved = sweep_bytes[dom] / (dom_ms * 1e-3) / 1e9
        traffic, fetch = measured_traffic(dom)
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                    "fetch_bytes_per_launch": fetch,
                    "kernel": f"gemv {dom[0]} M={dom[1]} (bf16 x, fp32 y)",
                    "avg_launch_us": round(dom_ms * 1e3 / len(launches), 3),
                    "bytes_per_launch": round(sweep_bytes[dom] / len(launches))}
    roofline_gemm = None
    if gemm_ids:
        gi = max(gemm_ids, key=lambda i: ms[("gemm", i)])
        fmt, M, N, K, _ = GEMMS[gi]
        gt = ms[("gemm", gi)]
        roofline_gemm = {"bound": "mfma", "achieved": round(2 * M * N * K / (gt * 1e-3) / 1e12, 1),
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(2 * M * N * K / (gt * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                         "kernel": f"gemm {fmt} {M}x{N}x{K}", "avg_launch_us": round(gt * 1e3, 3)}

    probes = platform_probes(torch, dev) if args.only is None else None
    shapes = None if (args.only is not None or args.no_shapes) else shape_timings(torch, lb, dev, args.seed)
    arithmetic = part_arithmetic(lb, sweeps, gemm_ids, launches, layers, ws_bytes, gws_bytes)
    cpu = None if args.no_cpu_baseline else cpu_baseline(args.cpu_seconds)

    out = {
        "metric": "low-bit GEMV HBM GB/s (% peak) + prefill GEMM TFLOP/s at 27B-class shapes",
        "value": round(value, 1) if value is not None else None, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded packed weights, N(0,1) activations)",
        "config": {"workload": "27B-class decode weight sweep (64 blocks of q/k/v/o 5120x5120, gate/up "
                               "17408x5120, down 5120x17408 + LM head 151936x5120; q1 then tq2; M=1 and M=16; "
                               "q/k/v and gate/up as fused launches, 257 per sweep) "
                               "+ prefill GEMM M=512 (q1 17408x5120, tq5 5120x17408)",
                   "hbm_fraction": round(value / HBM_PEAK_GBS, 4) if value is not None else None,
                   "only": args.only},
        "sweeps": per_sweep, "prefill_gemm": gemm_out, "arithmetic": arithmetic,
        "roofline": roofline, "roofline_gemm": roofline_gemm, "platform_probes": probes,
        "shapes": shapes, "cpu_baseline": cpu,
    }
    print(json.dumps(out))


def load_probes():
    """libprobes.so: the plain streaming-read, MFMA and empty kernels the
    platform probes time (built next to liblowbit.so; no part of the product)."""
    import ctypes
    path = os.path.join(ROOT, "ternary_group_scaled_q1_amd", "libprobes.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m ternary_group_scaled_q1_amd.build`")
    lib = ctypes.CDLL(path)
    i32, i64, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
    lib.probe_stream_read.restype, lib.probe_stream_read.argtypes = i32, [vp, i64, vp, i32, vp]
    lib.probe_mfma_bf16.restype, lib.probe_mfma_bf16.argtypes = i32, [vp, i32, i32, vp]
    lib.probe_empty.restype, lib.probe_empty.argtypes = i32, [vp]
    lib.probe_tile_read.restype, lib.probe_tile_read.argtypes = i32, [vp, i64, i32, i32, i32, vp, vp]
    return lib


def read_grid(nbytes):
    """Workgroups of 512 lanes for a streaming read of nbytes (about four
    16-byte loads per lane, at least one workgroup per CU)."""
    return int(min(max(nbytes // (16 * 512 * 4), 256), 8192))


def _graph_time_ms(torch, fn, reps=5, warm_ms=30.0):
    """Median over reps replays of a HIP graph holding fn's launches, after
    untimed replays that keep the GPU busy for at least warm_ms (a single
    warm-up replay left the clocks short of their loaded state: the first
    shape timed after a pause read up to 12% slower than the same launches
    timed again); HIP events on the replay stream."""
    import time as _time
    import warnings
    g = torch.cuda.CUDAGraph()
    with warnings.catch_warnings():
        warnings.simplefilter("error")  # an empty capture means launches went to another stream
        with torch.cuda.graph(g):
            fn()
    t0 = _time.perf_counter()
    n = 0
    while n < 2 or (_time.perf_counter() - t0) * 1e3 < warm_ms:
        g.replay()
        torch.cuda.synchronize()
        n += 1
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del g
    return sorted(times)[len(times) // 2]


def platform_probes(torch, dev):
    """What this machine sustains with plain kernels, as context for the
    rooflines (untimed by the step):
      * stream_read_GBps: the committed streaming-read kernel over 4 GiB;
      * hbm_copy_GBps: a 1 GiB device copy (read + write bytes);
      * mfma_bf16_TFLOPs: the committed MFMA kernel, four chains of
        v_mfma_f32_16x16x32_bf16 per wave with +-1 B operands that change
        every step, 16 waves per CU;
      * empty_launch_us: an empty kernel, per launch in a graph of 256;
      * dense_bf16_matmul_TFLOPs: torch's matmul (the platform BLAS) at the
        q1 prefill shape 512 x 17408 x 5120;
      * tile_read: the q1 gate/up weight bytes (2176 tiles of 16 rows x 5120)
        read in the decode kernels' order, each wave its own tile, 1 KB per
        step, with 2 or 4 steps in flight, from its first chunk, from a
        rotated chunk, or in a chunk-major layout; next to the streaming
        read of the same bytes.  Each launch reads another copy of a 1 GiB
        rotation pool; us per launch in a graph of 64."""
    pr = load_probes()

    def cs():  # the stream launches go to (graph capture switches it)
        return torch.cuda.current_stream(dev).cuda_stream

    out = {}
    sink = torch.zeros(4096, device=dev, dtype=torch.uint8)
    buf = torch.empty(4 << 30, device=dev, dtype=torch.uint8)
    n = buf.numel()
    ms = _graph_time_ms(torch, lambda: [pr.probe_stream_read(buf.data_ptr(), n, sink.data_ptr(), 8192, cs())
                                        for _ in range(4)])
    out["stream_read_GBps"] = round(4 * n / (ms * 1e-3) / 1e9, 1)
    del buf
    src = torch.empty(1 << 28, device=dev, dtype=torch.float32).normal_()
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    out["hbm_copy_GBps"] = round(2 * src.numel() * 4 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del src, dst
    mo = torch.zeros(4096, device=dev, dtype=torch.float32)
    grid, iters = 512, 20000
    ms = _graph_time_ms(torch, lambda: pr.probe_mfma_bf16(mo.data_ptr(), iters, grid, cs()), reps=3)
    out["mfma_bf16_TFLOPs"] = round(grid * 8 * 4 * iters * 16384 / (ms * 1e-3) / 1e12, 1)
    ms = _graph_time_ms(torch, lambda: [pr.probe_empty(cs()) for _ in range(256)])
    out["empty_launch_us"] = round(ms * 1e3 / 256, 3)
    M, N, K = 512, 17408, 5120
    a = torch.randn((M, K), device=dev).to(torch.bfloat16)
    b = torch.randn((K, N), device=dev).to(torch.bfloat16).contiguous()
    for _ in range(3):
        c = torch.matmul(a, b)
    e0.record()
    for _ in range(20):
        c = torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    out["dense_bf16_matmul_TFLOPs"] = round(2 * M * N * K * 20 / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
    out["dense_bf16_matmul_shape"] = f"{M}x{N}x{K}"
    del a, b, c
    T, tb = 2176, 10240
    nb = T * tb
    copies = POOL_BYTES // nb
    pool = torch.empty(copies * nb, device=dev, dtype=torch.uint8)
    base = pool.data_ptr()
    tr = {}

    def tile_reads(depth, mode):
        for i in range(64):
            if pr.probe_tile_read(base + (i % copies) * nb, tb, T, depth, mode, sink.data_ptr(), cs()) != 0:
                raise RuntimeError("probe_tile_read refused its arguments")

    for depth, mode, name in ((2, 0, "own_tile_2_in_flight_us"), (4, 0, "own_tile_4_in_flight_us"),
                              (2, 1, "rotated_start_2_in_flight_us"), (2, 2, "chunk_major_2_in_flight_us")):
        tr[name] = round(_graph_time_ms(torch, lambda: tile_reads(depth, mode)) * 1e3 / 64, 2)
    tr["stream_read_us"] = round(_graph_time_ms(torch, lambda: [
        pr.probe_stream_read(base + (i % copies) * nb, nb, sink.data_ptr(), read_grid(nb), cs())
        for i in range(64)]) * 1e3 / 64, 2)
    tr["bytes"] = nb
    out["tile_read"] = tr
    del pool
    return out


# Single-launch timings: (label, format, fused row counts, K, tokens, x dtype).
# The workload shapes of the 8B-class q1 decode, the 27B-class tq2 (and tq5)
# decode, and every distinct launch of the sweep; the first is the small
# latency case (L2-resident, no bandwidth claim).
SHAPES = ([("q1 256x1024 M=1 f16 (latency)", "q1", [256], 1024, 1, "f16")]
          + [(f"q1 {N}x{K} M=1 f16", "q1", [N], K, 1, "f16") for N, K in ((24576, 4096), (4096, 12288), (151936, 4096))]
          + [(f"tq2 {N}x{K} M={m} bf16", "tq2", [N], K, m, "bf16") for N, K in ((34816, 5120), (5120, 17408))
             for m in (1, 4, 8)]
          + [(f"tq5 {N}x{K} M={m} bf16", "tq5", [N], K, m, "bf16") for N, K in ((34816, 5120), (5120, 17408))
             for m in (1, 8)]
          + [(f"{f} sweep {name} M={m} bf16", f, Ns, K, m, "bf16") for f in ("q1", "tq2") for m in (1, 16)
             for name, Ns, K in (("qkv", [5120] * 3, 5120), ("o", [5120], 5120), ("gate_up", [17408] * 2, 5120),
                                 ("down", [5120], 17408), ("lm_head", [151936], 5120))])
POOL_BYTES = 1 << 30  # rotation pool: at least 4x the 256 MB last-level cache


def shape_timings(torch, lb, dev, seed):
    """Per-launch time of each shape in SHAPES, the launch repeated over a
    rotation pool of >= 1 GiB of distinct weight copies (so no launch finds
    its weights in a cache), next to the committed streaming-read kernel
    reading the same bytes of the same buffers; median of 5 graph replays."""
    pr = load_probes()
    sink = torch.zeros(4096, device=dev, dtype=torch.uint8)
    out = {}
    for label, fmt, Ns, K, M, xdt in SHAPES:
        latency = "latency" in label
        wbytes = sum(lb.packed_bytes(fmt, N, K) for N in Ns)
        copies = 1 if latency else max(4, -(-POOL_BYTES // wbytes))
        layers = [(N, K) for _ in range(copies) for N in Ns]
        buf, offs = gen_weights_gpu(torch, lb, fmt, layers, seed)
        x = torch.randn((M, K), device=dev).to(torch.bfloat16 if xdt == "bf16" else torch.float16)
        ys = [torch.empty((M, N), device=dev, dtype=torch.float32) for N in Ns]
        wsb = lb.gemv_multi_workspace_bytes(fmt, Ns, M, K)
        ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=dev)
        f, xd = lb.FORMATS[fmt], lb.DT_BF16 if xdt == "bf16" else lb.DT_F16
        base = buf.data_ptr()
        n_launch = 1000 if latency else copies * max(1, -(-32 // copies))

        def launches():
            s = torch.cuda.current_stream(dev).cuda_stream
            for i in range(n_launch):
                c = (i % copies) * len(Ns)
                if len(Ns) == 1:
                    lb.gemv_raw(f, base + offs[c], x.data_ptr(), xd, ys[0].data_ptr(), lb.DT_F32, M, Ns[0], K, s,
                                ws.data_ptr(), wsb)
                else:
                    lb.gemv_multi_raw(f, [base + offs[c + j] for j in range(len(Ns))], Ns, x.data_ptr(), xd,
                                      [y.data_ptr() for y in ys], lb.DT_F32, M, K, s, ws.data_ptr(), wsb)

        span = offs[len(Ns) - 1] + lb.packed_bytes(fmt, Ns[-1], K)  # the weights of one launch, contiguous

        def reads():
            s = torch.cuda.current_stream(dev).cuda_stream
            for i in range(n_launch):
                c = (i % copies) * len(Ns)
                pr.probe_stream_read(base + offs[c], span // 16 * 16, sink.data_ptr(), read_grid(span), s)

        us = _graph_time_ms(torch, launches) * 1e3 / n_launch
        rd = _graph_time_ms(torch, reads) * 1e3 / n_launch
        alg = wbytes + M * K * 2 + M * sum(Ns) * 4
        plan = lb.gemv_plan(fmt, Ns, M, K, x_dtype=xdt, workspace_bytes=wsb)
        e = {"us": round(us, 3), "read_probe_us": round(rd, 3), "bytes": alg,
             "kernel": f"{plan['kernel_name']} ({plan['operands_name']}, grid {plan['grid']}, "
                       f"{plan['k_ranges']} K ranges)"}
        if not latency:
            e.update({"GB_s": round(alg / (us * 1e-6) / 1e9, 1), "hbm_frac": round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                      "read_probe_GB_s": round(span / (rd * 1e-6) / 1e9, 1), "vs_read_probe": round(rd / us, 3),
                      "pool_copies": copies})
        out[label] = e
        del buf, x, ys, ws
        torch.cuda.empty_cache()
    progress(f"shape timings: {len(out)}")
    return out


def part_arithmetic(lb, sweeps, gemm_ids, launches, layers, ws_bytes, gws_bytes):
    """What each timed part multiplies, from the plan queries of its
    launches: kernel and operand types (fp8_fp4 = bf16 x as two exact fp8
    pieces x fp4 weights on the scaled MFMA; fp8x3_fp4 = fp16 x as three
    pieces, the same MFMA; bf16 / f16 = exact operands on
    v_mfma_f32_16x16x32); every part accumulates in fp32."""
    out = {}
    for fmt, m in sweeps:
        kinds = {}
        for L in launches:
            p = lb.gemv_plan(fmt, [layers[i][0] for i in L], m, layers[L[0]][1], workspace_bytes=ws_bytes)
            k = f"{p['kernel_name']} {p['operands_name']}"
            kinds[k] = kinds.get(k, 0) + 1
        out[f"{fmt}_M{m}"] = ", ".join(f"{k} x{v}" for k, v in sorted(kinds.items()))
    for i in gemm_ids:
        fmt, M, N, K, _ = GEMMS[i]
        p = lb.gemm_plan(fmt, M, N, K, workspace_bytes=gws_bytes)
        out[f"gemm_{fmt}"] = (f"{p['kernel_name']} {p['operands_name']}"
                              + (" (x converted to fp8 pieces by a pre-pass launch)" if p["x_pieces"] else ""))
    return out


def _source_digest():
    """sha256 over the code of the kernel sources and the launch planner, with
    line comments and blank lines left out, and over the compiler flags
    they are built with (any change to the code or its flags invalidates
    counters taken earlier; a change to a comment does not).  The
    measurement probes (probes.hip) are not part of what is measured."""
    import hashlib
    from ternary_group_scaled_q1_amd import build as bld
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "ternary_group_scaled_q1_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp", ".cpp")) and name != "probes.hip":
            with open(os.path.join(csrc, name), encoding="utf-8") as f:
                code = [ln.split("//", 1)[0].rstrip() for ln in f]
            h.update(name.encode() + b"\0" + "\n".join(ln for ln in code if ln).encode())
            h.update(" ".join(bld.HIPCC_FLAGS + bld.EXTRA_FLAGS.get(name, [])).encode())
    return h.hexdigest()


def measured_traffic(dom):
    """(traffic, fetch) in HBM bytes per launch of the dominant sweep from the
    committed counter summary: FETCH_SIZE and WRITE_SIZE, each scaled by the
    calibration copy.  traffic = fetch + write when both were measured; both
    are None when there is no summary or the kernels changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            kv = dict(l.split(":", 1) for l in f if ":" in l and not l.startswith(("#", "|", " ")))
    except OSError:
        return None, None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    name = f"{dom[0]}_M{dom[1]}"
    if kv.get("source_sha256") != _source_digest():
        return None, None
    # Per-sweep figures ("fetch_bytes_per_launch.<sweep>: ..."), or one sweep's
    # figures under a "sweep: <sweep>" line.
    suffix = f".{name}" if f"fetch_bytes_per_launch.{name}" in kv else ""
    if not suffix and kv.get("sweep") != name:
        return None, None

    def num(key):
        try:
            return int(float(kv[key + suffix]))
        except (KeyError, ValueError):
            return None

    fetch, write = num("fetch_bytes_per_launch"), num("write_bytes_per_launch")
    return (fetch + write if fetch is not None and write is not None else None), fetch


# Workload shapes of the CPU baseline: (label, format, N, K, tokens, x dtype,
# rows timed).  The oracle treats every weight row alike, so a block of rows
# of full K, timed and scaled by N / rows, gives the full-shape time.
CPU_CASES = [
    ("q1 GEMV 256x1024 M=1", "q1", 256, 1024, 1, "f16", 256),
    ("q1 GEMV 24576x4096 M=1", "q1", 24576, 4096, 1, "f16", 512),
    ("q1 GEMV 4096x12288 M=1", "q1", 4096, 12288, 1, "f16", 256),
    ("q1 GEMV 151936x4096 M=1", "q1", 151936, 4096, 1, "f16", 512),
    ("tq2 GEMV 34816x5120 M=1", "tq2", 34816, 5120, 1, "bf16", 384),
    ("tq2 GEMV 34816x5120 M=8", "tq2", 34816, 5120, 8, "bf16", 384),
    ("tq2 GEMV 5120x17408 M=1", "tq2", 5120, 17408, 1, "bf16", 128),
    ("tq2 GEMV 5120x17408 M=8", "tq2", 5120, 17408, 8, "bf16", 128),
    ("q1 GEMM 512x17408x5120", "q1", 17408, 5120, 512, "bf16", 256),
    ("tq5 GEMM 512x5120x17408", "tq5", 5120, 17408, 512, "bf16", 96),
]


def host_cpu():
    """(CPU model, logical CPUs this process may run on)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return model, n


def cpu_baseline(budget_s, cases=None):
    """The oracle as it stands (float64 numpy: its own unpack of the packed
    blob, then a dense float64 product) on the host cores, on 1 thread and on
    all of them, for every workload shape of configs 1-4.  Each shape is
    timed on a block of weight rows of full K for about budget_s seconds and
    scaled to its N.  value = packed GB/s of the decode shapes (configs 2
    and 3) on all threads."""
    import numpy as np

    import synth
    import ternary_group_scaled_q1_amd as lb
    from oracle import ref

    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_info, threadpool_limits = None, None
    model, ncpu = host_cpu()
    blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1]) if threadpool_info else 1
    out, dec_bytes, dec_s = {}, 0, 0.0
    for label, fmt, N, K, M, xdt, rows in cases or CPU_CASES:
        p0 = None if fmt == "q1" else (1.0 / 3.0 if fmt == "tq5" else 0.3)
        codes, sc = synth.draw_matrix(0, 90, len(out), rows, K, p0)
        blob = lb.pack(fmt, codes, sc)
        x = synth.draw_x(0, 90, len(out), M, K, xdt)
        del codes, sc
        res = {}
        for tag, limit in (("1", 1), ("all", None)):
            ctx = threadpool_limits(limits=limit) if (threadpool_limits and limit) else _nullctx()
            with ctx:
                calls, t0 = 0, time.perf_counter()
                while True:
                    ref.product_from_blob(fmt, blob, rows, K, x, xdt)
                    calls += 1
                    if time.perf_counter() - t0 >= budget_s:
                        break
                dt = (time.perf_counter() - t0) / calls * N / rows  # seconds per full-shape call
            wb = lb.packed_bytes(fmt, N, K)
            res[f"full_shape_s_{tag}"] = round(dt, 4)
            res[f"weights_per_s_{tag}"] = round(N * K / dt, 1)
            res[f"packed_GB_s_{tag}"] = round(wb / dt / 1e9, 5)
            res[f"tok_s_{tag}"] = round(M / dt, 3)
            if tag == "all" and "GEMV" in label and "256x1024" not in label:
                dec_bytes += wb + M * K * 2 + M * N * 4
                dec_s += dt
        res["rows_timed"] = rows
        out[label] = res
    return {"value": round(dec_bytes / dec_s / 1e9, 5) if dec_s else None, "unit": "GB/s",
            "cores": int(max(blas_threads, 1)), "kind": "oracle",
            "sample": ("the oracle (its own unpack of the packed blob, then a float64 numpy product) on every "
                       "workload shape of the 8B-class q1 decode, 27B-class tq2 decode and M=512 prefill; each shape "
                       f"timed on a block of weight rows of full K for about {budget_s:g} s per thread setting and "
                       "scaled to its N; value = packed GB/s over the decode shapes on all BLAS threads "
                       "(unpack runs on one thread)"),
            "cpu_model": model, "nproc": ncpu, "blas_threads_all": int(blas_threads), "per_shape": out}


class _nullctx:
    def __enter__(self):
        return self

    def __exit__(self, *a):
        return False


if __name__ == "__main__":
    main()
