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

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
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
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
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
    P(t=0) = 0.3, P(t=+-1) = 0.35 each, four whole 2-bit codes per byte.
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
        a = N * K // (8 if fmt == "q1" else 4)
        if fmt == "q1":
            plane = torch.randint(0, 256, (a,), dtype=torch.uint8, device="cuda", generator=gen)
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
        "sweeps": per_sweep, "prefill_gemm": gemm_out,
        "roofline": roofline, "roofline_gemm": roofline_gemm, "platform_probes": probes, "cpu_baseline": cpu,
    }
    print(json.dumps(out))


def platform_probes(torch, dev):
    """What this machine sustains outside this library, as context for the
    rooflines (untimed by the step): a 1 GiB device copy (HBM read + write)
    and torch's dense bf16 matmul (the platform BLAS) at the q1 prefill
    shape 512 x 17408 x 5120, with N(0,1) operands."""
    out = {}
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
    return out


def _source_digest():
    """sha256 over the code of the kernel sources and the launch planner, with
    line comments and blank lines left out (any change to the code
    invalidates counters taken earlier; a change to a comment does not)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "ternary_group_scaled_q1_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp", ".cpp")):
            with open(os.path.join(csrc, name), encoding="utf-8") as f:
                code = [ln.split("//", 1)[0].rstrip() for ln in f]
            h.update(name.encode() + b"\0" + "\n".join(ln for ln in code if ln).encode())
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
    if kv.get("source_sha256") != _source_digest() or kv.get("sweep") != f"{dom[0]}_M{dom[1]}":
        return None, None

    def num(key):
        try:
            return int(float(kv[key]))
        except (KeyError, ValueError):
            return None

    fetch, write = num("fetch_bytes_per_launch"), num("write_bytes_per_launch")
    return (fetch + write if fetch is not None and write is not None else None), fetch


def cpu_baseline(budget_s):
    """The oracle (float64 numpy: unpack the packed blob, then a dense
    product) on a bounded sample of the decode workload, on the host cores."""
    import numpy as np

    import synth
    import ternary_group_scaled_q1_amd as lb
    from oracle import ref

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    N, K, rows = 17408, 5120, 512
    sweep = synth.WORKLOADS["decode_sweep_27b"]["stream"]
    codes, sc = synth.draw_matrix(0, sweep, 0, rows, K, None)
    blob = lb.pack("q1", codes, sc)
    x = synth.draw_x(0, sweep, 0, 1, K, "bf16")
    per_call_bytes = lb.packed_bytes("q1", rows, K) + K * 2 + rows * 4
    t0 = time.perf_counter()
    calls = 0
    while True:
        ref.product_from_blob("q1", blob, rows, K, x, "bf16")
        calls += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(per_call_bytes * calls / dt / 1e9, 4), "unit": "GB/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"q1 GEMV M=1, {rows} of the {N} rows of the 17408x5120 gate projection, x bf16; "
                      f"{calls} calls in {dt:.1f} s (oracle unpacks the blob and takes a float64 product)"}


if __name__ == "__main__":
    main()
