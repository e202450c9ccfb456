"""Benchmark of the 4-bit group-wise hot path on one MI355X.

Default workload: a 7B-style decoder weight stream in NF4 (block 64, fp32
absmax): 32 layers of q/k/v/o (4096x4096), gate/up (11008x4096) and down
(4096x11008), all ~ N(0, 0.02^2) fp16, seeded.  q/k/v and gate/up, which share
their input, are stored as row-concatenated matrices (codes are row-local, so
the bytes are those of the separate matrices), giving 4 GEMV launches per
layer and 128 per token.

One step = one decode token: the 128 dequant-GEMVs (M = 1, bf16 activations)
over all 6,476,005,376 weights, run back to back as two chained launches of
64 GEMVs (q4_gemv_chain: one persistent kernel per 64 products, the weight
stream of the next product prefetched across the boundary).  The token's
activations are fixed synthetic inputs, so the products are independent
(Q4_TASK_NO_WAIT).  `value` is the weight bytes (codes + absmax) streamed per
token times tokens/s.  Reported beside it: the same chain with a grid-wide
wait before every product (each reading the previous outputs' memory order),
and the 128 single-product q4_gemv launches replayed from a HIP graph.

Also reported for the token: the 128 single-product launches back to back on
the plain stream.  The same run also measures, each with HIP events on the
launch stream:
  * the one-shot quantize of all weights (HBM-resident fp16 input),
  * dequantize of a 14336x4096 INT4-asym weight to bf16,
  * the prefill GEMM M=2048, N=14336, K=4096, INT4-asym g32, bf16 x
    (TFLOP/s against the dense bf16 matrix-core peak) and the backward
    product dX = dY . What on the same weight, after 400 warm-up calls each,
  * the unfused path (dequantize to bf16, then torch.matmul / hipBLASLt) at
    the prefill shape and at M = 16 on an 11008x4096 NF4 weight, beside the
    fused kernels, and both on the prefill weight at M = 64 ... 1024 (where
    the fused product stops beating the unfused path),
  * single-matrix GEMVs on cold weights (rotating copies over 512 MiB):
    NF4 g64 1024x1024 and INT4-sym g128 4096x4096 at M = 1, NF4 g64
    11008x4096 and 4096x11008 at M = 1, 4, 16,
  * a plain 1 GiB device copy and a 4 GiB read-only row sum (torch), the
    streaming ceilings read beside the rates,
  * quantize and dequantize of the single-matrix workloads in their own
    formats on cold buffers,
  * the CPU oracle on a time-bounded sample of the token, on one thread and
    on the host's cores (cpu_baseline), and on samples of the INT4-asym
    quantize, dequantize and GEMM reference (cpu_baseline.other_ops).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
WARM_MC = 400                # warm-up calls of the matrix-core legs
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 matrix cores, TFLOP/s

LAYERS = 32
HID, FFN = 4096, 11008
# fused launch matrices of one layer: (name, N, K, [(part, rows, seed index)])
LAYER_MATS = [
    ("qkv", 3 * HID, HID, [("q", HID, 0), ("k", HID, 1), ("v", HID, 2)]),
    ("o", HID, HID, [("o", HID, 3)]),
    ("gate_up", 2 * FFN, HID, [("gate", FFN, 4), ("up", FFN, 5)]),
    ("down", HID, FFN, [("down", HID, 6)]),
]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--layers", type=int, default=LAYERS,
                   help="decoder layers in the weight stream (32 for the 7B shape)")
    p.add_argument("--no-graph", action="store_true",
                   help="skip the graph-replayed single-launch comparison")
    p.add_argument("--no-dep", action="store_true",
                   help="skip the chain with a grid-wide wait before every product (its "
                        "cooperative launch; for profiler runs)")
    p.add_argument("--cpu-seconds", type=float, default=20.0,
                   help="time budget of the CPU-oracle sample (half on one thread, half on "
                        "all cores)")
    p.add_argument("--skip-extra", action="store_true",
                   help="time only the decode token (for profiler runs)")
    p.add_argument("--only", choices=["gemm", "gemm_dx", "quantize", "dequantize", "copy",
                                      "gemv_configs", "codec_configs"],
                   help="run one leg alone, a few times, and print its timing "
                        "(for profiler runs); 'copy' is a plain 1 GiB device copy, the "
                        "reference for scaling HBM byte counters; 'gemv_configs' and "
                        "'codec_configs' are the single-matrix GEMV and quantize / "
                        "dequantize workloads on cold weights")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic():
    """HBM bytes per chained-GEMV launch from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE scaled by a plain copy's readings), or
    None when the GEMV source has changed since the counters were taken."""
    import hashlib
    prof = os.path.join(ROOT, "profiles", "gemv_chain_nf4_decode_token_7b_traffic.md")
    src = os.path.join(ROOT, "bit_group_wise_amd", "csrc", "gemv.hip")
    try:
        fields = {}
        with open(prof) as f:
            for line in f:
                k, sep, v = line.strip().partition(": ")
                if sep:
                    fields[k] = v.strip()
        with open(src, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()[:16]
        if fields.get("gemv_source_sha256_16") != sha:
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; "
                          "--gpus N > 1 is not supported"}))
        sys.exit(2)

    import torch
    from bit_group_wise_amd import q4

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    stream = torch.cuda.current_stream()

    if args.only:
        print(json.dumps(one_leg(args.only, torch, q4, dev, stream)), flush=True)
        return

    # ---------------------------------------------------------- weights
    t0 = time.time()
    gen = torch.Generator(device=dev)
    fp16 = []       # per layer: list of fused fp16 matrices
    for layer in range(args.layers):
        mats = []
        for name, N, K, parts in LAYER_MATS:
            w = torch.empty((N, K), dtype=torch.float16, device=dev)
            r0 = 0
            for _, rows, idx in parts:
                gen.manual_seed(5000 + 7 * layer + idx)
                w[r0:r0 + rows].normal_(0.0, 0.02, generator=gen)
                r0 += rows
            mats.append(w)
        fp16.append(mats)
    torch.cuda.synchronize()
    log(f"generated fp16 weights in {time.time() - t0:.1f}s")

    qw = [[q4.alloc_quantized(q4.NF4, 64, w.shape[0], w.shape[1], dev) for w in mats]
          for mats in fp16]
    n_weights = sum(w.numel() for mats in fp16 for w in mats)
    w_bytes = sum(q.nbytes() for row in qw for q in row)

    # ---------------------------------------------------------- one-shot quantize
    def quantize_all():
        for mats, qs in zip(fp16, qw):
            for w, q in zip(mats, qs):
                q4.quantize(w, q4.NF4, 64, out=q)

    quantize_all()                              # warm (and the weights used below)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    quantize_all()
    e1.record(stream)
    torch.cuda.synchronize()
    quant_ms = e0.elapsed_time(e1)
    quant_bytes = n_weights * 2 + w_bytes
    # the same weights with double-quantized absmax (8-bit codes per block,
    # a binary32 constant per 256 blocks)
    qw_dq = [[q4.quantize(w, q4.NF4_DQ, 64) for w in mats] for mats in fp16]
    torch.cuda.synchronize()
    w_bytes_dq = sum(q.nbytes() for row in qw_dq for q in row)
    log("quantized all weights (NF4, then NF4 with double-quantized absmax)")
    del fp16
    torch.cuda.empty_cache()

    # ---------------------------------------------------------- decode token
    xg = torch.Generator(device="cpu")
    xg.manual_seed(5900)
    x_h = torch.randn((1, HID), generator=xg).to(torch.bfloat16).to(dev)
    xg.manual_seed(5901)
    x_f = torch.randn((1, FFN), generator=xg).to(torch.bfloat16).to(dev)
    outs = [[torch.empty((1, q.N), dtype=torch.bfloat16, device=dev) for q in row] for row in qw]
    flat_q = [q for row in qw for q in row]
    flat_y = [y for ys in outs for y in ys]
    flat_x = [x_f if q.K == FFN else x_h for q in flat_q]
    n_launch_gemv = len(flat_q)
    sync = q4.chain_sync(dev)

    def chains(flags):
        tasks = [(x, q, y, flags) for x, q, y in zip(flat_x, flat_q, flat_y)]
        return [tasks[i:i + q4.CHAIN_MAX] for i in range(0, len(tasks), q4.CHAIN_MAX)]
    indep = chains(q4.TASK_NO_WAIT)
    dep = chains(0)
    n_chain = len(indep)

    def token_single():
        for x, q, y in zip(flat_x, flat_q, flat_y):
            q4.gemv(x, q, out=y)

    def run_chains(cs):
        for c in cs:
            q4.gemv_chain(c, sync=sync)

    # reference outputs: single-product launches; every chain must give the
    # same bits
    token_single()
    torch.cuda.synchronize()
    ref = [y.clone() for y in flat_y]
    for name, cs in (("independent", indep),) + ((("dependent", dep),) if not args.no_dep else ()):
        for y in flat_y:
            y.zero_()
        run_chains(cs)
        torch.cuda.synchronize()
        if not all(torch.equal(a, b) for a, b in zip(flat_y, ref)):
            raise RuntimeError(f"{name} chain differs from single-product launches")
    if sync.any().item():
        raise RuntimeError("chain sync words not clear")

    # the chained launches of the timed steps are separated by events on the
    # launch stream, one before the first and one after each (the kernel's
    # average launch duration; a launch's span then also holds the short
    # dispatch gap after the previous one)
    lev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(indep) + 1)]
           for _ in range(args.steps)]

    def step(evs=None):
        if evs is not None:
            evs[0].record(stream)
        for i, c in enumerate(indep):
            q4.gemv_chain(c, sync=sync)
            if evs is not None:
                evs[i + 1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0.record(stream)
    t_wall = time.perf_counter()
    for k in range(args.steps):
        step(lev[k])
    e1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_wall) * 1e3
    ms = e0.elapsed_time(e1) / args.steps
    value = w_bytes / (ms * 1e-3) / 1e9
    log(f"decode token timed: {ms:.4f} ms per step, {value:.1f} GB/s")

    timed = _timer(torch, stream)
    reps = max(args.steps // 5, 3)
    dep_ms = None if args.no_dep else timed(lambda: run_chains(dep), reps)
    # the same 128 GEMVs as single launches back to back on the plain stream
    plain_ms = timed(token_single, reps)
    single_ms = None
    if not args.no_graph:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            token_single()                         # warm on the capture stream
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            token_single()
        single_ms = timed(graph.replay, reps)
        del graph
    # double-quantized decode token: same products, chained the same way;
    # checked against single launches, then timed
    flat_qd = [q for row in qw_dq for q in row]
    yd = [torch.empty((1, q.N), dtype=torch.bfloat16, device=dev) for q in flat_qd]
    tasks_dq = [(x, q, y, q4.TASK_NO_WAIT) for x, q, y in zip(flat_x, flat_qd, yd)]
    chains_dq = [tasks_dq[i:i + q4.CHAIN_MAX] for i in range(0, len(tasks_dq), q4.CHAIN_MAX)]
    ref_dq = [q4.gemv(x, q) for x, q in zip(flat_x, flat_qd)]
    run_chains(chains_dq)
    torch.cuda.synchronize()
    if not all(torch.equal(a, b) for a, b in zip(yd, ref_dq)):
        raise RuntimeError("double-quantized chain differs from single-product launches")
    del ref_dq
    dq_ms = timed(lambda: run_chains(chains_dq), max(args.steps // 2, 3))
    log("dependent chain, single launches and double-quantized token timed")
    launch_ms = [evs[i].elapsed_time(evs[i + 1]) for evs in lev for i in range(len(indep))]
    chain_avg_us = sum(launch_ms) / len(launch_ms) * 1e3
    bytes_per_chain = w_bytes / n_chain
    chain_gbs = bytes_per_chain / (chain_avg_us * 1e-6) / 1e9

    extra = {}
    if not args.skip_extra:
        extra = extra_legs(torch, q4, dev, stream)
        log("matrix-core, codec and single-matrix legs timed")
        extra["gemv_configs_cold"] = config_gemvs(torch, q4, dev, stream)
        extra["codec_configs_cold"] = codec_configs(torch, q4, dev, stream)
        extra["hbm_copy_ceiling"] = copy_ceiling(torch, dev, stream)
        extra["hbm_read_ceiling"] = read_ceiling(torch, dev, stream)

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(args.cpu_seconds)

    result = {
        "metric": "W4A16 dequant-GEMV weight GB/s (% HBM peak); GEMM TFLOP/s at M=2048",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "7B-style decode token: 32 layers x (qkv 12288x4096, o 4096x4096, "
                        "gate_up 22016x4096, down 4096x11008), NF4 block 64 fp32 absmax, "
                        "M=1 bf16 x, 128 dequant-GEMVs per step"
                        + ("" if args.layers == LAYERS else f" ({args.layers} layers)"),
            "weights": n_weights,
            "weight_bytes_per_token": w_bytes,
            "launch": f"{n_chain} chained launches of up to {q4.CHAIN_MAX} GEMVs "
                      "(independent products)",
            "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 1),
            "wall_ms_per_step": round(wall_ms / args.steps, 4),
            "dependent_chain_ms_per_step": None if dep_ms is None else round(dep_ms, 4),
            "dependent_chain_GBps": None if dep_ms is None
            else round(w_bytes / (dep_ms * 1e-3) / 1e9, 1),
            "single_launch_plain_ms_per_step": round(plain_ms, 4),
            "single_launch_plain_GBps": round(w_bytes / (plain_ms * 1e-3) / 1e9, 1),
            "single_launch_graph_ms_per_step": None if single_ms is None else round(single_ms, 4),
            "single_launch_graph_GBps": None if single_ms is None
            else round(w_bytes / (single_ms * 1e-3) / 1e9, 1),
            "dq_decode_token": {
                "format": "NF4 block 64, absmax double-quantized (8-bit codes, binary32 "
                          "constant per 256 blocks)",
                "weight_bytes_per_token": w_bytes_dq,
                "bits_per_weight": round(w_bytes_dq * 8 / n_weights, 4),
                "ms_per_step": round(dq_ms, 4),
                "GBps": round(w_bytes_dq / (dq_ms * 1e-3) / 1e9, 1),
                "speedup_vs_fp32_absmax": round(ms / dq_ms, 3),
            },
            "quantize_all_ms": round(quant_ms, 3),
            "quantize_all_GBps": round(quant_bytes / (quant_ms * 1e-3) / 1e9, 1),
            "device": props.name,
            "cus": props.multi_processor_count,
            **extra,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "gemv_chain_kernel<NF4, bf16> (64 GEMVs per launch)",
            "achieved": round(chain_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(chain_gbs / HBM_PEAK_GBS, 4),
            "avg_launch_us": round(chain_avg_us, 3),
            "bytes_per_launch": round(bytes_per_chain),
            "gemvs_per_launch": n_launch_gemv // n_chain,
            "traffic": measured_traffic(),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


def _timer(torch, stream):
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, reps, warm=1):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps
    return timed


def _prefill_inputs(torch, q4, dev):
    """The INT4-asym g32 14336x4096 weight (~ N(0.001, 0.02^2)) and the bf16
    2048x4096 x (~ N(0, 1)) of the prefill workload, drawn on the GPU."""
    N, K, M = 14336, 4096, 2048
    gen = torch.Generator(device=dev)
    gen.manual_seed(401)
    w = torch.empty((N, K), dtype=torch.float16, device=dev).normal_(0.001, 0.02, generator=gen)
    gen.manual_seed(402)
    x = torch.empty((M, K), dtype=torch.float32, device=dev).normal_(0.0, 1.0, generator=gen)
    return w, x.to(torch.bfloat16), q4.quantize(w, q4.INT4_ASYM, 32)


def one_leg(leg, torch, q4, dev, stream):
    """One leg alone, 5 timed repetitions (for profiler runs; the matrix-core
    legs after the same warm-up as in the full run)."""
    timed = _timer(torch, stream)
    if leg == "copy":
        n = 1 << 30
        a = torch.ones(n // 4, dtype=torch.int32, device=dev)
        b = torch.empty_like(a)
        ms = timed(lambda: b.copy_(a), 5)
        return {"leg": "copy", "bytes_read": n, "bytes_written": n, "ms": round(ms, 4),
                "GBps": round(2 * n / (ms * 1e-3) / 1e9, 1)}
    if leg == "gemv_configs":
        return {"leg": leg, **config_gemvs(torch, q4, dev, stream)}
    if leg == "codec_configs":
        return {"leg": leg, **codec_configs(torch, q4, dev, stream)}
    w, x, q = _prefill_inputs(torch, q4, dev)
    N, K = w.shape
    M = x.shape[0]
    if leg == "quantize":
        ms = timed(lambda: q4.quantize(w, q4.INT4_ASYM, 32, out=q), 5)
        nb = N * K * 2 + q.nbytes()
        return {"leg": leg, "ms": round(ms, 4), "GBps": round(nb / (ms * 1e-3) / 1e9, 1)}
    if leg == "dequantize":
        out = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
        ms = timed(lambda: q4.dequantize(q, torch.bfloat16, out=out), 5)
        nb = N * K * 2 + q.nbytes()
        return {"leg": leg, "ms": round(ms, 4), "GBps": round(nb / (ms * 1e-3) / 1e9, 1)}
    if leg == "gemm_dx":
        dy = torch.randn((M, N), device=dev).to(torch.bfloat16)
        dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        ms = timed(lambda: q4.gemm_dx(dy, q, out=dx), 5, warm=WARM_MC)
        return {"leg": leg, "ms": round(ms, 4),
                "TFLOPs": round(2.0 * M * N * K / (ms * 1e-3) / 1e12, 1)}
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ms = timed(lambda: q4.gemm(x, q, out=y), 5, warm=WARM_MC)
    return {"leg": "gemm", "ms": round(ms, 4),
            "TFLOPs": round(2.0 * M * N * K / (ms * 1e-3) / 1e12, 1)}


def _rotated_gemv(torch, q4, dev, stream, fmt, g, N, K, Ms, act, seed, min_bytes=512 << 20):
    """GEMV weight GB/s on cold weights: R copies of one quantized matrix
    (R * bytes >= 512 MiB, more than the 256 MB last-level cache), used in
    turn, timed per launch with HIP events (median and minimum), and the
    same R launches back to back from a HIP graph (per-launch average)."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    w = torch.empty((N, K), dtype=torch.float16, device=dev).normal_(0.0, 0.02, generator=gen)
    q0 = q4.quantize(w, fmt, g)
    nb = q0.nbytes()
    R = max(2, -(-min_bytes // nb))
    qs = [q0] + [q4.quantize(w, fmt, g) for _ in range(R - 1)]
    del w
    dt = torch.bfloat16 if act == q4.BF16 else torch.float16
    out = {}
    for M in Ms:
        x = torch.randn((M, K), generator=gen, device=dev).to(dt)
        y = torch.empty((M, N), dtype=dt, device=dev)
        for q in qs[:2]:
            q4.gemv(x, q, out=y)
        torch.cuda.synchronize()
        reps = 3 * R
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for i, (a, b) in enumerate(ev):
            a.record(stream)
            q4.gemv(x, qs[i % R], out=y)
            b.record(stream)
        torch.cuda.synchronize()
        us = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
        med = us[len(us) // 2]
        # the same launches back to back, replayed from a HIP graph
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for q in qs:
                q4.gemv(x, q, out=y)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for q in qs:
                q4.gemv(x, q, out=y)
        graph.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(3):
            graph.replay()
        b.record(stream)
        torch.cuda.synchronize()
        g_us = a.elapsed_time(b) * 1e3 / (3 * R)
        del graph
        out[f"M{M}"] = {"us_median": round(med, 2), "us_min": round(us[0], 2),
                        "weight_GBps": round(nb / (med * 1e-6) / 1e9, 1),
                        "pct_hbm_peak": round(100 * nb / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 1),
                        "graph_us_per_launch": round(g_us, 2),
                        "graph_weight_GBps": round(nb / (g_us * 1e-6) / 1e9, 1)}
    del qs
    torch.cuda.empty_cache()
    return {"weight_bytes": nb, "copies": R, **out}


def _codec_rates(torch, q4, dev, stream, fmt, g, N, K, out_dt, seed, mu=0.0,
                 min_bytes=512 << 20):
    """Quantize and dequantize GB/s on cold buffers: R copies of the fp16
    weight and of its quantized form (R * bytes >= 512 MiB, more than the
    256 MB last-level cache), used in turn; algorithmic bytes = fp16 read +
    codes and metadata written (quantize), codes and metadata read + N K
    16-bit values written (dequantize)."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    w0 = torch.empty((N, K), dtype=torch.float16, device=dev).normal_(mu, 0.02, generator=gen)
    q0 = q4.quantize(w0, fmt, g)
    nb = N * K * 2 + q0.nbytes()
    R = max(2, -(-min_bytes // nb))
    ws = [w0] + [w0.clone() for _ in range(R - 1)]
    qs = [q0] + [q4.quantize(w0, fmt, g) for _ in range(R - 1)]
    outs = [torch.empty((N, K), dtype=out_dt, device=dev) for _ in range(R)]
    timed = _timer(torch, stream)

    def quant_all():
        for w, q in zip(ws, qs):
            q4.quantize(w, fmt, g, out=q)

    def deq_all():
        for q, o in zip(qs, outs):
            q4.dequantize(q, out_dt, out=o)
    qt = timed(quant_all, 3) / R
    dt = timed(deq_all, 3) / R
    del ws, qs, outs
    torch.cuda.empty_cache()
    return {"copies": R, "bytes": nb,
            "quantize_us": round(qt * 1e3, 2), "quantize_GBps": round(nb / (qt * 1e-3) / 1e9, 1),
            "dequantize_us": round(dt * 1e3, 2),
            "dequantize_GBps": round(nb / (dt * 1e-3) / 1e9, 1)}


def codec_configs(torch, q4, dev, stream):
    """Quantize / dequantize of the single-matrix workloads in their own
    formats (NF4 g64 1024x1024 -> fp16; INT4-sym g128 4096x4096 -> fp16; NF4
    g64 11008x4096 -> bf16; INT4-asym g32 14336x4096 -> bf16)."""
    return {
        "c1_nf4_g64_1024x1024_f16": _codec_rates(torch, q4, dev, stream, q4.NF4, 64, 1024, 1024,
                                                 torch.float16, 101),
        "c2_sym_g128_4096x4096_f16": _codec_rates(torch, q4, dev, stream, q4.INT4_SYM, 128, 4096,
                                                  4096, torch.float16, 201),
        "c3_nf4_g64_11008x4096_bf16": _codec_rates(torch, q4, dev, stream, q4.NF4, 64, 11008, 4096,
                                                   torch.bfloat16, 301),
        "c4_asym_g32_14336x4096_bf16": _codec_rates(torch, q4, dev, stream, q4.INT4_ASYM, 32,
                                                    14336, 4096, torch.bfloat16, 401, mu=0.001),
    }


def copy_ceiling(torch, dev, stream):
    """A plain 1 GiB device-to-device copy (read + write), the streaming
    ceiling beside which the kernels' GB/s are read (context, not a peak)."""
    n = 1 << 30
    a = torch.ones(n // 4, dtype=torch.int32, device=dev)
    b = torch.empty_like(a)
    ms = _timer(torch, stream)(lambda: b.copy_(a), 10)
    del a, b
    torch.cuda.empty_cache()
    return {"bytes_moved": 2 * n, "ms": round(ms, 4),
            "GBps": round(2 * n / (ms * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100 * 2 * n / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 1)}


def read_ceiling(torch, dev, stream):
    """A read-only stream: torch's row sums of a 65536 x 16384 fp32 matrix
    (4 GiB read, 256 KiB written; of the library reductions tried, the
    fastest reader), beside which a weight stream that reads and barely
    writes is read (context, not a peak)."""
    n = 1 << 32
    a = torch.ones((65536, n // 4 // 65536), dtype=torch.float32, device=dev)
    out = torch.empty((65536,), dtype=torch.float32, device=dev)
    ms = _timer(torch, stream)(lambda: torch.sum(a, dim=1, out=out), 10)
    del a, out
    torch.cuda.empty_cache()
    return {"bytes_read": n, "ms": round(ms, 4),
            "GBps": round(n / (ms * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100 * n / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 1)}


def config_gemvs(torch, q4, dev, stream):
    """The single-matrix GEMV configurations on cold weights: NF4 g64
    1024x1024 (fp16 x, M = 1), INT4-sym g128
    4096x4096 (fp16 x, M = 1) and the NF4 g64 MLP shapes 11008x4096 and
    4096x11008 (bf16 x, M = 1, 4, 16)."""
    return {
        "c1_nf4_g64_1024x1024_f16": _rotated_gemv(torch, q4, dev, stream, q4.NF4, 64,
                                                  1024, 1024, [1], q4.F16, 102),
        "c2_sym_g128_4096x4096_f16": _rotated_gemv(torch, q4, dev, stream, q4.INT4_SYM, 128,
                                                   4096, 4096, [1], q4.F16, 203),
        "c3_nf4_g64_11008x4096_bf16": _rotated_gemv(torch, q4, dev, stream, q4.NF4, 64,
                                                    11008, 4096, [1, 4, 16], q4.BF16, 303),
        "c3_nf4_g64_4096x11008_bf16": _rotated_gemv(torch, q4, dev, stream, q4.NF4, 64,
                                                    4096, 11008, [1, 4, 16], q4.BF16, 304),
    }


def extra_legs(torch, q4, dev, stream):
    """Quantize, dequantize and prefill-GEMM legs on the INT4-asym g32
    14336x4096 weight."""
    timed = _timer(torch, stream)
    w, x, q = _prefill_inputs(torch, q4, dev)
    N, K = w.shape
    M = x.shape[0]
    qt = timed(lambda: q4.quantize(w, q4.INT4_ASYM, 32, out=q), 10)
    out = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    dt = timed(lambda: q4.dequantize(q, torch.bfloat16, out=out), 10)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    # matrix-core legs: steady state after 400 warm-up calls (about 0.1 s;
    # the first calls after a change of load run at a lower clock: the
    # M = 2048 GEMM took 257 us per call over its first 5 ms and 215 us after
    # 30 ms), the fused and the unfused legs alike
    gt = timed(lambda: q4.gemm(x, q, out=y), 30, warm=WARM_MC)
    flops = 2.0 * M * N * K
    codec_bytes = N * K * 2 + q.nbytes()
    # the pages' unfused path: dequantize to the compute dtype, then a
    # library 16-bit GEMM (hipBLASLt through torch.matmul)
    yb = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def unfused():
        q4.dequantize(q, torch.bfloat16, out=out)
        torch.matmul(x, out.t(), out=yb)
    ut = timed(unfused, 30, warm=WARM_MC)
    mt = timed(lambda: torch.matmul(x, out.t(), out=yb), 30, warm=WARM_MC)
    # the same at decode width: M = 16 on the c3 gate/up shape (NF4 g64)
    w16 = torch.empty((11008, 4096), dtype=torch.float16, device=dev).normal_(0.0, 0.02)
    q16 = q4.quantize(w16, q4.NF4, 64)
    x16 = torch.randn((16, 4096), device=dev).to(torch.bfloat16)
    o16 = torch.empty((11008, 4096), dtype=torch.bfloat16, device=dev)
    y16 = torch.empty((16, 11008), dtype=torch.bfloat16, device=dev)

    def unfused16():
        q4.dequantize(q16, torch.bfloat16, out=o16)
        torch.matmul(x16, o16.t(), out=y16)
    u16 = timed(unfused16, 20)
    f16t = timed(lambda: q4.gemv(x16, q16, out=y16), 20)
    # where the fused product stops beating the unfused path: the same
    # weight at prefill widths between the two
    sweep = {}
    for m in (64, 128, 256, 512, 1024):
        xm, ym, ybm = x[:m], y[:m], yb[:m]

        def unfused_m():
            q4.dequantize(q, torch.bfloat16, out=out)
            torch.matmul(xm, out.t(), out=ybm)
        fm = timed(lambda: q4.gemm(xm, q, out=ym), 20, warm=100)
        um = timed(unfused_m, 20, warm=100)
        sweep[f"M{m}"] = {"fused_ms": round(fm, 4), "unfused_ms": round(um, 4),
                          "fused_TFLOPs": round(2.0 * m * N * K / (fm * 1e-3) / 1e12, 1),
                          "fused_over_unfused": round(um / fm, 3)}
    # the backward product through the same frozen weight (QLoRA's dX):
    # dY [2048, 14336] . What -> [2048, 4096], and the unfused equivalent
    gen = torch.Generator(device=dev)
    gen.manual_seed(403)
    dy = torch.empty((M, N), dtype=torch.float32, device=dev).normal_(0.0, 1.0, generator=gen)
    dy = dy.to(torch.bfloat16)
    dxo = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    bt = timed(lambda: q4.gemm_dx(dy, q, out=dxo), 30, warm=WARM_MC)

    def unfused_dx():
        q4.dequantize(q, torch.bfloat16, out=out)
        torch.matmul(dy, out, out=dxo)
    but = timed(unfused_dx, 30, warm=WARM_MC)
    return {
        "gemm_dx": {"shape": f"dY {M}x{N} . W {N}x{K} int4_asym g32 bf16", "ms": round(bt, 4),
                    "TFLOPs": round(flops / (bt * 1e-3) / 1e12, 1),
                    "pct_bf16_peak": round(100 * flops / (bt * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 1),
                    "unfused_dequant_then_hipblaslt_ms": round(but, 4)},
        "gemm": {"shape": f"M={M} N={N} K={K} int4_asym g32 bf16", "ms": round(gt, 4),
                 "TFLOPs": round(flops / (gt * 1e-3) / 1e12, 1),
                 "pct_bf16_peak": round(100 * flops / (gt * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 1)},
        "unfused_dequant_then_hipblaslt": {
            "prefill_M2048_ms": round(ut, 4),
            "prefill_matmul_only_ms": round(mt, 4),
            "prefill_matmul_only_TFLOPs": round(flops / (mt * 1e-3) / 1e12, 1),
            "fused_over_unfused_prefill": round(ut / gt, 3),
            "decode_M16_nf4_11008x4096_unfused_ms": round(u16, 4),
            "decode_M16_nf4_11008x4096_fused_ms": round(f16t, 4),
            "fused_over_unfused_M16": round(u16 / f16t, 3),
            "prefill_m_sweep_int4asym_g32_14336x4096": sweep},
        "dequantize_14336x4096_asym_bf16": {"ms": round(dt, 4),
                                             "GBps": round(codec_bytes / (dt * 1e-3) / 1e9, 1)},
        "quantize_14336x4096_asym": {"ms": round(qt, 4),
                                      "GBps": round(codec_bytes / (qt * 1e-3) / 1e9, 1)},
    }


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(seconds: float):
    """The C oracle on the host cores, on a bounded sample of the token: the
    first 2048 rows of each matrix, layer by layer, in blocks of 64 rows (at
    most 512 blocks, drawn with the same seeds and distribution as the GPU
    run's weights but a different generator, so not the same bits), each
    quantized by the oracle beforehand (not timed).  Timed: dequantize each
    row to bf16 and form the fp64 product with x, as the reference does --
    first on one thread, then on T threads (the host's cores, at most 16),
    each for about half the budget, cycling over the blocks.  The oracle is
    plain scalar C; ctypes releases the interpreter lock during each call,
    so the threads run in parallel."""
    import concurrent.futures as cf
    import oracle
    from bit_group_wise_amd import synth

    T = max(1, min(len(os.sched_getaffinity(0)), 16))
    xs = {HID: synth.act_bits(1, HID, 5900, synth.BF16), FFN: synth.act_bits(1, FFN, 5901, synth.BF16)}
    specs = []
    for layer in range(LAYERS):
        for name, N, K, parts in LAYER_MATS:
            for part, rows, idx in parts:
                for r0 in range(0, min(rows, 2048), 64):
                    specs.append((f"{part}{layer}", K, 5000 + 7 * layer + idx, r0))
    specs = specs[:512]

    def prep(spec):
        name, K, seed, r0 = spec
        # the first rows of a row-major draw are the full matrix's first rows
        w = synth.weight_f16_bits(r0 + 64, K, seed=seed)[r0:r0 + 64]
        codes, scales, _ = oracle.quantize(oracle.NF4, 64, w)
        return name, K, codes, scales

    with cf.ThreadPoolExecutor(T) as ex:
        blocks = list(ex.map(prep, specs))
    row_bytes = {K: K // 2 + (K // 64) * 4 for K in (HID, FFN)}

    def run(block):
        name, K, codes, scales = block
        oracle.matmul(oracle.NF4, 64, oracle.BF16, xs[K], codes, scales, None, 64, K)
        return 64 * row_bytes[K]

    # one thread
    done1, t0, i = 0, time.perf_counter(), 0
    while time.perf_counter() - t0 < seconds / 2:
        done1 += run(blocks[i % len(blocks)])
        i += 1
    t1 = time.perf_counter() - t0
    # all T threads, in rounds of 4 T blocks
    doneT, t0, i = 0, time.perf_counter(), 0
    with cf.ThreadPoolExecutor(T) as ex:
        while time.perf_counter() - t0 < seconds / 2:
            batch = [blocks[(i + j) % len(blocks)] for j in range(4 * T)]
            i += 4 * T
            doneT += sum(ex.map(run, batch))
    tT = time.perf_counter() - t0
    others = _cpu_other_ops(T, max(2.0, seconds / 8))
    return {
        "value": round(doneT / tT / 1e9, 4),
        "unit": "GB/s",
        "cores": T,
        "kind": "oracle",
        "other_ops": others,
        "sample": f"{len(blocks)} blocks of 64 weight rows (the first 2048 rows of each of "
                  f"{blocks[0][0]} .. {blocks[-1][0]}), NF4 g64, M=1 bf16: dequantize + fp64 dot "
                  f"product, cycled for {tT:.1f}s on {T} threads ({doneT / 2**20:.0f} MiB); "
                  f"one thread: {done1 / t1 / 1e9:.4f} GB/s over {t1:.1f}s",
        "value_one_thread": round(done1 / t1 / 1e9, 4),
        "cpu_model": _cpu_model(),
    }


def _cpu_other_ops(T: int, seconds: float):
    """The oracle on the other ops, T threads, each cycled for about
    `seconds`: quantize and dequantize of the INT4-asym g32 prefill weight
    (blocks of 64 of its 14336 rows; algorithmic GB/s as on the GPU) and the
    fp64 GEMM reference on a row sample of that workload (64 rows of x
    against 256 weight rows at a time; GFLOP/s of 2 M N K)."""
    import concurrent.futures as cf
    import numpy as np
    import oracle
    from bit_group_wise_amd import synth

    K, g, rows = 4096, 32, 64
    w = [synth.weight_f16_bits(rows, K, seed=401 + i, mu=0.001) for i in range(4 * T)]
    q = [oracle.quantize(oracle.INT4_ASYM, g, b) for b in w]
    nb = rows * K * 2 + rows * K // 2 + rows * (K // g) * 2 + rows * (K // g) // 2
    x = synth.act_bits(64, K, 402, synth.BF16)
    wq = [oracle.quantize(oracle.INT4_ASYM, g, synth.weight_f16_bits(256, K, seed=450 + i,
                                                                      mu=0.001))
          for i in range(T)]

    def cycle(fn, items):
        done, t0, i = 0, time.perf_counter(), 0
        with cf.ThreadPoolExecutor(T) as ex:
            while time.perf_counter() - t0 < seconds:
                done += sum(ex.map(fn, [items[(i + j) % len(items)] for j in range(T)]))
                i += T
        return done / (time.perf_counter() - t0)

    qr = cycle(lambda b: (oracle.quantize(oracle.INT4_ASYM, g, b), nb)[1], w)
    dr = cycle(lambda c: (oracle.dequantize(oracle.INT4_ASYM, g, c[0], c[1], c[2], rows, K,
                                            oracle.BF16), nb)[1], q)
    fr = cycle(lambda c: (oracle.matmul(oracle.INT4_ASYM, g, oracle.BF16, x, c[0], c[1], c[2],
                                        256, K), 2.0 * 64 * 256 * K)[1], wq)
    return {"threads": T,
            "quantize_asym_g32_GBps": round(qr / 1e9, 4),
            "dequantize_asym_g32_bf16_GBps": round(dr / 1e9, 4),
            "gemm_reference_fp64_GFLOPs": round(fr / 1e9, 4),
            "sample": f"INT4-asym g32, K = 4096: blocks of {rows} weight rows (codec); "
                      f"64 x rows x 256 weight rows per GEMM sample; about {seconds:.1f}s each"}


if __name__ == "__main__":
    main()
