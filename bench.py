"""Throughput of quantized SDPA (FP8 Q/K/P/V) on one MI355X.

One step = one qsdpa_forward call over the Kontext-style 1024x1024 edit
sequence (512 text + 4096 output-image + 4096 context-image tokens, B=1,
H=24, head_dim 128): channel statistics, quantize, fused attention, bf16 out.
Inputs are seeded synthetic tensors already resident in HBM.

Prints one JSON line: TFLOP/s of the whole step (4 B H N^2 D per step), the
roofline of the dominant kernel (the fused attention, timed with HIP events
on the stream it runs on), the CPU oracle timed on a bounded sample, and the
GPU output's error against that oracle sample and against exact fp64
attention of the unquantized inputs.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP8_PEAK_TFLOPS = 5000.0    # MI355X dense FP8 MFMA
HBM_PEAK_GBS = 8000.0
# The attention kernel's roofline per mode.  FP8: dense FP8 MFMA.  MXFP4: half
# of the flops are Q.K^T on the FP4 MFMA (10.1 PFLOP/s dense) and half P.V on
# FP8 (5.0), so its peak is the harmonic mean of the two.  FP4 (fp32 scales per
# 16 channels): the dense FP8 peak, since its P.V is FP8 and its exact Q.K^T
# runs on f16 MFMAs plus FP8 correction MFMAs (the FP4 peak, 10.1, is noted in
# the record; the hardware's scaled FP4 MFMA cannot apply fp32 scales).
FP4_PEAK_TFLOPS = 10100.0
KERNEL_PEAK_TFLOPS = {"fp8": FP8_PEAK_TFLOPS, "fp4": FP8_PEAK_TFLOPS,
                      "mxfp4": 2.0 / (1.0 / FP4_PEAK_TFLOPS + 1.0 / FP8_PEAK_TFLOPS)}
PEAK_BASIS = {"fp8": "dense FP8 MFMA (Q.K^T and P.V)",
              "mxfp4": "Q.K^T at the dense FP4 peak, P.V at the dense FP8 peak (harmonic mean)",
              "fp4": "dense FP8 MFMA (P.V is FP8; the exact per-16-channel Q.K^T runs on f16 + FP8 "
                     "MFMAs); dense FP4 peak 10100 TFLOP/s"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="kontext1024")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-shapes", action="store_true",
                    help="skip the other FLUX shapes of the metric (N = 4608 and 16896, FP8)")
    ap.add_argument("--cpu-heads", type=int, default=16, help="(b,h) pairs of the CPU oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (for scaling HBM byte counters)")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic_attn_fp8_kontext1024.json"),
                    help="HBM bytes per attention launch measured with rocprofv3 counters (if present)")
    return ap.parse_args()


# At most this many oracle workers: the host share of one GPU on the machines
# this runs on.
MAX_CPU_WORKERS = 16


def _worker_init():
    """Oracle worker: single-threaded BLAS, so that the workers are the
    parallelism.  The thread counts are set before the worker loads NumPy's
    BLAS (read at load time), and limited again once it is loaded."""
    global _LIMITS
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS"):
        os.environ[var] = "1"
    import numpy  # noqa: F401  (loads BLAS with one thread)
    from threadpoolctl import threadpool_limits
    _LIMITS = threadpool_limits(limits=1)


def _oracle_head(task):
    """Quantize + attention of one (b, h) pair through the oracle (runs in a
    worker process).  Returns the output [N, 128] and the seconds it took."""
    qh, kh, vh, fmt, block_q, block_k = task
    import oracle
    from workloads import TAU
    t0 = time.perf_counter()
    z = oracle.quantize(qh, kh, vh, fmt=fmt, block_q=block_q, block_k=block_k)
    out = oracle.attend(z, TAU, 0, 0)
    return out, time.perf_counter() - t0


def start_cpu_pool(heads: int):
    """Worker processes for the oracle, forked now: before this process makes
    any GPU call, so the workers never touch the GPU.  One per host core this
    process may run on (os.sched_getaffinity), at most MAX_CPU_WORKERS and at
    most one per head of the sample."""
    import multiprocessing as mp
    n = max(1, min(len(os.sched_getaffinity(0)), MAX_CPU_WORKERS, heads))
    return mp.get_context("fork").Pool(n, initializer=_worker_init), n


def cpu_baseline(w, heads: int, got_bits, pool, workers: int):
    """The oracle on the first ``heads`` (b, h) pairs of batch 0 of the
    workload, one pair per task over ``workers`` worker processes (each with
    single-threaded BLAS): quantize of each head and every query row against
    every key, timed from the first task out to the last result back.  Then,
    untimed, the error of the GPU output on those heads (``got_bits``, bf16
    bits [heads, N, 128]) against the oracle's output and against exact
    attention.  Returns the baseline record and the accuracy record."""
    import numpy as np

    from workloads import draw

    qb, kb, vb = draw(w, batch=1, heads=heads)   # the same tensors as heads 0.. of batch 0
    tasks = [(qb[:, h:h + 1], kb[:, h:h + 1], vb[:, h:h + 1], w.fmt, w.block_q, w.block_k) for h in range(heads)]
    t0 = time.perf_counter()
    res = pool.map(_oracle_head, tasks, chunksize=1)
    dt = time.perf_counter() - t0
    outs = np.stack([r[0] for r in res])
    cpu_s = sum(r[1] for r in res)
    flops = 4.0 * heads * w.seq_len ** 2 * 128
    rec = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
           "sample": f"{heads} of the {w.batch * w.heads} (b,h) pairs of {w.name}, all {w.seq_len} query rows "
                     f"(quantize + attention), one pair per task on {workers} worker processes with "
                     f"single-threaded NumPy: {dt:.1f} s wall, {cpu_s:.1f} s of CPU work"}
    return rec, accuracy(w, got_bits, outs, (qb, kb, vb))


def accuracy(w, got_bits, want, inputs, rows_per_head: int = 256):
    """Part of the CPU-baseline leg: error of the GPU output (bf16 bits
    [heads, N, 128] of batch 0) against the oracle's output on the same
    heads, and against exact fp64 softmax attention of the unquantized inputs
    on sampled rows."""
    import numpy as np

    import oracle
    from workloads import TAU

    got = oracle.bf16_bits_to_f64(got_bits)
    d = np.abs(got - want)
    qb, kb, vb = inputs
    rng = np.random.default_rng(0)
    ex = []
    for h in range(want.shape[0]):
        rows = np.sort(rng.choice(w.seq_len, min(rows_per_head, w.seq_len), replace=False))
        q, k, v = (oracle.bf16_bits_to_f64(x[0, h]) for x in (qb, kb, vb))
        ex.append(np.abs(got[h, rows] - oracle.exact_attention(q, k, v, TAU, rows)))
    e = np.concatenate([x.ravel() for x in ex])
    return {"vs_oracle": {"max_abs": float(d.max()), "mean_abs": float(d.mean()),
                          "sample": f"{want.shape[0]} heads x {w.seq_len} rows"},
            "vs_exact_fp64": {"max_abs": float(e.max()), "mean_abs": float(e.mean()),
                              "sample": f"{want.shape[0]} heads x {min(rows_per_head, w.seq_len)} rows"},
            "tolerance_vs_oracle": {"max_abs": 1e-2, "mean_abs": 1e-3}}


# The GPU's clock ramps up over the first ~100 ms of load, so the warm-up runs
# the W steps asked for and, if they take less, more steps until this much
# time has passed; the timed steps then measure the steady state.
WARMUP_MIN_S = 0.25


def warm_up(step, warmup: int, dev):
    """Run ``warmup`` untimed steps, and more until WARMUP_MIN_S seconds have
    passed; returns (steps run, seconds)."""
    import torch

    t0 = time.perf_counter()
    n = 0
    for _ in range(warmup):
        step()
        n += 1
    torch.cuda.synchronize(dev)
    while time.perf_counter() - t0 < WARMUP_MIN_S:
        for _ in range(8):
            step()
            n += 1
        torch.cuda.synchronize(dev)
    return n, time.perf_counter() - t0


def time_forward(w, steps: int, warmup: int):
    """ms per qsdpa_forward call of workload ``w`` (inputs resident in HBM),
    timed with HIP events on the current stream."""
    import torch

    import precision_attention_qsdpa_amd as qs
    from workloads import TAU, draw

    qb, kb, vb = draw(w)
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x).view(torch.bfloat16).to(dev) for x in (qb, kb, vb))
    params = qs.make_params(w.batch, w.heads, w.seq_len, fmt=w.fmt, block_q=w.block_q, block_k=w.block_k,
                            softmax_scale=TAU)
    ws = qs.empty_workspace(params, dev)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream(dev)
    warm_up(lambda: qs.qsdpa_forward(q, k, v, out=out, workspace=ws, params=params, stream=stream), warmup, dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        qs.qsdpa_forward(q, k, v, out=out, workspace=ws, params=params, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize(dev)
    return e0.elapsed_time(e1) / steps


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "the path shards by (batch, head) with no exchange: each GPU would run this same "
              "kernel on its share of the heads", file=sys.stderr)
        sys.exit(2)
    pool = workers = None
    if not args.no_cpu_baseline and not args.copy_calibration:
        pool, workers = start_cpu_pool(args.cpu_heads)   # before the first GPU call
    import torch

    if args.copy_calibration:
        n = 256 << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "launches": 5}))
        return

    import precision_attention_qsdpa_amd as qs
    from workloads import TAU, WORKLOADS, draw

    w = WORKLOADS[args.workload]
    qb, kb, vb = draw(w)
    dev = torch.device("cuda:0")
    to = lambda x: torch.from_numpy(x).view(torch.bfloat16).to(dev)
    q, k, v = to(qb), to(kb), to(vb)
    params = qs.make_params(w.batch, w.heads, w.seq_len, fmt=w.fmt, block_q=w.block_q, block_k=w.block_k,
                            softmax_scale=TAU)
    ws = qs.empty_workspace(params, dev)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream(dev)

    def step():
        qs.qsdpa_forward(q, k, v, out=out, workspace=ws, params=params, stream=stream)

    warm_steps, warm_s = warm_up(step, args.warmup, dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / args.steps

    # single steps, each between its own pair of events (after the timed region,
    # so the clocks are already up): the median of 50, and the pages' protocol
    # of 2 warm-up calls followed by the mean of 10
    def single_steps(n):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in ev:
            a.record(stream)
            step()
            b.record(stream)
        torch.cuda.synchronize(dev)
        return [a.elapsed_time(b) for a, b in ev]
    single = sorted(single_steps(50))
    single_steps(2)
    ten = single_steps(10)
    per_step = {"median_of_50": round(single[25], 4), "min_of_50": round(single[0], 4),
                "max_of_50": round(single[-1], 4), "mean_of_10_after_2_warmups": round(sum(ten) / 10, 4)}

    # the quantize pass and the dominant kernel, timed alone on the same
    # stream.  The dominant kernel is the attention kernel of the timed step
    # (qsdpa_forward's, which quantizes Q in its prologue): it runs alone as
    # qsdpa_attention_bf16q on the K/V codes the timed steps left in the
    # workspace.  qsdpa_attention (on Q codes from qsdpa_quantize) is timed too.
    n_attn = max(args.steps, 20)
    ev = lambda: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    (a0, a1), (b0, b1), (c0, c1) = ev(), ev(), ev()
    a0.record(stream)
    for _ in range(n_attn):
        qs.qsdpa_attention_bf16q(q, ws, out, params, stream=stream)
    a1.record(stream)
    b0.record(stream)
    for _ in range(n_attn):
        qs.qsdpa_quantize(q, k, v, ws, params, stream=stream)
    b1.record(stream)
    c0.record(stream)
    for _ in range(n_attn):
        qs.qsdpa_attention(ws, out, params, stream=stream)
    c1.record(stream)
    torch.cuda.synchronize(dev)
    ms_attn = a0.elapsed_time(a1) / n_attn
    ms_quant = b0.elapsed_time(b1) / n_attn
    ms_attn_codes = c0.elapsed_time(c1) / n_attn

    flops = w.flops
    tflops = flops / (ms_step * 1e-3) / 1e12
    attn_tflops = flops / (ms_attn * 1e-3) / 1e12
    traffic = None
    if os.path.exists(args.traffic_json):
        with open(args.traffic_json) as f:
            tj = json.load(f)
        if tj.get("workload") == w.name and tj.get("kernel_source_sha") == kernel_sha():
            traffic = tj.get("hbm_bytes_per_launch")
    elem = w.batch * w.heads * w.seq_len * 128
    kernel = {"fp8": "attn_fp8_kernel<true>", "fp4": "attn_fp4_kernel<true>", "mxfp4": "attn_mx_kernel<true>"}[w.fmt]
    # quantize pass bytes per element: Q, K, V bf16 read (6) + K, V re-read by the
    # statistics pass (4) + codes and scales written; FP4 mode also reads the K
    # codes and scales again (0.75) and writes their f16 hi/lo expansion (4)
    quant_bpe = {"fp8": 6 + 4 + 3, "fp4": 6 + 4 + 2 + 0.5 + 0.75 + 4, "mxfp4": 6 + 4 + 2 + 2 / 32}[w.fmt]
    rec = {
        "metric": "quantized SDPA TFLOPS at FLUX shapes (N=4608/8704/16896) + % FP8 MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_run": {"steps": warm_steps, "seconds": round(warm_s, 3), "min_seconds": WARMUP_MIN_S},
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp8": "fp8_e4m3", "fp4": "fp4_e2m1+fp8_e4m3", "mxfp4": "mxfp4_e2m1+fp8_e4m3"}[w.fmt],
        "data": "synthetic (seeded N(0,1) Q/V, K with N(0,3) channel offsets; Kontext context tokens rho=0.8)",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "seq_len": w.seq_len,
                   "head_dim": 128, "qk_format": w.fmt, "block_q": w.block_q, "block_k": w.block_k,
                   "pct_fp8_peak": round(100.0 * tflops / FP8_PEAK_TFLOPS, 2)},
        "roofline": {"bound": "mfma", "kernel": kernel, "achieved": round(attn_tflops, 2),
                     "peak": round(KERNEL_PEAK_TFLOPS[w.fmt], 1), "peak_basis": PEAK_BASIS[w.fmt],
                     "unit": "TFLOP/s", "frac": round(attn_tflops / KERNEL_PEAK_TFLOPS[w.fmt], 4),
                     "traffic": traffic, "ms_per_launch": round(ms_attn, 4),
                     "ms_per_launch_on_q_codes": round(ms_attn_codes, 4)},
        "quantize": {"ms_per_launch": round(ms_quant, 4),
                     "algorithmic_GB_s": round(elem * quant_bpe / (ms_quant * 1e-3) / 1e9, 1),
                     "hbm_peak_GB_s": HBM_PEAK_GBS},
        "wall_s_timed": round(wall, 3),
        "system": system_info(dev),
        "per_step_ms": per_step,
    }
    if w.fmt == "fp8":
        # the selective correction (VC-Attention-style, rho = 0.005): the same
        # step with the ceil(rho N) highest-error query tokens of each head
        # recomputed without quantization; reported beside the headline
        rho = qs.VC_RHO
        vws = torch.empty(qs.qsdpa_vc_workspace_bytes(params, rho), dtype=torch.uint8, device=dev)
        for _ in range(10):
            qs.qsdpa_forward_vc(q, k, v, out=out, workspace=vws, rho=rho, params=params, stream=stream)
        v0, v1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        v0.record(stream)
        for _ in range(n_attn):
            qs.qsdpa_forward_vc(q, k, v, out=out, workspace=vws, rho=rho, params=params, stream=stream)
        v1.record(stream)
        torch.cuda.synchronize(dev)
        ms_vc = v0.elapsed_time(v1) / n_attn
        L = qs.qsdpa_vc_workspace_layout(params, rho)
        rec["vc_forward"] = {"rho": rho, "rows_per_head": L.count, "ms_per_step": round(ms_vc, 4),
                             "value": round(flops / (ms_vc * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                             "overhead_vs_forward": round(ms_vc / ms_step - 1.0, 4)}
    if not args.no_shapes and w.name == "kontext1024":
        # the metric's other FLUX shapes (FP8): one line each, not the headline value
        rec["shapes"] = []
        for name in ("dev1024", "gen2048_fp8"):
            ws_ = WORKLOADS[name]
            ms = time_forward(ws_, steps=30, warmup=10)
            tf = ws_.flops / (ms * 1e-3) / 1e12
            rec["shapes"].append({"workload": name, "batch": ws_.batch, "heads": ws_.heads,
                                  "seq_len": ws_.seq_len, "qk_format": ws_.fmt, "ms_per_step": round(ms, 4),
                                  "value": round(tf, 2), "unit": "TFLOP/s",
                                  "pct_fp8_peak": round(100.0 * tf / FP8_PEAK_TFLOPS, 2)})
    if not args.no_cpu_baseline:
        heads = min(args.cpu_heads, w.heads)
        got_bits = out[0, :heads].contiguous().view(torch.int16).cpu().numpy().view("uint16")
        rec["cpu_baseline"], rec["accuracy"] = cpu_baseline(w, heads, got_bits, pool, workers)
        pool.close()
        pool.join()
    print(json.dumps(rec), flush=True)


def system_info(dev) -> dict:
    """Device, architecture, compute units and HIP / PyTorch versions."""
    import torch

    pr = torch.cuda.get_device_properties(dev)
    return {"device": torch.cuda.get_device_name(dev), "arch": getattr(pr, "gcnArchName", None),
            "compute_units": pr.multi_processor_count, "hbm_GiB": round(pr.total_memory / 2 ** 30, 1),
            "hip": torch.version.hip, "torch": torch.__version__}


def kernel_sha() -> str:
    """Hash of the attention kernel source (the traffic counters are only
    valid for the kernel they were taken on)."""
    import hashlib
    p = os.path.join(ROOT, "precision_attention_qsdpa_amd", "csrc", "qsdpa_attn.hip")
    with open(p, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


if __name__ == "__main__":
    main()
