"""Benchmark of the W4A4 linear layer on one MI355X.

Metric: effective W4A4 TOPS of the runtime path (activation quantize + grouped GEMM) at
Llama-7B linear-layer shapes, as a fraction of the dense INT8 MFMA peak.

One step = for each Llama-7B shape (attention projection 256x4096x4096, MLP gate/up
1024x4096x11008, MLP down 2048x11008x4096): atom_quantize_act on a fresh fp16 activation
batch, then the grouped GEMM against pre-packed weights (atom_gemm_ws: shapes with few
output tiles split their groups over several workgroups through a preallocated workspace).
Outlier selection and weight packing are offline steps of the method and run once before
timing.  Effective TOPS = sum of 2*M*N*K over the shapes / step time.  Inputs rotate over several resident copies so that each step
reads its activations and packed weights from HBM rather than from the 256 MB Infinity
Cache.

Prints ONE JSON line on stdout (progress goes to stderr).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 256 * 2.4e9 * 8192 / 1e12      # 5033: 256 CUs x 2.4 GHz x 8192 int8 ops/clk/CU
# The INT4 groups run on the fp6 (e2m3) matrix cores, twice the int8 rate; this is the roofline
# peak of the GEMM (its one INT8 group per row runs at the int8 rate, so the true mixed peak is
# slightly lower and the reported fraction slightly conservative).
FP6_PEAK_TOPS = 256 * 2.4e9 * 16384 / 1e12      # 10066: dense fp6 / fp4 MFMA
HBM_PEAK_GBS = 8000.0
GEMM_SRC = os.path.join(ROOT, "bit_quantized_gemm_amd", "csrc", "gemm.hip")
QUANT_SRC = os.path.join(ROOT, "bit_quantized_gemm_amd", "csrc", "quantize.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_hbm_traffic.json")

WORKLOAD_SETS = {
    "llama7b": ["A", "B", "C"],
    "A": ["A"], "B": ["B"], "C": ["C"], "D": ["D"],
    # 16 tokens through the same weights: the few-rows GEMM, bound by reading the packed weights
    "decode": ["dA", "dB", "dC"],
    # the W4A8 variant (INT8 activations in every group) on the same Llama-7B shapes
    "w4a8": ["A", "B", "C"],
    "Dq": [],              # activation quantize alone on 8192 x 8192 fp16 (128 outlier channels x30)
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def sha256(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def quant_bytes(M, K):
    """Algorithmic HBM bytes of one activation quantize: read fp16 X, write codes and scales."""
    return M * (2 * K + ((K - 128) // 2 + 128) + 2 * (K // 128))


def gemm_bytes(M, N, K):
    """Compulsory HBM bytes of one GEMM: codes and scales of both operands, fp16 Y."""
    rb = (K - 128) // 2 + 128
    g = K // 128
    return M * rb + 2 * g * M + N * rb + 2 * g * N + 2 * M * N


def traffic_for_current_gemm():
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary, only while the
    GEMM source is unchanged since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    d = json.load(open(TRAFFIC_FILE))
    if d.get("gemm_source_sha256") != sha256(GEMM_SRC):
        return None
    return d.get("bytes_per_launch_by_workload")


def traffic_for_current_quantize():
    """HBM bytes per 8192 x 8192 quantize launch from the same counter summary, only while the
    quantize source is unchanged since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    d = json.load(open(TRAFFIC_FILE))
    if d.get("quantize_source_sha256") != sha256(QUANT_SRC):
        return None
    return d.get("quantize_8192_bytes_per_launch")


class _nullctx:
    def __enter__(self):
        return self

    def __exit__(self, *a):
        return False


def cpu_baseline(shapes, budget_rows, a8=False):
    """Time the CPU oracle (quantize + dequantise-then-fp64-matmul) on a row sample of every
    shape; weights are packed by the oracle beforehand, like the GPU path.  a8: INT8 codes in
    every activation group (the W4A8 variant)."""
    import synth
    from oracle import atom_oracle as O
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except Exception:                                      # pragma: no cover
        threadpool_limits = None
    cores = min(len(os.sched_getaffinity(0)), 16)
    ops = 0
    secs = 0.0
    parts = []
    blas = None
    with (threadpool_limits(limits=cores) if threadpool_limits else _nullctx()):
        for key in shapes:
            w = synth.get(key)
            x, wt, _ = synth.make_inputs(w)
            rows = min(w.M, budget_rows)
            perm = O.outlier_perm(x)
            qw, sw = O.quantize_rows(wt, perm)
            xs = np.ascontiguousarray(x[:rows])
            t0 = time.perf_counter()
            qx, sx = O.quantize_rows(xs, perm, all_int8=a8)
            y = O.to_fp16(O.gemm_ref(qx, sx, qw, sw))
            dt = time.perf_counter() - t0
            assert y.shape == (rows, w.N)
            ops += 2 * rows * w.N * w.K
            secs += dt
            parts.append(f"{key}: first {rows} of {w.M} rows x N={w.N} x K={w.K} in {dt:.2f}s")
            log(f"[cpu] {parts[-1]}")
        if threadpool_limits:
            info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
            blas = f'{info[0].get("internal_api")} x{info[0].get("num_threads")}' if info else None
    return {"value": ops / secs / 1e12, "unit": "TOP/s", "cores": cores, "kind": "oracle",
            "sample": "; ".join(parts) + f"; numpy oracle, BLAS {blas}, {cores} threads",
            "seconds": round(secs, 3)}


def quant_only(args, torch, bq, synth, dev, R):
    """Activation-quantize throughput on the 8192 x 8192 workload (HBM-bound kernel)."""
    x, _, _ = synth.quant_only_x()
    M, K = x.shape
    X0 = torch.from_numpy(x).to(dev)
    perm = bq.atom_select_outliers(bq.atom_channel_stat(X0))
    copies = []
    for r in range(R):
        Xr = X0.clone() if r == 0 else (X0 * (1.0 + 1e-3 * r)).to(torch.float16)
        copies.append(dict(X=Xr, Xq=torch.empty((M, bq.atom_row_bytes(K)), dtype=torch.uint8, device=dev),
                           sx=torch.empty((K // 128, M), dtype=torch.float16, device=dev)))
    del X0
    stream = torch.cuda.current_stream(dev)

    def step(i):
        c = copies[i % R]
        bq.atom_quantize_act(c["X"], perm, Xq=c["Xq"], sx=c["sx"], stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    qb = quant_bytes(M, K)
    gbs = qb / (ms * 1e-3) / 1e9
    line = {
        "metric": "activation quantize throughput (reorder + per-group absmax + INT4 pack + INT8 tail)",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16->int4/int8", "data": "synthetic",
        "config": {"workload": "quantize_only_8192x8192", "M": M, "K": K, "rotating_input_copies": R},
        "roofline": {"kernel": "row_quantize_kernel", "bound": "hbm", "achieved": round(gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic_for_current_quantize() if (M, K) == (8192, 8192) else None,
                     "bytes_per_launch": qb, "avg_launch_us": round(ms * 1e3, 3)},
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="llama7b", choices=sorted(WORKLOAD_SETS))
    ap.add_argument("--rotate", type=int, default=4, help="resident input copies cycled through")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=2048, help="rows per shape in the CPU oracle sample (2048: every row)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (steps times), to calibrate HBM byte counters")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import bit_quantized_gemm_amd as bq
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": max(1, args.steps)}), flush=True)
        return
    bq.load_library()
    keys = WORKLOAD_SETS[args.workload]
    R = max(1, args.rotate)
    if args.workload == "Dq":
        return quant_only(args, torch, bq, synth, dev, R)

    # ---------------------------------------------------------------- offline: inputs, perm, weight pack
    w4a8 = args.workload == "w4a8"
    sets = []
    for key in keys:
        w = synth.get(key)
        x, wt, _ = synth.make_inputs(w)
        X0 = torch.from_numpy(x).to(dev)
        W0 = torch.from_numpy(wt).to(dev)
        perm = bq.atom_select_outliers(bq.atom_channel_stat(X0))
        Wq0, sw0 = (bq.atom_pack_weights_w4a8 if w4a8 else bq.atom_pack_weights)(W0, perm)
        del W0
        copies = []
        for r in range(R):
            # distinct resident copies; activations get a tiny per-copy change so codes differ
            Xr = X0.clone() if r == 0 else (X0 * (1.0 + 1e-3 * r)).to(torch.float16)
            copies.append(dict(X=Xr, Wq=Wq0.clone(), sw=sw0.clone(),
                               Xq=torch.empty((w.M, w.K if w4a8 else bq.atom_row_bytes(w.K)), dtype=torch.uint8,
                                              device=dev),
                               sx=torch.empty((w.K // 128, w.M), dtype=torch.float16, device=dev),
                               Y=torch.empty((w.M, w.N), dtype=torch.float16, device=dev)))
        # split-K scratch for shapes with few output tiles (allocated once, outside the timed region)
        need = (bq.atom_gemm_w4a8_workspace_bytes if w4a8 else bq.atom_gemm_workspace_bytes)(w.M, w.N, w.K)
        ws = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
        sets.append(dict(key=key, w=w, perm=perm, copies=copies, ws=ws))
        log(f"[setup] {key} {w.name} ready ({R} copies)")
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)

    def step(i, evs=None):
        for si, s in enumerate(sets):
            c = s["copies"][i % R]
            w = s["w"]
            if evs is not None:
                evs[si][0].record(stream)
            if w4a8:
                bq.atom_quantize_act_a8(c["X"], s["perm"], Xq=c["Xq"], sx=c["sx"], stream=stream)
            else:
                bq.atom_quantize_act(c["X"], s["perm"], Xq=c["Xq"], sx=c["sx"], stream=stream)
            if evs is not None:
                evs[si][1].record(stream)
            if w4a8:
                bq.atom_gemm_w4a8_ws(c["Xq"], c["sx"], c["Wq"], c["sw"], w.K, s["ws"], Y=c["Y"], stream=stream)
            else:
                bq.atom_gemm_ws(c["Xq"], c["sx"], c["Wq"], c["sw"], w.K, s["ws"], Y=c["Y"], stream=stream)
            if evs is not None:
                evs[si][2].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- timed region: whole steps
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)
    ms_per_step = ms_total / args.steps

    # ---------------------------------------------------------------- per-kernel durations (HIP events)
    n_k = min(args.steps, 200)
    evl = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in sets] for _ in range(n_k)]
    torch.cuda.synchronize()
    for i in range(n_k):
        step(i, evl[i])
    torch.cuda.synchronize()
    per = {}
    for si, s in enumerate(sets):
        q = [evl[i][si][0].elapsed_time(evl[i][si][1]) for i in range(n_k)]
        g = [evl[i][si][1].elapsed_time(evl[i][si][2]) for i in range(n_k)]
        per[s["key"]] = dict(quant_us=1e3 * float(np.mean(q)), gemm_us=1e3 * float(np.mean(g)),
                             quant_us_p10_50_90=[round(1e3 * float(v), 2) for v in np.percentile(q, [10, 50, 90])],
                             gemm_us_p10_50_90=[round(1e3 * float(v), 2) for v in np.percentile(g, [10, 50, 90])])

    ops_step = sum(s["w"].ops for s in sets)
    value = ops_step / (ms_per_step * 1e-3) / 1e12

    gemm_ops = sum(s["w"].ops for s in sets)
    gemm_us = sum(per[s["key"]]["gemm_us"] for s in sets)
    gemm_tops = gemm_ops / (gemm_us * 1e-6) / 1e12
    gemm_bytes_step = sum(gemm_bytes(s["w"].M, s["w"].N, s["w"].K) for s in sets)
    gemm_gbs = gemm_bytes_step / (gemm_us * 1e-6) / 1e9
    shapes = {}
    for s in sets:
        w = s["w"]
        p = per[w.key]
        qb = quant_bytes(w.M, w.K) + (w.M * (w.K - (w.K - 128) // 2 - 128) if w4a8 else 0)   # A8 rows are K bytes
        shapes[w.key] = {
            "name": w.name, "M": w.M, "K": w.K, "N": w.N,
            "quant_us": round(p["quant_us"], 2), "gemm_us": round(p["gemm_us"], 2),
            "quant_us_p10_50_90": p["quant_us_p10_50_90"], "gemm_us_p10_50_90": p["gemm_us_p10_50_90"],
            "gemm_tops": round(w.ops / (p["gemm_us"] * 1e-6) / 1e12, 1),
            "gemm_frac_int8_peak": round(w.ops / (p["gemm_us"] * 1e-6) / 1e12 / INT8_PEAK_TOPS, 4),
            "gemm_frac_fp6_peak": round(w.ops / (p["gemm_us"] * 1e-6) / 1e12 / FP6_PEAK_TOPS, 4),
            "quant_gbs": round(qb / (p["quant_us"] * 1e-6) / 1e9, 1),
            "quant_frac_hbm": round(qb / (p["quant_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "eff_tops": round(w.ops / ((p["quant_us"] + p["gemm_us"]) * 1e-6) / 1e12, 1),
            "tokens_per_s": round(w.M / ((p["quant_us"] + p["gemm_us"]) * 1e-6), 0),
        }

    traffic = None
    tr = traffic_for_current_gemm()
    if tr is not None:
        vals = [tr.get(s["key"]) for s in sets]
        if all(v is not None for v in vals):
            traffic = float(np.mean(vals))

    line = {
        "metric": ("effective W4A8 TOPS (quant+GEMM) at Llama-7B shapes; % of INT8 MFMA peak" if w4a8 else
                   "effective W4A4 TOPS (quant+GEMM) at Llama-7B shapes; % of INT8 MFMA peak"),
        "value": round(value, 2),
        "unit": "TOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "frac_int8_peak": round(value / INT8_PEAK_TOPS, 4),
        "dtype": "int8 x int4 via int8 mfma" if w4a8 else "int4 via fp6e2m3 mfma + int8",
        "data": "synthetic",
        "config": {
            "workload": ("w4a8_" if w4a8 else "") + ("llama7b_linear_" + "_".join(s["w"].name for s in sets)
                                                      if len(sets) > 1 else sets[0]["w"].name),
            "shapes_MxKxN": [f'{s["w"].M}x{s["w"].K}x{s["w"].N}' for s in sets],
            "group": 128, "outlier_channels": 128,
            "weights": "pre-packed INT4 + INT8 outlier group" + (" (offset-binary nibbles)" if w4a8 else ""),
            "activations": "INT8 in every group" if w4a8 else "INT4 + INT8 outlier group",
            "rotating_input_copies": R,
        },
        "roofline": {
            # every W4A8 group runs on the int8 matrix cores
            "kernel": "gemm_w4a8_kernel", "bound": "mfma", "achieved": round(gemm_tops, 1),
            "peak": round(INT8_PEAK_TOPS, 1), "unit": "TOP/s", "frac": round(gemm_tops / INT8_PEAK_TOPS, 4),
            "traffic": None, "ops_per_launch": gemm_ops / len(sets), "avg_launch_us": round(gemm_us / len(sets), 3),
        } if w4a8 else {
            "kernel": "gemm_w4a4_kernel", "bound": "mfma", "achieved": round(gemm_tops, 1),
            "peak": round(FP6_PEAK_TOPS, 1), "unit": "TOP/s", "frac": round(gemm_tops / FP6_PEAK_TOPS, 4),
            "traffic": traffic, "ops_per_launch": gemm_ops / len(sets),
            "avg_launch_us": round(gemm_us / len(sets), 3),
        } if args.workload != "decode" else {
            # few rows: every weight byte is used at most 16 times, so the bound is HBM
            "kernel": "gemm_w4a4_small_kernel", "bound": "hbm", "achieved": round(gemm_gbs, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gemm_gbs / HBM_PEAK_GBS, 4),
            "traffic": None, "bytes_per_launch": gemm_bytes_step / len(sets),
            "avg_launch_us": round(gemm_us / len(sets), 3),
        },
        "shapes": shapes,
    }
    if not args.no_cpu_baseline:
        log("[cpu] timing the oracle on a row sample")
        line["cpu_baseline"] = cpu_baseline(keys, args.cpu_rows, a8=w4a8)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
