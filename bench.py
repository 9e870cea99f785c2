#!/usr/bin/env python
"""Benchmark of the calibration-Hessian GPTQ int4 path on one MI355X.

One step is one pass of the whole path over one synthetic batch, inputs already
resident in HBM:
    hessian_accumulate (one T-token bf16 chunk into a zeroed fp32 H)
    -> hessian_pack_tril -> hessian_unpack_tril (Bf16TrilDiagF32 storage)
    -> psd_project -> gptq_factor (damp 0.01, Cholesky, U) -> gptq_sweep (+ qerr,
       importance = the stored exact diagonal).
gptq_factor + gptq_sweep is exactly gptq_quantize split in two so each half is
timed on its own.  The headline value is weights quantised per second of whole
steps, N*K / step time, on the attention shape (T=8192, K=5120, N=10240).
Per-stage times, the Hessian TFLOP/s against the bf16 matrix-core peak, and the
dominant kernel's roofline are reported alongside.  Two more blocks of the same
JSON line time the same path on the MLP down-projection shape (K=17408,
"k17408") and on the 128-chunk streamed recipe with its four weight tensors
("stream"); the CPU oracle runs one whole step of the headline workload on the
host cores.

Usage: python bench.py [--gpus 1] [--steps 5] [--warmup 2] [--workload attn5120]
                       [--no-k17408] [--no-stream] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import re
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GPTQ int4 weights quantized/sec at K=5120/17408; Hessian TFLOP/s vs MFMA peak"
# MI355X published peaks (dense): HBM 8 TB/s; bf16 2.5 PFLOP/s; int8 5.0 POP/s; fp32 157.3;
# fp64 78.6 TFLOP/s
PEAK_TFLOPS = {"bf16": 2516.6, "i8": 5000.0, "f32": 157.3, "f64": 78.6}
PEAK_HBM_GBS = 8000.0
SWEEP_BLOCK = 128          # lazy-batch width of gptq_sweep (include/gq.h)

# HBM bytes per launch of the dominant kernel, from two rocprofv3 --pmc passes
# (FETCH_SIZE, WRITE_SIZE) scaled by what the same counters read for the copy
# kernel of known size in the same run (profiles/oz_gemm_attn5120_traffic.md).
# Valid only for the kernel sources they were taken on: any change to those
# files makes the figure stale and it is reported as null.
TRAFFIC = {
    "attn5120": {"fetch_bytes": 905149.9298780488 * 1.99970 * 1024, "write_bytes": 161280.0 * 1.00000 * 1024,
                 "sources_sha256_16": "8999b5b8080889cb"},
}
TRAFFIC_SOURCES = ("post_weight_quantization_accumulate_amd/csrc/ozaki.hip",
                   "post_weight_quantization_accumulate_amd/csrc/gq_internal.h")


def traffic_for(workload):
    import hashlib
    t = TRAFFIC.get(workload)
    if t is None:
        return None, None
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest()[:16] != t["sources_sha256_16"]:
        return None, "kernel sources changed since the counters were taken"
    return t["fetch_bytes"] + t["write_bytes"], {"fetch_bytes": t["fetch_bytes"], "write_bytes": t["write_bytes"]}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=5)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--workload", default="attn5120", choices=["attn5120", "mlpdown17408", "stored1024"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-k17408", action="store_true", help="skip the K=17408 block")
    p.add_argument("--no-stream", action="store_true", help="skip the 128-chunk streamed block")
    p.add_argument("--extra-steps", type=int, default=2, help="timed steps of the K=17408 and stream blocks")
    return p.parse_args()


def cpu_baseline(wl, X, W):
    """The CPU oracle on the whole workload: every stage of one step (Gram of the
    T x K chunk, storage, PSD projection, U, the sweep of all N rows, qerr), timed
    on the host's cores with nothing scaled or extrapolated."""
    import numpy as np
    import oracle
    Xs = X.float().cpu().numpy()
    Ws = W.cpu().numpy()
    K, G = wl.K, wl.group
    t = {}
    t0 = time.perf_counter(); H = oracle.gram(Xs).astype(np.float32); t["gram"] = time.perf_counter() - t0
    del Xs
    t0 = time.perf_counter(); blob = oracle.pack_tril(H); Hs = oracle.unpack_tril(blob, K)
    t["storage"] = time.perf_counter() - t0
    t0 = time.perf_counter(); P = oracle.psd_project(Hs); t["psd"] = time.perf_counter() - t0
    t0 = time.perf_counter(); st, U, _ = oracle.gptq_U(P, wl.damp); t["factor"] = time.perf_counter() - t0
    t0 = time.perf_counter(); c, sc = oracle.gptq_sweep(Ws, U, G); t["sweep"] = time.perf_counter() - t0
    t0 = time.perf_counter(); oracle.qerr(c, sc, Ws, blob[:4 * K].view(np.float32)); t["qerr"] = time.perf_counter() - t0
    full = sum(t.values())
    return {
        "value": wl.N[0] * wl.K / full,
        "unit": "weights/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": (f"one whole step of this workload (T={wl.T}, K={wl.K}, N={wl.N[0]}), every stage "
                   f"run by the oracle, nothing scaled"),
        "step_s": full,
        "stage_s": {k: round(v, 4) for k, v in t.items()},
    }


STAGES = ["accumulate", "pack", "unpack", "psd", "factor", "sweep"]


def progress(msg):
    print(f"bench: {msg}", file=sys.stderr, flush=True)


SWEEP64_MIN_K = 8193       # gptq_quantize sweeps with its state in fp64 from here on (include/gq.h)


def run_path(gq, torch, wl, chunks, Ws, dev, steps, warmup):
    """Time whole steps of the path: zero H, accumulate every chunk (one
    hessian_accumulate_chunks call when there are several), pack, unpack,
    project, factor once, sweep every weight tensor under that U (qerr with the
    stored diagonal as importance).  Stage times come from torch events on the
    current stream; psd_project's product launches are timed by the library
    with HIP events on the same stream.

    From K = 8193 on, gptq_quantize sweeps with its state in fp64 (U, working
    weights and errors): there the step runs its two halves with that state,
    gptq_factor_f64 and gptq_sweep_f64."""
    K, G, damp = wl.K, wl.group, wl.damp
    f64 = K >= SWEEP64_MIN_K
    H = torch.empty(K, K, dtype=torch.float32, device=dev)
    blob = torch.empty(gq.hessian_tril_bytes(K), dtype=torch.uint8, device=dev)
    Hs = torch.empty(K, K, dtype=torch.float32, device=dev)
    U = torch.empty(K, K, dtype=torch.float32, device=dev)
    outs = [(torch.empty(W.shape[0], K // 2, dtype=torch.uint8, device=dev),
             torch.empty(W.shape[0], K // G, dtype=torch.float32, device=dev)) for W in Ws]
    ws_psd = gq.workspace(gq.psd_project_workspace_size(K), dev)
    ws_fac = gq.workspace(gq.gptq_factor_workspace_size(K), dev)
    ws_swp = (gq.workspace(max(gq.gptq_sweep_f64_workspace_size(W.shape[0], K, G) for W in Ws), dev) if f64
              else gq.workspace(max(gq.gptq_sweep_workspace_size(W.shape[0], K, G) for W in Ws), dev))
    U64 = torch.empty(K, K, dtype=torch.float64, device=dev) if f64 else None
    imp = blob[: 4 * K].view(torch.float32)          # stored exact diagonal of H
    ev = {s: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for s in STAGES}
    acc = {s: 0.0 for s in STAGES}
    qerr = [None] * len(Ws)

    def sweeps():
        for t, (W, (c, sc)) in enumerate(zip(Ws, outs)):
            qerr[t] = gq.gptq_sweep(c, sc, W, U, imp, G, ws_swp)

    def sweeps64():
        for t, (W, (c, sc)) in enumerate(zip(Ws, outs)):
            qerr[t] = gq.gptq_sweep_f64(c, sc, W, U64, imp, G, ws_swp)

    ws_acc = (gq.workspace(max(gq.hessian_accumulate_chunks_workspace_size(K, len(chunks)), 1), dev)
              if len(chunks) > 1 else None)

    def accumulate():
        if len(chunks) > 1:
            gq.hessian_accumulate_chunks(H, chunks, ws_acc)
        else:
            gq.hessian_accumulate(H, chunks[0])

    def step(record):
        def run(name, fn):
            if record:
                ev[name][0].record()
            fn()
            if record:
                ev[name][1].record()
        H.zero_()
        run("accumulate", accumulate)
        run("pack", lambda: gq.hessian_pack_tril(blob, H))
        run("unpack", lambda: gq.hessian_unpack_tril(Hs, blob))
        run("psd", lambda: gq.psd_project(Hs, ws_psd))
        if f64:
            run("factor", lambda: gq.gptq_factor_f64(U64, Hs, damp, ws_fac))
            run("sweep", sweeps64)
        else:
            run("factor", lambda: gq.gptq_factor(U, Hs, damp, ws_fac))
            run("sweep", sweeps)
        if record:
            torch.cuda.synchronize()
            for s in STAGES:
                acc[s] += ev[s][0].elapsed_time(ev[s][1])

    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    # psd_project brackets each launch of its product kernel with HIP events on
    # this stream (two event records per launch)
    gq.gq_set_timing(True)
    prod = {"launches": 0, "ms": 0.0, "kernel": ""}
    t0 = time.perf_counter()
    for _ in range(steps):
        step(True)
        n_l, ms_l, name = gq.psd_project_last_timing()
        prod["launches"] += n_l
        prod["ms"] += ms_l
        prod["kernel"] = name
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gq.gq_set_timing(False)
    stage_ms = {s: acc[s] / steps for s in STAGES}
    if f64:
        gq.gptq_factor(U, Hs, damp, ws_fac)          # the fp32 U the variants' sweeps take (untimed)
    return {"ms_step": wall * 1e3 / steps, "stage_ms": stage_ms, "prod": prod,
            "qerr": qerr, "H": H, "Hs": Hs, "U": U, "blob": blob, "imp": imp, "sweep_state": "f64" if f64 else "f32"}


def update_flops(N, K):
    """Algorithmic flops of the sweep's block updates: 2 N per (column, later
    column) pair outside each 128-wide block."""
    return sum(2 * N * min(SWEEP_BLOCK, K - b0) * (K - b0 - min(SWEEP_BLOCK, K - b0))
               for b0 in range(0, K, SWEEP_BLOCK))


def moduli_of(kernel_name):
    """Residue products per emulated fp64 product, as psd_project names its
    product kernel ("... N moduli"); 1 for the fp64 products."""
    m = re.search(r"(\d+) moduli", kernel_name)
    return int(m.group(1)) if m else 1


def product_roofline(K, r, steps):
    """The sign iteration's product kernel: its ops per launch and live rate."""
    prod = r["prod"]
    emulated = prod["kernel"].startswith("oz_gemm")
    per_launch = K * K * (K + 1) * (moduli_of(prod["kernel"]) if emulated else 1)
    prod_ms = prod["ms"] / prod["launches"]
    tops = per_launch / (prod_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS["i8" if emulated else "f64"]
    return emulated, per_launch, prod_ms, tops, peak


def block_summary(wl, r, steps):
    """Per-workload figures of a run_path result."""
    K, G = wl.K, wl.group
    st = r["stage_ms"]
    Ns = wl.N
    emulated, per_launch, prod_ms, tops, peak = product_roofline(K, r, steps)
    gram_flops = wl.T * wl.chunks * K * (K + 1)
    gram_tflops = gram_flops / (st["accumulate"] * 1e-3) / 1e12
    weights = sum(Ns) * K
    return {
        "config": {"workload": wl.name, "T": wl.T, "chunks": wl.chunks, "K": K, "N": Ns, "group": G,
                   "damp": wl.damp, "x_dtype": wl.x_dtype, "seed": wl.seed},
        "steps": steps,
        "ms_per_step": r["ms_step"],
        "weights_per_s": weights / (r["ms_step"] * 1e-3),
        "tensors_per_s": len(Ns) * 1e3 / r["ms_step"],
        "stages_ms": {k: round(v, 4) for k, v in st.items()},
        "gptq_weights_per_s": weights / ((st["factor"] + st["sweep"]) * 1e-3),
        "hessian_tflops": gram_tflops,
        "hessian_frac_of_bf16_peak": gram_tflops / PEAK_TFLOPS["bf16"],
        "sweep_state": r["sweep_state"],
        "sweep_update_tflops": sum(update_flops(N, K) for N in Ns) / (st["sweep"] * 1e-3) / 1e12,
        "psd_products_per_call": r["prod"]["launches"] / steps,
        "psd_product_kernel": {"kernel": r["prod"]["kernel"], "avg_launch_ms": prod_ms, "per_launch_ops": per_launch,
                               "achieved": tops, "peak": peak, "unit": "TOP/s" if emulated else "TFLOP/s",
                               "frac": tops / peak},
        "qerr": r["qerr"],
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "sharding of this path is a design note, not a measured configuration.", file=sys.stderr)
        sys.exit(2)

    import torch
    import post_weight_quantization_accumulate_amd as gq
    import synthgen as g

    dev = "cuda:0"
    torch.cuda.set_device(0)
    wl = g.WORKLOADS[args.workload]
    T, K, N, G, damp = wl.T, wl.K, wl.N[0], wl.group, wl.damp
    X = g.x_chunk(wl, device=dev)
    W = g.weights(wl, device=dev)
    torch.cuda.synchronize()

    r = run_path(gq, torch, wl, [X], [W], dev, args.steps, args.warmup)
    progress(f"{wl.name}: {args.steps} steps, {r['ms_step']:.2f} ms per step")
    ms_step, stage_ms = r["ms_step"], r["stage_ms"]
    Hs, U, blob, imp = r["Hs"], r["U"], r["blob"], r["imp"]
    qerr = r["qerr"]

    gram_flops = T * K * (K + 1)
    gram_tflops = gram_flops / (stage_ms["accumulate"] * 1e-3) / 1e12
    prod_flops = K * K * (K + 1)                     # one symmetric product, lower triangle
    emulated, per_launch, prod_ms, prod_tops, peak = product_roofline(K, r, args.steps)
    n_prod = r["prod"]["launches"] / args.steps
    upd_flops = update_flops(N, K)
    gptq_ms = stage_ms["factor"] + stage_ms["sweep"]
    traffic, traffic_detail = traffic_for(wl.name)

    out = {
        "metric": METRIC,
        "value": N * K / (ms_step * 1e-3),
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "dtype_by_stage": {"accumulate": "bf16 products, f32 accumulate",
                           "psd": ("f64-class products: operands rounded per row to integers of 40 bits (12 "
                                   "moduli, K <= 8192) or 43-44 bits (13 moduli), exact int8 residue products, "
                                   "128-bit CRT, f64 epilogue"
                                   if emulated else "f64"),
                           "factor": "f64", "sweep": "f32", "storage": "u16/u32 bits"},
        "data": "synthetic",
        "config": {"workload": wl.name, "T": T, "K": K, "N": N, "group": G, "damp": damp,
                   "x_dtype": wl.x_dtype, "seed": wl.seed},
        "stages_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "hessian_tflops": gram_tflops,
        "hessian_frac_of_bf16_peak": gram_tflops / PEAK_TFLOPS["bf16"],
        "tensors_per_s": 1e3 / ms_step,
        "gptq_weights_per_s": N * K / (gptq_ms * 1e-3),
        "sweep_update_tflops": upd_flops / (stage_ms["sweep"] * 1e-3) / 1e12,
        "qerr": qerr[0],
        "psd_f64_equivalent_tflops": n_prod * prod_flops / (stage_ms["psd"] * 1e-3) / 1e12,
        "roofline": {
            "bound": "mfma",
            "kernel": r["prod"]["kernel"] + ", sign-iteration symmetric product; timed alone with HIP events",
            "achieved": prod_tops,
            "peak": peak,
            "unit": "TOP/s" if emulated else "TFLOP/s",
            "frac": prod_tops / peak,
            "traffic": traffic,
            "traffic_detail": traffic_detail,
            "algorithmic_bytes_per_launch": (
                {"read_residue_planes_A_B": 2 * moduli_of(r["prod"]["kernel"]) * K * K,
                 "write_residues_lower": moduli_of(r["prod"]["kernel"]) * K * (K + 1) // 2}
                if emulated else
                {"read_AB": 2 * K * K * 8, "read_cin_step_products": K * K * 8, "write_lower_and_mirror": K * K * 8}),
            "per_launch_ops": per_launch,
            "avg_launch_ms": prod_ms,
            "launches_per_step": n_prod,
        },
    }
    out["rtn"] = rtn_measure(gq, torch, W, imp, G, dev)
    out["hfqm"] = hfqm_measure(gq, blob, imp, K)
    out["hadamard"] = hadamard_measure(gq, torch, W, Hs, dev)
    out["variants"] = variants_measure(gq, torch, W, U, Hs, imp, G, damp, dev)
    out["rtn"]["qerr_gptq_over_rtn"] = qerr[0] / out["rtn"]["qerr"] if out["rtn"]["qerr"] else None
    progress("round to nearest, HFQM, rotation and variants measured")
    del r, Hs, U
    torch.cuda.empty_cache()
    if not args.no_k17408 and wl.name != "mlpdown17408":
        out["k17408"] = k17408_measure(gq, torch, g, dev, args.extra_steps)
        torch.cuda.empty_cache()
        progress(f"mlpdown17408: {out['k17408']['ms_per_step']:.1f} ms per step")
    if not args.no_stream:
        out["stream"] = stream_measure(gq, torch, g, dev, args.extra_steps)
        torch.cuda.empty_cache()
        progress(f"stream5120: {out['stream']['ms_per_step']:.1f} ms per step")
    if not args.no_cpu_baseline:
        progress("CPU oracle: one whole step of the headline workload")
        out["cpu_baseline"] = cpu_baseline(wl, X, W)
        progress(f"CPU oracle: {out['cpu_baseline']['step_s']:.1f} s")
    print(json.dumps(out))


def k17408_measure(gq, torch, g, dev, steps):
    """The MLP down-projection shape (T=8192, K=17408, N=5120, heavy-tailed bf16
    activations): whole steps of the same path as the headline, one warm-up."""
    wl = g.WORKLOADS["mlpdown17408"]
    X = g.x_chunk(wl, device=dev)
    W = g.weights(wl, device=dev)
    torch.cuda.synchronize()
    r = run_path(gq, torch, wl, [X], [W], dev, steps, 1)
    return block_summary(wl, r, steps)


def stream_measure(gq, torch, g, dev, steps):
    """The streamed recipe: 128 chunks of 8192 bf16 tokens at K=5120, generated
    and staged in HBM (10.7 GB) before timing, accumulated into one H per step,
    then storage, projection, one factor and the sweeps of the four weight
    tensors (N = 5120, 10240, 1024, 1024) that share it; one warm-up."""
    wl = g.WORKLOADS["stream5120"]
    chunks = [g.x_chunk(wl, c, device=dev) for c in range(wl.chunks)]
    Ws = [g.weights(wl, t, device=dev) for t in range(len(wl.N))]
    torch.cuda.synchronize()
    r = run_path(gq, torch, wl, chunks, Ws, dev, steps, 1)
    out = block_summary(wl, r, steps)
    out["hessian_target_ms_at_60pct"] = wl.T * wl.chunks * wl.K * (wl.K + 1) / (0.6 * PEAK_TFLOPS["bf16"] * 1e12) * 1e3
    return out


def hadamard_measure(gq, torch, W, H, dev, block=1024, reps=10):
    """The block Walsh-Hadamard rotation (blocks of 1024, random signs) of a copy of
    W (W R^T) and of the step's Hessian (R H R^T), timed after the steps with HIP
    events.  Algorithmic bytes: one read and one write of each matrix; the
    Hessian's two-sided rotation runs as rows, transpose, rows, copy (4x that)."""
    N, K = W.shape
    g = torch.Generator(device="cpu").manual_seed(1)
    signs = (torch.randint(0, 2, (K,), generator=g) * 2 - 1).float().to(dev)
    Wc, Hc = W.clone(), H.clone()
    ws = gq.workspace(gq.hadamard_rotate_hessian_workspace_size(K), dev)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {"block": block}
    for name, fn, nbytes in (("rows", lambda: gq.hadamard_rotate_rows(Wc, block, signs), 8 * N * K),
                             ("hessian", lambda: gq.hadamard_rotate_hessian(Hc, block, ws, signs), 8 * K * K)):
        fn()
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        res[name + "_ms"] = ms
        res[name + "_gb_per_s"] = nbytes / (ms * 1e-3) / 1e9
        res[name + "_frac_of_hbm_peak"] = nbytes / (ms * 1e-3) / 1e9 / 8000.0
    return res


def variants_measure(gq, torch, W, U, H, imp, G, damp, dev, reps=3):
    """The sweep's variants under the step's U (static groups, the NF4 codebook,
    both; "plain" is gptq_sweep_ex with no flag, the step's own sweep) and NF4
    round to nearest, each timed per API call with HIP events after the steps,
    with its qerr (same importance).  Act order needs the factor of the permuted
    Hessian, so it is timed as a whole gptq_quantize_ex call (permutation, permuted
    H, factor, permuted sweep, codes put back) beside the same call with static
    groups alone."""
    N, K = W.shape
    codes = torch.empty(N * (K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty(N * (K // G), dtype=torch.float32, device=dev)
    ws = gq.workspace(gq.gptq_sweep_workspace_size(N, K, G), dev)
    ws_r = gq.workspace(gq.rtn_quantize_workspace_size(N, K, G), dev)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {"sweep_ms": {}, "qerr": {}}
    calls = [(name, lambda f=f: gq.gptq_sweep_ex(codes, scales, W, U, imp, G, f, ws))
             for name, f in (("plain", 0), ("static", gq.GQ_STATIC_GROUPS), ("nf4", gq.GQ_NF4),
                             ("static_nf4", gq.GQ_STATIC_GROUPS | gq.GQ_NF4))]
    calls.append(("rtn_nf4", lambda: gq.rtn_quantize_ex(codes, scales, W, imp, G, gq.GQ_NF4, ws_r)))
    act = gq.GQ_STATIC_GROUPS | gq.GQ_ACT_ORDER
    ws_q = gq.workspace(gq.gptq_quantize_ex_workspace_size(N, K, G, act), dev)
    for name, f in (("quantize_static", gq.GQ_STATIC_GROUPS), ("quantize_static_act", act)):
        calls.append((name, lambda f=f: gq.gptq_quantize_ex(codes, scales, W, H, imp, G, damp, f, ws_q)))
    res["quantize_ms"] = {}
    for name, fn in calls:
        q = fn()
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        if name == "rtn_nf4":
            res["rtn_nf4_ms"] = a.elapsed_time(b) / reps
        elif name.startswith("quantize_"):
            res["quantize_ms"][name[len("quantize_"):]] = a.elapsed_time(b) / reps
        else:
            res["sweep_ms"][name] = a.elapsed_time(b) / reps
        res["qerr"][name] = q
    return res


def hfqm_measure(gq, blob, imp, K, reps=3):
    """The stored Hessian and its imatrix as a two-entry HFQM package: write to a
    temporary file and read back (index and both payloads), host to disk and back,
    after the timed steps; the device blob is copied to the host first (not timed)."""
    import tempfile
    ents = [("blk.0.hessian", gq.GQ_HFQM_HESSIAN, (K, K), 0, blob.cpu().numpy()),
            ("blk.0.imatrix", gq.GQ_HFQM_F32, (K,), 0, imp.cpu().numpy())]
    nbytes = sum(e[4].nbytes for e in ents)
    with tempfile.TemporaryDirectory() as d:
        p = os.path.join(d, "bench.calib.hfq")
        tw = tr = 0.0
        for _ in range(reps):
            t0 = time.perf_counter()
            gq.hfqm_write(p, 0, '{"producer":"bench"}', ents)
            t1 = time.perf_counter()
            _, _, idx = gq.hfqm_read(p)
            for i, e in enumerate(idx):
                gq.hfqm_read_payload(p, i, e[4])
            t2 = time.perf_counter()
            tw += t1 - t0
            tr += t2 - t1
        size = os.path.getsize(p)
    return {"payload_bytes": nbytes, "file_bytes": size, "write_mb_per_s": nbytes * reps / tw / 1e6,
            "read_mb_per_s": nbytes * reps / tr / 1e6, "where": "tempfile directory of the host"}


def rtn_measure(gq, torch, W, imp, G, dev, reps=10):
    """The round-to-nearest pack of the same weights on the same grid (with qerr,
    the same importance), timed after the GPTQ steps.  One kernel reads W and imp
    once and writes codes, scales and qerr's partial sums; ms_per_call is the
    whole API call (launches, status and qerr readback, host synchronisation)."""
    N, K = W.shape
    codes = torch.empty(N * (K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty(N * (K // G), dtype=torch.float32, device=dev)
    ws = gq.workspace(gq.rtn_quantize_workspace_size(N, K, G), dev)
    q = gq.rtn_quantize(codes, scales, W, imp, G, ws)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        gq.rtn_quantize(codes, scales, W, imp, G, ws)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    nbytes = 4 * N * K + N * K // 2 + 4 * N * K // G + 4 * K
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"ms_per_call": ms, "algorithmic_bytes": nbytes, "achieved_gb_per_s": gbs,
            "frac_of_hbm_peak": gbs / 8000.0, "weights_per_s": N * K / (ms * 1e-3), "qerr": q}


if __name__ == "__main__":
    main()
