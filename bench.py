#!/usr/bin/env python3
"""Benchmark of one routed-expert MoE FFN layer on one MI355X.

Headline: decode tokens/s of a DeepSeek-V4-Flash-class MoE layer (hidden
4096, 256 routed experts + 1 bf16 shared expert, intermediate 2048, top-8
softmax routing; gate/up in the 2.06-bit VQ2 codebook format, down in Q2K),
batch 1, with the achieved HBM bandwidth; prefill tokens/s at 2048 tokens is
reported beside it.  Inputs are synthetic and seeded (synth/).

A step is one moe_forward over one batch of tokens: route, dispatch, expert
FFNs (dequant fused), shared expert, combine.  The weights are held in R
replicas in distinct HBM so that consecutive steps never find them in the
256 MB last-level cache; every step uses a new token batch.  Decode steps are
replayed from HIP graphs of G consecutive steps (launch cost amortised).

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer decode tokens/s + achieved HBM GB/s; prefill tokens/s @2048"
HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0  # dense bf16 / fp16
MFMA_FP8_PEAK_TFLOPS = 5000.0  # dense fp8 (an FP8 x FP4 product runs at the FP8 rate)
MFMA_BF16_PEAK_TFLOPS = 2500.0


def _args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--workload", default="decode_b1")
    ap.add_argument("--replicas", type=int, default=8)
    ap.add_argument("--graph-steps", type=int, default=64)
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--marked-steps", type=int, default=40)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--extras", default="prefill_2048,decode_b16_zipf,verify_t6,verify_t96_zipf,"
                    "mxfp4_decode_b1,mxfp4_hash_decode_b1,mxfp4_a8_prefill_4096",
                    help="comma-separated extra workloads measured after the headline")
    ap.add_argument("--extra-steps", type=int, default=20)
    ap.add_argument("--extra-warmup", type=int, default=20)
    ap.add_argument("--no-cache-curve", action="store_true",
                    help="skip the routed-expert cache's decode-vs-hit-rate curve")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the HBM / matrix-core peak probes")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-MiB buffer 4 times (HBM counter calibration) and exit")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR",
                                                       "COPY_WRITE_DIR"),
                    help="summarise rocprofv3 FETCH_SIZE / WRITE_SIZE runs (this workload, then "
                         "the copy probe) into profiles/traffic.json and exit")
    ap.add_argument("--copy-mib", type=int, default=256)
    return ap.parse_args()


# --------------------------------------------------------------------------
# HBM traffic from hardware counters
# --------------------------------------------------------------------------

# marker name -> pattern (re.search) of the HIP kernel's symbol; the grouped
# GEMM markers take the routed weight formats only (Q2K, VQ2, MXFP4: template
# argument 1, 2 or 3), not the shared expert's bf16 instance
KERNEL_OF = {"decode_p1": r"k_dec_p1<", "decode_p2": r"k_dec_p2<", "decode_p3": r"k_dec_p3<",
             "router": r"k_router", "gemm_gateup": r"k_gemm(32|_dma)?<0, [123],",
             "gemm_down": r"k_gemm(32|_dma)?<1, [123],", "combine": r"k_combine\b",
             "select": r"k_select\(", "select_plan": r"k_select_plan", "routed_gateup": r"k_gateup",
             "routed_down": r"k_down", "shared_gateup": r"k_gateup", "shared_down": r"k_down",
             "a8_gemm_gateup": r"k_(gemm_a8|a8_dma)<0", "a8_gemm_down": r"k_(gemm_a8|a8_dma)<1",
             "act_quant": r"k_mx8_quant", "tokens_f16": r"k_tokens_f16"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


# kernel symbol substring -> the source file it is built from
SOURCE_OF = (("k_dec_", "decode.hip"), ("k_gemm_a8", "gemm_fp4.hip"), ("k_a8_dma", "gemm_fp4.hip"),
             ("k_mx8", "gemm_fp4.hip"), ("k_dense", "gemm.hip"),
             ("k_gemm", "gemm.hip"), ("k_tile_list", "gemm.hip"), ("k_tokens_f16", "gemm.hip"),
             ("k_skinny", "gemm.hip"), ("k_router", "route.hip"), ("k_select", "route.hip"),
             ("k_chunk", "route.hip"), ("k_plan", "route.hip"), ("k_gateup", "gemv.hip"),
             ("k_down", "gemv.hip"), ("k_dequant", "gemv.hip"), ("k_combine", "combine.hip"))


def sources_sha(kernel):
    """Digest of the sources kernel `kernel` (a symbol) is built from: its own
    .hip file, every shared header and the ABI header.  Counters recorded
    against another digest describe another kernel and are not reported."""
    import glob
    import hashlib

    src = next((f for sub, f in SOURCE_OF if sub in kernel), None)
    if src is None:
        return None
    csrc = os.path.join(ROOT, "routed_expert_ffn_router_amd", "csrc")
    files = [os.path.join(csrc, src)] + sorted(glob.glob(os.path.join(csrc, "*.h"))) + \
        [os.path.join(ROOT, "include", "moe.h")]
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _pmc_rows(d):
    import csv
    import glob

    out = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            out += list(csv.DictReader(fh))
    return out


def _per_kernel(rows, counter):
    acc = {}
    for r in rows:
        if r["Counter_Name"] == counter:
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return acc


def pmc_summary(args):
    fetch_d, write_d, cfetch_d, cwrite_d = args.pmc_summary
    nbytes = args.copy_mib << 20
    scale = {}
    for name, d, ctr in (("fetch", cfetch_d, "FETCH_SIZE"), ("write", cwrite_d, "WRITE_SIZE")):
        vals = [v for k, vs in _per_kernel(_pmc_rows(d), ctr).items() if "copyBuffer" in k for v in vs]
        got = max(vals) * 1024.0  # KiB -> bytes, the probe's big copy
        scale[name] = nbytes / got
    fetch = _per_kernel(_pmc_rows(fetch_d), "FETCH_SIZE")
    write = _per_kernel(_pmc_rows(write_d), "WRITE_SIZE")
    kernels = {}
    lines = [f"copy calibration: {args.copy_mib} MiB copy; FETCH_SIZE scale {scale['fetch']:.4f}, "
             f"WRITE_SIZE scale {scale['write']:.4f}",
             f"{'kernel':64s} {'launches':>8s} {'fetch MB':>10s} {'write MB':>10s} {'HBM MB':>10s}"]
    for k in sorted(fetch, key=lambda k: -np.mean(fetch[k])):
        if "copyBuffer" in k or "spin_kernel" in k or k not in write:
            continue
        f_b = float(np.mean(fetch[k])) * 1024.0 * scale["fetch"]
        w_b = float(np.mean(write[k])) * 1024.0 * scale["write"]
        kernels[k] = {"fetch_bytes": f_b, "write_bytes": w_b, "bytes": f_b + w_b,
                      "launches": len(fetch[k]), "sources_sha": sources_sha(k)}
        lines.append(f"{k[:64]:64s} {len(fetch[k]):8d} {f_b / 1e6:10.3f} {w_b / 1e6:10.3f} "
                     f"{(f_b + w_b) / 1e6:10.3f}")
    db = {}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as fh:
            db = json.load(fh)
    db[args.workload] = {"scale": scale, "kernels": kernels}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(db, fh, indent=1, sort_keys=True)
    print("\n".join(lines))


def measured_traffic(workload, marker):
    """HBM bytes per launch of `marker`'s kernel from the committed counter
    summary, or None when there is none or the kernels changed since."""
    if not os.path.exists(TRAFFIC_FILE) or marker not in KERNEL_OF:
        return None
    with open(TRAFFIC_FILE) as fh:
        rec = json.load(fh).get(workload)
    if not rec:
        return None
    hits = [(k, v) for k, v in rec["kernels"].items() if re.search(KERNEL_OF[marker], k)]
    if len(hits) != 1 or hits[0][1].get("sources_sha") != sources_sha(hits[0][0]):
        return None
    return hits[0][1]["bytes"]


def copy_probe(mib):
    import torch

    a = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(4):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_mib": mib}))


# --------------------------------------------------------------------------
# algorithmic bytes / flops
# --------------------------------------------------------------------------

def kernel_cost(name, L, T, U, n):
    """(algorithmic HBM bytes, algorithmic flops) of one launch of kernel `name`:
    every weight byte the launch needs read once, activations read and written
    once.  U: experts that received tokens; n = T*k bucket rows."""
    H, I, E, Is = L.H, L.I, L.E, L.I_shared
    gu = L.gate.nbytes_per_expert() + L.up.nbytes_per_expert()
    dn = L.down.nbytes_per_expert()
    cb = 1024 if L.gate.fmt == 2 else 0
    xb = T * H * 2
    table = {
        # fused batch-1 decode: (1) shared gate/up + router, (2) shared down +
        # select + routed gate/up, (3) routed down + combine with the shared row
        "decode_p1": (2 * Is * H * 2 + E * H * 2 + xb + Is * 4 + E * 4,
                      2 * T * (2 * Is * H + E * H)),
        "decode_p2": (U * gu + cb + xb + E * 4 + n * I * 4 + n * 8
                      + H * Is * 2 + Is * 4 + T * H * 4,
                      4 * n * I * H + 2 * T * H * Is),
        "decode_p3": (U * dn + T * H * 4 + n * I * 4 + n * 8 + T * H * 4,
                      2 * n * H * I),
        "router": (E * H * 2 + xb + T * E * 4, 2 * T * E * H),
        "shared_gateup": (2 * Is * H * 2 + xb + T * Is * 4, 4 * T * Is * H),
        "shared_down": (H * Is * 2 + T * Is * 4 + T * H * 4, 2 * T * H * Is),
        "shared_tile_list": (0, 0),
        "shared_gemm_gateup": (2 * Is * H * 2 + xb + T * Is * 2, 4 * T * Is * H),
        "shared_gemm_down": (H * Is * 2 + T * Is * 2 + T * H * 4, 2 * T * H * Is),
        "select_plan": (T * E * 4 + n * 16, 0),
        "select": (T * E * 4 + n * 8, 0),
        "dispatch_counts": (n * 4, 0),
        "dispatch_scan": (2 * ((n + 255) // 256) * E * 4, 0),
        "dispatch_scatter": (n * 4 * 4 + ((n + 255) // 256) * E * 4, 0),
        "plan": ((E + 1) * 4, 0),
        "tile_list": ((E + 1) * 4, 0),
        "routed_gateup": (U * gu + cb + xb + n * I * 4, 4 * n * I * H),
        "gateup_gemv": (U * gu + cb + xb + n * I * 4, 4 * n * I * H),
        "routed_down": (U * dn + n * I * 4 + n * H * 4, 2 * n * H * I),
        "down_gemv": (U * dn + n * I * 4 + n * H * 4, 2 * n * H * I),
        "gemm_gateup": (U * gu + cb + xb + n * I * 2, 4 * n * I * H),
        "gemm_down": (U * dn + n * I * 2 + n * H * 4, 2 * n * H * I),
        # MX-FP8 activations (1 byte + a scale byte per 32) on the FP4 matrix cores
        "act_quant": (xb + T * H + T * H // 32, 0),
        "tokens_f16": (2 * xb, 0),
        "shared_tokens_f16": (2 * xb, 0),
        "a8_gemm_gateup": (U * gu + T * H + T * H // 32 + n * I + n * I // 32, 4 * n * I * H),
        "a8_gemm_down": (U * dn + n * I + n * I // 32 + n * H * 4, 2 * n * H * I),
        "combine": (n * H * 4 + 2 * T * H * 4 + n * 8, 2 * n * H),
    }
    return table.get(name, (0, 0))


def step_bytes(L, T, U):
    """Weights streamed once per step + activations in and out."""
    gu = L.gate.nbytes_per_expert() + L.up.nbytes_per_expert()
    dn = L.down.nbytes_per_expert()
    shared = 3 * L.I_shared * L.H * 2
    router = L.E * L.H * 2
    cb = 1024 if L.gate.fmt == 2 else 0
    return U * (gu + dn) + shared + router + cb + T * L.H * 2 + T * L.H * 4


def step_flops(L, T):
    return 2 * T * (L.k * 3 * L.H * L.I + 3 * L.H * L.I_shared + L.E * L.H)


# --------------------------------------------------------------------------
# setup
# --------------------------------------------------------------------------

_LAYERS = {}  # LayerSpec -> (host layer, device replicas): one per spec for the whole run


def setup(wname, replicas, seed, npool, dev):
    import torch

    import routed_expert_ffn_router_amd as moe
    import synth

    w = synth.WORKLOADS[wname]
    if w.layer not in _LAYERS:
        for spec in list(_LAYERS):  # one layer family in device memory at a time
            if spec != w.layer:
                del _LAYERS[spec]
        torch.cuda.empty_cache()
        host = synth.gen_layer(w.layer, seed)
        _LAYERS[w.layer] = (host, [moe.DeviceLayer.upload(host, device=dev)])
    host, reps = _LAYERS[w.layer]
    while len(reps) < replicas:
        reps.append(reps[0].clone())
    layers = [r.with_route_mode(w.route).with_act(w.act) for r in reps[:replicas]]
    xs, lgs, tids = [], [], []
    for i in range(npool):
        x, lg, ti = synth.gen_step_inputs(w, seed, step=i)
        xs.append(torch.from_numpy(x.view(np.int16)).to(dev))
        lgs.append(None if lg is None else torch.from_numpy(lg).to(dev))
        tids.append(None if ti is None else torch.from_numpy(ti).to(dev))
    return w, host, layers, xs, lgs, tids


def unique_experts(f, layers, xs, lgs, tids, n=8):
    import torch

    us = []
    for i in range(min(n, len(xs))):
        f(xs[i], lgs[i], tids[i], layer=layers[i % len(layers)])
        torch.cuda.synchronize()
        us.append(len(torch.unique(f.idx)))
    return float(np.mean(us))


def time_steps(f, layers, xs, lgs, tids, steps, warmup, graph_steps, use_graph):
    """Seconds per step: the median over the timed steps (graph replays of G
    steps each: the median replay over G) of exactly `steps` steps, every one
    bracketed by a pair of events on the stream it runs on, the whole timed
    region by synchronisation."""
    import torch

    R, P = len(layers), len(xs)

    def run(i):
        f(xs[i % P], lgs[i % P], tids[i % P], layer=layers[i % R])

    if use_graph:
        G = max(g for g in range(1, graph_steps + 1) if steps % g == 0)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(warmup):
                run(i)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(G):
                run(i)
        g.replay()
        torch.cuda.synchronize()
        # the graph's last step must equal the same step run eagerly
        gout = f.out.clone()
        run(G - 1)
        torch.cuda.synchronize()
        if not torch.equal(gout, f.out):
            raise RuntimeError("graph replay differs from eager execution")
        reps = steps // G
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        torch.cuda.synchronize()
        for a, b in ev:
            a.record()
            g.replay()
            b.record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ev])) / 1e3 / G, G
    for i in range(warmup):
        run(i)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(ev):
        a.record()
        run(i)
        b.record()
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ev])) / 1e3, 1


def kernel_times(f, layers, xs, lgs, tids, steps):
    """Average duration (s) of each kernel of a step: moe_forward_marked launches
    every kernel with a pair of HIP events that the launch itself records at the
    kernel's start and end, on the stream the kernel runs on."""
    import torch

    R, P = len(layers), len(xs)
    nmax = 24
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(nmax)] for _ in range(steps)]
    for row in evs:  # torch creates the HIP event on first record
        for a, b in row:
            a.record()
            b.record()
    torch.cuda.synchronize()
    torch.cuda._sleep(60_000_000)  # keep the GPU busy while the host enqueues every step
    names = None
    for i in range(steps):
        nm = f.marked(xs[i % P], evs[i], lgs[i % P], tids[i % P], layer=layers[i % R])
        names = names or nm
    torch.cuda.synchronize()
    acc = {}
    for i in range(steps):
        for j, name in enumerate(names):
            a, b = evs[i][j]
            acc.setdefault(name, []).append(a.elapsed_time(b) / 1e3)
    return {k: float(np.median(v[1:] if len(v) > 2 else v)) for k, v in acc.items()}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(host, w, seed, budget_s, max_tokens=None):
    """The oracle (route, dequantize the selected experts, fp64 FFNs, combine)
    on the host: on all its threads for about budget_s, and single-threaded
    for about a third of that.  Decode workloads run whole steps; a prefill
    chunk runs a bounded sample of max_tokens of its tokens per call (tokens
    are independent: no capacity limit)."""
    import oracle
    import synth

    R = oracle.LayerRef(host, route_mode=w.route)
    all_threads = oracle.threads()

    def run(threads, budget):
        oracle.set_threads(threads)
        n, t_total = 0, 0.0
        while n < 1 or (t_total < budget and n < 1000):
            x, lg, ti = synth.gen_step_inputs(w, seed, step=10_000 + n)
            if max_tokens is not None:
                x = x[:max_tokens]
                lg = None if lg is None else lg[:max_tokens]
                ti = None if ti is None else ti[:max_tokens]
            t0 = time.perf_counter()
            R.forward(x, lg, ti)
            t_total += time.perf_counter() - t0
            n += 1
        return n, n * x.shape[0] / t_total, t_total

    n, v, t = run(all_threads, budget_s)
    n1, v1, t1 = run(1, budget_s / 3)
    oracle.set_threads(all_threads)
    what = (f"{w.name} (T={w.T})" if max_tokens is None else
            f"the first {max_tokens} tokens of {w.name} chunks (T={w.T})")
    return {"value": v, "unit": "tokens/s", "cores": all_threads, "kind": "oracle",
            "sample": f"{n} calls on {what} through the full oracle layer (route, dequantize "
                      f"the selected experts, fp64 FFNs, combine); {t:.1f} s",
            "single_thread": {"value": v1, "unit": "tokens/s", "cores": 1,
                              "sample": f"{n1} calls, {t1:.1f} s"},
            "nproc": os.cpu_count(), "cpu_model": cpu_model()}


def probe_peaks(dev):
    """Achievable peaks on this GPU: a streaming read of 4 GiB (16 times the
    last-level cache) and dense matrix-instruction loops on every CU."""
    import torch

    import routed_expert_ffn_router_amd as moe

    def timed(fn, reps):
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) / 1e3)
        return min(ts[1:])

    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.empty(moe.probe_sink_words(nbytes), dtype=torch.int32, device=dev)
    t = timed(lambda: moe.probe_hbm_read(buf, sink), 6)
    out = {"hbm_read_gbps": nbytes / t / 1e9}
    del buf, sink
    blocks, iters = 256 * 8, 400
    sink = torch.empty(blocks * 256 * 32, dtype=torch.float32, device=dev)
    for name, kind in (("mfma_bf16_tflops", moe.PROBE_BF16), ("mfma_f16_tflops", moe.PROBE_F16),
                       ("mfma_bf16_32x32_tflops", moe.PROBE_BF16_32),
                       ("mfma_f16_32x32_tflops", moe.PROBE_F16_32),
                       ("mfma_f8f4_tflops", moe.PROBE_F8F4)):
        fl = []
        t = timed(lambda: fl.append(moe.probe_mfma(kind, blocks, iters, sink)), 4)
        out[name] = fl[0] / t / 1e12
    del sink
    torch.cuda.empty_cache()
    out["method"] = ("moe_probe_hbm_read over 4 GiB (best of 5 launches); moe_probe_mfma, "
                     f"{blocks} workgroups x 4 waves x {iters} rounds of 8 independent "
                     "instructions (best of 3)")
    return out


def measure(wname, args, dev, headline):
    import routed_expert_ffn_router_amd as moe

    # decode steps touch ~0.1 GB of a replica: rotating over all replicas keeps
    # the 256 MB last-level cache from serving the shared expert and router
    w, host, layers, xs, lgs, tids = setup(
        wname, args.replicas if headline or w_is_decode(wname) else 2, 0,
        64 if w_is_decode(wname) else 4, dev)
    L = layers[0]
    f = moe.Forward(L, w.T, dev)
    U = unique_experts(f, layers, xs, lgs, tids)
    decode = w_is_decode(wname)
    steps = args.steps if headline else args.extra_steps
    warm = args.warmup if headline else args.extra_warmup
    sec, G = time_steps(f, layers, xs, lgs, tids, steps, warm, args.graph_steps,
                        decode and not args.no_graph)
    kt = kernel_times(f, layers, xs, lgs, tids, args.marked_steps if headline else 10)
    res = {"workload": wname, "T": w.T, "sec_per_step": sec, "tokens_per_s": w.T / sec,
           "unique_experts": U, "graph_steps": G,
           "hbm_bytes_per_step": step_bytes(L, w.T, U),
           "hbm_gbps": step_bytes(L, w.T, U) / sec / 1e9,
           "tflops": step_flops(L, w.T) / sec / 1e12,
           }
    per = {}
    for name, t in kt.items():
        nb, nf = kernel_cost(name, L, w.T, U, w.T * L.k)
        per[name] = {"us": t * 1e6, "bytes": nb, "flops": nf, "gbps": nb / t / 1e9,
                     "tflops": nf / t / 1e12}
    res["kernels"] = per
    dom = max(kt, key=kt.get)
    d = per[dom]
    # a launch whose flops per algorithmic byte exceed the chip's balance point
    # (2.5 PFLOP/s over 8 TB/s) is priced against the matrix cores
    # (the MX-FP8 x FP4 kernels against the FP8 matrix peak)
    peak = MFMA_FP8_PEAK_TFLOPS if dom.startswith("a8_") else MFMA_PEAK_TFLOPS
    mfma = d["flops"] > (peak * 1e12 / (HBM_PEAK_GBPS * 1e9)) * d["bytes"]
    if mfma:
        res["roofline"] = {"bound": "mfma", "kernel": dom, "achieved": d["tflops"],
                           "peak": peak, "unit": "TFLOP/s",
                           "frac": d["tflops"] / peak, "traffic": None,
                           "flops_per_launch": d["flops"], "us_per_launch": d["us"]}
    else:
        res["roofline"] = {"bound": "hbm", "kernel": dom, "achieved": d["gbps"],
                           "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                           "frac": d["gbps"] / HBM_PEAK_GBPS, "traffic": None,
                           "bytes_per_launch": d["bytes"], "us_per_launch": d["us"]}
    return res, host, w, L


def cache_curve(dev, hit_rates=(0.0, 0.25, 0.5, 0.75, 0.875, 1.0), n_slots=64, steps=64,
                seed=0):
    """decode_b1 with the routed experts in pinned host memory and n_slots of
    them resident in HBM (moe_forward_cached): tokens/s against the hit rate.
    Each step's logits pick round(h k) experts among the resident ones and
    the rest among the others, planned eagerly from the cache's own table
    (the device decides; the plan only reads it back between steps), then
    the same sequence is replayed from an emptied-and-warmed cache and timed
    step by step.  Roofline: the host link, measured as a pinned host -> HBM
    copy; each miss moves one expert (7,077,888 B at this layer)."""
    import torch

    import routed_expert_ffn_router_amd as moe
    import synth

    w = synth.WORKLOADS["decode_b1"]
    host = synth.gen_layer(w.layer, seed)
    cl = moe.CachedLayer(host, n_slots, dev)
    E, k = w.layer.E, w.layer.k
    per_expert = host.routed_bytes_per_expert()
    # the host link: one 512 MiB pinned -> device copy
    src = torch.empty(512 << 20, dtype=torch.uint8).pin_memory()
    dst = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    ts = []
    for _ in range(4):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src, non_blocking=True)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) / 1e3)
    link = (512 << 20) / min(ts[1:]) / 1e9
    del src, dst
    rng = np.random.default_rng(seed)
    xs = [torch.from_numpy(synth.gen_x(w.layer.H, 1, seed, step=i).view(np.int16)).to(dev)
          for i in range(16)]
    curve = []
    for h in hit_rates:
        n_hit = int(round(h * k))
        cl.reset()
        seq = []
        for s in range(n_slots // k + steps):
            res = cl.resident()
            warm = s < n_slots // k
            pool_res = np.flatnonzero(res >= 0)
            pool_non = np.flatnonzero(res < 0)
            nh = 0 if warm else n_hit
            chosen = np.concatenate([rng.choice(pool_res, nh, replace=False),
                                     rng.choice(pool_non, k - nh, replace=False)])
            lg = rng.standard_normal(E).astype(np.float32) - 10.0
            lg[chosen] = 10.0 - np.arange(k, dtype=np.float32)
            lt = torch.from_numpy(lg[None, :]).to(dev)
            seq.append(lt)
            cl(xs[s % 16], lt)
        cl.reset()
        nw = n_slots // k
        for s in range(nw):
            cl(xs[s % 16], seq[s])
        torch.cuda.synchronize()
        h0, m0 = cl.counts()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for i, (a, b) in enumerate(ev):
            a.record()
            cl(xs[(nw + i) % 16], seq[nw + i])
            b.record()
        torch.cuda.synchronize()
        h1, m1 = cl.counts()
        t = float(np.median([a.elapsed_time(b) for a, b in ev])) / 1e3
        miss_bytes = (m1 - m0) / steps * per_expert
        curve.append({"hit_rate": (h1 - h0) / max(h1 - h0 + m1 - m0, 1), "us_per_step": t * 1e6,
                      "tokens_per_s": 1.0 / t, "miss_bytes_per_step": miss_bytes,
                      "host_link_gbps": miss_bytes / t / 1e9,
                      "host_link_frac": miss_bytes / t / 1e9 / link})
    del cl
    torch.cuda.empty_cache()
    return {"n_slots": n_slots, "E": E, "k": k, "expert_bytes": per_expert,
            "host_link_probe_gbps": link, "steps": steps, "curve": curve}


def add_probed(roof, peaks):
    """Beside the spec peak: the probed one and the fraction of it."""
    if not peaks:
        return
    if roof["unit"] == "GB/s":
        p = peaks["hbm_read_gbps"]
    elif roof["kernel"].startswith("a8_"):
        p = peaks["mfma_f8f4_tflops"]
    else:  # the faster of the fp16 shapes: what this chip's matrix cores can give
        p = max(peaks["mfma_f16_tflops"], peaks["mfma_f16_32x32_tflops"])
    roof["peak_probed"] = p
    roof["frac_probed"] = roof["achieved"] / p


def w_is_decode(wname):
    import synth
    return synth.WORKLOADS[wname].T <= 64


def main():
    args = _args()
    if args.pmc_summary:
        pmc_summary(args)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "libmoe runs on one GPU: the layer is not sharded here "
                          "(see the sharding design note); run with --gpus 1"}))
        sys.exit(2)
    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    peaks = None if args.no_probes else probe_peaks(dev)
    head, host, w, L = measure(args.workload, args, dev, True)
    roof = head["roofline"]
    roof["traffic"] = measured_traffic(args.workload, roof["kernel"])
    add_probed(roof, peaks)
    extras = {}
    for name in [e for e in args.extras.split(",") if e and e != args.workload]:
        torch.cuda.empty_cache()
        r, xhost, xw, _ = measure(name, args, dev, False)
        r["roofline"]["traffic"] = measured_traffic(name, r["roofline"]["kernel"])
        add_probed(r["roofline"], peaks)
        if not args.no_cpu_baseline and xw.T >= 2048:
            r["cpu_baseline"] = cpu_baseline(xhost, xw, 0, args.cpu_seconds / 2, max_tokens=32)
        extras[name] = r
    if not args.no_cache_curve:
        _LAYERS.clear()
        torch.cuda.empty_cache()
        extras["decode_b1_expert_cache"] = cache_curve(dev)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(host, w, 0, args.cpu_seconds)
    fmt = {0: "bf16", 1: "q2k", 2: "vq2", 3: "mxfp4"}
    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["sec_per_step"] * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "H": L.H, "I": L.I, "E": L.E, "k": L.k,
                   "T": w.T, "I_shared": L.I_shared, "gate_up": fmt[L.gate.fmt],
                   "down": fmt[L.down.fmt], "shared": "bf16", "replicas": args.replicas},
        "hbm_gbps": head["hbm_gbps"],
        "hbm_frac": head["hbm_gbps"] / HBM_PEAK_GBPS,
        "hbm_bytes_per_step": head["hbm_bytes_per_step"],
        "unique_experts": head["unique_experts"],
        "kernels": head["kernels"],
        "roofline": roof,
        "cpu_baseline": cpu,
        "probed_peaks": peaks,
        "extras": extras,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
