#!/usr/bin/env python3
"""Benchmark of one quantized MoE layer (GLM-5.2 shape) on one MI355X.

A step is one moe_layer call -- router, permutation, routed and shared expert
FFNs, combine -- over one batch of synthetic inputs resident in HBM.  The
headline workload is single-token decode (hidden 6144, moe_inter 2048, 256
experts, top-8 of 4 kept groups out of 8, one shared expert, int4 weights with
fp16 scales per 32 inputs).  Weight sets are replicated and rotated so that no
step reads weights another step left in the 256 MB Infinity Cache.

Prints one JSON line.  Usage:
    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads a,b,...]
    python bench.py --copy-calibration      (plain copy kernel, for PMC scaling)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + weight-stream HBM GB/s (% peak); prefill MFMA util"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_F16_TFLOPS = 2500.0       # MI355X dense fp16/bf16 MFMA
PEAK_I8_TOPS = 5000.0          # MI355X dense int8 MFMA
ALL_WORKLOADS = ["decode", "verify4", "verify64", "prefill4k", "prefill16k", "nvfp4_512",
                 "decode_topp", "verify64_topp", "decode_stream", "decode_stream_warm",
                 "decode_int4_row", "decode_int8_row", "decode_int2_row", "verify4_int2_row",
                 "prefill4k_int4_row",
                 "prefill4k_int8_row", "prefill4k_w4a8", "prefill16k_w4a8", "verify64_w4a8"]
HEADLINE = "decode"
# expert streaming from host memory: the decode layer with its 256 routed
# experts in page-locked host RAM and this many HBM slots (moe_layer_cached)
STREAM_WORKLOADS = {"decode_stream": 64, "decode_stream_warm": 256}
PEAK_HOST_LINK_GBS = 64.0      # PCIe 5.0 x16, one direction


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workloads", default=",".join(ALL_WORKLOADS))
    ap.add_argument("--replicas", type=int, default=0, help="weight replicas (0: automatic)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-trace", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--json-out", default=None)
    return ap.parse_args()


# ---------------------------------------------------------------------------
# algorithmic bytes and flops
# ---------------------------------------------------------------------------

ROW_BITS = {"int4_row": 4, "int8_row": 8, "int2_row": 2}


def proj_bytes(N, K, wfmt):
    if wfmt == "int4":
        return N * K // 2 + (N * K // 32) * 2
    if wfmt in ROW_BITS:
        return N * K * ROW_BITS[wfmt] // 8 + 4 * N
    return N * K // 2 + N * K // 16 + 4


def expert_bytes(H, I, wfmt):
    return {"gate": proj_bytes(I, H, wfmt), "up": proj_bytes(I, H, wfmt),
            "down": proj_bytes(H, I, wfmt)}


def algorithmic(geom, wfmt, T, n_active):
    """Bytes the method must move and flops it must do for one layer call, and
    per kernel of the launch sequence (keys are the kernel names the library's
    trace reports).  Bytes count each operand once: the weights of every
    selected expert, activations in, results out."""
    H, I, E, k = geom["hidden"], geom["moe_inter"], geom["n_routed_experts"], geom["top_k"]
    Is = geom["shared_inter"] if geom["n_shared_experts"] else 0
    P = T * k
    eb = expert_bytes(H, I, wfmt)
    sb = expert_bytes(H, Is, wfmt) if Is else {"gate": 0, "up": 0, "down": 0}
    x_b, y_b = T * H * 2, T * H * 4
    router_b = E * H * 4 + E * 4
    layer_bytes = n_active * sum(eb.values()) + sum(sb.values()) + router_b + x_b + y_b
    layer_flops = P * 2 * H * I * 3 + T * 2 * H * Is * 3 + T * 2 * H * E
    rows = P + (T if Is else 0)                   # routed pairs + shared rows
    w_gu = n_active * (eb["gate"] + eb["up"]) + sb["gate"] + sb["up"]
    w_dn = n_active * eb["down"] + sb["down"]
    f_gu = P * 2 * H * I * 2 + T * 2 * H * Is * 2
    f_dn = P * 2 * H * I + T * 2 * H * Is
    # selection: logits and bias in; ids, weights, expert records (48 bytes),
    # per-pick expert/token words and the count out
    sel_b = T * E * 8 + E * 4 + P * 8 + n_active * 48 + P * 4 + 4
    # the shared expert's gate/up runs beside the selection (dec_fused_t1 for
    # one token, dec_select_permute otherwise); its down projection runs with
    # the routed ones
    sh_sel = Is > 0
    sh_gu_b = sb["gate"] + sb["up"] + T * Is * 2
    sh_gu_f = T * 2 * H * Is * 2
    kern = {
        # small-batch path
        "dec_router": dict(bytes=router_b + x_b + T * E * 8, flops=T * 2 * H * E),
        "dec_select_permute": dict(bytes=sel_b + (sh_gu_b if sh_sel else 0), flops=sh_gu_f if sh_sel else 0),
        "dec_gateup": dict(bytes=n_active * (eb["gate"] + eb["up"]) + x_b + P * I * 2,
                           flops=P * 2 * H * I * 2),
        "dec_down_combine": dict(bytes=w_dn + rows * I * 2 + y_b, flops=f_dn + 2 * P * H),
    }
    # one token: selection, gate/up and down in one launch (the three rows
    # above together)
    kern["dec_fused_t1"] = {m: sum(kern[k][m] for k in ("dec_select_permute", "dec_gateup", "dec_down_combine"))
                            for m in ("bytes", "flops")}
    # 2-4 tokens: selection and gate/up in one launch
    kern["dec_select_gateup"] = {m: sum(kern[k][m] for k in ("dec_select_permute", "dec_gateup"))
                                 for m in ("bytes", "flops")}
    kern.update({
        # large-batch path
        "route_logits": dict(bytes=router_b + x_b + T * E * 8, flops=T * 2 * H * E),
        "route_select": dict(bytes=T * E * 8 + E * 4 + P * 8, flops=0),
        "permute": dict(bytes=P * 4 * 3 + (E + 1) * 4, flops=0),
        "gemm_prep": dict(bytes=x_b * 2, flops=0),
        "gemm_gateup": dict(bytes=w_gu + x_b + rows * I * 2, flops=f_gu),
        "gemm_down": dict(bytes=w_dn + rows * I * 2 + rows * H * 4, flops=f_dn),
        "combine": dict(bytes=rows * H * 4 + P * 8 + y_b, flops=2 * P * H),
        # moe_expert_ffn_q4 on few tokens
        "gateup_gemv": dict(bytes=w_gu + x_b + rows * I * 2, flops=f_gu),
        # W4A8: the SwiGLU outputs to int8 rows between the projections
        "quant_h": dict(bytes=rows * I * 3 + rows * 8, flops=0),
        "down_gemv": dict(bytes=w_dn + rows * I * 2 + rows * H * 4, flops=f_dn),
    })
    return layer_bytes, layer_flops, kern


KERNEL_SOURCES = {
    "dec_": ["decode.hip", "select_token.h", "qmoe_device.h", "qmoe_internal.h"],
    "gemm_": ["gemm.hip", "gemm_i8.hip", "gemm_common.h", "qmoe_device.h", "qmoe_internal.h"],
    "quant_h": ["gemm_i8.hip", "gemm_common.h", "qmoe_device.h", "qmoe_internal.h"],
    "route_": ["route.hip", "decode.hip", "select_token.h", "qmoe_device.h", "qmoe_internal.h"],
    "permute": ["permute.hip", "qmoe_device.h", "qmoe_internal.h"],
    "combine": ["gemv.hip", "qmoe_device.h", "qmoe_internal.h"],
    "gateup_gemv": ["gemv.hip", "qmoe_device.h", "qmoe_internal.h"],
    "down_gemv": ["gemv.hip", "qmoe_device.h", "qmoe_internal.h"],
}


def strip_comments(src):
    """C/C++ source text without its comments (string and character literals
    kept as they are), so that a comment edit does not count as a change."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return "".join(out)


def source_code(src):
    """The code lines of a C/C++ source: comments stripped, blank lines and
    trailing spaces dropped."""
    return "\n".join(l.rstrip() for l in strip_comments(src).splitlines() if l.strip())


def kernel_source_hash(kernel):
    """sha256 over the code (source_code) of the sources a kernel is compiled
    from (None if unknown)."""
    import hashlib
    files = next((v for p, v in KERNEL_SOURCES.items() if kernel.startswith(p)), None)
    if files is None:
        return None
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "quantized_moe_02_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(source_code(fh.read()).encode())
    return h.hexdigest()


def traffic_for(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 PMC
    readings (FETCH_SIZE + WRITE_SIZE, each scaled by the same counter's
    reading for a copy kernel of known size); None when no reading exists or
    the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(f"{kernel}@{workload}")
    h = kernel_source_hash(kernel)
    if not rec or h is None or rec.get("sha256") != h:
        return None
    return rec["fetch_kib"] * 1024 * rec["fetch_scale"] + rec["write_kib"] * 1024 * rec["write_scale"]


def roofline_bound(kb):
    """A kernel is MFMA-bound when its arithmetic intensity exceeds the
    machine balance (dense fp16 flops per HBM byte), else HBM-bound."""
    return "mfma" if kb["flops"] > kb["bytes"] * (PEAK_F16_TFLOPS * 1e12) / (PEAK_HBM_GBS * 1e9) else "hbm"


# ---------------------------------------------------------------------------
# layer set-up
# ---------------------------------------------------------------------------

def clone_experts(qe):
    import synth
    c = lambda p: synth.QProj(p.q.clone(), p.scale.clone(), None if p.gscale is None else p.gscale.clone())
    return synth.QExperts(c(qe.gate), c(qe.up), c(qe.down))


class Bench:
    def __init__(self, name, replicas):
        import quantized_moe_02_amd as q
        import synth
        self.q = q
        self.name = name
        self.L = L = synth.make_layer(name, "cuda")
        self.geom, self.T, self.wfmt = L.geom, L.T, L.wfmt
        g = self.geom
        self.options = synth.WORKLOADS[name].get("options", 0)
        self.cfg = q.make_config(g, L.wfmt, self.options)
        self.sets = [(L.router_w, L.bias, L.routed, L.shared)]
        for _ in range(replicas - 1):
            self.sets.append((L.router_w.clone(), L.bias.clone(), clone_experts(L.routed),
                              clone_experts(L.shared) if L.shared is not None else None))
        torch.cuda.synchronize()

        def qx(qe):
            t = lambda p: (p.q, p.scale, p.gscale)
            return q.qexperts(t(qe.gate), t(qe.up), t(qe.down))
        self.qsets = [(rw, b, qx(r), qx(s) if s is not None else None) for rw, b, r, s in self.sets]
        self.ws = q.workspace(self.cfg, self.T)
        self.y = torch.empty(self.T, g["hidden"], device="cuda", dtype=torch.float32)
        self.ids = torch.empty(self.T, g["top_k"], device="cuda", dtype=torch.int32)
        self.tw = torch.empty(self.T, g["top_k"], device="cuda", dtype=torch.float32)

    def step(self, i, stream=None):
        rw, b, r, s = self.qsets[i % len(self.qsets)]
        self.q.moe_layer(self.cfg, self.T, self.L.x, rw, b, r, s, self.y, self.q.MOE_OUT_F32,
                         self.ids, self.tw, self.ws, stream=stream)

    def step_traced(self, i, trace):
        rw, b, r, s = self.qsets[i % len(self.qsets)]
        self.q.moe_layer_trace(self.cfg, self.T, self.L.x, rw, b, r, s, self.y, trace,
                               self.q.MOE_OUT_F32, self.ids, self.tw, self.ws)

    def n_active(self):
        # experts with at least one kept pick (-1: a pick the adaptive top-p dropped)
        return int(torch.unique(self.ids[self.ids >= 0]).numel())


def time_steps(B: Bench, steps, warmup, use_graph):
    """Whole-step throughput over exactly `steps` steps.  Decode-sized steps
    replay captured HIP graphs -- one of a step per replica, replayed
    steps // R times, and one of the remaining steps % R steps -- so that
    Python launch overhead does not idle the GPU."""
    R = len(B.qsets)
    for i in range(warmup):
        B.step(i)
    torch.cuda.synchronize()
    if use_graph:
        def capture(n_steps):
            g = torch.cuda.CUDAGraph()
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                with torch.cuda.graph(g, stream=s):
                    for i in range(n_steps):
                        B.step(i)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            return g
        g = capture(R)
        reps, rem = divmod(steps, R)
        g_rem = capture(rem) if rem else None
        t0 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        if g_rem is not None:
            g_rem.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        # per-step spread, from events around each replay of R steps (after
        # the timed run)
        nrep = max(1, reps)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(nrep + 1)]
        ev[0].record()
        for j in range(nrep):
            g.replay()
            ev[j + 1].record()
        torch.cuda.synchronize()
        per = [ev[j].elapsed_time(ev[j + 1]) * 1e3 / R for j in range(nrep)]
        return steps, (t1 - t0), per
    t0 = time.perf_counter()
    for i in range(steps):
        B.step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        B.step(i)
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(steps)]
    return steps, (t1 - t0), per


def trace_kernels(B: Bench, steps):
    """Average duration of each kernel of moe_layer, from HIP events recorded
    by the library at kernel boundaries on the launch stream.  The steps are
    queued behind a sleep kernel so that host launch gaps do not enter the
    intervals."""
    q = B.q
    per = {}
    traces = []
    evs = []
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2.4e9 * 0.02 + steps * 2.4e9 * 150e-6))   # ~20 ms + 150 us/step of cycles
    for i in range(steps):
        tr = q.MoeTrace()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(q.MOE_TRACE_MAX + 1)]
        for j, ev in enumerate(e):
            ev.record()   # materialise the event object
            tr.events[j] = ev.cuda_event
        B.step_traced(i, tr)
        traces.append(tr)
        evs.append(e)
    torch.cuda.synchronize()
    for tr, e in zip(traces, evs):
        for j in range(tr.n_kernels):
            name = tr.names[j].decode()
            per.setdefault(name, []).append(e[j].elapsed_time(e[j + 1]) * 1e3)   # us
    return {k: float(np.mean(v)) for k, v in per.items()}


def run_workload(name, args):
    T = __import__("synth").WORKLOADS[name]["tokens"]
    decode_like = T <= 64
    replicas = args.replicas or (8 if decode_like else 2)
    B = Bench(name, replicas)
    steps = args.steps or (400 if decode_like else (40 if T <= 4096 else 12))
    warmup = args.warmup if args.warmup is not None else (20 if decode_like else 3)
    n, dt, per_step = time_steps(B, steps, warmup, use_graph=decode_like)
    B.step(0)
    torch.cuda.synchronize()
    n_active = B.n_active()
    lb, lf, kern = algorithmic(B.geom, B.wfmt, B.T, n_active)
    s_per_step = dt / n
    res = dict(workload=name, tokens=B.T, steps=n, warmup=warmup, replicas=replicas,
               ms_per_step=s_per_step * 1e3, tokens_per_s=B.T / s_per_step,
               hbm_gbs=lb / s_per_step / 1e9, hbm_pct_peak=100 * lb / s_per_step / 1e9 / PEAK_HBM_GBS,
               tflops=lf / s_per_step / 1e12, active_experts=n_active,
               algorithmic_bytes=lb, algorithmic_flops=lf, graph=decode_like,
               # spread over a second run of the same steps, one event pair per step
               # (per graph replay of `replicas` steps for decode-sized workloads)
               step_us={"p10": float(np.percentile(per_step, 10)), "median": float(np.median(per_step)),
                        "p90": float(np.percentile(per_step, 90))})
    if not args.no_trace:
        ksteps = min(steps, 64 if decode_like else 8)
        kt = trace_kernels(B, ksteps)
        res["kernels_us"] = kt
        dom = max(kt, key=kt.get)
        kb = kern[dom]
        dur = kt[dom] * 1e-6
        if roofline_bound(kb) == "mfma":
            ach = kb["flops"] / dur / 1e12
            # the W4A8 path multiplies on the int8 matrix cores
            i8 = bool(B.options & 4)
            peak = PEAK_I8_TOPS if i8 else PEAK_F16_TFLOPS
            res["roofline"] = dict(kernel=dom, bound="mfma", achieved=ach, peak=peak,
                                   unit="TOP/s" if i8 else "TFLOP/s", frac=ach / peak,
                                   traffic=traffic_for(dom, name),
                                   algorithmic=kb["flops"], avg_us=kt[dom])
        else:
            ach = kb["bytes"] / dur / 1e9
            res["roofline"] = dict(kernel=dom, bound="hbm", achieved=ach, peak=PEAK_HBM_GBS,
                                   unit="GB/s", frac=ach / PEAK_HBM_GBS,
                                   traffic=traffic_for(dom, name),
                                   algorithmic=kb["bytes"], avg_us=kt[dom])
    del B
    torch.cuda.empty_cache()
    return res


def run_stream_workload(name, args):
    """Single-token decode with the routed experts streamed from host memory
    through an expert cache of n HBM slots (LRU, loads on miss): a step is one
    moe_layer_cached call on a fresh token (routing, one host synchronisation,
    the misses' host-to-device copies, the expert FFNs, the combine).
    decode_stream: 64 slots, cold start, warm-up steps fill the cache, then the
    steady state of uniform routing (about a quarter of the picks hit).
    decode_stream_warm: 256 slots, all experts prefetched first: every pick
    hits, so a step is the cached path's cost without transfers."""
    import quantized_moe_02_amd as q
    import synth
    n_slots = STREAM_WORKLOADS[name]
    L = synth.make_layer("decode", "cuda")
    g = L.geom
    cfg = q.make_config(g, L.wfmt)
    projs = (L.routed.gate, L.routed.up, L.routed.down)
    host = [tuple(None if t is None else t.cpu().pin_memory() for t in (p.q, p.scale, p.gscale))
            for p in projs]
    slots = [tuple(None if t is None else torch.empty((n_slots,) + tuple(t.shape[1:]), dtype=t.dtype,
                                                      device="cuda")
                   for t in (p.q, p.scale, p.gscale)) for p in projs]
    L.routed = None
    del projs
    torch.cuda.empty_cache()
    h_store, d_slots = q.qexperts(*host), q.qexperts(*slots)
    shared = q.qexperts(*[(p.q, p.scale, p.gscale) for p in (L.shared.gate, L.shared.up, L.shared.down)])
    cache = q.moe_cache_create(cfg, n_slots, h_store, d_slots)
    steps = args.steps or 200
    warmup = args.warmup if args.warmup is not None else 20
    H, k = g["hidden"], g["top_k"]
    X = synth.to_bf16(synth.randn((warmup + steps, H), synth.sub_seed(L.seed, 77), "cuda"))
    ws = q.workspace(cfg, 1)
    y = torch.empty(1, H, device="cuda")
    ids = torch.empty(1, k, dtype=torch.int32, device="cuda")
    tw = torch.empty(1, k, dtype=torch.float32, device="cuda")

    def step(i):
        q.moe_layer_cached(cache, 1, X[i:i + 1], L.router_w, L.bias, shared, y, q.MOE_OUT_F32, ids,
                           tw, ws)

    try:
        if n_slots == g["n_routed_experts"]:
            q.moe_cache_prefetch(cache, list(range(n_slots)))
        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        s0 = q.moe_cache_get_stats(cache)
        t0 = time.perf_counter()
        for i in range(steps):
            step(warmup + i)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        s1 = q.moe_cache_get_stats(cache)
    finally:
        q.moe_cache_destroy(cache)
    # the DMA engine's own rate on this machine: one 1 GiB page-locked host-to-device copy
    src = torch.empty(1 << 30, dtype=torch.uint8).pin_memory()
    dst = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    best = 0.0
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src, non_blocking=True)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, (1 << 30) / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    misses = s1["misses"] - s0["misses"]
    hits = s1["hits"] - s0["hits"]
    moved = s1["bytes_loaded"] - s0["bytes_loaded"]
    h2d = moved / dt / 1e9
    res = dict(workload=name, tokens=1, steps=steps, warmup=warmup, slots=n_slots,
               experts=g["n_routed_experts"], ms_per_step=dt / steps * 1e3,
               tokens_per_s=steps / dt, misses_per_token=misses / steps,
               hit_rate=hits / max(1, hits + misses), h2d_bytes_per_token=moved / steps,
               h2d_gbs=h2d, copy_ceiling_gbs=best,
               roofline=dict(kernel="host-to-device copies", bound="host_link", achieved=h2d,
                             peak=PEAK_HOST_LINK_GBS, unit="GB/s", frac=h2d / PEAK_HOST_LINK_GBS,
                             traffic=None, algorithmic=moved / steps))
    del src, dst, host, slots
    torch.cuda.empty_cache()
    return res


def cpu_baseline(name, budget_s=10.0, max_calls=16):
    """The fp64 oracle on tokens of the workload, on this host's cores: single-token
    calls (routing, dequantisation of the chosen experts, their FFNs, combine) until
    about budget_s seconds of CPU work, then one call on a single thread."""
    import oracle
    import synth
    from threadpoolctl import threadpool_info, threadpool_limits
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from helpers import oracle_inputs
    L = synth.make_layer(name, "cuda")

    def one(i):
        # fresh inputs, so that no dequantised expert is kept from a previous call
        x, Wr, b, cfg, routed, shared = oracle_inputs(L, lazy=True)
        t0 = time.perf_counter()
        oracle.layer(x, Wr, b, cfg, routed, shared, token_idx=np.array([i % L.T]))
        return time.perf_counter() - t0

    times = []
    while sum(times) < budget_s and len(times) < max_calls:
        times.append(one(len(times)))
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    with threadpool_limits(limits=1):
        t1 = one(0)
    n, dt = len(times), sum(times)
    return dict(value=n / dt, unit="tokens/s", cores=int(threads), kind="oracle",
                value_1thread=1.0 / t1,
                sample=f"{n} single-token calls on the {name} workload (fp64 route + "
                       f"{L.geom['top_k']} routed + shared expert FFNs incl. dequant), {dt:.1f} s; "
                       f"one call on 1 thread: {t1:.1f} s")


def copy_calibration():
    """Kernels of known traffic whose FETCH_SIZE / WRITE_SIZE readings scale the
    layer kernels' counters (libqmoe_calib.so): whole-line reads of 1 GiB,
    GEMM-shaped half-line reads (16 rows x 64 bytes per instruction) of
    349525 rows x 3072 bytes, whole-line writes of 1 GiB; five launches each."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "quantized_moe_02_amd", "libqmoe_calib.so"))
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.qmoe_calib_read_lines.argtypes = [vp, sz, vp, vp]
    lib.qmoe_calib_read_halflines.argtypes = [vp, sz, ctypes.c_uint32, vp, vp]
    lib.qmoe_calib_write_lines.argtypes = [vp, sz, vp]
    n = 1 << 30
    buf = torch.empty(n, dtype=torch.uint8, device="cuda")
    buf.random_(0, 256)
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rows, row_bytes = 349525, 3072
    for _ in range(5):
        assert lib.qmoe_calib_read_lines(buf.data_ptr(), n, sink.data_ptr(), st) == 0
    for _ in range(5):
        assert lib.qmoe_calib_read_halflines(buf.data_ptr(), rows, row_bytes, sink.data_ptr(), st) == 0
    for _ in range(5):
        assert lib.qmoe_calib_write_lines(buf.data_ptr(), n, st) == 0
    torch.cuda.synchronize()
    print(json.dumps(dict(read_lines_kernel=n, read_halflines_kernel=rows * row_bytes,
                          write_lines_kernel=n, launches=5)))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the path has no multi-GPU mode); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return
    names = [w for w in args.workloads.split(",") if w]
    results = {}
    for name in names:
        results[name] = (run_stream_workload if name in STREAM_WORKLOADS else run_workload)(name, args)
        print(f"# {name}: {results[name]['tokens_per_s']:.1f} tok/s "
              f"{results[name]['ms_per_step']:.4f} ms/step", file=sys.stderr, flush=True)
    plain = [n for n in names if n not in STREAM_WORKLOADS]
    head = HEADLINE if HEADLINE in results else (plain[0] if plain else names[0])
    h = results[head]
    import synth
    base = head if head in synth.WORKLOADS else "decode"      # the streamed layer is the decode one
    geom = synth.WORKLOADS[base]["geom"]
    line = {
        "metric": METRIC, "value": h["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": h["steps"], "warmup": h["warmup"], "ms_per_step": h["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"int4": "int4*bf16->f32", "nvfp4": "fp4*bf16->f32"}.get(
            synth.WORKLOADS[base]["wfmt"], synth.WORKLOADS[base]["wfmt"] + "*bf16->f32"),
        "data": "synthetic",
        "config": {"workload": head, "tokens": h["tokens"], "hidden": geom["hidden"],
                   "moe_inter": geom["moe_inter"], "experts": geom["n_routed_experts"],
                   "top_k": geom["top_k"], "n_group": geom["n_group"],
                   "topk_group": geom["topk_group"], "shared_inter": geom["shared_inter"],
                   "weights": synth.WORKLOADS[base]["wfmt"], "replicas": h.get("replicas")},
        "roofline": h.get("roofline"),
        "hbm_gbs": h.get("hbm_gbs"), "hbm_pct_peak": h.get("hbm_pct_peak"), "tflops": h.get("tflops"),
        "workloads": results,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(head)
    out = json.dumps(line)
    print(out, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(out + "\n")


if __name__ == "__main__":
    main()
