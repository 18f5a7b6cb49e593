#!/usr/bin/env python3
"""Throughput of the chunkwise delta-rule forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--no-others]

One step = one full forward pass (one delta_fwd call: the intra-chunk kernel, then the segment
summary, combine and output launches of the inter-chunk pass) over one batch of synthetic inputs
already resident in HBM.  W untimed warm-up steps, then K timed steps bracketed by device
synchronisation; `value` and `ms_per_step` come from them.  The same K steps are then run as
their four launches with HIP events between them (per-kernel durations: `kernels_ms`, the
roofline), replayed K times from a HIP graph of one step (`graph`), and called K times singly
between event pairs, warm and with the Infinity Cache flushed before each call
(`median_call_ms`).  Prints ONE JSON line on stdout; progress goes to stderr.

Default workload: Gated DeltaNet, B=2, H=16, L=8192, d_k=d_v=128, bf16 inputs, fp32 state,
chunk 64 (the H=16, d=128, L=8K shape the tokens/s metric is quoted on).  tokens = B * L.

The line carries:
  roofline      for the dominant (longest) launch: the forward pass's compulsory HBM bytes (q, k,
                v, O in the input dtype, beta and log g in fp32, S0 and S_final in fp32: 1032 B per
                token-head at d = 128 bf16) over that launch's mean duration (HIP events on the
                launch stream), against 8 TB/s.  `launch_bytes` is what that launch itself must
                move, `traffic` its HBM bytes from the committed rocprofv3 counters, and
                `traffic_step` / `traffic_ratio` the counter bytes of all four launches and their
                ratio to the compulsory bytes.
  step          the same compulsory bytes and the algorithmic flops (causal counts; `dense_flops`
                with full C x C tiles) over ms_per_step: % of HBM, % of bf16 MFMA peak, and the
                roofline fraction achieved FLOP/s / min(MFMA peak, 8 TB/s x intensity)
  cpu_baseline  the fp64 oracle on the host cores, on a bounded sample of the same workload
  others        the other workloads (DeltaNet 4x8x2K, DeltaProduct n_h=2, GDN 64K, and the
                batch-64 decode step), measured the same way, each with its own oracle baseline,
                unless --no-others
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA
MFMA_F32_PEAK_TFLOPS = 157.3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ algorithmic work per launch
#
# One prefill step is four launches: intra (T, A, gate prefix per chunk), summary (per segment:
# the state run from zero and the d_k x d_k transition), combine (segment start states) and
# outputs.  Bytes count every tensor a launch must read or write once; flops count the products
# the method computes (causal / triangular counts).


def _es(w):
    return 2 if w.dtype == "bf16" else 4


def _segments(w):
    import chunkwise_delta_rule_chunked_amd as D
    return D.segments(w.B, w.L, w.H, w.dk, w.dv, w.n_h, w.chunk, D.BF16 if w.dtype == "bf16" else D.F32)


def intra_bytes(w) -> int:
    """Reads k, beta, log g; writes T (input dtype) and the gate prefix."""
    es = _es(w)
    NT = -(-w.Lx // w.chunk)
    b = w.B * w.Lx * w.H * (w.dk * es + 4)
    if w.gate:
        b += w.B * w.L * w.H * 4
    b += w.B * w.H * NT * w.chunk * (w.chunk * es + 4)
    return b


def intra_flops(w) -> int:
    """Strictly-lower Gram and the triangular inverse."""
    C, dk = w.chunk, w.dk
    NT = -(-w.Lx // C)
    return w.B * w.H * NT * (C * (C - 1) * dk + C ** 3 // 3)


def _chain_flops(w, cols) -> int:
    """One chunk of the state chain on `cols` state columns: K S, T Y, K^T (D V~)."""
    C, dk = w.chunk, w.dk
    return 2 * C * dk * cols + C * (C + 1) * cols + 2 * C * dk * cols


def summary_bytes(w) -> int:
    """Segments 0..P-2: reads k, v, T, gate prefix, S0; writes each segment's summary."""
    P, NS = _segments(w)
    if P <= 1:
        return 0
    es = _es(w)
    nch = min(-(-w.Lx // w.chunk), (P - 1) * NS)
    pos = min(w.Lx, nch * w.chunk)
    b = w.B * pos * w.H * (w.dk + w.dv) * es + w.B * w.H * nch * w.chunk * (w.chunk * es + 4)
    # S0 read for segment 0 (and once more for its copy), segment 0's start state written
    b += w.B * w.H * w.dk * w.dv * 4 * (3 if w.s0 is not None else 1)
    # S_loc (fp32) of segments 0..P-2, M (element type) of segments 1..P-2
    b += w.B * w.H * ((P - 1) * w.dk * w.dv * 4 + (P - 2) * w.dk * w.dk * es)
    return b


def summary_flops(w) -> int:
    P, NS = _segments(w)
    if P <= 1:
        return 0
    NT = -(-w.Lx // w.chunk)
    seg0 = min(NS, NT)
    rest = min(NT, (P - 1) * NS) - seg0
    return w.B * w.H * (seg0 * _chain_flops(w, w.dv) + rest * _chain_flops(w, w.dv + w.dk))


def combine_bytes(w) -> int:
    """Reads S_loc of segments 0..P-2 and M of 1..P-2; writes the start states of 1..P-1."""
    P, _ = _segments(w)
    if P <= 1:
        return 0
    return w.B * w.H * ((P - 1) * w.dk * w.dv * 4 + (P - 2) * w.dk * w.dk * _es(w) + (P - 1) * w.dk * w.dv * 4)


def combine_flops(w) -> int:
    P, _ = _segments(w)
    return w.B * w.H * max(0, P - 2) * 2 * w.dk * w.dk * w.dv


def outputs_bytes(w) -> int:
    """Reads q, k, v, T, gate prefix and the segments' start states (S0 itself when the sequence
    is not split); writes O, S_final."""
    es = _es(w)
    P, _ = _segments(w)
    NT = -(-w.Lx // w.chunk)
    b = w.B * w.L * w.H * (w.dk + w.dv) * es           # q, O
    b += w.B * w.Lx * w.H * (w.dk + w.dv) * es         # k, v
    b += w.B * w.H * NT * w.chunk * (w.chunk * es + 4)  # T, gate prefix
    b += w.B * w.H * w.dk * w.dv * 4                    # S_final
    if P > 1:
        b += w.B * w.H * P * w.dk * w.dv * 4            # start states
    elif w.s0 is not None:
        b += w.B * w.H * w.dk * w.dv * 4                # S0
    return b


def outputs_flops(w) -> int:
    C, dk, dv, nh = w.chunk, w.dk, w.dv, w.n_h
    QR = C // nh
    reach = sum(t * nh + nh for t in range(QR))   # positions each token row reads
    # chain, Q S, A V~ and the causal Q K^T itself
    per_chunk = _chain_flops(w, dv) + 2 * QR * dk * dv + 2 * reach * dv + 2 * reach * dk
    return w.B * w.H * (-(-w.Lx // C)) * per_chunk


KERNELS = {  # phase -> (kernel symbol substring, bytes, flops)
    "intra": ("intra_chunk_kernel", intra_bytes, intra_flops),
    "summary": ("summary_kernel", summary_bytes, summary_flops),
    "combine": ("combine_kernel", combine_bytes, combine_flops),
    "outputs": ("seg_kernel", outputs_bytes, outputs_flops),
}


def decode_bytes(w, kda=False) -> int:
    """State read and written once, q, k, v, O, beta, and the gate (a float per head, or per key
    channel for KDA)."""
    es = 2 if w.dtype == "bf16" else 4
    BH = w.B * w.H
    gate = w.dk * 4 if kda else (4 if w.gate else 0)
    return BH * (2 * w.dk * w.dv * 4 + (w.dk + w.n_h * (w.dk + w.dv) + w.dv) * es + w.n_h * 4 + gate)


# ------------------------------------------------------------------ timing

def time_prefill(w, steps, warmup, copy_calibration_mib=0):
    import torch
    import chunkwise_delta_rule_chunked_amd as D
    import workloads as W
    log("[bench] generating %s" % (w,))
    inp = W.make_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def dev(x, d):
        return None if x is None else torch.from_numpy(x).to(d).cuda()

    q, k, v = dev(inp["q"], dt), dev(inp["k"], dt), dev(inp["v"], dt)
    beta, g, S0 = dev(inp["beta"], torch.float32), dev(inp["g_log"], torch.float32), dev(inp["S0"], torch.float32)
    del inp
    O = torch.empty((w.B, w.L, w.H, w.dv), dtype=dt, device="cuda")
    SF = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    code = D.BF16 if w.dtype == "bf16" else D.F32
    nbytes = D.workspace_bytes(w.B, w.L, w.H, w.dk, w.dv, w.n_h, w.chunk, code)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    if copy_calibration_mib:
        # the library's streaming copy (delta_measure_copy) over a known size, for scaling the HBM
        # byte counters of a profile run
        src = torch.ones(copy_calibration_mib << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        D.measure_copy(src, dst, unroll=4, blocks=4096)
        torch.cuda.synchronize()
        del src, dst
    # the calls of one step, in order, each timed by its own event pair on the launch stream
    calls = [
        ("intra", lambda: D.fwd_intra(k, beta, g, ws, n_h=w.n_h, chunk=w.chunk, dv=w.dv)),
        ("summary", lambda: D.scan_summary(k, v, S0, ws, n_h=w.n_h, chunk=w.chunk)),
        ("combine", lambda: D.scan_combine(ws, B=w.B, L=w.L, H=w.H, dk=w.dk, dv=w.dv, n_h=w.n_h, chunk=w.chunk,
                                           dtype=code)),
        ("outputs", lambda: D.scan_outputs(q, k, v, S0, ws, n_h=w.n_h, chunk=w.chunk, O=O, S_final=SF)),
    ]
    def step():  # one forward pass as a caller runs it: one delta_fwd call
        D.fwd(q, k, v, beta, g, S0, n_h=w.n_h, chunk=w.chunk, O=O, S_final=SF, workspace=ws)

    for _ in range(warmup):
        step()
        for _, c in calls:
            c()
    torch.cuda.synchronize()
    # timed region 1: whole steps back to back (the throughput reported as `value`)
    t0 = time.perf_counter()
    for i in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # timed region 2: the same steps as their four launches, each bracketed by events on the
    # launch stream (the per-kernel durations of the roofline; the events add their own gaps)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record()
        for j, (_, c) in enumerate(calls):
            c()
            ev[i][j + 1].record()
    torch.cuda.synchronize()
    wall_ev = time.perf_counter() - t1
    ms = {name: sum(e[j].elapsed_time(e[j + 1]) for e in ev) / steps for j, (name, _) in enumerate(calls)}
    # timed region 3: one step captured as a HIP graph and replayed (launch gaps removed)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(2):
        graph.replay()
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for i in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    wall_g = time.perf_counter() - t2
    # single calls, each bracketed by an event pair: warm (back to back) and cold (a 512 MiB
    # scratch buffer written between calls, outside the pair, so no input or workspace byte is
    # left in the 256 MB Infinity Cache); medians
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    single = {"warm": [], "cold": []}
    for mode in ("warm", "cold"):
        for i in range(steps):
            if mode == "cold":
                scratch.fill_(i & 255)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            step()
            e1.record()
            single[mode].append((e0, e1))
        torch.cuda.synchronize()
    del scratch
    med = {mode: sorted(a.elapsed_time(b) for a, b in pairs)[len(pairs) // 2] for mode, pairs in single.items()}
    return {"wall_s": wall, "ms_per_step": wall * 1e3 / steps, "kernel_ms": ms,
            "tokens_per_s": w.B * w.L * steps / wall, "ms_per_step_with_events": wall_ev * 1e3 / steps,
            "graph_ms_per_step": wall_g * 1e3 / steps, "graph_tokens_per_s": w.B * w.L * steps / wall_g,
            "median_call_ms": med}


FORWARD_SOURCES = ("chunk_scan.hip", "common.h", "intra_chunk.hip", "kernels.h", "scan_summary.hip")


def kernel_sources_sha():
    """Hash of the sources the forward step's kernels are built from, recorded with measured
    traffic so that a stale figure is dropped."""
    import hashlib
    h = hashlib.sha256()
    src = os.path.join(ROOT, "chunkwise_delta_rule_chunked_amd", "csrc")
    for f in FORWARD_SOURCES:
        with open(os.path.join(src, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(w, phase):
    """HBM bytes per launch of `phase` from the committed rocprofv3 counter summary of this
    workload (FETCH_SIZE + WRITE_SIZE, scaled by the copy calibration), or None when there is
    none or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_%s.md" % w.name)
    if not os.path.exists(path):
        return None
    sha, val = None, None
    with open(path) as fh:
        for line in fh:
            parts = line.split()
            if len(parts) >= 2 and parts[0] == "sources:":
                sha = parts[1]
            if len(parts) >= 3 and parts[0] == "traffic:" and parts[1] == phase:
                val = int(parts[2])
    return val if sha == kernel_sources_sha() else None


def compulsory_bytes(w) -> int:
    """HBM bytes one forward pass cannot avoid: q, k, v and O in the input dtype, beta and log g
    in fp32, S0 (when given) and S_final in fp32, each touched once (1032 B per token-head at
    d = 128, bf16, with S0)."""
    es = _es(w)
    b = w.B * w.L * w.H * (w.dk + w.dv) * es + w.B * w.Lx * w.H * ((w.dk + w.dv) * es + 4)
    if w.gate:
        b += w.B * w.L * w.H * 4
    b += w.B * w.H * w.dk * w.dv * 4 * (2 if w.s0 is not None else 1)
    return b


def method_flops(w, dense=False) -> float:
    """Flops of the chunkwise method: per expanded position 4 d_k d_v (W S and K^T V~),
    C (2 d_k + d_v) (K K^T, W = T K, U = T V, causal halves) and C^2 / 3 (the triangular solve); per
    output 2 d_k d_v (Q S) and C (d_k + d_v) (the causal Q K^T and its product with V~).  dense:
    the C-terms over full C x C tiles (twice the causal count)."""
    C, dk, dv = w.chunk, w.dk, w.dv
    m = 2 if dense else 1
    npos, nout = w.B * w.H * w.Lx, w.B * w.H * w.L
    return npos * (4 * dk * dv + m * C * (2 * dk + dv) + C * C / 3) + nout * (2 * dk * dv + m * C * (dk + dv))


def _mfma_peak(w):
    return (MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS) * 1e12


def roofline_of(w, r):
    """Roofline record of the dominant (longest) launch of one forward pass: the pass's
    compulsory bytes over that launch's mean duration."""
    phase = max(r["kernel_ms"], key=r["kernel_ms"].get)
    ms = r["kernel_ms"][phase]
    nb = compulsory_bytes(w)
    gbs = nb / (ms * 1e-3) / 1e9
    traffic = {ph: measured_traffic(w, ph) for ph in KERNELS}
    step_traffic = sum(traffic.values()) if all(v is not None for v in traffic.values()) else None
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic[phase],
            "kernel": phase, "kernel_ms": round(ms, 5), "bytes_per_launch": nb,
            "launch_bytes": KERNELS[phase][1](w), "traffic_step": step_traffic,
            "traffic_ratio": None if step_traffic is None else round(step_traffic / nb, 3)}


def step_roofline(w, ms_per_step):
    """The whole forward pass against the roofline: compulsory bytes and method flops over the
    measured time per step."""
    t = ms_per_step * 1e-3
    nb, F, Fd = compulsory_bytes(w), method_flops(w), method_flops(w, dense=True)
    peak = _mfma_peak(w)
    I = F / nb
    ceiling = min(peak, HBM_PEAK_GBS * 1e9 * I)
    return {"ms": round(ms_per_step, 5), "compulsory_bytes": nb, "alg_flops": round(F), "dense_flops": round(Fd),
            "intensity_flop_per_B": round(I, 1), "bound": "hbm" if ceiling < peak else "mfma",
            "hbm_GBs": round(nb / t / 1e9, 1), "hbm_frac": round(nb / t / (HBM_PEAK_GBS * 1e9), 4),
            "mfma_frac_alg": round(F / t / peak, 4), "mfma_frac_dense": round(Fd / t / peak, 4),
            "roofline_frac": round(F / t / ceiling, 4), "floor_us": round(nb / (HBM_PEAK_GBS * 1e9) * 1e6, 2)}


def backward_flops(w) -> float:
    """Flops of the chunkwise backward as the kernels evaluate it, causal halves counted once:
    per expanded position 16 d_k d_v (the two state chains re-run: K S, K^T V~, K G', K^T dY; the
    per-chunk products K S, K G', dY S^T, V~ G'^T), C (6 d_v + 5 d_k) (T Y, T^T dV~, P^T dO,
    dV~ Y^T, dO V~^T, K K^T, Q K^T, E1 K, E1^T Q, Gs K, each over the causal half) and C^2 (the
    two C x C x C products of the chunk-local algebra, triangular); per output 4 d_k d_v (Q^T dO
    in the adjoint chain, dO S^T) and C (d_k + d_v)."""
    C, dk, dv = w.chunk, w.dk, w.dv
    npos, nout = w.B * w.H * w.Lx, w.B * w.H * w.L
    return npos * (16 * dk * dv + C * (6 * dv + 5 * dk) + C * C) + nout * (4 * dk * dv + C * (dk + dv))


def time_backward(w, steps, warmup=2):
    """delta_bwd on the prefill workload with its seeded cotangents (dO, dS_final): `steps`
    back-to-back calls with preallocated gradients and workspace, timed with HIP events."""
    import torch
    import chunkwise_delta_rule_chunked_amd as D
    import workloads as W
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    inp, cot = W.make_inputs(w), W.make_cotangents(w)
    dev = {kk: (None if vv is None else torch.from_numpy(vv).to(torch.float32 if kk in ("beta", "g_log", "S0")
                                                            else dt).cuda()) for kk, vv in inp.items()}
    dO = torch.from_numpy(cot["dO"]).to(dt).cuda()
    dS = torch.from_numpy(cot["dS_final"]).cuda()
    ws = torch.empty(D.bwd_workspace_bytes(w.B, w.L, w.H, w.dk, w.dv, w.n_h, w.chunk,
                                           D.BF16 if w.dtype == "bf16" else D.F32), dtype=torch.uint8, device="cuda")

    def run(grads=None):
        return D.bwd(dev["q"], dev["k"], dev["v"], dev["beta"], dev["g_log"], dev["S0"], dO, dS, n_h=w.n_h,
                     chunk=w.chunk, grads=grads, workspace=ws)

    grads = run()
    for _ in range(warmup):
        run(grads)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        run(grads)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    F = backward_flops(w)
    peak = _mfma_peak(w)
    return {"ms_per_step": round(ms, 4), "tokens_per_s": round(w.B * w.L / (ms * 1e-3), 1), "steps": steps,
            "workspace_mib": round(ws.numel() / 2**20, 1),
            "roofline": {"bound": "mfma", "achieved": round(F / (ms * 1e-3) / 1e12, 2), "peak": round(peak / 1e12, 1),
                         "unit": "TFLOP/s", "frac": round(F / (ms * 1e-3) / peak, 4), "flops": round(F)}}


KDA_WORKLOAD = "kda_b2h16_l8k"   # the Gated DeltaNet workload's shape and inputs, decays per key channel
F32_VALU_PEAK_TFLOPS = 157.3


def time_kda(steps, warmup=2):
    """KDA forward on the 32-head, 8K-token shape (the Gated DeltaNet workload's inputs, decays per
    key channel), `steps` back-to-back calls of each form timed with HIP events:
      - chunked (delta_fwd_kda_chunked): against HBM, its compulsory bytes (q, k, v, O, beta, the
        per-channel log decays, S0 and S_final once each) over the time per call;
      - recurrent (delta_fwd_kda, the token recurrence): bound by the fp32 vector ALU (a chain of L
        dependent steps of ~7 d_k d_v flops per sequence), against the fp32 vector peak."""
    import torch
    import chunkwise_delta_rule_chunked_amd as D
    import workloads as W
    w = W.CONFIGS["gdn_b2h16_l8k"].replace(name=KDA_WORKLOAD)
    inp = W.make_inputs(w)
    a = torch.from_numpy(W.make_kda_decays(w)).cuda()
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = lambda x, d: torch.from_numpy(x).to(d).cuda()
    q, k, v = dev(inp["q"], dt), dev(inp["k"], dt), dev(inp["v"], dt)
    beta, S0 = dev(inp["beta"], torch.float32), dev(inp["S0"], torch.float32)
    O = torch.empty((w.B, w.L, w.H, w.dv), dtype=dt, device="cuda")
    SF = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    ws = torch.empty(D.kda_chunked_workspace_bytes(w.B, w.L, w.H), dtype=torch.uint8, device="cuda")

    def timed(run):
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            run()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms_c = timed(lambda: D.fwd_kda_chunked(q, k, v, beta, a, S0, O=O, S_final=SF, workspace=ws))
    ms = timed(lambda: D.fwd_kda(q, k, v, beta, a, S0, O=O, S_final=SF))
    th = w.B * w.L * w.H
    flops = th * 7 * w.dk * w.dv
    nb = compulsory_bytes(w) - w.B * w.L * w.H * 4 + th * w.dk * 4   # a per-channel log decay in place of g
    tf = flops / (ms * 1e-3) / 1e12
    gbs = nb / (ms_c * 1e-3) / 1e9
    return {"ms_per_step": round(ms_c, 4), "tokens_per_s": round(w.B * w.L / (ms_c * 1e-3), 1), "steps": steps,
            "form": "chunked", "workspace_mib": round(ws.numel() / 2**20, 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "compulsory_bytes": nb},
            "recurrent": {"ms_per_step": round(ms, 4), "tokens_per_s": round(w.B * w.L / (ms * 1e-3), 1),
                          "roofline": {"bound": "alu", "achieved": round(tf, 2), "peak": F32_VALU_PEAK_TFLOPS,
                                       "unit": "TFLOP/s", "frac": round(tf / F32_VALU_PEAK_TFLOPS, 4), "flops": flops,
                                       "hbm_frac": round(nb / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4)}}}


def time_layer(w, steps, width=4):
    """delta_layer_prologue and delta_layer_epilogue on the workload's shapes (seeded inputs),
    `steps` calls each timed with HIP events; GB/s from the bytes each must move (inputs read
    once, outputs written once, filters and weights)."""
    import torch
    import chunkwise_delta_rule_chunked_amd as D
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    es = 2 if w.dtype == "bf16" else 4
    g = torch.Generator(device="cpu").manual_seed(2026)
    mk = lambda *shape: torch.randn(*shape, generator=g).to(dt).cuda()
    Lx = w.L * w.n_h
    xq, xk, xv = mk(w.B, w.L, w.H, w.dk), mk(w.B, Lx, w.H, w.dk), mk(w.B, Lx, w.H, w.dv)
    wq, wk, wv = (torch.randn(w.H * d, width, generator=g).cuda() for d in (w.dk, w.dk, w.dv))
    o, gate = mk(w.B, w.L, w.H, w.dv), mk(w.B, w.L, w.H, w.dv)
    nw = torch.ones(w.dv, device="cuda")
    q, k, v = D.layer_prologue(xq, xk, xv, wq, wk, wv, n_h=w.n_h)
    y = D.layer_epilogue(o, gate, nw)
    out = {}
    for name, fn, nbytes in (
            ("prologue", lambda: D.layer_prologue(xq, xk, xv, wq, wk, wv, n_h=w.n_h, q=q, k=k, v=v),
             2 * es * (w.B * w.L * w.H * w.dk + w.B * Lx * w.H * (w.dk + w.dv)) + 4 * width * w.H * (2 * w.dk + w.dv)),
            ("epilogue", lambda: D.layer_epilogue(o, gate, nw, y=y), 3 * es * w.B * w.L * w.H * w.dv + 4 * w.dv)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        gbs = nbytes / (us * 1e-6) / 1e9
        out[name] = {"us_per_call": round(us, 2), "bytes": nbytes, "GB_s": round(gbs, 1),
                     "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    return out


def time_decode(w, steps, n_states=8, kda=False):
    """`steps` back-to-back decode calls cycling over n_states independent states (8 x 64 MiB
    exceeds the 256 MB Infinity Cache, so each step streams its state from HBM); the same loop on
    one state (warm); the cold loop replayed from a HIP graph; and, as the practical ceiling of a
    step that reads and writes its state once, a plain device copy of the same volume.  kda: the
    KDA step (delta_decode_kda, a decay per key channel) instead."""
    import torch
    import chunkwise_delta_rule_chunked_amd as D
    import workloads as W
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    log("[bench] generating decode inputs %s" % (w,))
    S0 = torch.from_numpy(W.make_decode_state(w)).cuda()
    states = [S0.clone() for _ in range(n_states)]
    steps_in = []
    for t in range(steps):
        x = W.make_decode_inputs(w, t)
        steps_in.append({kk: (None if vv is None else torch.from_numpy(vv).to(torch.float32 if kk in ("beta", "g_log")
                                                                              else dt).cuda())
                         for kk, vv in x.items()})
        if kda:
            steps_in[-1]["a_log"] = torch.from_numpy(W.make_kda_decay(w, t)).cuda()
    O = torch.empty((w.B, 1, w.H, w.dv), dtype=dt, device="cuda")

    def run(i, S):
        x = steps_in[i]
        if kda:
            D.decode_kda(x["q"], x["k"], x["v"], x["beta"], x["a_log"], S, O=O)
        else:
            D.decode(x["q"], x["k"], x["v"], x["beta"], x["g_log"], S, n_h=w.n_h, O=O)

    for i in range(min(5, steps)):
        run(i, states[i % n_states])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        run(i, states[i % n_states])
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1)
    per_step_us = ms * 1e3 / steps
    gbs = decode_bytes(w, kda) / (per_step_us * 1e-6) / 1e9
    # the same loop on one state (warm: it stays in the Infinity Cache)
    e0.record()
    for i in range(steps):
        run(i, states[0])
    e1.record()
    torch.cuda.synchronize()
    warm_us = e0.elapsed_time(e1) * 1e3 / steps
    # the same cold loop captured once in a HIP graph and replayed (no per-launch host overhead)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            run(i, states[i % n_states])
    g.replay()
    torch.cuda.synchronize()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    graph_us = e0.elapsed_time(e1) * 1e3 / steps
    del g
    # reference: a plain device copy moving the same state volume (read once, written once),
    # cycling n_states buffers like the loop above
    nel = w.B * w.H * w.dk * w.dv
    src = [torch.empty(nel, dtype=torch.float32, device="cuda").fill_(1.0) for _ in range(n_states)]
    dst = [torch.empty_like(x) for x in src]
    for i in range(n_states):
        dst[i].copy_(src[i])
    torch.cuda.synchronize()
    e0.record()
    for i in range(steps):
        dst[i % n_states].copy_(src[i % n_states])
    e1.record()
    torch.cuda.synchronize()
    copy_us = e0.elapsed_time(e1) * 1e3 / steps
    del src, dst
    ceil = stream_ceiling(nel * 4, n_buf=n_states)
    return {"us_per_step": round(per_step_us, 3), "tokens_per_s": w.B * steps / (ms * 1e-3),
            "stream_ceiling": {k: v for k, v in ceil.items() if k != "sweep_us"},
            "frac_of_stream_ceiling": round(ceil["us"] / per_step_us, 4),
            "wall_tokens_per_s": w.B * steps / wall, "achieved_GBs": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "warm_us_per_step": round(warm_us, 3),
            "warm_GBs": round(decode_bytes(w, kda) / (warm_us * 1e-6) / 1e9, 1),
            "graph_us_per_step": round(graph_us, 3), "graph_tokens_per_s": round(w.B / (graph_us * 1e-6), 1),
            "state_copy_us": round(copy_us, 3),
            "state_copy_GBs": round(2 * nel * 4 / (copy_us * 1e-6) / 1e9, 1)}


def stream_ceiling(nbytes, n_buf=8, reps=32):
    """The best rate of the library's plain streaming copy (delta_measure_copy) reading nbytes and
    writing nbytes, cycling n_buf buffer pairs so that nothing stays in the 256 MB Infinity Cache,
    over a sweep of its launch shapes: the practical ceiling of a kernel that moves each byte once."""
    import torch
    import chunkwise_delta_rule_chunked_amd as D
    src = [torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0) for _ in range(n_buf)]
    dst = [torch.empty_like(x) for x in src]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best, sweep = None, {}
    for unroll in (1, 2, 4, 8):
        for blocks in (1024, 2048, 4096, 8192):
            for nt in (0, 1):
                for i in range(n_buf):
                    D.measure_copy(src[i], dst[i], unroll=unroll, blocks=blocks, nontemporal=nt)
                e0.record()
                for i in range(reps):
                    D.measure_copy(src[i % n_buf], dst[i % n_buf], unroll=unroll, blocks=blocks, nontemporal=nt)
                e1.record()
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / reps
                sweep["u%d_b%d_nt%d" % (unroll, blocks, nt)] = round(us, 2)
                if best is None or us < best[0]:
                    best = (us, unroll, blocks, nt)
    del src, dst
    us, unroll, blocks, nt = best
    gbs = 2 * nbytes / (us * 1e-6) / 1e9
    return {"us": round(us, 3), "bytes": 2 * nbytes, "GBs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "unroll": unroll, "blocks": blocks, "nontemporal": bool(nt), "sweep_us": sweep}


def cpu_baseline_decode(w, steps):
    """The fp64 oracle on the decode workload: every (b, h) runs its `steps` tokens as one
    sequence from the same start state (the decode step is the recurrence's token step)."""
    import numpy as np
    import oracle
    import workloads as W
    xs = [W.make_decode_inputs(w, t) for t in range(steps)]
    cat = lambda key: None if xs[0][key] is None else np.concatenate([x[key] for x in xs], axis=1)
    S0 = W.make_decode_state(w)
    args = [cat(k) for k in ("q", "k", "v", "beta", "g_log")]
    t0 = time.perf_counter()
    oracle.fwd(*args, S0, n_h=w.n_h)
    dt = time.perf_counter() - t0
    return {"value": round(w.B * steps / dt, 1), "unit": "tokens/s", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": "all %d (b,h) sequences x %d steps (whole workload), fp64, %.2f s" % (w.B * w.H, steps, dt)}


def cpu_baseline(w, budget_s=15.0):
    """The fp64 oracle as it stands, on the host cores, on a bounded sample of the workload: all
    (b, h) sequences over a prefix of the tokens, sized for about `budget_s` seconds."""
    import oracle
    import workloads as W
    probe_L = 128
    x = W.make_inputs(w.replace(L=probe_L))
    t0 = time.perf_counter()
    oracle.fwd(x["q"], x["k"], x["v"], x["beta"], x["g_log"], x["S0"], n_h=w.n_h)
    per_tok = (time.perf_counter() - t0) / probe_L
    Ls = int(min(w.L, max(probe_L, budget_s / max(per_tok, 1e-9))))
    x = W.make_inputs(w.replace(L=Ls))
    t0 = time.perf_counter()
    oracle.fwd(x["q"], x["k"], x["v"], x["beta"], x["g_log"], x["S0"], n_h=w.n_h)
    dt = time.perf_counter() - t0
    return {"value": round(w.B * Ls / dt, 1), "unit": "tokens/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": "all %d (b,h) sequences, first %d of %d tokens (%s), fp64, %.1f s" % (
                w.B * w.H, Ls, w.L, "whole workload" if Ls == w.L else "prefix", dt)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gdn_b2h16_l8k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true")
    ap.add_argument("--layer-only", action="store_true",
                    help="time only the layer prologue/epilogue on the workload's shapes")
    ap.add_argument("--backward-only", action="store_true",
                    help="time only delta_bwd on the workload (--steps calls) and print its line")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (for HBM counter scaling)")
    ap.add_argument("--kda-only", action="store_true",
                    help="time only the KDA forward (chunked and recurrent) on the 32-head 8K-token shape and print its line")
    ap.add_argument("--decode-only", action="store_true",
                    help="time only the batch-64 decode step (scalar gate, then KDA) and print its line")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the library runs on exactly one GPU (one (b, h) shard of the work); "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import chunkwise_delta_rule_chunked_amd as D
    import workloads as W
    D.load_library()
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)

    w = W.get(args.workload)
    if args.copy_calibration_mib and (args.kda_only or args.decode_only):
        # the counter runs' reference: the library's streaming copy of a known size
        src = torch.ones(args.copy_calibration_mib << 18, dtype=torch.float32, device="cuda")
        D.measure_copy(src, torch.empty_like(src), unroll=4, blocks=4096)
        torch.cuda.synchronize()
        del src
    if args.kda_only:
        print(json.dumps({"workload": KDA_WORKLOAD, "kda": time_kda(args.steps, args.warmup)}), flush=True)
        return
    if args.decode_only:
        dec = time_decode(W.DECODE, W.DECODE_STEPS)
        kd = time_decode(W.DECODE, W.DECODE_STEPS, kda=True)
        print(json.dumps({"workload": W.DECODE.name, "decode": dec, "kda_decode": kd}), flush=True)
        return
    if args.layer_only:
        print(json.dumps({"workload": w.name, "layer": time_layer(w, args.steps)}), flush=True)
        return
    if args.backward_only:
        bw = time_backward(w, args.steps, args.warmup)
        print(json.dumps({"workload": w.name, "backward": bw}), flush=True)
        return
    r = time_prefill(w, args.steps, args.warmup, args.copy_calibration_mib)
    log("[bench] %s: %.3f ms/step (%s), %.3e tokens/s" % (
        w.name, r["ms_per_step"], ", ".join("%s %.4f ms" % kv for kv in r["kernel_ms"].items()), r["tokens_per_s"]))
    line = {
        "metric": "tokens/s of chunkwise delta-rule fwd (H=16,d=128,L=8K) + % MFMA/HBM roofline",
        "value": round(r["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded generators shaped like the pages' models)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "L": w.L, "dk": w.dk, "dv": w.dv,
                   "n_h": w.n_h, "chunk": w.chunk, "gate": w.gate, "state": "fp32",
                   "global_batch": w.B, "seq_len": w.L, "parallelism": "single GPU"},
        "roofline": roofline_of(w, r),
        "step": step_roofline(w, r["ms_per_step"]),
        "kernels_ms": {k: round(v, 5) for k, v in r["kernel_ms"].items()},
        "ms_per_step_with_events": round(r["ms_per_step_with_events"], 5),
        "graph": {"ms_per_step": round(r["graph_ms_per_step"], 5), "tokens_per_s": round(r["graph_tokens_per_s"], 1)},
        "median_call_ms": {k: round(v, 5) for k, v in r["median_call_ms"].items()},
        "segments": list(_segments(w)),
    }
    if not args.no_others:
        others = {}
        for name in ("deltanet_b4h8_l2k", "gdp2_b2h16_l4k", "gdn_b1h16_l64k"):
            if name == w.name:
                continue
            try:
                wo = W.get(name)
                ro = time_prefill(wo, max(20, args.steps // 2), 3)
                others[name] = {"tokens_per_s": round(ro["tokens_per_s"], 1), "ms_per_step": round(ro["ms_per_step"], 5),
                                "graph_tokens_per_s": round(ro["graph_tokens_per_s"], 1),
                                "median_call_ms": {k: round(v, 5) for k, v in ro["median_call_ms"].items()},
                                "kernels_ms": {k: round(v, 5) for k, v in ro["kernel_ms"].items()},
                                "roofline": roofline_of(wo, ro), "step": step_roofline(wo, ro["ms_per_step"])}
                if wo.n_h > 1:  # DeltaProduct: expanded positions (L * n_h per sequence) per second
                    others[name]["positions_per_s"] = round(ro["tokens_per_s"] * wo.n_h, 1)
                if not args.no_cpu_baseline:
                    others[name]["cpu_baseline"] = cpu_baseline(wo, budget_s=5.0)
                log("[bench] %s: %.3f ms/step, %.3e tokens/s" % (name, ro["ms_per_step"], ro["tokens_per_s"]))
            except Exception as e:  # an auxiliary line must not hide the main one
                others[name] = {"error": repr(e)}
        try:
            dec = time_decode(W.DECODE, W.DECODE_STEPS)
            if not args.no_cpu_baseline:
                dec["cpu_baseline"] = cpu_baseline_decode(W.DECODE, W.DECODE_STEPS)
            others[W.DECODE.name] = dec
            log("[bench] decode: %s" % dec)
            kd = time_decode(W.DECODE, W.DECODE_STEPS, kda=True)
            others["kda_" + W.DECODE.name] = kd
            log("[bench] kda decode: %s" % kd)
        except Exception as e:
            others[W.DECODE.name] = {"error": repr(e)}
        try:
            kd = time_kda(max(5, args.steps // 10))
            others[KDA_WORKLOAD] = kd
            log("[bench] kda prefill: %s" % kd)
        except Exception as e:
            others[KDA_WORKLOAD] = {"error": repr(e)}
        try:
            ly = time_layer(w, max(20, args.steps))
            others["layer_" + w.name] = ly
            log("[bench] layer steps %s: %s" % (w.name, ly))
        except Exception as e:
            others["layer_" + w.name] = {"error": repr(e)}
        try:
            bw = time_backward(w, max(5, args.steps // 10))
            others["bwd_" + w.name] = bw
            log("[bench] backward %s: %s" % (w.name, bw))
        except Exception as e:
            others["bwd_" + w.name] = {"error": repr(e)}
        line["others"] = others
    line["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
