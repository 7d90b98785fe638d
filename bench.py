#!/usr/bin/env python3
"""Attention forward+backward throughput on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic input:
fa_fwd (O and logsumexp) followed by fa_bwd (dQ, dK, dV) on the training
shape B=4, H=16, N=4096, d=128, causal, bf16, with iid N(0,1) inputs drawn
from a fixed seed and already resident in device memory when timing starts.

FLOP convention: forward 4*B*H*N^2*d, halved for causal; backward 2.5x the
forward (five N x N x d products: the recomputed scores, dP, dV, dK, dQ).

Printed: one JSON line with the whole-step TFLOP/s, the roofline of the
dominant launch (the backward call) and of the forward kernel, both timed with
HIP events on the stream the kernels run on, and the fp64 CPU oracle timed on
a bounded sample of the same workload as a reported baseline.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # 256 CUs x 4096 dense bf16 flop/clk/CU x 2.4 GHz
PEAK_FP8_TFLOPS = 5033.2   # dense fp8 MFMA: twice the bf16 rate
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "train_causal_traffic.json")


# Sources of the kernels the stored traffic describes (the forward and
# backward calls of the training step and their launch path).
TRAFFIC_SOURCES = ("fa_api.hip", "fa_bwd.hip", "fa_common.hpp", "fa_fwd.hip", "fa_launch.hpp", "fa_merge.hip")


def kernel_source_hash() -> str:
    """SHA-256 of the sources of the measured kernels; a stored traffic
    measurement is only reported while they are unchanged."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "exact_tiled_attention_37_amd", "csrc")
    for path in (os.path.join(csrc, name) for name in TRAFFIC_SOURCES):
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def stored_traffic(workload: str):
    """HBM bytes per launch measured by rocprofv3 (FETCH_SIZE / WRITE_SIZE,
    calibrated against a plain copy), or None if absent or stale."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != kernel_source_hash() or t.get("workload") != workload:
        return None
    return t


def fwd_flops(w) -> float:
    f = 4.0 * w.B * w.H * w.N * w.N * w.d
    return f / 2 if w.causal else f


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    # Defaults: about 0.1 s of untimed steps, so that the GPU's clock has
    # left the state the host-side input generation leaves it in, then
    # about 0.13 s of timed steps.
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=80)
    ap.add_argument("--workload", default="train_causal")
    ap.add_argument("--cpu-heads", type=int, default=16,
                    help="(batch, head) pairs of the workload whose forward+backward the CPU oracle "
                         "baseline runs (0 = skip the CPU baseline; each workload's forward is also "
                         "timed on a few pairs: about 20 s in all on 16 threads)")
    ap.add_argument("--no-sweep", action="store_true", help="skip the forward sweep over the other workloads")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-shaped calls")
    ap.add_argument("--no-bias", action="store_true", help="skip the additive-bias calls")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8 forward calls (per-head and microscaled)")
    ap.add_argument("--no-ring", action="store_true",
                    help="skip the key-chunk leg (one rank's share of the 16384-token sequence over 8 ranks)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (3 times) so that profiler byte "
                         "counters can be scaled against a transfer of known size")
    return ap.parse_args()


def time_calls(fn, n, stream):
    """Average duration (s) of fn() over n calls, HIP events on `stream`."""
    import torch

    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(n):
        fn()
    stop.record(stream)
    stop.synchronize()
    return start.elapsed_time(stop) / 1e3 / n


def time_each(fn, n, stream):
    """Durations (s) of n calls of fn(), each between its own pair of HIP
    events on `stream` (recorded back to back). Returns them sorted."""
    import torch

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    ev[-1][1].synchronize()
    return sorted(a.elapsed_time(b) / 1e3 for a, b in ev)


def cpu_info():
    """The host CPU: model name, physical cores, logical CPUs and the CPUs
    this process may run on."""
    model, cores = None, set()
    try:
        phys = core = None
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                key, _, val = line.partition(":")
                key, val = key.strip(), val.strip()
                if key == "model name" and model is None:
                    model = val
                elif key == "physical id":
                    phys = val
                elif key == "core id":
                    core = val
                elif not key and phys is not None:
                    cores.add((phys, core))
                    phys = core = None
            if phys is not None:
                cores.add((phys, core))
    except OSError:
        pass
    return {"model": model, "physical_cores": len(cores) or None, "logical_cpus": os.cpu_count(),
            "cpus_available": len(os.sched_getaffinity(0))}


def settle(fn, stream, seconds=0.1, max_calls=2000):
    """Untimed calls of fn() for about `seconds` of GPU time before a leg is
    timed. The leg's inputs are drawn on the host just before, which leaves
    the GPU idle long enough for its clock to drop; a few calls do not bring
    it back (the same kernels then time 10-15% slower than in the step loop)."""
    t = time_calls(fn, 3, stream)
    n = min(max_calls, int(seconds / max(t, 1e-6)))
    if n > 0:
        time_calls(fn, n, stream)


def settle_calls(flops, seconds=0.1, max_calls=2000):
    """A fixed number of untimed calls worth about `seconds` at 1 PFLOP/s (the
    sweep and FP8 legs use it instead of `settle`, so that their dispatches
    can be told apart by count in a profiler trace)."""
    return max(3, min(max_calls, int(seconds / (flops / 1e15))))


def cold_call_roofline(fn, wl, reps, stream):
    """Average duration of fn() with the caches flushed before each call
    (a 512 MiB fill between calls, outside the events), against HBM bandwidth:
    algorithmic bytes = Q, K, V read + O written (bf16) + logsumexp (fp32)."""
    import torch

    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    total = 0.0
    for i in range(reps):
        flush.fill_(i & 0xFF)
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        fn()
        stop.record(stream)
        stop.synchronize()
        total += start.elapsed_time(stop) / 1e3
    del flush
    s = total / reps
    nbytes = 4 * wl.B * wl.N * wl.H * wl.d * 2 + wl.B * wl.H * wl.N * 4
    return {"fwd_ms": round(s * 1e3, 4), "fwd_tflops": round(fwd_flops(wl) / s / 1e12, 2),
            "roofline": {"bound": "hbm", "achieved": round(nbytes / s / 1e9, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(nbytes / s / 1e9 / PEAK_HBM_GBS, 4),
                         "bytes_per_launch": nbytes}}


RING_RANKS = 8


def ring_rank_leg(fa, si, torch, dev, stream):
    """One rank's share of the 16384-token causal workload split over 8
    ranks (rank 7, the busiest): its 2048 query rows attend to the 2048-key
    chunks 0..7 with their global positions (fa_fwd_chunk, written straight
    into the stacked chunk buffer), then fa_merge combines the 8 results.
    FLOPs count 4*B*H*n^2*d per chunk, halved for the diagonal one; the merge
    is priced by its algorithmic bytes against HBM bandwidth."""
    w = si.WORKLOADS["long_causal"]
    n = w.N // RING_RANKS
    r = RING_RANKS - 1
    C = r + 1
    b = si.draw_workload(w)
    q, k, v = (si.bits_to_torch(b[t], dev) for t in ("q", "k", "v"))
    qc = q[:, r * n:(r + 1) * n].contiguous()
    kcs = [k[:, c * n:(c + 1) * n].contiguous() for c in range(C)]
    vcs = [v[:, c * n:(c + 1) * n].contiguous() for c in range(C)]
    del q, k, v
    o_parts = torch.empty((C, w.B, n, w.H, w.d), dtype=torch.float32, device=dev)
    l_parts = torch.empty((C, w.B, w.H, n), dtype=torch.float32, device=dev)
    o = torch.empty((w.B, n, w.H, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.H, n), dtype=torch.float32, device=dev)

    def chunks():
        for c in range(C):
            fa.fa_fwd_chunk(qc, kcs[c], vcs[c], True, r * n, c * n, w.scale, out=o_parts[c], lse=l_parts[c])

    def merge():
        fa.fa_merge(o_parts, l_parts, out=o, lse=lse)

    settle(chunks, stream)
    settle(merge, stream)
    t_chunks = time_calls(chunks, 10, stream)
    t_merge = time_calls(merge, 20, stream)
    flops = 4.0 * w.B * w.H * n * n * w.d * (C - 0.5)
    rows = w.B * n * w.H
    mbytes = C * rows * (w.d * 4 + 4) + rows * (w.d * 2 + 4)
    tf = flops / t_chunks / 1e12
    gbs = mbytes / t_merge / 1e9
    return {
        "config": f"rank {r} of {RING_RANKS}: B={w.B} H={w.H} d={w.d}, {n} query rows at position {r * n}, "
                  f"{C} causal key chunks of {n}",
        "chunks_ms": round(t_chunks * 1e3, 4), "chunks_tflops": round(tf, 2),
        "chunks_frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
        "merge_ms": round(t_merge * 1e3, 4),
        "merge_roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes_per_launch": int(mbytes)},
        "total_ms": round((t_chunks + t_merge) * 1e3, 4),
    }


def decode_leg(fa, si, torch, dev, stream):
    """Decode-shaped calls (a few query rows against a long key history):
    bound by streaming K and V from memory, so each is priced by its
    algorithmic bytes (K, V, Q read; O and logsumexp written) against HBM
    bandwidth; TFLOP/s (4*B*H*Nq*Nk*d) is reported beside it."""
    out = {}
    for name, w in si.DECODE_WORKLOADS.items():
        b = si.draw_decode(w)
        q, k, v = (si.bits_to_torch(b[t], dev) for t in ("q", "k", "v"))
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
        need = fa.fa_decode_workspace_bytes(w.B, w.Nq, w.Nk, w.H, w.d)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        call = lambda: fa.fa_decode(q, k, v, w.causal, w.scale, out=o, lse=lse, workspace=ws)
        settle(call, stream)
        t = time_calls(call, 50, stream)
        kv = 2 * w.B * w.Nk * w.H * w.d * 2
        byts = kv + 2 * (w.B * w.Nq * w.H * w.d * 2) + w.B * w.H * w.Nq * 4
        gbs = byts / t / 1e9
        out[name] = {"B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d, "causal": w.causal,
                     "ms": round(t * 1e3, 4),
                     "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                  "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes_per_launch": int(byts)},
                     "tflops": round(4.0 * w.B * w.H * w.Nq * w.Nk * w.d / t / 1e12, 2),
                     "workspace_bytes": int(need)}
        del q, k, v, o, lse, ws
    return out


def bias_leg(fa, si, torch, dev, stream):
    """Attention with an additive bias (a dense bf16 [B, H, N, N] matrix) on
    the bias workload: forward and backward (with dBias), each priced both
    by FLOPs against the MFMA peak and by algorithmic bytes against HBM (the
    bias makes the traffic quadratic in N)."""
    out = {}
    for name, w in si.BIAS_WORKLOADS.items():
        b = si.draw_with_bias(w.B, w.N, w.H, w.d, w.seed)
        q, k, v, do = (si.bits_to_torch(b[t], dev) for t in ("q", "k", "v", "do"))
        bias = fa.padded_bias(w.B, w.H, w.N, dev)
        bias.copy_(si.bits_to_torch(b["bias"], dev))
        del b
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        dbias = fa.padded_bias(w.B, w.H, w.N, dev)
        ws = torch.empty(fa.fa_bwd_workspace_bytes(w.B, w.N, w.H, w.d), dtype=torch.uint8, device=dev)
        fwd = lambda: fa.fa_fwd_bias(q, k, v, bias, w.causal, w.scale, out=o, lse=lse)
        bwd = lambda: fa.fa_bwd_bias(q, k, v, bias, o, lse, do, w.causal, w.scale, dq=dq, dk=dk, dv=dv,
                                     dbias=dbias, workspace=ws)
        settle(lambda: (fwd(), bwd()), stream)
        tf_, tb_ = time_calls(fwd, 20, stream), time_calls(bwd, 10, stream)
        ff = fwd_flops(w)
        tok = w.B * w.N * w.H * w.d * 2
        nn = w.B * w.H * w.N * w.N * 2
        rows = w.B * w.H * w.N * 4
        fbytes = 4 * tok + rows + nn
        bbytes = 5 * tok + rows + nn + 3 * tok + nn + 2 * rows
        def roof(flops, byts, t):
            return {"ms": round(t * 1e3, 4), "tflops": round(flops / t / 1e12, 2),
                    "mfma_frac": round(flops / t / 1e12 / PEAK_BF16_TFLOPS, 4),
                    "gbs": round(byts / t / 1e9, 1), "hbm_frac": round(byts / t / 1e9 / PEAK_HBM_GBS, 4),
                    "bytes_per_launch": int(byts), "flops_per_launch": flops}
        out[name] = {"B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                     "fwd": roof(ff, fbytes, tf_), "bwd": roof(2.5 * ff, bbytes, tb_)}
        del q, k, v, do, bias, o, lse, dq, dk, dv, dbias, ws
    return out


def fp8_leg(fa, si, torch, dev, stream):
    """FP8 (e4m3) forward on the FP8 workloads: per-head descales (fa_fwd_fp8)
    and E8M0 block scales (fa_fwd_mxfp8), TFLOP/s against the dense FP8 MFMA
    peak, with the bf16 forward of the same shape (random bf16 inputs) timed
    in the same window."""
    out = {}
    for (name, w), (mname, mw) in zip(si.FP8_WORKLOADS.items(), si.MXFP8_WORKLOADS.items()):
        assert (w.B, w.H, w.N, w.d, w.causal) == (mw.B, mw.H, mw.N, mw.d, mw.causal)
        b8 = si.draw_fp8(w.B, w.N, w.H, w.d, w.seed)
        t = {k: torch.from_numpy(v).to(dev) for k, v in b8.items()}
        b8 = si.draw_mxfp8(mw.B, mw.N, mw.H, mw.d, mw.seed)
        m = {k: torch.from_numpy(v).to(dev) for k, v in b8.items()}
        del b8
        o = torch.empty((w.B, w.N, w.H, w.d), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        call = lambda: fa.fa_fwd_fp8(t["q"], t["k"], t["v"], t["q_descale"], t["k_descale"], t["v_descale"],
                                     w.causal, w.scale, out=o, lse=lse)
        mcall = lambda: fa.fa_fwd_mxfp8(m["q"], m["q_scale"], m["k"], m["k_scale"], m["v"], m["v_scale"],
                                        w.causal, w.scale, out=o, lse=lse)
        bq = torch.randn((w.B, w.N, w.H, w.d), device=dev).to(torch.bfloat16)
        bk, bv = torch.randn_like(bq, dtype=torch.float32).to(torch.bfloat16), torch.randn_like(bq, dtype=torch.float32).to(torch.bfloat16)
        ref = lambda: fa.fa_fwd(bq, bk, bv, w.causal, w.scale, out=o, lse=lse)
        time_calls(lambda: (call(), mcall(), ref()), settle_calls(2 * fwd_flops(w)), stream)
        reps = 10 if w.N * w.N * w.B * w.H >= (1 << 30) else 30
        t8, tm, t16 = time_calls(call, reps, stream), time_calls(mcall, reps, stream), time_calls(ref, reps, stream)
        ff = fwd_flops(w)
        roof = lambda tt: {"bound": "mfma", "achieved": round(ff / tt / 1e12, 2), "peak": PEAK_FP8_TFLOPS,
                           "unit": "TFLOP/s", "frac": round(ff / tt / 1e12 / PEAK_FP8_TFLOPS, 4)}
        shape = {"B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal}
        out[name] = {**shape, "ms": round(t8 * 1e3, 4), "roofline": roof(t8), "bf16_fwd_ms": round(t16 * 1e3, 4),
                     "speedup_vs_bf16": round(t16 / t8, 3)}
        out[mname] = {**shape, "ms": round(tm * 1e3, 4), "roofline": roof(tm), "bf16_fwd_ms": round(t16 * 1e3, 4),
                      "speedup_vs_bf16": round(t16 / tm, 3), "time_vs_per_head_fp8": round(tm / t8, 3)}
        del t, m, o, lse, bq, bk, bv
    return out


# (batch, head) pairs each workload's oracle forward is timed on (the
# forward+backward of the step's workload takes --cpu-heads of its own).
CPU_FWD_SAMPLE_HEADS = {"tiny": 2, "short_noncausal": 32, "short_causal": 32, "mid_causal": 8,
                        "long_causal": 1, "train_causal": 8}


def cpu_baseline_leg(args, w, bits, ff, bf, si):
    """The fp64 oracle as it stands, timed on this host's cores: the step's
    forward+backward on --cpu-heads (batch, head) pairs (the headline), and
    per workload the forward alone on a few pairs (for the training workload
    also the forward+backward, so the backward's share is their difference).
    Each figure is also extrapolated to the whole workload."""
    import oracle
    from threadpoolctl import threadpool_info

    def run(wl, b_, heads, backward):
        x = {n: si.bf16_bits_to_f64(b_[n]) for n in (("q", "k", "v", "do") if backward else ("q", "k", "v"))}
        pairs = [(i // wl.H, i % wl.H) for i in range(heads)]
        t0 = time.perf_counter()
        for b, h in pairs:
            sl = (slice(b, b + 1), slice(None), slice(h, h + 1), slice(None))
            if backward:
                oracle.attention_backward(x["q"][sl], x["k"][sl], x["v"][sl], x["do"][sl], wl.causal, wl.scale)
            else:
                oracle.attention_forward(x["q"][sl], x["k"][sl], x["v"][sl], wl.causal, wl.scale)
        return (time.perf_counter() - t0) / heads

    heads = min(args.cpu_heads, w.B * w.H)
    per_head_step = run(w, bits, heads, True)
    threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    flops_head = (ff + bf) / (w.B * w.H)
    per_config = {}
    for name, wl in si.WORKLOADS.items():
        n = min(CPU_FWD_SAMPLE_HEADS.get(name, 1), wl.B * wl.H)
        b_ = bits if name == w.name else si.draw_workload(wl)
        t = run(wl, b_, n, False)
        f_head = fwd_flops(wl) / (wl.B * wl.H)
        e = {"sample_heads": n, "heads": wl.B * wl.H, "fwd_s_per_head": round(t, 5),
             "fwd_gflops": round(f_head / t / 1e9, 3), "fwd_s_whole_est": round(t * wl.B * wl.H, 2)}
        if name == w.name:
            tb = per_head_step - t
            e.update({"fwd_bwd_sample_heads": heads, "fwd_bwd_s_per_head": round(per_head_step, 5),
                      "bwd_s_per_head": round(tb, 5), "bwd_gflops": round(2.5 * f_head / tb / 1e9, 3),
                      "bwd_s_whole_est": round(tb * wl.B * wl.H, 2)})
        per_config[name] = e
    return {"value": round(flops_head / per_head_step / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"fp64 oracle forward+backward of {heads} of the {w.B * w.H} (batch, head) pairs of "
                      f"B={w.B} H={w.H} N={w.N} d={w.d} causal, {per_head_step * heads:.1f} s; NumPy/BLAS "
                      f"with {threads} BLAS threads",
            "cpu": cpu_info(), "per_config": per_config}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; sharding the path over "
                                   "several GPUs is designed but not built", "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import exact_tiled_attention_37_amd as fa
    import seeded_inputs as si

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    fa.load_library()
    dev = torch.device("cuda:0")
    w = si.WORKLOADS[args.workload]
    if not w.backward:
        raise SystemExit(f"workload {w.name} has no backward; pick one with backward=True")

    bits = si.draw_workload(w)
    q, k, v, do = (si.bits_to_torch(bits[n], dev) for n in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(fa.fa_bwd_workspace_bytes(w.B, w.N, w.H, w.d), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    resident = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    stream = torch.cuda.current_stream()

    def fwd():
        fa.fa_fwd(q, k, v, w.causal, w.scale, out=o, lse=lse)

    def bwd():
        fa.fa_bwd(q, k, v, o, lse, do, w.causal, w.scale, dq=dq, dk=dk, dv=dv, workspace=ws)

    for _ in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    # However few warm-up steps were asked for, about 0.1 s of untimed steps
    # follow, so that the timed window starts at a settled clock.
    settle(lambda: (fwd(), bwd()), stream)
    torch.cuda.synchronize()

    # Timed region: exactly K whole steps.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1, e2 in ev:
        e0.record(stream)
        fwd()
        e1.record(stream)
        bwd()
        e2.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_each = sorted(e0.elapsed_time(e1) for e0, e1, _ in ev)  # ms per call
    bwd_each = sorted(e1.elapsed_time(e2) for _, e1, e2 in ev)
    step_each = sorted(e0.elapsed_time(e2) for e0, _, e2 in ev)
    fwd_s = sum(fwd_each) / 1e3 / args.steps
    bwd_s = sum(bwd_each) / 1e3 / args.steps
    step_mean_s = ev[0][0].elapsed_time(ev[-1][2]) / 1e3 / args.steps
    step_s = step_each[len(step_each) // 2] / 1e3  # the median step
    peak_mem = torch.cuda.max_memory_allocated()

    ff = fwd_flops(w)
    bf = 2.5 * ff
    value = (ff + bf) / step_s / 1e12

    traffic = stored_traffic(w.name)

    def roof(flops, secs, kernel, launch_key):
        ach = flops / secs / 1e12
        t = None
        if traffic is not None and launch_key in traffic.get("bytes_per_launch", {}):
            t = int(traffic["bytes_per_launch"][launch_key])
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": t, "kernel": kernel,
                "avg_launch_ms": round(secs * 1e3, 4), "flops_per_launch": flops}

    detail = {
        "gpu": torch.cuda.get_device_name(0),
        "arch": torch.cuda.get_device_properties(0).gcnArchName,
        "fwd_ms": round(fwd_s * 1e3, 4),
        "bwd_ms": round(bwd_s * 1e3, 4),
        "fwd_ms_median": round(fwd_each[len(fwd_each) // 2], 4),
        "fwd_ms_min": round(fwd_each[0], 4),
        "bwd_ms_median": round(bwd_each[len(bwd_each) // 2], 4),
        "bwd_ms_min": round(bwd_each[0], 4),
        "fwd_tflops": round(ff / fwd_s / 1e12, 2),
        "bwd_tflops": round(bf / bwd_s / 1e12, 2),
        "fwd_frac_of_peak": round(ff / fwd_s / 1e12 / PEAK_BF16_TFLOPS, 4),
        "ms_per_step_mean": round(step_mean_s * 1e3, 4),
        "ms_per_step_min": round(step_each[0], 4),
        "value_from_mean_step": round((ff + bf) / step_mean_s / 1e12, 2),
        "wall_s_timed_region": round(wall, 4),
        "resident_bytes": int(resident),
        "peak_bytes_during_steps": int(peak_mem),
    }

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        detail["copy_calibration_bytes"] = n
        del src, dst

    if not args.no_sweep:
        sweep = {}
        for name, wl in si.WORKLOADS.items():
            b2 = si.draw(wl.B, wl.N, wl.H, wl.d, wl.seed)
            q2, k2, v2 = (si.bits_to_torch(b2[n], dev) for n in ("q", "k", "v"))
            o2 = torch.empty_like(q2)
            l2 = torch.empty((wl.B, wl.H, wl.N), dtype=torch.float32, device=dev)
            call = lambda: fa.fa_fwd(q2, k2, v2, wl.causal, wl.scale, out=o2, lse=l2)
            time_calls(call, settle_calls(fwd_flops(wl)), stream)
            reps = 50 if wl.N * wl.N * wl.B * wl.H < (1 << 30) else 10
            s = time_calls(call, reps, stream)
            each = time_each(call, reps, stream)
            med = each[len(each) // 2]
            tf = fwd_flops(wl) / s / 1e12
            sweep[name] = {"B": wl.B, "H": wl.H, "N": wl.N, "d": wl.d, "causal": wl.causal,
                           "fwd_ms": round(s * 1e3, 4), "fwd_tflops": round(tf, 2),
                           "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                           "fwd_ms_median": round(med * 1e3, 4), "fwd_ms_min": round(each[0] * 1e3, 4),
                           "frac_of_peak_median": round(fwd_flops(wl) / med / 1e12 / PEAK_BF16_TFLOPS, 4)}
            if wl.d == 64 and wl.N <= 512 and wl.B * wl.H >= 256:
                # Short sequences are bound by memory traffic (Q, K, V in, O and the
                # logsumexp out), so they are also timed with the caches flushed:
                # a 512 MiB buffer (more than the L2s and the 256 MiB Infinity
                # Cache) is overwritten before each call, outside its events.
                sweep[name]["cold_l2"] = cold_call_roofline(call, wl, reps=20, stream=stream)
            del q2, k2, v2, o2, l2
        detail["fwd_sweep"] = sweep

    if not args.no_ring:
        detail["ring_rank"] = ring_rank_leg(fa, si, torch, dev, stream)
    if not args.no_decode:
        detail["decode"] = decode_leg(fa, si, torch, dev, stream)
    if not args.no_bias:
        detail["bias"] = bias_leg(fa, si, torch, dev, stream)
    if not args.no_fp8:
        detail["fp8"] = fp8_leg(fa, si, torch, dev, stream)

    cpu = None
    if args.cpu_heads > 0:
        cpu = cpu_baseline_leg(args, w, bits, ff, bf, si)

    line = {
        "metric": "attention fwd/bwd TFLOP/s at 1 MI355X; % of bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"attention fwd+bwd B={w.B} H={w.H} N={w.N} d={w.d} "
                               f"{'causal' if w.causal else 'non-causal'}",
                   "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   "global_batch": w.B, "seq_len": w.N, "parallelism": "single GPU"},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "roofline": roof(bf, bwd_s, "fa_bwd call (bwd_dq_kernel, which also forms the row terms, + bwd_dkdv_kernel)", "fa_bwd"),
        "roofline_fwd": roof(ff, fwd_s, "fwd48_kernel (the causal d = 128 form with 192-row workgroups)", "fa_fwd"),
        "cpu_baseline": cpu,
        "detail": detail,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
