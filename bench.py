#!/usr/bin/env python3
"""Benchmark of the MI355X linear-attention recurrence library (one GPU).

Headline workload: gated-delta chunkwise prefill of one layer, B = 1, H = 16,
T = 1,048,576, d_k = d_v = 128, bf16 q/k/v/alpha/beta, fp32 state, seeded synthetic
inputs with the gated-delta recipe (synth.gdn_inputs).  One step = one complete
la_prefill over the whole sequence, run as its separate passes so that each pass is
timed with HIP events on the launch stream.  value = tokens/s, a token being one
position through all 16 heads.

Timing protocol (after the NoteBank paper's latency protocol, App. C.5: warm-up, timed
repetitions, medians): W untimed warm-up steps, then K timed steps; ms_per_step is the
K-step bracket divided by K, and the median, minimum and maximum of the per-step times
are reported beside it.  The other configurations are timed the same way (at least five
repetitions each).  Inputs are generated on the device before any timed region.

The headline prefill is timed a second time with slow decay (gate logits U(-8, -4)
instead of the recipe's U(-2, 4)): with the recipe's gates the transition over each
segment's last 8 chunks is exactly zero in fp32, so the map pass carries only those chunks
and the scan has nothing to chain; with slow decay the map pass carries whole segments and
the scan chains them (`prefill_slow_decay`).

Also measured in the same run: the fp32 additive configuration (1 head x 1024 tokens),
BASED prefill (B=4, H=16, T=8192), the 64K-token gated-delta prefill, the batched decode
step (256 sequences x 16 heads, gated-delta state 128 x 128 and BASED state 273 x 64 per
head, 1024 consecutive steps; plus the gated-delta step on a 1 GiB state set that the
256 MB Infinity Cache cannot hold), the 8-head x 256 gated-delta shape, the NoteBank
write/address steps, and the fp64 oracle on each configuration on the host cores.

The published peaks (HBM 8 TB/s, dense bf16 MFMA 2.5 PFLOP/s) are the roofline
denominators.  Beside them the run measures what the same device reaches on two plain
library operations, a 2 GiB device-to-device copy and an 8192^3 bf16 matrix product
(torch, i.e. the ROCm libraries), and reports the replay's rate against that copy rate
too; the device's properties as the runtime reports them are listed with them.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-decode]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "prefill tokens/sec (GDN, T=1M) + decode steps/sec, 1×MI355X, % of roofline"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published
FP32_VEC_PEAK_TFLOPS = 157.3
PROFILE_COUNTERS = ROOT / "profiles" / "gdn_prefill_1m_counters.txt"

# Algorithmic work per token-head of the gated-delta prefill at chunk 64, d = 128:
# bytes: q, k, v (3 x 128 x 2) + alpha, beta (2 x 2) + o (128 x 2): inputs read once,
# outputs written once (intermediates such as stored per-chunk transforms are the
# implementation's, not the method's, and appear only under measured traffic)
C_, D_ = 64, 128


def gdn_bytes_per_token_head(d):
    return 3 * d * 2 + 2 * 2 + d * 2


def gdn_flops_per_token_head(d, c=C_):
    # chunk form (multiply-add = 2): Grams K K^T and Q K^T, W, U~, A U (5 x 2 C^2 d),
    # W S^T, Q S^T, the state update (3 x 2 C d^2), the triangular solve (C^3 / 3)
    return (5 * 2 * c * c * d + 3 * 2 * c * d * d + c ** 3 / 3) / c


BYTES_PER_TOKEN_HEAD = gdn_bytes_per_token_head(D_)          # 1028
FLOPS_PER_TOKEN_HEAD = gdn_flops_per_token_head(D_)          # 181,589


def stats(xs):
    xs = [float(x) for x in xs]
    return {"median": round(statistics.median(xs), 4), "min": round(min(xs), 4),
            "max": round(max(xs), 4), "mean": round(sum(xs) / len(xs), 4), "n": len(xs)}


def kernel_source_hash() -> str:
    src = (ROOT / "gated_delta_rule_chunkwise_amd" / "csrc" / "chunk.hip").read_bytes()
    return hashlib.sha256(src).hexdigest()[:16]


def read_traffic(kernel_key: str):
    """HBM bytes per launch of `kernel_key` from the committed counter summary, scaled by
    the copy-kernel calibration recorded there; None if absent or taken on other code."""
    if not PROFILE_COUNTERS.exists():
        return None
    txt = PROFILE_COUNTERS.read_text()
    m = re.search(r"source_sha256_16:\s*(\w+)", txt)
    if not m or m.group(1) != kernel_source_hash():
        return None
    m = re.search(rf"^{re.escape(kernel_key)}\s+traffic_bytes_per_launch:\s*([0-9.eE+]+)", txt, re.M)
    return float(m.group(1)) if m else None


class Timer:
    """Repetitions of a callable on one stream, each bracketed by HIP events recorded on
    that stream; returns the per-repetition milliseconds divided by `per`."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def reps(self, fn, reps=5, warmup=2, per=1):
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        evs[0].record(self.stream)
        for i in range(reps):
            fn()
            evs[i + 1].record(self.stream)
        torch.cuda.synchronize()
        return [evs[i].elapsed_time(evs[i + 1]) / per for i in range(reps)]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--seq-len", type=int, default=1 << 20)
    ap.add_argument("--heads", type=int, default=16)
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-based", action="store_true")
    ap.add_argument("--no-notebank", action="store_true")
    ap.add_argument("--no-d256", action="store_true")
    ap.add_argument("--no-small", action="store_true")
    ap.add_argument("--no-reference-rates", action="store_true")
    ap.add_argument("--no-slow-decay", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run one plain 256 MiB copy (la_prefill with T = 0) so that HBM "
                         "byte counters can be scaled against a known size")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print("bench.py measures one GPU only: this build has no multi-GPU path "
                  "(every (batch, head) slice is independent; sharding is described in DESIGN.md)",
                  file=sys.stderr)
        sys.exit(2)

    import torch

    import gated_delta_rule_chunkwise_amd as la
    import synth

    la.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    timer = Timer(torch, stream)
    B, H, T, D = 1, args.heads, args.seq_len, D_

    if args.calibrate_copy:  # copy_or_zero_kernel: reads and writes exactly 256 MiB
        e = torch.empty((1, 4096, 0, 128), dtype=torch.bfloat16, device=dev)
        ea = torch.empty((1, 4096, 0), dtype=torch.bfloat16, device=dev)
        S0c = torch.randn((1, 4096, 128, 128), device=dev)
        la.prefill("gated_delta", e, e, e, ea, ea, S0=S0c)
        torch.cuda.synchronize()
        del S0c

    # ---------------------------------------------------------------- headline prefill
    pre = bench_gdn_prefill(torch, la, synth, dev, stream, B, H, T, D, args.steps, args.warmup, seed=3)
    ms_per_step = pre.pop("_ms_per_step")
    token_heads = B * H * T
    # the roofline kernel is the replay: it reads q, k, v, alpha, beta once and writes o once,
    # exactly the method's bytes per token-head (it is also the longest pass)
    dominant = pre.pop("_dominant")
    dom = "replay"
    t_dom = pre["ms_per_pass"][dom]["mean"] * 1e-3
    alg_b = token_heads * BYTES_PER_TOKEN_HEAD
    alg_f = token_heads * FLOPS_PER_TOKEN_HEAD
    hbm_bound = alg_b / (HBM_PEAK_GBS * 1e9) >= alg_f / (BF16_PEAK_TFLOPS * 1e12)
    if hbm_bound:
        ach, peak, unit, bound = alg_b / t_dom / 1e9, HBM_PEAK_GBS, "GB/s", "hbm"
    else:
        ach, peak, unit, bound = alg_f / t_dom / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s", "mfma"
    roofline = {
        "bound": bound, "achieved": round(ach, 1), "peak": peak, "unit": unit,
        "frac": round(ach / peak, 4), "traffic": read_traffic(dom),
        "kernel": pre["kernels"][dom],
        "ms_per_launch": round(t_dom * 1e3, 4),
        "ms_per_launch_stats": pre["ms_per_pass"][dom],
        "alg_bytes_per_launch": alg_b, "alg_bytes_per_unit": BYTES_PER_TOKEN_HEAD,
        "units_per_launch": token_heads, "unit_name": "token-head",
        "alg_flops_per_launch": alg_f, "longest_pass": dominant,
    }

    # the same prefill with slow decay, a ~ U(-8, -4) (alpha in [0.982, 0.9997]): the segment
    # transitions stay nonzero, so the map pass carries whole segments
    slow = None
    if not args.no_slow_decay:
        slow = bench_gdn_prefill(torch, la, synth, dev, stream, B, H, T, D, max(3, args.steps // 2),
                                 args.warmup, seed=3, a_range=(-8.0, -4.0))
        ms_slow = slow.pop("_ms_per_step")
        slow.pop("_dominant")
        slow["ms_per_step"] = round(ms_slow, 4)
        slow["tokens_per_s"] = round(B * T / (ms_slow * 1e-3), 1)
        slow["gates"] = "alpha = exp(-softplus(a)), a ~ U(-8, -4)"

    # ---------------------------------------------------------------- other configurations
    small = None if args.no_small else bench_small_configs(torch, la, synth, dev, stream, timer)
    based = None
    if not args.no_based:
        based = bench_based(torch, la, synth, dev, stream, timer)
        based["compact"] = bench_based(torch, la, synth, dev, stream, timer, "based_compact")
    decode = None if args.no_decode else bench_decode(torch, la, synth, dev, stream, timer, args.decode_steps)
    gdn256 = None if args.no_d256 else bench_gdn256(torch, la, synth, dev, stream, timer, args.steps,
                                                    args.warmup, args.seq_len)
    notebank = None if args.no_notebank else bench_notebank(torch, la, synth, dev, stream, timer)
    rates = None if args.no_reference_rates else bench_reference_rates(torch, dev, timer)
    if rates is not None:
        roofline["measured_copy_gbs"] = rates["copy"]["gbs"]
        roofline["frac_of_measured_copy"] = round(ach / rates["copy"]["gbs"], 4) if hbm_bound else None
    cpu = None if args.no_cpu_baseline else bench_cpu(args.cpu_seconds)

    out = {
        "metric": METRIC, "value": round(B * T / (ms_per_step * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"gated-delta chunkwise prefill, B={B} H={H} T={T} d_k=d_v={D}, "
                               "bf16 inputs, fp32 state, chunk 64", "batch": B, "heads": H,
                   "seq_len": T, "d_k": D, "d_v": D, "chunk": 64, "parallelism": "none (1 GPU)"},
        "timing": {"ms_per_step": pre["ms_per_step_stats"], "protocol":
                   f"{args.warmup} warm-up steps, {args.steps} timed steps, HIP events per step "
                   "and per pass on the launch stream"},
        "roofline": roofline,
        "prefill": pre,
        "prefill_slow_decay": slow,
        "configs": {"cfg0_additive_fp32": None if small is None else small["additive_fp32"],
                    "cfg1_based_prefill": based,
                    "cfg2_gdn_64k": None if small is None else small["gdn_64k"],
                    "cfg3_gdn_1m": "headline (value, prefill)",
                    "cfg4_decode": decode},
        "gdn_d256": gdn256,
        "notebank": notebank,
        "reference_rates": rates,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_gdn_prefill(torch, la, synth, dev, stream, B, H, T, D, steps, warmup, seed, a_range=None):
    """The gated-delta prefill as its separate passes, each bracketed by HIP events on the
    launch stream; returns per-pass and per-step statistics.  a_range: the gate logits'
    range (the recipe's U(-2, 4) by default)."""
    inp = synth.gdn_inputs(B, H, T, D, D, dtype=torch.bfloat16, seed=seed, device=dev,
                           **({} if a_range is None else {"a_range": a_range}))
    q, k, v, a, b = inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"]
    o = torch.empty((B, H, T, D), dtype=torch.bfloat16, device=dev)
    S_T = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    ws = torch.empty(max(la.workspace_size("gated_delta", la.BF16, B, H, T, D, D), 16), dtype=torch.uint8,
                     device=dev)
    nseg, seg_chunks = la.segments("gated_delta", la.BF16, B, H, T, D, D)
    passes = la.prefill_passes("gated_delta", la.BF16, B, H, T, D, D)
    names = {la.PASS_TRANSFORM: "transform", la.PASS_MAPS: "maps", la.PASS_SCAN: "scan",
             la.PASS_REPLAY: "replay"}

    def step(evs=None):
        for i, p in enumerate(passes):
            la.prefill("gated_delta", q, k, v, a, b, o=o, S_T=S_T, workspace=ws, pass_=p, stream=stream)
            if evs is not None:
                evs[i + 1].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    all_evs = []
    t_start.record(stream)
    for _ in range(steps):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(passes) + 1)]
        evs[0].record(stream)
        step(evs)
        all_evs.append(evs)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / steps
    per_pass = {names[p]: [e[i].elapsed_time(e[i + 1]) for e in all_evs] for i, p in enumerate(passes)}
    per_step = [e[0].elapsed_time(e[-1]) for e in all_evs]
    th = B * H * T
    alg_b = th * gdn_bytes_per_token_head(D)
    alg_f = th * gdn_flops_per_token_head(D)
    t_roof = max(alg_b / (HBM_PEAK_GBS * 1e9), alg_f / (BF16_PEAK_TFLOPS * 1e12))
    pass_stats = {kk: stats(vv) for kk, vv in per_pass.items()}
    dom = max(pass_stats, key=lambda kk: pass_stats[kk]["mean"])
    wide = "" if D == 128 else f", {D}"
    if D == 128:  # the map and replay passes form each chunk's solve: no transform pass
        kernels = {"replay": "replay_kernel<true> (replay pass, forming each chunk's solve from its keys)",
                   "maps": "map_kernel<true> (segment-map pass; helper waves form each chunk's solve blocks)",
                   "scan": "scan_delta_kernel (segment scan)"}
    else:
        kernels = {"replay": f"replay_kernel<true{wide}> (replay pass)",
                   "maps": f"map_kernel<true{wide}> (segment-map pass)",
                   "transform": f"tprep_kernel<{D}> (per-chunk UT transform pass)",
                   "scan": f"scan_delta_kernel<{D}> (segment scan)"}
    res = {"workload": f"gated-delta chunkwise prefill, B={B} H={H} T={T} d_k=d_v={D}, bf16 inputs, "
                       "fp32 state, chunk 64",
           "ms_per_step_stats": stats(per_step), "ms_per_pass": pass_stats,
           "segments": nseg, "chunks_per_segment": seg_chunks,
           "alg_bytes": alg_b, "alg_flops": alg_f, "roofline_time_ms": round(t_roof * 1e3, 4),
           "roofline_frac_whole_step": round(t_roof * 1e3 / ms_per_step, 4),
           "hbm_frac_whole_step": round(alg_b / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "bf16_mfma_frac_whole_step": round(alg_f / (ms_per_step * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
           "kernels": {names[p]: kernels[names[p]] for p in passes},
           "_ms_per_step": ms_per_step, "_dominant": dom}
    del inp, q, k, v, a, b, o, ws
    torch.cuda.empty_cache()
    return res


def bench_small_configs(torch, la, synth, dev, stream, timer):
    """The fp32 additive configuration (B=1, H=1, T=1024, d=64: one head, so launch
    latency bounds it) and the gated-delta prefill at 64K tokens (B=1, H=16, T=65536,
    d=128, bf16), each timed as whole la_prefill calls."""
    res = {}
    d0 = synth.additive_inputs(1, 1, 1024, 64, dtype=torch.float32, seed=0, device=dev)
    o0 = torch.empty_like(d0["v"])
    S0 = torch.empty((1, 1, 64, 64), dtype=torch.float32, device=dev)
    us = timer.reps(lambda: [la.prefill("additive", d0["q"], d0["k"], d0["v"], o=o0, S_T=S0, stream=stream)
                             for _ in range(100)], reps=7, warmup=1, per=100)
    us = [x * 1e3 for x in us]
    res["additive_fp32"] = {"workload": "additive linear attention, B=1 H=1 T=1024 d=64, fp32",
                            "us_per_call": stats(us),
                            "tokens_per_s": round(1024 / (statistics.median(us) * 1e-6), 1)}
    B, H, T, D = 1, 16, 65536, 128
    g = synth.gdn_inputs(B, H, T, D, D, dtype=torch.bfloat16, seed=2, device=dev)
    o2 = torch.empty_like(g["v"])
    S2 = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    ws = torch.empty(max(la.workspace_size("gated_delta", la.BF16, B, H, T, D, D), 16), dtype=torch.uint8, device=dev)
    ms = timer.reps(lambda: la.prefill("gated_delta", g["q"], g["k"], g["v"], g["alpha"], g["beta"], o=o2, S_T=S2,
                                       workspace=ws, stream=stream), reps=20, warmup=3)
    byt = B * H * T * BYTES_PER_TOKEN_HEAD
    flo = B * H * T * FLOPS_PER_TOKEN_HEAD
    t_roof = max(byt / (HBM_PEAK_GBS * 1e9), flo / (BF16_PEAK_TFLOPS * 1e12))
    nseg, sc = la.segments("gated_delta", la.BF16, B, H, T, D, D)
    med = statistics.median(ms)
    res["gdn_64k"] = {"workload": "gated-delta chunkwise prefill, B=1 H=16 T=65536 d_k=d_v=128, bf16, chunk 64",
                      "ms": stats(ms), "tokens_per_s": round(T / (med * 1e-3), 1), "segments": nseg,
                      "chunks_per_segment": sc, "alg_bytes": byt, "alg_flops": flo,
                      "roofline_time_ms": round(t_roof * 1e3, 4), "roofline_frac": round(t_roof * 1e3 / med, 4)}
    del g, o2, ws
    torch.cuda.empty_cache()
    return res


def bench_gdn256(torch, la, synth, dev, stream, timer, steps, warmup, T):
    """The gated-delta shape of the NoteBank paper's own backbone: 8 heads of width 256
    (d_k = d_v = 256, fp32 state 256 x 256 per head), bf16 inputs with the gated-delta
    recipe, T tokens (1M by default), its passes timed as for the headline; the 24-layer
    stack of it; then the decode step on 256 sequences x 8 heads of that width."""
    B, H, D = 1, 8, 256
    res = bench_gdn_prefill(torch, la, synth, dev, stream, B, H, T, D, steps, warmup, seed=6)
    ms = res.pop("_ms_per_step")
    res.pop("_dominant")
    res["ms"] = round(ms, 4)
    res["tokens_per_s"] = round(B * T / (ms * 1e-3), 1)
    rep = res["ms_per_pass"]["replay"]["mean"]
    res["replay_hbm_frac"] = round(B * H * T * gdn_bytes_per_token_head(D) / (rep * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    res["replay_traffic"] = read_traffic("d256_replay")
    # the recurrence's share of the pages' 24-layer GDN at this length: 24 whole-layer
    # prefills back to back (each layer reuses these inputs; projections, convolutions and
    # the other layer parts are outside the recurrence)
    inp = synth.gdn_inputs(B, H, T, D, D, dtype=torch.bfloat16, seed=6, device=dev)
    o = torch.empty((B, H, T, D), dtype=torch.bfloat16, device=dev)
    S_T = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    ws = torch.empty(max(la.workspace_size("gated_delta", la.BF16, B, H, T, D, D), 16), dtype=torch.uint8,
                     device=dev)
    stack = timer.reps(lambda: [la.prefill("gated_delta", inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                                           o=o, S_T=S_T, workspace=ws, stream=stream) for _ in range(24)],
                       reps=3, warmup=0)
    res["stack_24_layers_ms"] = stats(stack)
    del inp, o, ws
    torch.cuda.empty_cache()

    N, nsteps = 256 * 8, 256
    S = synth.gdn_state((N, D, D), seed=7, device=dev)
    g = synth.gdn_decode_inputs(nsteps, N, D, D, dtype=torch.bfloat16, seed=7, device=dev)
    od = torch.empty((N, D), dtype=torch.bfloat16, device=dev)

    def loop():
        for t in range(nsteps):
            la.decode_step("gated_delta", S, g["q"][t], g["k"][t], g["v"][t], g["alpha"][t], g["beta"][t],
                           S_out=S, o=od, stream=stream)
    us = [x * 1e3 for x in timer.reps(loop, reps=5, warmup=1, per=nsteps)]
    bd = 2 * N * D * D * 4 + N * (3 * D + 2 + D) * 2
    med = statistics.median(us)
    res["decode"] = {"states": N, "steps": nsteps, "us_per_step": stats(us),
                     "steps_per_s": round(1e6 / med, 1), "alg_bytes_per_step": bd,
                     "hbm_frac": round(bd / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    del S, g
    torch.cuda.empty_cache()
    return res


def bench_decode(torch, la, synth, dev, stream, timer, steps):
    """256 sequences x 16 heads; gated-delta and BASED decode (and BASED with the compact
    153-feature state), `steps` consecutive steps per repetition, five repetitions; then
    the gated-delta step on 16384 states (1 GiB, four times the Infinity Cache), so that
    the state streams from HBM itself."""
    N, D, dp, dv_b = 256 * 16, 128, 16, 64
    Dphi = 1 + dp + dp * dp
    Dc = 1 + dp + dp * (dp + 1) // 2
    res = {"states": N, "steps": steps}
    # gated delta: seeded N(0,1) start state, per-step q/k/v/alpha/beta resident in HBM
    S = synth.gdn_state((N, D, D), seed=4, device=dev)
    g = synth.gdn_decode_inputs(steps, N, D, D, dtype=torch.bfloat16, seed=4, device=dev)
    o = torch.empty((N, D), dtype=torch.bfloat16, device=dev)
    # BASED: start state = the end state of a 64-token warm-up prefill of the same batch
    w = synth.based_warmup_inputs(N, 64, dp, dv_b, dtype=torch.bfloat16, seed=4, device=dev)
    _, s, z = la.prefill("based", w["q"][None], w["k"][None], w["v"][None])
    s, z = s[0].contiguous(), z[0].contiguous()
    bd = synth.based_decode_inputs(steps, N, dp, dv_b, dtype=torch.bfloat16, seed=5, device=dev)
    ob = torch.empty((N, dv_b), dtype=torch.bfloat16, device=dev)
    _, sc, zc = la.prefill("based_compact", w["q"][None], w["k"][None], w["v"][None])
    sc, zc = sc[0].contiguous(), zc[0].contiguous()

    def loop(fn, n=steps):
        return lambda: [fn(t) for t in range(n)]

    def gdn_step(t):
        la.decode_step("gated_delta", S, g["q"][t], g["k"][t], g["v"][t], g["alpha"][t],
                       g["beta"][t], S_out=S, o=o, stream=stream)

    def based_step(t):
        la.decode_step("based", s, bd["q"][t], bd["k"][t], bd["v"][t], z=z, S_out=s, z_out=z,
                       o=ob, stream=stream)

    def compact_step(t):
        la.decode_step("based_compact", sc, bd["q"][t], bd["k"][t], bd["v"][t], z=zc, S_out=sc,
                       z_out=zc, o=ob, stream=stream)

    def both_step(t):
        gdn_step(t)
        based_step(t)

    def entry(fn, byts, extra=None):
        us = [x * 1e3 for x in timer.reps(loop(fn), reps=5, warmup=1, per=steps)]
        med = statistics.median(us)
        r = {"us_per_step": stats(us), "steps_per_s": round(1e6 / med, 1), "alg_bytes_per_step": byts,
             "hbm_frac": round(byts / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        r.update(extra or {})
        return r

    bytes_g = 2 * N * D * D * 4 + N * (3 * D + 2 + D) * 2
    bytes_b = 2 * N * (Dphi * dv_b + Dphi) * 4 + N * (2 * dp + 2 * dv_b) * 2
    bytes_c = 2 * N * (Dc * dv_b + Dc) * 4 + N * (2 * dp + 2 * dv_b) * 2
    res["gated_delta"] = entry(gdn_step, bytes_g)
    res["based"] = entry(based_step, bytes_b)
    res["based_compact"] = entry(compact_step, bytes_c, {"state_features": Dc})
    res["both"] = entry(both_step, bytes_g + bytes_b)
    del S, g, s, z, bd, sc, zc, w
    torch.cuda.empty_cache()

    # the same step on a state set four times the Infinity Cache: an HBM-only rate
    Nh, nst = 16384, 256
    Sh = synth.gdn_state((Nh, D, D), seed=14, device=dev)
    gh = synth.gdn_decode_inputs(nst, Nh, D, D, dtype=torch.bfloat16, seed=14, device=dev)
    oh = torch.empty((Nh, D), dtype=torch.bfloat16, device=dev)

    def hbm_step(t):
        la.decode_step("gated_delta", Sh, gh["q"][t], gh["k"][t], gh["v"][t], gh["alpha"][t], gh["beta"][t],
                       S_out=Sh, o=oh, stream=stream)
    us = [x * 1e3 for x in timer.reps(loop(hbm_step, nst), reps=5, warmup=1, per=nst)]
    med = statistics.median(us)
    bh = 2 * Nh * D * D * 4 + Nh * (3 * D + 2 + D) * 2
    res["gated_delta_1gib_states"] = {"states": Nh, "steps": nst, "us_per_step": stats(us),
                                      "steps_per_s": round(1e6 / med, 1), "alg_bytes_per_step": bh,
                                      "hbm_frac": round(bh / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    del Sh, gh
    torch.cuda.empty_cache()
    return res


def bench_based(torch, la, synth, dev, stream, timer, variant="based"):
    """BASED Taylor prefill, B=4, H=16, T=8192, d'=16, d_v=64, bf16 (all passes); the
    compact variant keeps a 153-feature state."""
    B, H, T, dp, dv = 4, 16, 8192, 16, 64
    d = synth.based_inputs(B, H, T, dp, dv, dtype=torch.bfloat16, seed=1, device=dev)
    Dphi = 1 + dp + dp * (dp + 1) // 2 if variant == "based_compact" else 1 + dp + dp * dp
    o = torch.empty((B, H, T, dv), dtype=torch.bfloat16, device=dev)
    s_T = torch.empty((B, H, Dphi, dv), dtype=torch.float32, device=dev)
    z_T = torch.empty((B, H, Dphi), dtype=torch.float32, device=dev)
    ws = torch.empty(max(la.workspace_size(variant, la.BF16, B, H, T, dp, dv), 16), dtype=torch.uint8,
                     device=dev)
    run = lambda: la.prefill(variant, d["q"], d["k"], d["v"], o=o, S_T=s_T, z_T=z_T, workspace=ws,
                             stream=stream)
    ms = timer.reps(run, reps=20, warmup=3)
    med = statistics.median(ms)
    th = B * H * T
    alg_bytes = th * (2 * dp * 2 + 2 * dv * 2) + 2 * B * H * Dphi * (dv + 1) * 4
    C = 64  # chunk-form FLOPs per token-head: QK^T, A V, Phi_Q s, Phi_K^T V, normaliser
    alg_flops = th * (2 * C * dp + 2 * C * dv + 4 * Dphi * dv + 2 * Dphi + C)
    t_roof = max(alg_bytes / (HBM_PEAK_GBS * 1e9), alg_flops / (BF16_PEAK_TFLOPS * 1e12))
    nseg, sc = la.segments(variant, la.BF16, B, H, T, dp, dv)
    return {"workload": f"BASED Taylor prefill B=4 H=16 T=8192 d'=16 d_v=64 bf16, {Dphi}-feature state",
            "ms": stats(ms), "tokens_per_s": round(B * T / (med * 1e-3), 1),
            "alg_bytes": alg_bytes, "alg_flops": alg_flops, "segments": nseg,
            "roofline_time_ms": round(t_roof * 1e3, 4), "roofline_frac": round(t_roof * 1e3 / med, 4)}


def bench_notebank(torch, la, synth, dev, stream, timer):
    """NoteBank write scoring over the 1M-token, 16-head keys (512-token write chunks, 48-token
    windows, 32-token tails) and addressing at the pages' archive size (4092 notes, 192 channels,
    d_rho = 16, a 128-token question, R = 8)."""
    B, H, T, D = 1, 16, 1 << 20, 128
    k = synth.gdn_inputs(B, H, T, D, D, dtype=torch.bfloat16, seed=3, device=dev)["k"]
    d_head = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    d_mean = torch.empty((B, T), dtype=torch.float32, device=dev)
    ms_s = timer.reps(lambda: la.write_scores(k, 512, d_head=d_head, d_mean=d_mean, stream=stream), reps=10)
    ms_w = timer.reps(lambda: la.write_windows(d_mean, 512, 48, 32, stream=stream), reps=10)
    bytes_s = B * H * T * (D * 2 + 4) + B * T * 4 + B * H * T * 4  # keys, d_head out, d_mean (read H rows, write 1)
    del k
    N, J, nQ, dr, R = 4092, 192, 128, 16, 8
    g = torch.Generator(device=dev).manual_seed(11)
    rho = torch.randn((N, J, dr), generator=g, device=dev).to(torch.bfloat16)
    u = torch.randn((nQ, J, dr), generator=g, device=dev).to(torch.bfloat16)
    pos = torch.arange(N, dtype=torch.int64, device=dev) * 256
    ms_v = timer.reps(lambda: la.address_votes(rho, u, R, pos, want_score=False, stream=stream), reps=10)
    flops_v = 2 * nQ * N * J * dr
    ms, mw, mv = (statistics.median(x) for x in (ms_s, ms_w, ms_v))
    return {"write_scores": {"workload": "keys B=1 H=16 T=1048576 d_k=128 bf16, 512-token write chunks",
                             "ms": stats(ms_s), "alg_bytes": bytes_s,
                             "hbm_frac": round(bytes_s / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
            "write_windows": {"ms": stats(ms_w), "chunks": T // 512},
            "address_votes": {"workload": f"{N} notes x {J} channels, d_rho={dr}, {nQ}-token question, R={R}",
                              "ms": stats(ms_v), "alg_flops": flops_v,
                              "fp32_vector_frac": round(flops_v / (mv * 1e-3) / (FP32_VEC_PEAK_TFLOPS * 1e12), 4)}}


def bench_reference_rates(torch, dev, timer):
    """What the device reaches on two plain library operations, as a check on the
    published peaks: a 2 GiB device-to-device copy (eight times the Infinity Cache; bytes
    read plus bytes written per second) and an 8192 x 8192 x 8192 bf16 matrix product
    (2 * 8192^3 FLOP, contiguous operands).  Also the device's properties as the runtime
    reports them."""
    props = torch.cuda.get_device_properties(dev)
    keep = ("name", "gcnArchName", "multi_processor_count", "total_memory", "L2_cache_size",
            "max_threads_per_multi_processor", "warp_size", "clock_rate", "memory_clock_rate",
            "memory_bus_width")
    device = {kk: getattr(props, kk) for kk in keep if isinstance(getattr(props, kk, None), (int, str))}
    n = 1 << 30  # bf16 elements: 2 GiB
    src = torch.empty(n, dtype=torch.bfloat16, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    ms = timer.reps(lambda: dst.copy_(src), reps=10, warmup=2)
    med = statistics.median(ms)
    copy = {"bytes": 4 * n, "ms": stats(ms), "gbs": round(4 * n / (med * 1e-3) / 1e9, 1),
            "frac_of_published_peak": round(4 * n / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del src, dst
    m = 8192
    a = torch.randn((m, m), device=dev).to(torch.bfloat16)
    b = torch.randn((m, m), device=dev).to(torch.bfloat16)
    ms = timer.reps(lambda: torch.mm(a, b), reps=10, warmup=3)
    med = statistics.median(ms)
    gemm = {"flops": 2 * m ** 3, "ms": stats(ms), "tflops": round(2 * m ** 3 / (med * 1e-3) / 1e12, 1),
            "frac_of_published_peak": round(2 * m ** 3 / (med * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
    del a, b
    torch.cuda.empty_cache()
    return {"device": device, "copy": copy, "bf16_gemm": gemm}


def bench_cpu(target_s):
    """The fp64 oracle, as it is, on every configuration, on this host's cores (inputs of
    the same recipes and shapes, generated on the host: the oracle's cost does not depend
    on the values).  Each figure is scaled from a bounded sample to the configuration's
    unit; the sample is stated.  The headline (1M tokens) grows its sample until it takes
    about target_s."""
    import torch

    import oracle
    import synth

    cores = len(os.sched_getaffinity(0))
    oracle._load()

    def wall(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    per = {}
    # cfg0: the whole configuration
    d0 = synth.additive_inputs(1, 1, 1024, 64, dtype=torch.float32, seed=0)
    dt = wall(lambda: oracle.prefill("additive", d0["q"], d0["k"], d0["v"], nthreads=cores))
    per["cfg0_additive_fp32"] = {"value": round(1024 / dt, 1), "unit": "tokens/s",
                                 "sample": f"the whole configuration (1024 tokens), {dt:.3f} s"}
    # cfg1: the first 2048 of the 8192 tokens of all 64 (b, h) slices
    d1 = synth.based_inputs(4, 16, 2048, 16, 64, seed=1)
    dt = wall(lambda: oracle.prefill("based", d1["q"], d1["k"], d1["v"], nthreads=cores))
    per["cfg1_based_prefill"] = {"value": round(4 * 2048 / dt, 1), "unit": "tokens/s",
                                 "sample": f"the first 2048 tokens of all 4 x 16 slices, {dt:.2f} s"}
    # cfg2: the first 16384 of the 65536 tokens of all 16 heads
    d2 = synth.gdn_inputs(1, 16, 16384, 128, 128, seed=2)
    dt = wall(lambda: oracle.prefill("gated_delta", d2["q"], d2["k"], d2["v"], d2["alpha"], d2["beta"],
                                     nthreads=cores))
    per["cfg2_gdn_64k"] = {"value": round(16384 / dt, 1), "unit": "tokens/s",
                           "sample": f"the first 16384 tokens of all 16 heads, {dt:.2f} s"}
    del d2
    # cfg4: 16 consecutive decode steps of all 4096 states, as one recurrence per state
    N, n = 4096, 16
    g = synth.gdn_decode_inputs(n, N, 128, 128, seed=4)
    S = synth.gdn_state((N, 128, 128), seed=4)
    tq = lambda t: t.transpose(0, 1).contiguous()[None]
    dt = wall(lambda: oracle.prefill("gated_delta", tq(g["q"]), tq(g["k"]), tq(g["v"]), tq(g["alpha"]),
                                     tq(g["beta"]), S0=S[None], nthreads=cores))
    per["cfg4_decode_gated_delta"] = {"value": round(n / dt, 2), "unit": "steps/s",
                                      "sample": f"{n} steps of all {N} states, {dt:.2f} s"}
    bd = synth.based_decode_inputs(n, N, 16, 64, seed=5)
    w = synth.based_warmup_inputs(N, 64, 16, 64, seed=4)
    _, s0, z0 = oracle.prefill("based", w["q"][None], w["k"][None], w["v"][None], nthreads=cores)
    dt = wall(lambda: oracle.prefill("based", tq(bd["q"]), tq(bd["k"]), tq(bd["v"]), S0=s0, z0=z0,
                                     nthreads=cores))
    per["cfg4_decode_based"] = {"value": round(n / dt, 2), "unit": "steps/s",
                                "sample": f"{n} steps of all {N} states, {dt:.2f} s"}
    del g, S, bd, w

    # cfg3 (headline): a prefix of the 16-head sequence, grown to about target_s
    def run3(Ts):
        d = synth.gdn_inputs(1, 16, Ts, 128, 128, seed=3)
        return wall(lambda: oracle.prefill("gated_delta", d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                           nthreads=cores))
    Ts = 4096
    dt = run3(Ts)
    Ts2 = int(min(max(Ts * target_s / max(dt, 1e-3), Ts), 1 << 20)) // 64 * 64
    if Ts2 > Ts:
        Ts, dt = Ts2, run3(Ts2)
    per["cfg3_gdn_1m"] = {"value": round(Ts / dt, 1), "unit": "tokens/s",
                          "sample": f"the first {Ts} tokens of the 16-head sequence, {dt:.1f} s"}
    head = per["cfg3_gdn_1m"]
    return {"value": head["value"], "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"fp64 oracle on the first {Ts} of the 1,048,576 tokens of the 16-head gated-delta "
                      f"prefill (all 128 value rows, d_k=d_v=128), {dt:.1f} s wall, {cores} threads",
            "per_config": per}


if __name__ == "__main__":
    main()
