#!/usr/bin/env python3
"""Benchmark of the MI355X linear-attention recurrence library (one GPU).

Headline workload: gated-delta chunkwise prefill of one layer, B = 1, H = 16,
T = 1,048,576, d_k = d_v = 128, bf16 q/k/v/alpha/beta, fp32 state, seeded synthetic
inputs with the gated-delta recipe (synth.gdn_inputs).  One step = one complete
la_prefill over the whole sequence (its four passes: per-chunk UT transforms, segment
maps, segment scan, replay).
value = tokens/s, a token being one position through all 16 heads.

Also measured in the same run: the batched decode step (256 sequences x 16 heads,
gated-delta state 128 x 128 and BASED state 273 x 64 per head, 1024 consecutive steps),
and the fp64 oracle on a bounded sample of the prefill workload on the host cores.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-decode]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "prefill tokens/sec (GDN, T=1M) + decode steps/sec, 1×MI355X, % of roofline"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published
PROFILE_COUNTERS = ROOT / "profiles" / "gdn_prefill_1m_counters.txt"

# algorithmic work per token-head of the gated-delta prefill at chunk 64, d = 128:
# bytes: q, k, v (3 x 128 x 2) + alpha, beta (2 x 2) + o (128 x 2)
BYTES_PER_TOKEN_HEAD = 3 * 128 * 2 + 2 * 2 + 128 * 2          # 1028
# FLOPs of the chunk form (multiply-add = 2): Grams K K^T and Q K^T, W, U~, A U
# (5 x 2 C^2 d), W S^T, Q S^T, state update (3 x 2 C d^2), triangular solve (C^3 / 3)
C_, D_ = 64, 128
FLOPS_PER_TOKEN_HEAD = (5 * 2 * C_ * C_ * D_ + 3 * 2 * C_ * D_ * D_ + C_ ** 3 / 3) / C_


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
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
    B, H, T, D = 1, args.heads, args.seq_len, 128

    if args.calibrate_copy:  # copy_or_zero_kernel: reads and writes exactly 256 MiB
        e = torch.empty((1, 4096, 0, 128), dtype=torch.bfloat16, device=dev)
        ea = torch.empty((1, 4096, 0), dtype=torch.bfloat16, device=dev)
        S0c = torch.randn((1, 4096, 128, 128), device=dev)
        la.prefill("gated_delta", e, e, e, ea, ea, S0=S0c)
        torch.cuda.synchronize()
        del S0c

    # ---------------------------------------------------------------- prefill
    inp = synth.gdn_inputs(B, H, T, D, D, dtype=torch.bfloat16, seed=3, device=dev)
    q, k, v, a, b = inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"]
    o = torch.empty((B, H, T, D), dtype=torch.bfloat16, device=dev)
    S_T = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    ws_n = la.workspace_size("gated_delta", la.BF16, B, H, T, D, D)
    ws = torch.empty(max(ws_n, 16), dtype=torch.uint8, device=dev)
    nseg, seg_chunks = la.segments("gated_delta", la.BF16, B, H, T, D, D)
    passes = [la.PASS_TRANSFORM, la.PASS_MAPS, la.PASS_SCAN, la.PASS_REPLAY] if nseg > 1 \
        else [la.PASS_TRANSFORM, la.PASS_REPLAY]
    names = {la.PASS_TRANSFORM: "transform", la.PASS_MAPS: "maps", la.PASS_SCAN: "scan",
             la.PASS_REPLAY: "replay"}

    def step(evs=None):
        for i, p in enumerate(passes):
            la.prefill("gated_delta", q, k, v, a, b, o=o, S_T=S_T, workspace=ws, pass_=p,
                       stream=stream)
            if evs is not None:
                evs[i + 1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    per_pass = {names[p]: 0.0 for p in passes}
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    all_evs = []
    t_start.record(stream)
    for _ in range(args.steps):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(passes) + 1)]
        evs[0].record(stream)
        step(evs)
        all_evs.append(evs)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    for evs in all_evs:
        for i, p in enumerate(passes):
            per_pass[names[p]] += evs[i].elapsed_time(evs[i + 1]) / args.steps
    ms_per_step = total_ms / args.steps
    tokens_per_s = B * T / (ms_per_step * 1e-3)
    token_heads = B * H * T
    alg_bytes = token_heads * BYTES_PER_TOKEN_HEAD
    alg_flops = token_heads * FLOPS_PER_TOKEN_HEAD

    # the dominant launch of the step, with the algorithmic bytes and FLOPs of that pass
    # (per token-head, C = 64, d = 128; a stored transform is 6 KB per chunk = 96 B per token):
    #   transform: k, alpha, beta in, the transform out (356 B); K K^T and the solve
    #              (2 C d + C^2 / 3 FLOP); every chunk
    #   maps:      k, v, alpha, beta, transform in (612 B); K S^T, TB Y (2 C d + C^2) and the
    #              state update for 256 state rows, B_seg and M_seg; every segment but the last
    #   scan:      per segment but the last, its 256 x 128 map read; every start state written;
    #              a 128 x 128 x 128 product per segment
    #   replay:    q, k, v, alpha, beta, transform in, o out (1124 B); Q K^T, A U, TB Y
    #              (4 x 2 C d) and K S^T, Q S^T, the state update (3 x 2 d^2); every chunk
    dom = max(per_pass, key=per_pass.get)
    map_frac = (nseg - 1) / nseg
    per_th = {"transform": (128 * 2 + 2 * 2 + 96, 2 * C_ * D_ + C_ * C_ / 3, 1.0),
              "maps": (2 * 128 * 2 + 2 * 2 + 96, 2 * 2 * C_ * D_ + 4 * 2 * D_ * D_, map_frac),
              "replay": (BYTES_PER_TOKEN_HEAD + 96, 4 * 2 * C_ * D_ + 3 * 2 * D_ * D_, 1.0)}
    pass_bytes = {kk: token_heads * vv[0] * vv[2] for kk, vv in per_th.items()}
    pass_flops = {kk: token_heads * vv[1] * vv[2] for kk, vv in per_th.items()}
    pass_bytes["scan"] = B * H * ((nseg - 1) * 2 * D * D * 4 + nseg * D * D * 4)
    pass_flops["scan"] = B * H * (nseg - 1) * 2 * D * D * D
    t_dom = per_pass[dom] * 1e-3
    t_hbm = pass_bytes[dom] / (HBM_PEAK_GBS * 1e9)
    t_mfma = pass_flops[dom] / (BF16_PEAK_TFLOPS * 1e12)
    if t_hbm >= t_mfma:
        ach, peak, unit, bound = pass_bytes[dom] / t_dom / 1e9, HBM_PEAK_GBS, "GB/s", "hbm"
    else:
        ach, peak, unit, bound = pass_flops[dom] / t_dom / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s", "mfma"
    kname = {"replay": "replay_kernel<true> (replay pass)",
             "maps": "map_kernel<true> (segment-map pass)",
             "transform": "tprep_kernel (per-chunk UT transform pass)",
             "scan": "scan_delta_kernel (segment scan)"}[dom]
    roofline = {
        "bound": bound, "achieved": round(ach, 1), "peak": peak, "unit": unit,
        "frac": round(ach / peak, 4), "traffic": read_traffic(dom), "kernel": kname,
        "ms_per_launch": round(per_pass[dom], 4),
        "alg_bytes_per_launch": pass_bytes[dom], "alg_flops_per_launch": pass_flops[dom],
    }
    prefill_detail = {
        "ms_per_pass": {kk: round(vv, 4) for kk, vv in per_pass.items()},
        "segments": nseg, "chunks_per_segment": seg_chunks,
        "alg_bytes": alg_bytes, "alg_flops": alg_flops,
        "hbm_frac_whole_step": round(alg_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "bf16_mfma_frac_whole_step": round(alg_flops / (ms_per_step * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
        "roofline_time_ms": round(max(alg_bytes / (HBM_PEAK_GBS * 1e9),
                                      alg_flops / (BF16_PEAK_TFLOPS * 1e12)) * 1e3, 4),
    }
    prefill_detail["roofline_frac_whole_step"] = round(prefill_detail["roofline_time_ms"] / ms_per_step, 4)

    # host copy of a prefix of the same inputs for the CPU oracle sample
    host = None
    if not args.no_cpu_baseline:
        Tmax = min(T, 1 << 19)
        host = {n: t[:, :, :Tmax].cpu() for n, t in inp.items()}

    # ---------------------------------------------------------------- decode
    decode = None
    del inp, q, k, v, a, b, o, ws
    torch.cuda.empty_cache()
    if not args.no_decode:
        decode = bench_decode(torch, la, synth, dev, stream, args.decode_steps)

    # ---------------------------------------------------------------- d = 256 gated delta
    gdn256 = None
    if not args.no_d256:
        gdn256 = bench_gdn256(torch, la, synth, dev, stream, args.steps, args.warmup, args.seq_len)

    # ---------------------------------------------------------------- the two smaller configs
    small = None
    if not args.no_small:
        small = bench_small_configs(torch, la, synth, dev, stream)

    # ---------------------------------------------------------------- BASED prefill
    based = None
    if not args.no_based:
        based = bench_based(torch, la, synth, dev, stream, args.steps)
        based["compact"] = bench_based(torch, la, synth, dev, stream, args.steps, "based_compact")

    # ---------------------------------------------------------------- NoteBank steps
    notebank = None
    if not args.no_notebank:
        notebank = bench_notebank(torch, la, synth, dev, stream)

    # ---------------------------------------------------------------- CPU oracle
    cpu = None
    if not args.no_cpu_baseline:
        cpu = bench_cpu(host, H, D, args.cpu_seconds)

    out = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"gated-delta chunkwise prefill, B={B} H={H} T={T} d_k=d_v={D}, "
                               "bf16 inputs, fp32 state, chunk 64", "batch": B, "heads": H,
                   "seq_len": T, "d_k": D, "d_v": D, "chunk": 64, "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "prefill": prefill_detail,
        "decode": decode,
        "gdn_d256": gdn256,
        "small_configs": small,
        "based_prefill": based,
        "notebank": notebank,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_small_configs(torch, la, synth, dev, stream):
    """The two smaller configurations: additive linear attention in fp32 (B=1, H=1, T=1024,
    d=64: one head, so launch latency bounds it) and the gated-delta prefill at 64K tokens
    (B=1, H=16, T=65536, d=128, bf16), each as la_prefill calls timed with HIP events."""
    def timed(fn, n):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n
    res = {}
    d0 = synth.additive_inputs(1, 1, 1024, 64, dtype=torch.float32, seed=0, device=dev)
    o0 = torch.empty_like(d0["v"])
    S0 = torch.empty((1, 1, 64, 64), dtype=torch.float32, device=dev)
    ms0 = timed(lambda: la.prefill("additive", d0["q"], d0["k"], d0["v"], o=o0, S_T=S0, stream=stream), 200)
    res["additive_fp32"] = {"workload": "additive linear attention, B=1 H=1 T=1024 d=64, fp32",
                            "us_per_call": round(ms0 * 1e3, 2), "tokens_per_s": round(1024 / (ms0 * 1e-3), 1)}
    B, H, T, D = 1, 16, 65536, 128
    g = synth.gdn_inputs(B, H, T, D, D, dtype=torch.bfloat16, seed=2, device=dev)
    o2 = torch.empty_like(g["v"])
    S2 = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    ws = torch.empty(max(la.workspace_size("gated_delta", la.BF16, B, H, T, D, D), 16), dtype=torch.uint8, device=dev)
    ms2 = timed(lambda: la.prefill("gated_delta", g["q"], g["k"], g["v"], g["alpha"], g["beta"], o=o2, S_T=S2,
                                   workspace=ws, stream=stream), 20)
    byt = B * H * T * BYTES_PER_TOKEN_HEAD
    flo = B * H * T * FLOPS_PER_TOKEN_HEAD
    t_roof = max(byt / (HBM_PEAK_GBS * 1e9), flo / (BF16_PEAK_TFLOPS * 1e12))
    nseg, sc = la.segments("gated_delta", la.BF16, B, H, T, D, D)
    res["gdn_64k"] = {"workload": "gated-delta chunkwise prefill, B=1 H=16 T=65536 d_k=d_v=128, bf16, chunk 64",
                      "ms": round(ms2, 4), "tokens_per_s": round(T / (ms2 * 1e-3), 1), "segments": nseg,
                      "chunks_per_segment": sc, "alg_bytes": byt, "alg_flops": flo,
                      "roofline_time_ms": round(t_roof * 1e3, 4), "roofline_frac": round(t_roof * 1e3 / ms2, 4)}
    return res


def bench_gdn256(torch, la, synth, dev, stream, steps, warmup, T):
    """The gated-delta shape of the NoteBank paper's own backbone: 8 heads of width 256
    (d_k = d_v = 256, fp32 state 256 x 256 per head), bf16 inputs with the gated-delta
    recipe, T tokens (1M by default): the four passes timed with HIP events on the launch
    stream; then the decode step on 256 sequences x 8 heads of that width."""
    B, H, D = 1, 8, 256
    inp = synth.gdn_inputs(B, H, T, D, D, dtype=torch.bfloat16, seed=6, device=dev)
    q, k, v, a, b = inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"]
    o = torch.empty((B, H, T, D), dtype=torch.bfloat16, device=dev)
    S_T = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    ws = torch.empty(max(la.workspace_size("gated_delta", la.BF16, B, H, T, D, D), 16), dtype=torch.uint8,
                     device=dev)
    nseg, sc = la.segments("gated_delta", la.BF16, B, H, T, D, D)
    passes = [la.PASS_TRANSFORM, la.PASS_MAPS, la.PASS_SCAN, la.PASS_REPLAY] if nseg > 1 \
        else [la.PASS_TRANSFORM, la.PASS_REPLAY]
    names = {la.PASS_TRANSFORM: "transform", la.PASS_MAPS: "maps", la.PASS_SCAN: "scan",
             la.PASS_REPLAY: "replay"}

    def run(evs=None):
        for i, p in enumerate(passes):
            la.prefill("gated_delta", q, k, v, a, b, o=o, S_T=S_T, workspace=ws, pass_=p, stream=stream)
            if evs is not None:
                evs[i + 1].record(stream)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    per_pass = {names[p]: 0.0 for p in passes}
    total = 0.0
    for _ in range(steps):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(passes) + 1)]
        evs[0].record(stream)
        run(evs)
        torch.cuda.synchronize()
        total += evs[0].elapsed_time(evs[-1]) / steps
        for i, p in enumerate(passes):
            per_pass[names[p]] += evs[i].elapsed_time(evs[i + 1]) / steps
    # algorithmic work per token-head at d = 256, chunk 64 (as for d = 128): q, k, v, o and
    # the two gates; chunk-form FLOPs 5 x 2 C^2 d + 3 x 2 C d^2 + C^3 / 3 per chunk
    th = B * H * T
    byt = th * (4 * D * 2 + 2 * 2)
    flo = th * (5 * 2 * C_ * C_ * D + 3 * 2 * C_ * D * D + C_ ** 3 / 3) / C_
    t_roof = max(byt / (HBM_PEAK_GBS * 1e9), flo / (BF16_PEAK_TFLOPS * 1e12))
    # the replay reads q, k, v, the gates and the stored transform (96 B per token) and writes o
    rep_b = th * (4 * D * 2 + 2 * 2 + 96)
    res = {"workload": f"gated-delta chunkwise prefill, B={B} H={H} T={T} d_k=d_v={D}, bf16 inputs, "
                       "fp32 state, chunk 64",
           "ms": round(total, 4), "tokens_per_s": round(B * T / (total * 1e-3), 1),
           "ms_per_pass": {kk: round(vv, 4) for kk, vv in per_pass.items()},
           "segments": nseg, "chunks_per_segment": sc, "alg_bytes": byt, "alg_flops": flo,
           "roofline_time_ms": round(t_roof * 1e3, 4), "roofline_frac": round(t_roof * 1e3 / total, 4),
           "bf16_mfma_frac": round(flo / (total * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
           "replay_hbm_frac": round(rep_b / (per_pass["replay"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "replay_traffic": read_traffic("d256_replay")}
    # the recurrence's share of the pages' 24-layer GDN at this length: 24 whole-layer
    # prefills back to back (each layer reuses these inputs; projections, convolutions and
    # the other layer parts are outside the recurrence)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(24):
        la.prefill("gated_delta", q, k, v, a, b, o=o, S_T=S_T, workspace=ws, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    res["stack_24_layers_ms"] = round(e0.elapsed_time(e1), 3)
    del inp, q, k, v, a, b, o, ws
    torch.cuda.empty_cache()

    N, nsteps = 256 * 8, 256
    S = synth.gdn_state((N, D, D), seed=7, device=dev)
    g = synth.gdn_decode_inputs(nsteps, N, D, D, dtype=torch.bfloat16, seed=7, device=dev)
    od = torch.empty((N, D), dtype=torch.bfloat16, device=dev)
    step = lambda t: la.decode_step("gated_delta", S, g["q"][t], g["k"][t], g["v"][t], g["alpha"][t],
                                    g["beta"][t], S_out=S, o=od, stream=stream)
    for t in range(8):
        step(t)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for t in range(nsteps):
        step(t)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / nsteps
    bd = 2 * N * D * D * 4 + N * (3 * D + 2 + D) * 2
    res["decode"] = {"states": N, "steps": nsteps, "us_per_step": round(ms * 1e3, 2),
                     "steps_per_s": round(1e3 / ms, 1), "alg_bytes_per_step": bd,
                     "hbm_frac": round(bd / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    return res


def bench_decode(torch, la, synth, dev, stream, steps):
    """256 sequences x 16 heads; gated-delta and BASED decode (and BASED with the compact
    153-feature state), `steps` consecutive steps."""
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

    def gdn_step(t):
        la.decode_step("gated_delta", S, g["q"][t], g["k"][t], g["v"][t], g["alpha"][t],
                       g["beta"][t], S_out=S, o=o, stream=stream)

    def based_step(t):
        la.decode_step("based", s, bd["q"][t], bd["k"][t], bd["v"][t], z=z, S_out=s, z_out=z,
                       o=ob, stream=stream)

    def compact_step(t):
        la.decode_step("based_compact", sc, bd["q"][t], bd["k"][t], bd["v"][t], z=zc, S_out=sc,
                       z_out=zc, o=ob, stream=stream)

    def timed(fn):
        for t in range(8):
            fn(t)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for t in range(steps):
            fn(t)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms_g = timed(gdn_step)
    ms_b = timed(based_step)
    ms_c = timed(compact_step)
    bytes_g = 2 * N * D * D * 4 + N * (3 * D + 2 + D) * 2
    bytes_b = 2 * N * (Dphi * dv_b + Dphi) * 4 + N * (2 * dp + 2 * dv_b) * 2
    res["gated_delta"] = {"us_per_step": round(ms_g * 1e3, 2), "steps_per_s": round(1e3 / ms_g, 1),
                          "alg_bytes_per_step": bytes_g,
                          "hbm_frac": round(bytes_g / (ms_g * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    res["based"] = {"us_per_step": round(ms_b * 1e3, 2), "steps_per_s": round(1e3 / ms_b, 1),
                    "alg_bytes_per_step": bytes_b,
                    "hbm_frac": round(bytes_b / (ms_b * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    bytes_c = 2 * N * (Dc * dv_b + Dc) * 4 + N * (2 * dp + 2 * dv_b) * 2
    res["based_compact"] = {"us_per_step": round(ms_c * 1e3, 2), "steps_per_s": round(1e3 / ms_c, 1),
                            "alg_bytes_per_step": bytes_c, "state_features": Dc,
                            "hbm_frac": round(bytes_c / (ms_c * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    res["both_steps_per_s"] = round(1e3 / (ms_g + ms_b), 1)
    return res


def bench_based(torch, la, synth, dev, stream, steps, variant="based"):
    """BASED Taylor prefill, B=4, H=16, T=8192, d'=16, d_v=64, bf16 (all three passes); the
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
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = max(steps, 10)
    e0.record(stream)
    for _ in range(n):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    th = B * H * T
    alg_bytes = th * (2 * dp * 2 + 2 * dv * 2) + 2 * B * H * Dphi * (dv + 1) * 4
    C = 64  # chunk-form FLOPs per token-head: QK^T, A V, Phi_Q s, Phi_K^T V, normaliser
    alg_flops = th * (2 * C * dp + 2 * C * dv + 4 * Dphi * dv + 2 * Dphi + C)
    t_roof = max(alg_bytes / (HBM_PEAK_GBS * 1e9), alg_flops / (BF16_PEAK_TFLOPS * 1e12))
    nseg, sc = la.segments(variant, la.BF16, B, H, T, dp, dv)
    return {"workload": f"BASED Taylor prefill B=4 H=16 T=8192 d'=16 d_v=64 bf16, {Dphi}-feature state",
            "ms": round(ms, 4), "tokens_per_s": round(B * T / (ms * 1e-3), 1),
            "alg_bytes": alg_bytes, "alg_flops": alg_flops, "segments": nseg,
            "roofline_time_ms": round(t_roof * 1e3, 4), "roofline_frac": round(t_roof * 1e3 / ms, 4)}


def bench_notebank(torch, la, synth, dev, stream):
    """NoteBank write scoring over the 1M-token, 16-head keys (512-token write chunks, 48-token
    windows, 32-token tails) and addressing at the pages' archive size (4092 notes, 192 channels,
    d_rho = 16, a 128-token question, R = 8)."""
    B, H, T, D = 1, 16, 1 << 20, 128
    k = synth.gdn_inputs(B, H, T, D, D, dtype=torch.bfloat16, seed=3, device=dev)["k"]
    d_head = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    d_mean = torch.empty((B, T), dtype=torch.float32, device=dev)

    def timed(fn, n=10):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    ms_s = timed(lambda: la.write_scores(k, 512, d_head=d_head, d_mean=d_mean, stream=stream))
    ms_w = timed(lambda: la.write_windows(d_mean, 512, 48, 32, stream=stream))
    bytes_s = B * H * T * (D * 2 + 4) + B * T * 4 + B * H * T * 4  # keys, d_head out, d_mean (read H rows, write 1)
    del k
    N, J, nQ, dr, R = 4092, 192, 128, 16, 8
    g = torch.Generator(device=dev).manual_seed(11)
    rho = torch.randn((N, J, dr), generator=g, device=dev).to(torch.bfloat16)
    u = torch.randn((nQ, J, dr), generator=g, device=dev).to(torch.bfloat16)
    pos = torch.arange(N, dtype=torch.int64, device=dev) * 256
    ms_v = timed(lambda: la.address_votes(rho, u, R, pos, want_score=False, stream=stream))
    flops_v = 2 * nQ * N * J * dr
    return {"write_scores": {"workload": "keys B=1 H=16 T=1048576 d_k=128 bf16, 512-token write chunks",
                             "ms": round(ms_s, 4), "alg_bytes": bytes_s,
                             "hbm_frac": round(bytes_s / (ms_s * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
            "write_windows": {"ms": round(ms_w, 4), "chunks": T // 512},
            "address_votes": {"workload": f"{N} notes x {J} channels, d_rho={dr}, {nQ}-token question, R={R}",
                              "ms": round(ms_v, 4), "alg_flops": flops_v,
                              "fp32_vector_frac": round(flops_v / (ms_v * 1e-3) / 157.3e12, 4)}}


def bench_cpu(host, H, D, target_s):
    """The fp64 oracle, as it is, on the first T_s tokens of the same 16-head sequence (all
    value rows, the same input values the GPU ran on), on this host's cores; T_s is grown
    until the run takes about target_s."""
    import oracle

    cores = len(os.sched_getaffinity(0))
    oracle._load()
    Tmax = host["q"].shape[2]

    def run(Ts):
        d = {n: t[:, :, :Ts] for n, t in host.items()}
        t0 = time.perf_counter()
        oracle.prefill("gated_delta", d["q"], d["k"], d["v"], d["alpha"], d["beta"], nthreads=cores)
        return time.perf_counter() - t0

    Ts = min(2048, Tmax)
    dt = run(Ts)
    Ts2 = int(min(max(Ts * target_s / max(dt, 1e-3), Ts), Tmax)) // 64 * 64
    if Ts2 == Ts:
        return {"value": round(Ts / dt, 1), "unit": "tokens/s", "cores": cores, "kind": "oracle",
                "sample": f"fp64 oracle on the first {Ts} tokens of the {H}-head gated-delta "
                          f"sequence (all 128 value rows, d_k=d_v={D}), {dt:.1f} s wall"}
    dt2 = run(Ts2)
    return {"value": round(Ts2 / dt2, 1), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"fp64 oracle on the first {Ts2} tokens of the {H}-head gated-delta "
                      f"sequence (all 128 value rows, d_k=d_v={D}), {dt2:.1f} s wall"}


if __name__ == "__main__":
    main()
