#!/usr/bin/env python3
"""Benchmark of the SwiAttn routed hot path on one MI355X.

One step = the whole hot path on one batch of synthetic input:
  router over the hidden states of a 32K-token sequence -> hard gate ->
  compaction of the full-branch tokens -> routed prefill (window branch for
  every row, far part of the full branch for the gathered rows, log-sum-exp
  merge) at N=32768, 16 query / 4 KV heads, d=128, W=1024, bf16;
  then one routed decode step for 64 sequences on a 32768-token shared bf16
  KV cache (16/4 heads, d=128, W=1024, per-sequence gate Bernoulli(0.13)).

The router inputs are H ~ N(0,1), r ~ N(0, 1/2048) and a bias set for a 13%
full-branch fraction; the hidden rows are i.i.d., so the gate bits are
i.i.d. Bernoulli(0.13).  Inputs are synthetic and seeded; they stand in for
the evaluation data of the SwiAttn report, which needs trained weights.

Prints ONE JSON line.  `value` is the routed prefill's useful TFLOP/s
(4*d per attended (query head, key) pair at the realized gate, timed from
the router to the merge); decode tokens/s and GB/s are reported beside it.
`roofline` covers the kernel with the largest share of the step's time,
timed with HIP events recorded on its launch stream inside the library;
its `traffic` (HBM bytes per launch) comes from the committed rocprofv3
counter summary under profiles/ and is null when the kernel sources have
changed since those counters were taken.
`cpu_baseline` times the float64 CPU reference on a bounded sample of the
same workload.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA

ROOT = os.path.dirname(os.path.abspath(__file__))
# rocprofv3 counter summary of this benchmark (FETCH_SIZE / WRITE_SIZE per
# dispatch, scaled by the counts of a plain copy of known size)
PROFILE = os.path.join(ROOT, "profiles", "kernels_prefill32k_decode64x32k.md")
# bench kernel key -> kernel function name in the profile
PROFILE_NAMES = {"attn": "attn_kernel", "decode_splitk": "decode_kernel"}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="time budget of the CPU reference sample (0 = skip)")
    ap.add_argument("--p", type=float, default=0.13, help="full-branch fraction")
    ap.add_argument("--serve-steps", type=int, default=20,
                    help="timed serving decode steps (route + append + decode; after the timed steps; 0 = skip)")
    ap.add_argument("--both-steps", type=int, default=3,
                    help="timed runs of the both-branch prefill (after the timed steps; 0 = skip)")
    ap.add_argument("--anchor-steps", type=int, default=10,
                    help="timed runs of the anchored prefill and decode (after the timed steps; 0 = skip)")
    ap.add_argument("--anchors", type=int, default=256,
                    help="global anchor keys of the window branch in the anchored runs")
    ap.add_argument("--rgrad-steps", type=int, default=10,
                    help="timed runs of the router gradient (after the timed steps; 0 = skip)")
    ap.add_argument("--bwd-steps", type=int, default=10,
                    help="timed runs of the attention backward (after the timed steps; 0 = skip)")
    ap.add_argument("--extra-steps", type=int, default=5,
                    help="timed runs of each extra configuration (layer, gate bounds, structured routing, "
                         "decode densities; after the timed steps; 0 = skip)")
    ap.add_argument("--stage-steps", type=int, default=20,
                    help="steps run after the timed ones with the library's stage events, for the "
                         "per-kernel times")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="run one plain device-to-device copy of this many MiB before the steps "
                         "(a known-size reference for hardware byte counters)")
    return ap.parse_args()


# ------------------------------------------------------------------ accounting
def prefill_pairs(gate, W, Hq, G, A=0):
    """Attended (query head, key) pairs: full rows see i+1 keys, window rows
    min(i+1, W) plus min(A, i-W+1) anchors when i-W+1 > 0.  Returns (useful
    total, window part, far part)."""
    B, N, _ = gate.shape
    i = np.arange(N, dtype=np.int64)
    band = np.minimum(i + 1, W) + np.minimum(A, np.maximum(i - W + 1, 0))
    far = i + 1 - band
    tot_b = tot_f = 0
    for h in range(Hq):
        g = gate[:, :, h * G // Hq].astype(bool)
        tot_b += int(band.sum()) * B
        tot_f += int((far[None, :] * g).sum())
    return tot_b + tot_f, tot_b, tot_f


def decode_bytes(gate, cache_len, W, Hq, Hkv, d, elem=2, A=0):
    """Algorithmic HBM bytes of one decode step: every attended key and value
    row of a KV head is read once for its Hq/Hkv query heads, plus q and o
    (a window pair also reads its min(A, L-W) anchors)."""
    B, G = gate.shape
    HK = Hq // Hkv
    keys = 0
    for b in range(B):
        L = int(cache_len[b])
        for kv in range(Hkv):
            full = any(gate[b, (kv * HK + j) * G // Hq] for j in range(HK))
            keys += L if full else min(L, W) + min(A, max(0, L - W))
    return keys * d * 2 * elem + B * Hq * d * 2 * elem, keys


def kernel_source_hash():
    """sha256 over the kernel sources, file by file in byte order of their paths."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "sliding_window_attention_router_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def profiled_traffic(path=PROFILE):
    """HBM bytes per launch by kernel name, from the committed counter
    summary; empty when the summary was taken on other kernel sources."""
    if not os.path.exists(path):
        return {}
    text = open(path, encoding="utf-8").read()
    m = [ln for ln in text.splitlines() if ln.startswith("kernel sources sha256:")]
    if not m or m[0].split(":", 1)[1].strip().strip("`") != kernel_source_hash():
        return {}
    out = {}
    section = text.split("## HBM traffic", 1)[-1].split("\n## ", 1)[0] if "## HBM traffic" in text else ""
    for ln in section.splitlines():
        cells = [c.strip().strip("`") for c in ln.strip().strip("|").split("|")]
        if len(cells) >= 5 and cells[0] in PROFILE_NAMES.values():
            try:
                out[cells[0]] = float(cells[4])
            except ValueError:
                pass
    return out


# ------------------------------------------------------------------ main
def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (got --gpus {args.gpus}); "
              "the multi-GPU sharding is described but not implemented.", file=sys.stderr)
        sys.exit(2)
    import torch

    import sliding_window_attention_router_amd as swa
    from sliding_window_attention_router_amd import binding, synth

    if not os.path.exists(binding.LIB_PATH):
        from sliding_window_attention_router_amd import build

        build.build()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    N, Hq, Hkv, d, W, hidden = 32768, 16, 4, 128, 1024, 2048
    B_dec, L_dec = 64, 32768
    t0 = time.time()
    pre = synth.long_prefill(seed=3, N=N, Hq=Hq, Hkv=Hkv, d=d, W=W, p=args.p, with_router=True,
                             hidden=hidden)
    bf = torch.bfloat16
    Q = torch.from_numpy(pre.Q).to(bf).to(dev)
    K = torch.from_numpy(pre.K).to(bf).to(dev)
    V = torch.from_numpy(pre.V).to(bf).to(dev)
    H = torch.from_numpy(pre.H).to(bf).to(dev)
    r = torch.from_numpy(pre.r).to(bf).to(dev)
    bias = torch.from_numpy(pre.bias).to(dev)
    dec = synth.decode_cache(seed=5, B=B_dec, Lmax=L_dec, Hq=Hq, Hkv=Hkv, d=d, W=W, p=args.p,
                             device=dev)
    q_d, Kc, Vc = dec["q"], dec["Kc"], dec["Vc"]
    gate_d = torch.from_numpy(dec["gate"]).to(dev)
    len_d = torch.from_numpy(dec["cache_len"]).to(dev)
    print(f"[bench] inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    G = 1
    gate = torch.empty((1, N, G), dtype=torch.uint8, device=dev)
    idx = torch.empty((1, G, N), dtype=torch.int32, device=dev)
    cnt = torch.empty((1, G), dtype=torch.int32, device=dev)
    O = torch.empty_like(Q)
    o_d = torch.empty_like(q_d)
    ws_p = torch.empty(swa.prefill_workspace_size(1, N, Hq, Hkv, G, d, W), dtype=torch.uint8, device=dev)
    ws_d = torch.empty(swa.decode_workspace_size(B_dec, L_dec, Hq, Hkv, G, d, W), dtype=torch.uint8,
                       device=dev)

    def new_events(n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in evs:
            e.record()
        return evs

    def step(ev=None):
        # ev: 3 events: [route start, prefill end = decode start, decode end]
        if ev is not None:
            ev[0].record()
        swa.route(H, r, bias, out=(gate, idx, cnt))
        swa.prefill(Q, K, V, gate, W, idx=idx, cnt=cnt, out=O, workspace=ws_p)
        if ev is not None:
            ev[1].record()
        swa.decode(q_d, Kc, Vc, len_d, gate_d, W, out=o_d, workspace=ws_d)
        if ev is not None:
            ev[2].record()

    def staged_step(ev):
        # ev: 9 events: [route start] + prefill stages 0..3 + decode stages 0..2 + [end]
        ev[0].record()
        swa.route(H, r, bias, out=(gate, idx, cnt))
        swa.prefill(Q, K, V, gate, W, idx=idx, cnt=cnt, out=O, workspace=ws_p, events=ev[1:5])
        swa.decode(q_d, Kc, Vc, len_d, gate_d, W, out=o_d, workspace=ws_d, events=ev[5:8])
        ev[8].record()

    if args.copy_mib > 0:
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evsets = [new_events(3) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(args.steps):
        step(evsets[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    print(f"[bench] {args.steps} timed steps in {wall:.3f}s", file=sys.stderr, flush=True)
    prefill_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evsets]))
    decode_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evsets]))
    step_ms = wall * 1e3 / args.steps

    # Per-kernel times from further steps with the library's stage events
    # (each event between two launches lengthens the step by a few us, so
    # the timed steps above carry none).
    stsets = [new_events(9) for _ in range(max(1, args.stage_steps))]
    torch.cuda.synchronize()
    for ev in stsets:
        staged_step(ev)
    torch.cuda.synchronize()

    def avg(i, j):
        return float(np.mean([e[i].elapsed_time(e[j]) for e in stsets]))

    t = {
        "route_compact": avg(0, 1),
        "far_schedule": avg(1, 2),
        "attn": avg(2, 3),
        "merge": avg(3, 4),
        "decode_splitk": avg(5, 6),
        "decode_merge": avg(6, 7),
    }

    g_host = gate.cpu().numpy()
    useful, band_pairs, far_pairs = prefill_pairs(g_host, W, Hq, G)
    fl = 4.0 * d
    prefill_tflops = useful * fl / (prefill_ms * 1e-3) / 1e12
    dbytes, dkeys = decode_bytes(dec["gate"], dec["cache_len"], W, Hq, Hkv, d)
    decode_gbs = dbytes / (decode_ms * 1e-3) / 1e9
    decode_tok_s = B_dec / (decode_ms * 1e-3)

    kern = {
        "attn": {"bound": "mfma", "work": useful * fl, "unit": "TFLOP/s", "peak": BF16_PEAK_TFLOPS},
        "decode_splitk": {"bound": "hbm", "work": dbytes, "unit": "GB/s", "peak": HBM_PEAK_GBS},
    }
    rooflines = {}
    traffic = profiled_traffic()
    for name, k in kern.items():
        ms = t[name]
        scale = 1e12 if k["unit"] == "TFLOP/s" else 1e9
        ach = k["work"] / (ms * 1e-3) / scale
        rooflines[name] = {"bound": k["bound"], "achieved": round(ach, 2), "peak": k["peak"],
                           "unit": k["unit"], "frac": round(ach / k["peak"], 4), "ms": round(ms, 4),
                           "traffic": traffic.get(PROFILE_NAMES[name])}
    dominant = max(kern, key=lambda n: t[n])

    both = (both_branch_run(swa, Q, K, V, gate, W, args.both_steps, H, r, bias)
            if args.both_steps > 0 else None)
    serve = (serve_run(swa, q_d, Kc, Vc, len_d, r, bias, W, args.serve_steps)
             if args.serve_steps > 0 else None)
    anch = (anchors_run(swa, Q, K, V, gate, idx, cnt, W, args.anchors, q_d, Kc, Vc, len_d, gate_d,
                        dec, args.anchor_steps)
            if args.anchor_steps > 0 else None)
    rgrad = (router_grad_run(swa, Q, K, V, W, H, r, bias, args.rgrad_steps)
             if args.rgrad_steps > 0 else None)
    bwd = (backward_run(swa, Q, K, V, O, gate, idx, cnt, W, useful, args.bwd_steps)
           if args.bwd_steps > 0 else None)

    extra = {}
    if args.extra_steps > 0:
        extra["layer_4k"] = layer_run(swa, args.extra_steps)
        extra["long_prefill_bounds"] = bounds_run(swa, Q, K, V, W, args.extra_steps)
        extra["structured"] = structured_run(swa, W, args.extra_steps)
        extra["decode_densities"] = decode_sweep(swa, dec, W, args.extra_steps)
        print("[bench] extra configurations done", file=sys.stderr, flush=True)

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(pre, g_host, W, args.cpu_seconds)

    realized_p = float(g_host.mean())
    out = {
        "metric": "routed prefill useful TFLOP/s + decode tok/s, N=32K W=1024, % roofline",
        "value": round(prefill_tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V/H and KV cache; router-made gate, i.i.d. Bernoulli(0.13))",
        "config": {
            "workload": "routed prefill N=32768 Hq=16 Hkv=4 d=128 W=1024 (router on hidden 2048) "
                        "+ routed decode B=64 cache 32768 Hq=16 Hkv=4 d=128 W=1024",
            "prefill": {"B": 1, "N": N, "Hq": Hq, "Hkv": Hkv, "d": d, "W": W, "hidden": hidden,
                        "gate_density": round(realized_p, 5), "useful_pairs": useful,
                        "useful_tflop": round(useful * fl / 1e12, 4), "ms": round(prefill_ms, 4),
                        "frac_of_bf16_peak": round(prefill_tflops / BF16_PEAK_TFLOPS, 4)},
            "decode": {"B": B_dec, "cache_len": L_dec, "Hq": Hq, "Hkv": Hkv, "d": d, "W": W,
                       "full_sequences": int(dec["gate"].sum()), "attended_kv_rows": dkeys,
                       "bytes": dbytes, "ms": round(decode_ms, 4),
                       "tok_per_s": round(decode_tok_s, 1), "GB_per_s": round(decode_gbs, 1),
                       "frac_of_hbm_peak": round(decode_gbs / HBM_PEAK_GBS, 4)},
            "both_branch": both,
            "serving_step": serve,
            "anchors": anch,
            "router_grad": rgrad,
            "attention_backward": bwd,
            **extra,
        },
        "kernel_ms": {k: round(v, 4) for k, v in t.items()},
        "roofline": dict(rooflines[dominant], kernel=dominant),
        "rooflines": rooflines,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


LEAD_CYCLES = 1_000_000  # about 0.4-0.5 ms of GPU clock


def gpu_lead():
    """Keep the GPU busy for a moment ahead of a start event (a bounded spin
    kernel), so that the host's enqueueing of the timed calls, which follows,
    is not inside the timed region: the events then bracket GPU work only,
    as in the back-to-back timed steps."""
    import torch
    torch.cuda._sleep(LEAD_CYCLES)


def time_ms(fn, iters, flush=None):
    """Median and minimum of the time of fn() between two events recorded on
    the launch stream (torch's current stream, which the binding launches
    on); with `flush`, that buffer is rewritten before every run (the write
    also keeps the GPU busy while the run is enqueued), else a spin kernel
    precedes the start event."""
    import torch
    fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(iters):
        if flush is not None:
            flush.fill_(1)
        else:
            gpu_lead()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return float(np.median(ts)), float(np.min(ts))


def layer_run(swa, steps):
    """One SwiAttn layer: the router over hidden states [4096, 2048] (bf16,
    bias for about 13 % full), compaction, then the routed prefill at
    N=4096 with 16 MHA heads, d=128, W=1024.  Route and prefill timed apart
    and together; useful TFLOP/s at the realized gate."""
    import torch
    from sliding_window_attention_router_amd import synth
    dev = torch.device("cuda", 0)
    bf = torch.bfloat16
    w = synth.layer()
    H, r, bias = (torch.from_numpy(w.H).to(bf).to(dev), torch.from_numpy(w.r).to(bf).to(dev),
                  torch.from_numpy(w.bias).to(dev))
    Q, K, V = (torch.from_numpy(x).to(bf).to(dev) for x in (w.Q, w.K, w.V))
    B, N, Hq, d = Q.shape
    G = 1
    gate = torch.empty((B, N, G), dtype=torch.uint8, device=dev)
    idx = torch.empty((B, G, N), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, G), dtype=torch.int32, device=dev)
    O = torch.empty_like(Q)
    ws = torch.empty(swa.prefill_workspace_size(B, N, Hq, K.shape[2], G, d, w.W), dtype=torch.uint8, device=dev)
    route = lambda: swa.route(H, r, bias, out=(gate, idx, cnt))
    pre = lambda: swa.prefill(Q, K, V, gate, w.W, idx=idx, cnt=cnt, out=O, workspace=ws)

    def both():
        route()
        pre()

    t_r, _ = time_ms(route, steps)
    t_p, _ = time_ms(pre, steps)
    t_b, _ = time_ms(both, steps)
    g = gate.cpu().numpy()
    useful = prefill_pairs(g, w.W, Hq, G)[0]
    flop = 4.0 * d * useful
    hbytes = H.numel() * 2
    return {"B": B, "N": N, "Hq": Hq, "Hkv": K.shape[2], "d": d, "W": w.W, "hidden": H.shape[2],
            "gate_density": round(float(g.mean()), 5), "useful_tflop": round(flop / 1e12, 5),
            "route_ms": round(t_r, 4), "route_GB_per_s": round(hbytes / (t_r * 1e-3) / 1e9, 1),
            "prefill_ms": round(t_p, 4), "prefill_tflops": round(flop / (t_p * 1e-3) / 1e12, 2),
            "route_prefill_ms": round(t_b, 4),
            "route_prefill_tflops": round(flop / (t_b * 1e-3) / 1e12, 2),
            "frac_of_bf16_peak": round(flop / (t_b * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}


def bounds_run(swa, Q, K, V, W, steps):
    """The long prefill's bounds on its own inputs: gate all zeros (pure
    window attention) and all ones (full causal attention through the
    routed path: every row gathered)."""
    import torch
    B, N, Hq, d = Q.shape
    dev = Q.device
    G = 1
    out = {}
    O = torch.empty_like(Q)
    ws = torch.empty(swa.prefill_workspace_size(B, N, Hq, K.shape[2], G, d, W), dtype=torch.uint8, device=dev)
    for name, val in (("gate_all_0", 0), ("gate_all_1", 1)):
        gate = torch.full((B, N, G), val, dtype=torch.uint8, device=dev)
        _, idx, cnt, _ = swa.route(None, gate=gate)
        t, tmin = time_ms(lambda: swa.prefill(Q, K, V, gate, W, idx=idx, cnt=cnt, out=O, workspace=ws), steps)
        useful = prefill_pairs(gate.cpu().numpy(), W, Hq, G)[0]
        flop = 4.0 * d * useful
        out[name] = {"useful_tflop": round(flop / 1e12, 4), "ms": round(t, 4), "min_ms": round(tmin, 4),
                     "tflops": round(flop / (t * 1e-3) / 1e12, 2),
                     "frac_of_bf16_peak": round(flop / (t * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
    return out


def structured_run(swa, W, steps):
    """Structured routing (contiguous runs of 64-512 tokens) at densities
    0.30 and 0.05 on N=32768 with 16 MHA heads, d=128: the hard-gate prefill
    (useful pairs at the realized gate) and the both-branch prefill with the
    per-token distance (full causal pairs)."""
    import torch
    from sliding_window_attention_router_amd import synth
    dev = torch.device("cuda", 0)
    bf = torch.bfloat16
    out = {}
    for p in (0.30, 0.05):
        w = synth.structured(p)
        Q, K, V = (torch.from_numpy(x).to(bf).to(dev) for x in (w.Q, w.K, w.V))
        gate = torch.from_numpy(w.gate).to(dev)
        B, N, Hq, d = Q.shape
        G = 1
        _, idx, cnt, _ = swa.route(None, gate=gate)
        O = torch.empty_like(Q)
        diff = torch.empty((B, N), dtype=torch.float32, device=dev)
        ws_h = torch.empty(swa.prefill_workspace_size(B, N, Hq, K.shape[2], G, d, W), dtype=torch.uint8,
                           device=dev)
        ws_b = torch.empty(swa.prefill_workspace_size(B, N, Hq, K.shape[2], G, d, W, both_branch=True),
                           dtype=torch.uint8, device=dev)
        th, _ = time_ms(lambda: swa.prefill(Q, K, V, gate, W, idx=idx, cnt=cnt, out=O, workspace=ws_h), steps)
        tb, _ = time_ms(lambda: swa.prefill(Q, K, V, gate, W, both_branch=True, out=O, diff=diff,
                                            workspace=ws_b), max(2, steps // 2))
        useful = prefill_pairs(w.gate, W, Hq, G)[0]
        fh = 4.0 * d * useful
        fb = 4.0 * d * Hq * B * N * (N + 1) / 2
        out[f"p{p:.2f}"] = {
            "realized_density": round(float(w.gate.mean()), 5), "Hq": Hq, "Hkv": K.shape[2],
            "hard_gate": {"useful_tflop": round(fh / 1e12, 4), "ms": round(th, 4),
                          "tflops": round(fh / (th * 1e-3) / 1e12, 2),
                          "frac_of_bf16_peak": round(fh / (th * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)},
            "both_branch": {"useful_tflop": round(fb / 1e12, 4), "ms": round(tb, 4),
                            "tflops": round(fb / (tb * 1e-3) / 1e12, 2),
                            "frac_of_bf16_peak": round(fb / (tb * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}}
        del Q, K, V, O, ws_h, ws_b
        torch.cuda.empty_cache()
    return out


def decode_sweep(swa, dec, W, steps):
    """Routed decode on the decode workload's cache (64 x 32768, GQA 16/4)
    at per-sequence full-branch densities 0, 0.05, 0.13 and 1 (seeded
    Bernoulli draws), each run after rewriting a 512 MiB buffer so that no
    key is served from the L2 or MALL.  The speedup of each density over
    the all-full decode is the same-run analogue of the pages' decode claim
    (4x for their standard routing distribution, 12x for the easy one, at
    32K with W=1024), which the pages do not tie to any hardware or
    density; densities 0.13 and 0.05 stand for standard and easy."""
    import torch
    q, Kc, Vc = dec["q"], dec["Kc"], dec["Vc"]
    B, Hq, d = q.shape
    Lmax, Hkv = Kc.shape[1], Kc.shape[2]
    dev = q.device
    lens = torch.from_numpy(dec["cache_len"]).to(dev)
    o = torch.empty_like(q)
    ws = torch.empty(swa.decode_workspace_size(B, Lmax, Hq, Hkv, 1, d, W), dtype=torch.uint8, device=dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    out = {}
    for p in (0.0, 0.05, 0.13, 1.0):
        g = (np.random.default_rng(55).random((B, 1)) < p).astype(np.uint8)
        gd = torch.from_numpy(g).to(dev)
        t, tmin = time_ms(lambda: swa.decode(q, Kc, Vc, lens, gd, W, out=o, workspace=ws), steps, flush=flush)
        byts, keys = decode_bytes(g, dec["cache_len"], W, Hq, Hkv, d)
        out[f"p{p:.2f}"] = {"full_sequences": int(g.sum()), "attended_kv_rows": keys, "bytes": byts,
                            "ms": round(t, 4), "min_ms": round(tmin, 4),
                            "tok_per_s": round(B / (t * 1e-3), 1),
                            "GB_per_s": round(byts / (t * 1e-3) / 1e9, 1),
                            "frac_of_hbm_peak": round(byts / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    t1 = out["p1.00"]["ms"]
    out["speedup_vs_all_full"] = {k: round(t1 / v["ms"], 2) for k, v in out.items() if k.startswith("p")}
    out["pages_claim"] = "4x (standard routing distribution) to 12x (easy) at 32K, W=1024; no hardware named"
    del flush
    torch.cuda.empty_cache()
    return out


def serve_run(swa, q, Kc, Vc, cache_len, r, bias, W, steps):
    """Serving decode steps on the decode workload's cache (outside the timed
    steps): each routes 64 new tokens (hidden states drawn from a seeded
    N(0,1), router as in the prefill), appends their keys and values at
    position L-1 of the full cache (the lengths are set to L-1 before each
    step) and decodes over L keys.  The steps run back to back, each timed
    with events around the whole call; the median is reported."""
    import torch
    B, Hq, d = q.shape
    Hkv = Kc.shape[2]
    dev = q.device
    hidden = r.shape[0]
    gen = torch.Generator(device=dev).manual_seed(23)
    Hn = torch.randn(B, hidden, generator=gen, device=dev).to(r.dtype)
    k = torch.randn(B, Hkv, d, generator=gen, device=dev).to(q.dtype)
    v = torch.randn(B, Hkv, d, generator=gen, device=dev).to(q.dtype)
    before = (cache_len - 1).to(torch.int32)
    L = before.clone()
    o = torch.empty_like(q)
    gate = torch.empty((B, r.shape[1]), dtype=torch.uint8, device=dev)
    G = r.shape[1]
    ws = torch.empty(swa.decode_workspace_size(B, Kc.shape[1], Hq, Hkv, G, d, W), dtype=torch.uint8,
                     device=dev)
    swa.decode_step(Hn, r, bias, q, k, v, Kc, Vc, L, W, gate=gate, out=o, workspace=ws)
    torch.cuda.synchronize()
    # steps back to back, as in a serving loop (the lengths are reset by a
    # small copy before each step, outside its events); one synchronisation
    # at the end
    evs = []
    gpu_lead()
    for _ in range(steps):
        L.copy_(before)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        swa.decode_step(Hn, r, bias, q, k, v, Kc, Vc, L, W, gate=gate, out=o, workspace=ws)
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
    g = gate.cpu().numpy()
    lens = L.cpu().numpy()
    dbytes, keys = decode_bytes(g, lens, W, Hq, Hkv, d)
    byts = dbytes + B * hidden * 2 + 2 * B * Hkv * d * 2  # + router input + appended rows
    return {"B": B, "cache_len_after": int(lens.max()), "hidden": hidden,
            "full_sequences": int(g.sum()), "attended_kv_rows": keys, "bytes": byts,
            "ms": round(ms, 4), "tok_per_s": round(B / (ms * 1e-3), 1),
            "GB_per_s": round(byts / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def anchors_run(swa, Q, K, V, gate, idx, cnt, W, A, q_d, Kc, Vc, len_d, gate_d, dec, steps):
    """Anchored prefill and decode on the same inputs and gates (outside the
    timed steps): the window branch also sees the first A keys.  Stage times
    from events recorded inside the library; useful work counts the anchors
    (prefill) and the anchor rows read (decode)."""
    import torch
    B, N, Hq, d = Q.shape
    Hkv = K.shape[2]
    dev = Q.device
    G = gate.shape[2]
    O = torch.empty_like(Q)
    o = torch.empty_like(q_d)
    ws_p = torch.empty(swa.prefill_workspace_size(B, N, Hq, Hkv, G, d, W), dtype=torch.uint8, device=dev)
    ws_d = torch.empty(swa.decode_workspace_size(q_d.shape[0], Kc.shape[1], Hq, Hkv, gate_d.shape[1], d, W),
                       dtype=torch.uint8, device=dev)

    def run(ev=None):
        swa.prefill(Q, K, V, gate, W, idx=idx, cnt=cnt, out=O, workspace=ws_p, anchors=A,
                    events=ev[0:4] if ev is not None else None)
        swa.decode(q_d, Kc, Vc, len_d, gate_d, W, out=o, workspace=ws_d, anchors=A,
                   events=ev[4:7] if ev is not None else None)

    def new_sets(n):
        sets = []
        for _ in range(steps):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
            for e in ev:
                e.record()
            sets.append(ev)
        return sets

    run()
    torch.cuda.synchronize()
    # whole calls first, with events only around them; then the stage times
    # from the library's events (which lengthen a call by a few us)
    ends = new_sets(3)
    torch.cuda.synchronize()
    gpu_lead()
    for ev in ends:
        ev[0].record()
        swa.prefill(Q, K, V, gate, W, idx=idx, cnt=cnt, out=O, workspace=ws_p, anchors=A)
        ev[1].record()
        swa.decode(q_d, Kc, Vc, len_d, gate_d, W, out=o, workspace=ws_d, anchors=A)
        ev[2].record()
    torch.cuda.synchronize()
    sets = new_sets(7)
    torch.cuda.synchronize()
    gpu_lead()
    for ev in sets:
        run(ev)
    torch.cuda.synchronize()

    def avg(i, j):
        return float(np.mean([ev[i].elapsed_time(ev[j]) for ev in sets]))

    pre_ms = float(np.mean([ev[0].elapsed_time(ev[1]) for ev in ends]))
    dec_ms = float(np.mean([ev[1].elapsed_time(ev[2]) for ev in ends]))
    attn_ms, split_ms = avg(1, 2), avg(4, 5)
    useful = prefill_pairs(gate.cpu().numpy(), W, Hq, G, A)[0]
    flop = 4.0 * d * useful
    dbytes, keys = decode_bytes(dec["gate"], dec["cache_len"], W, Hq, Hkv, d, A=A)
    return {"anchors": A,
            "prefill": {"useful_tflop": round(flop / 1e12, 4), "ms": round(pre_ms, 4),
                        "tflops": round(flop / (pre_ms * 1e-3) / 1e12, 2),
                        "kernel_ms": {"far_schedule": round(avg(0, 1), 4), "attn": round(attn_ms, 4),
                                      "merge": round(avg(2, 3), 4)},
                        "attn_frac_of_bf16_peak": round(flop / (attn_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)},
            "decode": {"attended_kv_rows": keys, "bytes": dbytes, "ms": round(dec_ms, 4),
                       "tok_per_s": round(q_d.shape[0] / (dec_ms * 1e-3), 1),
                       "GB_per_s": round(dbytes / (dec_ms * 1e-3) / 1e9, 1),
                       "splitk_frac_of_hbm_peak": round(dbytes / (split_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}}


def backward_run(swa, Q, K, V, O, gate, idx, cnt, W, pairs, steps):
    """Attention backward of the routed prefill (outside the timed steps) on
    the timed step's inputs, gate and output, with dO ~ N(0,1) from a seeded
    generator.  Useful work: 10*d FLOP per attended (query head, key) pair
    (scores, dP, dV, dQ, dK); for bfloat16 every product runs on the matrix
    cores, so the roofline is the dense bf16 MFMA peak."""
    import torch
    d = Q.shape[3]
    dev = Q.device
    gen = torch.Generator(device=dev).manual_seed(31)
    dO = torch.randn(Q.shape, generator=gen, device=dev).to(Q.dtype)
    out = (torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V))
    B, N, Hq = Q.shape[:3]
    ws = torch.empty(int(swa.lib().swiattn_prefill_backward_workspace_size(B, N, Hq)), dtype=torch.uint8,
                     device=dev)
    swa.prefill_backward(Q, K, V, O, dO, gate, W, idx=idx, cnt=cnt, out=out, workspace=ws)
    torch.cuda.synchronize()
    times = []
    for _ in range(steps):
        gpu_lead()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        swa.prefill_backward(Q, K, V, O, dO, gate, W, idx=idx, cnt=cnt, out=out, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = float(np.median(times))
    flop = 10.0 * d * pairs
    tf = flop / (ms * 1e-3) / 1e12
    return {"useful_tflop": round(flop / 1e12, 4), "ms": round(ms, 3), "tflops": round(tf, 2),
            "bound": "mfma", "peak_tflops": BF16_PEAK_TFLOPS,
            "frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4)}


def router_grad_run(swa, Q, K, V, W, H, r, bias, steps):
    """Router gradient through the straight-through gate on the prefill
    layer (outside the timed steps): the two branch outputs come from one
    both-branch pass (swiattn_prefill_branches, timed as
    branch_outputs_pass_ms), dO ~ N(0,1) from a seeded generator, z from the
    router.  Timed with events around the call (three
    launches); algorithmic bytes: dO, O_FULL, O_SWA and H read once, dH
    written once, plus z, dz and the split partials."""
    import torch
    B, N, Hq, d = Q.shape
    dev = Q.device
    hidden, G = r.shape
    gate, _, _, z = swa.route(H, r, bias, want_z=True)
    # both branch outputs of every token from one both-branch pass
    t_br, _ = time_ms(lambda: swa.prefill_branches(Q, K, V, gate, W), 3)
    _, _, O_full, O_swa = swa.prefill_branches(Q, K, V, gate, W)
    gen = torch.Generator(device=dev).manual_seed(29)
    dO = torch.randn(Q.shape, generator=gen, device=dev).to(Q.dtype)
    out = (torch.empty((B, N, G), dtype=torch.float32, device=dev), torch.empty_like(H),
           torch.empty((hidden, G), dtype=torch.float32, device=dev),
           torch.empty((G,), dtype=torch.float32, device=dev))
    ws = torch.empty(int(swa.lib().swiattn_router_backward_workspace_size(B, N, hidden, G)),
                     dtype=torch.uint8, device=dev)
    swa.router_backward(dO, O_full, O_swa, z, H, r, out=out, workspace=ws)
    torch.cuda.synchronize()
    times = []
    for _ in range(steps):
        gpu_lead()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        swa.router_backward(dO, O_full, O_swa, z, H, r, out=out, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = float(np.median(times))
    el = Q.element_size()
    splits = (B * N + 31) // 32
    byts = (3 * B * N * Hq * d * el + 2 * B * N * hidden * el + 3 * 4 * B * N * G
            + 2 * 4 * splits * G * (hidden + 1))
    return {"B": B, "N": N, "Hq": Hq, "d": d, "hidden": hidden, "G": G, "bytes": byts,
            "ms": round(ms, 4), "GB_per_s": round(byts / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "branch_outputs_pass_ms": round(t_br, 4)}


def both_branch_run(swa, Q, K, V, gate, W, steps, H, r, bias):
    """Both-branch prefill on the same inputs (outside the timed steps): every
    row takes both branches and the per-token distance is written; then the
    adaptive regulariser on that distance, the router's logits and a seeded
    synthetic NLL (uniform in [0, 6]).  Useful work of the prefill is the
    full causal branch (the window branch's keys are a subset of it):
    4*d*Hq*sum_i (i+1) FLOP; the regulariser moves 16 bytes per token and
    gate group."""
    import torch
    B, N, Hq, d = Q.shape
    dev = Q.device
    G = gate.shape[2]
    ws = torch.empty(swa.prefill_workspace_size(B, N, Hq, K.shape[2], G, d, W, both_branch=True),
                     dtype=torch.uint8, device=dev)
    O = torch.empty_like(Q)
    diff = torch.empty((B, N), dtype=torch.float32, device=dev)
    z = swa.route(H, r, bias, want_z=True)[3]
    nll = torch.from_numpy(np.random.default_rng(17).uniform(0.0, 6.0, (B, N)).astype(np.float32)).to(dev)
    loss = torch.empty_like(z)
    swa.prefill(Q, K, V, gate, W, both_branch=True, out=O, diff=diff, workspace=ws)
    swa.regularizer(z, nll, diff, out=loss)
    torch.cuda.synchronize()
    sets = []
    for _ in range(steps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        for e in ev:
            e.record()
        sets.append(ev)
    torch.cuda.synchronize()
    gpu_lead()
    for ev in sets:
        swa.prefill(Q, K, V, gate, W, both_branch=True, out=O, diff=diff, workspace=ws, events=ev[:5])
        swa.regularizer(z, nll, diff, out=loss)
        ev[5].record()
    torch.cuda.synchronize()
    stage = [float(np.mean([ev[i].elapsed_time(ev[i + 1]) for ev in sets])) for i in range(5)]
    ms = sum(stage[:4])
    flop = 4.0 * d * Hq * B * N * (N + 1) / 2
    reg_bytes = 4 * (2 * z.numel() + 2 * B * N)
    return {"ms": round(ms, 4), "useful_tflop": round(flop / 1e12, 4),
            "tflops": round(flop / (ms * 1e-3) / 1e12, 2),
            "frac_of_bf16_peak": round(flop / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "kernel_ms": {"far_schedule": round(stage[0], 4), "attn": round(stage[1], 4),
                          "merge": round(stage[2], 4), "diff": round(stage[3], 4)},
            "regularizer": {"ms": round(stage[4], 4), "bytes": reg_bytes,
                            "GB_per_s": round(reg_bytes / (stage[4] * 1e-3) / 1e9, 1)}}


CPU_POOL_MAX = 16  # the host share of one GPU on the measuring machines


def _cpu_worker_init():
    from threadpoolctl import threadpool_limits

    threadpool_limits(1)  # one BLAS thread per worker: `cores` counts processes


def _cpu_rows(task):
    """One chunk of oracle rows in a worker process (inputs memory-mapped)."""
    folder, W, rows = task
    import oracle

    Q, K, V = (np.load(os.path.join(folder, f + ".npy"), mmap_mode="r") for f in ("Q", "K", "V"))
    gate = np.load(os.path.join(folder, "gate.npy"))
    oracle.prefill(Q, K, V, gate, W, rows=rows)
    Hq = Q.shape[2]
    return int(sum(Hq * ((i + 1) if gate[0, i, 0] else min(i + 1, W)) for i in rows))


def cpu_baseline(pre, gate, W, budget_s):
    """Float64 CPU reference (oracle.prefill) on the routed prefill's rows:
    evenly spaced rows (every 13th, shuffled) in chunks of 16 rows x every
    head, spread over a process pool of min(os.cpu_count(), 16) spawned
    workers with one BLAS thread each, for about budget_s seconds of wall
    time; then one worker alone for a quarter of that.  Scaled to useful
    TFLOP/s at 4*d FLOP per attended pair (the same count as the GPU
    figure).  The gate is the router's (computed on the GPU, the same bits
    the oracle's router gives outside |z| < 1e-5)."""
    import multiprocessing as mp
    import shutil
    import tempfile

    from threadpoolctl import threadpool_limits

    Hq, d = pre.Q.shape[2], pre.Q.shape[3]
    N = pre.Q.shape[1]
    rows_all = np.arange(0, N, 13)  # coprime with every tile size: rows spread over all positions
    np.random.default_rng(0).shuffle(rows_all)
    chunks = [np.sort(rows_all[s:s + 16]) for s in range(0, rows_all.size, 16)]
    folder = tempfile.mkdtemp(prefix="swiattn_cpu_")
    try:
        for name, arr in (("Q", pre.Q), ("K", pre.K), ("V", pre.V), ("gate", gate)):
            np.save(os.path.join(folder, name + ".npy"), np.ascontiguousarray(arr))
        workers = max(1, min(os.cpu_count() or 1, CPU_POOL_MAX))
        ctx = mp.get_context("spawn")
        pairs, done = 0, 0
        with ctx.Pool(workers, initializer=_cpu_worker_init) as pool:
            # start-up and page-in, untimed
            pool.map_async(_cpu_rows, [(folder, W, chunks[0][:1])] * workers).get(timeout=300)
            t0 = time.perf_counter()
            it = pool.imap_unordered(_cpu_rows, [(folder, W, c) for c in chunks])
            for _ in chunks:
                # a bounded wait: a pool whose workers fail would otherwise wait forever
                pairs += it.next(timeout=120)
                done += 1
                if time.perf_counter() - t0 > budget_s:
                    break
            el = time.perf_counter() - t0
            pool.terminate()
        # one core: the same work in this process, one BLAS thread
        pairs1, done1 = 0, 0
        with threadpool_limits(1):
            t1 = time.perf_counter()
            for c in chunks:
                pairs1 += _cpu_rows((folder, W, c))
                done1 += 1
                if time.perf_counter() - t1 > budget_s / 4:
                    break
            el1 = time.perf_counter() - t1
    finally:
        shutil.rmtree(folder, ignore_errors=True)
    fl = 4.0 * d
    return {"value": round(pairs * fl / el / 1e12, 6), "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
            "sample": f"{done} chunks of 16 evenly spaced prefill rows x {Hq} heads ({pairs} useful pairs) "
                      f"in {el:.1f}s over {workers} worker processes (one BLAS thread each), float64 numpy",
            "one_core": {"value": round(pairs1 * fl / el1 / 1e12, 6), "unit": "TFLOP/s", "cores": 1,
                         "sample": f"{done1} chunks ({pairs1} useful pairs) in {el1:.1f}s, one process, "
                                   "one BLAS thread"}}


if __name__ == "__main__":
    main()
