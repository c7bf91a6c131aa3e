#!/usr/bin/env python3
"""Benchmark of the MoE feed-forward hot path (dots.llm1 shapes) on one MI355X.

Default workload (c2/c4 shapes): one step is one pass of the whole path over one batch:
  - routing (softmax, biased top-k, weights, counts);
  - permutation into block-aligned expert segments;
  - the grouped SwiGLU GEMMs (gate/up with the fused SwiGLU, down);
  - the weighted combine;
  - then the backward: combine backward, dgrad (down with the fused SwiGLU backward, gate/up),
    wgrad (down, gate/up) and the unpermute backward.
It uses T=8192 tokens, hidden 4096, 128 experts top-6, intermediate 1408, block 128, with uniform
routing (every expert gets exactly 384 rows). The routing stage runs on logits that encode that
assignment, so the selection kernel runs but decides nothing else.

Other workloads (forward only, routing computed from x): `--workload c3` is the skewed full layer
(T=16384, Zipf logit offsets, 2 shared experts, block 128); `--workload c5` is decode (T=256,
random routing, 2 shared experts, block 16). `--workload dense` runs the default step on a dense
SwiGLU FFN expressed as one group (E = K = 1, intermediate 11264). `--workload ep8` runs it on one
GPU's share of the default layer under 8-way expert parallelism: 16 local experts with 3072 rows
each (8192 tokens top-6 over 16 experts; the exchange between GPUs is not part of it).

Prints one JSON line. `value` is the useful grouped-GEMM TFLOP/s of the whole step (padding
excluded). It also carries the dominant kernel's roofline, timed with HIP events on the launch
stream, and the CPU oracle's throughput on a bounded sample of the same workload. With the default
workload it also times, outside the step, the router backward on the step's routing (dlogits, then
dWg and the router's share of dx in fp32) and the load-balancing bias update.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "grouped-GEMM bf16 TFLOP/s (% MFMA peak) and MoE-layer tokens/s, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
PEAK_FP32_TFLOPS = 157.3    # MI355X dense fp32 (matrix and vector)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def _bf(np, torch, bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "grouped_gemm_fp32_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch measured with rocprofv3 counters for this exact kernel source, or None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    e = d.get(f"{workload}:{kernel}")
    if not e or e.get("source_hash") != kernel_source_hash():
        return None
    return e.get("bytes_per_launch")


def _threads():
    from threadpoolctl import threadpool_info
    return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))


def cpu_baseline_fwd_bwd(cfg, x, w1, w2, logits, dy, sample_tokens):
    """The CPU oracle, as it is, on the first `sample_tokens` tokens of the workload (fwd + bwd)."""
    from oracle import moe_oracle as O

    T = sample_tokens
    probs = O.softmax_probs(logits[:T])
    kw = dict(T=T, H=cfg.H, E=cfg.E, K=cfg.K, I=cfg.I, S=cfg.S)
    t0 = time.perf_counter()
    f = O.moe_forward(x[:T], w1, w2, B=cfg.block_m, probs=probs, **kw)
    O.moe_backward(f, dy[:T], w1, w2, **kw)
    dt = time.perf_counter() - t0
    rows = T * cfg.K + cfg.S * T
    flops = 18.0 * cfg.H * cfg.I * rows
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": _threads(), "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": f"first {T} tokens of the workload ({rows} expert rows), forward + backward, "
                      f"float64 NumPy oracle; useful FLOPs / oracle seconds"}


def cpu_baseline_fwd(cfg, x, w1, w2, wg, logit_bias, sel_bias, sample_tokens):
    """The CPU oracle on the first `sample_tokens` tokens, forward from x (router included)."""
    from oracle import moe_oracle as O

    T = sample_tokens
    kw = dict(T=T, H=cfg.H, E=cfg.E, K=cfg.K, I=cfg.I, S=cfg.S)
    t0 = time.perf_counter()
    O.moe_forward(x[:T], w1, w2, B=cfg.block_m, w_gate=wg, logit_bias=logit_bias,
                  sel_bias=sel_bias, **kw)
    dt = time.perf_counter() - t0
    rows = T * cfg.K + cfg.S * T
    flops = 6.0 * cfg.H * cfg.I * rows
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": _threads(), "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": f"first {T} tokens of the workload ({rows} expert rows), forward from x, "
                      f"float64 NumPy oracle; useful grouped-GEMM FLOPs / oracle seconds"}


def _time_steps(torch, np, step, nstages, steps, warmup):
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(nstages + 1)]
              for _ in range(steps)]
    log(f"[bench] timing {steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        step(events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage_ms = [float(np.mean([ev[i].elapsed_time(ev[i + 1]) for ev in events]))
                for i in range(nstages)]
    return wall * 1e3 / steps, stage_ms


def _time_call(torch, np, fn, reps):
    """Mean HIP-event time (ms) of fn() on the current stream, after one untimed call."""
    fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    for k in range(reps):
        ev[k].record()
        fn()
    ev[reps].record()
    torch.cuda.synchronize()
    return float(np.mean([ev[k].elapsed_time(ev[k + 1]) for k in range(reps)]))


def router_backward_timing(torch, np, M, Sy, cfg, s, b, X, dev, reps=20):
    """The router backward on the step's own routing and weight gradients (not part of the step):
    dlogits alone, then with dWg = dlogits^T x and dx_router = dlogits Wg; the bias update; the
    sequence-wise balance loss with its gradient."""
    T, H, E = cfg.T, cfg.H, cfg.E
    WG = torch.from_numpy(Sy.draw_wg(cfg)).to(dev)
    dz = torch.empty(T, E, device=dev)
    dwg = torch.empty(E, H, device=dev)
    dxr = torch.empty(T, H, device=dev)
    sb = torch.zeros(E, device=dev)
    args = (s, b["dtopk_w"], b["topk_idx"], b["probs"], X, WG, dz)
    t_dz = _time_call(torch, np, lambda: M.moe_route_bwd(*args, None, None), reps)
    t_dwg = _time_call(torch, np, lambda: M.moe_route_bwd(*args, dwg, None), reps) - t_dz
    t_dx = _time_call(torch, np, lambda: M.moe_route_bwd(*args, None, dxr), reps) - t_dz
    t_all = _time_call(torch, np, lambda: M.moe_route_bwd(*args, dwg, dxr), reps)
    t_bias = _time_call(torch, np, lambda: M.moe_bias_update(s, b["expert_counts"], 1e-3, sb), reps)
    loss = torch.empty(1, device=dev)   # the batch as one sequence of T tokens (8K, the pages' length)
    ws = torch.empty(M.moe_balance_workspace_size(s, T) // 4, device=dev)
    t_bal = _time_call(torch, np, lambda: M.moe_balance_loss(s, T, 1e-3, b["probs"], b["topk_idx"],
                                                             loss, dz, ws), reps)
    flops = 2.0 * T * E * H                # each of dWg and dx_router, fp32
    return {"ms": round(t_all, 4), "dlogits_ms": round(t_dz, 4),
            "dwg_ms": round(t_dwg, 4), "dwg_tflops": round(flops / (t_dwg * 1e-3) / 1e12, 2),
            "dx_ms": round(t_dx, 4), "dx_tflops": round(flops / (t_dx * 1e-3) / 1e12, 2),
            "fp32_peak_tflops": PEAK_FP32_TFLOPS, "bias_update_ms": round(t_bias, 4),
            "balance_loss_ms": round(t_bal, 4)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=("c2", "c3", "c5", "dense", "ep8"), default="c2",
                    help="c2: forward+backward at the uniform 8192-token shape (default); c3: skewed "
                         "16384-token full layer forward; c5: 256-token decode forward; dense: "
                         "forward+backward of a dense SwiGLU FFN (intermediate 11264) as one group; "
                         "ep8: forward+backward of one GPU's 16-expert share under 8-way expert "
                         "parallelism (3072 rows per expert)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="before warmup, copy a cold buffer of this many MiB (a plain copy of known "
                         "size that scales the HBM byte counters)")
    ap.add_argument("--materialize", action="store_true",
                    help="c3/c5: write x_perm in moe_permute and run grouped_gemm_fwd on it instead "
                         "of gathering x's rows inside the gate/up product")
    ap.add_argument("--cpu-sample", type=int, default=None,
                    help="tokens of the workload the CPU oracle runs (0 = skip the CPU baseline); "
                         "default 384 for c2, 256 for c3, all 256 for c5")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for {max(args.gpus, world)}): the library "
              f"implements the single-GPU path only; sharding the experts across GPUs (an "
              f"all-to-all of the permuted rows each way) is not implemented.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import grouped_gemm_fp32_amd as M
    import synth as Sy

    dev = "cuda:0"
    cfg = Sy.get_config(args.workload)
    T, H, E, K, I, S, B = cfg.T, cfg.H, cfg.E, cfg.K, cfg.I, cfg.S, cfg.block_m
    log(f"[bench] {args.workload}: generating inputs T={T} H={H} E={E} K={K} I={I} S={S} B={B}")
    t0 = time.perf_counter()
    x, w1, w2 = Sy.draw_x(cfg), Sy.draw_w1_all(cfg), Sy.draw_w2_all(cfg)
    fwd_bwd = args.workload in ("c2", "dense", "ep8")
    if fwd_bwd:
        dy, logits = Sy.draw_dy(cfg), Sy.uniform_logits(cfg)
    else:
        wg, lb, sb = Sy.draw_wg(cfg), Sy.draw_logit_bias(cfg), Sy.draw_sel_bias(cfg)
    log(f"[bench] inputs ready in {time.perf_counter() - t0:.1f}s; uploading")
    s = M.make_shape(T, H, E, K, I, S, B)
    b = M.alloc_buffers(s, dev, backward=fwd_bwd, save_h=fwd_bwd)
    X, W1, W2 = _bf(np, torch, x, dev), _bf(np, torch, w1, dev), _bf(np, torch, w2, dev)
    if fwd_bwd:
        DY, LG = _bf(np, torch, dy, dev), torch.from_numpy(logits).to(dev)
        route_args = (None, None, None, None, LG)
    else:
        WG = torch.from_numpy(wg).to(dev)
        LB = torch.from_numpy(lb).to(dev) if lb is not None else None
        SB = torch.from_numpy(sb).to(dev)
        route_args = (X, WG, LB, SB, b["logits"])
    torch.cuda.synchronize()

    # Forward-only workloads gather x's rows inside the gate/up product (no x_perm); the training
    # step keeps x_perm, which the gate/up weight gradient reads.
    gather = not fwd_bwd and not args.materialize
    if gather:
        del b["x_perm"]
    stages = ["route", "permute", "fwd_gateup", "fwd_down", "combine"]
    if fwd_bwd:
        stages += ["combine_bwd", "dgrad_down", "dgrad_gateup", "wgrad_down", "wgrad_gateup",
                   "unpermute_bwd"]
    h_save = b.get("h_save")

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        M.moe_route(s, *route_args, b["probs"], b["topk_idx"], b["topk_w"], b["expert_counts"])
        mark(1)
        if gather:   # maps only: the gate/up product reads x through row_token
            M.moe_permute(s, b["topk_idx"], None, b["seg_offsets"], b["tile_group"],
                          b["total_rows"], b["row_token"], b["pos"], None, b["ws"])
            mark(2)
            M.grouped_gemm_fwd_gather(s, M.MOE_FWD_GATEUP, X, b["row_token"], b["seg_offsets"],
                                      b["tile_group"], b["total_rows"], W1, W2, h_save, b["a"],
                                      b["y_perm"])
        else:
            M.moe_permute(s, b["topk_idx"], X, b["seg_offsets"], b["tile_group"],
                          b["total_rows"], b["row_token"], b["pos"], b["x_perm"], b["ws"])
            mark(2)
            M.grouped_gemm_fwd(s, M.MOE_FWD_GATEUP, b["x_perm"], b["seg_offsets"],
                               b["tile_group"], b["total_rows"], W1, W2, h_save, b["a"],
                               b["y_perm"])
        mark(3)
        M.grouped_gemm_fwd(s, M.MOE_FWD_DOWN, None, b["seg_offsets"], b["tile_group"],
                           b["total_rows"], W1, W2, h_save, b["a"], b["y_perm"])
        mark(4)
        M.moe_combine(s, b["y_perm"], b["pos"], b["topk_w"], b["seg_offsets"], b["y"])
        mark(5)
        if not fwd_bwd:
            return
        M.moe_combine_bwd(s, DY, b["y_perm"], b["pos"], b["topk_w"], b["seg_offsets"],
                          b["row_token"], b["total_rows"], b["dy_perm"], b["dtopk_w"])
        for i, which in enumerate((M.MOE_DGRAD_DOWN, M.MOE_DGRAD_GATEUP, M.MOE_WGRAD_DOWN,
                                   M.MOE_WGRAD_GATEUP)):
            mark(6 + i)
            M.grouped_gemm_bwd(s, which, b["x_perm"], b["h_save"], b["a"], b["dy_perm"],
                               b["seg_offsets"], b["tile_group"], b["total_rows"], W1, W2, b["dh"],
                               b["dx_perm"], b["dw1"], b["dw2"])
        mark(10)
        M.moe_unpermute_bwd(s, b["dx_perm"], b["pos"], b["seg_offsets"], b["dx"])
        mark(11)

    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * 2 ** 20 // 4
        src = torch.ones(n, dtype=torch.int32, device=dev)
        flush = torch.ones(2 * n, dtype=torch.int32, device=dev)   # evicts src from the caches
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.add(src, 1, out=dst)   # an ordinary elementwise kernel: reads and writes N MiB
        torch.cuda.synchronize()
        log(f"[bench] calibration copy: {args.calib_copy_mib} MiB read + written")
        del src, flush, dst
    log(f"[bench] warmup {args.warmup}")
    step()
    torch.cuda.synchronize()
    counts = b["expert_counts"].cpu().numpy()
    if fwd_bwd:   # the uniform assignment gives every expert T*K/E rows
        assert np.all(counts == T * K // E), "uniform routing not reproduced"
    ms_step, st_ms = _time_steps(torch, np, step, len(stages), args.steps, args.warmup)
    stage_ms = dict(zip(stages, st_ms))
    router_bwd = (router_backward_timing(torch, np, M, Sy, cfg, s, b, X, dev)
                  if args.workload == "c2" else None)

    rows = T * K + S * T                       # useful rows (padding excluded)
    per_row = {"fwd_gateup": 4.0 * H * I, "fwd_down": 2.0 * H * I}
    if fwd_bwd:
        per_row.update({"dgrad_down": 2.0 * H * I, "dgrad_gateup": 4.0 * H * I,
                        "wgrad_down": 2.0 * H * I, "wgrad_gateup": 4.0 * H * I})
    step_flops = sum(per_row.values()) * rows
    value = step_flops / (ms_step * 1e-3) / 1e12
    dom = max(per_row, key=lambda k: stage_ms[k])
    touched = int(np.sum(counts > 0)) + S      # groups whose weights are read
    if args.workload == "c5":
        # decode: each launch streams the weights of every touched expert once
        wbytes = {"fwd_gateup": touched * 2 * I * H * 2, "fwd_down": touched * H * I * 2}
        dom = max(wbytes, key=lambda k: stage_ms[k])
        gbs = wbytes[dom] / (stage_ms[dom] * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                    "traffic": load_traffic(dom, args.workload), "kernel": dom,
                    "per_unit": f"{wbytes[dom] // touched} weight bytes per touched expert x "
                                f"{touched} experts per launch",
                    "avg_launch_ms": round(stage_ms[dom], 4)}
    else:
        dom_flops = per_row[dom] * rows
        achieved = dom_flops / (stage_ms[dom] * 1e-3) / 1e12
        traffic = load_traffic(dom, args.workload)
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                    "traffic": traffic, "kernel": dom,
                    "traffic_gbs": (round(traffic / (stage_ms[dom] * 1e-3) / 1e9, 1)
                                    if traffic is not None else None),
                    "per_unit": f"{per_row[dom]:.0f} FLOP per useful row x {rows} rows per launch",
                    "avg_launch_ms": round(stage_ms[dom], 4)}
    desc = {"dense": "dense SwiGLU FFN as one group, forward+backward (T=8192, hidden=4096, "
                     "intermediate=11264, block_m=128)",
            "c2": "grouped-GEMM MoE FFN forward+backward, uniform routing (T=8192, hidden=4096, "
                  "128 experts top-6, intermediate=1408, block_m=128, 384 rows per expert)",
            "ep8": "one GPU's share of the 128-expert layer under 8-way expert parallelism, "
                   "forward+backward: 16 experts x 3072 rows (T=8192 top-6 uniform over 16 "
                   "experts, hidden=4096, intermediate=1408, block_m=128)",
            "c3": "MoE FFN full layer forward from x, skewed routing (T=16384, hidden=4096, 128 "
                  "experts top-6 with Zipf(1.1) logit offsets + 2 shared experts, intermediate=1408, "
                  "block_m=128)",
            "c5": "MoE FFN decode forward from x, random routing (T=256, hidden=4096, 128 experts "
                  "top-6 + 2 shared experts, intermediate=1408, block_m=16)"}[args.workload]
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": desc, "T": T, "H": H, "E": E, "K": K, "I": I, "S": S, "block_m": B},
        "roofline": roofline,
        "tokens_per_s": round(T / (ms_step * 1e-3), 1),
        "mfma_frac": round(value / PEAK_BF16_TFLOPS, 4),
        "step_useful_tflop": round(step_flops / 1e12, 4),
        "stages_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "stages_tflops": {k: round(per_row[k] * rows / (stage_ms[k] * 1e-3) / 1e12, 1)
                          for k in per_row},
        "experts_touched": touched,
        "permutation": ("rows of x gathered inside the gate/up GEMM (moe_permute writes the maps "
                        "only, no x_perm)") if gather else "x_perm written by moe_permute",
    }
    # The forward, data-gradient and weight-gradient passes, each its two grouped GEMMs.
    passes = {"fwd": ("fwd_gateup", "fwd_down"), "dx": ("dgrad_down", "dgrad_gateup"),
              "dw": ("wgrad_down", "wgrad_gateup")}
    out["passes"] = {}
    for name, ks in passes.items():
        if not all(k in per_row for k in ks):
            continue
        t = sum(stage_ms[k] for k in ks)
        tf = sum(per_row[k] for k in ks) * rows / (t * 1e-3) / 1e12
        out["passes"][name] = {"ms": round(t, 4), "tflops": round(tf, 1),
                               "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
    if router_bwd is not None:
        out["router_backward"] = router_bwd
    if args.workload == "c2":
        # The fp32-gradient variant of the two weight-gradient GEMMs on the step's own operands.
        dw1f = torch.empty(E, 2 * I, H, device=dev)
        dw2f = torch.empty(E, H, I, device=dev)
        wg32 = {}
        for name, which in (("wgrad_down", M.MOE_WGRAD_DOWN), ("wgrad_gateup", M.MOE_WGRAD_GATEUP)):
            t = _time_call(torch, np, lambda: M.grouped_gemm_wgrad_f32(
                s, which, b["x_perm"], b["a"], b["dy_perm"], b["dh"], b["seg_offsets"], dw1f, dw2f),
                10)
            wg32[name] = {"ms": round(t, 4),
                          "tflops": round(per_row[name] * rows / (t * 1e-3) / 1e12, 1)}
        out["wgrad_fp32_dw"] = wg32
        del dw1f, dw2f
        # Context only: the gate/up product as a plain batched library GEMM (torch.bmm, served by
        # hipBLASLt) over the 128 experts' 384-row segments, operands made contiguous first.
        Xb = b["x_perm"][:T * K].view(E, T * K // E, H)
        W1t = W1.view(E, 2 * I, H).transpose(1, 2).contiguous()
        t_lib = _time_call(torch, np, lambda: torch.bmm(Xb, W1t), 20)
        out["library_gemm_ref"] = {
            "what": "torch.bmm of the 128 segments [384,H] by W1_e^T [H,2I] in bf16 (the gate/up "
                    "forward GEMM without the SwiGLU)",
            "ms": round(t_lib, 4), "tflops": round(4.0 * T * K * H * I / (t_lib * 1e-3) / 1e12, 1),
            "this_library_fwd_gateup_ms": round(stage_ms["fwd_gateup"], 4)}
        del W1t
    if args.workload == "dense":
        # Context only: the same gate/up product as one plain library GEMM (torch.mm, which ROCm
        # serves with hipBLASLt), on the same operands, outside the step.
        W1t = W1.view(2 * I, H).t().contiguous()
        t_lib = _time_call(torch, np, lambda: torch.mm(X, W1t), 20)
        out["library_gemm_ref"] = {
            "what": "torch.mm of x [T,H] by W1^T [H,2I] in bf16 (the gate/up forward GEMM)",
            "ms": round(t_lib, 4), "tflops": round(4.0 * T * H * I / (t_lib * 1e-3) / 1e12, 1),
            "this_library_fwd_gateup_ms": round(stage_ms["fwd_gateup"], 4)}
        del W1t
    sample = args.cpu_sample if args.cpu_sample is not None else {"c2": 384, "c3": 256, "dense": 8192,
                                                                   "c5": 256, "ep8": 384}[args.workload]
    if sample > 0:
        log(f"[bench] CPU oracle on {sample} tokens")
        out["cpu_baseline"] = (cpu_baseline_fwd_bwd(cfg, x, w1, w2, logits, dy, sample) if fwd_bwd
                               else cpu_baseline_fwd(cfg, x, w1, w2, wg, lb, sb, sample))
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
