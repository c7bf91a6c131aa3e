#!/usr/bin/env python3
"""Benchmark of the MoE feed-forward hot path (dots.llm1 shapes) on one MI355X.

A step is one pass of the whole path over one batch: routing (softmax, biased top-k, weights,
counts), permutation into block-aligned expert segments, the grouped SwiGLU GEMMs (gate/up with the
fused SwiGLU, down), the weighted combine, then the backward: combine backward, dgrad (down with
the fused SwiGLU backward, gate/up), wgrad (down, gate/up) and the unpermute backward.

Default workload: T=8192 tokens, hidden 4096, 128 experts top-6, intermediate 1408, block 128,
uniform routing (every expert gets exactly 384 rows). The routing stage runs on logits that encode
that assignment, so the selection kernel runs but decides nothing else.

Prints one JSON line: value = useful grouped-GEMM TFLOP/s of the whole step (padding excluded),
with the dominant kernel's roofline (timed with HIP events on the launch stream) and the CPU
oracle's throughput on a bounded sample of the same workload.
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


def cpu_baseline(cfg, x, w1, w2, logits, dy, sample_tokens):
    """The CPU oracle, as it is, on the first `sample_tokens` tokens of the workload (fwd + bwd)."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from oracle import moe_oracle as O

    T = sample_tokens
    probs = O.softmax_probs(logits[:T])
    idx, w = O.select_topk(probs, None, cfg.K)
    kw = dict(T=T, H=cfg.H, E=cfg.E, K=cfg.K, I=cfg.I, S=cfg.S)
    t0 = time.perf_counter()
    f = O.moe_forward(x[:T], w1, w2, B=cfg.block_m, probs=probs, **kw)
    O.moe_backward(f, dy[:T], w1, w2, **kw)
    dt = time.perf_counter() - t0
    rows = T * cfg.K + cfg.S * T
    flops = 18.0 * cfg.H * cfg.I * rows
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": f"first {T} tokens of the workload ({rows} expert rows), forward + backward, "
                      f"float64 NumPy oracle; useful FLOPs / oracle seconds"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="before warmup, copy a cold buffer of this many MiB (a plain copy of known "
                         "size that scales the HBM byte counters)")
    ap.add_argument("--cpu-sample", type=int, default=384,
                    help="tokens of the workload the CPU oracle runs (0 = skip the CPU baseline)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for {max(args.gpus, world)}): this build "
              f"implements the single-GPU path only; sharding across GPUs is described in DESIGN.md "
              f"but not implemented.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import grouped_gemm_fp32_amd as M
    from synth import get_config, draw_x, draw_w1_all, draw_w2_all, draw_dy, uniform_logits

    dev = "cuda:0"
    cfg = get_config("c2")
    T, H, E, K, I, S, B = cfg.T, cfg.H, cfg.E, cfg.K, cfg.I, cfg.S, cfg.block_m
    log(f"[bench] generating inputs T={T} H={H} E={E} K={K} I={I} S={S} B={B}")
    t0 = time.perf_counter()
    x, w1, w2, dy, logits = draw_x(cfg), draw_w1_all(cfg), draw_w2_all(cfg), draw_dy(cfg), \
        uniform_logits(cfg)
    log(f"[bench] inputs ready in {time.perf_counter() - t0:.1f}s; uploading")
    s = M.make_shape(T, H, E, K, I, S, B)
    buf = M.alloc_buffers(s, dev, backward=True)
    X, W1, W2, DY = _bf(np, torch, x, dev), _bf(np, torch, w1, dev), _bf(np, torch, w2, dev), \
        _bf(np, torch, dy, dev)
    LG = torch.from_numpy(logits).to(dev)
    torch.cuda.synchronize()

    stages = ["route", "permute", "fwd_gateup", "fwd_down", "combine", "combine_bwd",
              "dgrad_down", "dgrad_gateup", "wgrad_down", "wgrad_gateup", "unpermute_bwd"]
    b = buf

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        M.moe_route(s, None, None, None, None, LG, b["probs"], b["topk_idx"], b["topk_w"],
                    b["expert_counts"])
        mark(1)
        M.moe_permute(s, b["topk_idx"], X, b["seg_offsets"], b["tile_group"], b["total_rows"],
                      b["row_token"], b["pos"], b["x_perm"], b["ws"])
        mark(2)
        M.grouped_gemm_fwd(s, M.MOE_FWD_GATEUP, b["x_perm"], b["seg_offsets"], b["tile_group"],
                           b["total_rows"], W1, W2, b["h_save"], b["a"], b["y_perm"])
        mark(3)
        M.grouped_gemm_fwd(s, M.MOE_FWD_DOWN, b["x_perm"], b["seg_offsets"], b["tile_group"],
                           b["total_rows"], W1, W2, b["h_save"], b["a"], b["y_perm"])
        mark(4)
        M.moe_combine(s, b["y_perm"], b["pos"], b["topk_w"], b["seg_offsets"], b["y"])
        mark(5)
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
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # routing sanity: the uniform assignment gives every expert T*K/E rows
    counts = buf["expert_counts"].cpu().numpy()
    assert np.all(counts == T * K // E), "uniform routing not reproduced"

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(12)] for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    stage_ms = {name: float(np.mean([ev[i].elapsed_time(ev[i + 1]) for ev in events]))
                for i, name in enumerate(stages)}

    rows = T * K + S * T                       # useful rows (padding excluded)
    per_row = {"fwd_gateup": 4.0 * H * I, "fwd_down": 2.0 * H * I, "dgrad_down": 2.0 * H * I,
               "dgrad_gateup": 4.0 * H * I, "wgrad_down": 2.0 * H * I, "wgrad_gateup": 4.0 * H * I}
    step_flops = sum(per_row.values()) * rows
    value = step_flops / (ms_step * 1e-3) / 1e12
    dom = max(per_row, key=lambda k: stage_ms[k])
    dom_flops = per_row[dom] * rows
    achieved = dom_flops / (stage_ms[dom] * 1e-3) / 1e12
    traffic = load_traffic(dom, "c2")
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic, "kernel": dom,
                "traffic_gbs": (round(traffic / (stage_ms[dom] * 1e-3) / 1e9, 1)
                                if traffic is not None else None),
                "per_unit": f"{per_row[dom]:.0f} FLOP per routed row x {rows} rows per launch",
                "avg_launch_ms": round(stage_ms[dom], 4)}
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "grouped-GEMM MoE FFN forward+backward, uniform routing "
                               "(T=8192, hidden=4096, 128 experts top-6, intermediate=1408, "
                               "block_m=128, 384 rows per expert)",
                   "T": T, "H": H, "E": E, "K": K, "I": I, "S": S, "block_m": B},
        "roofline": roofline,
        "tokens_per_s": round(T / (ms_step * 1e-3), 1),
        "mfma_frac": round(value / PEAK_BF16_TFLOPS, 4),
        "step_useful_tflop": round(step_flops / 1e12, 4),
        "stages_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "stages_tflops": {k: round(per_row[k] * rows / (stage_ms[k] * 1e-3) / 1e12, 1)
                          for k in per_row},
    }
    if args.cpu_sample > 0:
        log(f"[bench] CPU oracle on {args.cpu_sample} tokens")
        out["cpu_baseline"] = cpu_baseline(cfg, x, w1, w2, logits, dy, args.cpu_sample)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
