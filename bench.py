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

The default run also times, as sub-objects of the same line, the two forward workloads the metric
names: `layer_c3`, the full MoE layer forward from x on the skewed 16384-token batch (router with
Zipf logit offsets, 2 shared experts, block 128; tokens/s and the fraction of bf16 MFMA peak), and
`decode_c5`, the 256-token decode forward (random routing, 2 shared experts, block 16; the weight
stream as a fraction of HBM bandwidth). Both gather x's rows inside the gate/up product.

Other workloads: `--workload c3` / `c5` make those forwards the main line; `--workload dense`
runs the default step on a dense SwiGLU FFN expressed as one group (E = K = 1, intermediate
11264); `--workload ep8` runs it on one GPU's share of the default layer under 8-way expert
parallelism: 16 local experts with 3072 rows each (the exchange between GPUs is not part of it);
`--workload c4z` runs the default step with Zipf(1.1)-skewed routing (segments from 0 to several
thousand rows).

Prints one JSON line. `value` is the useful grouped-GEMM TFLOP/s of the whole step (padding
excluded). It also carries the dominant kernel's roofline, timed with HIP events on the launch
stream, the shader clock read from the GPU's metrics over a few seconds of back-to-back steps
after the timed ones, and the CPU oracle's throughput on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "grouped-GEMM bf16 TFLOP/s (% MFMA peak) and MoE-layer tokens/s, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
PEAK_FP32_TFLOPS = 157.3    # MI355X dense fp32 (matrix and vector)
NOMINAL_CLOCK_MHZ = 2400.0  # the clock the peaks above assume

DESC = {
    "dense": "dense SwiGLU FFN as one group, forward+backward (T=8192, hidden=4096, "
             "intermediate=11264, block_m=128)",
    "c2": "grouped-GEMM MoE FFN forward+backward, uniform routing (T=8192, hidden=4096, "
          "128 experts top-6, intermediate=1408, block_m=128, 384 rows per expert)",
    "ep8": "one GPU's share of the 128-expert layer under 8-way expert parallelism, "
           "forward+backward: 16 experts x 3072 rows (T=8192 top-6 uniform over 16 "
           "experts, hidden=4096, intermediate=1408, block_m=128)",
    "c3": "MoE FFN full layer forward from x, skewed routing (T=16384, hidden=4096, 128 "
          "experts top-6 with Zipf(1.1) logit offsets + 2 shared experts, intermediate=1408, "
          "block_m=128)",
    "c4z": "grouped-GEMM MoE FFN forward+backward, Zipf(1.1)-skewed routing (T=8192, "
           "hidden=4096, 128 experts top-6, intermediate=1408, block_m=128)",
    "c5": "MoE FFN decode forward from x, random routing (T=256, hidden=4096, 128 experts "
          "top-6 + 2 shared experts, intermediate=1408, block_m=16)",
}


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


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class ClockSampler:
    """The GPU's shader (GFX) clock while a workload runs back to back, through amdsmi's GPU
    metrics. The firmware refreshes them about once a second, so a summary needs a window of a few
    seconds: only readings the firmware published after the window opened count, averaged over the
    8 XCDs. summary() is None where amdsmi, the metrics or fresh readings are unavailable."""

    def __init__(self, period=0.05):
        self.period, self.samples, self._stop, self._th, self._h = period, [], None, None, None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._amdsmi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
            self._read()
        except Exception:   # no amdsmi, no device access: no clock in the line
            self._h = None

    def _read(self):
        m = self._amdsmi.amdsmi_get_gpu_metrics_info(self._h)
        clks = [float(c) for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float))]
        if not clks and isinstance(m.get("current_gfxclk"), (int, float)):
            clks = [float(m["current_gfxclk"])]
        return m.get("system_clock_counter"), clks

    def _run(self):
        first, seen = None, set()
        while not self._stop.is_set():
            try:
                stamp, clks = self._read()
                if first is None:
                    first = stamp          # published before the window opened: not counted
                elif stamp != first and stamp not in seen and clks:
                    seen.add(stamp)
                    self.samples.append(sum(clks) / len(clks))
            except Exception:
                pass
            self._stop.wait(self.period)

    def __enter__(self):
        if self._h is not None:
            self.samples, self._stop = [], threading.Event()
            self._th = threading.Thread(target=self._run, daemon=True)
            self._th.start()
        return self

    def __exit__(self, *exc):
        if self._th is not None:
            self._stop.set()
            self._th.join()
            self._th = None

    def summary(self):
        s = sorted(v for v in self.samples if v > 0)
        if not s:
            return None
        return {"median_mhz": s[len(s) // 2], "min_mhz": s[0], "max_mhz": s[-1], "samples": len(s),
                "source": "amdsmi GPU metrics (mean over the 8 XCDs of each once-a-second "
                          "firmware reading) during a window of back-to-back steps after timing"}


def sample_clock(torch, clock, step, seconds=3.0):
    """Run `step` back to back for about `seconds` under the clock sampler; its summary."""
    if clock is None or clock._h is None:
        return None
    with clock:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(8):
                step()
            torch.cuda.synchronize()
    return clock.summary()


def cpu_baseline_fwd_bwd(cfg, x, w1, w2, logits, dy, stride):
    """The CPU oracle, as it is, on one token in `stride` of the uniformly routed workload,
    forward + backward. With stride 8 (or 16, 32) the sampled tokens route to 48 (24, 12) experts
    with exactly 128 rows each, one whole block: the sample has no padding rows."""
    import numpy as np
    from oracle import moe_oracle as O

    sel = np.arange(0, cfg.T, stride)
    T = len(sel)
    probs = O.softmax_probs(logits[sel])
    kw = dict(T=T, H=cfg.H, E=cfg.E, K=cfg.K, I=cfg.I, S=cfg.S)
    t0 = time.perf_counter()
    f = O.moe_forward(x[sel], w1, w2, B=cfg.block_m, probs=probs, **kw)
    O.moe_backward(f, dy[sel], w1, w2, **kw)
    dt = time.perf_counter() - t0
    rows = T * cfg.K + cfg.S * T
    padded = int(f["total_rows"])
    flops = 18.0 * cfg.H * cfg.I * rows
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": _threads(), "kind": "oracle",
            "cpu_model": cpu_model(), "seconds": round(dt, 3), "rows_useful": rows,
            "rows_padded": padded, "padded_over_useful": round(padded / rows, 4),
            "sample": f"one token in {stride} of the workload ({T} tokens, {rows} expert rows, "
                      f"{padded} after padding), forward + backward, float64 NumPy oracle; useful "
                      f"FLOPs / oracle seconds"}


def cpu_baseline_fwd(cfg, x, w1, w2, wg, logit_bias, sel_bias, sample_tokens):
    """The CPU oracle on the first `sample_tokens` tokens, forward from x (router included)."""
    from oracle import moe_oracle as O

    T = sample_tokens
    kw = dict(T=T, H=cfg.H, E=cfg.E, K=cfg.K, I=cfg.I, S=cfg.S)
    t0 = time.perf_counter()
    f = O.moe_forward(x[:T], w1, w2, B=cfg.block_m, w_gate=wg, logit_bias=logit_bias,
                      sel_bias=sel_bias, **kw)
    dt = time.perf_counter() - t0
    rows = T * cfg.K + cfg.S * T
    padded = int(f["total_rows"])
    flops = 6.0 * cfg.H * cfg.I * rows
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": _threads(), "kind": "oracle",
            "cpu_model": cpu_model(), "seconds": round(dt, 3), "rows_useful": rows,
            "rows_padded": padded, "padded_over_useful": round(padded / rows, 4),
            "sample": f"first {T} tokens of the workload ({rows} expert rows, {padded} after "
                      f"padding), forward from x, float64 NumPy oracle; useful grouped-GEMM FLOPs "
                      f"/ oracle seconds"}


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


# ------------------------------------------------------------------------------------------------
# forward from x (the skewed full layer, the decode)
# ------------------------------------------------------------------------------------------------
def run_forward(torch, np, M, Sy, name, W1, W2, dev, steps, warmup, materialize=False, clock=None,
                block_m=None):
    """Time the forward from x of workload `name` (router, permutation, gate/up, down, combine).
    W1/W2 are the device weights [G, 2I, H] / [G, H, I] (the workload's own draw). Returns the
    measurement dict; the useful FLOPs exclude padding rows. block_m overrides the workload's."""
    cfg = Sy.get_config(name, **({"block_m": block_m} if block_m else {}))
    T, H, E, K, I, S, B = cfg.T, cfg.H, cfg.E, cfg.K, cfg.I, cfg.S, cfg.block_m
    x, wg, lb, sb = Sy.draw_x(cfg), Sy.draw_wg(cfg), Sy.draw_logit_bias(cfg), Sy.draw_sel_bias(cfg)
    s = M.make_shape(T, H, E, K, I, S, B)
    b = M.alloc_buffers(s, dev, backward=False, save_h=False)
    X = _bf(np, torch, x, dev)
    WG = torch.from_numpy(wg).to(dev)
    LB = torch.from_numpy(lb).to(dev) if lb is not None else None
    SB = torch.from_numpy(sb).to(dev)
    gather = not materialize
    if gather:
        del b["x_perm"]
    stages = ["route", "permute", "fwd_gateup", "fwd_down", "combine"]

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        M.moe_route(s, X, WG, LB, SB, b["logits"], b["probs"], b["topk_idx"], b["topk_w"],
                    b["expert_counts"])
        mark(1)
        if gather:   # maps only: the gate/up product reads x through row_token
            M.moe_permute(s, b["topk_idx"], None, b["seg_offsets"], b["tile_group"],
                          b["total_rows"], b["row_token"], b["pos"], None, b["ws"])
            mark(2)
            M.grouped_gemm_fwd_gather(s, M.MOE_FWD_GATEUP, X, b["row_token"], b["seg_offsets"],
                                      b["tile_group"], b["total_rows"], W1, W2, None, b["a"],
                                      b["y_perm"])
        else:
            M.moe_permute(s, b["topk_idx"], X, b["seg_offsets"], b["tile_group"],
                          b["total_rows"], b["row_token"], b["pos"], b["x_perm"], b["ws"])
            mark(2)
            M.grouped_gemm_fwd(s, M.MOE_FWD_GATEUP, b["x_perm"], b["seg_offsets"],
                               b["tile_group"], b["total_rows"], W1, W2, None, b["a"],
                               b["y_perm"])
        mark(3)
        M.grouped_gemm_fwd(s, M.MOE_FWD_DOWN, None, b["seg_offsets"], b["tile_group"],
                           b["total_rows"], W1, W2, None, b["a"], b["y_perm"])
        mark(4)
        M.moe_combine(s, b["y_perm"], b["pos"], b["topk_w"], b["seg_offsets"], b["y"])
        mark(5)

    step()
    torch.cuda.synchronize()
    counts = b["expert_counts"].cpu().numpy()
    seg = b["seg_offsets"].cpu().numpy()
    ms, st_ms = _time_steps(torch, np, step, len(stages), steps, warmup)
    stage_ms = dict(zip(stages, st_ms))
    rows = T * K + S * T                        # useful rows
    padded = int(seg[-1])                      # rows the grouped GEMMs run (segments padded to B)
    touched = int(np.sum(counts > 0)) + S      # groups whose weights are read
    per_row = {"fwd_gateup": 4.0 * H * I, "fwd_down": 2.0 * H * I}
    gemm_flops = sum(per_row.values()) * rows
    layer_flops = gemm_flops + 2.0 * T * H * E                  # plus the router's fp32 logits
    out = {"workload": DESC[name], "T": T, "H": H, "E": E, "K": K, "I": I, "S": S, "block_m": B,
           "ms": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
           "useful_tflops": round(layer_flops / (ms * 1e-3) / 1e12, 2),
           "frac": round(layer_flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "stages_ms": {k: round(v, 4) for k, v in stage_ms.items()},
           "stages_tflops": {k: round(per_row[k] * rows / (stage_ms[k] * 1e-3) / 1e12, 1)
                             for k in per_row},
           "rows_useful": rows, "rows_padded": padded,
           "padding_excess": round(padded / rows - 1.0, 4),
           "experts_touched": touched,
           "permutation": ("rows of x gathered inside the gate/up GEMM (moe_permute writes the "
                           "maps only, no x_perm)") if gather else "x_perm written by moe_permute"}
    if B < 128:
        # decode: each launch streams the weights of every touched expert once
        wbytes = {"fwd_gateup": touched * 2 * I * H * 2, "fwd_down": touched * H * I * 2}
        gbs = {k: wbytes[k] / (stage_ms[k] * 1e-3) / 1e9 for k in wbytes}
        both = sum(wbytes.values()) / ((stage_ms["fwd_gateup"] + stage_ms["fwd_down"]) * 1e-3) / 1e9
        out["weight_stream_gbs"] = {k: round(v, 1) for k, v in gbs.items()}
        out["hbm_frac"] = round(both / PEAK_HBM_GBS, 4)
        dom = max(wbytes, key=lambda k: stage_ms[k])
        out["roofline"] = {"bound": "hbm", "achieved": round(gbs[dom], 1), "peak": PEAK_HBM_GBS,
                           "unit": "GB/s", "frac": round(gbs[dom] / PEAK_HBM_GBS, 4),
                           "traffic": load_traffic(dom, name), "kernel": dom,
                           "per_unit": f"{wbytes[dom] // touched} weight bytes per touched expert x "
                                       f"{touched} experts per launch",
                           "avg_launch_ms": round(stage_ms[dom], 4)}
    else:
        dom = max(per_row, key=lambda k: stage_ms[k])
        ach = per_row[dom] * rows / (stage_ms[dom] * 1e-3) / 1e12
        traffic = load_traffic(dom, name)
        out["roofline"] = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                           "traffic": traffic, "kernel": dom,
                           "per_unit": f"{per_row[dom]:.0f} FLOP per useful row x {rows} rows "
                                       f"per launch",
                           "avg_launch_ms": round(stage_ms[dom], 4)}
    out["clock"] = sample_clock(torch, clock, step)
    return out, (x, wg, lb, sb, cfg)


# ------------------------------------------------------------------------------------------------
# the training step (forward + backward)
# ------------------------------------------------------------------------------------------------
def run_train_step(torch, np, M, Sy, name, x, w1, w2, W1, W2, dev, args, clock):
    cfg = Sy.get_config(name)
    T, H, E, K, I, S, B = cfg.T, cfg.H, cfg.E, cfg.K, cfg.I, cfg.S, cfg.block_m
    dy = Sy.draw_dy(cfg)
    logits = Sy.skewed_logits(cfg) if cfg.routing == "zipf" else Sy.uniform_logits(cfg)
    s = M.make_shape(T, H, E, K, I, S, B)
    b = M.alloc_buffers(s, dev, backward=True, save_h=True)
    X = _bf(np, torch, x, dev)
    DY, LG = _bf(np, torch, dy, dev), torch.from_numpy(logits).to(dev)
    stages = ["route", "permute", "fwd_gateup", "fwd_down", "combine", "combine_bwd", "dgrad_down",
              "dgrad_gateup", "wgrad_down", "wgrad_gateup", "unpermute_bwd"]
    # The unpermute backward needs only dx_perm, so it runs on a second stream beside the two
    # weight-gradient GEMMs (it takes little LDS and few registers, so its workgroups fit on the
    # CUs beside theirs); the step ends when both streams are done. Its own events are on that
    # stream.
    side = torch.cuda.Stream() if not args.serial else None
    side_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
               for _ in range(args.steps)]
    side_k = [0]
    # Default: moe_permute writes only the maps and the gate/up product gathers x's rows itself,
    # writing x_perm (which the gate/up weight gradient reads) from the rows it stages.
    gather = not args.materialize

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        M.moe_route(s, None, None, None, None, LG, b["probs"], b["topk_idx"], b["topk_w"],
                    b["expert_counts"])
        mark(1)
        M.moe_permute(s, b["topk_idx"], None if gather else X, b["seg_offsets"], b["tile_group"],
                      b["total_rows"], b["row_token"], b["pos"], None if gather else b["x_perm"],
                      b["ws"])
        mark(2)
        if gather:
            M.grouped_gemm_fwd_gather(s, M.MOE_FWD_GATEUP, X, b["row_token"], b["seg_offsets"],
                                      b["tile_group"], b["total_rows"], W1, W2, b["h_save"],
                                      b["a"], b["y_perm"], x_perm=b["x_perm"])
        else:
            M.grouped_gemm_fwd(s, M.MOE_FWD_GATEUP, b["x_perm"], b["seg_offsets"],
                               b["tile_group"], b["total_rows"], W1, W2, b["h_save"], b["a"],
                               b["y_perm"])
        mark(3)
        M.grouped_gemm_fwd(s, M.MOE_FWD_DOWN, None, b["seg_offsets"], b["tile_group"],
                           b["total_rows"], W1, W2, b["h_save"], b["a"], b["y_perm"])
        mark(4)
        M.moe_combine(s, b["y_perm"], b["pos"], b["topk_w"], b["seg_offsets"], b["y"])
        mark(5)
        M.moe_combine_bwd(s, DY, b["y_perm"], b["pos"], b["topk_w"], b["seg_offsets"],
                          b["row_token"], b["total_rows"], b["dy_perm"], b["dtopk_w"])
        for i, which in enumerate((M.MOE_DGRAD_DOWN, M.MOE_DGRAD_GATEUP, M.MOE_WGRAD_DOWN,
                                   M.MOE_WGRAD_GATEUP)):
            mark(6 + i)
            if side is not None and which == M.MOE_WGRAD_DOWN:
                done = torch.cuda.Event()
                done.record()
                side.wait_event(done)
                with torch.cuda.stream(side):
                    if ev is not None:
                        side_ev[side_k[0]][0].record()
                    M.moe_unpermute_bwd(s, b["dx_perm"], b["pos"], b["seg_offsets"], b["dx"])
                    if ev is not None:
                        side_ev[side_k[0]][1].record()
            M.grouped_gemm_bwd(s, which, b["x_perm"], b["h_save"], b["a"], b["dy_perm"],
                               b["seg_offsets"], b["tile_group"], b["total_rows"], W1, W2, b["dh"],
                               b["dx_perm"], b["dw1"], b["dw2"])
        mark(10)
        if side is None:
            M.moe_unpermute_bwd(s, b["dx_perm"], b["pos"], b["seg_offsets"], b["dx"])
        else:
            joined = torch.cuda.Event()
            joined.record(side)
            torch.cuda.current_stream().wait_event(joined)
            if ev is not None:
                side_k[0] += 1
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
    if cfg.routing != "zipf":
        assert np.all(counts == T * K // E), "uniform routing not reproduced"
    ms_step, st_ms = _time_steps(torch, np, step, len(stages), args.steps, args.warmup)
    stage_ms = dict(zip(stages, st_ms))
    if side is not None:   # on its own stream, beside the weight-gradient GEMMs
        stage_ms["unpermute_bwd"] = float(np.mean([e[0].elapsed_time(e[1]) for e in side_ev]))

    rows = T * K + S * T                       # useful rows (padding excluded)
    per_row = {"fwd_gateup": 4.0 * H * I, "fwd_down": 2.0 * H * I, "dgrad_down": 2.0 * H * I,
               "dgrad_gateup": 4.0 * H * I, "wgrad_down": 2.0 * H * I, "wgrad_gateup": 4.0 * H * I}
    step_flops = sum(per_row.values()) * rows
    value = step_flops / (ms_step * 1e-3) / 1e12
    dom = max(per_row, key=lambda k: stage_ms[k])
    dom_flops = per_row[dom] * rows
    achieved = dom_flops / (stage_ms[dom] * 1e-3) / 1e12
    traffic = load_traffic(dom, name)
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic, "kernel": dom,
                "traffic_gbs": (round(traffic / (stage_ms[dom] * 1e-3) / 1e9, 1)
                                if traffic is not None else None),
                "per_unit": f"{per_row[dom]:.0f} FLOP per useful row x {rows} rows per launch",
                "avg_launch_ms": round(stage_ms[dom], 4)}
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": DESC[name], "T": T, "H": H, "E": E, "K": K, "I": I, "S": S,
                   "block_m": B},
        "roofline": roofline,
        "training_step_tokens_per_s": round(T / (ms_step * 1e-3), 1),
        "mfma_frac": round(value / PEAK_BF16_TFLOPS, 4),
        "step_useful_tflop": round(step_flops / 1e12, 4),
        "stages_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "stages_tflops": {k: round(per_row[k] * rows / (stage_ms[k] * 1e-3) / 1e12, 1)
                          for k in per_row},
        "experts_touched": int(np.sum(counts > 0)) + S,
        "permutation": ("maps only; the gate/up product gathers x's rows and writes x_perm from "
                        "its staged rows" if gather else "x_perm written by moe_permute"),
        "streams": ("the unpermute backward on a second stream beside the weight-gradient GEMMs"
                    if side is not None else "one stream"),
    }
    # The forward, data-gradient and weight-gradient passes, each its two grouped GEMMs.
    out["passes"] = {}
    for pname, ks in (("fwd", ("fwd_gateup", "fwd_down")), ("dx", ("dgrad_down", "dgrad_gateup")),
                      ("dw", ("wgrad_down", "wgrad_gateup"))):
        t = sum(stage_ms[k] for k in ks)
        tf = sum(per_row[k] for k in ks) * rows / (t * 1e-3) / 1e12
        out["passes"][pname] = {"ms": round(t, 4), "tflops": round(tf, 1),
                                "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
    out["clock"] = sample_clock(torch, clock, step)
    if out["clock"]:
        c = out["clock"]["median_mhz"]
        # the same fractions against the dense bf16 peak at the sampled clock
        out["passes_frac_at_sampled_clock"] = {
            k: round(v["frac"] * NOMINAL_CLOCK_MHZ / c, 4) for k, v in out["passes"].items()}
    if name == "c2":
        out["router_backward"] = router_backward_timing(torch, np, M, Sy, cfg, s, b, X, dev)
        # The fp32-gradient variant of the two weight-gradient GEMMs on the step's own operands.
        dw1f = torch.empty(E, 2 * I, H, device=dev)
        dw2f = torch.empty(E, H, I, device=dev)
        wg32 = {}
        for wname, which in (("wgrad_down", M.MOE_WGRAD_DOWN), ("wgrad_gateup", M.MOE_WGRAD_GATEUP)):
            t = _time_call(torch, np, lambda: M.grouped_gemm_wgrad_f32(
                s, which, b["x_perm"], b["a"], b["dy_perm"], b["dh"], b["seg_offsets"], dw1f, dw2f),
                10)
            wg32[wname] = {"ms": round(t, 4),
                           "tflops": round(per_row[wname] * rows / (t * 1e-3) / 1e12, 1)}
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
    if name == "dense":
        # Context only: the same gate/up product as one plain library GEMM (torch.mm, which ROCm
        # serves with hipBLASLt), on the same operands, outside the step.
        W1t = W1.view(2 * I, H).t().contiguous()
        t_lib = _time_call(torch, np, lambda: torch.mm(X, W1t), 20)
        out["library_gemm_ref"] = {
            "what": "torch.mm of x [T,H] by W1^T [H,2I] in bf16 (the gate/up forward GEMM)",
            "ms": round(t_lib, 4), "tflops": round(4.0 * T * H * I / (t_lib * 1e-3) / 1e12, 1),
            "this_library_fwd_gateup_ms": round(stage_ms["fwd_gateup"], 4)}
        del W1t
    del b
    return out, (dy, logits)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=("c2", "c3", "c5", "dense", "ep8", "c4z"), default="c2",
                    help="c2: forward+backward at the uniform 8192-token shape (default; the line "
                         "also carries the c3 and c5 forwards); c3: skewed 16384-token full layer "
                         "forward; c5: 256-token decode forward; dense: forward+backward of a dense "
                         "SwiGLU FFN (intermediate 11264) as one group; ep8: forward+backward of one "
                         "GPU's 16-expert share under 8-way expert parallelism (3072 rows per expert); "
                         "c4z: the default forward+backward with Zipf(1.1)-skewed routing")
    ap.add_argument("--serial", action="store_true",
                    help="training step: run the unpermute backward after the weight gradients on "
                         "the one stream instead of beside them on a second stream")
    ap.add_argument("--no-forwards", action="store_true",
                    help="c2: leave out the c3 and c5 forward sub-objects")
    ap.add_argument("--forward-steps", type=int, default=10,
                    help="timed steps of each c3/c5 forward sub-object")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="before warmup, copy a cold buffer of this many MiB (a plain copy of known "
                         "size that scales the HBM byte counters)")
    ap.add_argument("--block-m", type=int, default=None,
                    help="c3/c5: pad the segments to this block size instead of the workload's")
    ap.add_argument("--materialize", action="store_true",
                    help="write x_perm in moe_permute and run grouped_gemm_fwd on it instead of "
                         "gathering x's rows inside the gate/up product (the training step and "
                         "the c3/c5 forwards)")
    ap.add_argument("--cpu-sample", type=int, default=None,
                    help="CPU oracle sample (0 = skip the CPU baseline): for the training workloads "
                         "the token stride (default 8: 1024 tokens, 48 experts x 128 rows, no "
                         "padding), for c3/c5 the number of leading tokens (default 256)")
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
    clock = ClockSampler()
    name = args.workload
    cfg = Sy.get_config(name)
    log(f"[bench] {name}: generating inputs {cfg}")
    t0 = time.perf_counter()
    extras = name == "c2" and not args.no_forwards
    if name in ("c2", "c3"):
        # c3's 130 groups share their first 128 with c2 (the same per-group streams, seed 0)
        w_cfg = Sy.get_config("c3") if (name == "c3" or extras) else cfg
    else:
        w_cfg = cfg
    w1, w2 = Sy.draw_w1_all(w_cfg), Sy.draw_w2_all(w_cfg)
    log(f"[bench] weights ready in {time.perf_counter() - t0:.1f}s; uploading")
    W1a, W2a = _bf(np, torch, w1, dev), _bf(np, torch, w2, dev)
    G = cfg.E + cfg.S
    W1, W2 = W1a[:G], W2a[:G]
    torch.cuda.synchronize()

    if name in ("c3", "c5"):
        fwd, (x, wg, lb, sb, _) = run_forward(torch, np, M, Sy, name, W1, W2, dev, args.steps,
                                              args.warmup, args.materialize, clock, args.block_m)
        if args.block_m:
            cfg = Sy.get_config(name, block_m=args.block_m)
        rows, T = fwd["rows_useful"], cfg.T
        out = {"metric": METRIC, "value": fwd["useful_tflops"], "unit": "TFLOP/s", "n_gpus": 1,
               "steps": args.steps, "warmup": args.warmup, "ms_per_step": fwd["ms"],
               "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
               "data": "synthetic",
               "config": {"workload": DESC[name], "T": T, "H": cfg.H, "E": cfg.E, "K": cfg.K,
                          "I": cfg.I, "S": cfg.S, "block_m": cfg.block_m},
               "roofline": fwd.pop("roofline"), "tokens_per_s": fwd["tokens_per_s"],
               "mfma_frac": fwd["frac"]}
        out.update({k: v for k, v in fwd.items() if k not in out})
        sample = args.cpu_sample if args.cpu_sample is not None else 256
        if sample > 0:
            log(f"[bench] CPU oracle on {sample} tokens")
            out["cpu_baseline"] = cpu_baseline_fwd(cfg, x, w1[:G], w2[:G], wg, lb, sb, sample)
        else:
            out["cpu_baseline"] = None
        print(json.dumps(out), flush=True)
        return

    x = Sy.draw_x(cfg)
    out, (dy, logits) = run_train_step(torch, np, M, Sy, name, x, w1, w2, W1, W2, dev, args, clock)
    if extras:
        log("[bench] c3 forward (skewed full layer)")
        out["layer_c3"], _ = run_forward(torch, np, M, Sy, "c3", W1a, W2a, dev, args.forward_steps,
                                         3, args.materialize, clock)
        log("[bench] c5 forward (decode): drawing its weights")
        del W1a, W2a, W1, W2
        torch.cuda.empty_cache()
        c5 = Sy.get_config("c5")
        W15 = _bf(np, torch, Sy.draw_w1_all(c5), dev)
        W25 = _bf(np, torch, Sy.draw_w2_all(c5), dev)
        out["decode_c5"], _ = run_forward(torch, np, M, Sy, "c5", W15, W25, dev,
                                          max(args.forward_steps, 20), 5, args.materialize, clock)
        del W15, W25
    # The sample is padding-free only under uniform routing; the skewed step skips it by default.
    stride = args.cpu_sample if args.cpu_sample is not None else (0 if name == "c4z" else 8)
    if stride > 0:
        log(f"[bench] CPU oracle on one token in {stride}")
        G = cfg.E + cfg.S
        out["cpu_baseline"] = cpu_baseline_fwd_bwd(cfg, x, w1[:G], w2[:G], logits, dy, stride)
        out["cpu_baseline"]["gpu_over_cpu"] = round(out["value"] / out["cpu_baseline"]["value"], 1)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
