"""Summaries of rocprofv3 CSV output for this library's kernels.

    python -m grouped_gemm_fp32_amd.profiling stats <kernel_stats.csv>
    python -m grouped_gemm_fp32_amd.profiling traffic <fetch_dir> <write_dir> --calib-mib N \
        [--workload NAME] [--json OUT]
    python -m grouped_gemm_fp32_amd.profiling mfma <counter_dir>
    python -m grouped_gemm_fp32_amd.profiling units <lds_counter_dir> <ta_counter_dir>

`stats` prints the per-kernel table (calls, average and total duration, share of GPU time).
`traffic` reads two `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs (KiB per dispatch) of
the same deterministic program, scales each counter by what it reads for a plain copy of a known
size in the same run (the dispatch with the largest FETCH_SIZE outside this library: bench.py's
`--calib-copy-mib` elementwise copy of a cold buffer, `calib` MiB read and written; the same
dispatch id in the WRITE_SIZE run), and reports HBM bytes per launch.
`mfma` reads one `rocprofv3 --pmc SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE` run and
reports, per kernel, the matrix instructions per launch, the fraction of SIMD cycles the matrix
unit was busy, and the shader clock the launch ran at (GRBM_GUI_ACTIVE sums the busy cycles of
every XCD; dividing by the XCD count and by the dispatch's duration gives the clock).
`units` reads a run of `SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE` and one of
`TA_TA_BUSY SQ_WAIT_INST_LDS SQ_WAVE_CYCLES GRBM_GUI_ACTIVE` and reports, per kernel, the share of
all CU cycles in which LDS served indexed (non-DMA) accesses, the share stalled by bank conflicts,
the share in which the texture addresser (the front of the vector memory path, which the
direct-to-LDS loads and the stores share) was busy, and the share of wavefront cycles spent
waiting for LDS results.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import json
import os
import re
import sys

# rocprofv3 kernel name -> the stage names bench.py reports
STAGE_OF = {
    "ggemm_tall8_kernel<0,false>": "fwd_gateup", "ggemm_tall8_kernel<1,false>": "fwd_down",
    "ggemm_tall8_kernel<2,false>": "dgrad_down", "ggemm_tall8_kernel<3,false>": "dgrad_gateup",
    "ggemm_tall8_kernel<0,true>": "fwd_gateup",   # rows gathered through row_token
    "ggemm_wgrad8_kernel<4,false>": "wgrad_down", "ggemm_wgrad8_kernel<5,false>": "wgrad_gateup",
    "gather_rows_kernel": "permute", "gather_sum_kernel<true>": "combine",
    "combine_bwd_kernel": "combine_bwd", "gather_sum_kernel<false>": "unpermute_bwd",
    "route_kernel<1>": "route",
}


# Kernels the benchmark times outside the step (extra measurements and context).
OUTSIDE_STEP = {
    "ggemm_wgrad8_kernel<4,true>": "fp32-dW wgrad down (outside the step)",
    "ggemm_wgrad8_kernel<5,true>": "fp32-dW wgrad gate/up (outside the step)",
    "route_bwd_kernel<true>": "router backward (outside the step)",
    "router_dwg_kernel<true>": "router backward (outside the step)",
    "router_dwg_kernel<false>": "router backward (outside the step)",
    "router_dx_kernel": "router backward (outside the step)",
    "balance_hist_kernel": "balance loss (outside the step)",
    "balance_kernel": "balance loss (outside the step)",
    "balance_reduce_kernel": "balance loss (outside the step)",
    "bias_update_kernel": "bias update (outside the step)",
}


# Other kernels of a stage (labels only: STAGE_OF keeps one kernel per stage for the traffic table).
PART_OF = {
    "router_logits_kernel<4,4>": "route (router logits)", "router_logits_kernel<2,4>": "route (router logits)",
    "router_logits_kernel<1,8>": "route (router logits)",
    "router_logits_dma_kernel<1>": "route (router logits)", "router_logits_dma_kernel<2>": "route (router logits)",
    "fill_i32_kernel": "route (count clear)", "count_kernel": "route (expert counts)",
    "count_kernel<false>": "route (expert counts)", "count_kernel<true>": "route (expert counts)",
    "perm_clear_rows_kernel": "permute (maps)",
    "perm_small_kernel": "permute (segments and maps, one workgroup)",
    "perm_hist_kernel": "permute (segments)", "perm_segment_kernel": "permute (segments)",
    "perm_scatter_kernel": "permute (maps)", "zero_pad_rows_kernel": "combine_bwd (padding rows)",
    "ggemm_kernel<0,16,256,16,1>": "fwd_gateup (16-row tiles)",
    "ggemm_kernel<1,16,256,16,1>": "fwd_down (16-row tiles)",
    "ggemm_kernel<0,32,256,32,1>": "fwd_gateup (32-row tiles)",
    "ggemm_kernel<1,32,256,32,1>": "fwd_down (32-row tiles)",
    "ggemm_block64_kernel<0>": "fwd_gateup (64-row tiles)", "ggemm_block64_kernel<1>": "fwd_down (64-row tiles)",
}


def label(k: str) -> str:
    if k in STAGE_OF:
        return STAGE_OF[k]
    if k in PART_OF:
        return PART_OF[k]
    if k in OUTSIDE_STEP:
        return OUTSIDE_STEP[k]
    if k.startswith("Cijk_"):
        return "library GEMM reference (outside the step)"
    return ""


def short_name(n: str) -> str:
    m = re.search(r"moe::\(anonymous namespace\)::(\w+)(<[^(]*>)?", n)
    if m:
        return m.group(1) + (m.group(2) or "").replace(" ", "")
    return n.split("(")[0][:60]


def _csv(path_or_dir: str, suffix: str) -> str:
    if os.path.isdir(path_or_dir):
        hits = glob.glob(os.path.join(path_or_dir, "**", "*" + suffix), recursive=True)
        if not hits:
            raise FileNotFoundError(f"no *{suffix} under {path_or_dir}")
        return hits[0]
    return path_or_dir


def stats_table(path: str) -> str:
    rows = list(csv.DictReader(open(_csv(path, "kernel_stats.csv"))))
    out = ["| kernel | stage | calls | avg (us) | total (ms) | share |", "|---|---|---|---|---|---|"]
    for r in rows:
        k = short_name(r["Name"])
        out.append(f"| {k} | {label(k)} | {r['Calls']} | "
                   f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['TotalDurationNs']) / 1e6:.3f} | "
                   f"{float(r['Percentage']):.1f}% |")
    return "\n".join(out)


def counter_rows(path: str) -> list:
    return list(csv.DictReader(open(_csv(path, "counter_collection.csv"))))


def counter_means(path: str) -> dict:
    d = collections.defaultdict(list)
    for r in counter_rows(path):
        d[(short_name(r["Kernel_Name"]), r["Counter_Name"])].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in d.items()}


def traffic(fetch_dir: str, write_dir: str, calib_mib: float) -> dict:
    known = calib_mib * 2 ** 20
    fr, wr = counter_rows(fetch_dir), counter_rows(write_dir)
    # The calibration copy is the first kernel outside this library that reads at least a quarter
    # of its size (the fills that prepare it read nothing; library GEMMs timed later come after).
    foreign = [r for r in fr if "moe::" not in r["Kernel_Name"]
               and float(r["Counter_Value"]) * 1024.0 >= known / 4]
    if not foreign:
        raise ValueError("no calibration copy found in the FETCH_SIZE run")
    cal = min(foreign, key=lambda r: int(r["Dispatch_Id"]))
    cal_w = [r for r in wr if r["Dispatch_Id"] == cal["Dispatch_Id"]]
    if not cal_w or cal_w[0]["Kernel_Name"] != cal["Kernel_Name"]:
        raise ValueError("the FETCH_SIZE and WRITE_SIZE runs do not line up by dispatch id")
    out = {}
    for name, rows, crow, counter in (("fetch", fr, cal, "FETCH_SIZE"),
                                      ("write", wr, cal_w[0], "WRITE_SIZE")):
        measured = float(crow["Counter_Value"]) * 1024.0
        scale = known / measured
        out[f"{name}_calibration"] = {"kernel": short_name(crow["Kernel_Name"]),
                                      "dispatch": int(crow["Dispatch_Id"]), "known_bytes": known,
                                      "counter_bytes": measured, "scale": scale}
        d = collections.defaultdict(list)
        for r in rows:
            if r["Counter_Name"] == counter:
                d[short_name(r["Kernel_Name"])].append(float(r["Counter_Value"]))
        for k, v in d.items():
            e = out.setdefault("kernels", {}).setdefault(k, {})
            e[f"{name}_bytes"] = sum(v) / len(v) * 1024.0 * scale
            e[f"{name}_bytes_raw"] = sum(v) / len(v) * 1024.0
    for k, e in out.get("kernels", {}).items():
        e["bytes_per_launch"] = e.get("fetch_bytes", 0.0) + e.get("write_bytes", 0.0)
    return out


# MI355X: 8 XCDs of 32 CUs, 4 SIMDs per CU.
N_XCD, N_SIMD = 8, 256 * 4


def mfma_util(path: str) -> dict:
    """Per kernel: mean over its dispatches of the MFMA-busy fraction of all SIMD cycles, the
    shader clock (GHz), the duration (us), MFMA instructions per launch and busy cycles per
    instruction. Dispatches that lack one of the three counters are skipped."""
    disp = collections.defaultdict(dict)
    for r in counter_rows(path):
        key = (short_name(r["Kernel_Name"]), int(r["Dispatch_Id"]))
        d = disp[key]
        d[r["Counter_Name"]] = float(r["Counter_Value"])
        d["_ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    per = collections.defaultdict(list)
    need = ("SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")
    for (k, _), d in disp.items():
        if not all(n in d for n in need) or d["SQ_INSTS_MFMA"] <= 0 or d["_ns"] <= 0:
            continue
        cyc = d["GRBM_GUI_ACTIVE"] / N_XCD
        per[k].append({"busy_frac": d["SQ_VALU_MFMA_BUSY_CYCLES"] / (N_SIMD * cyc),
                       "clock_ghz": cyc / d["_ns"],
                       "us": d["_ns"] / 1e3,
                       "mfma_insts": d["SQ_INSTS_MFMA"],
                       "cycles_per_inst": d["SQ_VALU_MFMA_BUSY_CYCLES"] / d["SQ_INSTS_MFMA"]})
    out = {}
    for k, v in per.items():
        out[k] = {f: sum(e[f] for e in v) / len(v) for f in v[0]}
        out[k]["dispatches"] = len(v)
    return out


def mfma_table(path: str) -> str:
    rows = ["| kernel | stage | dispatches | avg (us) | MFMA instr / launch | busy cycles / instr "
            "| clock (GHz) | MFMA busy (of SIMD cycles) |", "|---|---|---|---|---|---|---|---|"]
    for k, e in sorted(mfma_util(path).items(), key=lambda kv: -kv[1]["us"]):
        rows.append(f"| {k} | {label(k)} | {e['dispatches']} | {e['us']:.1f} | "
                    f"{e['mfma_insts']:.0f} | {e['cycles_per_inst']:.1f} | {e['clock_ghz']:.2f} | "
                    f"{100 * e['busy_frac']:.1f}% |")
    return "\n".join(rows)


N_CU = 256


def _per_dispatch(path: str) -> dict:
    disp = collections.defaultdict(dict)
    for r in counter_rows(path):
        d = disp[(short_name(r["Kernel_Name"]), int(r["Dispatch_Id"]))]
        d[r["Counter_Name"]] = float(r["Counter_Value"])
        d["_ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    return disp


def unit_util(lds_path: str, ta_path: str) -> dict:
    """Per kernel, means over its dispatches of: lds_active and lds_bank_conflict (fractions of
    all CU cycles, the SQ_ counters summed over every CU), ta_busy (TA_TA_BUSY over all CU
    cycles) and lds_wait (SQ_WAIT_INST_LDS over SQ_WAVE_CYCLES). A kernel missing from either run,
    or a dispatch without GRBM_GUI_ACTIVE, is skipped."""
    def means(path, need, f):
        per = collections.defaultdict(list)
        for (k, _), d in _per_dispatch(path).items():
            if all(n in d for n in need) and d["GRBM_GUI_ACTIVE"] > 0:
                per[k].append(f(d, d["GRBM_GUI_ACTIVE"] / N_XCD * N_CU) | {"us": d["_ns"] / 1e3})
        return {k: {c: sum(e[c] for e in v) / len(v) for c in v[0]} for k, v in per.items()}
    lds = means(lds_path, ("SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "GRBM_GUI_ACTIVE"),
                lambda d, cu: {"lds_active": d["SQ_LDS_IDX_ACTIVE"] / cu,
                               "lds_bank_conflict": d["SQ_LDS_BANK_CONFLICT"] / cu})
    ta = means(ta_path, ("TA_TA_BUSY", "SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE"),
               lambda d, cu: {"ta_busy": d["TA_TA_BUSY"] / cu,
                              "lds_wait": (d["SQ_WAIT_INST_LDS"] / d["SQ_WAVE_CYCLES"]
                                           if d["SQ_WAVE_CYCLES"] > 0 else 0.0)})
    return {k: lds[k] | {c: v for c, v in ta[k].items() if c != "us"} for k in lds if k in ta}


def units_table(lds_path: str, ta_path: str) -> str:
    rows = ["| kernel | stage | avg (us) | LDS active | LDS bank-conflict stall | TA busy "
            "| wave cycles waiting on LDS |", "|---|---|---|---|---|---|---|"]
    for k, e in sorted(unit_util(lds_path, ta_path).items(), key=lambda kv: -kv[1]["us"]):
        rows.append(f"| {k} | {label(k)} | {e['us']:.1f} | {100 * e['lds_active']:.1f}% | "
                    f"{100 * e['lds_bank_conflict']:.1f}% | {100 * e['ta_busy']:.1f}% | "
                    f"{100 * e['lds_wait']:.1f}% |")
    return "\n".join(rows)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    m = sub.add_parser("mfma")
    m.add_argument("dir")
    u = sub.add_parser("units")
    u.add_argument("lds_dir")
    u.add_argument("ta_dir")
    t = sub.add_parser("traffic")
    t.add_argument("fetch")
    t.add_argument("write")
    t.add_argument("--calib-mib", type=float, required=True)
    t.add_argument("--workload", default="c2")
    t.add_argument("--json", default=None, help="merge per-stage bytes into this traffic.json")
    t.add_argument("--source-hash", default=None)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        print(stats_table(a.csv))
        return
    if a.cmd == "mfma":
        print(mfma_table(a.dir))
        return
    if a.cmd == "units":
        print(units_table(a.lds_dir, a.ta_dir))
        return
    tr = traffic(a.fetch, a.write, a.calib_mib)
    print(json.dumps(tr, indent=1))
    if a.json:
        d = json.load(open(a.json)) if os.path.exists(a.json) else {}
        for k, e in tr["kernels"].items():
            if k in STAGE_OF:
                d[f"{a.workload}:{STAGE_OF[k]}"] = {
                    "bytes_per_launch": round(e["bytes_per_launch"]),
                    "fetch_bytes": round(e.get("fetch_bytes", 0)),
                    "write_bytes": round(e.get("write_bytes", 0)),
                    "fetch_scale": tr["fetch_calibration"]["scale"],
                    "write_scale": tr["write_calibration"]["scale"],
                    "source_hash": a.source_hash}
        with open(a.json, "w") as f:
            json.dump(d, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main(sys.argv[1:])
