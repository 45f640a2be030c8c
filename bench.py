"""Benchmark of the MSA routed-layer hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--workload prefill|decode|interleave|backward|linear|encode|stack|scan100m]
                    [--no-cpu-baseline]

A step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM:

  prefill (default; the 1M-token bank: 2048 docs x 512 tokens, 32/8 heads,
           head dim 128, bf16, 2048-token prefill, top-16):
      route -> top-k -> gather -> attention; the offline stage (pool K, pool V,
      pool K_r + norms into the bank) is timed apart in the same run and
      reported as `offline_pool` (encoded tokens/s, HBM fraction)
  decode  (the same bank; 32 sequences x 1 token, 4096 cached tokens, top-16):
      route -> top-k -> gather -> split-KV attention (the bank is pooled once,
      outside the timed region, as the offline stage of the pipeline); the
      routing scan is also timed warm and cold (`route_scan_warm_cold`)
  interleave (the prefill workload with 3 routing rounds, Memory Interleave at
           kernel level: each round routes its own planted router query and
           keeps the top-16 documents no earlier round took; the 48 documents'
           memory, 384 pooled rows, then joins the prefill attention):
      route+top-k x3 -> gather -> attention (the bank is pooled outside the step)
  backward (training step of the routed layer's attention at the prefill
           shapes: 2048 tokens, 128 gathered memory rows, 2048 local rows,
           32/8 heads): attention forward -> attention backward (dq; dk, dv of
           the memory and local rows)
  linear  (the linear-layer variant on the 1M-token bank: 32 sequences x 1
           token, top-16, 8 heads x 128): route -> top-k -> sum of the
           selected documents' states -> one gated-delta step from that state
           (the 2048 document states are encoded beforehand, timed apart)
  encode  (offline encoder: 2048 documents of 256..768 tokens, ~1M tokens,
           8 KV heads x 128, bf16): chunk offsets -> encode K (document-wise
           RoPE, base 1e6) -> encode V -> encode K_r (+ norms)
  scan100m (one GPU's share of a 100M-token memory: 195,313 docs x 512
           tokens around 1024 cluster centres, a 3.2 GB router bank in HBM, the
           pooled content K/V in pinned host memory; 4 x 512 router query
           tokens, top-16): route -> top-k -> host-tier fetch of the 64
           selected docs; also a routing sweep over T_tot = 1 .. 2048 query
           tokens (`route_sweep`) and the host-tier fetch in both modes, alone
           and overlapped with the next step's routing (`host_tier`)
  stack   (18 routed layers at a 10M-token memory, each with its own bank of
           19,532 docs x 512 tokens, 8192-token prefill, top-32, 32/8 heads):
           (route -> top-k -> gather -> attention) for every layer; the banks
           are pooled beforehand (the offline stage), timed apart

Prints one JSON line.  `value` is query tokens per second of the whole step
(for the default workload the online step, route -> top-k -> gather ->
attention; its offline pooling has its own entry).
W eager warm-up steps, then K eager steps with HIP events around every launch
(on the stream the kernels run on: the per-kernel durations, `stages` and
`roofline`, which describes the kernel with the largest share of the step),
then the step captured once in a HIP graph and K replays timed: `ms_per_step`
and `value` (the route, decode, interleave, linear and stack steps; the eager figure
is `ms_per_step_eager`).  The replays run the same kernels on the same data
without the host's per-launch cost between short kernels.
`cpu_baseline` times the float64 CPU oracle on a bounded sample of the same
workload and scales it to the full step.

Profiles (run on the GPU, summaries land in profiles/):
    rocprofv3 --kernel-trace --stats --output-format csv -d D -o run -- python3 bench.py --steps 5 --no-cpu-baseline
    python bench.py --summarize-stats D/run_kernel_stats.csv profiles/<name>.md "<title>" "<command>"
HBM traffic of each stage (`roofline.traffic`): four counter runs into DIR,
    rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/copy_fetch -o run -- python3 bench.py --copy-probe
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR/copy_write -o run -- python3 bench.py --copy-probe
    rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/<workload>_fetch -o run -- python3 bench.py --workload <workload> --steps 2 --warmup 1 --no-cpu-baseline
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR/<workload>_write -o run -- python3 bench.py --workload <workload> --steps 2 --warmup 1 --no-cpu-baseline
then `python bench.py --summarize-traffic DIR`.  The copy probe moves a known
1 GiB each way; the ratio of that to what the counters read scales every
kernel's counters to bytes.  A stage's entry is kept only while its source
file is unchanged (sha256 recorded beside it).
"""

import argparse
import dataclasses
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", choices=["prefill", "decode", "interleave", "backward", "linear", "encode", "stack",
                                          "scan100m"],
                   default="prefill")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--step-only", action="store_true",
                   help="time the step alone: no routing sweep, host-tier or warm/cold extras (for profiling)")
    # profiling helpers (see "Profiles" in the module docstring)
    p.add_argument("--copy-probe", action="store_true",
                   help="run a plain elementwise 1 GiB read + 1 GiB write five times and exit")
    p.add_argument("--summarize-stats", nargs=4, metavar=("STATS_CSV", "OUT_MD", "TITLE", "COMMAND"),
                   help="write a markdown summary of a rocprofv3 --stats kernel_stats.csv and exit")
    p.add_argument("--summarize-counters", nargs="+", metavar="ARG",
                   help="OUT_MD TITLE COMMANDS DIR [DIR ...]: per-kernel derived metrics (MFMA busy, VALU and LDS "
                        "activity, bank conflicts, instruction mix) from rocprofv3 --pmc runs, then exit")
    p.add_argument("--summarize-traffic", metavar="DIR",
                   help="turn rocprofv3 FETCH_SIZE / WRITE_SIZE runs under DIR into profiles/traffic.json")
    return p.parse_args()


# ---------------------------------------------------------------------------
# algorithmic work per launch (bytes that must cross HBM, flops that must be done)
# ---------------------------------------------------------------------------

def work_pool(cfg, with_norm):
    rows = cfg.n_doc * cfg.doc_len
    row_b = cfg.heads_kv * cfg.dim * 2
    n_ch = cfg.n_chunks
    b = rows * row_b + n_ch * row_b + (n_ch * cfg.heads_kv * 4 if with_norm else 0)
    return {"bound": "hbm", "bytes": b, "flops": rows * cfg.heads_kv * cfg.dim}


def work_route(cfg):
    t_tot = cfg.batch * cfg.q_len
    row = cfg.heads_kv * cfg.dim
    flops = 2 * t_tot * cfg.n_chunks * row
    b = cfg.n_chunks * row * 2 + cfg.n_chunks * cfg.heads_kv * 4 + t_tot * row * 2 + cfg.batch * cfg.n_doc * 4
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    return {"bound": "mfma" if flops / b > ridge else "hbm", "bytes": b, "flops": flops}


def work_rounds(cfg, rounds):
    # the routing of every round (MFMA-bound at 2048 tokens); the top-k launches are latency
    w = work_route(cfg)
    return {"bound": w["bound"], "bytes": rounds * (w["bytes"] + work_topk(cfg)["bytes"]),
            "flops": rounds * w["flops"]}


def work_topk(cfg):
    return {"bound": "hbm", "bytes": cfg.batch * cfg.n_doc * 4 + cfg.batch * cfg.topk * 8, "flops": 0}


def work_gather(cfg):
    b = 2 * 2 * cfg.batch * cfg.mem_len * cfg.heads_kv * cfg.dim * 2 + cfg.batch * cfg.topk * 4
    return {"bound": "hbm", "bytes": b, "flops": 0}


def work_attn(cfg):
    b_, t_, m, l_ = cfg.batch, cfg.q_len, cfg.mem_len, cfg.loc_len
    pairs = t_ * m + sum(l_ - t_ + t + 1 for t in range(t_))
    flops = 4 * cfg.dim * cfg.heads_q * b_ * pairs
    row_kv = cfg.heads_kv * cfg.dim * 2
    b = (2 * b_ * t_ * cfg.heads_q * cfg.dim * 2            # q in, o out
         + 2 * b_ * (m + l_) * row_kv                       # k/v memory + local
         + b_ * cfg.heads_q * t_ * 4)                       # lse
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    return {"bound": "mfma" if flops / b > ridge else "hbm", "bytes": b, "flops": flops}


def host_threads():
    """Host threads the oracle runs on: `cores` is the BLAS thread count (its
    matrix products use them; its element-wise NumPy work runs on one), beside
    the cores this process may use (os.sched_getaffinity)."""
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        blas = 1
    return {"cores": int(blas), "blas_threads": int(blas), "affinity_cores": len(os.sched_getaffinity(0))}


def roofline_entry(work, ms):
    s = ms / 1e3
    if work["bound"] == "mfma":
        achieved = work["flops"] / s / 1e12
        return {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / MFMA_BF16_PEAK_TFLOPS}
    achieved = work["bytes"] / s / 1e9
    return {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS}


# ---------------------------------------------------------------------------
# measured HBM traffic (rocprofv3 counters), valid only for the source it was taken on
# ---------------------------------------------------------------------------

def kernel_source_sha(src_files):
    """Hash of kernel sources (names separated by |) and of the local headers they include."""
    csrc = os.path.join(ROOT, "routed_sparse_attention_msa_amd", "csrc")
    h = hashlib.sha256()
    todo, seen = src_files.split("|"), set()
    while todo:
        name = todo.pop(0)
        path = os.path.normpath(os.path.join(csrc, name))
        if path in seen or not os.path.exists(path):
            continue
        seen.add(path)
        with open(path, "rb") as f:
            data = f.read()
        h.update(data)
        todo += re.findall(r'#include "([^"]+)"', data.decode("utf-8", "replace"))
    return h.hexdigest()[:16]


INTERLEAVE_ROUNDS = 3

# stage -> (kernel-name patterns separated by |, source file[, launches of each kernel per stage call:
#           one count for all, or a count per pattern])
STAGE_KERNELS = {
    "prefill": {"pool": ("pool_kernel", "pool.hip"), "route": ("route_", "route.hip"),
                "topk": ("topk", "topk.hip"), "gather": ("gather", "gather.hip"),
                "attn": ("attn_prefill", "attn_prefill.hip")},
    "decode": {"route": ("route_", "route.hip"), "topk": ("topk", "topk.hip"),
               "gather": ("gather", "gather.hip"), "attn": ("attn_decode", "attn_decode.hip")},
    # (the rounds' routing is one launch over all rounds' queries; each round has its own top-k launch)
    "interleave": {"rounds": ("route_|topk", "route.hip|topk.hip", {"route_": 1, "topk": INTERLEAVE_ROUNDS}),
                   "gather": ("gather", "gather.hip"),
                   "attn": ("attn_prefill", "attn_prefill.hip")},
    "backward": {"attn": ("attn_prefill", "attn_prefill.hip"), "attn_bwd": ("attn_bwd", "attn_backward.hip")},
    # (the backward stage is two kernels, dq then dk/dv; its entry covers both)
    "linear": {"route": ("route_", "route.hip"), "topk": ("topk", "topk.hip"),
               "state_sum": ("gdn_state_sum", "gdn.hip"), "gdn": ("gdn_kernel<unsigned short, 128, true>", "gdn.hip")},
    "encode": {"offsets": ("chunk_offsets", "encode.hip"),
               "encode_rope": ("encode_kernel<unsigned short, true>", "encode.hip"),
               "encode": ("encode_kernel<unsigned short, false>", "encode.hip")},
    # (the two plain encode launches share one kernel; its entry is their median)
    "scan100m": {"route": ("route_", "route.hip"), "topk": ("topk", "topk.hip"), "fetch": ("gather", "gather.hip")},
    "stack": {"route": ("route_", "route.hip"), "topk": ("topk", "topk.hip"),
              "gather": ("gather", "gather.hip"), "attn": ("attn_prefill", "attn_prefill.hip")},
}
COPY_PROBE_BYTES = 1 << 30


def measured_traffic(workload, stage):
    """HBM bytes per launch of `stage` from profiles/traffic.json, or None when
    absent or taken on a different version of the stage's source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(workload, {}).get(stage)
    if not rec or rec.get("source_sha") != kernel_source_sha(STAGE_KERNELS[workload][stage][1]):
        return None
    return rec["bytes_per_launch"]


def _counter_rows(run_dir):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def _per_kernel_median(rows):
    """kernel name -> median of the counter over its dispatches (KiB)."""
    by = {}
    for r in rows:
        by.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: sorted(v)[len(v) // 2] for k, v in by.items()}


def _short_kernel(name):
    import re
    m = re.search(r"msa::\(anonymous namespace\)::([a-z_0-9]+(?:<[^>(]*>)?)", name)
    return m.group(1) if m else name


def summarize_traffic(d):
    copy = {}
    for kind in ("fetch", "write"):
        med = _per_kernel_median(_counter_rows(os.path.join(d, f"copy_{kind}")))
        probe = [v for k, v in med.items() if "neg" in k]
        if not probe:
            raise SystemExit(f"no copy-probe kernel in {d}/copy_{kind}")
        copy[kind] = probe[0]
    fetch_factor = COPY_PROBE_BYTES / (copy["fetch"] * 1024)
    write_factor = COPY_PROBE_BYTES / (copy["write"] * 1024)
    out = {"calibration": {"copy_probe_bytes_each_way": COPY_PROBE_BYTES, "copy_fetch_kib": copy["fetch"],
                           "copy_write_kib": copy["write"], "fetch_factor": fetch_factor,
                           "write_factor": write_factor}}
    md = ["# HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
          "Commands (repository root, one MI355X; DIR = gpurun_out/traffic):", "", "```"]
    md += ["export TMPDIR=/tmp",
           "rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/copy_fetch -o run -- python3 bench.py --copy-probe",
           "rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR/copy_write -o run -- python3 bench.py --copy-probe"]
    for wl in STAGE_KERNELS:
        extra = " --step-only" if wl == "scan100m" else ""
        md += [f"rocprofv3 --pmc {c} --output-format csv -d DIR/{wl}_{c.split('_')[0].lower()} -o run -- "
               f"python3 bench.py --workload {wl} --steps 2 --warmup 1 --no-cpu-baseline{extra}"
               for c in ("FETCH_SIZE", "WRITE_SIZE")]
    md += ["python bench.py --summarize-traffic DIR", "```", "",
           f"Calibration: a 1 GiB elementwise read+write reads {copy['fetch']:.0f} KiB (FETCH_SIZE) and writes "
           f"{copy['write']:.0f} KiB (WRITE_SIZE); factors {fetch_factor:.4f} and {write_factor:.4f} turn "
           "counter KiB into bytes.", "",
           "| workload | stage | kernels | read MB | written MB | total MB per launch |", "|---|---|---|---|---|---|"]
    for wl, stages in STAGE_KERNELS.items():
        fm = _per_kernel_median(_counter_rows(os.path.join(d, f"{wl}_fetch")))
        wm = _per_kernel_median(_counter_rows(os.path.join(d, f"{wl}_write")))
        if not fm or not wm:
            continue
        out[wl] = {}
        for stage, spec in stages.items():
            pat, src = spec[0], spec[1]
            per_call = spec[2] if len(spec) > 2 else 1          # launches of each kernel per stage call
            names = sorted(k for k in fm if "msa::" in k and any(p in k for p in pat.split("|")))
            if not names:
                continue

            def launches(name):
                if isinstance(per_call, dict):
                    return next(n for p, n in per_call.items() if p in name)
                return per_call

            rd = sum(launches(k) * fm[k] for k in names) * 1024 * fetch_factor
            wr = sum(launches(k) * wm.get(k, 0.0) for k in names) * 1024 * write_factor
            out[wl][stage] = {"source_sha": kernel_source_sha(src), "read_bytes": rd, "write_bytes": wr,
                              "bytes_per_launch": rd + wr, "kernels": names}
            short = ", ".join(sorted({_short_kernel(n) for n in names}))
            md.append(f"| {wl} | {stage} | `{short}` | {rd / 1e6:.1f} | {wr / 1e6:.1f} | {(rd + wr) / 1e6:.1f} |")
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(out, f, indent=1)
    with open(os.path.join(ROOT, "profiles", "hbm-traffic_per-stage_all-workloads.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    print(json.dumps(out, indent=1))


N_XCD, N_CU = 8, 256      # MI355X: 8 XCDs, 256 CUs (4 SIMDs each)


def summarize_counters(out_md, title, commands, dirs):
    """Per-kernel medians of every counter in the rocprofv3 --pmc runs under
    `dirs`, and the ratios read from them:
      MFMA busy  = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs)
      VALU, LDS, wait fractions = SQ_ACTIVE_INST_VALU, SQ_ACTIVE_INST_LDS, SQ_WAIT_INST_ANY
                   over SQ_WAVE_CYCLES (per-wave shares of its lifetime)
      bank-conflict share = SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS
      VALU per MFMA = SQ_INSTS_VALU / SQ_INSTS_MFMA (SQ_INSTS_VALU counts the MFMAs too)."""
    import csv
    import glob
    vals = {}
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    if "msa::" not in r["Kernel_Name"]:
                        continue
                    key = (_short_kernel(r["Kernel_Name"]), r["Counter_Name"])
                    vals.setdefault(key, []).append(float(r["Counter_Value"]))
    med = {k: _median(v) for k, v in vals.items()}
    kernels = sorted({k for k, _ in med})
    names = sorted({c for _, c in med})
    g = lambda k, c: med.get((k, c))

    def ratio(a, b, scale=1.0):
        return None if a is None or not b else a / (b * scale)
    lines = [f"# {title}", "", "Commands (repository root, one MI355X):", "", "```", *commands, "```", "",
             "Derived (medians over dispatches): MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs "
             "x 1024 SIMDs); VALU / LDS / wait = SQ_ACTIVE_INST_VALU, SQ_ACTIVE_INST_LDS, SQ_WAIT_INST_ANY over "
             "SQ_WAVE_CYCLES; conflict = SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS; VALU/MFMA = SQ_INSTS_VALU / "
             "SQ_INSTS_MFMA (SQ_INSTS_VALU includes the MFMAs).", "",
             "| kernel | MFMA busy | VALU | LDS | wait | LDS conflict | VALU/MFMA |", "|---|---|---|---|---|---|---|"]
    fmt = lambda x: "—" if x is None else f"{x:.3f}"
    for k in kernels:
        busy = ratio(g(k, "SQ_VALU_MFMA_BUSY_CYCLES"), g(k, "GRBM_GUI_ACTIVE"), 4 * N_CU / N_XCD)
        wc = g(k, "SQ_WAVE_CYCLES")
        lines.append(f"| `{k}` | {fmt(busy)} | {fmt(ratio(g(k, 'SQ_ACTIVE_INST_VALU'), wc))} | "
                     f"{fmt(ratio(g(k, 'SQ_ACTIVE_INST_LDS'), wc))} | {fmt(ratio(g(k, 'SQ_WAIT_INST_ANY'), wc))} | "
                     f"{fmt(ratio(g(k, 'SQ_LDS_BANK_CONFLICT'), g(k, 'SQ_ACTIVE_INST_LDS')))} | "
                     f"{fmt(ratio(g(k, 'SQ_INSTS_VALU'), g(k, 'SQ_INSTS_MFMA')))} |")
    lines += ["", "Raw medians per dispatch:", "", "| kernel | " + " | ".join(names) + " |",
              "|---|" + "---|" * len(names)]
    for k in kernels:
        lines.append(f"| `{k}` | " + " | ".join("—" if g(k, c) is None else f"{g(k, c):.4g}" for c in names) + " |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_stats(csv_path, out_md, title, command):
    import csv
    with open(csv_path) as fh:
        rows = list(csv.DictReader(fh))
    ours, other_ns = [], 0
    for r in rows:
        if "msa::" not in r["Name"]:
            other_ns += int(r["TotalDurationNs"])
            continue
        ours.append((_short_kernel(r["Name"]), int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]),
                     float(r["MaxNs"]), int(r["TotalDurationNs"])))
    with open(out_md, "w") as f:
        f.write(f"# {title}\n\nCommand (repository root, one MI355X):\n\n```\n{command}\n```\n\n")
        f.write("| kernel | calls | avg us | min us | max us | total us |\n|---|---|---|---|---|---|\n")
        for name, c, a, mn, mx, t in sorted(ours, key=lambda x: -x[5]):
            f.write(f"| `{name}` | {c} | {a / 1e3:.1f} | {mn / 1e3:.1f} | {mx / 1e3:.1f} | {t / 1e3:.1f} |\n")
        f.write(f"\nOther kernels (torch input synthesis, copies): {other_ns / 1e3:.1f} us total.\n")


def copy_probe():
    import torch
    n = COPY_PROBE_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print("copy probe done", float(dst[0]))


# ---------------------------------------------------------------------------
# the GPU step
# ---------------------------------------------------------------------------

class Step:
    """Preallocated buffers and the sequence of ABI calls of one step."""

    def __init__(self, cfg, workload, seed, dev, rounds=1):
        import torch
        import msa_inputs as mi
        import routed_sparse_attention_msa_amd as msa
        self.torch, self.msa, self.cfg, self.workload, self.rounds = torch, msa, cfg, workload, rounds
        t = mi.draw_layer(cfg if workload != "decode" else mi.PREFILL, seed=seed, device=dev)
        if workload == "decode":
            d = mi.draw_layer(cfg, seed=seed + 1, device=dev, with_raw=False)
            for k in ("q", "k_loc", "v_loc", "q_r"):
                t[k] = d[k]
        self.t = t
        cpd = cfg.chunks_per_doc
        e = lambda *shape, dt=torch.bfloat16: torch.empty(shape, dtype=dt, device=dev)
        self.kbar = e(cfg.n_chunks, cfg.heads_kv, cfg.dim)
        self.vbar = e(cfg.n_chunks, cfg.heads_kv, cfg.dim)
        self.kbar_r = e(cfg.n_chunks, cfg.heads_kv, cfg.dim)
        self.knorm = e(cfg.n_chunks, cfg.heads_kv, dt=torch.float32)
        self._pool()
        if "q_r" not in t:
            t["q_r"] = mi.plant_router_queries(self.kbar_r, t["planted"], t["q_r_noise"], cfg)
        if workload == "interleave":
            # round r > 0: its own planted documents and noise (a later seed)
            qs = [t["q_r"]]
            for r in range(1, rounds):
                d = mi.draw_layer(cfg, seed=seed + 100 * r, device=dev, with_raw=False)
                qs.append(mi.plant_router_queries(self.kbar_r, d["planted"], d["q_r_noise"], cfg))
            t["q_r_rounds"] = torch.stack(qs).contiguous()
        kk = rounds * cfg.topk
        self.scores = e(cfg.batch, cfg.n_doc, dt=torch.float32)
        self.ids = e(cfg.batch, kk, dt=torch.int32)
        self.top = e(cfg.batch, kk, dt=torch.float32)
        self.k_sel = e(cfg.batch, rounds * cfg.mem_len, cfg.heads_kv, cfg.dim)
        self.v_sel = e(cfg.batch, rounds * cfg.mem_len, cfg.heads_kv, cfg.dim)
        self.out = torch.empty_like(t["q"])
        self.lse = e(cfg.batch, cfg.heads_q, cfg.q_len, dt=torch.float32)
        u8 = lambda n: torch.empty(max(n, 16), dtype=torch.uint8, device=dev)
        self.ws_route = u8(msa.msa_route_scores_workspace(cfg.batch, cfg.q_len, cfg.heads_kv, cfg.dim,
                                                          cfg.n_doc, cpd, torch.bfloat16))
        self.ws_topk = u8(msa.msa_topk_docs_workspace(cfg.batch, cfg.n_doc, cfg.topk))
        self.ws_attn = u8(msa.msa_sparse_attn_workspace(cfg.batch, cfg.q_len, cfg.heads_q, cfg.heads_kv,
                                                        cfg.dim, rounds * cfg.mem_len, cfg.loc_len,
                                                        torch.bfloat16))
        if workload == "interleave":
            self.ws_rounds = u8(msa.msa_route_rounds_workspace(rounds, cfg.batch, cfg.q_len, cfg.heads_kv,
                                                               cfg.dim, cfg.n_doc, cpd, cfg.topk,
                                                               torch.bfloat16))
        torch.cuda.synchronize()

    def _pool(self):
        c = self.cfg.chunk
        self.msa.msa_pool_chunks(self.t["k"], c, xbar=self.kbar)
        self.msa.msa_pool_chunks(self.t["v"], c, xbar=self.vbar)
        self.msa.msa_pool_chunks(self.t["k_r"], c, xbar=self.kbar_r, xbar_norm=self.knorm)

    def calls(self):
        """(stage, callable) in step order."""
        msa, t, cfg, c = self.msa, self.t, self.cfg, self.cfg.chunk
        seq = []
        if self.workload == "interleave":
            seq += [("rounds", lambda: msa.msa_route_rounds(t["q_r_rounds"], self.kbar_r, self.knorm,
                                                            cfg.chunks_per_doc, cfg.topk, topk_ids=self.ids,
                                                            topk_scores=self.top, ws=self.ws_rounds))]
        else:
            seq += [
                ("route", lambda: msa.msa_route_scores(t["q_r"], self.kbar_r, self.knorm, cfg.chunks_per_doc,
                                                       doc_scores=self.scores, ws=self.ws_route)),
                ("topk", lambda: msa.msa_topk_docs(self.scores, cfg.topk, topk_ids=self.ids,
                                                   topk_scores=self.top, ws=self.ws_topk))]
        seq += [
            ("gather", lambda: msa.msa_gather_kv(self.kbar, self.vbar, self.ids, cfg.chunks_per_doc,
                                                 k_sel=self.k_sel, v_sel=self.v_sel)),
            ("attn", lambda: msa.msa_sparse_attn(t["q"], self.k_sel, self.v_sel, t["k_loc"], t["v_loc"],
                                                 out=self.out, lse=self.lse, ws=self.ws_attn)),
        ]
        return seq

    def pool_calls(self):
        """The offline stage (S1): pool K, V and K_r (+ norms) into the bank."""
        msa, t, c = self.msa, self.t, self.cfg.chunk
        return [("pool", lambda: msa.msa_pool_chunks(t["k"], c, xbar=self.kbar)),
                ("pool", lambda: msa.msa_pool_chunks(t["v"], c, xbar=self.vbar)),
                ("pool", lambda: msa.msa_pool_chunks(t["k_r"], c, xbar=self.kbar_r, xbar_norm=self.knorm))]

    def run(self, steps, events, seq=None):
        torch = self.torch
        seq = self.calls() if seq is None else seq
        marks = []
        for _ in range(steps):
            for stage, fn in seq:
                if events:
                    a = torch.cuda.Event(enable_timing=True)
                    b = torch.cuda.Event(enable_timing=True)
                    a.record()
                    fn()
                    b.record()
                    marks.append((stage, a, b))
                else:
                    fn()
        return marks


class EncodeStep:
    """Offline encoder over variable-length documents: the seeded recipe draws
    2048 lengths uniform in [256, 768] (about 1M tokens) and N(0,1)/sqrt(128)
    bf16 rows for K, V and K_r; K is rotated at document-local positions."""

    N_DOCS, LEN_LO, LEN_HI, HEADS, DIM, CHUNK, ROPE_BASE = 2048, 256, 768, 8, 128, 64, 1.0e6

    def __init__(self, seed, dev):
        import numpy as np
        import torch
        import routed_sparse_attention_msa_amd as msa
        self.torch, self.msa = torch, msa
        rng = np.random.default_rng(seed)
        lens = rng.integers(self.LEN_LO, self.LEN_HI + 1, self.N_DOCS)
        self.doc_off_h = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        self.rows = int(self.doc_off_h[-1])
        self.chunks = int(((lens + self.CHUNK - 1) // self.CHUNK).sum())
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        mk = lambda: (torch.randn((self.rows, self.HEADS, self.DIM), generator=g, device=dev)
                      / math.sqrt(self.DIM)).to(torch.bfloat16)
        self.k, self.v, self.k_r = mk(), mk(), mk()
        self.doc_off = torch.as_tensor(self.doc_off_h, device=dev)
        self.chunk_off = torch.empty_like(self.doc_off)
        e = lambda: torch.empty((self.chunks, self.HEADS, self.DIM), dtype=torch.bfloat16, device=dev)
        self.kbar, self.vbar, self.kbar_r = e(), e(), e()
        self.knorm = torch.empty((self.chunks, self.HEADS), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()

    def calls(self):
        msa, c = self.msa, self.CHUNK
        enc = lambda x, out, rope, norm: msa.msa_encode_docs(x, self.doc_off, self.chunk_off, self.chunks, c,
                                                             rope_base=rope, xbar=out, xbar_norm=norm)
        return [("offsets", lambda: msa.msa_chunk_offsets(self.doc_off, c, chunk_off=self.chunk_off)),
                ("encode_rope", lambda: enc(self.k, self.kbar, self.ROPE_BASE, None)),
                ("encode", lambda: enc(self.v, self.vbar, 0.0, None)),
                ("encode", lambda: enc(self.k_r, self.kbar_r, 0.0, self.knorm))]

    run = Step.run

    def work(self, stage):
        rb = self.HEADS * self.DIM * 2
        if stage == "offsets":
            return {"bound": "hbm", "bytes": 2 * 8 * (self.N_DOCS + 1), "flops": 0}
        # K (rotated) alone; V and K_r (+ norms) averaged
        b = self.rows * rb + self.chunks * rb + (0 if stage == "encode_rope" else self.chunks * self.HEADS * 2)
        return {"bound": "hbm", "bytes": b, "flops": self.rows * self.HEADS * self.DIM}

    def cpu_baseline(self):
        from oracle import encode_docs
        # every document: about 10 s of float64 work on the host
        docs = range(self.N_DOCS)
        secs, rows = 0.0, 0
        for n in docs:
            a, b = int(self.doc_off_h[n]), int(self.doc_off_h[n + 1])
            rows += b - a
            for x, rope in ((self.k, self.ROPE_BASE), (self.v, None), (self.k_r, None)):
                xs = x[a:b].float().cpu().double().numpy()
                t0 = time.perf_counter()
                encode_docs(xs, [0, b - a], self.CHUNK, rope)
                secs += time.perf_counter() - t0
        return {"value": rows / secs, "unit": "encoded tokens/s", **host_threads(), "kind": "oracle",
                "sample": f"the whole step: {self.N_DOCS} documents ({rows} rows) x 3 tensors",
                "seconds_per_step": secs}


class BackwardStep:
    """Attention forward + backward at the prefill layer's shapes (a training
    step of the routed layer's attention; the gathered memory rows are drawn
    directly, N(0,1)/sqrt(128) like every other value, and dL/dO is N(0,1))."""

    def __init__(self, seed, dev):
        import torch
        import msa_inputs as mi
        import routed_sparse_attention_msa_amd as msa
        self.torch, self.msa, self.cfg = torch, msa, mi.PREFILL
        cfg = self.cfg
        t = mi.draw_layer(cfg, seed=seed, device=dev, with_raw=False)
        g = torch.Generator(device=dev)
        g.manual_seed(seed + 7)
        mem = (cfg.batch, cfg.mem_len, cfg.heads_kv, cfg.dim)
        self.q, self.k_loc, self.v_loc = t["q"], t["k_loc"], t["v_loc"]
        self.k_sel = (torch.randn(mem, generator=g, device=dev) * cfg.value_scale).to(torch.bfloat16)
        self.v_sel = (torch.randn(mem, generator=g, device=dev) * cfg.value_scale).to(torch.bfloat16)
        self.d_out = torch.randn(self.q.shape, generator=g, device=dev).to(torch.bfloat16)
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty((cfg.batch, cfg.heads_q, cfg.q_len), dtype=torch.float32, device=dev)
        self.grads = (torch.empty_like(self.q), torch.empty_like(self.k_sel), torch.empty_like(self.v_sel),
                      torch.empty_like(self.k_loc), torch.empty_like(self.v_loc))
        u8 = lambda n: torch.empty(max(n, 16), dtype=torch.uint8, device=dev)
        self.ws = u8(msa.msa_sparse_attn_backward_workspace(cfg.batch, cfg.q_len, cfg.heads_q, cfg.heads_kv,
                                                            cfg.dim, cfg.mem_len, cfg.loc_len, torch.bfloat16))
        torch.cuda.synchronize()

    def calls(self):
        msa = self.msa
        return [("attn", lambda: msa.msa_sparse_attn(self.q, self.k_sel, self.v_sel, self.k_loc, self.v_loc,
                                                     out=self.out, lse=self.lse)),
                ("attn_bwd", lambda: msa.msa_sparse_attn_backward(self.q, self.k_sel, self.v_sel, self.k_loc,
                                                                  self.v_loc, self.out, self.lse, self.d_out,
                                                                  grads=self.grads, ws=self.ws))]

    run = Step.run

    def work(self, stage):
        fwd = work_attn(self.cfg)
        if stage == "attn":
            return fwd
        # flash-attention accounting: S recomputed, dP, dQ, dK, dV = 2.5 x the forward's products;
        # bytes: q, k, v, o, dO, lse read, dq, dk, dv written
        c = self.cfg
        row_kv = c.heads_kv * c.dim * 2
        q_b = c.batch * c.q_len * c.heads_q * c.dim * 2
        kv_b = 2 * c.batch * (c.mem_len + c.loc_len) * row_kv
        b = 4 * q_b + 2 * kv_b + c.batch * c.heads_q * c.q_len * 4
        return {"bound": "mfma", "bytes": b, "flops": 2.5 * fwd["flops"]}

    def cpu_baseline(self):
        import numpy as np
        from oracle import sparse_attention_backward
        c = self.cfg
        f = lambda x: x.detach().float().cpu().double().numpy()
        # one KV group (its 4 query heads) of the 8, scaled to all of them
        gs, hs = slice(0, 1), slice(0, c.heads_q // c.heads_kv)
        args = [f(self.q[:, :, hs]), f(self.k_sel[:, :, gs]), f(self.v_sel[:, :, gs]), f(self.k_loc[:, :, gs]),
                f(self.v_loc[:, :, gs]), f(self.d_out[:, :, hs])]
        t0 = time.perf_counter()
        sparse_attention_backward(*args, scale=1.0 / math.sqrt(c.dim))
        secs = (time.perf_counter() - t0) * c.heads_kv
        tokens = c.batch * c.q_len
        return {"value": tokens / secs, "unit": "query tokens/s", **host_threads(), "kind": "oracle",
                "sample": f"backward of 1 of {c.heads_kv} KV groups (all tokens), scaled to all groups; "
                          "the forward not timed",
                "seconds_per_step": secs}


class LinearStep:
    """Linear-layer variant on the 1M-token bank (decode shape): the router
    bank and queries follow decode-1M-bf16; each document's state comes from
    the gated delta rule over its 512 tokens (K unit-norm, V N(0,1)/sqrt(128),
    log-decay -U(0, 0.1), beta U(0, 1)), encoded once before timing; the query
    token's q, k, v, gates are drawn the same way."""

    def __init__(self, seed, dev):
        import torch
        import msa_inputs as mi
        import routed_sparse_attention_msa_amd as msa
        self.torch, self.msa, self.cfg = torch, msa, mi.DECODE
        c = self.cfg
        base = mi.draw_layer(mi.PREFILL, seed=seed, device=dev)
        t = mi.draw_layer(c, seed=seed + 1, device=dev, with_raw=False)
        self.kbar_r = torch.empty((c.n_chunks, c.heads_kv, c.dim), dtype=torch.bfloat16, device=dev)
        self.knorm = torch.empty((c.n_chunks, c.heads_kv), dtype=torch.float32, device=dev)
        msa.msa_pool_chunks(base["k_r"], c.chunk, xbar=self.kbar_r, xbar_norm=self.knorm)
        self.q_r = t["q_r"]
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed + 5)
        h, d = c.heads_kv, c.dim

        def seq(n, t_len):
            k = torch.randn((n, t_len, h, d), generator=gen, device=dev)
            k = (k / torch.linalg.vector_norm(k, dim=-1, keepdim=True)).to(torch.bfloat16)
            v = (torch.randn((n, t_len, h, d), generator=gen, device=dev) / math.sqrt(d)).to(torch.bfloat16)
            g = -0.1 * torch.rand((n, t_len, h), generator=gen, device=dev)
            b = torch.rand((n, t_len, h), generator=gen, device=dev)
            return k, v, g, b

        # offline: every document's state (outputs not needed)
        dk_, dv_, dg, db = seq(c.n_doc, c.doc_len)
        self.doc_states = torch.empty((c.n_doc, h, d, d), dtype=torch.float32, device=dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        # token-by-token form first (its time is reported beside the chunked one), then the chunked
        # form whose states the step uses
        e0.record()
        msa.msa_gated_delta_rule(None, dk_, dv_, dg, db, final_state=self.doc_states, with_out=False)
        e1.record()
        torch.cuda.synchronize()
        self.encode_recurrent_ms = e0.elapsed_time(e1)
        msa.msa_gated_delta_rule_chunked(None, dk_, dv_, dg, db, final_state=self.doc_states, with_out=False)
        torch.cuda.synchronize()
        e0.record()
        msa.msa_gated_delta_rule_chunked(None, dk_, dv_, dg, db, final_state=self.doc_states, with_out=False)
        e1.record()
        torch.cuda.synchronize()
        self.encode_ms = e0.elapsed_time(e1)
        del dk_, dv_, dg, db
        self.k, self.v, self.g, self.beta = seq(c.batch, c.q_len)
        self.q = (torch.randn((c.batch, c.q_len, h, d), generator=gen, device=dev) / math.sqrt(d)).to(torch.bfloat16)
        self.scores = torch.empty((c.batch, c.n_doc), dtype=torch.float32, device=dev)
        self.ids = torch.empty((c.batch, c.topk), dtype=torch.int32, device=dev)
        self.s_ext = torch.empty((c.batch, h, d, d), dtype=torch.float32, device=dev)
        self.out = torch.empty((c.batch, c.q_len, h, d), dtype=torch.bfloat16, device=dev)
        self.final = torch.empty_like(self.s_ext)
        u8 = lambda n: torch.empty(max(n, 16), dtype=torch.uint8, device=dev)
        self.ws_route = u8(msa.msa_route_scores_workspace(c.batch, c.q_len, h, d, c.n_doc, c.chunks_per_doc,
                                                          torch.bfloat16))
        self.ws_topk = u8(msa.msa_topk_docs_workspace(c.batch, c.n_doc, c.topk))
        torch.cuda.synchronize()

    def calls(self):
        msa, c = self.msa, self.cfg
        return [("route", lambda: msa.msa_route_scores(self.q_r, self.kbar_r, self.knorm, c.chunks_per_doc,
                                                       doc_scores=self.scores, ws=self.ws_route)),
                ("topk", lambda: msa.msa_topk_docs(self.scores, c.topk, topk_ids=self.ids, with_scores=False,
                                                   ws=self.ws_topk)),
                ("state_sum", lambda: msa.msa_gdn_state_sum(self.doc_states, self.ids, s_ext=self.s_ext)),
                ("gdn", lambda: msa.msa_gated_delta_rule(self.q, self.k, self.v, self.g, self.beta,
                                                         initial_state=self.s_ext, out=self.out,
                                                         final_state=self.final))]

    run = Step.run

    def work(self, stage):
        c = self.cfg
        st = c.heads_kv * c.dim * c.dim * 4
        if stage == "route":
            return work_route(c)
        if stage == "topk":
            return work_topk(c)
        if stage == "state_sum":
            return {"bound": "hbm", "bytes": c.batch * (c.topk + 1) * st + c.batch * c.topk * 4, "flops": 0}
        # one step per sequence: the state read and written, q/k/v/out
        b = 2 * c.batch * st + 4 * c.batch * c.q_len * c.heads_kv * c.dim * 2
        return {"bound": "hbm", "bytes": b, "flops": 6 * c.batch * c.q_len * c.heads_kv * c.dim * c.dim}

    def cpu_baseline(self):
        import numpy as np
        from oracle import gated_delta_rule, inject_states, route_scores, topk_docs
        c = self.cfg
        f = lambda x: x.detach().float().cpu().double().numpy()
        # the whole step (the selected documents' states copied to the host first, untimed)
        q_r, kb = f(self.q_r), f(self.kbar_r)
        t0 = time.perf_counter()
        sc = route_scores(q_r, kb, c.chunks_per_doc)
        ids, _ = topk_docs(sc, c.topk)
        secs = time.perf_counter() - t0
        st = f(self.doc_states[self.ids.flatten().long()])
        t0 = time.perf_counter()
        s_ext = inject_states(st, np.arange(c.batch * c.topk).reshape(c.batch, c.topk))
        gated_delta_rule(f(self.q), f(self.k), f(self.v), f(self.g), f(self.beta), initial_state=s_ext)
        secs += time.perf_counter() - t0
        return {"value": c.batch * c.q_len / secs, "unit": "query tokens/s", **host_threads(), "kind": "oracle",
                "sample": "the whole step (route over all documents, top-k, state sum and the step for all "
                          f"{c.batch} sequences)", "seconds_per_step": secs}


class StackStep:
    """The 18-layer stack at a 10M-token memory: every layer has its own bank
    (19,532 documents x 512 tokens, 8 KV heads x 128, bf16, N(0,1) values),
    router queries, queries and local KV (8192-token prefill), and routes
    independently.  Each layer's raw K, V and K_r are drawn in slabs of 512
    documents and pooled on the GPU as they are drawn (the offline stage,
    outside the step).  One step: route -> top-32 -> gather -> attention for
    each of the 18 layers."""

    SLAB_DOCS = 512

    def __init__(self, seed, dev):
        import torch
        import msa_inputs as mi
        import routed_sparse_attention_msa_amd as msa
        self.torch, self.msa, self.cfg = torch, msa, mi.STACK18
        cfg = self.cfg
        cpd, n_ch, hkv, d = cfg.chunks_per_doc, cfg.n_chunks, cfg.heads_kv, cfg.dim
        e = lambda *shape, dt=torch.bfloat16: torch.empty(shape, dtype=dt, device=dev)
        u8 = lambda n: torch.empty(max(n, 16), dtype=torch.uint8, device=dev)
        self.layers = []
        t0 = time.perf_counter()
        for layer in range(cfg.layers):
            t = mi.draw_layer(cfg, seed=seed + 1000 * layer, device=dev, with_raw=False)
            g = torch.Generator(device=dev)
            g.manual_seed(seed + 1000 * layer + 1)
            L = {"q": t["q"], "k_loc": t["k_loc"], "v_loc": t["v_loc"], "q_r": t["q_r"],
                 "kbar": e(n_ch, hkv, d), "vbar": e(n_ch, hkv, d), "kbar_r": e(n_ch, hkv, d),
                 "knorm": e(n_ch, hkv, dt=torch.float32)}
            for name in ("kbar", "vbar", "kbar_r"):
                for d0 in range(0, cfg.n_doc, self.SLAB_DOCS):
                    d1 = min(cfg.n_doc, d0 + self.SLAB_DOCS)
                    raw = (torch.randn((d1 - d0, cfg.doc_len, hkv, d), generator=g, device=dev)
                           * cfg.value_scale).to(torch.bfloat16)
                    dst = L[name][d0 * cpd:d1 * cpd]
                    if name == "kbar_r":
                        msa.msa_pool_chunks(raw, cfg.chunk, xbar=dst, xbar_norm=L["knorm"][d0 * cpd:d1 * cpd])
                    else:
                        msa.msa_pool_chunks(raw, cfg.chunk, xbar=dst)
                    del raw
            L["out"] = torch.empty_like(t["q"])
            L["lse"] = e(cfg.batch, cfg.heads_q, cfg.q_len, dt=torch.float32)
            self.layers.append(L)
            torch.cuda.synchronize()
        self.pool_s = time.perf_counter() - t0
        self.scores = e(cfg.batch, cfg.n_doc, dt=torch.float32)
        self.ids = e(cfg.batch, cfg.topk, dt=torch.int32)
        self.top = e(cfg.batch, cfg.topk, dt=torch.float32)
        self.k_sel = e(cfg.batch, cfg.mem_len, hkv, d)
        self.v_sel = e(cfg.batch, cfg.mem_len, hkv, d)
        self.ws_route = u8(msa.msa_route_scores_workspace(cfg.batch, cfg.q_len, hkv, d, cfg.n_doc, cpd,
                                                          torch.bfloat16))
        self.ws_topk = u8(msa.msa_topk_docs_workspace(cfg.batch, cfg.n_doc, cfg.topk))
        self.ws_attn = u8(msa.msa_sparse_attn_workspace(cfg.batch, cfg.q_len, cfg.heads_q, hkv, d, cfg.mem_len,
                                                        cfg.loc_len, torch.bfloat16))
        torch.cuda.synchronize()

    def calls(self):
        msa, cfg, cpd = self.msa, self.cfg, self.cfg.chunks_per_doc
        seq = []
        for L in self.layers:
            seq += [
                ("route", lambda L=L: msa.msa_route_scores(L["q_r"], L["kbar_r"], L["knorm"], cpd,
                                                           doc_scores=self.scores, ws=self.ws_route)),
                ("topk", lambda: msa.msa_topk_docs(self.scores, cfg.topk, topk_ids=self.ids, topk_scores=self.top,
                                                   ws=self.ws_topk)),
                ("gather", lambda L=L: msa.msa_gather_kv(L["kbar"], L["vbar"], self.ids, cpd, k_sel=self.k_sel,
                                                         v_sel=self.v_sel)),
                ("attn", lambda L=L: msa.msa_sparse_attn(L["q"], self.k_sel, self.v_sel, L["k_loc"], L["v_loc"],
                                                         out=L["out"], lse=L["lse"], ws=self.ws_attn)),
            ]
        return seq

    run = Step.run

    def work(self, stage):
        return {"route": work_route, "topk": work_topk, "gather": work_gather, "attn": work_attn}[stage](self.cfg)

    def cpu_baseline(self):
        """The oracle on one layer's bounded sample, scaled to the layer and then to the 18 layers."""
        import numpy as np
        from oracle import route_scores, sparse_attention_rows, topk_docs
        cfg, L, torch = self.cfg, self.layers[0], self.torch
        f = lambda x: x.detach().float().cpu().double().numpy()
        rng = np.random.default_rng(0)
        cpd = cfg.chunks_per_doc
        secs = 0.0
        n_route = 16
        sample = rng.choice(cfg.n_doc, n_route, replace=False)
        rows = torch.as_tensor((sample[:, None] * cpd + np.arange(cpd)).ravel(), device=L["kbar_r"].device)
        kb, q_r = f(L["kbar_r"][rows]), f(L["q_r"])
        t0 = time.perf_counter()
        route_scores(q_r, kb, cpd)
        secs += (time.perf_counter() - t0) * cfg.n_doc / n_route
        self.msa.msa_route_scores(L["q_r"], L["kbar_r"], L["knorm"], cpd, doc_scores=self.scores, ws=self.ws_route)
        self.msa.msa_topk_docs(self.scores, cfg.topk, topk_ids=self.ids, topk_scores=self.top, ws=self.ws_topk)
        self.msa.msa_gather_kv(L["kbar"], L["vbar"], self.ids, cpd, k_sel=self.k_sel, v_sel=self.v_sel)
        sc = f(self.scores)
        t0 = time.perf_counter()
        topk_docs(sc, cfg.topk)
        secs += time.perf_counter() - t0
        ks, vs, kl, vl, q = f(self.k_sel), f(self.v_sel), f(L["k_loc"]), f(L["v_loc"]), f(L["q"])
        n_rows_total = cfg.q_len * cfg.heads_q
        n_att = 256
        g = cfg.heads_q // cfg.heads_kv
        picks = rng.integers(0, n_rows_total, n_att)
        t0 = time.perf_counter()
        for r in picks:
            h, tt = int(r % cfg.heads_q), int(r // cfg.heads_q)
            n_loc = cfg.loc_len - cfg.q_len + tt + 1
            keys = np.concatenate([ks[0, :, h // g], kl[0, :n_loc, h // g]])
            vals = np.concatenate([vs[0, :, h // g], vl[0, :n_loc, h // g]])
            sparse_attention_rows(q[0, tt, h], keys, vals, 1.0 / math.sqrt(cfg.dim))
        secs += (time.perf_counter() - t0) * n_rows_total / n_att
        secs *= cfg.layers
        return {"value": cfg.q_len / secs, "unit": "query tokens/s", **host_threads(), "kind": "oracle",
                "sample": (f"layer 0: route all {cfg.q_len} tokens vs {n_route}/{cfg.n_doc} docs; top-k whole; "
                           f"attention {n_att}/{n_rows_total} rows; each stage scaled to the layer, the layer "
                           f"to the {cfg.layers} layers"),
                "seconds_per_step": secs}


class ScanStep:
    """The routing scan at one GPU's share of a 100M-token memory
    (scan-100M-share-bf16): 195,313 documents x 512 tokens drawn around 1024
    Gaussian cluster centres (sigma 0.3) in slabs and pooled on the GPU into a
    3.2 GB router bank (the offline stage, timed apart); the pooled content
    K-bar / V-bar in pinned host memory (6.4 GB, doc-major).  One step: route
    4 x 512 router query tokens over the whole bank -> top-16 per sequence ->
    fetch of the 64 selected documents' content from the host tier (the GPU
    reads the pinned rows directly)."""

    SLAB = 2048

    def __init__(self, seed, dev):
        import torch
        import msa_inputs as mi
        import routed_sparse_attention_msa_amd as msa
        self.torch, self.msa, self.mi, self.cfg, self.dev = torch, msa, mi, mi.SCAN100M, dev
        cfg = self.cfg
        cpd, n_ch, hkv, d = cfg.chunks_per_doc, cfg.n_chunks, cfg.heads_kv, cfg.dim
        e = lambda *shape, dt=torch.bfloat16: torch.empty(shape, dtype=dt, device=dev)
        self.kbar_r = e(n_ch, hkv, d)
        self.knorm = e(n_ch, hkv, dt=torch.float32)
        t0 = time.perf_counter()
        for d0 in range(0, cfg.n_doc, self.SLAB):
            d1 = min(cfg.n_doc, d0 + self.SLAB)
            raw = mi.draw_scan_bank_slab(cfg, seed, d0, d1, dev)
            msa.msa_pool_chunks(raw, cfg.chunk, xbar=self.kbar_r[d0 * cpd:d1 * cpd],
                                xbar_norm=self.knorm[d0 * cpd:d1 * cpd])
            del raw
        torch.cuda.synchronize()
        self.pool_s = time.perf_counter() - t0
        t0 = time.perf_counter()
        self.hk = torch.empty((n_ch, hkv, d), dtype=torch.bfloat16, pin_memory=True)
        self.hv = torch.empty((n_ch, hkv, d), dtype=torch.bfloat16, pin_memory=True)
        for d0 in range(0, cfg.n_doc, 16384):
            d1 = min(cfg.n_doc, d0 + 16384)
            k, v = mi.draw_scan_content_slab(cfg, seed, d0, d1, dev)
            self.hk[d0 * cpd:d1 * cpd].copy_(k)
            self.hv[d0 * cpd:d1 * cpd].copy_(v)
        torch.cuda.synchronize()
        self.host_s = time.perf_counter() - t0
        self.q_r = mi.draw_scan_queries(cfg, seed, dev)
        self.bufs = [self._buffers() for _ in range(2)]     # two sets: the two-stream pipeline
        self.scores, self.ids, self.top = self.bufs[0]["scores"], self.bufs[0]["ids"], self.bufs[0]["top"]
        self.k_sel, self.v_sel = self.bufs[0]["k_sel"], self.bufs[0]["v_sel"]
        torch.cuda.synchronize()

    def _buffers(self):
        torch, msa, cfg, dev = self.torch, self.msa, self.cfg, self.dev
        e = lambda *shape, dt=torch.bfloat16: torch.empty(shape, dtype=dt, device=dev)
        u8 = lambda n: torch.empty(max(n, 16), dtype=torch.uint8, device=dev)
        return {"scores": e(cfg.batch, cfg.n_doc, dt=torch.float32), "ids": e(cfg.batch, cfg.topk, dt=torch.int32),
                "top": e(cfg.batch, cfg.topk, dt=torch.float32),
                "k_sel": e(cfg.batch, cfg.mem_len, cfg.heads_kv, cfg.dim),
                "v_sel": e(cfg.batch, cfg.mem_len, cfg.heads_kv, cfg.dim),
                "ws_route": u8(msa.msa_route_scores_workspace(cfg.batch, cfg.q_len, cfg.heads_kv, cfg.dim,
                                                              cfg.n_doc, cfg.chunks_per_doc, torch.bfloat16)),
                "ws_topk": u8(msa.msa_topk_docs_workspace(cfg.batch, cfg.n_doc, cfg.topk))}

    def _route(self, B):
        return lambda: self.msa.msa_route_scores(self.q_r, self.kbar_r, self.knorm, self.cfg.chunks_per_doc,
                                                 doc_scores=B["scores"], ws=B["ws_route"])

    def _topk(self, B):
        return lambda: self.msa.msa_topk_docs(B["scores"], self.cfg.topk, topk_ids=B["ids"], topk_scores=B["top"],
                                              ws=B["ws_topk"])

    def _fetch(self, B, host_memcpy=False):
        return lambda: self.msa.msa_gather_kv(self.hk, self.hv, B["ids"], self.cfg.chunks_per_doc,
                                              k_sel=B["k_sel"], v_sel=B["v_sel"], host_memcpy=host_memcpy)

    def calls(self):
        B = self.bufs[0]
        return [("route", self._route(B)), ("topk", self._topk(B)), ("fetch", self._fetch(B))]

    run = Step.run

    def work(self, stage):
        cfg = self.cfg
        if stage == "fetch":      # the selected rows cross the host link once and land in HBM once
            b = 2 * cfg.batch * cfg.mem_len * cfg.heads_kv * cfg.dim * 2
            return {"bound": "hbm", "bytes": b + cfg.batch * cfg.topk * 4, "flops": 0}
        return {"route": work_route, "topk": work_topk}[stage](cfg)

    def sweep(self, reps):
        """Routing over the 3.2 GB bank at T_tot = 1, 4, 32, 128, 512, 2048 query
        tokens: where the scan is HBM-bound (T_tot below the ridge, about 315)
        and where it turns MFMA-bound."""
        torch, msa, cfg = self.torch, self.msa, self.cfg
        import dataclasses as dc
        q = self.q_r
        shapes = [(1, 1, q[:1, :1]), (4, 1, q[:, :1]), (32, 1, q[:, :8].reshape(32, 1, 8, 128)),
                  (128, 1, q[:, :32].reshape(128, 1, 8, 128)), (4, 128, q[:, :128]), (4, 512, q)]
        out = []
        for b, t, qq in shapes:
            qq = qq.contiguous()
            sc = torch.empty((b, cfg.n_doc), dtype=torch.float32, device=self.dev)
            ws = torch.empty(max(16, msa.msa_route_scores_workspace(b, t, cfg.heads_kv, cfg.dim, cfg.n_doc,
                                                                    cfg.chunks_per_doc, torch.bfloat16)),
                             dtype=torch.uint8, device=self.dev)
            fn = lambda: msa.msa_route_scores(qq, self.kbar_r, self.knorm, cfg.chunks_per_doc, doc_scores=sc, ws=ws)
            fn()
            ms = time_launches(fn, reps)
            w = work_route(dc.replace(cfg, batch=b, q_len=t))
            hbm = roofline_entry(dict(w, bound="hbm"), ms)
            mf = roofline_entry(dict(w, bound="mfma"), ms)
            out.append({"t_tot": b * t, "batch": b, "q_len": t, "path": "scan" if b * t <= 128 else "tiled",
                        "bound": w["bound"], "ms": ms, "bytes": w["bytes"], "flops": w["flops"],
                        "GB/s": hbm["achieved"], "frac_hbm": hbm["frac"], "TFLOP/s": mf["achieved"],
                        "frac_mfma": mf["frac"]})
            print(f"[bench] sweep T_tot={b * t}: {ms:.3f} ms, {hbm['achieved']:.0f} GB/s ({hbm['frac']:.3f} of HBM), "
                  f"{mf['achieved']:.0f} TFLOP/s", file=sys.stderr, flush=True)
        return out

    def host_tier(self, reps, units=8):
        """The host-tier fetch of the 64 selected documents (2 MiB of pooled
        content over the host link), both modes, alone and overlapped with the
        next unit's routing on a second stream."""
        import torch
        B = self.bufs[0]
        self._route(B)()
        self._topk(B)()
        torch.cuda.synchronize()
        nbytes = self.work("fetch")["bytes"]
        res = {"bytes": nbytes}
        for mode, memcpy in (("zero_copy", False), ("memcpy", True)):
            fn = self._fetch(B, memcpy)
            fn()
            walls = []

            def timed():
                t0 = time.perf_counter()
                fn()
                walls.append(time.perf_counter() - t0)
            ms = time_launches(timed, reps)
            res[mode] = {"fetch_ms": ms, "GB/s_pcie_inclusive": nbytes / (ms / 1e3) / 1e9,
                         "host_call_ms": 1e3 * _median(walls)}
        # pipelines of `units` steps over two streams: unit u routes on stream u % 2
        # while the host waits for unit u-1's ids and its copies run
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]

        def pipeline(fetch_mode):
            cur = torch.cuda.current_stream()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(cur)
            for st in streams:
                st.wait_stream(cur)
            for u in range(units + 1):
                if u < units:
                    Bu = self.bufs[u % 2]
                    with torch.cuda.stream(streams[u % 2]):
                        self._route(Bu)()
                        self._topk(Bu)()
                        if fetch_mode == "zero_copy":
                            self._fetch(Bu)()
                if u > 0 and fetch_mode == "memcpy":
                    with torch.cuda.stream(streams[(u - 1) % 2]):
                        self._fetch(self.bufs[(u - 1) % 2], True)()
            for st in streams:
                cur.wait_stream(st)
            b.record(cur)
            torch.cuda.synchronize()
            return a.elapsed_time(b) / units

        pipeline(None)
        base = _median([pipeline(None) for _ in range(3)])
        res["pipeline"] = {"units": units, "route_topk_ms_per_unit": base}
        for mode in ("zero_copy", "memcpy"):
            pipeline(mode)
            with_f = _median([pipeline(mode) for _ in range(3)])
            res["pipeline"][f"with_{mode}_fetch_ms_per_unit"] = with_f
            res["pipeline"][f"{mode}_fetch_exposed_ms"] = with_f - base
        return res

    def cpu_baseline(self):
        """The oracle on a bounded sample: all 4 x 512 tokens routed against 4096
        of the 195,313 documents (scaled to the bank), the whole top-k on the
        GPU's scores, and the gather of the 64 selected documents from the host
        bank."""
        import numpy as np
        from oracle import gather_kv, route_scores, topk_docs
        torch, cfg = self.torch, self.cfg
        f = lambda x: x.detach().float().cpu().double().numpy()
        rng = np.random.default_rng(0)
        cpd = cfg.chunks_per_doc
        n_route = 4096
        sample = rng.choice(cfg.n_doc, n_route, replace=False)
        rows = torch.as_tensor((sample[:, None] * cpd + np.arange(cpd)).ravel(), device=self.dev)
        kb, q_r = f(self.kbar_r[rows]), f(self.q_r)
        secs = 0.0
        t0 = time.perf_counter()
        route_scores(q_r, kb, cpd)
        secs += (time.perf_counter() - t0) * cfg.n_doc / n_route
        self._route(self.bufs[0])()
        self._topk(self.bufs[0])()
        sc = f(self.bufs[0]["scores"])
        t0 = time.perf_counter()
        ids, _ = topk_docs(sc, cfg.topk)
        secs += time.perf_counter() - t0
        raw = lambda t: t.view(torch.int16).numpy()
        t0 = time.perf_counter()
        gather_kv(raw(self.hk), raw(self.hv), ids, cpd)
        secs += time.perf_counter() - t0
        tokens = cfg.batch * cfg.q_len
        return {"value": tokens / secs, "unit": "query tokens/s", **host_threads(), "kind": "oracle",
                "sample": (f"route all {tokens} tokens vs {n_route}/{cfg.n_doc} docs (scaled to the bank); "
                           "top-k whole; gather of the 64 selected docs from the host bank"),
                "seconds_per_step": secs}


def main_scan(args):
    import torch
    print("[bench] building inputs for scan-100M-share-bf16 (pooling a 3.2 GB router bank, 6.4 GB of pinned "
          "host content)", file=sys.stderr, flush=True)
    step = ScanStep(args.seed, "cuda:0")
    print(f"[bench] bank pooled in {step.pool_s:.1f} s, host content in {step.host_s:.1f} s; warmup {args.warmup}",
          file=sys.stderr, flush=True)
    step.run(args.warmup, events=False)
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    marks = step.run(args.steps, events=True)
    end.record()
    torch.cuda.synchronize()
    eager_ms = start.elapsed_time(end) / args.steps
    print(f"[bench] timing {args.steps} graph replays", file=sys.stderr, flush=True)
    graph_ms = graph_replay_ms(step, args.steps)
    ms_per_step = graph_ms if graph_ms is not None else eager_ms
    stages = stage_summary(step, marks, args.steps)
    dom = max(stages, key=lambda k: stages[k]["ms_per_step"])
    roof = {k: stages[dom][k] for k in ("bound", "achieved", "peak", "unit", "frac")}
    roof.update({"kernel": dom, "avg_launch_ms": stages[dom]["avg_launch_ms"],
                 "traffic": measured_traffic("scan100m", dom)})
    sweep = host = None
    if not args.step_only:
        print("[bench] routing sweep over the 3.2 GB bank", file=sys.stderr, flush=True)
        sweep = step.sweep(max(5, min(args.steps, 20)))
        print("[bench] host-tier fetch, alone and overlapped", file=sys.stderr, flush=True)
        host = step.host_tier(max(5, min(args.steps, 20)))
    c = step.cfg
    rec = {
        "metric": "query tokens/s of the routing scan at a 100M-token share (3.2 GB router bank) with the "
                  "host-tier fetch of the selected documents",
        "value": c.batch * c.q_len / (ms_per_step / 1e3), "unit": "query tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step, "ms_per_step_eager": eager_ms,
        "step_timing": "hip graph replay" if graph_ms is not None else "eager", "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "scan-100M-share-bf16", "n_docs": c.n_doc, "doc_len": c.doc_len, "chunk": c.chunk,
                   "n_chunks": c.n_chunks, "heads_kv": c.heads_kv, "dim": c.dim, "batch": c.batch, "q_len": c.q_len,
                   "topk": c.topk, "clusters": c.clusters, "cluster_sigma": c.cluster_sigma,
                   "step": "route 4 x 512 tokens over the bank -> top-16 -> host-tier fetch (zero-copy) of the "
                           "64 selected docs",
                   "offline_pooling_s": step.pool_s},
        "roofline": roof, "stages": stages, "route_sweep": sweep, "host_tier": host,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = step.cpu_baseline()
    print(json.dumps(rec))


def main_stack(args):
    import torch
    print("[bench] building inputs for stack18-10M-bf16 (pooling 18 banks of 10M tokens)", file=sys.stderr,
          flush=True)
    step = StackStep(args.seed, "cuda:0")
    print(f"[bench] banks pooled in {step.pool_s:.1f} s; warmup {args.warmup}", file=sys.stderr, flush=True)
    step.run(args.warmup, events=False)
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    marks = step.run(args.steps, events=True)
    end.record()
    torch.cuda.synchronize()
    eager_ms = start.elapsed_time(end) / args.steps
    print(f"[bench] timing {args.steps} graph replays", file=sys.stderr, flush=True)
    graph_ms = graph_replay_ms(step, args.steps)
    ms_per_step = graph_ms if graph_ms is not None else eager_ms
    stages = stage_summary(step, marks, args.steps)
    dom = max(stages, key=lambda k: stages[k]["ms_per_step"])
    roof = {k: stages[dom][k] for k in ("bound", "achieved", "peak", "unit", "frac")}
    roof.update({"kernel": dom, "avg_launch_ms": stages[dom]["avg_launch_ms"],
                 "traffic": measured_traffic("stack", dom)})
    c = step.cfg
    rec = {
        "metric": "end-to-end query tokens/s of the 18-layer routed stack at 10M-token memory (prefill)",
        "value": c.batch * c.q_len / (ms_per_step / 1e3), "unit": "query tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step, "ms_per_step_eager": eager_ms,
        "step_timing": "hip graph replay" if graph_ms is not None else "eager", "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "stack18-10M-bf16", "layers": c.layers, "n_docs": c.n_doc, "doc_len": c.doc_len,
                   "chunk": c.chunk, "batch": c.batch, "q_len": c.q_len, "loc_len": c.loc_len,
                   "heads_q": c.heads_q, "heads_kv": c.heads_kv, "dim": c.dim, "topk": c.topk,
                   "mem_len": c.mem_len, "step": "(route -> top-32 -> gather -> attention) x 18 layers",
                   "offline_pooling_s": step.pool_s},
        "roofline": roof, "stages": stages,
        "cpu_baseline": None if args.no_cpu_baseline else step.cpu_baseline(),
    }
    print(json.dumps(rec))


def main_linear(args):
    import torch
    print("[bench] building inputs for linear-1M-decode-bf16 (encoding 2048 document states)", file=sys.stderr,
          flush=True)
    step = LinearStep(args.seed, "cuda:0")
    step.run(args.warmup, events=False)
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    marks = step.run(args.steps, events=True)
    end.record()
    torch.cuda.synchronize()
    eager_ms = start.elapsed_time(end) / args.steps
    print(f"[bench] timing {args.steps} graph replays", file=sys.stderr, flush=True)
    graph_ms = graph_replay_ms(step, args.steps)
    ms_per_step = graph_ms if graph_ms is not None else eager_ms
    stages = stage_summary(step, marks, args.steps)
    dom = max(stages, key=lambda k: stages[k]["ms_per_step"])
    roof = {k: stages[dom][k] for k in ("bound", "achieved", "peak", "unit", "frac")}
    roof.update({"kernel": dom, "avg_launch_ms": stages[dom]["avg_launch_ms"],
                 "traffic": measured_traffic("linear", dom)})
    c = step.cfg
    rec = {
        "metric": "query tokens/s of the linear-layer variant at 1M-token memory (decode step)",
        "value": c.batch * c.q_len / (ms_per_step / 1e3), "unit": "query tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step, "ms_per_step_eager": eager_ms,
        "step_timing": "hip graph replay" if graph_ms is not None else "eager", "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "linear-1M-decode-bf16", "n_docs": c.n_doc, "doc_len": c.doc_len, "batch": c.batch,
                   "q_len": c.q_len, "heads": c.heads_kv, "dk": c.dim, "dv": c.dim, "topk": c.topk,
                   "step": "route -> top-k -> state sum -> gated-delta step",
                   "offline_document_states_ms": step.encode_ms,
                   "offline_document_states_form": "chunked (msa_gated_delta_rule_chunked)",
                   "offline_document_states_ms_token_by_token": step.encode_recurrent_ms},
        "roofline": roof, "stages": stages,
        "cpu_baseline": None if args.no_cpu_baseline else step.cpu_baseline(),
    }
    print(json.dumps(rec))


def main_backward(args):
    import torch
    dev = "cuda:0"
    print("[bench] building inputs for backward-1M-layer-bf16", file=sys.stderr, flush=True)
    step = BackwardStep(args.seed, dev)
    step.run(args.warmup, events=False)
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    marks = step.run(args.steps, events=True)
    end.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    stages = stage_summary(step, marks, args.steps)
    dom = max(stages, key=lambda k: stages[k]["ms_per_step"])
    roof = {k: stages[dom][k] for k in ("bound", "achieved", "peak", "unit", "frac")}
    roof.update({"kernel": dom, "avg_launch_ms": stages[dom]["avg_launch_ms"],
                 "traffic": measured_traffic("backward", dom)})
    c = step.cfg
    tokens = c.batch * c.q_len
    rec = {
        "metric": "query tokens/s of the routed layer's attention forward + backward (training step)",
        "value": tokens / (ms_per_step / 1e3), "unit": "query tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "backward-1M-layer-bf16", "batch": c.batch, "q_len": c.q_len,
                   "loc_len": c.loc_len, "mem_len": c.mem_len, "heads_q": c.heads_q, "heads_kv": c.heads_kv,
                   "dim": c.dim, "step": "attention forward -> attention backward"},
        "roofline": roof, "stages": stages,
        "cpu_baseline": None if args.no_cpu_baseline else step.cpu_baseline(),
    }
    print(json.dumps(rec))


def graph_replay_ms(step, steps, warmup=2):
    """Capture one step's launches in a HIP graph (torch's CUDAGraph over HIP)
    and time exactly `steps` replays; None when the capture fails.  The step
    makes no allocation and no host synchronisation, and the library records
    no memset, so the graph holds only the step's kernels.  Replays remove
    the per-launch host cost (the Python binding and the launches) that the
    eager loop pays between short kernels."""
    import torch
    seq = step.calls()
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _, fn in seq:
                fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _, fn in seq:
                fn()
    except Exception as e:  # pragma: no cover - reported, eager timing stands
        print(f"[bench] graph capture failed ({e}); eager timing only", file=sys.stderr, flush=True)
        return None
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def _median(xs):
    xs = sorted(xs)
    return xs[len(xs) // 2]


def time_launches(fn, reps, before=None):
    """Median duration (ms) of `fn`'s launches over `reps` repetitions, with HIP
    events on the current stream around each; `before` runs untimed ahead of
    every repetition."""
    import torch
    marks = []
    for _ in range(reps):
        if before is not None:
            before()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        marks.append((a, b))
    torch.cuda.synchronize()
    return _median([a.elapsed_time(b) for a, b in marks])


def route_scan_warm_cold(step, cfg, reps):
    """The decode step's routing scan over the 1M-token bank (32 MiB of K_r-bar,
    which the 256 MB MALL holds between steps) timed warm (back to back) and
    cold (a 512 MiB read between repetitions evicts it; a read, because the
    write-back of a written flush would land inside the timed scan)."""
    import torch
    msa = step.msa
    fn = lambda: msa.msa_route_scores(step.t["q_r"], step.kbar_r, step.knorm, cfg.chunks_per_doc,
                                      doc_scores=step.scores, ws=step.ws_route)
    flush = torch.ones((512 << 20) // 4, dtype=torch.float32, device=step.kbar_r.device)
    sink = torch.empty((), dtype=torch.float32, device=step.kbar_r.device)
    w = work_route(cfg)
    out = {}
    for name, before in (("warm", None), ("cold", lambda: sink.copy_(flush.sum()))):
        fn()
        ms = time_launches(fn, max(reps, 10), before)
        e = roofline_entry(dict(w, bound="hbm"), ms)
        out[name] = {"ms": ms, "GB/s": e["achieved"], "frac_hbm": e["frac"]}
    out["bytes"] = w["bytes"]
    del flush
    return out


def stage_summary(step, marks, steps):
    per, counts = {}, {}
    for stage, a, b in marks:
        per[stage] = per.get(stage, 0.0) + a.elapsed_time(b)
        counts[stage] = counts.get(stage, 0) + 1
    stages = {}
    for stage in per:
        avg = per[stage] / counts[stage]
        entry = roofline_entry(step.work(stage), avg)
        entry.update({"avg_launch_ms": avg, "launches_per_step": counts[stage] // steps,
                      "ms_per_step": per[stage] / steps})
        stages[stage] = entry
    return stages


def main_encode(args):
    import torch
    dev = "cuda:0"
    print("[bench] building inputs for encode-1M-varlen-bf16", file=sys.stderr, flush=True)
    step = EncodeStep(args.seed, dev)
    step.run(args.warmup, events=False)
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    marks = step.run(args.steps, events=True)
    end.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    per, counts = {}, {}
    for stage, a, b in marks:
        per[stage] = per.get(stage, 0.0) + a.elapsed_time(b)
        counts[stage] = counts.get(stage, 0) + 1
    stages = {}
    for stage in per:
        avg = per[stage] / counts[stage]
        entry = roofline_entry(step.work(stage), avg)
        entry.update({"avg_launch_ms": avg, "launches_per_step": counts[stage] // args.steps,
                      "ms_per_step": per[stage] / args.steps})
        stages[stage] = entry
    dom = max(stages, key=lambda k: stages[k]["ms_per_step"])
    roof = {k: stages[dom][k] for k in ("bound", "achieved", "peak", "unit", "frac")}
    roof.update({"kernel": dom, "avg_launch_ms": stages[dom]["avg_launch_ms"],
                 "traffic": measured_traffic("encode", dom)})
    rec = {
        "metric": "encoded document tokens/s (offline encoder, variable-length documents)",
        "value": step.rows / (ms_per_step / 1e3), "unit": "encoded tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "encode-1M-varlen-bf16", "n_docs": step.N_DOCS,
                   "doc_len_range": [step.LEN_LO, step.LEN_HI], "total_rows": step.rows,
                   "total_chunks": step.chunks, "chunk": step.CHUNK, "heads_kv": step.HEADS, "dim": step.DIM,
                   "rope_base": step.ROPE_BASE,
                   "step": "chunk offsets -> encode K (RoPE) -> encode V -> encode K_r (+ norms)"},
        "roofline": roof, "stages": stages,
        "cpu_baseline": None if args.no_cpu_baseline else step.cpu_baseline(),
    }
    print(json.dumps(rec))


def cpu_baseline(step, cfg, workload):
    """Time the float64 oracle on a bounded sample of the step and scale it up."""
    import numpy as np
    import torch
    from oracle import pool_chunks_mean, route_scores, sparse_attention_rows, topk_docs, topk_docs_excluding
    f = lambda x: x.detach().float().cpu().double().numpy()
    rng = np.random.default_rng(0)
    cpd = cfg.chunks_per_doc
    secs = 0.0
    parts = []
    pool_secs = None
    if workload == "prefill":
        # the offline stage, reported beside the step (not part of it)
        n_pool = 64
        pool_secs = 0.0
        docs = torch.as_tensor(rng.choice(cfg.n_doc, n_pool, replace=False), device=step.t["k"].device)
        for name in ("k", "v", "k_r"):
            x = f(step.t[name][docs])
            t0 = time.perf_counter()
            pool_chunks_mean(x, cfg.chunk)
            pool_secs += (time.perf_counter() - t0) * cfg.n_doc / n_pool
    n_route = 256
    sample = rng.choice(cfg.n_doc, n_route, replace=False)
    rows = torch.as_tensor((sample[:, None] * cpd + np.arange(cpd)).ravel(), device=step.kbar_r.device)
    kb = f(step.kbar_r[rows])
    q_rounds = [step.t["q_r"]] if workload != "interleave" else list(step.t["q_r_rounds"])
    for q_r in q_rounds:
        q_r = f(q_r)
        t0 = time.perf_counter()
        route_scores(q_r, kb, cpd)
        secs += (time.perf_counter() - t0) * cfg.n_doc / n_route
    parts.append(f"route all tokens vs {n_route}/{cfg.n_doc} docs" +
                 (f", each of {len(q_rounds)} rounds" if len(q_rounds) > 1 else ""))
    if workload == "interleave":
        # whole top-k of every round, on Gaussian scores of the same shape
        sc = rng.standard_normal((cfg.batch, cfg.n_doc))
        prev = np.empty((cfg.batch, 0), dtype=np.int64)
        t0 = time.perf_counter()
        for _ in q_rounds:
            ids, _ = topk_docs_excluding(sc, cfg.topk, prev)
            prev = np.concatenate([prev, ids], axis=1)
        secs += time.perf_counter() - t0
        parts.append("top-k excluding earlier rounds, whole, every round")
    else:
        sc = f(step.scores)
        t0 = time.perf_counter()
        topk_docs(sc, cfg.topk)
        secs += time.perf_counter() - t0
        parts.append("top-k whole")
    # gather is a copy; attention on sampled rows (uniform over (b, t, h))
    ks, vs = f(step.k_sel), f(step.v_sel)
    kl, vl, q = f(step.t["k_loc"]), f(step.t["v_loc"]), f(step.t["q"])
    n_rows_total = cfg.batch * cfg.q_len * cfg.heads_q
    n_att = min(2048, n_rows_total)
    g = cfg.heads_q // cfg.heads_kv
    picks = rng.integers(0, n_rows_total, n_att)
    t0 = time.perf_counter()
    for r in picks:
        h = int(r % cfg.heads_q)
        tt = int((r // cfg.heads_q) % cfg.q_len)
        b = int(r // (cfg.heads_q * cfg.q_len))
        n_loc = cfg.loc_len - cfg.q_len + tt + 1
        keys = np.concatenate([ks[b, :, h // g], kl[b, :n_loc, h // g]])
        vals = np.concatenate([vs[b, :, h // g], vl[b, :n_loc, h // g]])
        sparse_attention_rows(q[b, tt, h], keys, vals, 1.0 / math.sqrt(cfg.dim))
    secs += (time.perf_counter() - t0) * n_rows_total / n_att
    parts.append(f"attention {n_att}/{n_rows_total} rows")
    tokens = cfg.batch * cfg.q_len
    rec = {"value": tokens / secs, "unit": "query tokens/s", **host_threads(), "kind": "oracle",
           "sample": "; ".join(parts) + "; each stage's time scaled to the full step",
           "seconds_per_step": secs}
    if pool_secs is not None:
        rec["offline_pool_seconds"] = pool_secs
        rec["offline_pool_sample"] = f"pool {n_pool}/{cfg.n_doc} docs x3 tensors, scaled to the bank"
    return rec


def main():
    args = parse()
    if args.summarize_stats:
        summarize_stats(*args.summarize_stats)
        return
    if args.summarize_traffic:
        summarize_traffic(args.summarize_traffic)
        return
    if args.summarize_counters:
        a = args.summarize_counters
        summarize_counters(a[0], a[1], a[2].split(" ;; "), a[3:])
        return
    if args.copy_probe:
        copy_probe()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported. The path would "
              "shard documents across GPUs (each routes its shard, one all-gather of k candidates per "
              "sequence, a final top-k), but only the single-GPU share is built and timed.", file=sys.stderr)
        sys.exit(2)
    if args.workload == "encode":
        main_encode(args)
        return
    if args.workload == "backward":
        main_backward(args)
        return
    if args.workload == "linear":
        main_linear(args)
        return
    if args.workload == "stack":
        main_stack(args)
        return
    if args.workload == "scan100m":
        main_scan(args)
        return
    import torch
    import msa_inputs as mi
    dev = "cuda:0"
    cfg = mi.DECODE if args.workload == "decode" else mi.PREFILL
    rounds = INTERLEAVE_ROUNDS if args.workload == "interleave" else 1
    name = cfg.name if rounds == 1 else f"interleave{rounds}-1M-bf16"
    print(f"[bench] building inputs for {name}", file=sys.stderr, flush=True)
    step = Step(cfg, args.workload, args.seed, dev, rounds=rounds)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    step.run(args.warmup, events=False)
    torch.cuda.synchronize()

    # timed region: exactly K steps, per-launch events inside
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    marks = step.run(args.steps, events=True)
    end.record()
    torch.cuda.synchronize()
    eager_ms = start.elapsed_time(end) / args.steps
    print(f"[bench] timing {args.steps} graph replays", file=sys.stderr, flush=True)
    graph_ms = graph_replay_ms(step, args.steps)
    ms_per_step = graph_ms if graph_ms is not None else eager_ms

    mem_cfg = dataclasses.replace(cfg, topk=rounds * cfg.topk)      # the memory all rounds gathered
    works = {"pool": None, "route": work_route(cfg), "topk": work_topk(cfg), "gather": work_gather(mem_cfg),
             "attn": work_attn(mem_cfg), "rounds": work_rounds(cfg, rounds)}
    per = {}
    counts = {}
    for stage, a, b in marks:
        per[stage] = per.get(stage, 0.0) + a.elapsed_time(b)
        counts[stage] = counts.get(stage, 0) + 1
    stages = {}
    for stage in per:
        n_launch = counts[stage]
        avg = per[stage] / n_launch
        w = works[stage] if stage != "pool" else work_pool(cfg, with_norm=False)
        entry = roofline_entry(w, avg)
        entry.update({"avg_launch_ms": avg, "launches_per_step": n_launch // args.steps,
                      "ms_per_step": per[stage] / args.steps})
        stages[stage] = entry
    dom = max(stages, key=lambda s: stages[s]["ms_per_step"])
    roof = {k: stages[dom][k] for k in ("bound", "achieved", "peak", "unit", "frac")}
    roof["kernel"] = dom
    roof["avg_launch_ms"] = stages[dom]["avg_launch_ms"]
    roof["traffic"] = measured_traffic(args.workload, dom)

    tokens = cfg.batch * cfg.q_len
    offline = None
    if args.workload == "prefill":
        # S1, the offline stage of the pipeline, timed apart from the step
        print(f"[bench] timing {args.steps} passes of the offline pooling", file=sys.stderr, flush=True)
        pool_seq = step.pool_calls()
        step.run(1, events=False, seq=pool_seq)
        torch.cuda.synchronize()
        pmarks = step.run(args.steps, events=True, seq=pool_seq)
        torch.cuda.synchronize()
        pool_ms = [a.elapsed_time(b) for _, a, b in pmarks]
        avg = sum(pool_ms) / len(pool_ms)
        offline = roofline_entry(work_pool(cfg, with_norm=False), avg)
        offline.update({"kernel": "pool", "avg_launch_ms": avg, "launches_per_pass": 3,
                        "ms_per_pass": 3 * avg, "traffic": measured_traffic("prefill", "pool"),
                        "encoded_tokens_per_s": cfg.n_doc * cfg.doc_len / (3 * avg / 1e3),
                        "pass": "pool K, pool V, pool K_r (+ norms): 2048 docs x 512 tokens each"})
    route_cold = None
    if args.workload == "decode" and not args.step_only:
        route_cold = route_scan_warm_cold(step, cfg, args.steps)
    rec = {
        "metric": ("query tokens/s at 1M-token memory (routing-scan GB/s + sparse-attn TFLOP/s in stages)"
                   if rounds == 1 else
                   f"query tokens/s at 1M-token memory with {rounds} routing rounds (Memory Interleave)"),
        "value": tokens / (ms_per_step / 1e3),
        "unit": "query tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "ms_per_step_eager": eager_ms,
        "step_timing": "hip graph replay" if graph_ms is not None else "eager",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "n_docs": cfg.n_doc, "doc_len": cfg.doc_len, "chunk": cfg.chunk,
                   "batch": cfg.batch, "q_len": cfg.q_len, "loc_len": cfg.loc_len, "heads_q": cfg.heads_q,
                   "heads_kv": cfg.heads_kv, "dim": cfg.dim, "topk": cfg.topk, "rounds": rounds,
                   "mem_len": rounds * cfg.mem_len,
                   "step": {"prefill": "route -> top-k -> gather -> attention (the bank pooled offline, "
                                       "timed apart: offline_pool)",
                            "decode": "route -> top-k -> gather -> split-KV attention",
                            "interleave": f"(route -> top-k excluding earlier picks) x{rounds} -> gather -> "
                                          "attention"}[args.workload]},
        "roofline": roof,
        "stages": stages,
    }
    if offline is not None:
        rec["offline_pool"] = offline
    if route_cold is not None:
        rec["route_scan_warm_cold"] = route_cold
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(step, cfg, args.workload)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
