"""Throughput of the OneLA GDN beam decode step on one MI355X.

Workload: 32 concurrent requests x 16 heads, d_k = d_v = 128, beam width 256,
5 decode steps per episode, parents chosen per request as the top W of 4W
beam-search-like candidates. S0 is prompt-derived: a 5120-token synthetic
prompt per request is folded on the GPU by the prefill kernel (--s0 normal
draws S0 ~ N(0, 0.05^2) instead; the decode step's cost does not depend on
S0's values). One bench step is one
episode: every request is rewound (host-only) and advanced through all 5
decode steps of one GDN layer, one library launch per decode step. All inputs
of the 5 steps are resident in HBM before timing starts.

Prints one JSON line: beam-steps/s (value), microseconds per decode step, the
per-depth breakdown, the HBM roofline fraction of the step kernel (algorithmic
bytes per launch over its average duration: one pair of HIP events brackets
the timed region's back-to-back launches on their stream) and the float64
oracle timed on a bounded sample on the host cores. The per-depth breakdown
comes from a separate pass with events around every launch: each event is a
marker the GPU processes between two kernels, so that pass runs a few
microseconds slower per launch and stays out of the timed region.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from workload import bf16_bits_to_f32, make_episode, shape_of  # noqa: E402

METRIC = "GDN beam-steps/sec + µs/decode-step at W=256,d_k=d_v=128; % HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
KERNEL_NAME = "step_kernel"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "step_kernel_r32_h16_w256_t5_traffic.txt")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "step_kernel_r32_h16_w256_t5_counters.txt")
KERNEL_SOURCE = os.path.join(ROOT, "linear_attention_beam_gdn_amd", "csrc", "onela_kernels.hip")


# --------------------------------------------------------------- counters
# Kernels summarised from counter runs of this bench, by a fragment of their names.
COUNTER_KERNELS = [
    ("step_kernel<128, 128, false, *>", "::step_kernel<128, 128, false,"),
    ("step_kernel<128, 128, true, *> (raw projections in)", "::step_kernel<128, 128, true,"),
    ("prefill_kernel<128, 128, true> (5120-token prompts)", "::prefill_kernel<128, 128, true>"),
    ("projection probe, operands streamed", "projection_kernel"),
    ("projection probe, operands L2-resident", "projection_kernel"),
    ("projection probe, operands L2-resident, W = 1024", "projection_kernel"),
    ("MFMA loop probe", "mfma_loop_kernel"),
    ("copy probe", "::copy_kernel"),
]


def counters_from(dirs, command: str) -> str:
    """Summarise rocprofv3 --pmc runs of this bench (one counter set per run,
    each with GRBM_GUI_ACTIVE) into COUNTERS_FILE and return its text.

    Per kernel, averaged over its dispatches: MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES
    over (GRBM_GUI_ACTIVE per XCD x SIMDs); LDS busy = SQ_LDS_IDX_ACTIVE over
    (GRBM_GUI_ACTIVE per XCD x CUs); bank-conflict share = SQ_LDS_BANK_CONFLICT
    over SQ_LDS_IDX_ACTIVE; wave time waiting / issuing = SQ_WAIT_ANY /
    SQ_ACTIVE_INST_ANY over SQ_WAVE_CYCLES; VALU busy (an estimate) = 4 cycles per
    non-MFMA VALU instruction (SQ_INSTS_VALU - SQ_INSTS_MFMA) over the same SIMD cycles;
    instructions per wave from SQ_INSTS_*
    over SQ_WAVES. A step kernel row takes both instantiations (the first step's,
    which gathers no records, and the general one). The projection probe's
    dispatches are split in launch order:
    the bench runs the streamed form first, then the L2-resident one, then
    the L2-resident one with W = 1024.
    """
    import csv
    import glob

    agent, per, n_disp = {}, {}, {}   # per[label][counter] -> list of per-dispatch values
    for d in dirs:
        rows = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                rows.setdefault((int(r["Dispatch_Id"]), r["Kernel_Name"]), {})[r["Counter_Name"]] = float(r["Counter_Value"])
        for f in glob.glob(os.path.join(d, "**", "*agent_info.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r.get("Name", "").startswith("gfx"):
                    agent = {k: int(r[k]) for k in ("Simd_Count", "Cu_Count", "Num_Xcc")}
        for label, frag in COUNTER_KERNELS:
            disp = [c for (i, n), c in sorted(rows.items()) if frag in n]
            if frag == "projection_kernel":   # three equal runs, in this order
                third = len(disp) // 3
                part = 0 if "streamed" in label else 2 if "1024" in label else 1
                disp = disp[part * third:(part + 1) * third]
            n_disp[label] = max(n_disp.get(label, 0), len(disp))
            for c in disp:
                for name, v in c.items():
                    per.setdefault(label, {}).setdefault(name, []).append(v)
                if "GRBM_GUI_ACTIVE" in c and agent:
                    g = c["GRBM_GUI_ACTIVE"] / agent["Num_Xcc"]
                    derived = per.setdefault(label, {})
                    if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
                        derived.setdefault("mfma_busy", []).append(c["SQ_VALU_MFMA_BUSY_CYCLES"] / (g * agent["Simd_Count"]))
                    if "SQ_LDS_IDX_ACTIVE" in c:
                        derived.setdefault("lds_busy", []).append(c["SQ_LDS_IDX_ACTIVE"] / (g * agent["Cu_Count"]))
                    if "SQ_INSTS_VALU" in c and "SQ_INSTS_MFMA" in c:
                        # a wave64 VALU instruction occupies a 16-lane SIMD for 4 cycles
                        # (SQ_INSTS_VALU counts the MFMA instructions too)
                        valu = c["SQ_INSTS_VALU"] - c["SQ_INSTS_MFMA"]
                        derived.setdefault("valu_busy", []).append(4.0 * valu / (g * agent["Simd_Count"]))
    if not agent:
        raise SystemExit("no agent information under the counter directories")
    mean = lambda xs: sum(xs) / len(xs) if xs else float("nan")
    head = ("| kernel | dispatches | MFMA busy | VALU busy (est.) | LDS busy | LDS bank-conflict share | wave time waiting | "
            "wave time issuing | VALU / wave | MFMA / wave | LDS / wave | VMEM rd / wave | VMEM wr / wave | "
            "bf16 MFMA GFLOP / dispatch |")
    lines = [head, "|" + "---|" * (head.count("|") - 1)]
    for label, _ in COUNTER_KERNELS:
        c = {k: mean(v) for k, v in per.get(label, {}).items()}
        if not c:
            continue
        waves = c.get("SQ_WAVES", float("nan"))
        ratio = lambda a, b: c[a] / c[b] if c.get(a) is not None and c.get(b) else float("nan")
        lines.append(
            f"| {label} | {n_disp[label]} | {100 * c.get('mfma_busy', float('nan')):.1f}% | "
            f"{100 * c.get('valu_busy', float('nan')):.0f}% | "
            f"{100 * c.get('lds_busy', float('nan')):.1f}% | {100 * ratio('SQ_LDS_BANK_CONFLICT', 'SQ_LDS_IDX_ACTIVE'):.1f}% | "
            f"{100 * ratio('SQ_WAIT_ANY', 'SQ_WAVE_CYCLES'):.0f}% | {100 * ratio('SQ_ACTIVE_INST_ANY', 'SQ_WAVE_CYCLES'):.0f}% | "
            f"{c.get('SQ_INSTS_VALU', float('nan')) / waves:.0f} | {c.get('SQ_INSTS_MFMA', float('nan')) / waves:.0f} | "
            f"{c.get('SQ_INSTS_LDS', float('nan')) / waves:.0f} | {c.get('SQ_INSTS_VMEM_RD', float('nan')) / waves:.0f} | "
            f"{c.get('SQ_INSTS_VMEM_WR', float('nan')) / waves:.0f} | "
            f"{c.get('SQ_INSTS_VALU_MFMA_MOPS_BF16', float('nan')) * 512 / 1e9:.2f} |")
    step = {k: mean(v) for k, v in per.get(COUNTER_KERNELS[0][0], {}).items()}
    sratio = lambda a, b: step[a] / step[b] if step.get(a) is not None and step.get(b) else float("nan")
    text = "\n".join([
        "# Hardware counters of the decode-step kernels and the probes (rocprofv3 --pmc, one MI355X;",
        "# r32_h16_d128_w256_t5 for the step kernels, all depths averaged)",
        f"# commands (one counter set per run): {command}",
        f"kernel_source_sha = {kernel_source_sha()}",
        f"agent = {agent}",
        f"step_kernel_mfma_busy = {step.get('mfma_busy', float('nan')):.4f}",
        f"step_kernel_lds_bank_conflict_share = {sratio('SQ_LDS_BANK_CONFLICT', 'SQ_LDS_IDX_ACTIVE'):.4f}",
        f"step_kernel_wave_time_waiting = {sratio('SQ_WAIT_ANY', 'SQ_WAVE_CYCLES'):.4f}",
        "",
        *lines,
        "",
    ])
    os.makedirs(os.path.dirname(COUNTERS_FILE), exist_ok=True)
    open(COUNTERS_FILE, "w").write(text)
    return text


def read_counters():
    """The step kernel's counter summary, if taken on this kernel source."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    kv = {}
    for line in open(COUNTERS_FILE):
        if "=" in line and not line.lstrip().startswith(("#", "|")):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha") != kernel_source_sha():
        return None
    try:
        return {"mfma_busy": float(kv["step_kernel_mfma_busy"]),
                "lds_bank_conflict_share": float(kv["step_kernel_lds_bank_conflict_share"]),
                "wave_time_waiting": float(kv["step_kernel_wave_time_waiting"]),
                "source": os.path.relpath(COUNTERS_FILE, ROOT)}
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------- timing
def time_episodes(run, stream, episodes: int, T: int, instrumented: int = 10):
    """run(events) enqueues one episode of T launches on `stream`; events is
    None, or T (start, end) HIP event pairs to record around the launches.

    Returns the mean launch duration in seconds over `episodes` back-to-back
    episodes bracketed by one pair of HIP events (nothing else enqueued
    between the launches), the wall time per episode in seconds, and the
    median duration per depth in microseconds from a separate pass of
    `instrumented` episodes with events around every launch."""
    import torch

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(episodes):
        run(None)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean_launch_s = e0.elapsed_time(e1) * 1e-3 / (episodes * T)
    evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in range(T)]
           for _ in range(instrumented)]
    for i in range(instrumented):
        run(evs[i])
    torch.cuda.synchronize()
    per = np.array([[evs[i][t][0].elapsed_time(evs[i][t][1]) for t in range(T)] for i in range(instrumented)]) * 1e3
    return mean_launch_s, wall / episodes, np.median(per, axis=0), per


def evict_caches(buf) -> None:
    """Enqueue a read of `buf` (512 MiB or more): it replaces what the 256 MB
    last-level cache and the L2s hold with clean lines of its own. (A write
    would leave that much dirty data behind, whose write-backs the next kernel
    would then pay for.)"""
    import torch

    torch.amax(buf.view(torch.int32))


def depth_stats(per_us: np.ndarray) -> dict:
    """Median, p10 and p90 per depth (columns) of instrumented launch times in microseconds."""
    return {"median": [round(float(x), 2) for x in np.median(per_us, axis=0)],
            "p10": [round(float(x), 2) for x in np.percentile(per_us, 10, axis=0)],
            "p90": [round(float(x), 2) for x in np.percentile(per_us, 90, axis=0)],
            "episodes": int(per_us.shape[0])}



# ------------------------------------------------------------- accounting
def unique_ancestors(parents_req: np.ndarray, t: int) -> int:
    """Distinct records the W beams of one request read at step t (1-based)."""
    if t < 2:
        return 0
    total = 0
    reach = np.unique(parents_req[t - 1])            # beams of step t-1 with a child at step t
    for s in range(t - 1, 0, -1):
        total += len(reach)
        if s > 1:
            reach = np.unique(parents_req[s - 1][reach])
    return total


def step_bytes(shape, parents, t: int) -> dict:
    """Algorithmic HBM bytes of one decode step at depth t over all requests and heads."""
    R, H, W, dk, dv = shape.R, shape.H, shape.W, shape.dk, shape.dv
    rec = 4 + 4 * dv + 2 * dk
    uniq = sum(unique_ancestors(parents[:, r, :], t) for r in range(R))
    b = {
        "s0": R * H * 4 * dv * dk,                      # hi + lo bf16 planes = fp32 bytes
        "inputs": R * W * H * (2 * dk + 2 * dk + 2 * dv + 8),
        "records_read": uniq * H * rec,
        "records_append": R * W * H * rec,
        "o": R * W * H * 4 * dv,
        "ancestry": (R * W * 4 * (1 + 2 * (t - 1) - 1)) if t >= 2 else 0,
    }
    b["total"] = sum(b.values())
    b["unique_records"] = uniq
    return b


def step_flops(shape, t: int) -> dict:
    R, H, W, dk, dv = shape.R, shape.H, shape.W, shape.dk, shape.dv
    proj = R * H * 4 * W * dv * dk                       # S0 [k q] for 2W vectors
    replay = R * H * W * (t - 1) * (4 * dk + 4 * dv)
    epi = R * H * W * (2 * dk + 6 * dv)
    return {"projection": proj, "total": proj + replay + epi}


def kernel_source_sha() -> str:
    return hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch measured by rocprofv3 counters, if taken on this kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha") != kernel_source_sha():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def traffic_from_counters(fetch_dir: str, write_dir: str, copy_mib: int, command: str) -> str:
    """Per-launch HBM traffic of the step kernel from two rocprofv3 --pmc runs.

    fetch_dir / write_dir hold run_counter_collection.csv of a run with
    FETCH_SIZE / WRITE_SIZE (KiB per dispatch) that also ran one plain device
    copy of copy_mib MiB. Each counter is scaled by known bytes / counted
    bytes of that copy. Writes TRAFFIC_FILE and returns its text.
    """
    import csv
    import glob

    def per_kernel(d, counter):
        rows = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] == counter:
                    rows[int(r["Dispatch_Id"])] = (r["Kernel_Name"], float(r["Counter_Value"]) * 1024.0)
        step = [v for k, (n, v) in sorted(rows.items()) if f"::{KERNEL_NAME}<" in n]   # not fs_step_kernel
        copy = [v for k, (n, v) in sorted(rows.items()) if "copyBuffer" in n]
        if not step or not copy:
            raise SystemExit(f"no {KERNEL_NAME} or copy dispatches with {counter} under {d}")
        return step, max(copy)

    known = copy_mib * 2.0 ** 20
    fetch, fetch_copy = per_kernel(fetch_dir, "FETCH_SIZE")
    write, write_copy = per_kernel(write_dir, "WRITE_SIZE")
    f_scale, w_scale = known / fetch_copy, known / write_copy
    per_launch = (sum(fetch) / len(fetch)) * f_scale + (sum(write) / len(write)) * w_scale
    text = "\n".join([
        "# HBM traffic of step_kernel on r32_h16_d128_w256_t5 (bytes per launch, all 5 depths averaged)",
        f"# command: {command}",
        f"kernel_source_sha = {kernel_source_sha()}",
        f"copy_probe_bytes = {known:.0f}",
        f"fetch_scale = {f_scale:.4f}",
        f"write_scale = {w_scale:.4f}",
        f"launches = {len(fetch)}",
        f"fetch_bytes_per_launch = {sum(fetch) / len(fetch) * f_scale:.0f}",
        f"write_bytes_per_launch = {sum(write) / len(write) * w_scale:.0f}",
        f"hbm_bytes_per_launch = {per_launch:.0f}",
        "fetch_bytes_by_dispatch = " + " ".join(f"{x * f_scale:.0f}" for x in fetch),
        "write_bytes_by_dispatch = " + " ".join(f"{x * w_scale:.0f}" for x in write),
        "",
    ])
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    open(TRAFFIC_FILE, "w").write(text)
    return text


def _counter_rows(d):
    """{(dispatch id, kernel name): {counter: value}} of one rocprofv3 --pmc output directory."""
    import csv
    import glob

    rows = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            rows.setdefault((int(r["Dispatch_Id"]), r["Kernel_Name"]), {})[r["Counter_Name"]] = float(r["Counter_Value"])
    return rows


def profile_by_depth(leg: str, fetch_dir: str, write_dir: str, counter_dirs, copy_mib: int, command: str,
                     out_dir: str = "") -> str:
    """Per-depth HBM traffic and counters of step_kernel in a run of one bench
    leg alone (`bench.py --only stress` or `--only multi_layer` under
    rocprofv3 --pmc): FETCH_SIZE and WRITE_SIZE scaled by the same counters on
    a plain copy of copy_mib MiB in the same run, set against the algorithmic
    bytes of each depth from the realised parents; the other counter runs give
    wave waiting, L1-to-L2 read requests and MFMA / LDS activity per depth.
    Writes <out_dir or profiles/>/<kernel>_<workload>_by_depth.txt and returns its text."""
    if leg == "stress":
        from workload.gen_device import all_parents

        shape = shape_of(4)
        parents = all_parents(shape)
        per_step = 1                                  # launches per decode step
        fname = "step_kernel_r64_h32_w1024_t7_zipf_by_depth.txt"
        what = "stress workload r64_h32_d128_w1024_t7, Zipf(1.2) parents"
    elif leg == "multi_layer":
        from workload.gen import parents_for

        shape = shape_of(3)
        parents = np.stack([parents_for(shape, r) for r in range(shape.R)], axis=1)
        per_step = 4
        fname = "step_kernel_4layers_r32_h16_w256_t5_by_depth.txt"
        what = ("4 GDN layers of r32_h16_d128_w256_t5 sharing one ancestry index, eager and graph-replayed "
                "decode steps (each layer-step is one launch)")
    else:
        raise SystemExit(f"no per-depth profile for leg {leg!r}")
    T = shape.T
    known = copy_mib * 2.0 ** 20

    def step_disp(rows, counter):
        step = [c[counter] for (i, n), c in sorted(rows.items()) if f"::{KERNEL_NAME}<" in n and counter in c]
        copy = [c[counter] for (i, n), c in sorted(rows.items()) if "copyBuffer" in n and counter in c]
        return step, copy

    fr, wr = _counter_rows(fetch_dir), _counter_rows(write_dir)
    fetch, fcopy = step_disp(fr, "FETCH_SIZE")
    write, wcopy = step_disp(wr, "WRITE_SIZE")
    if not fetch or not write or not fcopy or not wcopy:
        raise SystemExit("missing step_kernel or copy dispatches in the FETCH_SIZE / WRITE_SIZE runs")
    f_scale, w_scale = known / (max(fcopy) * 1024.0), known / (max(wcopy) * 1024.0)
    depth_of = lambda i: (i // per_step) % T
    alg = [step_bytes(shape, parents, t + 1)["total"] for t in range(T)]
    byd = {t: {"fetch": [], "write": []} for t in range(T)}
    for i, x in enumerate(fetch):
        byd[depth_of(i)]["fetch"].append(x * 1024.0 * f_scale)
    for i, x in enumerate(write):
        byd[depth_of(i)]["write"].append(x * 1024.0 * w_scale)
    import csv
    import glob

    agent = {}
    for d in counter_dirs or []:
        for f in glob.glob(os.path.join(d, "**", "*agent_info.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r.get("Name", "").startswith("gfx"):
                    agent = {k: int(r[k]) for k in ("Simd_Count", "Cu_Count", "Num_Xcc")}
    cnt = {t: {} for t in range(T)}
    for d in counter_dirs or []:
        rows = _counter_rows(d)
        disp = [c for (i, n), c in sorted(rows.items()) if f"::{KERNEL_NAME}<" in n]
        for i, c in enumerate(disp):
            for k, v in c.items():
                cnt[depth_of(i)].setdefault(k, []).append(v)
            if "GRBM_GUI_ACTIVE" in c and agent:
                g = c["GRBM_GUI_ACTIVE"] / agent["Num_Xcc"]            # kernel cycles per XCD
                if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
                    cnt[depth_of(i)].setdefault("mfma_busy", []).append(
                        c["SQ_VALU_MFMA_BUSY_CYCLES"] / (g * agent["Simd_Count"]))
                if "SQ_LDS_IDX_ACTIVE" in c:
                    cnt[depth_of(i)].setdefault("lds_busy", []).append(c["SQ_LDS_IDX_ACTIVE"] / (g * agent["Cu_Count"]))
    mean = lambda xs: sum(xs) / len(xs) if xs else float("nan")
    head = ("| depth | launches | fetch MB | write MB | HBM MB (counters) | algorithmic MB | counters / algorithmic | "
            "wave time waiting | L1->L2 read requests (M) | MFMA busy | LDS busy |")
    lines = [head, "|" + "---|" * (head.count("|") - 1)]
    tot_c = tot_a = 0.0
    for t in range(T):
        f, w = mean(byd[t]["fetch"]), mean(byd[t]["write"])
        c = {k: mean(v) for k, v in cnt[t].items()}
        ratio = lambda a, b: c[a] / c[b] if c.get(a) is not None and c.get(b) else float("nan")
        tot_c += f + w
        tot_a += alg[t]
        lines.append(f"| {t + 1} | {len(byd[t]['fetch'])} | {f / 1e6:.1f} | {w / 1e6:.1f} | {(f + w) / 1e6:.1f} | "
                     f"{alg[t] / 1e6:.1f} | {(f + w) / alg[t]:.3f} | {100 * ratio('SQ_WAIT_ANY', 'SQ_WAVE_CYCLES'):.0f}% | "
                     f"{c.get('TCP_TCC_READ_REQ_sum', c.get('TCP_TCC_READ_REQ', float('nan'))) / 1e6:.1f} | "
                     f"{100 * c.get('mfma_busy', float('nan')):.1f}% | {100 * c.get('lds_busy', float('nan')):.1f}% |")
    text = "\n".join([
        f"# step_kernel per depth: {what}",
        "# HBM bytes per launch from FETCH_SIZE and WRITE_SIZE (rocprofv3 --pmc, KiB per dispatch), each scaled",
        "# by known bytes / counted bytes of one plain device copy in the same run; algorithmic bytes per launch",
        "# as the bench counts them (distinct ancestral records from the realised parents). Wave time waiting =",
        "# SQ_WAIT_ANY / SQ_WAVE_CYCLES; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES over the SIMDs' cycles, LDS busy =",
        "# SQ_LDS_IDX_ACTIVE over the CUs' cycles (GRBM_GUI_ACTIVE per XCD); L1->L2 read requests =",
        "# TCP_TCC_READ_REQ summed over the chip. FETCH_SIZE counts L2 fetches from the fabric, which the",
        "# 256 MB last-level cache may serve before HBM.",
        f"# commands: {command}",
        f"kernel_source_sha = {kernel_source_sha()}",
        f"copy_probe_bytes = {known:.0f}",
        f"fetch_scale = {f_scale:.4f}",
        f"write_scale = {w_scale:.4f}",
        f"hbm_bytes_per_launch_mean = {tot_c / T:.0f}",
        f"algorithmic_bytes_per_launch_mean = {tot_a / T:.0f}",
        f"counters_over_algorithmic = {tot_c / tot_a:.4f}",
        "",
        *lines,
        "",
    ])
    path = os.path.join(out_dir or os.path.join(ROOT, "profiles"), fname)
    os.makedirs(os.path.dirname(path), exist_ok=True)
    open(path, "w").write(text)
    return text


def prompt_s0(lay, shape, prompt_len, reqs, dev, stream, need_f32):
    """Fold a synthetic prompt per request into the layer's S0 on the GPU and time it.

    Returns (float32 S0 [R][H][dv][dk] for the comparator or None, prefill record).
    The recurrence itself is 5 d_v d_k flops per token and head (S k, then the
    decayed rank-one update); the chunked kernel computes it as products over
    pairs of 16-token chunks on the matrix cores, whose issued bf16 flops are
    reported beside it against the bf16 peak.
    """
    import torch

    from linear_attention_beam_gdn_amd import prefill
    from workload.gen_device import prompt_tokens_device

    pshape = shape_of(shape.cfg, s0="prompt", prompt_len=prompt_len)
    toks = prompt_tokens_device(pshape, dev, reqs=reqs)
    args = (toks["k"], toks["v"], toks["alpha"], toks["beta"])
    # warm-up (and the state the bench decodes from): the fold is the run's first GPU work,
    # so enough untimed launches for the clocks to settle (fewer gave 15% slower times)
    for _ in range(20):
        lay.init_requests_from_prompts(reqs, *args)
    reps = 5
    ev = [torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
    ev[0].record(stream)
    for _ in range(reps):                             # each launch folds the same prompts again
        lay.init_requests_from_prompts(reqs, *args)
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    S0 = prefill(*args, stream=stream) if need_f32 else None
    torch.cuda.synchronize()
    del toks, args
    flops = 5.0 * len(reqs) * prompt_len * shape.H * shape.dv * shape.dk
    tflops = flops / (ms * 1e-3) / 1e12
    # 16x16x32 products per pair of 16-token chunks and (sequence, head): the two
    # chunks' K K^T and the keys between them (3 x d/32), and per wave of d/16:
    # P for both chunks (2 d/16), the two solves and the coupling (6), update (2 d/16)
    kc, nw = shape.dk // 16, shape.dv // 16
    pairs = len(reqs) * shape.H * -(-prompt_len // 32)
    mfma_flops = pairs * (3 * (shape.dk // 32) + nw * (4 * kc + 6)) * 2 * 16 * 16 * 32
    mfma_tflops = mfma_flops / (ms * 1e-3) / 1e12
    return S0, {
        "kernel": "prefill_kernel",
        "what": f"S0 of {len(reqs)} requests x {shape.H} heads from {prompt_len}-token prompts, one launch "
                "(onela_init_requests_from_prompts, written as the step kernel's bf16 planes); mean of 5 "
                "back-to-back launches after 20 untimed ones",
        "ms": ms,
        "tokens_per_s": len(reqs) * prompt_len / (ms * 1e-3),
        "recurrence_tflops": tflops,
        "roofline": {"bound": "mfma", "achieved": mfma_tflops, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": mfma_tflops / BF16_PEAK_TFLOPS, "flops_per_launch": mfma_flops,
                     "note": "issued bf16 MFMA flops of the chunked form; the recurrence's own 5 d_v d_k flops per "
                             "token and head are in recurrence_tflops"},
    }


def probe_leg(shape, q, k, S0):
    """The box's practical peaks and the projection on its own.

    copy: a 1 GiB device-to-device copy (2 GiB moved per launch); MFMA loop:
    1024 workgroups x 8 waves x 2000 x 8 register-only 16x16x32 bf16 MFMAs;
    projection: S0 [k q] of the step-1 vectors for all (request, head) pairs
    with the step kernel's tiling (onela_probe_projection), repeated so that
    its 96 MB of operands come from the 256 MB last-level cache, which is the
    projection-only measurement the HBM-bound fused step cannot give.
    """
    import torch

    from linear_attention_beam_gdn_amd import probes

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device=q[0].device)
    dst = torch.empty_like(src)
    t_copy = timed(lambda: probes.copy(src, dst), 10)
    copy_gbs = 2 * n * 4 / t_copy / 1e9
    del src, dst
    n_wg, iters = 1024, 2000
    buf = torch.empty(n_wg * 512, dtype=torch.float32, device=q[0].device)
    t_mfma = timed(lambda: probes.mfma_loop(buf, n_wg, iters), 5)
    loop_tflops = n_wg * 8 * iters * 8 * 16384 / t_mfma / 1e12
    R, H, W, dk, dv = shape.R, shape.H, shape.W, shape.dk, shape.dv
    colsum = torch.empty((R * H, dv), dtype=torch.float32, device=q[0].device)
    pl = probes.planes(S0)                                            # the step kernel's form of S0
    t_proj = timed(lambda: probes.projection(pl, k[0], q[0], W, colsum), 20)
    t_res = timed(lambda: probes.projection(pl, k[0], q[0], W, colsum, resident_pairs=8), 20)
    flops = R * H * 2 * W * 2 * dv * dk
    tflops = flops / t_proj / 1e12
    res_tflops = flops / t_res / 1e12
    # the same probe with four times the beams per pair (W = 1024, drawn unit-norm-scale operands,
    # 8 resident pairs): how much of the W = 256 rate is the fixed cost of each pair (its 64 KB of S0
    # fragments, the first chunk's staging) rather than the matrix cores
    W4 = 4 * W
    g = torch.Generator(device=q[0].device).manual_seed(5)
    k4 = (torch.randn((R * W4, H, dk), generator=g, device=q[0].device) / dk ** 0.5).to(torch.bfloat16).view(torch.int16)
    q4 = (torch.randn((R * W4, H, dk), generator=g, device=q[0].device) / dk ** 0.5).to(torch.bfloat16).view(torch.int16)
    t_w4 = timed(lambda: probes.projection(pl, k4, q4, W4, colsum, resident_pairs=8), 20)
    w4_tflops = 4 * flops / t_w4 / 1e12
    del k4, q4
    operands = R * W * H * 2 * dk * 2 + R * H * dv * dk * 4          # k, q (bf16) and S0
    p_bytes = R * 2 * W * H * dv * 4                                  # P itself, were it written in float32
    cap = lambda nbytes: flops / (nbytes / (HBM_PEAK_GBS * 1e9)) / 1e12 / BF16_PEAK_TFLOPS
    return ({"copy_gbs": copy_gbs, "copy_bytes_per_launch": 2 * n * 4, "mfma_loop_tflops": loop_tflops,
             "mfma_loop_frac_of_peak": loop_tflops / BF16_PEAK_TFLOPS},
            {"method": "projection-only probe (onela_probe_projection): the step kernel's 16x16x32 bf16 tiles and "
                       "split-bf16 S0 read from hi/lo planes in A-fragment order (as the step kernel holds it), k and "
                       "q staged through LDS 64 beams at a time (next chunk in flight), per-row "
                       "sums in place of the replay; all 512 (request, head) pairs, 2W = 512 vectors each. "
                       "'achieved' reads the operands of 8 pairs only (workgroup p reads pair p mod 8), which stay "
                       "in L2: the projection's matrix-core rate; 'full_footprint' streams all 96 MB of operands",
             "us_per_launch": t_res * 1e6,
             "algorithmic_gflop_per_launch": flops / 1e9,
             "achieved_tflops": res_tflops, "peak_tflops": BF16_PEAK_TFLOPS, "frac": res_tflops / BF16_PEAK_TFLOPS,
             "issued_tflops": 2 * res_tflops, "issued_frac": 2 * res_tflops / BF16_PEAK_TFLOPS,
             "issued_frac_of_measured_mfma_loop": 2 * res_tflops / loop_tflops,
             "w1024_resident": {"us_per_launch": t_w4 * 1e6, "achieved_tflops": w4_tflops,
                                "frac": w4_tflops / BF16_PEAK_TFLOPS, "issued_frac": 2 * w4_tflops / BF16_PEAK_TFLOPS},
             "full_footprint": {"us_per_launch": t_proj * 1e6, "achieved_tflops": tflops,
                                "frac": tflops / BF16_PEAK_TFLOPS, "issued_frac": 2 * tflops / BF16_PEAK_TFLOPS,
                                "operand_gbs": operands / t_proj / 1e9},
             "hbm_cap_frac": {"operands_from_hbm": cap(operands), "operands_and_fp32_P": cap(operands + p_bytes),
                              "in_fused_step_S0_only": cap(R * H * dv * dk * 4)}})


def fused_leg(shape, ep, q, k, v, al, be, par, S0, bytes_t, runs=20):
    """The same decode steps through onela_step_raw (input-side fusion: q, k
    normalised, alpha and beta formed from raw projections inside the launch,
    o written as bf16). Raw inputs of the same shapes stand in for the
    projections (the cost does not depend on their values). Returns the
    launch time per depth and the HBM rate of its algorithmic bytes (the
    decode step's, with o at 2 bytes per element)."""
    import torch

    from linear_attention_beam_gdn_amd import Onela
    from workload import gate_params

    R, H, W, T = shape.R, shape.H, shape.W, shape.T
    stream = torch.cuda.current_stream()
    lay = Onela(R, H, shape.dk, shape.dv, W, T, stream=stream)
    for r in range(R):
        lay.init_request(r, S0[r].contiguous())
    g = gate_params(shape)
    A = torch.from_numpy(g["A_log"]).cuda()
    D = torch.from_numpy(g["dt_bias"]).cuda()
    o16 = torch.empty((R * W, H, shape.dv), dtype=torch.int16, device=q[0].device)
    reqs = list(range(R))

    def episode(events):
        for r in reqs:
            lay.reset(r)
        for t in range(T):
            if events is not None:
                events[t][0].record(stream)
            lay.step_raw(reqs, q[t], k[t], v[t], al[t], be[t], A, D, par[t], o16)
            if events is not None:
                events[t][1].record(stream)

    for _ in range(2):
        episode(None)
    mean_s, _, us, _ = time_episodes(episode, stream, runs, T)
    lay.sync()
    lay.close()
    nbytes = [b["total"] - R * W * H * 2 * shape.dv for b in bytes_t]     # o at 2 B instead of 4
    gbs = float(np.mean(nbytes)) / mean_s / 1e9
    return {
        "what": "onela_step_raw: per-head q/k L2 normalisation, alpha = exp(-exp(A_log) softplus(a + dt_bias)), "
                "beta = sigmoid(b) inside the launch, o as bf16",
        "kernel": "step_kernel<128, 128, true>",
        "kernel_us_mean": mean_s * 1e6,
        "us_by_depth_instrumented": [round(float(x), 2) for x in us],
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": float(np.mean(nbytes))},
    }


def multi_layer_leg(shape, n_layers, q, k, v, al, be, par, S0, episodes=10):
    """A decode step of n_layers GDN layers sharing one ancestry index, eager vs
    one HIP graph per decode step (graph mode: step counters on the device).

    Every layer gets the same inputs (the cost does not depend on their
    values). Returns microseconds per decode step (all layers), the median
    over the episodes of each episode's time divided by its T steps.
    """
    import torch

    from linear_attention_beam_gdn_amd import Onela

    R, H, W, T = shape.R, shape.H, shape.W, shape.T
    s = torch.cuda.Stream()
    layers = [Onela(R, H, shape.dk, shape.dv, W, T, stream=s)]
    layers += [Onela(R, H, shape.dk, shape.dv, W, T, stream=s, share_index_of=layers[0]) for _ in range(n_layers - 1)]
    reqs = list(range(R))
    outs = [torch.empty((R * W, H, shape.dv), dtype=torch.float32, device=q[0].device) for _ in layers]
    for lay in layers:
        for r in reqs:
            lay.init_request(r, S0[r].contiguous())

    def decode_step(t):
        for lay, o in zip(layers, outs):
            lay.step(reqs, q[t], k[t], v[t], al[t], be[t], par[t] if t else par[1], o)

    def run(replay):
        # one event pair per episode around its decode steps (the resets, which
        # launch counter updates in graph mode, stay outside); no
        # synchronisation inside the loop: the queue stays ahead of the GPU
        ev = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
              for _ in range(episodes + 2)]
        for it in range(episodes + 2):
            for lay in layers:
                for r in reqs:
                    lay.reset(r)
            ev[it][0].record(s)
            for t in range(T):
                replay(t)
            ev[it][1].record(s)
        s.synchronize()
        for lay in layers:
            lay.sync()
        return float(np.median([ev[it][0].elapsed_time(ev[it][1]) for it in range(2, episodes + 2)])) * 1e3 / T

    with torch.cuda.stream(s):
        eager = run(decode_step)
        for lay in layers:
            lay.set_graph_mode(True)
        graphs = []
        for t in range(T):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                decode_step(t)
            graphs.append(g)
        graph = run(lambda t: graphs[t].replay())
    del graphs
    for lay in reversed(layers):
        lay.close()
    return {
        "what": f"one decode step of {n_layers} GDN layers sharing one ancestry index (all {R} requests), "
                "eager onela_step calls vs one captured HIP graph per decode step",
        "layers": n_layers,
        "eager_us_per_decode_step": eager,
        "graph_us_per_decode_step": graph,
    }


def replay_leg(shape, q, k, v, al, be, par, o, S0, stream, onela_launch_s, onela_ms_per_step, onela_mem):
    """Same workload through the replay comparator (every beam rebuilds its
    state from S0 and its own ancestral records at every step)."""
    import torch

    from linear_attention_beam_gdn_amd import ReplayState

    R, H, W, T = shape.R, shape.H, shape.W, shape.T
    rs = ReplayState(R, H, shape.dk, shape.dv, W, T, stream=stream)
    for r in range(R):
        rs.init_request(r, S0[r].contiguous())
    reqs = list(range(R))

    def episode(events):
        for r in reqs:
            rs.reset(r)
        for t in range(T):
            if events is not None:
                events[t][0].record(stream)
            rs.step(reqs, q[t], k[t], v[t], al[t], be[t], par[t], o)
            if events is not None:
                events[t][1].record(stream)

    episode(None)
    mean_s, wall, by_depth, _ = time_episodes(episode, stream, 5, T, instrumented=2)
    rs.sync()
    rs_mem = rs.memory()
    rs.close()
    return {
        "what": "the same decode steps with every beam rebuilding its d_v x d_k state from S0 and its own "
                "ancestral records (full rank-one updates) at every step; nothing shared between beams",
        "kernel_us_mean": mean_s * 1e6,
        "us_per_decode_step": wall / T * 1e6,
        "us_by_depth_instrumented": [round(float(x), 1) for x in by_depth],
        "speedup_kernel": mean_s / onela_launch_s,
        "speedup_step": wall / T * 1e3 / (onela_ms_per_step / T),
        "persistent_state_bytes": {"replay": rs_mem,
                                   "onela": onela_mem["s0_bytes"] + onela_mem["record_bytes"] + onela_mem["index_bytes"]},
    }


# Shapes of the operator sweep: beam width, head dimension, decode steps and
# (requests, heads); parents chosen as the top W of 4W random scores.
SWEEP_W = (64, 256, 1024)
SWEEP_D = (64, 128)
SWEEP_T = (3, 7)
SWEEP_RH = ((4, 16), (32, 16))
SWEEP_FS_MAX_BYTES = 40 << 30       # full-state stores above this are skipped


def sweep_leg(episodes=2):
    """OneLA against the full-state and replay comparators over a grid of
    operator shapes (W x d x T x (requests, heads)), on seeded inputs drawn on
    the GPU. Per shape: mean launch time of each path over at least
    `episodes` episodes, and enough for a ~3 ms window (one event pair),
    after one untimed and one sizing episode; speedups, and the persistent-state reduction
    against W full states per request and head. Returns the per-shape rows
    and the medians over the shapes."""
    import torch

    from linear_attention_beam_gdn_amd import FullState, Onela, ReplayState
    from workload.gen_device import all_parents, s0_device, step_inputs

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    rows = []
    for (R, H) in SWEEP_RH:
        for W in SWEEP_W:
            for d in SWEEP_D:
                for T in SWEEP_T:
                    shape = shape_of(1, name=f"sweep_r{R}_h{H}_d{d}_w{W}_t{T}", R=R, H=H, dk=d, dv=d, W=W, T=T)
                    parents = all_parents(shape)
                    S0 = s0_device(shape, dev)
                    ins = [step_inputs(shape, t, dev) for t in range(T)]
                    par = [None] + [torch.from_numpy(parents[t].astype(np.int32)).to(dev) for t in range(1, T)]
                    o = torch.empty((R * W, H, d), dtype=torch.float32, device=dev)
                    reqs = list(range(R))

                    def run(ctx):
                        for r in reqs:
                            ctx.init_request(r, S0[r].contiguous())

                        def episode():
                            for r in reqs:
                                ctx.reset(r)
                            for t in range(T):
                                x = ins[t]
                                ctx.step(reqs, x["q"], x["k"], x["v"], x["alpha"], x["beta"], par[t], o)

                        episode()
                        torch.cuda.synchronize()
                        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                        # one timed episode sizes the run: at least `episodes`, and enough
                        # for a window of ~3 ms, so that microsecond launches are not timed
                        # over a handful of events
                        e0.record(stream)
                        episode()
                        e1.record(stream)
                        torch.cuda.synchronize()
                        n_ep = int(min(50, max(episodes, math.ceil(3.0 / max(e0.elapsed_time(e1), 1e-3)))))
                        e0.record(stream)
                        for _ in range(n_ep):
                            episode()
                        e1.record(stream)
                        torch.cuda.synchronize()
                        ctx.sync()
                        return e0.elapsed_time(e1) * 1e-3 / (n_ep * T)

                    ol = Onela(R, H, d, d, W, T, stream=stream)
                    t_ol = run(ol)
                    mem = ol.memory()
                    ol.close()
                    rs = ReplayState(R, H, d, d, W, T, stream=stream)
                    t_rs = run(rs)
                    rs.close()
                    per_beam = R * H * W * d * d * 4
                    t_fs = None
                    if 2 * per_beam <= SWEEP_FS_MAX_BYTES:
                        fs = FullState(R, H, d, d, W, T, stream=stream)
                        t_fs = run(fs)
                        fs.close()
                    onela_bytes = mem["s0_bytes"] + mem["record_bytes"] + mem["index_bytes"]
                    rows.append({"R": R, "H": H, "d": d, "W": W, "T": T, "onela_us": t_ol * 1e6,
                                 "replay_us": t_rs * 1e6, "fullstate_us": None if t_fs is None else t_fs * 1e6,
                                 "speedup_vs_replay": t_rs / t_ol,
                                 "speedup_vs_fullstate": None if t_fs is None else t_fs / t_ol,
                                 "state_reduction": per_beam / onela_bytes})
                    del ins, par, o, S0
                    torch.cuda.empty_cache()
    med = lambda key: float(np.median([r[key] for r in rows if r[key] is not None]))
    return {
        "what": "mean launch time per decode step of OneLA, the replay comparator and the full-state comparator "
                f"over {len(rows)} shapes (W in {SWEEP_W}, d in {SWEEP_D}, T in {SWEEP_T}, (requests, heads) in "
                f"{SWEEP_RH}; top-W-of-4W parents); state reduction = W full float32 states per request and head "
                "over OneLA's S0 planes + records + index",
        "median_speedup_vs_replay": med("speedup_vs_replay"),
        "median_speedup_vs_fullstate": med("speedup_vs_fullstate"),
        "median_state_reduction": med("state_reduction"),
        "shapes": rows,
    }


def latency_leg(episodes=20, warmup=3, flush_mib=512):
    """Per-step latency of the single-request workloads: tiny (1 x 1 head,
    d = 32, W = 8, T = 3), r1_h16 W = 256 T = 3, and r1_h16 W = 256 T = 7 with
    S0 folded on the GPU from a 1024-token synthetic prompt.

    Per depth, median, p10 and p90 over `episodes` episodes with a HIP event
    pair around each launch, taken twice: warm (caches hold the previous
    episode's inputs and records) and cold (a `flush_mib` MiB buffer is
    read, untimed, before every step, which evicts the 256 MB last-level
    cache and the L2s). Also the mean per launch of back-to-back warm episodes
    with no event between the launches (an event marker between two kernels
    costs the GPU a few microseconds, a visible share of launches this short),
    and the algorithmic bytes per step with the HBM fraction they give.
    """
    import torch

    from linear_attention_beam_gdn_amd import Onela

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    flush = torch.ones(flush_mib << 20, dtype=torch.uint8, device=dev)
    res = {}
    for cfg in (0, 1, 2):
        shape = shape_of(cfg)
        R, H, W, T, dk, dv = shape.R, shape.H, shape.W, shape.T, shape.dk, shape.dv
        ep = make_episode(shape)
        up = lambda a: (torch.from_numpy(np.ascontiguousarray(a)).view(torch.int16) if a.dtype == np.uint16
                        else torch.from_numpy(np.ascontiguousarray(a))).to(dev)
        ins = [[up(ep[key][t]) for key in ("q", "k", "v", "alpha", "beta")] for t in range(T)]
        par = [None] + [up(ep["parents"][t].astype(np.int32)) for t in range(1, T)]
        o = torch.empty((R * W, H, dv), dtype=torch.float32, device=dev)
        lay = Onela(R, H, dk, dv, W, T, stream=stream)
        reqs = list(range(R))
        if shape.s0 == "prompt":
            prompt_s0(lay, shape, shape.prompt_len, reqs, dev, stream, need_f32=False)
            s0_label = f"prompt-derived on the GPU ({shape.prompt_len} synthetic tokens)"
        else:
            for r in reqs:
                lay.init_request(r, up(ep["S0"][r]))
            s0_label = f"N(0, {shape.s0_sigma}^2)"

        def episode(events=None, cold=False):
            for r in reqs:
                lay.reset(r)
            for t in range(T):
                if cold:
                    evict_caches(flush)                     # untimed: before the event pair
                if events is not None:
                    events[t][0].record(stream)
                lay.step(reqs, *ins[t], par[t], o)
                if events is not None:
                    events[t][1].record(stream)

        def instrumented(cold):
            evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in range(T)]
                   for _ in range(episodes)]
            for i in range(episodes):
                episode(evs[i], cold)
            torch.cuda.synchronize()
            return np.array([[evs[i][t][0].elapsed_time(evs[i][t][1]) for t in range(T)]
                             for i in range(episodes)]) * 1e3

        for _ in range(warmup):
            episode()
        torch.cuda.synchronize()
        warm = instrumented(False)
        cold = instrumented(True)
        reps = 10 * episodes
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            episode()
        e1.record(stream)
        torch.cuda.synchronize()
        b2b_us = e0.elapsed_time(e1) * 1e3 / (reps * T)
        lay.sync()
        lay.close()
        bytes_t = [step_bytes(shape, ep["parents"], t + 1)["total"] for t in range(T)]
        frac = lambda us: [round(b / (x * 1e-6) / 1e9 / HBM_PEAK_GBS, 4) for b, x in zip(bytes_t, us)]
        ws, cs = depth_stats(warm), depth_stats(cold)
        res[shape.name] = {
            "what": f"{R} request x {H} heads, d = {dk}, W = {W}, T = {T}, S0 {s0_label}, parents {shape.parents}",
            "algorithmic_bytes_by_depth": bytes_t,
            "cold_us_by_depth": cs,
            "warm_us_by_depth": ws,
            "cold_hbm_frac_by_depth": frac(cs["median"]),
            "warm_hbm_frac_by_depth": frac(ws["median"]),
            "warm_us_per_step_back_to_back": b2b_us,
            "warm_beam_steps_per_s_back_to_back": R * W / (b2b_us * 1e-6),
            "cold_us_per_step_mean_of_medians": float(np.mean(cs["median"])),
        }
        del ins, par, o
    del flush
    torch.cuda.empty_cache()
    return res


def stress_leg(episodes=3):
    """The stress workload: 64 requests x 32 heads, d = 128, W = 1024, T = 7,
    Zipf(1.2) parents (deep shared ancestry), inputs drawn on the GPU for all
    7 steps before timing (about 11 GB). Same timing method as the main leg:
    one event pair around back-to-back episodes, per-depth durations from a
    separate pass with events around every launch."""
    import torch

    from linear_attention_beam_gdn_amd import Onela
    from workload.gen_device import all_parents, s0_device, step_inputs

    shape = shape_of(4)
    R, H, W, T, d = shape.R, shape.H, shape.W, shape.T, shape.dk
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    parents = all_parents(shape)
    S0 = s0_device(shape, dev)
    ins = [step_inputs(shape, t, dev) for t in range(T)]
    par = [None] + [torch.from_numpy(parents[t].astype(np.int32)).to(dev) for t in range(1, T)]
    lay = Onela(R, H, d, d, W, T, stream=stream)
    for r in range(R):
        lay.init_request(r, S0[r].contiguous())
    del S0
    o = torch.empty((R * W, H, d), dtype=torch.float32, device=dev)
    reqs = list(range(R))

    def episode(events):
        for r in reqs:
            lay.reset(r)
        for t in range(T):
            x = ins[t]
            if events is not None:
                events[t][0].record(stream)
            lay.step(reqs, x["q"], x["k"], x["v"], x["alpha"], x["beta"], par[t], o)
            if events is not None:
                events[t][1].record(stream)

    episode(None)
    mean_s, wall, by_depth, per = time_episodes(episode, stream, episodes, T, instrumented=5)
    lay.sync()
    mem = lay.memory()
    lay.close()
    del ins, par, o
    torch.cuda.empty_cache()
    bytes_t = [step_bytes(shape, parents, t + 1) for t in range(T)]
    nbytes = float(np.mean([b["total"] for b in bytes_t]))
    gbs = nbytes / mean_s / 1e9
    return {
        "workload": shape.name,
        "what": "64 requests x 32 heads, d = 128, W = 1024, T = 7, parents Zipf(1.2) over the previous beams",
        "us_per_decode_step": wall / T * 1e6,
        "beam_steps_per_s": R * W * T / wall,
        "kernel_us_mean": mean_s * 1e6,
        "us_by_depth_instrumented": [round(float(x), 1) for x in by_depth],
        "us_by_depth_instrumented_stats": depth_stats(per),
        "hbm_frac_by_depth_instrumented": [round(b["total"] / (x * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                                           for b, x in zip(bytes_t, by_depth)],
        "unique_records_by_depth": [b["unique_records"] for b in bytes_t],
        "persistent_state_bytes": mem["s0_bytes"] + mem["record_bytes"] + mem["index_bytes"],
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": nbytes},
    }


def fullstate_leg(shape, q, k, v, al, be, par, o, S0, stream, onela_launch_s, onela_ms_per_step, onela_mem):
    """Same workload through the full-state comparator (a full state per beam)."""
    import torch

    from linear_attention_beam_gdn_amd import FullState

    R, H, W, T = shape.R, shape.H, shape.W, shape.T
    fs = FullState(R, H, shape.dk, shape.dv, W, T, stream=stream)
    for r in range(R):
        fs.init_request(r, S0[r].contiguous())
    reqs = list(range(R))
    ev = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in range(T)]
    per_t, walls = [], []
    for it in range(4):
        for r in reqs:
            fs.reset(r)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(T):
            ev[t][0].record(stream)
            fs.step(reqs, q[t], k[t], v[t], al[t], be[t], par[t], o)
            ev[t][1].record(stream)
        torch.cuda.synchronize()
        if it:
            walls.append(time.perf_counter() - t0)
            per_t.append([ev[t][0].elapsed_time(ev[t][1]) for t in range(T)])
    fs.sync()
    fs_mem = fs.memory()
    fs.close()
    sz = shape.dv * shape.dk * 4
    fs_launch_s = float(np.mean(per_t)) * 1e-3
    onela_persistent = onela_mem["s0_bytes"] + onela_mem["record_bytes"] + onela_mem["index_bytes"]
    per_beam_states = R * H * W * sz
    return {
        "what": "the same decode steps with a full d_v x d_k float32 state per beam (gather the parent's, write the new)",
        "kernel_us_mean": fs_launch_s * 1e6,
        "us_per_decode_step": float(np.median(walls)) / T * 1e6,
        "us_per_decode_step_by_depth": [round(float(x) * 1e3, 1) for x in np.median(np.array(per_t), axis=0)],
        "speedup_kernel": fs_launch_s / onela_launch_s,
        "speedup_step": float(np.median(walls)) / T * 1e3 / (onela_ms_per_step / T),
        "persistent_state_bytes": {"onela": onela_persistent, "fullstate_per_beam_states": per_beam_states,
                                   "fullstate_allocated": fs_mem},
        "state_reduction": per_beam_states / onela_persistent,
    }


# ------------------------------------------------------------ CPU baseline
def _oracle_pair(args):
    import oracle

    S0, q, k, v, a, b, par, gpu = args
    t0 = time.perf_counter()
    ref = oracle.full_state_episode(S0, q, k, v, a, b, par)
    cpu_s = time.perf_counter() - t0
    if gpu is None:
        return cpu_s, None, None
    g_o, g_d = gpu                                  # the GPU's o and delta of this pair, [T][W][dv]
    return cpu_s, float(np.max(np.abs(g_o - ref["o"]))), float(np.max(np.abs(g_d - ref["delta"])))


def baseline_pairs(shape, n_pairs: int):
    """The (request, head) pairs the CPU baseline runs (seeded)."""
    rng = np.random.default_rng(7)
    return [(int(rng.integers(shape.R)), int(rng.integers(shape.H))) for _ in range(n_pairs)]


def cpu_baseline(shape, ep, n_pairs: int, S0=None, gpu_outputs=None, s0_label="the run's S0"):
    """Oracle (float64 full state per beam) on n_pairs (request, head) pairs, all steps.

    S0: the run's S0 per request [R][H][dv][dk] (host float32), or None for the
    episode's drawn one. gpu_outputs: {(request, head): (o, delta)} of the GPU
    path on the same inputs for some of the pairs; the oracle's results for
    those are compared with them (max-abs), the same arithmetic the timing
    runs anyway."""
    import multiprocessing as mp

    visible = len(os.sched_getaffinity(0))
    # every host core this process may run on, unless the environment sets a
    # smaller CPU share (OMP_NUM_THREADS, the per-GPU share on shared hosts)
    share = os.environ.get("OMP_NUM_THREADS", "")
    cores = max(1, min(visible, int(share)) if share.isdigit() and int(share) > 0 else visible)
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"                     # one BLAS thread per worker
    pairs = baseline_pairs(shape, n_pairs)
    W = shape.W
    S0 = ep["S0"] if S0 is None else S0
    gpu_outputs = gpu_outputs or {}
    jobs = []
    for (r, h) in pairs:
        sl = slice(r * W, (r + 1) * W)
        f = lambda key: bf16_bits_to_f32(ep[key][:, sl, h, :])
        jobs.append((S0[r, h], f("q"), f("k"), f("v"), ep["alpha"][:, sl, h], ep["beta"][:, sl, h],
                     ep["parents"][:, r, :], gpu_outputs.get((r, h))))
    ctx = mp.get_context("fork")
    with ctx.Pool(min(cores, n_pairs)) as pool:
        t0 = time.perf_counter()
        per_pair = pool.map(_oracle_pair, jobs)
        wall = time.perf_counter() - t0
    beam_steps = W * shape.T * n_pairs / shape.H       # a beam-step covers all H heads
    checked = [x for x in per_pair if x[1] is not None]
    return {
        "value": beam_steps / wall,
        "unit": "beam-steps/s",
        "cores": min(cores, n_pairs),
        "kind": "oracle",
        "sample": (f"{n_pairs} (request, head) pairs of {shape.name}, all {shape.T} steps, float64 full state "
                   f"per beam, from {s0_label}; {wall:.1f} s wall, {sum(x[0] for x in per_pair):.1f} s CPU; "
                   f"scaled by {shape.H} heads per beam-step"),
        "max_abs_err_vs_gpu": ({"o": max(x[1] for x in checked), "delta": max(x[2] for x in checked),
                                "pairs": len({pr for pr in pairs if pr in gpu_outputs}), "bound": 1e-3,
                                "what": "the GPU path's o and delta of one untimed episode of the same inputs "
                                        "against the oracle's, over all steps and beams of these pairs"}
                               if checked else None),
        "cpu_model": _cpu_model(),
        "host_cpus_visible": visible,
        "workers": min(cores, n_pairs),
        "worker_rule": "len(os.sched_getaffinity(0)), capped by OMP_NUM_THREADS when the environment sets it "
                       "(the host's CPU share per GPU); BLAS threads 1 per worker",
    }


def _cpu_model() -> str:
    """The host CPU as /proc/cpuinfo names it: model name, family/model/stepping, sockets."""
    fields, sockets = {}, set()
    try:
        for line in open("/proc/cpuinfo"):
            if ":" not in line:
                continue
            key, val = (x.strip() for x in line.split(":", 1))
            if key == "physical id":
                sockets.add(val)
            elif key in ("model name", "cpu family", "model", "stepping", "vendor_id") and key not in fields:
                fields[key] = val
    except OSError:
        return "unknown"
    name = fields.get("model name", "unknown")
    return (f"{name} (vendor {fields.get('vendor_id', '?')}, family {fields.get('cpu family', '?')}, "
            f"model {fields.get('model', '?')}, stepping {fields.get('stepping', '?')}, "
            f"{max(1, len(sockets))} socket(s))")


# ------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50, help="timed episodes")
    ap.add_argument("--warmup", type=int, default=5, help="untimed episodes")
    ap.add_argument("--beams-per-block", type=int, default=0)
    ap.add_argument("--cpu-pairs", type=int, default=256, help="(request, head) pairs the oracle runs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fullstate", action="store_true", help="skip the full-state comparator leg")
    ap.add_argument("--s0", choices=("prompt", "normal"), default="prompt",
                    help="S0 folded on the GPU from a synthetic prompt (default) or drawn N(0, 0.05^2)")
    ap.add_argument("--prompt-len", type=int, default=5120, help="prompt tokens per request for --s0 prompt")
    ap.add_argument("--no-fused", action="store_true", help="skip the input-side fusion leg")
    ap.add_argument("--no-probes", action="store_true", help="skip the copy / MFMA-loop / projection probes")
    ap.add_argument("--no-replay", action="store_true", help="skip the replay-comparator leg")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the operator sweep (OneLA vs both comparators over 24 shapes)")
    ap.add_argument("--no-stress", action="store_true",
                    help="skip the stress-workload leg (64 requests x 32 heads, W = 1024, T = 7)")
    ap.add_argument("--no-latency", action="store_true",
                    help="skip the single-request latency leg (tiny, W = 256 T = 3, W = 256 T = 7 prompt-derived)")
    ap.add_argument("--layers", type=int, default=4,
                    help="layers of the multi-layer decode-step leg (eager vs HIP graph); 0 skips it")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="run one plain device copy of MIB MiB first (reference for hardware traffic counters)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) into the traffic file and exit")
    ap.add_argument("--traffic-command", default="", help="command recorded in the traffic file")
    ap.add_argument("--counters-from", nargs="+", metavar="DIR",
                    help="summarise rocprofv3 --pmc runs of this bench into the counters file and exit")
    ap.add_argument("--counters-command", default="", help="commands recorded in the counters file")
    ap.add_argument("--only", choices=("stress", "multi_layer", "latency"),
                    help="run this leg alone (after the copy probe) and print its JSON, for per-depth profiles")
    ap.add_argument("--profile-by-depth", nargs="+", metavar="DIR",
                    help="with --only LEG: FETCH_DIR WRITE_DIR [COUNTER_DIR ...] of rocprofv3 --pmc runs of that leg "
                         "alone; write its per-depth traffic and counter summary under profiles/ and exit")
    args = ap.parse_args()
    if args.counters_from:
        print(counters_from(args.counters_from, args.counters_command))
        return
    if args.traffic_from:
        print(traffic_from_counters(args.traffic_from[0], args.traffic_from[1], args.copy_probe or 256,
                                    args.traffic_command))
        return
    if args.profile_by_depth:
        if args.only not in ("stress", "multi_layer") or len(args.profile_by_depth) < 2:
            raise SystemExit("--profile-by-depth needs --only stress|multi_layer and at least FETCH_DIR WRITE_DIR")
        print(profile_by_depth(args.only, args.profile_by_depth[0], args.profile_by_depth[1],
                               args.profile_by_depth[2:], args.copy_probe or 256, args.counters_command))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(requests and heads would shard across GPUs with no exchange inside a step).", file=sys.stderr)
        sys.exit(2)

    import torch

    from linear_attention_beam_gdn_amd import Onela

    if args.copy_probe:
        src = torch.ones(args.copy_probe << 18, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.only == "stress":
        print(json.dumps({"stress_workload": stress_leg()}), flush=True)
        return
    if args.only == "latency":
        print(json.dumps({"latency_configs": latency_leg()}), flush=True)
        return
    shape = shape_of(3)
    R, H, W, T, dk, dv = shape.R, shape.H, shape.W, shape.T, shape.dk, shape.dv
    t_gen = time.perf_counter()
    ep = make_episode(shape)
    t_gen = time.perf_counter() - t_gen
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def up(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(torch.int16) if a.dtype == np.uint16 else t).to(dev)

    q = [up(ep["q"][t]) for t in range(T)]
    k = [up(ep["k"][t]) for t in range(T)]
    v = [up(ep["v"][t]) for t in range(T)]
    al = [up(ep["alpha"][t]) for t in range(T)]
    be = [up(ep["beta"][t]) for t in range(T)]
    par = [None] + [up(ep["parents"][t].astype(np.int32)) for t in range(1, T)]
    o = torch.empty((R * W, H, dv), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    if args.only == "multi_layer":
        print(json.dumps({"multi_layer": multi_layer_leg(shape, max(args.layers, 1), q, k, v, al, be, par,
                                                         up(ep["S0"]))}), flush=True)
        return
    lay = Onela(R, H, dk, dv, W, T, stream=stream)
    if args.beams_per_block:
        lay.set_beams_per_block(args.beams_per_block)
    reqs = list(range(R))
    prefill_out = None
    if args.s0 == "prompt":
        S0_dev, prefill_out = prompt_s0(lay, shape, args.prompt_len, reqs, dev, stream,
                                        need_f32=not (args.no_fullstate and args.no_fused and args.no_probes) or args.layers > 0)
        s0_label = (f"prompt-derived: the GDN recurrence over {args.prompt_len} synthetic tokens per request "
                    "and head, folded on the GPU (prefill_kernel)")
    else:
        for r in range(R):
            lay.init_request(r, up(ep["S0"][r]))
        S0_dev = None
        s0_label = "N(0, 0.05^2) float32 per head"

    def episode(events=None):
        for r in reqs:
            lay.reset(r)
        for t in range(T):
            if events is not None:
                events[t][0].record(stream)
            lay.step(reqs, q[t], k[t], v[t], al[t], be[t], par[t], o)
            if events is not None:
                events[t][1].record(stream)

    for _ in range(args.warmup):
        episode()
    lay.sync()
    torch.cuda.synchronize()

    # Timed region: args.steps episodes back to back, bracketed by
    # synchronisations and one pair of HIP events on the launch stream.
    mean_launch_s, wall_per_episode, med_t_us, per_t_us = time_episodes(episode, stream, args.steps, T,
                                                                        instrumented=20)
    lay.sync()
    # Cold pass (outside the timed region): the 256 MB last-level cache evicted by an
    # untimed 512 MiB read before every step, events around each launch. A layer that
    # steps alone finds part of the previous steps' records in that cache; inside a model
    # the other layers' steps evict them.
    flush = torch.ones(512 << 20, dtype=torch.uint8, device=dev)
    evict_caches(flush)
    cold_per = []
    for i in range(10):
        for r in reqs:
            lay.reset(r)
        evc = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in range(T)]
        for t in range(T):
            evict_caches(flush)
            evc[t][0].record(stream)
            lay.step(reqs, q[t], k[t], v[t], al[t], be[t], par[t], o)
            evc[t][1].record(stream)
        torch.cuda.synchronize()
        cold_per.append([evc[t][0].elapsed_time(evc[t][1]) * 1e3 for t in range(T)])
    del flush
    lay.sync()
    cold_per = np.array(cold_per)

    bytes_t = [step_bytes(shape, ep["parents"], t + 1) for t in range(T)]
    flops_t = [step_flops(shape, t + 1) for t in range(T)]
    bytes_per_launch = float(np.mean([b["total"] for b in bytes_t]))
    achieved_gbs = bytes_per_launch / mean_launch_s / 1e9
    proj_tflops = float(np.mean([f["projection"] for f in flops_t])) / mean_launch_s / 1e12

    ms_per_step = wall_per_episode * 1e3
    value = R * W * T / wall_per_episode
    traffic = read_traffic()
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "beam-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "precision": ("inputs q, k, v bf16; alpha, beta float32; S0 held as two bf16 planes hi + lo "
                      "(hi = rne(S0), lo = rne(S0 - hi): about 16 significant bits, ~2^-17 relative); "
                      "projection bf16 x bf16 products accumulated in float32 on the matrix cores; "
                      "replay, delta and o in float32; delta records float32"),
        "config": {
            "workload": shape.name,
            "requests": R, "heads": H, "d_k": dk, "d_v": dv, "beam_width": W, "decode_steps": T,
            "s0": s0_label, "parents": "top W of 4W candidates per request",
            "inputs": "bf16 q, k (L2-normalised), v; float32 alpha, beta",
            "step": "one episode = host rewind + 5 decode steps of one GDN layer, one launch each",
        },
        "us_per_decode_step": ms_per_step * 1e3 / T,
        "us_by_depth_instrumented": [round(float(x), 2) for x in med_t_us],
        "us_by_depth_instrumented_stats": depth_stats(per_t_us),
        "cold_cache": {
            "what": ("the same launches with the 256 MB last-level cache evicted (an untimed 512 MiB read) "
                     "before every step, events around each launch, 10 episodes; hbm_frac from the mean "
                     "of the per-depth medians (event markers included, as in us_by_depth_instrumented)"),
            "us_by_depth": depth_stats(cold_per),
            "us_per_launch": float(np.mean(np.median(cold_per, axis=0))),
            "hbm_frac": bytes_per_launch / (float(np.mean(np.median(cold_per, axis=0))) * 1e-6) / 1e9 / HBM_PEAK_GBS,
        },
        "kernel_us_mean": mean_launch_s * 1e6,
        "unique_records_by_depth": [b["unique_records"] for b in bytes_t],
        "roofline": {
            "bound": "hbm",
            "achieved": achieved_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved_gbs / HBM_PEAK_GBS,
            "traffic": traffic,
            "kernel": KERNEL_NAME,
            "algorithmic_bytes_per_launch": bytes_per_launch,
            "launch_duration": "HIP events around the timed region's back-to-back launches, divided by their number",
        },
        "counters": read_counters(),
        "input_generation_s": round(t_gen, 1),
    }
    if not args.no_probes:
        out["probes"], out["mfma_projection"] = probe_leg(shape, q, k, S0_dev if S0_dev is not None else up(ep["S0"]))
        out["mfma_projection"]["in_fused_step"] = {
            "achieved_tflops": proj_tflops, "frac": proj_tflops / BF16_PEAK_TFLOPS,
            "note": "the projection's flops over the whole fused launch, which HBM bounds"}
        mp = out["mfma_projection"]
        out["roofline_mfma"] = {
            "bound": "mfma", "kernel": "S0 [k q] projection phase of step_kernel",
            "achieved": mp["achieved_tflops"], "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": mp["frac"],
            "issued_frac": mp["issued_frac"],
            "flops": "algorithmic: 4 W d_v d_k per (request, head); issued counts the hi and lo MFMA of every "
                     "product (2x)",
            "method": "projection-only probe with the step kernel's tiles and S0 planes, operands of 8 pairs "
                      "resident in L2",
            "streamed_frac": mp["full_footprint"]["frac"],
            "w1024_resident_frac": mp["w1024_resident"]["frac"],
            "in_fused_step_frac": proj_tflops / BF16_PEAK_TFLOPS,
            "hbm_cap_frac": mp["hbm_cap_frac"],
            "target_frac": 0.4,
            "target_met_algorithmic": mp["frac"] >= 0.4,
        }
    if prefill_out is not None:
        out["prefill"] = prefill_out
    # One untimed episode whose o and delta the CPU baseline checks for its first
    # pairs (the same inputs and S0 as the timed episodes).
    gpu_check, S0_host = {}, None
    if not args.no_cpu_baseline and (S0_dev is not None or args.s0 != "prompt"):
        S0_host = S0_dev.cpu().numpy() if S0_dev is not None else None
        check = list(dict.fromkeys(baseline_pairs(shape, args.cpu_pairs)[:32]))   # (distinct pairs)
        d_chk = torch.empty_like(o)
        for r in reqs:
            lay.reset(r)
        got = {pr: ([], []) for pr in check}
        for t in range(T):
            lay.step(reqs, q[t], k[t], v[t], al[t], be[t], par[t], o, d_chk)
            torch.cuda.synchronize()
            for (r, h) in check:
                got[(r, h)][0].append(o[r * W:(r + 1) * W, h].cpu().numpy())
                got[(r, h)][1].append(d_chk[r * W:(r + 1) * W, h].cpu().numpy())
        lay.sync()
        gpu_check = {pr: (np.stack(a), np.stack(b)) for pr, (a, b) in got.items()}
        del d_chk
    mem = lay.memory()
    lay.close()
    if not args.no_fused:
        out["fused_inputs"] = fused_leg(shape, ep, q, k, v, al, be, par,
                                        S0_dev if S0_dev is not None else up(ep["S0"]), bytes_t)
    if args.layers > 0:
        S0_ml = S0_dev if S0_dev is not None else up(ep["S0"])
        out["multi_layer"] = multi_layer_leg(shape, args.layers, q, k, v, al, be, par, S0_ml)
        # the same layers for the first request alone: launches of a few microseconds,
        # where replaying a captured graph saves the per-launch host and dispatch work
        cut = lambda xs: [x[:W] for x in xs]
        out["multi_layer_one_request"] = multi_layer_leg(
            shape_of(shape.cfg, R=1), args.layers, cut(q), cut(k), cut(v), cut(al), cut(be),
            [None] + [x[:1] for x in par[1:]], S0_ml[:1])
    if not args.no_fullstate:
        out["fullstate_comparator"] = fullstate_leg(shape, q, k, v, al, be, par, o,
                                                    up(ep["S0"]) if S0_dev is None else S0_dev, stream,
                                                    mean_launch_s, ms_per_step, mem)
    if not args.no_replay:
        out["replay_comparator"] = replay_leg(shape, q, k, v, al, be, par, o,
                                              up(ep["S0"]) if S0_dev is None else S0_dev, stream,
                                              mean_launch_s, ms_per_step, mem)
    if not args.no_latency:
        out["latency_configs"] = latency_leg()
    if not args.no_stress:
        out["stress_workload"] = stress_leg()
    if not args.no_sweep:
        out["operator_sweep"] = sweep_leg()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(
            shape, ep, args.cpu_pairs, S0=S0_host, gpu_outputs=gpu_check,
            s0_label=("the run's S0" if (S0_host is not None or args.s0 != "prompt") else
                      "a drawn S0 (the oracle's cost does not depend on S0's values)"))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
