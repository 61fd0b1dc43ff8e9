"""Benchmark of the exact relative-position attention hot path on one MI355X.

A step is one forward + backward pass of all four mechanisms (T5, Shaw, DeBERTa, T-XL) over the
long-context workload B=4, H=8, L=8192, d=64, bidirectional, bf16 inputs with fp32 accumulation
(T5 32 buckets / max_distance 1024, Shaw k=256, DeBERTa k=512, T-XL full span).  The value is
the whole step's algorithmic TFLOP/s: F_fwd = 4 N d + F_rel and F_bwd = 10 N d + 3 F_rel per
mechanism, N = attended pairs, F_rel = 2 d x distinct (row, table-row) relation products (0 for
T5, N for T-XL).  Inputs are resident in HBM before the timed region.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Profiling helpers (rocprofv3 runs and their committed summaries under profiles/):
    python bench.py --only txl --copy-calibration-mib 1024 ...   (run under rocprofv3 --pmc)
    python bench.py --summarize-pmc FETCH.csv WRITE.csv --copy-mib 1024 --out profiles/X.md --cmd "..."
    python bench.py --summarize-stats kernel_stats.csv --out profiles/X.md --cmd "..."
The roofline's `traffic` is read from profiles/hbm_traffic_*.md, and only while the kernel
sources hash to the value recorded there (else null: the counters predate the kernel).
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0

MECH_ORDER = ("t5", "shaw", "deberta", "txl")
MECH_ID = {"t5": 0, "shaw": 1, "txl": 2, "deberta": 3}   # relpos_mech values
CSRC = os.path.join(ROOT, "exact_attention_relative_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
CFG_NAME = {"t5": "long_t5_L8192", "shaw": "long_shaw_L8192", "deberta": "long_deberta_L8192",
            "txl": "long_txl_L8192"}


# ------------------------------------------------------------------ algorithmic flop counts
def _allowed_count_per_row(L, wl, wr):
    i = np.arange(L)
    lo = np.zeros(L, dtype=np.int64) if wl < 0 else np.maximum(0, i - wl)
    hi = np.full(L, L - 1, dtype=np.int64) if wr < 0 else np.minimum(L - 1, i + wr)
    return lo, hi


def _distinct_clamped(lo_off, hi_off, lo_clip, hi_clip):
    """Number of distinct values of clamp(x, lo_clip, hi_clip) for integer x in [lo_off, hi_off]."""
    a = np.clip(lo_off, lo_clip, hi_clip)
    b = np.clip(hi_off, lo_clip, hi_clip)
    return np.where(hi_off >= lo_off, b - a + 1, 0)


def flop_counts(mech, B, H, L, d, wl, wr, span):
    """(N, F_rel) for one call: attended pairs and relation-product flops."""
    lo, hi = _allowed_count_per_row(L, wl, wr)
    per_row = np.maximum(hi - lo + 1, 0)
    n_pairs = int(per_row.sum()) * B * H
    i = np.arange(L)
    if mech in ("t5", "alibi"):
        rel = 0
    elif mech == "txl":
        rel = n_pairs
    elif mech == "shaw":
        # row i reads clamp(j - i, -k, k) for j in [lo, hi]
        rel = int(_distinct_clamped(lo - i, hi - i, -span, span).sum()) * B * H
    elif mech == "deberta":
        # c2p: clamp(i - j + k) per query row; p2c: clamp(j - i + k) per key column
        c2p = _distinct_clamped(i - hi, i - lo, -span, span - 1).sum()
        jlo, jhi = _allowed_count_per_row(L, wr, wl)   # queries attending key j
        p2c = _distinct_clamped(i - jhi, i - jlo, -span, span - 1).sum()
        rel = int(c2p + p2c) * B * H
    else:
        raise ValueError(mech)
    return n_pairs, 2 * d * rel


def pass_flops(mech, B, H, L, d, wl, wr, span):
    n, frel = flop_counts(mech, B, H, L, d, wl, wr, span)
    return {"fwd": 4 * n * d + frel, "bwd": 10 * n * d + 3 * frel,
            # split of the backward between its two kernels (accounting convention)
            "bwd_dq": 2 * n * d + 2 * frel, "bwd_dkdv": 8 * n * d + frel, "pairs": n}


# ------------------------------------------------------------------ profile summaries
def kernel_source_sha():
    """Hash of every kernel source file: counters taken on other sources are stale."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h")) and not f.startswith(("relpos_probe", "relpos_proj")):
            h.update(f.encode())
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


_KNAME = re.compile(r"(fwd|bwd)_kernel(?:_\dwg)?<([^>]*)>")


def pass_of_kernel(name):
    """(mechanism, pass) of a library kernel name, or None for helpers (prep, aggregation)."""
    m = _KNAME.search(name)
    if not m:
        return None
    # template arguments: element type, then the integers (mechanism[, direction, part])
    args = [int(a) for a in (x.strip() for x in m.group(2).split(",")) if a.lstrip("-").isdigit()]
    inv = {v: k for k, v in MECH_ID.items()}
    if args[0] not in inv:
        return None
    if m.group(1) == "fwd":
        return inv[args[0]], "fwd"
    return inv[args[0]], ("bwd_dq" if args[1] == 0 else "bwd_dkdv")


def _pmc_rows(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def summarize_pmc(fetch_csv, write_csv, copy_mib, out, cmd):
    """HBM bytes per pass from FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each divided by the
    factor the same counter reads for a plain copy of copy_mib MiB; a pass's kernels are weighted
    by their dispatches per pass."""
    known_kib = copy_mib * 1024.0
    res = {}
    for ctr, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = [r for r in _pmc_rows(path) if r["Counter_Name"] == ctr]
        copies = [float(r["Counter_Value"]) for r in rows if "copy" in r["Kernel_Name"].lower()]
        factor = max(copies) / known_kib
        per = {}
        for r in rows:
            key = pass_of_kernel(r["Kernel_Name"])
            if key is None:
                continue
            name = r["Kernel_Name"].replace("relpos::", "")
            per.setdefault(key, {}).setdefault(name, []).append(float(r["Counter_Value"]))
        res[ctr] = (factor, per)
    f_fetch, per_fetch = res["FETCH_SIZE"]
    f_write, per_write = res["WRITE_SIZE"]
    sha = kernel_source_sha()
    lines = ["# HBM traffic per launch from rocprofv3 counters (long-context workload, L=8192)", "",
             "Commands (run from the repository root on one MI355X; one counter per run):", "",
             "```", cmd, "```", "",
             f"Copy calibration: a plain {copy_mib} MiB device copy reads FETCH_SIZE = "
             f"{f_fetch:.4f} x its bytes and WRITE_SIZE = {f_write:.4f} x its bytes; the kernel "
             "counters below are divided by these factors.", "",
             "| pass | kernel | dispatches | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | "
             "calibrated MB/dispatch |", "|---|---|---:|---:|---:|---:|"]
    records = []
    for key in sorted(per_fetch):
        # a pass may be several kernels, some dispatched more than once per pass (the folded
        # launches): the kernel dispatched least often runs once per pass
        passes = min(len(vals) for vals in per_fetch[key].values())
        total = 0.0
        for name, vals in sorted(per_fetch[key].items()):
            fv = float(np.mean(vals))
            wv = float(np.mean(per_write.get(key, {}).get(name, [0.0])))
            b = (fv / f_fetch + wv / f_write) * 1024.0
            total += b * len(vals) / passes
            lines.append(f"| {key[0]} {key[1]} | `{name[:70]}` | {len(vals)} | {fv:.1f} | {wv:.1f} | "
                         f"{b / 1e6:.1f} |")
        records.append({"mech": key[0], "pass": key[1], "source_sha": sha,
                        "bytes_per_pass": total})
    lines += ["", f"Kernel sources hash: `{sha}`.", ""]
    for r in records:
        lines.append("traffic-record: " + json.dumps(r))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def summarize_stats(stats_csv, out, cmd, title):
    rows = _pmc_rows(stats_csv)
    lines = [f"# {title}", "", "Command (run from the repository root on one MI355X):", "",
             "```", cmd, "```", "",
             "| kernel | pass | calls | avg (us) | min (us) | max (us) | share of GPU time |",
             "|---|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        name = r["Name"].replace("relpos::", "").replace("|", "/")
        key = pass_of_kernel(r["Name"])
        tag = f"{key[0]} {key[1]}" if key else "helper"
        if len(name) > 80:
            name = name[:80] + "..."
        lines.append(f"| `{name}` | {tag} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.2f}% |")
    lines += ["", f"Kernel sources hash: `{kernel_source_sha()}`."]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def summarize_trace_by_grid(trace_csv, out, cmd, title, pattern):
    """Mean / min duration per (kernel, grid size) of the kernels whose name contains `pattern`,
    from a rocprofv3 kernel trace (one row per dispatch)."""
    rows = _pmc_rows(trace_csv)
    groups = {}
    for r in rows:
        if pattern not in r["Kernel_Name"]:
            continue
        name = r["Kernel_Name"].replace("relpos::", "").replace("(anonymous namespace)::", "")
        name = re.sub(r"\(.*", "", name).replace("void ", "")
        grid = int(r["Grid_Size_X"]) // max(int(r["Workgroup_Size_X"]), 1)
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        groups.setdefault((name, grid), []).append(dur)
    lines = [f"# {title}", "", "Commands (run from the repository root on one MI355X):", "",
             "```", cmd, "```", "",
             "| kernel | workgroups | dispatches | mean (us) | min (us) |",
             "|---|---:|---:|---:|---:|"]
    for (name, grid), d in sorted(groups.items()):
        lines.append(f"| `{name}` | {grid} | {len(d)} | {float(np.mean(d)):.1f} | {min(d):.1f} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


SQ_SET1 = ("SQ_WAVES SQ_INSTS_VALU SQ_INSTS_SALU SQ_INSTS_LDS SQ_INSTS_VALU_TRANS_F32 "
           "SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_WAVE_CYCLES SQ_BUSY_CYCLES")
SQ_SET2 = ("SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_WAIT_INST_LDS SQ_LDS_BANK_CONFLICT "
           "SQ_LDS_IDX_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_WAIT_ANY GRBM_GUI_ACTIVE")


def summarize_sq(csv1, csv2, out, cmd, steps_per_wave=128):
    """Per-kernel instruction mix (per wave and 64-row step) and pipe utilisation from the two
    SQ counter runs.  GRBM_GUI_ACTIVE is summed over the 8 XCDs; MFMA-busy cycles are divided
    by (GUI / 8) x 1024 SIMDs."""
    data, cnt = {}, {}
    for path in (csv1, csv2):
        for r in _pmc_rows(path):
            key = pass_of_kernel(r["Kernel_Name"])
            if key is None:
                continue
            name = r["Kernel_Name"].replace("relpos::", "")
            d = data.setdefault((key, name), {})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            cnt[(key, name, r["Counter_Name"])] = cnt.get((key, name, r["Counter_Name"]), 0) + 1
    lines = ["# SQ counters per kernel (long-context workload, L=8192)", "",
             "Commands (run from the repository root on one MI355X; two counter sets, one run each):",
             "", "```", cmd, "```", "",
             "Per wave and 64-row step (`/ step`: SQ_INSTS_* / SQ_WAVES / 128 steps; general passes "
             "sweep only part of the steps, so theirs read low). `MFMA busy` = "
             "SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024 SIMDs). `VALU active` = "
             "SQ_ACTIVE_INST_VALU x 4 on the same base. `wait` = SQ_WAIT_ANY / SQ_WAVE_CYCLES. "
             "`bank conflicts` = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE. `LDS active` = "
             "SQ_LDS_IDX_ACTIVE / (GRBM_GUI_ACTIVE / 8 x 256 CUs).", "",
             "| pass | kernel | VALU / step | SALU / step | LDS / step | exp / step | MFMA ops / step | "
             "MFMA busy | VALU active | LDS active | wait | bank conflicts |",
             "|---|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for (key, name), d in sorted(data.items()):
        g = lambda c: d.get(c, 0.0) / max(cnt.get((key, name, c), 0), 1)
        waves = g("SQ_WAVES")
        if waves <= 0:
            continue
        ws = waves * steps_per_wave
        simd = g("GRBM_GUI_ACTIVE") / 8 * 1024
        lines.append(
            f"| {key[0]} {key[1]} | `{name[:48]}` | {g('SQ_INSTS_VALU') / ws:.0f} | "
            f"{g('SQ_INSTS_SALU') / ws:.0f} | {g('SQ_INSTS_LDS') / ws:.0f} | "
            f"{g('SQ_INSTS_VALU_TRANS_F32') / ws:.1f} | {g('SQ_INSTS_VALU_MFMA_MOPS_BF16') / ws / 64:.1f} | "
            f"{g('SQ_VALU_MFMA_BUSY_CYCLES') / max(simd, 1):.3f} | "
            f"{4 * g('SQ_ACTIVE_INST_VALU') / max(simd, 1):.3f} | "
            f"{g('SQ_LDS_IDX_ACTIVE') / max(simd / 4, 1):.3f} | "
            f"{g('SQ_WAIT_ANY') / max(g('SQ_WAVE_CYCLES'), 1):.3f} | "
            f"{g('SQ_LDS_BANK_CONFLICT') / max(g('SQ_LDS_IDX_ACTIVE'), 1):.3f} |")
    lines += ["", "`MFMA ops / step` counts 32x32x16 bf16 MFMAs (MOPS_BF16 / 64).", "",
              f"Kernel sources hash: `{kernel_source_sha()}`."]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def recorded_traffic(mech, pass_name):
    """Calibrated HBM bytes of one (mech, pass) pass, if counters exist for these sources."""
    sha = kernel_source_sha()
    for path in sorted(glob.glob(os.path.join(PROFILES, "hbm_traffic_*.md"))):
        with open(path) as f:
            for line in f:
                if line.startswith("traffic-record: "):
                    r = json.loads(line[len("traffic-record: "):])
                    if r["mech"] == mech and r["pass"] == pass_name and r["source_sha"] == sha:
                        return r["bytes_per_pass"], os.path.relpath(path, ROOT)
    return None, None


# ------------------------------------------------------------------ GPU side
def build_mech(mech, torch):
    from exact_attention_relative_amd import runner
    from exact_attention_relative_amd.inputs import make_config
    case = make_config(CFG_NAME[mech])
    desc = runner.desc_for(case)
    dev = runner.to_device(case)
    ws_f, nf = runner.workspace(desc, 0)
    ws_b, nb = runner.workspace(desc, 1)
    o = torch.empty_like(dev["q"])
    lse = torch.empty(dev["q"].shape[:-1], dtype=torch.float32, device="cuda")
    grads = runner.alloc_grads(desc, dev)
    cfg = case["config"]
    B, H, L, d = case["shape"]
    fl = pass_flops(mech, B, H, L, d, cfg["window"][0], cfg["window"][1], cfg.get("rel_span", 0))
    return dict(mech=mech, case=case, desc=desc, dev=dev, ws_f=ws_f, ws_b=ws_b, o=o, lse=lse,
                grads=grads, flops=fl)


def run_fwd(m):
    from exact_attention_relative_amd import relpos_attn_fwd
    from exact_attention_relative_amd.runner import slots
    d = m["dev"]
    relpos_attn_fwd(m["desc"], d["q"], d["k"], d["v"], *slots(d), m["o"], m["lse"], m["ws_f"],
                    m["ws_f"].numel())


def run_bwd(m):
    from exact_attention_relative_amd import runner
    runner.backward(m["desc"], m["dev"], m["o"], m["lse"], ws=m["ws_b"], grads=m["grads"])


GROUP_WORKGROUPS = 512   # the library's wave of workgroups (two per CU on 256 CUs)


def pass_launches(case, mech, kernel):
    """Launches of one pass kernel per call, by the library's launch rule: the T-XL key-side pass
    runs its batch entries as `fold` consecutive launches (the fewest groups of batch entries that
    give one wave of workgroups) when one batch entry gives at most one wave, else slice groups.
    Shaw and DeBERTa passes are two kernels (light, general) and are not counted here."""
    B, H, L, _ = case["shape"]
    nb = (L + 127) // 128
    if mech in ("shaw", "deberta"):
        return None
    if mech == "txl" and kernel == "bwd_dkdv":
        if H * nb <= GROUP_WORKGROUPS:
            ng = next((g for g in range(1, B + 1) if g * H * nb >= GROUP_WORKGROUPS), B)
            return -(-B // ng)
        group = max(1, min(B * H, GROUP_WORKGROUPS // nb))
        return -(-(B * H) // group)
    return 1


def step(mechs, hook=None):
    """One pass of the hot path.  hook = (mech, kernel_id, start, stop) records one kernel."""
    from exact_attention_relative_amd import relpos_profile_events, RELPOS_PROF_OFF
    for m in mechs:
        on = hook is not None and hook[0] == m["mech"]
        if on:
            relpos_profile_events(hook[2], hook[3], hook[1])
        run_fwd(m)
        run_bwd(m)
        if on:
            relpos_profile_events(None, None, RELPOS_PROF_OFF)


def measured_mfma_peak(torch):
    """Sustained dense bf16 MFMA rate of this device (measurement-only probe library)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "exact_attention_relative_amd", "librelpos_probe.so"))
    lib.relpos_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                           ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
    blocks = 2048
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    val = ctypes.c_double(0.0)
    rc = lib.relpos_probe_mfma_bf16(500, blocks, ctypes.c_void_p(out.data_ptr()), ctypes.byref(val),
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if rc != 0:
        raise RuntimeError(f"MFMA probe failed ({rc})")
    return val.value


def measured_valu_rates(torch):
    """Sustained vector-ALU rates of this device in giga lane-operations per second: the base-2
    exponential (v_exp_f32) and the fp32 fused multiply-add (measurement-only probe library)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "exact_attention_relative_amd", "librelpos_probe.so"))
    lib.relpos_probe_valu.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                      ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
    blocks = 2048
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    rates = {}
    for kind, name in ((0, "exp2_Glane_ops_per_s"), (1, "fma_f32_Glane_ops_per_s")):
        val = ctypes.c_double(0.0)
        rc = lib.relpos_probe_valu(kind, 2000, blocks, ctypes.c_void_p(out.data_ptr()),
                                   ctypes.byref(val),
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"vector-ALU probe {kind} failed ({rc})")
        rates[name] = val.value
    return rates


def probe_overlap(torch, iters=4000):
    """How much vector work hides under matrix work on one SIMD (measurement-only probe
    library).  For each workgroup count: matrix units alone, vector units alone, both in every
    wave, and both split over the two halves of 512-thread workgroups (the same number of them:
    one wave of each kind per SIMD, the same work as the first two together).  `hidden` is the
    share of the shorter alone-time that disappears: 1 = full overlap (the time is the longer
    alone-time), 0 = none (their sum)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "exact_attention_relative_amd", "librelpos_probe.so"))
    lib.relpos_probe_overlap.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                         ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
    res = []
    for blocks in (256, 512):   # one or two workgroups per CU, all resident
        out = torch.empty(2 * blocks * 256, dtype=torch.float32, device="cuda")
        t = {}
        for mode, nb in ((0, blocks), (1, blocks), (2, blocks), (3, blocks)):
            val = ctypes.c_double(0.0)
            rc = lib.relpos_probe_overlap(mode, iters, nb, ctypes.c_void_p(out.data_ptr()),
                                          ctypes.byref(val),
                                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            if rc != 0:
                raise RuntimeError(f"overlap probe mode {mode} failed ({rc})")
            t[mode] = val.value
        lo, hi = min(t[0], t[1]), max(t[0], t[1])
        res.append({"workgroups_per_cu": blocks / 256, "matrix_ms": t[0], "vector_ms": t[1],
                    "in_wave_ms": t[2], "across_waves_ms": t[3],
                    "hidden_in_wave": (t[0] + t[1] - t[2]) / lo,
                    "hidden_across_waves": (t[0] + t[1] - t[3]) / lo})
    return res


PASS_REPS = 10   # repetitions behind each per-mechanism forward / backward median


def time_kernel(torch, mechs, mech, kid, reps=50):
    evs = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    for a, b in evs:
        step([m for m in mechs if m["mech"] == mech], hook=(mech, kid, a, b))
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in evs]))


def cpu_baseline(budget_heads=1):
    """The fp64 oracle, as it stands, on one (batch, head) slice of each mechanism's workload
    (forward + backward), timed on the host cores; scaled to TFLOP/s by the slice's flops."""
    from exact_attention_relative_amd.inputs import make_config
    from oracle import relpos_oracle as orc
    cores = len(os.sched_getaffinity(0))
    threads = int(os.environ.get("OMP_NUM_THREADS", cores))
    tot_s, tot_f, fwd_s, bwd_s = 0.0, 0.0, 0.0, 0.0
    for mech in MECH_ORDER:
        case = make_config(CFG_NAME[mech])
        p = orc.Params(**case["params"])
        tab = {n: t.astype(np.float64) for n, t in case["tables"].items()}
        cfg = case["config"]
        B, H, L, d = case["shape"]
        fl = pass_flops(mech, 1, budget_heads, L, d, cfg["window"][0], cfg["window"][1],
                        cfg.get("rel_span", 0))
        for h in range(budget_heads):
            t0 = time.time()
            orc.forward_rows(p, case["q"], case["k"], case["v"], tab, 0, h)
            t1 = time.time()
            orc.backward_head(p, case["q"], case["k"], case["v"], tab, case["dout"], 0, h)
            t2 = time.time()
            fwd_s += t1 - t0
            bwd_s += t2 - t1
            tot_s += t2 - t0
        tot_f += fl["fwd"] + fl["bwd"]
        del case, tab
    return {"value": tot_f / tot_s / 1e12, "unit": "TFLOP/s", "cores": min(cores, threads),
            "kind": "oracle", "fwd_seconds": fwd_s, "bwd_seconds": bwd_s,
            "sample": f"forward + backward of {budget_heads} (batch, head) slice(s) of each of the "
                      f"four mechanisms at L=8192 (fp64 NumPy oracle), {tot_s:.1f} s"}


STRESS_SETTINGS = {"t5": dict(num_buckets=32, max_distance=1024), "shaw": dict(rel_span=256),
                   "deberta": dict(rel_span=512), "txl": {}, "alibi": {}}
STRESS_MECHS = MECH_ORDER + ("alibi",)


STRESS_WARMUP = 4   # untimed forward + backward calls per case before the timed ones


def run_stress(torch, lengths, reps=10, windows=None):
    """Fixed token budget B * L = 32768 (H = 8, d = 64, bf16) at several lengths, or at
    L = 8192 with several symmetric local windows: forward and backward time, algorithmic
    TFLOP/s (pairs inside the window only), peak memory and workspace."""
    from exact_attention_relative_amd import runner, relpos_attn_fwd
    from exact_attention_relative_amd.inputs import make_case
    out = []
    cases = [(L, -1) for L in lengths] if windows is None else [(8192, w) for w in windows]
    for mech in STRESS_MECHS:
        for L, win in cases:
            B = max(1, 32768 // L)
            c = make_case(mech, B, 8, L, 64, dtype="bf16", window=(win, win), seed=L + max(win, 0),
                          sub=STRESS_MECHS.index(mech), **STRESS_SETTINGS[mech])
            desc = runner.desc_for(c)
            torch.cuda.synchronize()
            base = torch.cuda.memory_allocated()
            dev = runner.to_device(c)
            ws_f, _ = runner.workspace(desc, 0)
            ws_b, _ = runner.workspace(desc, 1)
            o = torch.empty_like(dev["q"])
            lse = torch.empty(dev["q"].shape[:-1], dtype=torch.float32, device="cuda")
            grads = runner.alloc_grads(desc, dev)
            fwd = lambda: relpos_attn_fwd(desc, dev["q"], dev["k"], dev["v"], *runner.slots(dev), o,
                                          lse, ws_f, ws_f.numel())
            bwd = lambda: runner.backward(desc, dev, o, lse, ws=ws_b, grads=grads)
            torch.cuda.reset_peak_memory_stats()
            fwd(); bwd()
            torch.cuda.synchronize()
            peak = torch.cuda.max_memory_allocated() - base
            for _ in range(STRESS_WARMUP - 1):   # (the first call above is one warm-up)
                fwd(); bwd()
            torch.cuda.synchronize()
            tf, tb = [], []
            for _ in range(reps):
                e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
                e[0].record(); fwd(); e[1].record(); bwd(); e[2].record()
                torch.cuda.synchronize()
                tf.append(e[0].elapsed_time(e[1]))
                tb.append(e[1].elapsed_time(e[2]))
            fl = pass_flops(mech, B, 8, L, 64, win, win, STRESS_SETTINGS[mech].get("rel_span", 0))
            mf, mb = float(np.median(tf)), float(np.median(tb))
            out.append({"mech": mech, "B": B, "L": L, "window": win, "fwd_ms": mf, "bwd_ms": mb,
                        "fwd_TFLOPs": fl["fwd"] / mf / 1e9, "bwd_TFLOPs": fl["bwd"] / mb / 1e9,
                        "peak_mem_GiB": peak / 2**30, "workspace_bwd_GiB": ws_b.numel() / 2**30,
                        "naive_fp32_bias_GiB": B * 8 * L * L * 4 / 2**30})
            print(f"[stress] {mech} L={L} window={win}: fwd {mf:.2f} ms, bwd {mb:.2f} ms", file=sys.stderr,
                  flush=True)
            del dev, ws_f, ws_b, o, lse, grads
            torch.cuda.empty_cache()
    return out


PROJ_SHAPES = (("txl_L8192_causal", 8192, 512, 8, 64, "sinusoid", 0),
               ("txl_L8192_full", 16383, 512, 8, 64, "sinusoid", None),
               ("deberta_span512", 1024, 64, 2, 64, "normal", None))


def run_projections(torch, reps=20, per=20):
    """The relation-table projections around the attention calls (T-XL r = R W_r; DeBERTa
    Kr | Qr = P [W_r^k | W_r^q]) at the long-context shapes: forward, dW alone (T-XL's R is
    fixed) and dX + dW, bf16 and fp32 operands; per call, the median over `reps` replays
    of a graph of `per` calls."""
    import exact_attention_relative_amd as ear
    from exact_attention_relative_amd.inputs import make_projection_case
    from exact_attention_relative_amd.runner import tensor_from_f32
    out = []
    for name, N, F, H, d, basis, first in PROJ_SHAPES:
        for dt in ("bf16", "fp32"):
            c = make_projection_case(N, F, H, d, dtype=dt, basis=basis, first_offset=first, seed=1)
            X, W = tensor_from_f32(c["X"], dt), tensor_from_f32(c["W"], dt)
            drel = tensor_from_f32(c["drel"], "fp32")
            desc = ear.make_proj_desc(N, F, H, d, dtype=dt)
            rel = torch.empty((H, N, d), device="cuda",
                              dtype=torch.bfloat16 if dt == "bf16" else torch.float32)
            dX = torch.empty((N, F), device="cuda")
            dW = torch.empty((F, H * d), device="cuda")
            n = ear.relpos_project_workspace_size(desc)
            ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
            calls = {"fwd": lambda: ear.relpos_project_fwd(desc, X, W, rel),
                     "bwd_dW": lambda: ear.relpos_project_bwd(desc, X, W, drel, None, dW, ws, n),
                     "bwd_dX_dW": lambda: ear.relpos_project_bwd(desc, X, W, drel, dX, dW, ws, n)}
            e = 2 if dt == "bf16" else 4
            flops = {"fwd": 2.0 * N * F * H * d, "bwd_dW": 2.0 * N * F * H * d,
                     "bwd_dX_dW": 4.0 * N * F * H * d}
            nbytes = {"fwd": e * (N * F + F * H * d + N * H * d),
                      "bwd_dW": e * (N * F) + 4 * (N * H * d + F * H * d),
                      "bwd_dX_dW": e * (N * F + F * H * d) + 4 * (N * H * d + N * F + F * H * d)}
            row = {"shape": name, "N": N, "F": F, "H": H, "d": d, "dtype": dt,
                   "dW_slices": max(1, n // (F * H * d * 4))}
            for k, fn in calls.items():
                # device time only: `per` calls back to back in a captured graph, so host
                # marshalling between calls does not idle the GPU inside the timed region
                fn()
                torch.cuda.synchronize()
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph):
                    for _ in range(per):
                        fn()
                graph.replay()
                torch.cuda.synchronize()
                evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                       for _ in range(reps)]
                for a, b in evs:
                    a.record(); graph.replay(); b.record()
                torch.cuda.synchronize()
                ms = float(np.median([a.elapsed_time(b) for a, b in evs])) / per
                del graph
                row[k + "_us"] = ms * 1e3
                row[k + "_TFLOPs"] = flops[k] / ms / 1e9
                row[k + "_GBs"] = nbytes[k] / ms / 1e6
            print(f"[proj] {name} {dt}: fwd {row['fwd_us']:.1f} us, dW {row['bwd_dW_us']:.1f} us, "
                  f"dX+dW {row['bwd_dX_dW_us']:.1f} us", file=sys.stderr, flush=True)
            out.append(row)
            del X, W, drel, rel, dX, dW, ws
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stress", default=None, metavar="L1,L2,...",
                    help="length stress at a fixed token budget (prints its own JSON line)")
    ap.add_argument("--windows", default=None, metavar="W1,W2,...",
                    help="symmetric local windows at L=8192 (prints its own JSON line)")
    ap.add_argument("--probe-overlap", action="store_true",
                    help="time matrix / vector work alone, in one wave and across waves")
    ap.add_argument("--projections", action="store_true",
                    help="time the relation-table projections (prints its own JSON line)")
    ap.add_argument("--only", default=None,
                    help="comma-separated mechanisms (profiling runs; the value then covers only them)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this size first (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--summarize-stats", metavar="KERNEL_STATS_CSV")
    ap.add_argument("--summarize-sq", nargs=2, metavar=("SET1_CSV", "SET2_CSV"))
    ap.add_argument("--summarize-trace", nargs=2, metavar=("KERNEL_TRACE_CSV", "NAME_PATTERN"),
                    help="per (kernel, grid) durations from a kernel trace")
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--out")
    ap.add_argument("--cmd", default="")
    ap.add_argument("--title", default="rocprofv3 kernel statistics")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, args.copy_mib, args.out, args.cmd)
        return
    if args.summarize_stats:
        summarize_stats(args.summarize_stats, args.out, args.cmd, args.title)
        return
    if args.summarize_sq:
        summarize_sq(*args.summarize_sq, args.out, args.cmd)
        return
    if args.summarize_trace:
        trace_csv, pattern = args.summarize_trace
        summarize_trace_by_grid(trace_csv, args.out, args.cmd, args.title, pattern)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(the workload shards over (batch, head) with no exchange except a table-gradient "
              "all-reduce, which is not implemented)", file=sys.stderr)
        sys.exit(2)

    import torch
    from exact_attention_relative_amd import (RELPOS_PROF_BWD_DKDV, RELPOS_PROF_BWD_DQ,
                                              RELPOS_PROF_FWD)
    torch.cuda.init()
    if args.stress:
        lengths = [int(x) for x in args.stress.split(",") if x]
        print(json.dumps({"stress": run_stress(torch, lengths), "tokens_per_batch": 32768,
                          "heads": 8, "head_dim": 64, "dtype": "bf16", "data": "synthetic"}))
        return
    if args.windows:
        wins = [int(x) for x in args.windows.split(",") if x]
        print(json.dumps({"windows": run_stress(torch, [], windows=wins), "L": 8192, "B": 4,
                          "heads": 8, "head_dim": 64, "dtype": "bf16", "data": "synthetic"}))
        return
    if args.projections:
        print(json.dumps({"projections": run_projections(torch), "data": "synthetic"}))
        return
    if args.probe_overlap:
        print(json.dumps({"overlap": probe_overlap(torch)}))
        return
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * 2**20 // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()
    order = MECH_ORDER if args.only is None else tuple(x for x in args.only.split(",") if x)
    mechs = []
    per_mech = {}
    for mech in order:
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        m = build_mech(mech, torch)
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        run_fwd(m)
        torch.cuda.synchronize()
        peak_fwd = torch.cuda.max_memory_allocated() - base
        run_bwd(m)
        torch.cuda.synchronize()
        peak_all = torch.cuda.max_memory_allocated() - base
        mechs.append(m)
        B_, H_, L_, d_ = m["case"]["shape"]
        io = B_ * H_ * L_ * d_ * 2 * 8 + B_ * H_ * L_ * 4 * 2   # q k v o dout dq dk dv (bf16), lse, D
        tab = sum(t.size for t in m["case"]["tables"].values()) * (2 + 4)   # tables + fp32 grads
        per_mech[mech] = {"peak_mem_fwd_GiB": peak_fwd / 2**30, "peak_mem_fwd_bwd_GiB": peak_all / 2**30,
                          "analytic_min_GiB": (io + tab) / 2**30,
                          "workspace_fwd_GiB": m["ws_f"].numel() / 2**30,
                          "workspace_bwd_GiB": m["ws_b"].numel() / 2**30,
                          "naive_fp32_bias_GiB": 4 * m["case"]["shape"][0] * m["case"]["shape"][1] * m["case"]["shape"][2] ** 2 / 2**30}
        print(f"[bench] built {mech}", file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        step(mechs)
    torch.cuda.synchronize()

    # per-pass times of each mechanism (separate from the timed region)
    kid = {"fwd": RELPOS_PROF_FWD, "bwd_dq": RELPOS_PROF_BWD_DQ, "bwd_dkdv": RELPOS_PROF_BWD_DKDV}
    kernel_ms = {}
    for m in mechs:
        mech = m["mech"]
        for name, k in kid.items():
            kernel_ms[(mech, name)] = time_kernel(torch, mechs, mech, k)
        # per-mechanism forward / backward: medians over PASS_REPS event-timed repetitions
        evs3 = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(PASS_REPS)]
        for ev in evs3:
            ev[0].record(); run_fwd(m); ev[1].record(); run_bwd(m); ev[2].record()
        torch.cuda.synchronize()
        tf = float(np.median([ev[0].elapsed_time(ev[1]) for ev in evs3]))
        tb = float(np.median([ev[1].elapsed_time(ev[2]) for ev in evs3]))
        fl = m["flops"]
        per_mech[mech].update({
            "fwd_ms": tf, "bwd_ms": tb,
            "fwd_TFLOPs": fl["fwd"] / tf / 1e9, "bwd_TFLOPs": fl["bwd"] / tb / 1e9,
            "fwd_bwd_TFLOPs": (fl["fwd"] + fl["bwd"]) / (tf + tb) / 1e9,
            "fwd_bwd_frac_bf16_peak": (fl["fwd"] + fl["bwd"]) / (tf + tb) / 1e9 / PEAK_BF16_TFLOPS,
            "kernel_ms": {n: kernel_ms[(mech, n)] for n in kid}})
    dom = max(kernel_ms, key=kernel_ms.get)
    dom_mech, dom_kernel = dom
    dm = next(m for m in mechs if m["mech"] == dom_mech)

    # ---- timed region ----
    evs = []
    for _ in range(args.steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(); b.record()
        evs.append((a, b))
    t_start, t_stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for s in range(args.steps):
        step(mechs, hook=(dom_mech, kid[dom_kernel], evs[s][0], evs[s][1]))
    t_stop.record()
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_stop) / args.steps
    dom_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))

    step_flops = sum(m["flops"]["fwd"] + m["flops"]["bwd"] for m in mechs)
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    dom_flops = dm["flops"][dom_kernel]
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12
    traffic, traffic_src = recorded_traffic(dom_mech, dom_kernel)
    peak_meas = measured_mfma_peak(torch)
    valu_meas = measured_valu_rates(torch)
    # the pass may be several launches of one kernel: flops, time and traffic are per pass
    nl = pass_launches(dm["case"], dom_mech, dom_kernel)
    traffic_launch = traffic / nl if (traffic is not None and nl) else None
    roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                "traffic_per_launch": traffic_launch,
                "kernel": f"{dom_kernel} pass kernel, {dom_mech}", "avg_ms": dom_ms,
                "launches": nl, "avg_launch_ms": dom_ms / nl if nl else None,
                "flops_per_launch": dom_flops, "traffic_source": traffic_src,
                "peak_measured": peak_meas, "frac_of_measured": achieved / peak_meas,
                "valu_measured": valu_meas,
                "kernel_source_sha": kernel_source_sha()}

    cpu = None
    if not args.no_cpu_baseline:
        for m in mechs:
            del m["dev"]
        mechs.clear()
        torch.cuda.empty_cache()
        cpu = cpu_baseline()

    out = {
        "metric": "fwd+bwd TFLOP/s and % bf16 MFMA peak at L=8192 per mechanism; peak memory",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "frac_bf16_peak": value / PEAK_BF16_TFLOPS,
        "config": {"workload": "long-context relative-position attention: B=4 H=8 L=8192 d=64, "
                               "bidirectional; T5 32 buckets max_distance 1024, Shaw k=256, "
                               "DeBERTa k=512, T-XL full span; fwd+bwd of all four per step",
                   "global_batch": 4, "seq_len": 8192, "heads": 8, "head_dim": 64,
                   "mechanisms": [m for m in order]},
        "per_mechanism": per_mech,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
