"""Summarise rocprofv3 CSV output of bench.py into short text reports.

    python -m paged_kv_cache_226_amd.rocprof_summary --workload llama2_7b \
        [--kv-dtype fp16|fp8] \
        --kernel-trace DIR [--fetch DIR --write DIR --tcc DIR --sq DIR --valu DIR] \
        --command "..." --out-dir profiles
    python -m paged_kv_cache_226_amd.rocprof_summary --workload llama2_7b \
        --sweep-profile SWEEP.jsonl --fetch DIR --out-dir profiles

Inputs are the directories rocprofv3 wrote with `--output-format csv`
(`*_kernel_stats.csv`, `*_counter_collection.csv`).  Writes (the tag is the
workload name, with `_fp8` appended for E4M3 caches):
  pa_decode_<tag>_kernel_trace.md   per-kernel durations
  pa_decode_<tag>_counters.md       per prefetch mode: HBM bytes, L2 hit
                                         rate, stall share, instructions,
                                         VALU busy, MFMA utilisation
  pa_decode_<tag>_traffic.txt       HBM bytes per launch, read by bench.py
                                         while the kernel sources are unchanged
  pa_decode_sweep_<workload>_fetch.md  HBM read bytes per point of the
                                         batch x context sweep

FETCH_SIZE and WRITE_SIZE are scaled by what the same counters read for
kernels of known size in the same process (bench.py --profile runs a 1 GiB
streaming read and a 1 GiB fp16 elementwise copy).
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

MODE_NAMES = {0: "off", 1: "l2", 2: "reg", 3: "both", 4: "reg2", 5: "lds", 6: "lds2",
              10: "two_loop_off", 11: "two_loop_l2", 12: "two_loop_reg", 13: "two_loop_both"}
# pa_decode_kernel<PF, DBG, KV8, TWO, EVEN>; the two-loop instances count as
# modes 10 + PF; the even split's instances count as their look-ahead mode
DECODE_RE = re.compile(r"pa_decode_kernel<(\d), (true|false), (true|false)"
                       r"(?:, (true|false))?(?:, (true|false))?>")
KV8 = False  # which cache type's kernels the summary counts (set by main)


def _rows(d, suffix):
    out = []
    for f in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
        with open(f) as fh:
            out.extend(csv.DictReader(fh))
    return out


def counters(d):
    """{(kernel name, counter): [values per dispatch]}"""
    agg = collections.defaultdict(list)
    for r in _rows(d, "_counter_collection.csv"):
        agg[(r["Kernel_Name"], r["Counter_Name"])].append(float(r["Counter_Value"]))
    return agg


def mean(v):
    return sum(v) / len(v) if v else float("nan")


def decode_mode(name):
    m = DECODE_RE.search(name)
    if not m or m.group(2) != "false" or (m.group(3) == "true") != KV8:
        return None
    return int(m.group(1)) + (10 if m.group(4) == "true" else 0)


def per_mode(agg, counter):
    out = {}
    for (k, c), v in agg.items():
        if c == counter and decode_mode(k) is not None:
            out[decode_mode(k)] = mean(v)
    return out


def calibration(agg, counter, kind):
    """Known bytes / counter bytes for a calibration kernel."""
    best = None
    for (k, c), v in agg.items():
        if c != counter:
            continue
        if kind == "stream" and "stream_read_kernel" in k:
            best = mean(v)
        if kind == "copy" and "elementwise_kernel" in k:
            val = mean(v)
            if best is None or val > best:
                best = val
    if not best:
        return None
    return (1 << 30) / (best * 1024.0)


def kernel_stats(d):
    rows = _rows(d, "_kernel_stats.csv")
    return [(r["Name"], int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
             float(r["MaxNs"]) / 1e3, float(r["Percentage"])) for r in rows]


def sweep_fetch(profile_jsonl, fetch_dir, workload, out_dir, command):
    """FETCH_SIZE per point of a `bench.py --sweep --profile` run: the decode
    dispatches, in launch order, are matched to the points the run printed
    (modes x launches each), scaled by the 1 GiB streaming-read calibration
    and divided by the point's algorithmic KV bytes."""
    points = [json.loads(l) for l in open(profile_jsonl) if l.startswith('{"sweep_profile"')]
    rows = sorted(_rows(fetch_dir, "_counter_collection.csv"), key=lambda r: int(r["Dispatch_Id"]))
    per_dispatch = collections.OrderedDict()
    for r in rows:
        if r["Counter_Name"] == "FETCH_SIZE":
            key = int(r["Dispatch_Id"])
            if key not in per_dispatch:
                per_dispatch[key] = [r["Kernel_Name"], 0.0]
            per_dispatch[key][1] += float(r["Counter_Value"])
    fk = calibration({(n, "FETCH_SIZE"): [v] for n, v in per_dispatch.values()}, "FETCH_SIZE",
                     "stream")
    decode = [(decode_mode(n), v) for n, v in per_dispatch.values() if decode_mode(n) is not None]
    lines = [f"# FETCH_SIZE per point of the batch x context sweep: {workload}", "", "```",
             "command:", *["    " + c for c in command.split(" ;; ") if c],
             f"FETCH_SIZE scale: {fk} (1 GiB streaming read in the same process)", "```", "",
             "HBM read bytes / algorithmic KV bytes, per look-ahead mode (mean over the "
             "launches of each mode):", "",
             "| batch | context | KV bytes | partitions | off | reg | l2 |",
             "|---|---|---|---|---|---|---|"]
    i = 0
    for pt in points:
        ratios = {}
        for m in pt["modes"]:
            vals = []
            for _ in range(pt["launches_per_mode"]):
                mode, v = decode[i]
                i += 1
                assert mode == m, (pt, mode, m)
                vals.append(v)
            ratios[m] = sum(vals) / len(vals) * 1024 * fk / pt["kv_bytes"]
        lines.append(f"| {pt['batch']} | {pt['context']} | {pt['kv_bytes']} | "
                     f"{pt['partitions']} | {ratios[0]:.4f} | {ratios[2]:.4f} | {ratios[1]:.4f} |")
    assert i == len(decode), (i, len(decode))
    path = os.path.join(out_dir, f"pa_decode_sweep_{workload}_fetch.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


def sweep_timing(jsonl, workload, out_dir, command):
    """µs and GB/s per point of a `bench.py --sweep` run, look-ahead off and
    in the default mode, with the sampled parity of the default mode."""
    points = [json.loads(l) for l in open(jsonl) if l.startswith('{"sweep"')]
    lines = [f"# Batch x context sweep, timings: {workload}", "", "```", "command:",
             *["    " + c for c in command.split(" ;; ") if c], "```", "",
             "One decode step per point (prepared call, event-timed mean over the steps); "
             "KV bytes = 2 * Hkv * 128 * 2 B * batch * context.  Every context of a point "
             "is the point's context, which the calls pass as min_context_hint.  'on' is "
             "the library's default look-ahead and 'off' the look-ahead off, each on its "
             "own plan; parity is the default mode's output on the first and last "
             "sequence (every head) against the fp64 oracle.  'partitions' is the plan's: "
             "per sequence for a fixed split, the most one sequence may get for a balanced "
             "one (sized on the device).  'W / cap' is the default mode's waves per "
             "work-group and residency cap (- = none).", "",
             "| batch | context | KV bytes | split | partitions | W / cap | us off | us on |"
             " GB/s off | GB/s on | % of 8 TB/s on | on vs off | parity abs | parity rel |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for p in points:
        off_gbps = p["kv_bytes"] / p["us_off"] / 1e3
        split = "one" if p["partitions"] == 1 else ("balanced" if p.get("balanced") else "fixed")
        wc = f"{p.get('waves_per_wg', '?')} / {p.get('resident_wgs') or '-'}"
        lines.append(f"| {p['batch']} | {p['context']} | {p['kv_bytes']} | {split} | "
                     f"{p['partitions']} | {wc} | {p['us_off']:.2f} | {p['us_on']:.2f} | "
                     f"{off_gbps:.0f} | "
                     f"{p['GBps_on']:.0f} | {p['pct_hbm_peak_on']:.1f} | "
                     f"{p['speedup_on_vs_off']:.3f} | {p['parity_abs']:.2e} | "
                     f"{p['parity_rel']:.2e} |")
    path = os.path.join(out_dir, f"pa_decode_sweep_{workload}_timing.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


def timeline_table(jsonl, workload, kv_dtype, out_dir, command):
    """Per-XCD table of a `bench.py --timeline` run."""
    r = [json.loads(l) for l in open(jsonl) if l.startswith('{"timeline"')][-1]
    tag = workload + ("_fp8" if kv_dtype == "fp8" else "") + \
        ("" if r["min_context_hint"] else "_nohint")
    c = r["cu_last_end_us"]
    lines = [f"# pa_decode per-work-group timeline: {tag}", "", "```", "command:",
             *["    " + x for x in command.split(" ;; ") if x], "```", "",
             "The timed plan run once more in the checked kernel variant with the debug "
             "timeline: each work-group's start and end (s_memrealtime, 100 MHz) and the "
             "HW_ID / XCC_ID of its CU.  Times are from the launch's first start; the run "
             "whose span is the median of five is shown.", "",
             f"- plan: {r['waves_per_wg']} waves per work-group, residency cap "
             f"{r['resident_wgs'] or '-'}, {r['workgroups']} work-groups, "
             f"min_context_hint {r['min_context_hint']}",
             f"- kernel (event-timed mean): {r['kernel_us_plain']} us plain, "
             f"{r['kernel_us_traced']} us with the timeline; span of the shown run: "
             f"{r['span_us']} us",
             f"- CUs seen: {r['cus_seen']}; each CU's last work-group ends between "
             f"{c['min']} and {c['max']} us (median {c['median']})",
             "- share of CUs still busy at 80 / 90 / 95 % of the span: " +
             " / ".join(f"{100 * v:.0f} %" for v in r["cus_busy_at_80_90_95_pct_of_span"]),
             f"- KV bytes {r['kv_bytes']}: {r['kv_bytes'] / r['span_us'] / 1e3:.0f} GB/s over "
             "the span", "",
             "| XCD | work-groups | work-group index mod 8 | mean work-group us | last end us |",
             "|---|---|---|---|---|"]
    for x in r["per_xcd"]:
        lines.append(f"| {x['xcd']} | {x['workgroups']} | "
                     f"{','.join(str(v) for v in x['wg_index_mod_8'])} | {x['mean_wg_us']} | "
                     f"{x['last_end_us']} |")
    path = os.path.join(out_dir, f"pa_decode_{tag}_timeline.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


# Derived figures of the request-path passes, per decode launch.  The SQ
# clock count GRBM_GUI_ACTIVE is summed over the 8 XCDs; per-CU figures
# divide by the 256 CUs (one TA and one TCP each).
REQUEST_PATH_DERIVED = [
    ("kernel us", None),
    ("TCP->TCC read requests", lambda c, k: c["TCP_TCC_READ_REQ_sum"]),
    ("TCP->TCC mean read latency (cycles)",
     lambda c, k: c["TCP_TCC_READ_REQ_LATENCY_sum"] / c["TCP_TCC_READ_REQ_sum"]),
    ("TCP->TCC reads in flight per CU",
     lambda c, k: c["TCP_TCC_READ_REQ_LATENCY_sum"] / (c["GRBM_GUI_ACTIVE"] / 8) / 256),
    ("TA address stage stalled by TCP (% of CU cycles)",
     lambda c, k: 100 * c["TA_ADDR_STALLED_BY_TC_CYCLES_sum"] / (c["GRBM_GUI_ACTIVE"] / 8) / 256),
    ("TA busy (% of CU cycles)",
     lambda c, k: 100 * c["TA_TA_BUSY_sum"] / (c["GRBM_GUI_ACTIVE"] / 8) / 256),
    ("TCP stalled on data pending from L2 (% of CU cycles)",
     lambda c, k: 100 * c["TCP_PENDING_STALL_CYCLES_sum"] / (c["GRBM_GUI_ACTIVE"] / 8) / 256),
    ("TCP read tag-conflict stall cycles", lambda c, k: c["TCP_READ_TAGCONFLICT_STALL_CYCLES_sum"]),
    ("L2 (TCC) requests", lambda c, k: c["TCC_REQ_sum"]),
    ("L2 tag stall cycles", lambda c, k: c["TCC_TAG_STALL_sum"]),
    ("HBM (EA) read requests", lambda c, k: c["TCC_EA0_RDREQ_sum"]),
    ("HBM (EA) reads in flight", lambda c, k: c["TCC_EA0_RDREQ_LEVEL_sum"] / (c["GRBM_GUI_ACTIVE"] / 8)),
    ("HBM (EA) mean read latency (cycles)",
     lambda c, k: c["TCC_EA0_RDREQ_LEVEL_sum"] / c["TCC_EA0_RDREQ_sum"]),
    ("DRAM credit stall cycles", lambda c, k: c["TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum"]),
    ("address-translation misses (UTCL1)", lambda c, k: c["TCP_UTCL1_TRANSLATION_MISS_sum"]),
]


def request_path_table(dirs, tag, head, out_dir, kernel_us):
    """Per look-ahead mode, the mean per launch of every counter in the given
    passes (summed over the instances rocprofv3 reports, e.g. TCC channels
    and XCDs), next to the kernel-trace duration, and the derived figures of
    REQUEST_PATH_DERIVED."""
    per = collections.defaultdict(dict)
    names = []
    for d in dirs:
        agg = collections.defaultdict(float)
        launches = collections.defaultdict(set)
        for r in _rows(d, "_counter_collection.csv"):
            m = decode_mode(r["Kernel_Name"])
            if m is None:
                continue
            agg[(m, r["Counter_Name"])] += float(r["Counter_Value"])
            launches[(m, r["Counter_Name"])].add(r["Dispatch_Id"])
        for (m, c), v in agg.items():
            per[m][c] = v / max(1, len(launches[(m, c)]))
            if c not in names:
                names.append(c)

    def fmt(v):
        return f"{v:.4g}" if isinstance(v, float) else str(v)

    def derived(m, f):
        try:
            return fmt(float(f(per[m], kernel_us.get(m))))
        except (KeyError, ZeroDivisionError, TypeError):
            return ""

    modes = sorted(per)
    lines = ["# pa_decode memory request path per look-ahead mode: " + tag, "", "```", *head,
             "```", "",
             "Per decode launch (mean over the profiled launches of each mode).  "
             "GRBM_GUI_ACTIVE is summed over the 8 XCDs, so per-CU figures use "
             "GRBM_GUI_ACTIVE / 8 cycles and 256 CUs; 'in flight' is a latency sum "
             "divided by the cycles (Little's law).", "",
             "| figure | " + " | ".join(MODE_NAMES[m] for m in modes) + " |",
             "|---|" + "---|" * len(modes)]
    for label, f in REQUEST_PATH_DERIVED:
        if f is None:
            cells = [f"{kernel_us[m]:.2f}" if m in kernel_us else "" for m in modes]
        else:
            cells = [derived(m, f) for m in modes]
        lines.append(f"| {label} | " + " | ".join(cells) + " |")
    lines += ["", "Raw counters (sums over instances, per launch):", "",
              "| counter | " + " | ".join(MODE_NAMES[m] for m in modes) + " |",
              "|---|" + "---|" * len(modes)]
    for c in names:
        lines.append(f"| {c} | " + " | ".join(fmt(per[m].get(c, float('nan'))) for m in modes)
                     + " |")
    path = os.path.join(out_dir, f"pa_decode_{tag}_request_path.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


# (mode, look-ahead distance, structure) of each profiled mode, as bench.py
# runs them (0 = the library's default distance)
MODE_OPTIONS = {0: (0, 1, 0), 1: (1, 1, 0), 2: (2, 1, 0), 3: (3, 1, 0), 4: (2, 2, 0),
                5: (4, 1, 0), 6: (4, 2, 0), 10: (0, 1, 1), 11: (1, 1, 1), 12: (2, 1, 1),
                13: (3, 1, 1)}


def mode_plans(w, kv8, hint):
    """Each mode's own plan for workload w on the MI355X figures, with the
    caller's context hint as bench.py passes it: 'waves W, cap R, P parts'."""
    from paged_kv_cache_226_amd import _native as nat
    from paged_kv_cache_226_amd import inputs as gen
    ctx = gen.workload_context_lens(w)
    MB = w.max_blocks_per_seq or max(-(-int(c) // 16) for c in ctx)
    sh = nat.make_shape(w.num_seqs, w.num_q_heads, w.num_kv_heads, MB, w.pool_blocks or 1,
                        kv_dtype=nat.KV_E4M3 if kv8 else nat.KV_F16)
    dev = dict(compute_units=256, lds_bytes_per_cu=163840, lds_bytes_per_workgroup=163840)
    out = {}
    for m, (pf, dist, structure) in MODE_OPTIONS.items():
        if kv8 and structure:
            continue
        o = nat.default_options()
        o.prefetch, o.prefetch_distance, o.structure = pf, dist, structure
        o.min_context_hint = hint
        p = nat.plan(sh, o, device=dev)
        if p["even_split"]:
            out[m] = (f"{p['waves_per_wg']} waves, cap {p['resident_wgs']}, even split over "
                      f"{p['workgroups']} shares")
        else:
            out[m] = (f"{p['waves_per_wg']} waves, cap {p['resident_wgs'] or '-'}, "
                      f"{p['num_partitions']} partition(s)" +
                      (" balanced" if p["balanced"] else ""))
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--kv-dtype", choices=("fp16", "fp8"), default="fp16")
    ap.add_argument("--no-context-hint", action="store_true",
                    help="the profiled runs planned without min_context_hint (bench.py "
                         "--no-context-hint): summaries are tagged _nohint")
    ap.add_argument("--kernel-trace")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--tcc")
    ap.add_argument("--sq")
    ap.add_argument("--valu", help="pass with SQ_ACTIVE_INST_VALU SQ_VALU_MFMA_BUSY_CYCLES "
                                   "SQ_INSTS SQ_WAVE_CYCLES GRBM_GUI_ACTIVE")
    ap.add_argument("--request-path", nargs="*", default=[],
                    help="counter directories of passes over the memory request path "
                         "(TA / TD / TCP / TCC / EA counters): one table of their per-mode "
                         "means, pa_decode_<tag>_request_path.md")
    ap.add_argument("--sweep-timing", help="JSON lines of `bench.py --sweep`: writes the "
                                           "per-point timing table")
    ap.add_argument("--timeline", help="JSON line of `bench.py --timeline`: writes "
                                       "pa_decode_<tag>_timeline.md")
    ap.add_argument("--command", default="", help="the command lines that produced the inputs")
    ap.add_argument("--source-hash", default="")
    ap.add_argument("--out-dir", default="profiles")
    ap.add_argument("--sweep-profile", help="JSON lines of `bench.py --sweep --profile`; with "
                                            "--fetch, writes the per-point FETCH_SIZE table")
    a = ap.parse_args(argv)

    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from paged_kv_cache_226_amd import accounting as acc
    from paged_kv_cache_226_amd import inputs as gen

    global KV8
    KV8 = a.kv_dtype == "fp8"
    if a.sweep_profile:
        print(sweep_fetch(a.sweep_profile, a.fetch, a.workload, a.out_dir, a.command))
        return 0
    if a.sweep_timing:
        print(sweep_timing(a.sweep_timing, a.workload, a.out_dir, a.command))
        return 0
    if a.timeline:
        print(timeline_table(a.timeline, a.workload, a.kv_dtype, a.out_dir, a.command))
        return 0
    tag = a.workload + ("_fp8" if KV8 else "") + ("_nohint" if a.no_context_hint else "")
    w = gen.WORKLOADS[a.workload]
    ctx = gen.workload_context_lens(w)
    kv = acc.step_kv_bytes(w.num_kv_heads, 128, ctx, elem_bytes=1 if KV8 else 2)
    other = acc.step_other_bytes(w.num_seqs, w.num_q_heads, 128, ctx)
    os.makedirs(a.out_dir, exist_ok=True)
    head = [f"workload: {a.workload} ({w.description}), KV cache {'E4M3' if KV8 else 'fp16'}",
            f"algorithmic KV bytes per launch: {kv}  (Q, output, block tables: {other})",
            "command:", *["    " + c for c in a.command.split(" ;; ") if c]]
    if a.source_hash:
        head.append(f"kernel_source_hash: {a.source_hash} (bench.py kernel_source_hash of the "
                    "profiled sources)")
    hint = 0 if a.no_context_hint else max(int(min(ctx)), 0)
    head.append(f"plans (each mode on its own plan, min_context_hint {hint} as bench.py "
                "passes it; 256 CUs):")
    head.extend(f"    {MODE_NAMES[m]}: {desc}" for m, desc in mode_plans(w, KV8, hint).items())

    if a.kernel_trace:
        lines = ["# pa_decode kernel trace: " + tag, "", "```", *head, "```", "",
                 "| kernel | calls | avg us | min us | max us | % time | effective KV GB/s |",
                 "|---|---|---|---|---|---|---|"]
        for name, calls, avg, mn, mx, pct in sorted(kernel_stats(a.kernel_trace),
                                                     key=lambda r: -r[5]):
            gbps = f"{kv / avg / 1e3:.0f}" if decode_mode(name) is not None else ""
            lines.append(f"| `{name[:70]}` | {calls} | {avg:.2f} | {mn:.2f} | {mx:.2f} | "
                         f"{pct:.1f} | {gbps} |")
        with open(os.path.join(a.out_dir, f"pa_decode_{tag}_kernel_trace.md"), "w") as f:
            f.write("\n".join(lines) + "\n")

    # average duration of each mode's decode kernel (kernel trace)
    kernel_us = {}
    if a.kernel_trace:
        for name, calls, avg, mn, mx, pct in kernel_stats(a.kernel_trace):
            if decode_mode(name) is not None:
                kernel_us[decode_mode(name)] = avg

    if a.request_path:
        request_path_table(a.request_path, tag, head, a.out_dir, kernel_us)

    if a.fetch and a.write:
        fa, wa = counters(a.fetch), counters(a.write)
        fk_stream = calibration(fa, "FETCH_SIZE", "stream")
        fk_copy = calibration(fa, "FETCH_SIZE", "copy")
        wk_copy = calibration(wa, "WRITE_SIZE", "copy")
        fk = fk_stream or fk_copy
        fetch = per_mode(fa, "FETCH_SIZE")
        write = per_mode(wa, "WRITE_SIZE")
        tcc = counters(a.tcc) if a.tcc else {}
        hit, miss = per_mode(tcc, "TCC_HIT"), per_mode(tcc, "TCC_MISS")
        sq = counters(a.sq) if a.sq else {}
        wait, wcyc = per_mode(sq, "SQ_WAIT_INST_ANY"), per_mode(sq, "SQ_WAVE_CYCLES")
        wait_any = per_mode(sq, "SQ_WAIT_ANY")
        valu, waves = per_mode(sq, "SQ_INSTS_VALU"), per_mode(sq, "SQ_WAVES")
        vmem = per_mode(sq, "SQ_INSTS_VMEM_RD")
        va = counters(a.valu) if a.valu else {}
        v_act, v_mfma = per_mode(va, "SQ_ACTIVE_INST_VALU"), per_mode(va, "SQ_VALU_MFMA_BUSY_CYCLES")
        v_insts, v_wcyc = per_mode(va, "SQ_INSTS"), per_mode(va, "SQ_WAVE_CYCLES")
        v_gui = per_mode(va, "GRBM_GUI_ACTIVE")
        lines = ["# pa_decode counters per look-ahead mode: " + tag, "", "```", *head,
                 f"FETCH_SIZE scale: {fk_stream} (1 GiB streaming read), {fk_copy} (1 GiB copy)",
                 f"WRITE_SIZE scale: {wk_copy} (1 GiB copy)", "```", "",
                 "GRBM_GUI_ACTIVE is summed over the 8 XCDs in the CSV: divided by 8.",
                 "VALU busy = 100 * SQ_ACTIVE_INST_VALU / 256 CUs / GRBM_GUI_ACTIVE "
                 "(rocprofv3's VALUBusy); MFMA util = 100 * SQ_VALU_MFMA_BUSY_CYCLES / "
                 "(GRBM_GUI_ACTIVE * 1024 SIMDs) (its MfmaUtil); cycles / instruction = "
                 "4 * SQ_WAVE_CYCLES / SQ_INSTS (per wave); stall cycles / instruction = "
                 "4 * SQ_WAIT_INST_ANY / SQ_INSTS (cycles a wave waits per instruction it "
                 "issues; the two counters come from different passes over the same launches); "
                 "wait share = SQ_WAIT_ANY / SQ_WAVE_CYCLES (waiting for anything, "
                 "s_waitcnt included).",
                 "",
                 "| mode | HBM read bytes | read / algorithmic | HBM write bytes | L2 hit rate |"
                 " stall share (SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES) | VALU insts / wave |"
                 " VMEM reads / wave | VALU busy | MFMA util | cycles / instruction |"
                 " stall cycles / instruction | wait share (SQ_WAIT_ANY / SQ_WAVE_CYCLES) |",
                 "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
        traffic, evidence = {}, {}
        for m in sorted(fetch):
            rb = fetch[m] * 1024 * fk if fk else float("nan")
            wb = write.get(m, float("nan")) * 1024 * (wk_copy or 1.0)
            traffic[m] = rb + wb
            hr = hit[m] / (hit[m] + miss[m]) if m in hit and (hit[m] + miss[m]) else float("nan")
            st = wait[m] / wcyc[m] if m in wait and wcyc.get(m) else float("nan")
            vw = valu[m] / waves[m] if m in valu and waves.get(m) else float("nan")
            mw = vmem[m] / waves[m] if m in vmem and waves.get(m) else float("nan")
            gui = v_gui.get(m, float("nan")) / 8
            vb = 100 * v_act.get(m, float("nan")) / 256 / gui if gui else float("nan")
            mu = 100 * v_mfma.get(m, float("nan")) / (gui * 1024) if gui else float("nan")
            cpi = 4 * v_wcyc[m] / v_insts[m] if v_insts.get(m) and m in v_wcyc else float("nan")
            spi = 4 * wait[m] / v_insts[m] if v_insts.get(m) and m in wait else float("nan")
            wa = wait_any[m] / wcyc[m] if m in wait_any and wcyc.get(m) else float("nan")
            evidence[m] = (hr, wa, st, spi, cpi)
            lines.append(f"| {MODE_NAMES[m]} | {rb:.4g} | {rb / kv:.4f} | {wb:.4g} | "
                         f"{100 * hr:.2f} % | {100 * st:.1f} % | {vw:.0f} | {mw:.0f} | "
                         f"{vb:.1f} % | {mu:.1f} % | {cpi:.1f} | {spi:.1f} | {100 * wa:.1f} % |")
        with open(os.path.join(a.out_dir, f"pa_decode_{tag}_counters.md"), "w") as f:
            f.write("\n".join(lines) + "\n")
        with open(os.path.join(a.out_dir, f"pa_decode_{tag}_traffic.txt"), "w") as f:
            f.write("# HBM bytes per decode-kernel launch (FETCH_SIZE + WRITE_SIZE, scaled)\n")
            f.write(f"# workload: {tag}\n")
            f.write(f"kernel_source_hash: {a.source_hash}\n")
            f.write(f"fetch_scale: {fk}\nwrite_scale: {wk_copy}\n")
            f.write(f"algorithmic_kv_bytes: {kv}\n")
            for m, v in sorted(traffic.items()):
                f.write(f"hbm_bytes_per_launch_{MODE_NAMES[m]}: {v:.0f}\n")
            # the look-ahead evidence per mode: L2 hit rate, wait share
            # (SQ_WAIT_ANY / SQ_WAVE_CYCLES), issue-stall share
            # (SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES) as fractions; stall cycles
            # per instruction and cycles per instruction of a wave; the
            # kernel-trace average duration; nan if not taken
            for m, (hr, wa, st, spi, cpi) in sorted(evidence.items()):
                f.write(f"l2_hit_rate_{MODE_NAMES[m]}: {hr:.4f}\n")
                f.write(f"wait_share_{MODE_NAMES[m]}: {wa:.4f}\n")
                f.write(f"issue_stall_share_{MODE_NAMES[m]}: {st:.4f}\n")
                f.write(f"stall_cycles_per_inst_{MODE_NAMES[m]}: {spi:.2f}\n")
                f.write(f"cycles_per_inst_{MODE_NAMES[m]}: {cpi:.2f}\n")
            for m, us in sorted(kernel_us.items()):
                f.write(f"kernel_us_{MODE_NAMES[m]}: {us:.2f}\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
