"""Benchmark: paged decode attention on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--also NAMES]
                    [--prefetch MODE] [--kv-dtype fp16|fp8]

A step is one paged_attn_decode call over the whole batch (the decode kernel,
plus the cross-partition reduce when the plan splits contexts), i.e. one
layer's decode attention, with every input already resident in HBM.  The
printed JSON line reports, for the headline workload (--workload, default the
Llama2-7B-shaped MHA layer), effective KV GB/s (algorithmic KV bytes / time)
as `value`, µs/step, the fraction of the 8 TB/s HBM peak, the roofline of the
decode kernel, per-prefetch-mode timings, the streaming-read ceiling measured
in the same run, the fp64 CPU oracle timed on the host cores, and the parity
of the timed call's own output against the oracle.  Every workload of --also
(default: the Llama3-8B-shaped GQA 4:1 layer) gets the same block, without
the CPU timing, under `targets`.

Inputs are synthetic (seeded N(0,1) Q/K/V, shuffled block tables) with the
shapes of the workload; see paged_kv_cache_226_amd/inputs.py.  The caches
live in one pool with each (block, KV head)'s K and V slices side by side
(--kv-layout separate: two pools, vLLM's layout).  With
--kv-dtype fp8 the same draw is quantized to OCP E4M3 with per-tensor scales
and the KV bytes count one byte per value.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode attention µs/step + effective KV GB/s (% of HBM peak), 1 GPU"
KERNEL_SOURCES = ["paged_kv_cache_226_amd/csrc/pa_kernels.hip",
                  "paged_kv_cache_226_amd/csrc/pa_api.cpp",
                  "paged_kv_cache_226_amd/csrc/pa_internal.h"]


# (mode, distance, structure) of the per-mode timings: the four modes at
# distance 1, the register look-ahead two blocks ahead, the LDS-staged
# look-ahead, and (fp16 only) the four modes of the two-loop structure.
# Each runs on its own plan for the workload (with the same context hint as
# the timed call), as a caller switching the mode would get it.
MODE_RUNS = [(0, 1, 0), (1, 1, 0), (2, 1, 0), (3, 1, 0), (2, 2, 0), (4, 1, 0), (4, 2, 0),
             (0, 1, 1), (1, 1, 1), (2, 1, 1), (3, 1, 1)]
# modes timed again on the timed call's own shape (waves, partitions, order,
# residency): only the look-ahead differs from the timed call
SAME_SHAPE_RUNS = [(0, 1, 0), (1, 1, 0), (3, 1, 0)]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def profile_tag(workload: str, kv_dtype: str, hint: bool = True) -> str:
    return ((workload if kv_dtype == "fp16" else f"{workload}_{kv_dtype}") +
            ("" if hint else "_nohint"))


def _profile_figures(workload: str):
    """key: value pairs of the committed rocprofv3 summary of this workload,
    if it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"pa_decode_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_hash") != kernel_source_hash():
        return None
    return kv


def read_traffic(workload: str, mode_name: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    kv = _profile_figures(workload)
    key = f"hbm_bytes_per_launch_{mode_name}"
    return float(kv[key]) if kv and key in kv else None


# look-ahead evidence per mode in the committed counter summaries (fractions
# or per-instruction cycle counts; rocprof_summary writes them):
#   l2_hit_rate        TCC_HIT / (TCC_HIT + TCC_MISS)
#   issue_stall_share  SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (the stall share of
#                      the measurement plan: waves waiting to issue)
#   stall_cycles_per_inst  4 * SQ_WAIT_INST_ANY / SQ_INSTS
#   cycles_per_inst    4 * SQ_WAVE_CYCLES / SQ_INSTS (CPI of a wave)
#   wait_share         SQ_WAIT_ANY / SQ_WAVE_CYCLES (waiting for anything,
#                      s_waitcnt on loads included)
#   kernel_us          rocprofv3 kernel-trace average duration
LOOKAHEAD_FIGURES = ("l2_hit_rate", "issue_stall_share", "stall_cycles_per_inst",
                     "cycles_per_inst", "wait_share", "kernel_us")


def read_lookahead_counters(workload: str, mode_name: str):
    """The look-ahead evidence of the committed counter summary (same
    current-sources rule as the traffic) with the look-ahead off, as an L2
    touch, as both, and in the timed mode; None if absent."""
    kv = _profile_figures(workload)
    if not kv:
        return None
    out = {"source": f"profiles/pa_decode_{workload}_counters.md"}
    for fig in LOOKAHEAD_FIGURES:
        vals = {m: float(kv[f"{fig}_{m}"]) for m in ("off", "l2", "both", mode_name)
                if f"{fig}_{m}" in kv}
        if vals:
            out[fig] = {m: round(v, 4) for m, v in vals.items()}
    return out if len(out) > 1 else None


def read_kernel_us(workload: str, mode_name: str):
    """rocprofv3's average duration of the decode kernel of this mode, from
    the committed summary of the current kernel sources; None if absent."""
    kv = _profile_figures(workload)
    key = f"kernel_us_{mode_name}"
    return float(kv[key]) if kv and key in kv else None


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed steps before the timed region (and at least 250 ms of them)")
    ap.add_argument("--workload", default="llama2_7b",
                    help="the headline workload (its figures are the line's value)")
    ap.add_argument("--also", default="llama3_8b",
                    help="comma-separated further workloads measured the same way and "
                         "reported under `targets` ('' for none)")
    ap.add_argument("--prefetch", type=int, default=-1, help="-1 = library default")
    ap.add_argument("--kv-layout", choices=("separate", "adjacent"), default="adjacent",
                    help="separate K and V pools (vLLM's layout), or one pool with each "
                         "(block, head)'s K and V slices side by side")
    ap.add_argument("--kv-dtype", choices=("fp16", "fp8"), default="fp16",
                    help="KV cache element type (fp8 = OCP E4M3 with per-tensor scales)")
    ap.add_argument("--prefetch-distance", type=int, default=0,
                    help="L2-touch distance k in wave iterations (modes 1, 3); 0 = 1")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall-time budget of the oracle baseline (repeated full steps)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context-hint", action="store_true",
                    help="plan without the shortest context as min_context_hint")
    ap.add_argument("--profile", action="store_true",
                    help="short run for rocprofv3: every prefetch mode, no CPU leg")
    ap.add_argument("--timeline", action="store_true",
                    help="per-work-group timeline of the headline workload's timed plan "
                         "(debug kernel variant): one JSON line of per-XCD and per-CU "
                         "finish times")
    ap.add_argument("--sweep", action="store_true",
                    help="batch x context sweep of one workload's head shape: one JSON "
                         "line per point (look-ahead off vs on, sampled parity)")
    ap.add_argument("--sweep-batches", default="8,16,32,64,128,256")
    ap.add_argument("--sweep-contexts", default="1024,2048,4096,8192,16384,32768")
    ap.add_argument("--sweep-max-gb", type=float, default=16.0,
                    help="skip points whose K+V pool exceeds this many GB")
    return ap.parse_args()


# sweep counter pass: modes off, register look-ahead, L2 touch; launches each
SWEEP_PROFILE_MODES = [0, 2, 1]
SWEEP_PROFILE_LAUNCHES = 2


def calibrate_counters(torch, ops):
    """Kernels of known size for scaling the HBM byte counters: a 1 GiB
    streaming read (reads 2^30 B) and a 1 GiB fp16 elementwise copy (reads
    and writes 2^30 B each), three times each."""
    src = torch.empty(1 << 29, dtype=torch.float16, device="cuda").normal_()
    dst = torch.empty_like(src)
    for _ in range(3):
        ops.stream_read(src)
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": {"stream_read_bytes": 1 << 30, "copy_read_bytes": 1 << 30,
                                      "copy_write_bytes": 1 << 30}}), flush=True)


def run_sweep(args):
    """Batch x context sweep (the review's section 5.4 figure, at kernel level):
    for each point, µs/step and KV GB/s with the look-ahead off and with the
    default look-ahead, and the oracle on two sampled sequences."""
    import numpy as np
    import torch

    from oracle import oracle as orc
    from paged_kv_cache_226_amd import accounting as acc
    from paged_kv_cache_226_amd import inputs as gen
    from paged_kv_cache_226_amd import ops

    w = gen.WORKLOADS[args.workload]
    batches = [int(v) for v in args.sweep_batches.split(",")]
    contexts = [int(v) for v in args.sweep_contexts.split(",")]
    stream = torch.cuda.current_stream()
    steps = min(args.steps, 100)
    for bi, B in enumerate(batches):
        for ci, ctx in enumerate(contexts):
            kv_bytes = acc.step_kv_bytes(w.num_kv_heads, 128, [ctx] * B)
            if kv_bytes > args.sweep_max_gb * 1e9:
                continue
            d = gen.make_case_device(B, w.num_q_heads, w.num_kv_heads, ctx,
                                     seed=10_000 + 100 * bi + ci)
            out = torch.empty_like(d["q"])
            # every context of a sweep point is `ctx`: the caller's hint
            hint = 0 if args.no_context_hint else ctx
            plan = ops.plan(d["q"], d["k_cache"], d["block_tables"], min_context_hint=hint)
            if args.profile:
                # for a counter pass: a fixed number of launches per mode, in
                # this order, so the dispatches can be mapped back to points
                for pf in SWEEP_PROFILE_MODES:
                    for _ in range(SWEEP_PROFILE_LAUNCHES):
                        ops.paged_attn_decode(d["q"], d["k_cache"], d["v_cache"],
                                              d["block_tables"], d["context_lens"], d["scale"],
                                              out, prefetch=pf, min_context_hint=hint)
                torch.cuda.synchronize()
                print(json.dumps({"sweep_profile": args.workload, "batch": B, "context": ctx,
                                  "kv_bytes": kv_bytes, "partitions": plan["num_partitions"],
                                  "modes": SWEEP_PROFILE_MODES,
                                  "launches_per_mode": SWEEP_PROFILE_LAUNCHES}), flush=True)
                del d, out
                torch.cuda.empty_cache()
                continue
            times = {}
            for pf in (0, plan["prefetch"]):
                f = ops.prepare_decode(d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                       d["context_lens"], d["scale"], out, prefetch=pf,
                                       min_context_hint=hint)
                # warm up for at least 50 ms: the GPU runs slower for a while
                # after the input generation or an idle gap
                t_end = time.perf_counter() + 0.05
                while True:
                    for _ in range(10):
                        f()
                    torch.cuda.synchronize()
                    if time.perf_counter() >= t_end:
                        break
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for _ in range(steps):
                    f()
                b.record(stream)
                torch.cuda.synchronize()
                times[pf] = a.elapsed_time(b) * 1e3 / steps
            seqs = [0, B - 1]
            x = gen.host_subset(d, seqs)
            rows = np.array([[i, h] for i in range(len(seqs)) for h in range(w.num_q_heads)])
            ref = orc.paged_attention_rows_f64(x.q, x.k_cache, x.v_cache, x.block_tables,
                                               x.context_lens, x.scale, rows)
            got = out[seqs].float().cpu().numpy().reshape(-1, 128).astype(np.float64)
            diff = np.abs(got - ref)
            on = times[plan["prefetch"]]
            print(json.dumps({
                "sweep": args.workload, "batch": B, "context": ctx, "kv_bytes": kv_bytes,
                "partitions": plan["num_partitions"], "balanced": plan["balanced"],
                "waves_per_wg": plan["waves_per_wg"], "resident_wgs": plan["resident_wgs"],
                "min_context_hint": hint,
                "us_off": round(times[0], 2), "us_on": round(on, 2),
                "GBps_on": round(kv_bytes / on / 1e3, 1),
                "pct_hbm_peak_on": round(100 * kv_bytes / on / 1e3 / acc.HBM_PEAK_GBPS, 2),
                "speedup_on_vs_off": round(times[0] / on, 4),
                "parity_abs": float(diff.max()),
                "parity_rel": float((diff / np.maximum(np.abs(ref), 1e-3)).max())}), flush=True)
            del d, out
            torch.cuda.empty_cache()
    if args.profile:
        calibrate_counters(torch, ops)


def run_timeline(args):
    """The timed plan of --workload once more with the debug timeline (the
    checked kernel variant): when each work-group started and ended, on which
    CU and XCD.  Prints one JSON line: the launch span, the kernel's own
    event-timed duration, and per XCD the work-groups, the mean work-group
    duration and when its last work-group ended."""
    import numpy as np
    import torch
    from paged_kv_cache_226_amd import accounting as acc
    from paged_kv_cache_226_amd import inputs as gen
    from paged_kv_cache_226_amd import ops

    w = gen.WORKLOADS[args.workload]
    x = gen.make_inputs(w)
    fp8 = args.kv_dtype == "fp8"
    d = {k: torch.from_numpy(getattr(x, k)).cuda() for k in ("q", "block_tables", "context_lens")}
    if fp8:
        x8 = gen.to_fp8(x)
        d["k_cache"] = torch.from_numpy(gen.pack_k_fp8(x8.k8)).cuda()
        d["v_cache"] = torch.from_numpy(x8.v8).cuda()
    else:
        d["k_cache"] = torch.from_numpy(gen.pack_k(x.k_cache)).cuda()
        d["v_cache"] = torch.from_numpy(x.v_cache).cuda()
    d["k_cache"], d["v_cache"] = gen.side_by_side(d["k_cache"], d["v_cache"])
    hint = 0 if args.no_context_hint else max(int(x.context_lens.min()), 0)
    kw = dict(prefetch=args.prefetch, prefetch_distance=args.prefetch_distance,
              min_context_hint=hint)
    plan = ops.plan(d["q"], d["k_cache"], d["block_tables"], **kw)
    tl = torch.zeros(plan["workgroups"], 4, dtype=torch.int64, device="cuda")
    out = torch.empty_like(d["q"])
    extra = (x8.k_scale, x8.v_scale) if fp8 else ()
    prep = ops.prepare_decode_fp8 if fp8 else ops.prepare_decode
    plain = prep(d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["context_lens"],
                 x.scale, *extra, out, **kw)
    traced = prep(d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["context_lens"],
                  x.scale, *extra, out, debug_timeline=tl, **kw)
    stream = torch.cuda.current_stream()

    def event_us(f, n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            f()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / n

    t_end = time.perf_counter() + 0.3  # out of idle first
    while time.perf_counter() < t_end:
        event_us(plain, 20)
    plain_us = event_us(plain, 50)
    traced_us = event_us(traced, 20)
    spans = []
    keep = None
    for _ in range(5):  # the run whose span is the median is reported
        traced()
        torch.cuda.synchronize()
        t = tl.cpu().numpy().copy()
        spans.append(((t[:, 1].max() - t[:, 0].min()) / 100.0, t))
    spans.sort(key=lambda r: r[0])
    span_us, t = spans[len(spans) // 2]
    t0 = t[:, 0].min()
    start = (t[:, 0] - t0) / 100.0
    end = (t[:, 1] - t0) / 100.0
    hw, xcc = t[:, 2].astype(np.int64), (t[:, 3].astype(np.int64) & 0xF)
    cu = [(int(a), (int(h) >> 13) & 7, (int(h) >> 12) & 1, (int(h) >> 8) & 0xF)
          for a, h in zip(xcc, hw)]
    last = {}
    for k, e in zip(cu, end):
        last[k] = max(last.get(k, 0.0), float(e))
    cu_ends = np.array(sorted(last.values()))
    kv_bytes = acc.step_kv_bytes(w.num_kv_heads, 128, x.context_lens, elem_bytes=1 if fp8 else 2)
    wg = np.arange(len(xcc))
    per_xcd = []
    for xi in sorted(set(xcc.tolist())):
        m = xcc == xi
        per_xcd.append({"xcd": int(xi), "workgroups": int(m.sum()),
                        "mean_wg_us": round(float((end[m] - start[m]).mean()), 2),
                        "last_end_us": round(float(end[m].max()), 2),
                        "wg_index_mod_8": sorted(set((wg[m] % 8).tolist()))})
    busy_at = lambda f: float((cu_ends >= f * span_us).mean())
    print(json.dumps({
        "timeline": args.workload, "kv_dtype": args.kv_dtype, "min_context_hint": hint,
        "waves_per_wg": plan["waves_per_wg"], "resident_wgs": plan["resident_wgs"],
        "workgroups": plan["workgroups"], "cus_seen": len(last),
        "kernel_us_plain": round(plain_us, 2), "kernel_us_traced": round(traced_us, 2),
        "span_us": round(float(span_us), 2), "kv_bytes": kv_bytes,
        "cu_last_end_us": {"min": round(float(cu_ends.min()), 2),
                           "median": round(float(np.median(cu_ends)), 2),
                           "max": round(float(cu_ends.max()), 2)},
        "cus_busy_at_80_90_95_pct_of_span": [round(busy_at(f), 3) for f in (0.8, 0.9, 0.95)],
        "per_xcd": per_xcd}), flush=True)


def mode_name_of(nat, pf: int, dist: int, structure: int = 0) -> str:
    """Name of a (mode, distance, structure) run, as in the profiles."""
    ring = pf in (nat.PREFETCH_REG, nat.PREFETCH_LDS)
    return (("two_loop_" if structure else "") + nat.PREFETCH_NAMES[pf] +
            ("2" if ring and dist == 2 else ""))


def parity_of(got_f16, ref_f64):
    """abs = max |g - r|, rel = max |g - r| / max(|r|, 1e-3) over every element."""
    import numpy as np
    diff = np.abs(got_f16.astype(np.float64) - ref_f64)
    return {"abs": float(diff.max()),
            "rel": float((diff / np.maximum(np.abs(ref_f64), 1e-3)).max())}


def measure_workload(args, name, env, cpu_leg):
    """Time one workload's decode step and check the timed call's output
    against the fp64 oracle.  Returns (block for the JSON line, extras)."""
    import numpy as np
    torch, ops, nat, acc, gen = env["torch"], env["ops"], env["nat"], env["acc"], env["gen"]
    dev, stream = env["dev"], env["stream"]
    w = gen.WORKLOADS[name]
    t0 = time.time()
    x = gen.make_inputs(w)
    print(f"[bench] generated {name} in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    fp8 = args.kv_dtype == "fp8"
    d = {k: torch.from_numpy(getattr(x, k)).to(dev) for k in ("q", "block_tables", "context_lens")}
    x8 = None
    if fp8:
        x8 = gen.to_fp8(x)
        d["k_cache"] = torch.from_numpy(gen.pack_k_fp8(x8.k8)).to(dev)
        d["v_cache"] = torch.from_numpy(x8.v8).to(dev)
    else:
        d["k_cache"] = torch.from_numpy(gen.pack_k(x.k_cache)).to(dev)
        d["v_cache"] = torch.from_numpy(x.v_cache).to(dev)
    if args.kv_layout == "adjacent":
        # one pool [block][head][K slice | V slice]; K and V are strided views
        d["k_cache"], d["v_cache"] = gen.side_by_side(d["k_cache"], d["v_cache"])
    Hkv = x.k_cache.shape[1]
    kv_bytes = acc.step_kv_bytes(Hkv, 128, x.context_lens, elem_bytes=1 if fp8 else 2)
    # the caller knows its context lengths: the shortest one is the hint that
    # lets the plan take the streaming shape when every context fills the
    # block table (it changes no result)
    hint = 0 if args.no_context_hint else max(int(x.context_lens.min()), 0)
    plan = ops.plan(d["q"], d["k_cache"], d["block_tables"], prefetch=args.prefetch,
                    prefetch_distance=args.prefetch_distance, min_context_hint=hint)
    if plan["even_split"]:
        shape_kw = dict(even_split=nat.EVEN_SPLIT_ON, waves_per_wg=plan["waves_per_wg"],
                        max_resident_wgs=plan["resident_wgs"])
    else:
        shape_kw = dict(waves_per_wg=plan["waves_per_wg"], seq_order=plan["seq_order"],
                        max_resident_wgs=plan["resident_wgs"], even_split=nat.EVEN_SPLIT_OFF,
                        partition_blocks=0 if plan["balanced"] else plan["partition_blocks"])

    # One prepared call per configuration, each with its own output tensor
    # and its own workspace (sized for its own plan): a step is then one C
    # call into the library, as for a C caller, and every configuration's
    # output stays readable after the timings.
    calls, outs = {}, {}

    plans = {}

    def step(key):
        # key: (mode, distance, structure, on the timed call's shape?)
        if key not in calls:
            pf, dist, structure, same = key
            outs[key] = torch.empty_like(d["q"])
            kw = dict(prefetch=pf, prefetch_distance=dist, min_context_hint=hint)
            if same:
                kw.update(shape_kw)
            if structure:
                kw["structure"] = structure
            plans[key] = ops.plan(d["q"], d["k_cache"], d["block_tables"], **kw)
            if fp8:
                calls[key] = ops.prepare_decode_fp8(
                    d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["context_lens"],
                    x.scale, x8.k_scale, x8.v_scale, outs[key], **kw)
            else:
                calls[key] = ops.prepare_decode(
                    d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["context_lens"],
                    x.scale, outs[key], **kw)
        calls[key]()

    def timed(key, steps, warmup, min_warm_s=0.0):
        # Warm-up: `warmup` steps, and at least `min_warm_s` seconds of them.
        # Coming out of idle (e.g. after the host built the inputs) the first
        # tens of milliseconds of GPU work run measurably slower.
        t_end = time.perf_counter() + min_warm_s
        done = 0
        while done < warmup or time.perf_counter() < t_end:
            for _ in range(max(1, min(warmup - done, 50)) if done < warmup else 50):
                step(key)
                done += 1
            torch.cuda.synchronize()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            step(key)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / steps  # µs per step

    def per_launch(key, steps):
        """Average single-launch duration: an event pair around each call."""
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for a, b in evs:
            a.record(stream)
            step(key)
            b.record(stream)
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
        pick = lambda f: ts[min(len(ts) - 1, int(f * len(ts)))]
        return sum(ts) / len(ts), ts[len(ts) // 2], pick(0.1), pick(0.9)

    mode = plan["prefetch"]
    dist = plan["prefetch_distance"]  # the library's default unless given
    mode_label = mode_name_of(nat, mode, dist)
    timed_key = (mode, args.prefetch_distance, 0, False)

    if args.profile:
        # Coming out of idle (the host has just built the inputs) the GPU
        # runs slower for a while; the profilers average every dispatch of a
        # kernel, so the first mode's would carry that.  Warm up on a kernel
        # the summaries do not read (a torch sum) for 0.3 s first.
        warm = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        t_end = time.perf_counter() + 0.3
        while time.perf_counter() < t_end:
            for _ in range(20):
                warm.sum()
            torch.cuda.synchronize()
        del warm
        for pf, dist_r, structure in MODE_RUNS:
            if not (fp8 and structure):
                timed((pf, dist_r, structure, False), args.steps, args.warmup)
        return None, None

    def shape_of_plan(p):
        return {k: p[k] for k in ("waves_per_wg", "partition_blocks", "num_partitions",
                                  "seq_order", "resident_wgs", "balanced", "even_split",
                                  "workgroups")}

    us = timed(timed_key, args.steps, args.warmup, min_warm_s=0.25)
    launch_avg, launch_med, launch_p10, launch_p90 = per_launch(timed_key, args.steps)
    modes = {}
    for pf, dist_r, structure in MODE_RUNS:
        if fp8 and structure:
            continue
        key = (pf, dist_r, structure, False)
        u = timed(key, max(20, args.steps // 4), 5)
        p = plans[key]
        modes[mode_name_of(nat, pf, dist_r, structure)] = {
            "us_per_step": round(u, 2), "GBps": round(kv_bytes / u / 1e3, 1),
            "waves_per_wg": p["waves_per_wg"], "resident_wgs": p["resident_wgs"],
            "num_partitions": p["num_partitions"]}
    same_shape = {}
    for pf, dist_r, structure in SAME_SHAPE_RUNS:
        key = (pf, dist_r, structure, True)
        u = timed(key, max(20, args.steps // 4), 5)
        same_shape[mode_name_of(nat, pf, dist_r, structure)] = {
            "us_per_step": round(u, 2), "GBps": round(kv_bytes / u / 1e3, 1)}

    # the streaming read over exactly this step's KV bytes: the ramp-up and
    # drain of a launch weigh more on a shorter read than on the 4 GiB one
    buf = env["stream_buf"]
    n_same = min(kv_bytes, buf.numel()) // 16 * 16
    sink = ops.stream_read(buf[:n_same])
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(10):
        ops.stream_read(buf[:n_same], sink)
    b.record(stream)
    torch.cuda.synchronize()
    stream_same_gbps = n_same / (a.elapsed_time(b) * 1e3 / 10) / 1e3

    # The decode kernel is the dominant kernel.  With one partition it is the
    # only kernel of a step, and its average duration is the timed region over
    # the steps; otherwise the step also holds the reduce kernel and the
    # figure covers both.
    tag = profile_tag(name, args.kv_dtype, not args.no_context_hint)
    decode_only = plan["num_partitions"] == 1
    achieved = kv_bytes / us / 1e3
    kernel_us_rocprof = read_kernel_us(tag, mode_label)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": acc.HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / acc.HBM_PEAK_GBPS, 4),
                "traffic": read_traffic(tag, mode_label),
                "kernel": "pa_decode_kernel" + ("" if decode_only else " + pa_reduce_kernel"),
                "step_us_avg": round(us, 2),
                "kernel_us_rocprof": kernel_us_rocprof,
                "kernel_us_rocprof_source": (f"profiles/pa_decode_{tag}_kernel_trace.md"
                                             if kernel_us_rocprof is not None else None),
                "event_pair_us_avg": round(launch_avg, 2),
                "event_pair_us_median": round(launch_med, 2),
                "event_pair_us_p10": round(launch_p10, 2),
                "event_pair_us_p90": round(launch_p90, 2)}

    off_us = modes["off"]["us_per_step"]
    block = {
        "workload": name,
        "config": {"workload": name, "kv_dtype": "e4m3" if fp8 else "f16",
                   "kv_layout": args.kv_layout,
                   "batch": w.num_seqs, "q_heads": w.num_q_heads,
                   "kv_heads": w.num_kv_heads, "head_dim": 128, "block_size": 16,
                   "context_sum": int(np.maximum(x.context_lens, 0).sum()),
                   "context_min": int(x.context_lens.min()),
                   "context_max": int(x.context_lens.max()),
                   "prefetch": mode_label, "prefetch_distance": dist,
                   "min_context_hint": hint, "resident_wgs": plan["resident_wgs"],
                   "waves_per_wg": plan["waves_per_wg"],
                   "partition_blocks": plan["partition_blocks"],
                   "num_partitions": plan["num_partitions"],
                   "even_split": plan["even_split"],
                   "seq_order": nat.ORDER_NAMES.get(plan["seq_order"], plan["seq_order"]),
                   "parallelism": "single GPU"},
        "us_per_step": round(us, 2),
        "GBps": round(achieved, 1),
        "pct_hbm_peak": round(100 * achieved / acc.HBM_PEAK_GBPS, 2),
        "kv_bytes_per_step": kv_bytes,
        "other_bytes_per_step": acc.step_other_bytes(w.num_seqs, w.num_q_heads, 128,
                                                     x.context_lens),
        "flops_per_step": acc.step_flops(w.num_q_heads, 128, x.context_lens),
        "roofline": roofline,
        "lookahead": {"off_us_per_step": off_us, "timed_mode": mode_label,
                      "timed_us_per_step": round(us, 2),
                      "speedup_timed_vs_off": round(off_us / us, 4),
                      "off_same_shape_us_per_step": same_shape["off"]["us_per_step"],
                      "speedup_timed_vs_off_same_shape":
                          round(same_shape["off"]["us_per_step"] / us, 4)},
        "prefetch_modes": modes,
        "prefetch_modes_on_the_timed_shape": same_shape,
        "stream_read_same_size_GBps": round(stream_same_gbps, 1),
        "pct_of_same_size_stream": round(100 * achieved / stream_same_gbps, 1),
        "lookahead_counters": read_lookahead_counters(tag, mode_label),
        "inputs_sha256": {k: v[:16] for k, v in gen.digests(x).items()},
    }

    # Parity of the timed call's own output (and of every other
    # configuration's) against the fp64 oracle on the same host inputs.
    from oracle import oracle as orc

    def oracle_step():
        if fp8:
            return orc.paged_attention_fp8_f64(x8.q, x8.k8, x8.v8, x8.block_tables,
                                               x8.context_lens, x8.scale, x8.k_scale,
                                               x8.v_scale)
        return orc.paged_attention_f64(x.q, x.k_cache, x.v_cache, x.block_tables,
                                       x.context_lens, x.scale)

    runs = []
    deadline = time.time() + (args.cpu_seconds if cpu_leg else 0.0)
    while True:
        t1 = time.perf_counter()
        ref = oracle_step()
        runs.append(time.perf_counter() - t1)
        if time.time() > deadline or len(runs) >= 200:
            break
    torch.cuda.synchronize()
    got = outs[timed_key].cpu().numpy()
    par = parity_of(got, ref)
    par.update({"rows_checked": int(w.num_seqs * w.num_q_heads), "elements_checked": int(got.size),
                "output_of": f"the timed call ({mode_label})", "abs_tol": 2e-3, "rel_tol": 1e-2,
                "pass": par["abs"] <= 2e-3 and par["rel"] <= 1e-2})
    # every run against the oracle; the runs on the timed call's own shape
    # (same waves, partitions, order) must also give its bits
    bitwise = {}
    timed_shape = shape_of_plan(plans[timed_key])
    for key, o in outs.items():
        if key == timed_key:
            continue
        nm = mode_name_of(nat, *key[:3])
        gk = o.cpu().numpy()
        pk = parity_of(gk, ref)
        table = same_shape if key[3] else modes
        if nm in table:
            table[nm]["parity_abs"] = pk["abs"]
            table[nm]["parity_rel"] = pk["rel"]
        if key[2] == 0 and shape_of_plan(plans[key]) == timed_shape:
            tag_ = nm + ("@timed_shape" if key[3] else "")
            bitwise[tag_] = bool(np.array_equal(gk.view(np.uint16), got.view(np.uint16)))
    par["bitwise_equal_to_timed"] = bitwise
    block["parity"] = par
    t_cpu = sorted(runs)[len(runs) // 2]
    block["oracle_wall_s"] = round(t_cpu, 3)
    return block, {"t_cpu": t_cpu, "runs": runs, "kv_bytes": kv_bytes, "us": us}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this bench runs on exactly one GPU; the decode kernel "
                                   "is a single-GPU path (no collectives). Use --gpus 1."}))
        sys.exit(2)

    import torch

    from paged_kv_cache_226_amd import accounting as acc
    from paged_kv_cache_226_amd import inputs as gen
    from paged_kv_cache_226_amd import ops
    from paged_kv_cache_226_amd import _native as nat

    nat.lib()  # fail loudly if the HIP library is not built
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(3)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.sweep:
        run_sweep(args)
        return
    if args.timeline:
        run_timeline(args)
        return
    stream = torch.cuda.current_stream()
    env = dict(torch=torch, ops=ops, nat=nat, acc=acc, gen=gen, dev=dev, stream=stream)

    if args.profile:
        measure_workload(args, args.workload, env, cpu_leg=False)
        calibrate_counters(torch, ops)
        print(json.dumps({"profile_run": args.workload, "kv_dtype": args.kv_dtype,
                          "steps": args.steps}), flush=True)
        return

    # streaming-read ceiling over a buffer larger than every cache
    buf = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
    sink = ops.stream_read(buf)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(10):
        ops.stream_read(buf, sink)
    b.record(stream)
    torch.cuda.synchronize()
    stream_gbps = (4 << 30) / (a.elapsed_time(b) * 1e3 / 10) / 1e3
    env["stream_buf"] = buf

    cpu_leg = not args.no_cpu_baseline
    head, hx = measure_workload(args, args.workload, env, cpu_leg=cpu_leg)
    targets = {args.workload: head}
    for name in [n for n in args.also.split(",") if n and n != args.workload]:
        torch.cuda.empty_cache()
        blk, _ = measure_workload(args, name, env, cpu_leg=False)
        targets[name] = blk
    del buf, env["stream_buf"]

    us = hx["us"]
    result = {
        "metric": METRIC,
        "value": head["GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 5),
        "us_per_step": head["us_per_step"],
        "pct_hbm_peak": head["pct_hbm_peak"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "accumulate": "f32",
        "data": "synthetic",
        "config": head["config"],
        "kv_bytes_per_step": head["kv_bytes_per_step"],
        "other_bytes_per_step": head["other_bytes_per_step"],
        "flops_per_step": head["flops_per_step"],
        "prefetch_modes": head["prefetch_modes"],
        "prefetch_modes_on_the_timed_shape": head["prefetch_modes_on_the_timed_shape"],
        "stream_read_ceiling_GBps": round(stream_gbps, 1),
        "pct_of_stream_ceiling": round(100 * head["GBps"] / stream_gbps, 1),
        "stream_read_same_size_GBps": head["stream_read_same_size_GBps"],
        "pct_of_same_size_stream": head["pct_of_same_size_stream"],
        "roofline": head["roofline"],
        "lookahead": head["lookahead"],
        "lookahead_counters": head["lookahead_counters"],
        "parity": head["parity"],
        "kernel_source_hash": kernel_source_hash(),
        "inputs_sha256": head["inputs_sha256"],
        "targets": {n: {k: v for k, v in blk.items() if k not in ("inputs_sha256",)}
                    for n, blk in targets.items()},
    }
    if cpu_leg:
        from oracle import oracle as orc
        runs, t_cpu = hx["runs"], hx["t_cpu"]
        w = gen.WORKLOADS[args.workload]
        result["cpu_baseline"] = {
            "value": round(hx["kv_bytes"] / t_cpu / 1e9, 3), "unit": "GB/s",
            "us_per_step": round(t_cpu * 1e6, 1), "cores": orc.max_threads(), "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "sample": f"the whole {args.workload} step ({args.kv_dtype} KV, all "
                      f"{w.num_seqs * w.num_q_heads} (sequence, head) rows), fp64, median of "
                      f"{len(runs)} run(s) over {sum(runs):.1f} s of wall time"}
        result["gpu_speedup_vs_cpu_oracle"] = round(t_cpu * 1e6 / us, 1)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
