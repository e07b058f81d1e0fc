"""Kernel-name matching of the rocprofv3 summariser (CPU)."""
from paged_kv_cache_226_amd import rocprof_summary as rs


def test_decode_mode_selects_the_cache_type_and_skips_debug_instances():
    names = {n: f"void pa::pa_decode_kernel<{n[0]}, {n[1]}, {n[2]}>(pa::DecodeArgs)"
             for n in [(m, d, k) for m in range(4) for d in ("false", "true")
                       for k in ("false", "true")]}
    try:
        for kv8 in (False, True):
            rs.KV8 = kv8
            for (m, d, k), name in names.items():
                want = m if d == "false" and (k == "true") == kv8 else None
                assert rs.decode_mode(name) == want, (name, kv8)
        assert rs.decode_mode("void pa::pa_reduce_kernel(pa::DecodeArgs)") is None
        rs.KV8 = False
        for m in range(4):
            assert rs.decode_mode(f"void pa::pa_decode_kernel<{m}, false, false, false>(x)") == m
            assert rs.decode_mode(f"void pa::pa_decode_kernel<{m}, false, false, true>(x)") \
                == 10 + m
            assert rs.MODE_NAMES[10 + m].startswith("two_loop_")
            # with all five template arguments spelled out: fused, two-loop,
            # even split (its look-ahead mode), and the E4M3 / debug ones skipped
            five = "void pa::pa_decode_kernel<{}, {}, {}, {}, {}>(pa::DecodeArgs)"
            assert rs.decode_mode(five.format(m, "false", "false", "false", "false")) == m
            assert rs.decode_mode(five.format(m, "false", "false", "true", "false")) == 10 + m
            assert rs.decode_mode(five.format(m, "false", "false", "false", "true")) == m
            assert rs.decode_mode(five.format(m, "true", "false", "false", "true")) is None
            assert rs.decode_mode(five.format(m, "false", "true", "false", "true")) is None
    finally:
        rs.KV8 = False


def test_sweep_fetch_maps_dispatches_to_points(tmp_path):
    import json

    pts = [{"sweep_profile": "w", "batch": 8, "context": 1024, "kv_bytes": 1 << 20,
            "partitions": 2, "modes": [0, 2, 1], "launches_per_mode": 2},
           {"sweep_profile": "w", "batch": 16, "context": 1024, "kv_bytes": 1 << 21,
            "partitions": 1, "modes": [0, 2, 1], "launches_per_mode": 2}]
    (tmp_path / "p.jsonl").write_text("".join(json.dumps(p) + "\n" for p in pts))
    # FETCH_SIZE in KiB at half the true bytes (scale 2), one row per dispatch
    rows, did = [], 0

    def add(name, kib):
        nonlocal did
        did += 1
        rows.append(f'{did},{did},"Agent 1",1,1,1,1,1,"{name}",256,0,0,8,0,8,"FETCH_SIZE",{kib},0,0')

    dec = "void pa::pa_decode_kernel<{}, false, false, false>(pa::DecodeArgs)"
    for p, extra in zip(pts, (0.0, 0.25)):
        add("void at::native::normal_kernel(x)", 99.0)
        for m in p["modes"]:
            for _ in range(2):
                add(dec.format(m), p["kv_bytes"] / 1024 / 2 * (1 + (extra if m == 1 else 0)))
            add("void pa::pa_reduce_kernel(pa::DecodeArgs)", 7.0)
    add("pa::stream_read_kernel(unsigned int __vector(4) const*, long, unsigned", (1 << 20) / 2)
    head = ('"Correlation_Id","Dispatch_Id","Agent_Id","Queue_Id","Process_Id","Thread_Id",'
            '"Grid_Size","Kernel_Id","Kernel_Name","Workgroup_Size","LDS_Block_Size",'
            '"Scratch_Size","VGPR_Count","Accum_VGPR_Count","SGPR_Count","Counter_Name",'
            '"Counter_Value","Start_Timestamp","End_Timestamp"')
    d = tmp_path / "fetch"
    d.mkdir()
    (d / "x_counter_collection.csv").write_text(head + "\n" + "\n".join(rows) + "\n")
    rs.KV8 = False
    path = rs.sweep_fetch(str(tmp_path / "p.jsonl"), str(d), "w", str(tmp_path), "cmd")
    table = [l for l in open(path) if l.startswith("| 8 ") or l.startswith("| 16 ")]
    assert table[0].split("|")[5:8] == [" 1.0000 ", " 1.0000 ", " 1.0000 "]
    assert table[1].split("|")[5:8] == [" 1.0000 ", " 1.0000 ", " 1.2500 "]


def test_request_path_table_derives_little_law_figures(tmp_path):
    """Per-mode means of summed counters and the derived figures: mean latency
    = latency sum / requests, in flight = latency sum / cycles (per XCD clock,
    over 256 CUs for per-CU figures)."""
    head = ('"Correlation_Id","Dispatch_Id","Agent_Id","Queue_Id","Process_Id","Thread_Id",'
            '"Grid_Size","Kernel_Id","Kernel_Name","Workgroup_Size","LDS_Block_Size",'
            '"Scratch_Size","VGPR_Count","Accum_VGPR_Count","SGPR_Count","Counter_Name",'
            '"Counter_Value","Start_Timestamp","End_Timestamp"')
    dec = "void pa::pa_decode_kernel<{}, false, false, false>(pa::DecodeArgs)"
    rows, did = [], 0
    for m, scale in ((0, 1.0), (1, 2.0)):
        for _ in range(2):  # two launches per mode, same values
            did += 1
            for c, v in (("GRBM_GUI_ACTIVE", 8000.0), ("TCP_TCC_READ_REQ_sum", 100.0 * scale),
                         ("TCP_TCC_READ_REQ_LATENCY_sum", 256000.0 * scale),
                         ("TCC_EA0_RDREQ_sum", 50.0), ("TCC_EA0_RDREQ_LEVEL_sum", 5000.0)):
                rows.append(f'{did},{did},"A",1,1,1,1,1,"{dec.format(m)}",256,0,0,8,0,8,'
                            f'"{c}",{v},0,0')
    d = tmp_path / "rq"
    d.mkdir()
    (d / "x_counter_collection.csv").write_text(head + "\n" + "\n".join(rows) + "\n")
    rs.KV8 = False
    path = rs.request_path_table([str(d)], "w", ["h"], str(tmp_path), {0: 10.0, 1: 12.5})
    lines = {l.split("|")[1].strip(): [c.strip() for c in l.split("|")[2:-1]]
             for l in open(path) if l.startswith("| ")}
    assert lines["kernel us"] == ["10.00", "12.50"]
    assert lines["TCP->TCC read requests"] == ["100", "200"]
    assert lines["TCP->TCC mean read latency (cycles)"] == ["2560", "2560"]
    # 256000 latency-cycles over 1000 cycles per XCD = 256 in flight, 1 per CU
    assert lines["TCP->TCC reads in flight per CU"] == ["1", "2"]
    assert lines["HBM (EA) reads in flight"] == ["5", "5"]
    assert lines["HBM (EA) mean read latency (cycles)"] == ["100", "100"]


def test_sweep_timing_table(tmp_path):
    import json
    pts = [{"sweep": "w", "batch": 8, "context": 1024, "kv_bytes": 8000000, "partitions": 4,
            "us_off": 10.0, "us_on": 8.0, "GBps_on": 1000.0, "pct_hbm_peak_on": 12.5,
            "speedup_on_vs_off": 1.25, "parity_abs": 1e-5, "parity_rel": 2e-4,
            "waves_per_wg": 2, "resident_wgs": 0}]
    (tmp_path / "s.jsonl").write_text("noise\n" + "".join(json.dumps(p) + "\n" for p in pts))
    path = rs.sweep_timing(str(tmp_path / "s.jsonl"), "w", str(tmp_path), "cmd a ;; cmd b")
    text = open(path).read()
    assert "    cmd a\n    cmd b\n" in text
    row = [l for l in text.splitlines() if l.startswith("| 8 ")][0].split("|")
    assert [c.strip() for c in row[4:12]] == ["fixed", "4", "2 / -", "10.00", "8.00", "800",
                                              "1000", "12.5"]


def test_mode_plans_follow_the_library(native_lib):
    """The per-mode plans the summary header lists are the library's, with the
    shortest context as the hint: llama2_7b's register look-ahead on 1-wave
    work-groups capped at 2 per CU, the look-ahead off at 4 per CU."""
    from paged_kv_cache_226_amd import inputs as gen
    plans = rs.mode_plans(gen.WORKLOADS["llama2_7b"], False, 2048)
    assert plans[2] == "1 waves, cap 2, 1 partition(s)"
    assert plans[0] == "1 waves, cap 4, 1 partition(s)"
    assert plans[1].startswith("4 waves, cap -")
    assert 10 in plans and 4 in plans
    assert 10 not in rs.mode_plans(gen.WORKLOADS["llama2_7b"], True, 2048)


def test_timeline_table(tmp_path):
    import json
    r = {"timeline": "w", "kv_dtype": "fp16", "min_context_hint": 0, "waves_per_wg": 4,
         "resident_wgs": 0, "workgroups": 16, "cus_seen": 8, "kernel_us_plain": 10.0,
         "kernel_us_traced": 11.0, "span_us": 10.5, "kv_bytes": 1000000,
         "cu_last_end_us": {"min": 9.0, "median": 10.0, "max": 10.5},
         "cus_busy_at_80_90_95_pct_of_span": [1.0, 0.5, 0.25],
         "per_xcd": [{"xcd": 0, "workgroups": 2, "mean_wg_us": 9.5, "last_end_us": 10.5,
                      "wg_index_mod_8": [0]}]}
    (tmp_path / "t.jsonl").write_text("noise\n" + json.dumps(r) + "\n")
    path = rs.timeline_table(str(tmp_path / "t.jsonl"), "w", "fp16", str(tmp_path), "cmd")
    assert path.endswith("pa_decode_w_nohint_timeline.md")
    text = open(path).read()
    assert "| 0 | 2 | 0 | 9.5 | 10.5 |" in text and "100 % / 50 % / 25 %" in text
    assert "95 GB/s" in text
