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
