"""The C ABI without a GPU: symbols, host-only validation, plans (CPU).

No call here reaches a kernel launch: every decode call is built to fail the
host-side checks first.
"""
import ctypes
import os
import re
import subprocess

import pytest

from paged_kv_cache_226_amd import _native as nat

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "paged_attn.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(paged_attn_\w+)\s*\(", text)))


def test_library_exports_every_declared_function(native_lib):
    names = declared_functions()
    assert len(names) >= 8
    nm = subprocess.run(["nm", "-D", "--defined-only", nat.LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)$", nm, re.M))
    for n in names:
        assert n in exported, n
        assert hasattr(native_lib, n)


def test_version_and_error_strings(native_lib):
    assert native_lib.paged_attn_abi_version() == nat.ABI_VERSION == 8
    assert nat.error_string(0) == "ok"
    for code in range(1, 5):
        assert nat.error_string(code) not in ("ok", "unknown status")
    assert nat.error_string(99) == "unknown status"


def test_a_library_of_another_abi_version_is_refused(native_lib, monkeypatch):
    """A stale build would read the structs with another layout: the binding
    refuses it instead of calling it."""
    monkeypatch.setattr(nat, "_lib", None)
    monkeypatch.setattr(nat, "ABI_VERSION", nat.ABI_VERSION + 1)
    with pytest.raises(nat.NativeLibraryMissing, match="ABI version"):
        nat.lib()


def test_struct_layouts_match_header(native_lib, tmp_path):
    """Every field offset and struct size of the ctypes mirror equals what a C
    compiler makes of include/paged_attn.h."""
    structs = {"pa_shape": nat.PaShape, "pa_options": nat.PaOptions,
               "pa_plan_info": nat.PaPlanInfo, "pa_device_info": nat.PaDeviceInfo}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "paged_attn.h"',
             'int main(void) {']
    for cname, py in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'  printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines.append('  return 0; }')
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)],
                   check=True)
    got = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    for line in filter(None, got):
        cname, field, value = line.split()
        py = structs[cname]
        want = ctypes.sizeof(py) if field == "size" else getattr(py, field).offset
        assert int(value) == want, line
    o = nat.default_options()
    assert o.prefetch == -1 and o.partition_blocks == 0 and o.waves_per_wg == 0
    assert o.prefetch_distance == 0 and o.seq_order == 0 and o.structure == 0
    assert o.workspace is None and o.debug_gather_k is None


FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation


def call(shape, opts=None, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, ctx=FAKE, out=FAKE, scale=0.088):
    return nat.lib().paged_attn_decode(
        ctypes.c_void_p(q), ctypes.c_void_p(k), ctypes.c_void_p(v), ctypes.c_void_p(bt),
        ctypes.c_void_p(ctx), ctypes.c_float(scale), ctypes.c_void_p(out),
        ctypes.byref(shape) if shape is not None else None,
        ctypes.byref(opts) if opts is not None else None, None)


def good_shape(**kw):
    d = dict(num_seqs=2, num_q_heads=8, num_kv_heads=2, max_blocks_per_seq=4096, num_blocks=64)
    d.update(kw)
    return nat.make_shape(**d)


@pytest.mark.parametrize("case,code", [
    (dict(q=0), nat.PA_ERR_INVALID_ARG),
    (dict(out=0), nat.PA_ERR_INVALID_ARG),
    (dict(bt=0), nat.PA_ERR_INVALID_ARG),
    (dict(q=FAKE + 8), nat.PA_ERR_INVALID_ARG),
    (dict(bt=FAKE + 2), nat.PA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), nat.PA_ERR_INVALID_ARG),
    (dict(shape=None), nat.PA_ERR_INVALID_ARG),
    (dict(shape=dict(num_seqs=0)), nat.PA_ERR_INVALID_ARG),
    (dict(shape=dict(num_q_heads=6, num_kv_heads=4)), nat.PA_ERR_INVALID_ARG),
    (dict(shape=dict(num_blocks=0)), nat.PA_ERR_INVALID_ARG),
    (dict(shape=dict(k_head_stride=4104)), nat.PA_ERR_INVALID_ARG),
    (dict(shape=dict(v_block_stride=-16)), nat.PA_ERR_INVALID_ARG),
    (dict(shape=dict(k_head_stride=2048)), nat.PA_ERR_INVALID_ARG),
    (dict(shape=dict(v_head_stride=8192, v_block_stride=8192)), nat.PA_ERR_INVALID_ARG),
    (dict(shape=dict(k_block_stride=1 << 60)), nat.PA_ERR_UNSUPPORTED),
    (dict(shape=dict(head_dim=64)), nat.PA_ERR_UNSUPPORTED),
    (dict(shape=dict(block_size=32)), nat.PA_ERR_UNSUPPORTED),
    (dict(shape=dict(num_q_heads=34, num_kv_heads=2)), nat.PA_ERR_UNSUPPORTED),
    (dict(opts=dict(prefetch=5)), nat.PA_ERR_INVALID_ARG),
    (dict(opts=dict(prefetch=4, prefetch_distance=3)), nat.PA_ERR_UNSUPPORTED),
    (dict(shape=dict(kv_dtype=2)), nat.PA_ERR_INVALID_ARG),
    (dict(shape=dict(kv_dtype=-1)), nat.PA_ERR_INVALID_ARG),
    # an E4M3 shape given to the fp16 entry point
    (dict(shape=dict(kv_dtype=nat.KV_E4M3)), nat.PA_ERR_INVALID_ARG),
    # three fp16 LDS slots per wave for 8 waves: 192 KiB
    (dict(opts=dict(prefetch=4, prefetch_distance=2, waves_per_wg=8)), nat.PA_ERR_UNSUPPORTED),
    (dict(opts=dict(prefetch=4, structure=1)), nat.PA_ERR_UNSUPPORTED),
    (dict(opts=dict(waves_per_wg=3)), nat.PA_ERR_INVALID_ARG),
    (dict(opts=dict(prefetch_distance=64)), nat.PA_ERR_INVALID_ARG),
    (dict(opts=dict(prefetch_distance=-1)), nat.PA_ERR_INVALID_ARG),
    (dict(opts=dict(prefetch=2, prefetch_distance=3)), nat.PA_ERR_UNSUPPORTED),
    (dict(opts=dict(partition_blocks=-1)), nat.PA_ERR_INVALID_ARG),
    (dict(opts=dict(partition_blocks=2048)), nat.PA_ERR_UNSUPPORTED),
    (dict(opts=dict(seq_order=3)), nat.PA_ERR_INVALID_ARG),
    (dict(opts=dict(seq_order=-1)), nat.PA_ERR_INVALID_ARG),
    (dict(opts=dict(structure=2)), nat.PA_ERR_INVALID_ARG),
    (dict(opts=dict(structure=1, prefetch_distance=2)), nat.PA_ERR_UNSUPPORTED),
    (dict(shape=dict(num_seqs=257), opts=dict(seq_order=2)), nat.PA_ERR_UNSUPPORTED),
    # too much LDS: the two-loop scores of 1024 blocks x 16 heads (1 MiB)
    (dict(shape=dict(num_q_heads=32, num_kv_heads=2),
          opts=dict(structure=1, partition_blocks=1024)), nat.PA_ERR_UNSUPPORTED),
    # 4096 blocks per sequence need several partitions: no workspace given
    (dict(), nat.PA_ERR_WORKSPACE),
    (dict(opts=dict(workspace=FAKE, workspace_bytes=16)), nat.PA_ERR_WORKSPACE),
])
def test_validation_codes(native_lib, case, code):
    case = dict(case)
    sh = case.pop("shape", {})
    shape = None if sh is None else good_shape(**sh)
    o = nat.default_options()
    for k2, v2 in case.pop("opts", {}).items():
        setattr(o, k2, v2)
    assert call(shape, o, **case) == code


def test_noalloc_validation_codes(native_lib):
    """paged_attn_decode_noalloc checks its arguments as paged_attn_decode does
    and refuses, before any device call, a plan whose partials exceed its
    scratch array; a caller's workspace is ignored."""
    def noalloc(shape, opts=None, q=FAKE, out=FAKE):
        return native_lib.paged_attn_decode_noalloc(
            ctypes.c_void_p(q), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
            ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), ctypes.c_float(0.088),
            ctypes.c_void_p(out), ctypes.byref(shape) if shape is not None else None,
            ctypes.byref(opts) if opts is not None else None, None)
    m = re.search(r"#define PA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == nat.NOALLOC_SCRATCH_BYTES
    assert noalloc(good_shape(), q=0) == nat.PA_ERR_INVALID_ARG
    assert noalloc(good_shape(), out=FAKE + 8) == nat.PA_ERR_INVALID_ARG
    assert noalloc(None) == nat.PA_ERR_INVALID_ARG
    assert noalloc(good_shape(head_dim=64)) == nat.PA_ERR_UNSUPPORTED
    assert noalloc(good_shape(kv_dtype=nat.KV_E4M3)) == nat.PA_ERR_INVALID_ARG
    # 255 sequences x 16 heads in partitions of 16 blocks of a 1024-block table
    big = good_shape(num_seqs=255, num_q_heads=16, num_kv_heads=1, max_blocks_per_seq=1024)
    o = nat.default_options()
    o.partition_blocks = 16
    need = native_lib.paged_attn_workspace_size(ctypes.byref(big), ctypes.byref(o))
    assert need > nat.NOALLOC_SCRATCH_BYTES
    o.workspace, o.workspace_bytes = FAKE, need  # ignored by this entry point
    assert noalloc(big, o) == nat.PA_ERR_WORKSPACE


def test_plans_of_the_workloads(native_lib):
    from paged_kv_cache_226_amd import inputs as gen
    # (partitions, waves, balanced, even split) of the auto plan without a
    # hint; under the balanced split the partitions are the most one
    # sequence can get
    expect = {"tiny": (1, 8, 0, 0), "llama2_7b": (1, 4, 0, 0), "llama3_8b": (1, 2, 0, 1),
              "qwen25_7b": (1, 2, 0, 1), "qwen25_14b": (1, 2, 0, 1),
              "llama3_8b_tp2": (1, 2, 0, 1), "llama3_8b_tp4": (1, 2, 0, 1),
              "llama3_8b_tp8": (8, 8, 1, 0), "qwen25_14b_tp2": (1, 2, 0, 1),
              "qwen25_14b_tp4": (1, 2, 0, 1), "qwen25_14b_tp8": (1, 2, 0, 1)}
    for name, w in gen.WORKLOADS.items():
        MB = w.max_blocks_per_seq or max(-(-c // 16) for c in w.context_lens)
        nb = w.pool_blocks or 1
        p = nat.plan(nat.make_shape(w.num_seqs, w.num_q_heads, w.num_kv_heads, MB, nb))
        got = (p["num_partitions"], p["waves_per_wg"], p["balanced"], p["even_split"])
        assert got == expect[name], name
        if p["even_split"]:
            # one share per CU, two records of g rows per share and one
            # piece record per (sequence, KV head)
            g = w.num_q_heads // w.num_kv_heads
            assert p["workgroups"] == 256 and p["resident_wgs"] == 1
            assert p["workspace_bytes"] == (2 * 256 * g * 130 + 2 * w.num_seqs * w.num_kv_heads) * 4
            continue
        if p["balanced"]:
            # one grid row per CU and KV head (256 CUs), the smallest size 16
            assert p["workgroups"] == 256 // w.num_kv_heads * w.num_kv_heads
            assert p["partition_blocks"] == 16
            header = -(-w.num_seqs // 4) * 4
        else:
            assert p["num_partitions"] * p["partition_blocks"] >= MB
            assert p["workgroups"] == p["num_partitions"] * w.num_kv_heads * w.num_seqs
            header = 0
        want = 0 if p["num_partitions"] == 1 else \
            (header + w.num_seqs * w.num_q_heads * p["num_partitions"] * 130) * 4
        assert p["workspace_bytes"] == want


def test_explicit_partition_size_and_workspace_size(native_lib):
    sh = good_shape(max_blocks_per_seq=100)
    o = nat.default_options()
    o.partition_blocks = 16
    p = nat.plan(sh, o)
    assert p["partition_blocks"] == 16 and p["num_partitions"] == 7
    assert native_lib.paged_attn_workspace_size(ctypes.byref(sh), ctypes.byref(o)) == 2 * 8 * 7 * 130 * 4
    bad = good_shape(head_dim=64)
    assert native_lib.paged_attn_workspace_size(ctypes.byref(bad), None) == 0


def test_stream_read_sink_is_one_word_per_cu(native_lib):
    assert native_lib.paged_attn_stream_read_sink_bytes(1 << 30) == \
        16 * nat.device_info()["compute_units"]


def test_stream_read_validation(native_lib):
    f = native_lib.paged_attn_stream_read
    assert f(None, 1024, ctypes.c_void_p(FAKE), None) == nat.PA_ERR_INVALID_ARG
    assert f(ctypes.c_void_p(FAKE), 1000, ctypes.c_void_p(FAKE), None) == nat.PA_ERR_INVALID_ARG
    assert f(ctypes.c_void_p(FAKE + 4), 1024, ctypes.c_void_p(FAKE), None) == nat.PA_ERR_INVALID_ARG


@pytest.mark.parametrize("B,Hkv,MB,order,want", [
    (1, 2, 16, 0, 1),      # one sequence: nothing to order
    (2, 2, 16, 0, 1),      # 4 work-groups, all resident at once
    (96, 8, 64, 0, 1),     # 768 4-wave work-groups: 3 per CU on 256 CUs
    (97, 8, 64, 0, 2),     # 776: some wait for a CU, so the longest go first
    (64, 8, 512, 0, 2),    # 512 8-wave work-groups, one per CU at a time
    (256, 8, 512, 0, 2),
    (257, 8, 512, 0, 1),   # more sequences than the in-kernel ranking takes
    (64, 2, 16, 1, 1), (1, 2, 16, 2, 2), (256, 2, 16, 2, 2)])
def test_sequence_order_of_the_plan(native_lib, B, Hkv, MB, order, want):
    o = nat.default_options()
    o.seq_order = order
    o.even_split = nat.EVEN_SPLIT_OFF  # (64 and 256 x 8 x 512 blocks would take it)
    sh = good_shape(num_seqs=B, num_q_heads=4 * Hkv, num_kv_heads=Hkv, max_blocks_per_seq=MB)
    assert nat.plan(sh, o)["seq_order"] == want


@pytest.mark.parametrize("B,Hkv,MB,waves,P,PB", [
    (256, 4, 2048, 4, 2, 1024),   # long contexts, many pairs: 1024-block partitions
    (8, 8, 64, 8, 4, 16),         # 64 pairs, short table: four 16-block partitions, 8 waves
    (8, 8, 128, 8, 4, 32),        # four 32-block partitions
    (4, 32, 1024, 8, 4, 256),     # 128 pairs: capped at 256 blocks
    (2, 1, 4096, 8, 64, 64),      # 2 pairs: 128 partitions of 32 would overload the reduce: 64 blocks
    (2, 1, 1024, 8, 16, 64),      # 64 partitions of 16 wanted: 64-block ones instead
    (1, 1, 10, 8, 1, 10),
    (64, 8, 512, 8, 1, 512),
    (64, 8, 511, 4, 1, 511),      # narrower table: 4 waves
    (96, 8, 512, 4, 1, 512),      # 768 pairs: 4 waves
])
def test_auto_plan_rule(native_lib, B, Hkv, MB, waves, P, PB):
    """The fixed split rule (an explicit sequence order keeps a split plan on
    it; with the auto order, batches of 2..256 sequences take the balanced
    split instead)."""
    o = nat.default_options()
    o.seq_order = nat.ORDER_NATURAL
    p = nat.plan(nat.make_shape(B, Hkv * 4, Hkv, MB, 1000), o)
    assert (p["waves_per_wg"], p["num_partitions"], p["partition_blocks"]) == (waves, P, PB)
    assert p["balanced"] == 0
    auto = nat.plan(nat.make_shape(B, Hkv * 4, Hkv, MB, 1000))
    even = 2 <= B <= 256 and 160 <= MB <= 1024 and 2 * B * Hkv >= 256
    assert auto["even_split"] == even
    if even:
        assert (auto["workgroups"], auto["num_partitions"]) == (256, 1)
        return
    assert auto["balanced"] == (1 if P > 1 and 2 <= B <= 256 and B * Hkv < 256 else 0)
    if not auto["balanced"]:
        assert (auto["waves_per_wg"], auto["num_partitions"], auto["partition_blocks"]) == \
            (waves, P, PB)


@pytest.mark.parametrize("B,Hkv,MB,cus,rows,P", [
    (8, 8, 64, 256, 32, 4),      # 32 rows per KV head; 4 partitions of 16 at most
    (64, 1, 512, 256, 256, 8),   # the llama3_8b TP8 shard: 8 partitions below 64 blocks
    (255, 1, 188, 256, 256, 2),  # one spare row: at most 2 partitions per sequence
    (2, 1, 4096, 256, 256, 64),  # 2 sequences of 4096 blocks: 64 partitions of 64
    (200, 1, 1024, 256, 256, 16),
    (4, 2, 8192, 16, 32, 29),    # few CUs: rows for 8 partitions of 1024 per sequence
])
def test_balanced_split_plan(native_lib, B, Hkv, MB, cus, rows, P):
    """Rows per KV head (at least one per CU, at least what the largest size
    needs), the most partitions one sequence can get (its table in partitions
    of the smallest size; at most 8 unless they hold 64 blocks or more; at
    most rows - B + 1), and the workspace (partials, then partition counts)."""
    dev = dict(MI355X, compute_units=cus)
    o = nat.default_options()
    o.even_split = nat.EVEN_SPLIT_OFF  # (200 x 1 x 1024 blocks would take the even split)
    p = nat.plan(nat.make_shape(B, 4 * Hkv, Hkv, MB, 1), o, device=dev)
    assert p["balanced"] == 1
    assert (p["workgroups"], p["num_partitions"], p["partition_blocks"]) == (rows * Hkv, P, 16)
    assert p["seq_order"] == nat.ORDER_NATURAL and p["waves_per_wg"] == 8
    assert p["workspace_bytes"] == (-(-B // 4) * 4 + B * 4 * Hkv * P * 130) * 4


@pytest.mark.parametrize("g,PB", [(1, 32), (4, 32), (8, 32), (16, 32)])
def test_two_loop_plan_keeps_the_scores_in_lds(native_lib, g, PB):
    o = nat.default_options()
    o.structure = nat.STRUCTURE_TWO_LOOP
    p = nat.plan(nat.make_shape(4, 2 * g, 2, 512, 100), o)
    assert (p["structure"], p["waves_per_wg"], p["partition_blocks"]) == (1, 4, PB)
    assert p["num_partitions"] == -(-512 // PB)


def call8(shape, opts=None):
    return nat.lib().paged_attn_decode_fp8(
        *[ctypes.c_void_p(FAKE)] * 5, ctypes.c_float(0.1), ctypes.c_float(1.0),
        ctypes.c_float(1.0), ctypes.c_void_p(FAKE), ctypes.byref(shape),
        ctypes.byref(opts) if opts is not None else None, None)


def test_two_loop_rejects_e4m3_and_debug_outputs(native_lib):
    o = nat.default_options()
    o.structure = nat.STRUCTURE_TWO_LOOP
    sh8 = good_shape(max_blocks_per_seq=16, kv_dtype=nat.KV_E4M3)
    assert call8(sh8, o) == nat.PA_ERR_UNSUPPORTED
    with pytest.raises(ValueError, match="unsupported"):
        nat.plan(sh8, o)
    sh = good_shape(max_blocks_per_seq=16)
    o.debug_error_word = FAKE
    assert call(sh, o) == nat.PA_ERR_UNSUPPORTED


def test_e4m3_entry_point_needs_an_e4m3_shape(native_lib):
    # 4096 blocks per sequence need partitions, so a shape that passes every
    # other check stops at the missing workspace, before any launch
    assert call8(good_shape()) == nat.PA_ERR_INVALID_ARG
    assert call8(good_shape(kv_dtype=nat.KV_E4M3)) == nat.PA_ERR_WORKSPACE
    assert call(good_shape(kv_dtype=nat.KV_E4M3)) == nat.PA_ERR_INVALID_ARG
    assert call(good_shape()) == nat.PA_ERR_WORKSPACE


@pytest.mark.parametrize("kv,pf,dist", [
    (0, 0, 1), (0, 1, 1), (0, 2, 1), (0, 3, 1), (0, 4, 1),
    (1, 0, 1), (1, 1, 1), (1, 2, 2), (1, 3, 1), (1, 4, 2)])
def test_default_lookahead_distance_depends_on_the_cache_type(native_lib, kv, pf, dist):
    o = nat.default_options()
    o.prefetch = pf
    p = nat.plan(good_shape(max_blocks_per_seq=16, kv_dtype=kv), o)
    assert (p["prefetch"], p["prefetch_distance"]) == (pf, dist)
    o.prefetch_distance = 1
    assert nat.plan(good_shape(max_blocks_per_seq=16, kv_dtype=kv), o)["prefetch_distance"] == 1


@pytest.mark.parametrize("kv,dist,waves", [(0, 1, 8), (0, 2, 4), (1, 1, 8), (1, 2, 8)])
def test_lds_ring_slots_count_in_the_wave_choice(native_lib, kv, dist, waves):
    """8 waves need (dist + 1) slots of one block's K and V each: 128 KiB for
    two fp16 slots fit in 160 KiB, 192 KiB for three do not (4 waves then);
    E4M3 slots are half the size."""
    o = nat.default_options()
    o.prefetch = nat.PREFETCH_LDS
    o.prefetch_distance = dist
    p = nat.plan(nat.make_shape(64, 32, 8, 512, 1000, kv_dtype=kv), o)
    assert (p["waves_per_wg"], p["num_partitions"]) == (waves, 1)


def test_binding_refuses_debug_outputs_of_the_wrong_size(native_lib):
    """The kernel writes the debug outputs at their full documented size, so a
    smaller (or otherwise shaped) tensor is refused by the binding."""
    import torch
    from paged_kv_cache_226_amd import ops
    B, Hkv, MB = 3, 2, 5
    ops.check_debug_shapes(B, Hkv, MB, torch.empty(B, Hkv, MB * 16, 128),
                           torch.empty(B, Hkv, MB, 2), torch.empty(1))
    for bad in (dict(debug_gather_k=torch.empty(B, Hkv, MB * 16 - 1, 128)),
                dict(debug_gather_k=torch.empty(B, Hkv, MB, 16, 128)),
                dict(debug_trace=torch.empty(B, Hkv, MB - 1, 2)),
                dict(debug_trace=torch.empty(B, Hkv + 1, MB, 2)),
                dict(debug_error_word=torch.empty(0))):
        with pytest.raises(ValueError):
            ops.check_debug_shapes(B, Hkv, MB, **bad)


def test_binding_refuses_broadcast_pools(native_lib):
    """A zero byte stride reaches the library as 'dense': an expanded (stride
    0) block or head dimension of a cache is refused instead."""
    import torch
    from paged_kv_cache_226_amd import ops
    q = torch.empty(2, 4, 128, dtype=torch.float16)
    bt = torch.zeros(2, 4, dtype=torch.int32)
    one = torch.empty(1, 2, 16, 16, 8, dtype=torch.float16)
    sh = ops.shape_of(q, one, bt)  # one block: stride 0 is not needed
    assert sh.num_blocks == 1
    with pytest.raises(ValueError, match="stride 0"):
        ops.shape_of(q, one.expand(64, 2, 16, 16, 8), bt)
    head = torch.empty(8, 1, 16, 16, 8, dtype=torch.float16)
    with pytest.raises(ValueError, match="stride 0"):
        ops.shape_of(q, head.expand(8, 2, 16, 16, 8), bt)
    v1 = torch.empty(1, 2, 16, 128, dtype=torch.float16)
    with pytest.raises(ValueError, match="v_cache"):
        ops.shape_of(q, torch.empty(64, 2, 16, 16, 8, dtype=torch.float16), bt,
                     v1.expand(64, 2, 16, 128))
    ok = ops.shape_of(q, torch.empty(64, 2, 16, 16, 8, dtype=torch.float16), bt,
                      torch.empty(64, 2, 16, 128, dtype=torch.float16))
    assert ok.num_blocks == 64 and ok.v_block_stride == 2 * 16 * 128 * 2


MI355X = dict(compute_units=256, lds_bytes_per_cu=163840, lds_bytes_per_workgroup=163840)


def test_device_figures_without_a_device_are_the_mi355x_ones(native_lib):
    """Here no device can be queried: the library plans with the MI355X
    figures, and planning for those figures explicitly gives the same plans."""
    import torch
    info = nat.device_info()
    if torch.cuda.is_available():
        pytest.skip("a device is visible: its own figures are used")
    assert info == dict(MI355X, queried=0)
    from paged_kv_cache_226_amd import inputs as gen
    for name, w in gen.WORKLOADS.items():
        MB = w.max_blocks_per_seq or max(-(-c // 16) for c in w.context_lens)
        sh = nat.make_shape(w.num_seqs, w.num_q_heads, w.num_kv_heads, MB, w.pool_blocks or 1)
        for pf in (-1, 0, 4):
            o = nat.default_options()
            o.prefetch = pf
            assert nat.plan(sh, o) == nat.plan(sh, o, device=MI355X), (name, pf)


@pytest.mark.parametrize("bad", [dict(compute_units=0), dict(compute_units=70000),
                                 dict(lds_bytes_per_workgroup=512),
                                 dict(lds_bytes_per_cu=65536)])
def test_plan_for_device_refuses_bad_figures(native_lib, bad):
    dev = dict(MI355X, **bad)
    with pytest.raises(ValueError, match="invalid argument"):
        nat.plan(good_shape(), device=dev)


@pytest.mark.parametrize("cus", [32, 64, 128, 256, 304, 512])
def test_plan_rules_follow_the_cu_count(native_lib, cus):
    """The partition, wave and order rules scale with the device's CU count:
    one partition per sequence iff there are at least as many (sequence, KV
    head) units as CUs; 8 waves for such unsplit long tables while there are
    fewer than three units per CU; longest-first order iff the grid holds
    more work-groups than the CUs keep resident (three 4-wave ones each);
    the even split (one share per CU, 2 waves) for at least half as many
    units as CUs over a long table."""
    dev = dict(MI355X, compute_units=cus)
    for B in (1, 2, 4, 8, 16, 32, 64, 96, 128, 200, 256):
        units = B * 8
        p = nat.plan(nat.make_shape(B, 32, 8, 512, 1), device=dev)
        even = B >= 2 and 2 * units >= cus
        assert p["even_split"] == even, (B, p)
        if even:
            assert (p["workgroups"], p["waves_per_wg"], p["num_partitions"]) == (cus, 2, 1)
            continue
        assert (p["num_partitions"] == 1) == (units >= cus), (B, p)
        if units >= cus:
            assert p["waves_per_wg"] == (8 if units < 3 * cus else 4), (B, p)
        else:
            assert p["num_partitions"] >= min(-(-cus // units), 2) and p["waves_per_wg"] == 8
        # short tables (no even split): 4 waves, one partition when units >= cus
        q = nat.plan(nat.make_shape(B, 32, 8, 64, 1), device=dev)
        assert q["even_split"] == 0
        if units >= cus:
            want = nat.ORDER_LONGEST_FIRST if B >= 2 and units > 3 * cus else nat.ORDER_NATURAL
            assert (q["waves_per_wg"], q["num_partitions"], q["seq_order"]) == (4, 1, want), (B, q)


def test_plan_lds_rules_follow_the_device(native_lib):
    """The LDS limits come from the device: a plan whose work-group needs more
    LDS than the device allows is refused, and the residency count that
    decides the order uses the LDS per CU."""
    sh = good_shape(max_blocks_per_seq=64)
    o = nat.default_options()
    o.prefetch, o.prefetch_distance, o.waves_per_wg = 4, 2, 4  # 96 KiB of LDS slots
    assert nat.plan(sh, o, device=MI355X)["prefetch"] == 4
    small = dict(MI355X, lds_bytes_per_cu=65536, lds_bytes_per_workgroup=65536)
    with pytest.raises(ValueError, match="unsupported"):
        nat.plan(sh, o, device=small)
    # 20 sequences x 8 KV heads, 4-wave work-groups with 64 KiB of LDS ring
    # each (2 per CU by LDS): 256 CUs hold the whole grid at once, 64 CUs
    # only 128 of its 160 work-groups
    sh2 = nat.make_shape(20, 64, 8, 64, 1)
    o2 = nat.default_options()
    o2.prefetch, o2.prefetch_distance, o2.waves_per_wg = 4, 1, 4
    assert nat.plan(sh2, o2, device=MI355X)["seq_order"] == nat.ORDER_NATURAL
    few = dict(MI355X, compute_units=64)
    assert nat.plan(sh2, o2, device=few)["seq_order"] == nat.ORDER_LONGEST_FIRST


def test_pack_k_validation(native_lib):
    f = native_lib.paged_attn_pack_k
    A, B = ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE + (1 << 24))
    assert f(None, B, 4, 2, nat.KV_F16, None) == nat.PA_ERR_INVALID_ARG
    assert f(A, ctypes.c_void_p(FAKE + (1 << 24) + 8), 4, 2, nat.KV_F16, None) == \
        nat.PA_ERR_INVALID_ARG
    assert f(A, B, 0, 2, nat.KV_F16, None) == nat.PA_ERR_INVALID_ARG
    assert f(A, B, 4, 0, nat.KV_F16, None) == nat.PA_ERR_INVALID_ARG
    assert f(A, B, 4, 2, 7, None) == nat.PA_ERR_INVALID_ARG
    # the output overlaps the input: 4 blocks x 2 heads x 4 KiB = 32 KiB
    assert f(A, ctypes.c_void_p(FAKE + 16384), 4, 2, nat.KV_F16, None) == nat.PA_ERR_INVALID_ARG
    assert f(A, B, 1 << 62, 2, nat.KV_F16, None) == nat.PA_ERR_UNSUPPORTED


def hinted(min_ctx, **kw):
    o = nat.default_options()
    o.min_context_hint = min_ctx
    for k, v in kw.items():
        setattr(o, k, v)
    return o


# (B, Hq, Hkv, kv_dtype) -> (waves, cap) on 256 CUs with every context at
# the table's width: a whole number u of (sequence, KV head) units per CU
@pytest.mark.parametrize("B,Hq,Hkv,kv,want", [
    (8, 32, 32, nat.KV_F16, (2, 0)),     # u = 1
    (16, 32, 32, nat.KV_F16, (1, 0)),    # u = 2
    (128, 28, 4, nat.KV_F16, (1, 0)),    # u = 2, GQA 7:1
    (24, 32, 32, nat.KV_F16, (2, 1)),    # u = 3
    (32, 32, 32, nat.KV_F16, (1, 2)),    # u = 4 (the llama2_7b shape)
    (128, 40, 8, nat.KV_F16, (1, 2)),    # u = 4, GQA 5:1
    (48, 32, 32, nat.KV_F16, (1, 2)),    # u = 6
    (32, 32, 32, nat.KV_E4M3, (1, 4)),   # u = 4, E4M3
])
def test_streaming_shape_for_uniform_contexts(native_lib, B, Hq, Hkv, kv, want):
    MB = 256
    sh = nat.make_shape(B, Hq, Hkv, MB, 1, kv_dtype=kv)
    p = nat.plan(sh, hinted(MB * 16), device=MI355X)
    assert (p["waves_per_wg"], p["resident_wgs"]) == want
    assert p["prefetch"] == nat.PREFETCH_REG and p["num_partitions"] == 1
    assert p["seq_order"] == nat.ORDER_NATURAL
    # two sequences per work-group where 1-wave work-groups capped at 2 per
    # CU still fill whole rounds of the cap with the grid halved
    chained = want == (1, 2) and (B * Hkv) % (2 * 2 * 256) == 0
    assert p["seqs_per_wg"] == (2 if chained else 1)
    assert p["workgroups"] == B * Hkv // p["seqs_per_wg"]
    if want[1]:
        # cap work-groups of the LDS fill a CU, cap + 1 do not
        share = 163840 // want[1] // 1024 * 1024 - 1024
        assert p["lds_bytes"] == share
        assert want[1] * (share + 1024) <= 163840 < (want[1] + 1) * (share + 256)
    # the hint is the only difference from the default plan
    base = nat.plan(sh, device=MI355X)
    assert base["resident_wgs"] == 0 or base["even_split"] == 1
    assert (base["waves_per_wg"], base["resident_wgs"], base["even_split"]) != want + (0,)


@pytest.mark.parametrize("case", [
    "no hint", "ragged", "short table", "short gqa table", "split table", "not a multiple",
    "u = 5", "u = 8", "u = 16", "e4m3 u = 2",
    "explicit waves", "l2 touch", "lds ring", "fp16 two blocks ahead", "e4m3 one block ahead",
    "explicit partitions",
    "explicit cap", "two-loop"])
def test_streaming_shape_needs_every_condition(native_lib, case):
    B, Hq, Hkv, MB, kv, hint, kw = 32, 32, 32, 128, nat.KV_F16, 128 * 16, {}
    if case == "no hint":
        hint = 0
    elif case == "ragged":
        hint = 128 * 16 * 7 // 8 - 1  # one token under 7/8 of the table
    elif case == "short table":
        MB, hint = 63, 63 * 16
    elif case == "short gqa table":
        # (without the hint this table takes the even split)
        B, Hq, Hkv, MB, hint = 128, 32, 8, 255, 255 * 16
        kw = dict(even_split=nat.EVEN_SPLIT_OFF)
    elif case == "split table":
        MB, hint = 1025, 1025 * 16
    elif case == "not a multiple":
        B = 33
    elif case == "u = 8":
        B = 64
    elif case == "u = 5":
        B = 40
    elif case == "u = 16":
        B = 128
    elif case == "e4m3 u = 2":
        B, kv = 16, nat.KV_E4M3
    elif case == "explicit waves":
        kw = dict(waves_per_wg=4)
    elif case == "l2 touch":
        kw = dict(prefetch=nat.PREFETCH_L2)
    elif case == "lds ring":
        kw = dict(prefetch=nat.PREFETCH_LDS)
    elif case == "fp16 two blocks ahead":
        kw = dict(prefetch_distance=2)
    elif case == "e4m3 one block ahead":
        kv, kw = nat.KV_E4M3, dict(prefetch_distance=1)
    elif case == "explicit partitions":
        kw = dict(partition_blocks=128)
    elif case == "explicit cap":
        kw = dict(max_resident_wgs=3)
    elif case == "two-loop":
        kw = dict(structure=nat.STRUCTURE_TWO_LOOP)
    sh = nat.make_shape(B, Hq, Hkv, MB, 1, kv_dtype=kv)
    p = nat.plan(sh, hinted(hint, **kw), device=MI355X)
    q = nat.plan(sh, hinted(0, **kw), device=MI355X)
    assert p == q, case


# the same, look-ahead off: one block in flight per wave, so about 4 waves
# per CU (8 for E4M3)
@pytest.mark.parametrize("B,Hq,Hkv,kv,want", [
    (8, 32, 32, nat.KV_F16, (4, 0)),     # u = 1
    (16, 32, 32, nat.KV_F16, (2, 0)),    # u = 2
    (24, 32, 32, nat.KV_F16, (4, 1)),    # u = 3
    (32, 32, 32, nat.KV_F16, (1, 4)),    # u = 4
    (48, 32, 32, nat.KV_F16, (2, 2)),    # u = 6
    (8, 32, 32, nat.KV_E4M3, (8, 0)),    # u = 1
    (32, 32, 32, nat.KV_E4M3, (2, 4)),   # u = 4
])
def test_streaming_shape_with_the_lookahead_off(native_lib, B, Hq, Hkv, kv, want):
    sh = nat.make_shape(B, Hq, Hkv, 128, 1, kv_dtype=kv)
    p = nat.plan(sh, hinted(128 * 16, prefetch=nat.PREFETCH_OFF), device=MI355X)
    assert (p["prefetch"], p["waves_per_wg"], p["resident_wgs"]) == (0, *want)


@pytest.mark.parametrize("kv,dist", [(nat.KV_F16, 1), (nat.KV_E4M3, 2)])
def test_explicit_default_distance_keeps_the_streaming_shape(native_lib, kv, dist):
    sh = nat.make_shape(32, 32, 32, 128, 1, kv_dtype=kv)
    auto = nat.plan(sh, hinted(128 * 16), device=MI355X)
    expl = nat.plan(sh, hinted(128 * 16, prefetch=nat.PREFETCH_REG, prefetch_distance=dist),
                    device=MI355X)
    assert auto == expl and auto["resident_wgs"] > 0


def test_the_hint_at_exactly_seven_eighths_of_the_table(native_lib):
    sh = nat.make_shape(32, 32, 32, 128, 1)
    assert nat.plan(sh, hinted(128 * 16 * 7 // 8), device=MI355X)["resident_wgs"] == 2
    assert nat.plan(sh, hinted(128 * 16 * 7 // 8 - 1), device=MI355X)["resident_wgs"] == 0


@pytest.mark.parametrize("cap", [1, 2, 3, 4, 5, 6, 7, 8])
def test_residency_cap_sizes_the_lds(native_lib, cap):
    sh = nat.make_shape(32, 32, 8, 64, 1)
    p = nat.plan(sh, hinted(0, max_resident_wgs=cap), device=MI355X)
    base = nat.plan(sh, device=MI355X)
    share = max(163840 // cap // 1024 * 1024 - 1024, 0)
    assert p["resident_wgs"] == cap
    assert p["lds_bytes"] == max(share, base["lds_bytes"])
    assert p["lds_bytes"] + 1024 <= 163840
    # cap work-groups fit with up to 1 KiB each of compiler LDS and rounding;
    # cap + 1 do not, even with only the kernel's 256 B
    assert cap * (share + 1024) <= 163840 < (cap + 1) * (share + 256)
    # nothing else changes
    for k in ("prefetch", "waves_per_wg", "partition_blocks", "num_partitions", "workgroups",
              "workspace_bytes", "prefetch_distance", "balanced"):
        assert p[k] == base[k], k


@pytest.mark.parametrize("bad", [dict(max_resident_wgs=-1), dict(max_resident_wgs=9),
                                 dict(min_context_hint=-5)])
def test_hint_and_cap_are_validated(native_lib, bad):
    with pytest.raises(ValueError, match="invalid argument"):
        nat.plan(good_shape(max_blocks_per_seq=16), hinted(0, **bad))
    assert call(good_shape(max_blocks_per_seq=16), hinted(0, **bad)) == nat.PA_ERR_INVALID_ARG


def test_lds_limit_leaves_room_for_the_compilers_lds(native_lib):
    """A work-group's dynamic LDS plus what the compiler adds (256 B here,
    1 KiB allowed) must fit the device's LDS per work-group: a plan whose
    dynamic LDS alone would just fit is refused."""
    sh = good_shape(max_blocks_per_seq=64)
    o = nat.default_options()
    o.prefetch, o.prefetch_distance, o.waves_per_wg = 4, 2, 4  # 96 KiB of LDS slots + table
    need = nat.plan(sh, o, device=MI355X)["lds_bytes"]
    fits = dict(MI355X, lds_bytes_per_cu=163840, lds_bytes_per_workgroup=need + 1024)
    assert nat.plan(sh, o, device=fits)["lds_bytes"] == need
    tight = dict(MI355X, lds_bytes_per_cu=163840, lds_bytes_per_workgroup=need + 512)
    with pytest.raises(ValueError, match="unsupported"):
        nat.plan(sh, o, device=tight)


# fewer units than CUs, uniform: the balanced split keeps one work-group per
# CU; from 256 table blocks per CU it takes 2 waves (4 with the look-ahead
# off) instead of 8
@pytest.mark.parametrize("B,Hq,Hkv,MB,pf,want", [
    (4, 32, 32, 512, -1, 2),     # 512 x 128 units = 256 blocks per CU
    (8, 32, 8, 1024, -1, 2),
    (128, 5, 1, 512, -1, 2),
    (4, 32, 32, 512, 0, 4),
    (16, 32, 8, 256, -1, 8),     # 128 blocks per CU: 8 waves
    (4, 32, 32, 256, -1, 8),
    (8, 32, 8, 1024, 1, 8),      # the L2 touch: no streaming shape
])
def test_streaming_waves_for_balanced_uniform_batches(native_lib, B, Hq, Hkv, MB, pf, want):
    sh = nat.make_shape(B, Hq, Hkv, MB, 1)
    p = nat.plan(sh, hinted(MB * 16, prefetch=pf), device=MI355X)
    assert p["balanced"] == 1 and p["waves_per_wg"] == want and p["resident_wgs"] == 0
    q = nat.plan(sh, hinted(0, prefetch=pf, even_split=nat.EVEN_SPLIT_OFF), device=MI355X)
    assert q["balanced"] == 1 and q["waves_per_wg"] == 8
    e4 = nat.plan(nat.make_shape(B, Hq, Hkv, MB, 1, kv_dtype=nat.KV_E4M3),
                  hinted(MB * 16, prefetch=pf), device=MI355X)
    assert e4["waves_per_wg"] == 8


def test_debug_timeline_pointer_must_be_8_byte_aligned(native_lib):
    o = nat.default_options()
    o.debug_timeline = FAKE + 4
    assert call(good_shape(max_blocks_per_seq=16), o) == nat.PA_ERR_INVALID_ARG


def test_binding_refuses_a_timeline_of_the_wrong_size(native_lib):
    import torch
    from paged_kv_cache_226_amd import ops
    ops.check_debug_timeline(torch.empty(256, 4, dtype=torch.int64), 256)
    for bad in (torch.empty(255, 4, dtype=torch.int64), torch.empty(256, 3, dtype=torch.int64),
                torch.empty(256, 4, dtype=torch.int32)):
        with pytest.raises(ValueError, match="debug_timeline"):
            ops.check_debug_timeline(bad, 256)


@pytest.mark.parametrize("B,Hkv,waves,cap,order,want", [
    (64, 16, 1, 2, 0, 2),                          # explicit: 1024 units, 512 work-groups
    (64, 16, 1, 2, nat.ORDER_LONGEST_FIRST, 2),    # ranked pairs y and B-1-y
    (63, 16, 1, 2, 0, 1),                          # odd batch
    (32, 16, 1, 2, 0, 1),                          # 512 units: half a round of the cap
    (64, 16, 2, 2, 0, 1),                          # 2-wave work-groups
    (64, 16, 1, 3, 0, 1),                          # another cap
    (64, 16, 1, 0, 0, 1),                          # no cap
])
def test_two_sequences_per_work_group(native_lib, B, Hkv, waves, cap, order, want):
    sh = nat.make_shape(B, 2 * Hkv, Hkv, 64, 64 * B)
    p = nat.plan(sh, hinted(0, waves_per_wg=waves, max_resident_wgs=cap, seq_order=order,
                            partition_blocks=64), device=MI355X)
    assert (p["waves_per_wg"], p["num_partitions"]) == (waves, 1)
    assert p["seqs_per_wg"] == want
    assert p["workgroups"] == B * Hkv // want
    if order:
        assert p["seq_order"] == order
