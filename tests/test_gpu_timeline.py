"""The debug timeline on the GPU (MI355X): one row per decode work-group with
its start and end on the constant 100 MHz clock and the HW_ID / XCC_ID
registers of its CU.

Checked here: every work-group of the grid records a start no later than its
end, all within the span of the launch as the host times it; the CUs named
are distinct hardware CUs, at most as many as the device has; the output is
bitwise the plain call's (the timeline only adds stores); grid rows with no
work (a balanced split's spare rows, empty sequences) record both times too.
"""
import time

import numpy as np
import pytest
import torch

from paged_kv_cache_226_amd import _native as nat
from paged_kv_cache_226_amd import inputs as gen
from paged_kv_cache_226_amd import ops

from parity import assert_close, bits, oracle, run, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(native_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def cu_key(hw_id, xcc_id):
    """(XCC, SE, SH, CU) from the HW_ID fields cu_id[11:8], sh_id[12],
    se_id[15:13] and XCC_ID[3:0]."""
    return (int(xcc_id) & 0xF, (int(hw_id) >> 13) & 0x7, (int(hw_id) >> 12) & 0x1,
            (int(hw_id) >> 8) & 0xF)


def check_timeline(tl, wall_s):
    start, end = tl[:, 0], tl[:, 1]
    assert (start > 0).all() and (end >= start).all()
    span_s = (end.max() - start.min()) / 100e6
    assert 0 < span_s <= wall_s + 1e-3, (span_s, wall_s)
    keys = {cu_key(h, x) for h, x in zip(tl[:, 2], tl[:, 3])}
    assert 1 <= len(keys) <= nat.device_info()["compute_units"]
    return keys


@pytest.mark.parametrize("hint", [0, 2048])
def test_timeline_of_a_uniform_batch(hint):
    """MHA 32 x 2048 tokens: 1024 work-groups (4 waves, or 1 wave at most 2
    per CU with the hint)."""
    x = gen.make_case(32, 32, 32, [2048] * 32, seed=800)
    dev = to_device(x)
    plan = ops.plan(dev["q"], dev["k_cache"], dev["block_tables"], min_context_hint=hint)
    tl = torch.zeros(plan["workgroups"], 4, dtype=torch.int64, device="cuda")
    plain = run(x, dev, min_context_hint=hint)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    got = run(x, dev, min_context_hint=hint, debug_timeline=tl)
    wall = time.perf_counter() - t0
    assert np.array_equal(bits(got), bits(plain))
    keys = check_timeline(tl.cpu().numpy(), wall)
    if nat.device_info()["compute_units"] == 256:
        assert len(keys) == 256  # 1024 work-groups reach every CU


def test_timeline_records_idle_rows_of_a_balanced_split():
    """A ragged small batch on the balanced split: rows past the last
    partition and an empty sequence's partition still record their times."""
    lens = [0, 17, 5000, 300, 12000, 1]
    x = gen.make_case(len(lens), 16, 2, lens, seed=810, extra_pool_blocks=3)
    dev = to_device(x)
    plan = ops.plan(dev["q"], dev["k_cache"], dev["block_tables"])
    assert plan["balanced"] == 1
    tl = torch.zeros(plan["workgroups"], 4, dtype=torch.int64, device="cuda")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    got = run(x, dev, debug_timeline=tl)
    wall = time.perf_counter() - t0
    check_timeline(tl.cpu().numpy(), wall)
    assert_close(got, oracle(x), "balanced with timeline")


def test_timeline_of_the_e4m3_kernel():
    x8 = gen.to_fp8(gen.make_case(8, 8, 2, [700, 1, 0, 2100, 33, 160, 999, 4000], seed=820))
    d = {k: torch.from_numpy(getattr(x8, k)).cuda() for k in ("q", "block_tables", "context_lens")}
    d["k_cache"] = torch.from_numpy(gen.pack_k_fp8(x8.k8)).cuda()
    d["v_cache"] = torch.from_numpy(x8.v8).cuda()
    plan = ops.plan(d["q"], d["k_cache"], d["block_tables"])
    tl = torch.zeros(plan["workgroups"], 4, dtype=torch.int64, device="cuda")
    dec = lambda **kw: ops.paged_attn_decode_fp8(
        d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["context_lens"], x8.scale,
        x8.k_scale, x8.v_scale, **kw).cpu().numpy()
    plain = dec()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    got = dec(debug_timeline=tl)
    wall = time.perf_counter() - t0
    assert np.array_equal(bits(got), bits(plain))
    check_timeline(tl.cpu().numpy(), wall)
