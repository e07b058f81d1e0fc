"""paged_attn_decode_noalloc through the C ABI (MI355X).

The entry point for callers that cannot allocate takes its partition partials
from the library's per-device scratch array instead of a caller's workspace.
It runs the same kernels and plan as paged_attn_decode, so its output must be
bitwise that of paged_attn_decode with a workspace (and within tolerance of
the fp64 oracle).  Two calls in a row, the second on a smaller input, check
that a call does not depend on what the previous one left in the array.
"""
import ctypes

import numpy as np
import pytest
import torch

from paged_kv_cache_226_amd import _native as nat
from paged_kv_cache_226_amd import inputs as gen
from paged_kv_cache_226_amd import ops

from parity import assert_close, bits, oracle, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(native_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def c_call(name, d, scale, out, opts):
    """One call of entry point `name` through the C ABI on torch's current
    stream; returns the status code."""
    sh = ops.shape_of(d["q"], d["k_cache"], d["block_tables"], d["v_cache"])
    ptrs = [ctypes.c_void_p(d[k].data_ptr())
            for k in ("q", "k_cache", "v_cache", "block_tables", "context_lens")]
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return getattr(nat.lib(), name)(*ptrs, ctypes.c_float(scale), ctypes.c_void_p(out.data_ptr()),
                                    ctypes.byref(sh), ctypes.byref(opts), st)


def with_workspace(d, x, **kw):
    out = torch.empty_like(d["q"])
    o = ops.options(**kw)
    need = ops.workspace_bytes(d["q"], d["k_cache"], d["block_tables"], **kw)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=d["q"].device)
    o.workspace, o.workspace_bytes = ws.data_ptr(), ws.numel()
    assert c_call("paged_attn_decode", d, x.scale, out, o) == nat.PA_OK
    torch.cuda.synchronize()
    return out.cpu().numpy()


# (B, Hq, Hkv, context lengths, options): every case plans several partitions
# (so the scratch array is used), the second of each pair on a smaller input
PAIRS = [
    ((4, 32, 8, [4000, 1, 3333, 2900], {}),
     (2, 8, 2, [900, 17], {})),
    ((3, 28, 4, [8192, 5000, 64], dict(prefetch=4, partition_blocks=32)),
     (1, 7, 1, [1000], dict(prefetch=0, partition_blocks=16, waves_per_wg=2))),
    ((2, 16, 1, [16384, 9000], dict(prefetch=1, prefetch_distance=3)),
     (2, 4, 1, [600, 2000], dict(prefetch=3))),
]


@pytest.mark.parametrize("pair", range(len(PAIRS)))
def test_noalloc_matches_the_workspace_entry_point_twice_in_a_row(pair):
    for k, (B, Hq, Hkv, ctx, kw) in enumerate(PAIRS[pair]):
        print(f"[noalloc] pair {pair} call {k}: B={B} Hq={Hq} Hkv={Hkv} ctx={ctx} {kw}",
              flush=True)
        x = gen.make_case(B, Hq, Hkv, ctx, seed=900 + 10 * pair + k, extra_pool_blocks=5,
                          poison=True)
        d = to_device(x)
        p = ops.plan(d["q"], d["k_cache"], d["block_tables"], **kw)
        assert p["num_partitions"] > 1 and 0 < p["workspace_bytes"] <= nat.NOALLOC_SCRATCH_BYTES
        want = with_workspace(d, x, **kw)
        out = torch.full_like(d["q"], float("nan"))
        assert c_call("paged_attn_decode_noalloc", d, x.scale, out, ops.options(**kw)) == nat.PA_OK
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(bits(got), bits(want)), f"pair {pair} call {k}"
        assert_close(got, oracle(x), f"noalloc pair {pair} call {k}")


def test_noalloc_single_partition_and_empty_sequences():
    """A plan without partials, with empty and one-token sequences."""
    x = gen.make_case(300, 8, 1, [0, 1, 17] + [40] * 297, seed=950, poison=True)
    d = to_device(x)
    assert ops.plan(d["q"], d["k_cache"], d["block_tables"])["num_partitions"] == 1
    want = with_workspace(d, x)
    out = torch.full_like(d["q"], float("nan"))
    assert c_call("paged_attn_decode_noalloc", d, x.scale, out, ops.options()) == nat.PA_OK
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.array_equal(bits(got), bits(want))
    assert_close(got, oracle(x), "noalloc single partition")


def test_noalloc_calls_allocate_no_device_memory():
    """After a first call on the device, further calls leave the device's free
    memory unchanged (the scratch array was placed when the library's code
    was loaded)."""
    x = gen.make_case(4, 32, 8, [4000, 3000, 2000, 1000], seed=960)
    d = to_device(x)
    out = torch.empty_like(d["q"])
    o = ops.options()
    assert c_call("paged_attn_decode_noalloc", d, x.scale, out, o) == nat.PA_OK
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for _ in range(5):
        assert c_call("paged_attn_decode_noalloc", d, x.scale, out, o) == nat.PA_OK
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0


def test_noalloc_refuses_a_plan_beyond_the_scratch_before_any_launch():
    """Partials beyond PA_NOALLOC_SCRATCH_BYTES: PA_ERR_WORKSPACE, out untouched."""
    x = gen.make_case(1, 16, 1, [16], seed=970)
    d = to_device(x)
    # 255 sequences x 16 heads x 64 partitions of 16 blocks: 8.5e7 bytes of partials
    sh_kw = dict(q=torch.empty(255, 16, 128, dtype=torch.float16, device="cuda"),
                 block_tables=torch.zeros(255, 1024, dtype=torch.int32, device="cuda"),
                 context_lens=torch.ones(255, dtype=torch.int32, device="cuda"))
    big = dict(d, **sh_kw)
    o = ops.options(partition_blocks=16)
    need = ops.workspace_bytes(big["q"], big["k_cache"], big["block_tables"], partition_blocks=16)
    assert need > nat.NOALLOC_SCRATCH_BYTES
    out = torch.full_like(big["q"], 7.0)
    assert c_call("paged_attn_decode_noalloc", big, x.scale, out, o) == nat.PA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
