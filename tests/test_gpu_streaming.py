"""The streaming shape on the GPU (MI355X): batches whose contexts all fill
the block table (the caller's min_context_hint says so) with a whole number
u of (sequence, KV head) units per CU run on 1- or 2-wave work-groups under
a residency cap, which the launch enforces through its LDS request.

Checked here: the hinted plan is the streaming one; its output against the
fp64 oracle; the residency cap changes no bits (the same waves and look-ahead
without the cap give the same output); every look-ahead mode on the same
plan gives the same bits; a wrong hint on a ragged batch changes speed only,
never the result; E4M3.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from paged_kv_cache_226_amd import _native as nat
from paged_kv_cache_226_amd import inputs as gen
from paged_kv_cache_226_amd import ops

from parity import assert_close, bits, oracle, run, same_plan, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(native_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def cus():
    return nat.device_info()["compute_units"]


# (units per CU, query heads, KV heads, context tokens) -> expected (waves, cap)
CASES = [
    (1, 32, 32, 1024, (2, 0)),
    (2, 32, 32, 1024, (1, 0)),
    (2, 28, 4, 4096, (1, 0)),
    (3, 32, 32, 1024, (2, 1)),
    (4, 32, 32, 1024, (1, 2)),
    (4, 40, 8, 4112, (1, 2)),   # 257 blocks, the last one partial
    (6, 32, 32, 1024, (1, 2)),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_streaming_shape_against_the_oracle(case):
    u, Hq, Hkv, ctx, want = CASES[case]
    C = cus()
    if (u * C) % Hkv:
        pytest.skip(f"{C} CUs: {u} units per CU is not a whole batch of {Hkv} KV heads")
    B = u * C // Hkv
    print(f"[streaming] case {case}: u={u} B={B} Hq={Hq} Hkv={Hkv} ctx={ctx}", flush=True)
    x = gen.make_case(B, Hq, Hkv, [ctx] * B, seed=700 + case, extra_pool_blocks=5, poison=True)
    dev = to_device(x)
    plan = ops.plan(dev["q"], dev["k_cache"], dev["block_tables"], min_context_hint=ctx)
    if C == 256:
        assert (plan["waves_per_wg"], plan["resident_wgs"]) == want
    assert plan["num_partitions"] == 1
    got = run(x, dev, min_context_hint=ctx)
    assert_close(got, oracle(x), f"streaming case {case}")
    # the cap changes no bits
    free = run(x, dev, **same_plan(plan, max_resident_wgs=0))
    assert np.array_equal(bits(got), bits(free)), "cap"
    # every look-ahead mode on the same plan gives the same bits
    for pf in (0, 1, 3):
        o = run(x, dev, prefetch=pf, **same_plan(plan))
        assert np.array_equal(bits(o), bits(got)), f"mode {pf}"


def test_wrong_hint_on_a_ragged_batch_changes_no_result():
    """The hint claims every context fills the table; half of them are short.
    The streaming plan is taken and the output is still the oracle's."""
    C = cus()
    B, Hq, Hkv = 4 * C // 32, 32, 32
    lens = [1024 if i % 2 else 1 + 29 * i for i in range(B)]
    x = gen.make_case(B, Hq, Hkv, lens, seed=760, extra_pool_blocks=3, poison=True)
    dev = to_device(x)
    plan = ops.plan(dev["q"], dev["k_cache"], dev["block_tables"], min_context_hint=1024)
    if C == 256:
        assert plan["resident_wgs"] == 2
    got = run(x, dev, min_context_hint=1024)
    assert_close(got, oracle(x), "wrong hint")
    assert np.array_equal(bits(got), bits(run(x, dev, **same_plan(plan, max_resident_wgs=0))))


@pytest.mark.parametrize("cap", [1, 3, 8])
def test_explicit_residency_caps_change_no_bits(cap):
    x = gen.make_case(64, 16, 4, None, seed=770, ctx_range=(1, 3000), extra_pool_blocks=2)
    dev = to_device(x)
    off = dict(even_split=nat.EVEN_SPLIT_OFF)  # (the auto plan would take the even split)
    ref = run(x, dev, **off)
    got = run(x, dev, max_resident_wgs=cap, **off)
    assert np.array_equal(bits(got), bits(ref))
    assert_close(got, oracle(x), f"cap {cap}")


def test_streaming_shape_over_an_e4m3_cache():
    C = cus()
    B, Hq, Hkv, ctx = 4 * C // 32, 32, 32, 1024
    x8 = gen.to_fp8(gen.make_case(B, Hq, Hkv, [ctx] * B, seed=780))
    d = {k: torch.from_numpy(getattr(x8, k)).cuda() for k in ("q", "block_tables", "context_lens")}
    d["k_cache"] = torch.from_numpy(gen.pack_k_fp8(x8.k8)).cuda()
    d["v_cache"] = torch.from_numpy(x8.v8).cuda()
    plan = ops.plan(d["q"], d["k_cache"], d["block_tables"], min_context_hint=ctx)
    if C == 256:
        assert (plan["waves_per_wg"], plan["resident_wgs"]) == (1, 4)
    dec = lambda **kw: ops.paged_attn_decode_fp8(
        d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["context_lens"], x8.scale,
        x8.k_scale, x8.v_scale, **kw).cpu().numpy()
    got = dec(min_context_hint=ctx)
    ref = orc.paged_attention_fp8_f64(x8.q, x8.k8, x8.v8, x8.block_tables, x8.context_lens,
                                      x8.scale, x8.k_scale, x8.v_scale)
    assert_close(got, ref, "e4m3 streaming")
    assert np.array_equal(bits(got), bits(dec(**same_plan(plan, max_resident_wgs=0))))
    assert np.array_equal(bits(got), bits(dec(prefetch=0, **same_plan(plan))))


@pytest.mark.parametrize("B,Hq,Hkv,ctx", [(4, 32, 32, 8192), (128, 5, 1, 8192), (3, 16, 4, 96000)])
def test_streaming_waves_of_a_balanced_split(B, Hq, Hkv, ctx):
    """Fewer units than CUs, every context at the table's width: the balanced
    split on 2-wave work-groups (where the walk per CU is long enough)."""
    x = gen.make_case(B, Hq, Hkv, [ctx] * B, seed=790 + B, extra_pool_blocks=3, poison=True)
    dev = to_device(x)
    plan = ops.plan(dev["q"], dev["k_cache"], dev["block_tables"], min_context_hint=ctx)
    assert plan["balanced"] == 1
    if cus() == 256:
        assert plan["waves_per_wg"] == 2
    got = run(x, dev, min_context_hint=ctx)
    assert_close(got, oracle(x), f"balanced streaming {B}x{ctx}")
    for pf in (0, 1, 3):
        o = run(x, dev, prefetch=pf, **same_plan(plan))
        assert np.array_equal(bits(o), bits(got)), f"mode {pf}"


@pytest.mark.parametrize("order", [0, nat.ORDER_LONGEST_FIRST])
def test_two_sequences_per_work_group_on_a_ragged_batch(order):
    """1-wave work-groups capped at 2 per CU walk sequence ranks y and B-1-y
    in turn (under longest-first order a long sequence pairs with a short
    one); empty sequences on either side of a pair give zeros.  The same
    waves, order and partitions under another cap (one sequence per
    work-group) give the same bits."""
    C = cus()
    Hkv = 16
    B = 4 * C // Hkv
    rng = np.random.default_rng(830)
    lens = rng.integers(1, 1025, size=B)
    lens[[0, 3, B - 1, B // 2]] = 0
    lens[[1, 5]] = 1024
    x = gen.make_case(B, 2 * Hkv, Hkv, [int(v) for v in lens], seed=831, extra_pool_blocks=3,
                      poison=True)
    dev = to_device(x)
    kw = dict(waves_per_wg=1, partition_blocks=64, seq_order=order)
    plan = ops.plan(dev["q"], dev["k_cache"], dev["block_tables"], max_resident_wgs=2, **kw)
    print(f"[chain] order={order} B={B} plan={plan}", flush=True)
    assert plan["seqs_per_wg"] == 2 and plan["num_partitions"] == 1
    got = run(x, dev, max_resident_wgs=2, **kw)
    assert_close(got, oracle(x), f"two per work-group, order {order}")
    one = run(x, dev, max_resident_wgs=3, **kw)
    assert np.array_equal(bits(got), bits(one))
    for pf in (0, 1, 3):
        o = run(x, dev, prefetch=pf, max_resident_wgs=2, **kw)
        assert np.array_equal(bits(o), bits(got)), f"mode {pf}"
