"""The even split on the GPU (MI355X): every work-group takes an equal share
of the batch's (block, KV head) pairs, whole units are written directly and
the pieces of the units that cross a share boundary are merged by the
reduce kernel.

Checked here, against the fp64 oracle: ragged batches with empty sequences;
fewer blocks than shares (most shares empty); one unit cut into a piece per
share; an all-empty batch; explicit waves and residency; every look-ahead
mode on the same plan gives the same bits; E4M3; the no-allocation entry
point gives the workspace call's bits.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from paged_kv_cache_226_amd import _native as nat
from paged_kv_cache_226_amd import inputs as gen
from paged_kv_cache_226_amd import ops

from parity import assert_close, bits, oracle, run, to_device

pytestmark = pytest.mark.gpu

EVEN = nat.EVEN_SPLIT_ON


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(native_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


CASES = [
    # (B, Hq, Hkv, context lengths or a range, seed, extra options)
    (64, 32, 8, (1, 8192), 900, {}),
    (64, 4, 1, (512, 8192), 901, {}),
    (16, 16, 2, [0, 17, 5000, 300, 12000, 1, 0, 4096, 16, 15, 33, 8000, 0, 2, 999, 1024], 902, {}),
    (1, 8, 1, [40], 903, {}),                        # 3 blocks over 256 shares
    (1, 16, 1, [16384], 904, {}),                    # one unit in a piece per share
    (3, 8, 8, [0, 0, 0], 905, {}),                   # nothing to attend
    (128, 40, 8, (1, 4096), 906, dict(waves_per_wg=1, max_resident_wgs=2)),
    (200, 28, 4, (1, 2000), 907, dict(waves_per_wg=4, max_resident_wgs=1)),
    (32, 32, 32, [2048] * 32, 908, {}),              # uniform: shares align with units
    (7, 64, 4, (1, 3000), 909, dict(waves_per_wg=8)),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_even_split_against_the_oracle(case):
    B, Hq, Hkv, lens, seed, kw = CASES[case]
    if isinstance(lens, tuple):
        x = gen.make_case(B, Hq, Hkv, None, seed=seed, ctx_range=lens, extra_pool_blocks=3,
                          poison=True)
    else:
        x = gen.make_case(B, Hq, Hkv, lens, seed=seed, extra_pool_blocks=3, poison=True)
    dev = to_device(x)
    plan = ops.plan(dev["q"], dev["k_cache"], dev["block_tables"], even_split=EVEN, **kw)
    print(f"[even] case {case}: B={B} Hq={Hq} Hkv={Hkv} plan={plan}", flush=True)
    assert plan["even_split"] == 1
    got = run(x, dev, even_split=EVEN, **kw)
    assert_close(got, oracle(x), f"even split case {case}")
    # every look-ahead mode on the same shares gives the same bits
    W, R = plan["waves_per_wg"], plan["resident_wgs"]
    for pf in (0, 1, 3, 4):
        kw2 = dict(prefetch=pf, even_split=EVEN, waves_per_wg=W, max_resident_wgs=R)
        try:
            ops.plan(dev["q"], dev["k_cache"], dev["block_tables"], **kw2)
        except ValueError:  # the LDS ring's slots do not fit beside 8 waves of 16 heads
            assert pf == 4
            continue
        o = run(x, dev, **kw2)
        assert np.array_equal(bits(o), bits(got)), f"mode {pf}"


def test_even_split_twice_with_fewer_blocks():
    """One workspace, filled with 0xFF bytes (NaN floats, -1 records), for a
    long batch, then a shorter one: every record the merge reads was written
    by the same call."""
    x1 = gen.make_case(32, 32, 8, None, seed=920, ctx_range=(2000, 8000))
    x2 = gen.make_case(32, 32, 8, None, seed=921, ctx_range=(1, 300), max_blocks_per_seq=500)
    devs = [to_device(x) for x in (x1, x2)]
    need = max(ops.workspace_bytes(d["q"], d["k_cache"], d["block_tables"], even_split=EVEN)
               for d in devs)
    ws = torch.full((need,), 255, dtype=torch.uint8, device="cuda")
    for x, dev in zip((x1, x2), devs):
        got = run(x, dev, even_split=EVEN, workspace=ws)
        assert_close(got, oracle(x), "even split, reused workspace")


@pytest.mark.parametrize("case", ["asked", "auto", "auto below C/2"])
def test_even_split_over_an_e4m3_cache(case):
    """Asked for (512 units), and taken by the auto plan (192 units over 256
    table blocks; and C/4 units of GQA 4/1, below the fp16 rule's C/2: 8
    waves, one block ahead)."""
    auto = case != "asked"
    B, Hq, Hkv = {"asked": (64, 32, 8), "auto": (24, 32, 8),
                  "auto below C/2": (nat.device_info()["compute_units"] // 4, 4, 1)}[case]
    print(f"[even e4m3] {case}: B={B} Hq={Hq} Hkv={Hkv}", flush=True)
    x8 = gen.to_fp8(gen.make_case(B, Hq, Hkv, None, seed=930 + B, ctx_range=(1, 4096),
                                  max_blocks_per_seq=256))
    d = {k: torch.from_numpy(getattr(x8, k)).cuda() for k in ("q", "block_tables", "context_lens")}
    d["k_cache"] = torch.from_numpy(gen.pack_k_fp8(x8.k8)).cuda()
    d["v_cache"] = torch.from_numpy(x8.v8).cuda()
    kw = {} if auto else dict(even_split=EVEN)
    plan = ops.plan(d["q"], d["k_cache"], d["block_tables"], **kw)
    assert plan["even_split"] == 1
    if auto and nat.device_info()["compute_units"] == 256:
        assert (plan["waves_per_wg"], plan["prefetch_distance"]) == (8, 1)
    dec = lambda **k2: ops.paged_attn_decode_fp8(
        d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["context_lens"], x8.scale,
        x8.k_scale, x8.v_scale, **kw, **k2).cpu().numpy()
    got = dec()
    ref = orc.paged_attention_fp8_f64(x8.q, x8.k8, x8.v8, x8.block_tables, x8.context_lens,
                                      x8.scale, x8.k_scale, x8.v_scale)
    assert_close(got, ref, "e4m3 even split")
    # the look-ahead two blocks ahead on the same shares: the same bits
    two = dec(prefetch=nat.PREFETCH_REG, prefetch_distance=2, even_split=EVEN,
              waves_per_wg=plan["waves_per_wg"]) if auto else dec(prefetch_distance=2)
    assert np.array_equal(bits(two), bits(got))


def test_even_split_without_allocation_matches_the_workspace_call():
    x = gen.make_case(48, 16, 4, None, seed=940, ctx_range=(1, 5000), extra_pool_blocks=2)
    dev = to_device(x)
    ref = run(x, dev, even_split=EVEN)
    out = torch.empty_like(dev["q"])
    ops.paged_attn_decode_noalloc(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                  dev["context_lens"], x.scale, out, even_split=EVEN)
    assert np.array_equal(bits(out.cpu().numpy()), bits(ref))


def test_even_split_timeline_and_checked_variant():
    x = gen.make_case(16, 8, 2, None, seed=950, ctx_range=(0, 3000))
    dev = to_device(x)
    plan = ops.plan(dev["q"], dev["k_cache"], dev["block_tables"], even_split=EVEN)
    tl = torch.zeros(plan["workgroups"], 4, dtype=torch.int64, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = run(x, dev, even_split=EVEN, debug_timeline=tl, debug_error_word=err)
    assert np.array_equal(bits(got), bits(run(x, dev, even_split=EVEN)))
    t = tl.cpu().numpy()
    assert (t[:, 0] > 0).all() and (t[:, 1] >= t[:, 0]).all()
    assert int(err.item()) == 0


@pytest.mark.parametrize("units_per_cu,MB", [(0.75, 256), (1, 160), (2, 200)])
def test_the_auto_plan_takes_the_even_split(units_per_cu, MB):
    """Ragged sequences x 8 KV heads from 3/4 to 2 units per CU over tables
    of 160..256 blocks: the auto plan is the even split, against the oracle
    and against the plan without it (another split of the same work)."""
    C = nat.device_info()["compute_units"]
    B = int(units_per_cu * C) // 8
    print(f"[even auto] B={B} MB={MB}", flush=True)
    x = gen.make_case(B, 16, 8, None, seed=960 + MB, ctx_range=(1, MB * 16),
                      max_blocks_per_seq=MB, poison=True)
    dev = to_device(x)
    plan = ops.plan(dev["q"], dev["k_cache"], dev["block_tables"])
    assert plan["even_split"] == 1 and plan["workgroups"] == C
    ref = oracle(x)
    assert_close(run(x, dev), ref, "auto even split")
    assert_close(run(x, dev, even_split=nat.EVEN_SPLIT_OFF), ref, "without the even split")
