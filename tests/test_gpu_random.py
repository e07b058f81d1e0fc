"""Seeded random configurations against the oracle (MI355X).

Each case draws a shape (batch, query and KV heads, ragged context lengths
with empty and partial-block sequences), a plan (partition size, waves), a
look-ahead mode and distance, a sequence order, a cache placement and the
cache type.  Every output element must be within tolerance of the fp64
oracle, and bitwise equal to the plain walk (no look-ahead) on the same
plan.  A second set asks for the even split on larger ragged batches."""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from paged_kv_cache_226_amd import _native as nat
from paged_kv_cache_226_amd import inputs as gen
from paged_kv_cache_226_amd import ops

from parity import assert_close, bits, same_plan

pytestmark = pytest.mark.gpu

N_CASES = 200


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(native_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def draw(seed):
    rng = np.random.default_rng(seed)
    Hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 16]))
    B = int(rng.integers(1, 9))
    lens = [int(rng.choice([0, 1, int(rng.integers(1, 2500)), 16 * int(rng.integers(1, 40))]))
            for _ in range(B)]
    if max(lens) == 0:
        lens[0] = 33
    pf = int(rng.choice([0, 1, 2, 3, 4]))
    dist = int(rng.choice([0, 1, 2])) if pf in (2, 4) else int(rng.choice([0, 1, 3]))
    return dict(B=B, Hq=Hkv * g, Hkv=Hkv, lens=lens, fp8=bool(rng.random() < 0.3),
                pf=pf, dist=dist, pb=int(rng.choice([0, 0, 1, 5, 16, 64])),
                waves=int(rng.choice([0, 0, 1, 2, 4, 8])), order=int(rng.choice([0, 1, 2])),
                layout=str(rng.choice(["dense", "adjacent", "padded"])),
                extra=int(rng.integers(0, 4)))


def place(kc, vc, layout):
    """The caches as views into a pool of the given placement."""
    if layout == "dense":
        return kc, vc
    NB, H = kc.shape[:2]
    n = kc[0, 0].numel()
    if layout == "adjacent":
        pool = torch.empty((NB, H, 2, n), dtype=kc.dtype, device=kc.device)
        pool[:, :, 0] = kc.reshape(NB, H, n)
        pool[:, :, 1] = vc.reshape(NB, H, n)
        return pool[:, :, 0].view(kc.shape), pool[:, :, 1].view(vc.shape)
    pad = 64 // kc.element_size()  # padded: 64 spare bytes after every slice
    kp = torch.zeros((NB, H, n + pad), dtype=kc.dtype, device=kc.device)
    vp = torch.zeros((NB, H, n + pad), dtype=vc.dtype, device=vc.device)
    kp[:, :, :n] = kc.reshape(NB, H, n)
    vp[:, :, :n] = vc.reshape(NB, H, n)
    return kp[:, :, :n].view(kc.shape), vp[:, :, :n].view(vc.shape)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_configuration(seed):
    c = draw(7000 + seed)
    print(f"[random] seed {7000 + seed}: {c}", flush=True)
    x = gen.make_case(c["B"], c["Hq"], c["Hkv"], c["lens"], seed=7000 + seed,
                      extra_pool_blocks=c["extra"])
    q = torch.from_numpy(x.q).cuda()
    bt = torch.from_numpy(x.block_tables).cuda()
    ctx = torch.from_numpy(x.context_lens).cuda()
    if c["fp8"]:
        x8 = gen.to_fp8(x)
        kc = torch.from_numpy(gen.pack_k_fp8(x8.k8)).cuda()
        vc = torch.from_numpy(x8.v8).cuda()
        ref = orc.paged_attention_fp8_f64(x8.q, x8.k8, x8.v8, x8.block_tables, x8.context_lens,
                                          x8.scale, x8.k_scale, x8.v_scale)
        dec = lambda k, v, **kw: ops.paged_attn_decode_fp8(q, k, v, bt, ctx, x8.scale,
                                                           x8.k_scale, x8.v_scale, **kw)
    else:
        kc = torch.from_numpy(gen.pack_k(x.k_cache)).cuda()
        vc = torch.from_numpy(x.v_cache).cuda()
        ref = orc.paged_attention_f64(x.q, x.k_cache, x.v_cache, x.block_tables,
                                      x.context_lens, x.scale)
        dec = lambda k, v, **kw: ops.paged_attn_decode(q, k, v, bt, ctx, x.scale, **kw)
    k, v = place(kc, vc, c["layout"])
    kw = dict(partition_blocks=c["pb"], waves_per_wg=c["waves"], seq_order=c["order"])
    try:
        plan = ops.plan(q, k, bt, prefetch=c["pf"], prefetch_distance=c["dist"], **kw)
    except ValueError as e:  # an option the plan rejects (e.g. LDS slots for 8 waves)
        assert "unsupported" in str(e), e
        with pytest.raises(RuntimeError, match="unsupported"):
            dec(k, v, prefetch=c["pf"], prefetch_distance=c["dist"], **kw)
        return
    got = dec(k, v, prefetch=c["pf"], prefetch_distance=c["dist"], **kw)
    same = same_plan(plan)
    plain = dec(k, v, prefetch=0, **same)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    assert_close(got, ref, f"seed {7000 + seed} {c}")
    assert np.array_equal(bits(got), bits(plain.cpu().numpy())), f"seed {7000 + seed} {c}"


def draw_even(seed):
    rng = np.random.default_rng(seed)
    Hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 5, 7, 8]))
    B = int(rng.integers(1, 49))
    lens = [int(rng.choice([0, 1, int(rng.integers(1, 3000)), 16 * int(rng.integers(1, 120))]))
            for _ in range(B)]
    if max(lens) == 0:
        lens[0] = 17
    pf = int(rng.choice([0, 1, 2, 3, 4]))
    return dict(B=B, Hq=Hkv * g, Hkv=Hkv, lens=lens, fp8=bool(rng.random() < 0.3), pf=pf,
                dist=int(rng.choice([0, 1, 2])) if pf in (2, 4) else 0,
                waves=int(rng.choice([0, 1, 2, 4, 8])), cap=int(rng.choice([0, 1, 2, 3])),
                layout=str(rng.choice(["dense", "adjacent", "padded"])),
                extra=int(rng.integers(0, 4)))


@pytest.mark.parametrize("seed", range(60))
def test_random_even_split(seed):
    """The even split asked for on random ragged batches (empty sequences,
    one-token ones, tables of 1..120 blocks, 1 to 3 shares per CU): within
    tolerance of the oracle, and bitwise equal to the walk without the
    look-ahead over the same shares."""
    c = draw_even(9000 + seed)
    print(f"[random even] seed {9000 + seed}: {c}", flush=True)
    x = gen.make_case(c["B"], c["Hq"], c["Hkv"], c["lens"], seed=9000 + seed,
                      extra_pool_blocks=c["extra"], poison=True)
    q = torch.from_numpy(x.q).cuda()
    bt = torch.from_numpy(x.block_tables).cuda()
    ctx = torch.from_numpy(x.context_lens).cuda()
    if c["fp8"]:
        x8 = gen.to_fp8(x)
        kc = torch.from_numpy(gen.pack_k_fp8(x8.k8)).cuda()
        vc = torch.from_numpy(x8.v8).cuda()
        ref = orc.paged_attention_fp8_f64(x8.q, x8.k8, x8.v8, x8.block_tables, x8.context_lens,
                                          x8.scale, x8.k_scale, x8.v_scale)
        dec = lambda k, v, **kw: ops.paged_attn_decode_fp8(q, k, v, bt, ctx, x8.scale,
                                                           x8.k_scale, x8.v_scale, **kw)
    else:
        kc = torch.from_numpy(gen.pack_k(x.k_cache)).cuda()
        vc = torch.from_numpy(x.v_cache).cuda()
        ref = orc.paged_attention_f64(x.q, x.k_cache, x.v_cache, x.block_tables,
                                      x.context_lens, x.scale)
        dec = lambda k, v, **kw: ops.paged_attn_decode(q, k, v, bt, ctx, x.scale, **kw)
    k, v = place(kc, vc, c["layout"])
    kw = dict(even_split=nat.EVEN_SPLIT_ON, waves_per_wg=c["waves"],
              max_resident_wgs=c["cap"])
    try:
        plan = ops.plan(q, k, bt, prefetch=c["pf"], prefetch_distance=c["dist"], **kw)
    except ValueError as e:  # e.g. LDS ring slots for 8 waves of 16 heads
        assert "unsupported" in str(e), e
        return
    assert plan["even_split"] == 1
    got = dec(k, v, prefetch=c["pf"], prefetch_distance=c["dist"], **kw).cpu().numpy()
    plain = dec(k, v, prefetch=0, even_split=nat.EVEN_SPLIT_ON,
                waves_per_wg=plan["waves_per_wg"], max_resident_wgs=plan["resident_wgs"])
    torch.cuda.synchronize()
    assert_close(got, ref, f"seed {9000 + seed} {c}")
    assert np.array_equal(bits(got), bits(plain.cpu().numpy())), f"seed {9000 + seed} {c}"
