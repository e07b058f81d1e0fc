"""E4M3 (FP8) KV caches on the GPU: parity with the fp64 E4M3 oracle (MI355X).

The oracle decodes each byte with its own E4M3 decoder and multiplies by the
per-tensor scale; the kernel widens bytes to fp16 with the hardware
conversion and folds the scales into the softmax scale and the output.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from oracle import schedule as sch
from paged_kv_cache_226_amd import inputs as gen
from paged_kv_cache_226_amd import ops

from parity import assert_close, bits, same_plan

pytestmark = pytest.mark.gpu

MODES = [0, 1, 2, 3, 4]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(native_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def to_device8(x8, device="cuda"):
    return dict(q=torch.from_numpy(x8.q).to(device),
                k_cache=torch.from_numpy(gen.pack_k_fp8(x8.k8)).to(device),
                v_cache=torch.from_numpy(x8.v8).to(device),
                block_tables=torch.from_numpy(x8.block_tables).to(device),
                context_lens=torch.from_numpy(x8.context_lens).to(device))


def run8(x8, dev=None, **kw):
    d = dev if dev is not None else to_device8(x8)
    out = ops.paged_attn_decode_fp8(d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                    d["context_lens"], x8.scale, x8.k_scale, x8.v_scale, **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle8(x8):
    return orc.paged_attention_fp8_f64(x8.q, x8.k8, x8.v8, x8.block_tables, x8.context_lens,
                                       x8.scale, x8.k_scale, x8.v_scale)


def case8(B, Hq, Hkv, lens, seed, extra=3, k_scale=gen.FP8_K_SCALE, v_scale=gen.FP8_V_SCALE):
    return gen.to_fp8(gen.make_case(B, Hq, Hkv, lens, seed=seed, extra_pool_blocks=extra),
                      k_scale, v_scale)


CASES = [
    (200, 1, 1, 1, [1]),
    (201, 2, 2, 2, [15, 16]),
    (202, 3, 4, 4, [17, 31, 33]),
    (203, 2, 8, 4, [100, 257]),
    (204, 2, 7, 1, [321, 48]),
    (205, 3, 16, 4, [65, 130, 500]),
    (206, 1, 8, 1, [2049]),
    (207, 4, 32, 8, [600, 1, 16, 1025]),
    (208, 2, 28, 4, [777, 4096]),
]


@pytest.mark.parametrize("seed,B,Hq,Hkv,lens", CASES)
def test_fp8_random_shapes_all_modes(seed, B, Hq, Hkv, lens):
    x8 = case8(B, Hq, Hkv, lens, seed)
    ref = oracle8(x8)
    dev = to_device8(x8)
    outs = {pf: run8(x8, dev, prefetch=pf) for pf in MODES}
    outs["reg2"] = run8(x8, dev, prefetch=2, prefetch_distance=2)
    for pf, o in outs.items():
        assert_close(o, ref, f"fp8 {seed} pf={pf}")
        assert np.array_equal(bits(o), bits(outs[0])), f"mode {pf} differs from mode 0"


@pytest.mark.parametrize("k_scale,v_scale", [(1.0, 1.0), (0.0375, 0.011), (2.0 ** -7, 0.5)])
def test_fp8_scales(k_scale, v_scale):
    """Non-power-of-two scales too: they enter the oracle as exact products."""
    x = gen.make_case(3, 8, 2, [300, 45, 1000], seed=210, extra_pool_blocks=2)
    # draws of N(0, 1) divided by the scale must stay inside E4M3's range
    x.k_cache = (x.k_cache.astype(np.float32) * min(1.0, 64 * k_scale)).astype(np.float16)
    x.v_cache = (x.v_cache.astype(np.float32) * min(1.0, 64 * v_scale)).astype(np.float16)
    x8 = gen.to_fp8(x, k_scale, v_scale)
    assert_close(run8(x8), oracle8(x8), f"k_scale={k_scale} v_scale={v_scale}")


@pytest.mark.parametrize("waves", [1, 2, 8])
@pytest.mark.parametrize("pb", [1, 3, 16])
def test_fp8_waves_and_partitions(waves, pb):
    x8 = case8(3, 8, 2, [700, 33, 1], seed=220)
    ref = oracle8(x8)
    dev = to_device8(x8)
    for pf in (0, 3, 4):
        assert_close(run8(x8, dev, prefetch=pf, waves_per_wg=waves, partition_blocks=pb), ref,
                     f"fp8 w={waves} pb={pb} pf={pf}")


def test_fp8_debug_gather_is_the_exact_widening():
    """The widened K the kernel computes on is exactly the E4M3 value of each
    gathered byte: pins the hardware conversion and the layout at once."""
    x8 = case8(3, 8, 2, [200, 31, 64], seed=230, extra=7)
    # every one of the 256 codes appears in the cache (NaN codes aside)
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    flat = x8.k8.reshape(-1)
    flat[: codes.size] = codes
    dev = to_device8(x8)
    B, MB = x8.block_tables.shape
    Hkv = x8.k8.shape[1]
    # block 0 (which holds the code table) becomes sequence 0's first block
    x8.block_tables[0, 0] = 0
    dev["block_tables"] = torch.from_numpy(x8.block_tables).cuda()
    dev["k_cache"] = torch.from_numpy(gen.pack_k_fp8(x8.k8)).cuda()
    for pf in MODES:
        dump = torch.full((B, Hkv, MB * 16, 128), float("nan"), dtype=torch.float16,
                          device="cuda")
        run8(x8, dev, prefetch=pf, debug_gather_k=dump, partition_blocks=4)
        got = dump.cpu().numpy()
        for b, L in enumerate(x8.context_lens):
            t = np.arange(L)
            want = gen.dequantize_e4m3_fp16(x8.k8[x8.block_tables[b, t // 16], :, t % 16, :])
            assert np.array_equal(bits(got[b, :, :L, :]), bits(np.transpose(want, (1, 0, 2)))), \
                f"b={b} pf={pf}"


def test_fp8_context_one_gives_scaled_v0_bitwise():
    x8 = case8(3, 8, 2, [1, 1, 1], seed=240, extra=2)
    for pf in MODES:
        o = run8(x8, prefetch=pf)
        for b in range(3):
            for h in range(8):
                v0 = gen.dequantize_e4m3_fp16(x8.v8[x8.block_tables[b, 0], h // 4, 0])
                want = (v0.astype(np.float64) * x8.v_scale).astype(np.float16)
                assert np.array_equal(bits(o[b, h]), bits(want))


def test_fp8_poison_gives_bitwise_clean_result():
    x = gen.make_case(4, 8, 2, [200, 31, 17, 64], seed=250, extra_pool_blocks=9)
    x8 = gen.to_fp8(x)
    clean = {pf: run8(x8, prefetch=pf) for pf in MODES}
    gen.apply_poison(x)
    p8 = gen.to_fp8(x)
    assert (p8.k8 == gen.FP8_NAN_BYTE).any() and (p8.v8 == gen.FP8_NAN_BYTE).any()
    for pf in MODES:
        dirty = run8(p8, prefetch=pf)
        assert np.isfinite(dirty.astype(np.float32)).all()
        assert np.array_equal(bits(dirty), bits(clean[pf]))


@pytest.mark.parametrize("pf", MODES)
def test_fp8_trace_follows_the_lookahead_schedule(pf):
    x8 = case8(3, 4, 2, [400, 90, 2000], seed=260, extra=2)
    dev = to_device8(x8)
    B, MB = x8.block_tables.shape
    Hkv = x8.k8.shape[1]
    trace = torch.full((B, Hkv, MB, 2), -1, dtype=torch.int32, device="cuda")
    run8(x8, dev, debug_trace=trace, prefetch=pf, partition_blocks=8)
    tr = trace.cpu().numpy()
    plan = ops.plan(dev["q"], dev["k_cache"], dev["block_tables"], prefetch=pf,
                    partition_blocks=8)
    W, PB = plan["waves_per_wg"], plan["partition_blocks"]
    for b, L in enumerate(x8.context_lens):
        nb = -(-int(L) // 16)
        for h in range(Hkv):
            for s in range(0, nb, PB):
                # the register and LDS rings over E4M3 run two blocks ahead by default
                exp = sch.expected_trace(s, min(nb, s + PB), W, 2 if pf in (2, 4) else 1)
                for j, (wave, it, fetcher) in exp.items():
                    assert tr[b, h, j, 0] == (wave << 16 | it), (b, h, j)
                    assert tr[b, h, j, 1] == (-1 if pf == 0 else fetcher), (b, h, j, pf)
        assert (tr[b, :, nb:, :] == -1).all()


@pytest.mark.parametrize("pf", MODES)
def test_fp8_debug_error_word_flags_a_bad_block_id(pf):
    x8 = case8(2, 4, 2, [40, 20], seed=270, extra=2)
    dev = to_device8(x8)
    dev["block_tables"][0, 1] = x8.k8.shape[0] + 1000
    dev["block_tables"][0, 2] = -7
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = ops.paged_attn_decode_fp8(dev["q"], dev["k_cache"], dev["v_cache"],
                                    dev["block_tables"], dev["context_lens"], x8.scale,
                                    x8.k_scale, x8.v_scale, debug_error_word=err, prefetch=pf)
    torch.cuda.synchronize()
    assert int(err.item()) & 1
    assert torch.isfinite(out.float()).all()


def test_fp8_float8_dtype_is_accepted_and_equal():
    x8 = case8(2, 8, 2, [100, 37], seed=280)
    dev = to_device8(x8)
    a = run8(x8, dev)
    dev8 = dict(dev, k_cache=dev["k_cache"].view(torch.float8_e4m3fn),
                v_cache=dev["v_cache"].view(torch.float8_e4m3fn))
    assert np.array_equal(bits(run8(x8, dev8)), bits(a))


def test_fp8_repeated_runs_are_bitwise_identical():
    x8 = case8(4, 32, 8, [900, 33, 4000, 129], seed=290, extra=0)
    dev = to_device8(x8)
    first = run8(x8, dev)
    for _ in range(9):
        assert np.array_equal(bits(run8(x8, dev)), bits(first))


@pytest.mark.parametrize("name", ["llama2_7b", "llama3_8b", "qwen25_7b", "qwen25_14b"])
def test_fp8_workload_full_output(name):
    print(f"[fp8 workload] {name}: generating", flush=True)
    x8 = gen.to_fp8(gen.make_inputs(name))
    dev = to_device8(x8)
    hint = int(x8.context_lens.min())
    print(f"[fp8 workload] {name}: decode (hint {hint})", flush=True)
    dec = lambda **kw: ops.paged_attn_decode_fp8(dev["q"], dev["k_cache"], dev["v_cache"],
                                                 dev["block_tables"], dev["context_lens"],
                                                 x8.scale, x8.k_scale, x8.v_scale, **kw)
    out = dec(min_context_hint=hint)
    plan = ops.plan(dev["q"], dev["k_cache"], dev["block_tables"], min_context_hint=hint)
    torch.cuda.synchronize()
    for pf, dist in ((0, 0), (1, 0), (3, 0), (2, 1), (2, 2)):
        o2 = dec(prefetch=pf, prefetch_distance=dist, **same_plan(plan))
        torch.cuda.synchronize()
        assert torch.equal(o2.view(torch.int16), out.view(torch.int16)), f"mode {pf}"
    no_hint = dec().cpu().numpy()
    # the LDS-staged look-ahead may plan fewer waves; on the same plan it
    # matches the register look-ahead bit for bit
    for dist in (1, 2):
        lds_plan = ops.plan(dev["q"], dev["k_cache"], dev["block_tables"], prefetch=4,
                            prefetch_distance=dist)
        same = same_plan(lds_plan, prefetch_distance=dist)
        lds = dec(prefetch=4, **same)
        reg = dec(prefetch=2, **same)
        torch.cuda.synchronize()
        assert torch.equal(lds.view(torch.int16), reg.view(torch.int16)), f"lds vs reg {same}"
    # the bench's launch: K and V side by side in one pool, prepared call
    ks, vs = gen.side_by_side(dev["k_cache"], dev["v_cache"])
    bench_out = torch.empty_like(out)
    call = ops.prepare_decode_fp8(dev["q"], ks, vs, dev["block_tables"], dev["context_lens"],
                                  x8.scale, x8.k_scale, x8.v_scale, bench_out,
                                  min_context_hint=hint)
    call()
    call()
    torch.cuda.synchronize()
    assert torch.equal(bench_out.view(torch.int16), out.view(torch.int16)), "side-by-side pool"
    del ks, vs, call, bench_out
    got, got_lds = out.cpu().numpy(), lds.cpu().numpy()
    del dev, out, lds, reg
    print(f"[fp8 workload] {name}: oracle on all {got.shape[0] * got.shape[1]} rows",
          flush=True)
    ref = orc.paged_attention_fp8_f64(x8.q, x8.k8, x8.v8, x8.block_tables, x8.context_lens,
                                      x8.scale, x8.k_scale, x8.v_scale)
    e = assert_close(got, ref, name)
    assert_close(got_lds, ref, name + " lds")
    assert_close(no_hint, ref, name + " without the hint")
    print(f"[fp8 workload] {name}: {e}", flush=True)


def test_fp8_longest_first_order_changes_no_bits():
    lens = [33, 700, 1, 0, 2100, 129, 700]
    x8 = case8(len(lens), 8, 2, lens, seed=295)
    dev = to_device8(x8)
    a = run8(x8, dev, seq_order=1)
    b = run8(x8, dev, seq_order=2)
    assert np.array_equal(bits(a), bits(b))
    assert_close(b, oracle8(x8), "fp8 order")
