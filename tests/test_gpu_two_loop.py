"""The two-loop walk (all Q.K^T with a K look-ahead, then all P.V with a V
look-ahead) against the fp64 oracle (MI355X)."""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from paged_kv_cache_226_amd import inputs as gen
from paged_kv_cache_226_amd import ops

from parity import assert_close, bits, oracle, run, to_device

pytestmark = pytest.mark.gpu

MODES = [0, 1, 2, 3]
TWO = 1


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(native_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


CASES = [
    (300, 1, 1, 1, [1]),
    (301, 2, 2, 2, [15, 16]),
    (302, 3, 4, 4, [17, 31, 33]),
    (303, 2, 8, 4, [100, 257]),
    (304, 2, 7, 1, [321, 48]),
    (305, 3, 16, 4, [65, 130, 500]),
    (306, 1, 8, 1, [2049]),
    (307, 4, 32, 8, [600, 1, 16, 1025]),
    (308, 2, 32, 2, [777, 4096]),
]


@pytest.mark.parametrize("seed,B,Hq,Hkv,lens", CASES)
def test_two_loop_random_shapes_all_modes(seed, B, Hq, Hkv, lens):
    x = gen.make_case(B, Hq, Hkv, lens, seed=seed, extra_pool_blocks=3)
    ref = oracle(x)
    dev = to_device(x)
    outs = {pf: run(x, dev, prefetch=pf, structure=TWO) for pf in MODES}
    for pf, o in outs.items():
        assert_close(o, ref, f"two-loop {seed} pf={pf}")
        assert np.array_equal(bits(o), bits(outs[0])), f"mode {pf} differs from mode 0"


@pytest.mark.parametrize("waves", [1, 2, 4, 8])
@pytest.mark.parametrize("pb", [0, 1, 3, 8])
def test_two_loop_waves_and_partitions(waves, pb):
    x = gen.make_case(3, 8, 2, [700, 33, 1], seed=310, extra_pool_blocks=3)
    ref = oracle(x)
    dev = to_device(x)
    for pf in (0, 3):
        assert_close(run(x, dev, prefetch=pf, waves_per_wg=waves, partition_blocks=pb,
                         structure=TWO), ref, f"two-loop w={waves} pb={pb} pf={pf}")


def test_two_loop_poison_and_empty_contexts():
    x = gen.make_case(5, 8, 2, [200, 0, 31, 17, 64], seed=311, extra_pool_blocks=9)
    clean = {pf: run(x, prefetch=pf, structure=TWO) for pf in MODES}
    assert not clean[0][1].any()
    assert_close(clean[0], oracle(x), "two-loop clean")
    gen.apply_poison(x)
    for pf in MODES:
        dirty = run(x, prefetch=pf, structure=TWO)
        assert np.isfinite(dirty.astype(np.float32)).all()
        assert np.array_equal(bits(dirty), bits(clean[pf]))


def test_two_loop_context_one_gives_v0():
    x = gen.make_case(3, 8, 2, [1, 1, 1], seed=312, extra_pool_blocks=2)
    o = run(x, structure=TWO)
    for b in range(3):
        for h in range(8):
            assert np.array_equal(bits(o[b, h]), bits(x.v_cache[x.block_tables[b, 0], h // 4, 0]))


@pytest.mark.parametrize("name", ["llama2_7b", "llama3_8b"])
def test_two_loop_workload_full_output(name):
    print(f"[two-loop workload] {name}", flush=True)
    x = gen.make_inputs(name)
    dev = to_device(x)
    outs = {}
    for pf in MODES:
        outs[pf] = ops.paged_attn_decode(dev["q"], dev["k_cache"], dev["v_cache"],
                                         dev["block_tables"], dev["context_lens"], x.scale,
                                         prefetch=pf, structure=TWO)
        torch.cuda.synchronize()
        assert torch.equal(outs[pf].view(torch.int16), outs[0].view(torch.int16)), f"mode {pf}"
    got = outs[0].cpu().numpy()
    del dev, outs
    ref = orc.paged_attention_f64(x.q, x.k_cache, x.v_cache, x.block_tables, x.context_lens,
                                  x.scale)
    e = assert_close(got, ref, name)
    print(f"[two-loop workload] {name}: {e}", flush=True)
