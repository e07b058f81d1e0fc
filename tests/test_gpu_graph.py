"""The decode call captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: every replay must give the eager result's bits, also after the
inputs are changed in place and with the workspace overwritten between
replays (MI355X).  Plans: a split batch with the reduce, whole units, E4M3,
and the even split."""
import numpy as np
import pytest
import torch

from paged_kv_cache_226_amd import inputs as gen
from paged_kv_cache_226_amd import ops

from parity import bits, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(native_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _call(dev, scale, out, ws, fp8=None, pf=-1):
    if fp8 is not None:
        return ops.paged_attn_decode_fp8(dev["q"], dev["k_cache"], dev["v_cache"],
                                         dev["block_tables"], dev["context_lens"], scale,
                                         fp8[0], fp8[1], out, workspace=ws, prefetch=pf)
    return ops.paged_attn_decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                 dev["context_lens"], scale, out, workspace=ws, prefetch=pf)


@pytest.mark.parametrize("pf", [-1, 4])  # the default mode and the LDS ring
@pytest.mark.parametrize("case", ["split", "whole", "fp8", "even"])
def test_graph_replays_match_eager(case, pf):
    if case == "whole":  # 256 (sequence, KV head) pairs: one partition, no reduce
        x = gen.make_case(64, 16, 4, list(np.random.default_rng(1).integers(1, 300, 64)),
                          seed=501)
    elif case == "even":  # 192 pairs over 256 table blocks: the even split (default mode)
        x = gen.make_case(24, 16, 8, list(np.random.default_rng(2).integers(1, 4097, 24)),
                          seed=502, max_blocks_per_seq=256)
    else:                # 32 pairs: split contexts and the reduce kernel
        x = gen.make_case(4, 32, 8, [900, 33, 4000, 129], seed=500)
    fp8 = None
    if case == "fp8":
        x8 = gen.to_fp8(x)
        dev = {"q": torch.from_numpy(x8.q).cuda(),
               "k_cache": torch.from_numpy(gen.pack_k_fp8(x8.k8)).cuda(),
               "v_cache": torch.from_numpy(x8.v8).cuda(),
               "block_tables": torch.from_numpy(x8.block_tables).cuda(),
               "context_lens": torch.from_numpy(x8.context_lens).cuda()}
        fp8 = (x8.k_scale, x8.v_scale)
    else:
        dev = to_device(x)
    p = ops.plan(dev["q"], dev["k_cache"], dev["block_tables"], prefetch=pf)
    if case == "even":
        assert p["even_split"] == (pf == -1)
    else:
        assert (p["num_partitions"] > 1) == (case != "whole")
    out = torch.empty_like(dev["q"])
    ws = ops.new_workspace(dev["q"], dev["k_cache"], dev["block_tables"], prefetch=pf)
    eager = _call(dev, x.scale, out, ws, fp8, pf).clone()
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _call(dev, x.scale, out, ws, fp8, pf)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _call(dev, x.scale, out, ws, fp8, pf)
    for _ in range(5):
        out.fill_(1.0)   # eager work between the replays
        ws.fill_(0xFF)   # the workspace may hold anything
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out.cpu().numpy()), bits(eager.cpu().numpy()))

    # new inputs in the captured buffers: replay equals a fresh eager call
    dev["q"].mul_(-0.5)
    dev["context_lens"].sub_(1).clamp_(min=0)
    g.replay()
    torch.cuda.synchronize()
    replayed = out.clone()
    fresh = _call(dev, x.scale, torch.empty_like(out), ws, fp8, pf)
    torch.cuda.synchronize()
    assert np.array_equal(bits(replayed.cpu().numpy()), bits(fresh.cpu().numpy()))
    assert not np.array_equal(bits(replayed.cpu().numpy()), bits(eager.cpu().numpy()))
