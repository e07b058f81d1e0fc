"""Shared helpers for the GPU parity tests.

Tolerance: outputs are fp16, accumulation is fp32.
  abs  = max |gpu - ref|                               must be <= 2e-3
  rel  = max |gpu - ref| / max(|ref|, 1e-3)            must be <= 1e-2
The 1e-3 floor keeps near-zero outputs from making the relative error
meaningless: below it they must be right to 1e-5 absolute, which fp32
accumulation (~1e-7) plus fp16 output rounding (<= 4.9e-7 there) meets.
A row-normwise figure max_d|g - r| / max_d|r| is reported alongside.
"""
import numpy as np
import torch

from oracle import oracle as orc
from paged_kv_cache_226_amd import inputs as gen
from paged_kv_cache_226_amd import _native as nat
from paged_kv_cache_226_amd import ops

ABS_TOL = 2e-3
REL_TOL = 1e-2
REL_FLOOR = 1e-3


def to_device(x, device="cuda"):
    return dict(q=torch.from_numpy(x.q).to(device),
                k_cache=torch.from_numpy(gen.pack_k(x.k_cache)).to(device),
                v_cache=torch.from_numpy(x.v_cache).to(device),
                block_tables=torch.from_numpy(x.block_tables).to(device),
                context_lens=torch.from_numpy(x.context_lens).to(device))


def run(x, dev=None, **kw):
    """Run the HIP path on inputs x; returns fp16 numpy [B, Hq, D]."""
    d = dev if dev is not None else to_device(x)
    out = ops.paged_attn_decode(d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                d["context_lens"], x.scale, **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle(x):
    return orc.paged_attention_f64(x.q, x.k_cache, x.v_cache, x.block_tables,
                                   x.context_lens, x.scale)


def errors(got_f16, ref_f64):
    g = got_f16.astype(np.float64)
    diff = np.abs(g - ref_f64)
    ab = float(diff.max()) if diff.size else 0.0
    rel = float((diff / np.maximum(np.abs(ref_f64), REL_FLOOR)).max()) if diff.size else 0.0
    denom = np.abs(ref_f64).max(axis=-1)
    rn = float((diff.max(axis=-1) / np.maximum(denom, 1e-30)).max()) if diff.size else 0.0
    return dict(abs=ab, rel=rel, rel_norm=rn)


def assert_close(got_f16, ref_f64, what=""):
    assert np.isfinite(got_f16.astype(np.float32)).all(), f"non-finite output {what}"
    e = errors(got_f16, ref_f64)
    assert e["abs"] <= ABS_TOL and e["rel"] <= REL_TOL, f"{what}: {e}"
    return e


def bits(a):
    return np.ascontiguousarray(a).view(np.uint16)


def same_plan(plan, **extra):
    """Options that reproduce `plan` (waves, partitions, order) for another
    look-ahead mode: a balanced split is reproduced by asking for it again
    (auto partitions and order with the same waves), a fixed one by its
    partition size and order.  A residency cap is kept (it changes no bits,
    only how many work-groups share a CU).  An even split is asked for again
    with the same waves and residency (the shares follow from them)."""
    if plan["even_split"]:
        kw = dict(even_split=nat.EVEN_SPLIT_ON, waves_per_wg=plan["waves_per_wg"])
    elif plan["balanced"]:
        kw = dict(partition_blocks=0, waves_per_wg=plan["waves_per_wg"], seq_order=0,
                  even_split=nat.EVEN_SPLIT_OFF)
    else:
        kw = dict(partition_blocks=plan["partition_blocks"], waves_per_wg=plan["waves_per_wg"],
                  seq_order=plan["seq_order"], even_split=nat.EVEN_SPLIT_OFF)
    kw["max_resident_wgs"] = plan["resident_wgs"]
    kw.update(extra)
    return kw
