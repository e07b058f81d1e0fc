"""Seeded synthetic inputs for paged decode attention.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  Both the HIP path (through the tests and the bench)
and the CPU oracle are fed from it.

Workloads follow the attention shapes of the four models the asynchronous-KV-
prefetch review evaluates (section 5.1 model table: Llama2-7B MHA 32:32,
Llama3-8B GQA 32:8, Qwen2.5-7B GQA 28:4, Qwen2.5-14B GQA 40:8) with FP16 KV
(section 5.1 setup) in 16-token blocks of head_dim 128 (section 4.2).  The
review measures inside vLLM on real model weights and prompts; none of that
is available or needed here: Q, K and V are N(0, 1) draws and the block
tables are seeded permutations of the physical pool, which gives the same
shapes, sizes and scattered-block access pattern.

Draw order per workload (numpy PCG64 seeded with the workload's seed):
  1. ragged context lengths, if the workload has them: integers in [lo, hi];
  2. a permutation of the physical pool; sequence b takes the next
     ceil(ctx_b / block_size) entries, padding is -1;
  3. Q: standard normal float32, rounded to fp16;
  4. the whole K pool, then the whole V pool, the same way (in chunks;
     chunking does not change the stream).
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

HEAD_DIM = 128
BLOCK_SIZE = 16
FP16_NAN_BITS = 0x7E00
_CHUNK = 1 << 24


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    seed: int
    context_lens: Optional[Tuple[int, ...]] = None  # fixed lengths, one per sequence
    ctx_range: Optional[Tuple[int, int]] = None     # ragged: uniform integers, inclusive
    pool_blocks: Optional[int] = None               # None: exactly the blocks in use
    max_blocks_per_seq: Optional[int] = None        # None: the longest sequence's blocks
    head_dim: int = HEAD_DIM
    block_size: int = BLOCK_SIZE
    description: str = ""

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


def _fixed(n: int, ctx: int) -> Tuple[int, ...]:
    return tuple([ctx] * n)


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny", 2, 4, 4, seed=0, context_lens=(256, 200), pool_blocks=64,
                 description="batch 2, 4 Q = 4 KV heads, contexts 256 and 200, "
                             "blocks scattered in a 64-block pool"),
        Workload("llama2_7b", 32, 32, 32, seed=1, context_lens=_fixed(32, 2048),
                 pool_blocks=4096,
                 description="Llama2-7B-shaped MHA layer: batch 32, 32 Q = 32 KV "
                             "heads, every context 2048 tokens, 4096-block pool"),
        Workload("llama3_8b", 64, 32, 8, seed=2, ctx_range=(512, 8192),
                 max_blocks_per_seq=512,
                 description="Llama3-8B-shaped GQA 4:1 layer: batch 64, 32 Q / 8 "
                             "KV heads, ragged contexts uniform in [512, 8192]"),
        Workload("qwen25_7b", 128, 28, 4, seed=3, context_lens=_fixed(128, 4096),
                 description="Qwen2.5-7B-shaped GQA 7:1 layer: batch 128, 28 Q / 4 "
                             "KV heads, every context 4096 tokens"),
        Workload("qwen25_14b", 128, 40, 8, seed=4, context_lens=_fixed(128, 8192),
                 description="Qwen2.5-14B-shaped GQA 5:1 layer: batch 128, 40 Q / 8 "
                             "KV heads, every context 8192 tokens (4 GiB of KV)"),
    ]
}

# One GPU's share of a tensor-parallel layer (the review's section 5.5 runs
# Llama3-8B and Qwen2.5-14B at TP 2, 4 and 8): the KV heads, their query
# heads and their pool are split evenly, the batch and the contexts are not.
# Same seeds as the full layer, so the context lengths match it.
for _base, _tp in [(b, t) for b in ("llama3_8b", "qwen25_14b") for t in (2, 4, 8)]:
    _w = WORKLOADS[_base]
    WORKLOADS[f"{_base}_tp{_tp}"] = dataclasses.replace(
        _w, name=f"{_base}_tp{_tp}", num_q_heads=_w.num_q_heads // _tp,
        num_kv_heads=_w.num_kv_heads // _tp,
        description=f"one GPU of {_base} at tensor parallelism {_tp}: "
                    f"{_w.num_q_heads // _tp} Q / {_w.num_kv_heads // _tp} KV heads")


@dataclasses.dataclass
class PagedInputs:
    q: np.ndarray             # fp16 [B, Hq, D]
    k_cache: np.ndarray       # fp16 [NB, Hkv, T, D]
    v_cache: np.ndarray       # fp16 [NB, Hkv, T, D]
    block_tables: np.ndarray  # int32 [B, MB], -1 padding
    context_lens: np.ndarray  # int32 [B]
    scale: float              # fp32 value, 1/sqrt(D)
    name: str = "case"

    @property
    def shape(self) -> Dict[str, int]:
        B, Hq, D = self.q.shape
        NB, Hkv, T, _ = self.k_cache.shape
        return dict(num_seqs=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                    block_size=T, max_blocks_per_seq=self.block_tables.shape[1],
                    num_blocks=NB)


def blocks_for(ctx: int, block_size: int = BLOCK_SIZE) -> int:
    return max(0, -(-int(ctx) // block_size))


def _fill_normal(rng: np.random.Generator, out: np.ndarray) -> None:
    flat = out.reshape(-1)
    for i in range(0, flat.size, _CHUNK):
        n = min(_CHUNK, flat.size - i)
        flat[i:i + n] = rng.standard_normal(n, dtype=np.float32)


def _layout(rng, ctx: Sequence[int], block_size: int, pool_blocks: Optional[int],
            max_blocks: Optional[int]):
    nbs = [blocks_for(c, block_size) for c in ctx]
    used = sum(nbs)
    NB = used if pool_blocks is None else int(pool_blocks)
    if NB < used:
        raise ValueError(f"pool of {NB} blocks cannot hold {used}")
    MB = max([1] + nbs) if max_blocks is None else int(max_blocks)
    if MB < max(nbs, default=0):
        raise ValueError("max_blocks_per_seq smaller than the longest sequence")
    perm = rng.permutation(NB).astype(np.int32)
    bt = np.full((len(ctx), MB), -1, dtype=np.int32)
    off = 0
    for b, nb in enumerate(nbs):
        bt[b, :nb] = perm[off:off + nb]
        off += nb
    return bt, NB


def make_case(num_seqs: int, num_q_heads: int, num_kv_heads: int,
              context_lens: Sequence[int], seed: int, *, head_dim: int = HEAD_DIM,
              block_size: int = BLOCK_SIZE, pool_blocks: Optional[int] = None,
              extra_pool_blocks: int = 0, max_blocks_per_seq: Optional[int] = None,
              ctx_range: Optional[Tuple[int, int]] = None, poison: bool = False,
              name: str = "case") -> PagedInputs:
    """Draw one input set.  With ctx_range, context_lens is ignored and the
    lengths are drawn first.  poison=True fills every byte the attention must
    never read (unused pool blocks, slots past the context in a sequence's
    last block) with fp16 NaN; block-table padding is -1 either way."""
    if num_q_heads % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    rng = np.random.default_rng(seed)
    if ctx_range is not None:
        lo, hi = ctx_range
        ctx = rng.integers(lo, hi + 1, size=num_seqs).astype(np.int32)
    else:
        ctx = np.asarray(context_lens, dtype=np.int32).reshape(num_seqs)
    if pool_blocks is None and extra_pool_blocks:
        pool_blocks = sum(blocks_for(c, block_size) for c in ctx) + extra_pool_blocks
    bt, NB = _layout(rng, ctx.tolist(), block_size, pool_blocks, max_blocks_per_seq)
    q = np.empty((num_seqs, num_q_heads, head_dim), dtype=np.float16)
    _fill_normal(rng, q)
    k = np.empty((NB, num_kv_heads, block_size, head_dim), dtype=np.float16)
    _fill_normal(rng, k)
    v = np.empty_like(k)
    _fill_normal(rng, v)
    scale = float(np.float32(1.0 / np.sqrt(head_dim)))
    out = PagedInputs(q, k, v, bt, ctx, scale, name)
    if poison:
        apply_poison(out)
    return out


@dataclasses.dataclass
class PagedInputsFP8:
    q: np.ndarray             # fp16 [B, Hq, D]
    k8: np.ndarray            # uint8 E4M3 [NB, Hkv, T, D] (token-major, logical)
    v8: np.ndarray            # uint8 E4M3 [NB, Hkv, T, D]
    block_tables: np.ndarray  # int32 [B, MB]
    context_lens: np.ndarray  # int32 [B]
    scale: float
    k_scale: float            # a cached K value is decode(byte) * k_scale
    v_scale: float
    name: str = "case_fp8"


# Per-tensor scales of the synthetic FP8 caches: powers of two, so a value
# N(0, 1) / scale stays below E4M3's 448 with a wide margin and every
# dequantized value is exact in fp16.
FP8_K_SCALE = 2.0 ** -5
FP8_V_SCALE = 2.0 ** -5
FP8_NAN_BYTE = 0x7F


def quantize_e4m3(x: np.ndarray, scale: float) -> np.ndarray:
    """x / scale rounded to OCP FP8 E4M3 (torch's float8_e4m3fn conversion,
    round to nearest even), returned as uint8 codes."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32) / np.float32(scale))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def dequantize_e4m3_fp16(codes: np.ndarray) -> np.ndarray:
    """E4M3 codes to fp16 (exact: E4M3 is a subset of fp16), before scaling."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(
        torch.float8_e4m3fn).to(torch.float16).numpy()


def to_fp8(x: PagedInputs, k_scale: float = FP8_K_SCALE,
           v_scale: float = FP8_V_SCALE) -> PagedInputsFP8:
    """The same draw as an E4M3 cache: K and V quantized with the scales (NaN
    fp16 poison becomes the E4M3 NaN code)."""
    k8 = quantize_e4m3(x.k_cache.astype(np.float32), k_scale)
    v8 = quantize_e4m3(x.v_cache.astype(np.float32), v_scale)
    k8[np.isnan(x.k_cache)] = FP8_NAN_BYTE
    v8[np.isnan(x.v_cache)] = FP8_NAN_BYTE
    return PagedInputsFP8(x.q, k8, v8, x.block_tables, x.context_lens, x.scale,
                          float(k_scale), float(v_scale), x.name + "_fp8")


def pack_k_fp8(k8: np.ndarray) -> np.ndarray:
    """E4M3 K pool in the kernel's layout [NB][Hkv][D/16][T][16]: a 16-byte
    piece holds dims 16g..16g+15 of one token; pure reindexing."""
    NB, H, T, D = k8.shape
    return np.ascontiguousarray(k8.reshape(NB, H, T, D // 16, 16).transpose(0, 1, 3, 2, 4))


def unpack_k_fp8(kp: np.ndarray) -> np.ndarray:
    NB, H, G16, T, X = kp.shape
    return np.ascontiguousarray(kp.transpose(0, 1, 3, 2, 4).reshape(NB, H, T, G16 * X))


def make_inputs(workload, *, poison: bool = False) -> PagedInputs:
    """Inputs of a named workload (a key of WORKLOADS or a Workload)."""
    w = WORKLOADS[workload] if isinstance(workload, str) else workload
    return make_case(w.num_seqs, w.num_q_heads, w.num_kv_heads,
                     w.context_lens or (), w.seed, head_dim=w.head_dim,
                     block_size=w.block_size, pool_blocks=w.pool_blocks,
                     max_blocks_per_seq=w.max_blocks_per_seq, ctx_range=w.ctx_range,
                     poison=poison, name=w.name)


def workload_context_lens(workload) -> np.ndarray:
    """The context lengths make_inputs(workload) draws, without drawing the
    pools (the lengths are the first draw of the seeded stream)."""
    w = WORKLOADS[workload] if isinstance(workload, str) else workload
    if w.ctx_range is not None:
        rng = np.random.default_rng(w.seed)
        lo, hi = w.ctx_range
        return rng.integers(lo, hi + 1, size=w.num_seqs).astype(np.int32)
    return np.asarray(w.context_lens, dtype=np.int32)


def apply_poison(x: PagedInputs) -> None:
    """NaN into every pool byte that no (sequence, token < ctx) refers to."""
    T = x.k_cache.shape[2]
    used = np.zeros(x.k_cache.shape[0], dtype=bool)
    nan = np.array([FP16_NAN_BITS], dtype=np.uint16).view(np.float16)[0]
    for b, c in enumerate(x.context_lens.tolist()):
        nb = blocks_for(c, T)
        ids = x.block_tables[b, :nb]
        used[ids] = True
        if nb and c % T:
            last = ids[-1]
            x.k_cache[last, :, c % T:, :] = nan
            x.v_cache[last, :, c % T:, :] = nan
    x.k_cache[~used] = nan
    x.v_cache[~used] = nan


def pack_k(k_cache: np.ndarray) -> np.ndarray:
    """K pool in the kernel's layout [NB][Hkv][D/8][T][8]: inside a 4 KiB
    (block, head) slice, the 16 tokens' values of dims 8g..8g+7 are 256
    contiguous bytes (group g), so one 16-byte piece holds 8 dims of one
    token.  A pure reindexing: unpack_k(pack_k(k)) == k bit for bit."""
    NB, H, T, D = k_cache.shape
    return np.ascontiguousarray(
        k_cache.reshape(NB, H, T, D // 8, 8).transpose(0, 1, 3, 2, 4))


def unpack_k(k_packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_k: back to token-major [NB][Hkv][T][D]."""
    NB, H, G8, T, X = k_packed.shape
    return np.ascontiguousarray(k_packed.transpose(0, 1, 3, 2, 4).reshape(NB, H, T, G8 * X))


def digests(x: PagedInputs) -> Dict[str, str]:
    """SHA-256 of every array, to log which exact inputs a result came from."""
    out = {}
    for k in ("q", "k_cache", "v_cache", "block_tables", "context_lens"):
        out[k] = hashlib.sha256(np.ascontiguousarray(getattr(x, k)).tobytes()).hexdigest()
    return out


def make_case_device(num_seqs: int, num_q_heads: int, num_kv_heads: int, context_len: int,
                     seed: int, device="cuda", head_dim: int = HEAD_DIM,
                     block_size: int = BLOCK_SIZE) -> Dict[str, object]:
    """Large inputs drawn directly in device memory (torch's seeded generator
    on the device), for sweeps whose pools are too big to draw on the host.
    Every sequence has `context_len` tokens; the pool holds exactly the
    blocks in use, shuffled.  K is drawn in the kernel's grouped layout
    (pack_k's layout; the values are i.i.d., so drawing them grouped is the
    same distribution).  Draw order: permutation, Q, K pool, V pool."""
    import torch

    nb = blocks_for(context_len, block_size)
    NB = num_seqs * nb
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    perm = torch.randperm(NB, generator=g, device=device, dtype=torch.int64)
    bt = perm.to(torch.int32).reshape(num_seqs, nb).contiguous()
    ctx = torch.full((num_seqs,), context_len, dtype=torch.int32, device=device)

    def normal(shape):
        out = torch.empty(shape, dtype=torch.float16, device=device)
        flat = out.view(-1)
        for i in range(0, flat.numel(), _CHUNK):
            n = min(_CHUNK, flat.numel() - i)
            flat[i:i + n] = torch.randn(n, generator=g, device=device, dtype=torch.float32)
        return out

    q = normal((num_seqs, num_q_heads, head_dim))
    k = normal((NB, num_kv_heads, head_dim // 8, block_size, 8))
    v = normal((NB, num_kv_heads, block_size, head_dim))
    scale = float(np.float32(1.0 / np.sqrt(head_dim)))
    return dict(q=q, k_cache=k, v_cache=v, block_tables=bt, context_lens=ctx, scale=scale)


def side_by_side(k_cache, v_cache):
    """Device views (k, v) into one new pool [NB][Hkv][2][slice] in which
    each (block, KV head)'s K slice is followed by its V slice; the values
    are copied from the given dense caches (K in the kernel's packed layout,
    V token-major, fp16 or E4M3 bytes).  The views keep the dense shapes and
    carry the pool's block and head strides."""
    import torch

    NB, H = k_cache.shape[:2]
    n = k_cache[0, 0].numel()
    if v_cache.shape[:2] != k_cache.shape[:2] or v_cache[0, 0].numel() != n:
        raise ValueError("K and V caches must have the same pool shape and slice size")
    pool = torch.empty((NB, H, 2, n), dtype=k_cache.dtype, device=k_cache.device)
    pool[:, :, 0] = k_cache.reshape(NB, H, n)
    pool[:, :, 1] = v_cache.reshape(NB, H, n)
    return pool[:, :, 0].view(k_cache.shape), pool[:, :, 1].view(v_cache.shape)


def host_subset(dev_case: Dict[str, object], seqs: Sequence[int]) -> PagedInputs:
    """Copy the given sequences of a device case back to the host as a small
    PagedInputs (their blocks only, renumbered, K unpacked to token-major),
    so the CPU oracle can check those rows."""
    import torch

    bt = dev_case["block_tables"][list(seqs)].cpu().numpy()
    ctx = dev_case["context_lens"][list(seqs)].cpu().numpy().astype(np.int32)
    used = sorted(set(int(v) for v in bt[bt >= 0].ravel()))
    remap = {p: i for i, p in enumerate(used)}
    idx = torch.tensor(used, dtype=torch.int64, device=dev_case["k_cache"].device)
    kp = dev_case["k_cache"].index_select(0, idx).cpu().numpy()
    v = dev_case["v_cache"].index_select(0, idx).cpu().numpy()
    bt2 = np.vectorize(lambda p: remap.get(int(p), -1))(bt).astype(np.int32)
    q = dev_case["q"][list(seqs)].cpu().numpy()
    return PagedInputs(q, unpack_k(kp), v, bt2, ctx, dev_case["scale"], "subset")
