"""PyTorch-facing binding of the paged decode-attention library.

Argument marshalling only: shapes, dtypes and devices are checked, device
pointers and the current HIP stream are handed to libpaged_attn.so, and every
step of the computation runs in the HIP kernels.  torch supplies device
memory (including the partition workspace) and streams.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _native as nat


def _stream_handle(stream: Optional[torch.cuda.Stream], device: torch.device) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    if s.device != device:
        raise ValueError(f"the stream is on {s.device}, the tensors on {device}")
    return ctypes.c_void_p(s.cuda_stream)


def _same_device(index: int, **tensors):
    for name, t in tensors.items():
        if t is not None and t.get_device() != index:
            raise ValueError(f"{name} is on {t.device}, q on cuda:{index}")


def _check(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-d tensor")


def _slice_contiguous(t: torch.Tensor) -> bool:
    """Dims 2.. (one (block, head) slice) contiguous; dims 0-1 may be strided."""
    expect = 1
    for d in range(t.dim() - 1, 1, -1):
        if t.shape[d] != 1 and t.stride(d) != expect:
            return False
        expect *= t.shape[d]
    return True


def _pool_strides_nonzero(t: torch.Tensor, name: str):
    """A zero byte stride means 'dense' to the library, so a pool whose block
    or head dimension is a broadcast (stride 0, e.g. from expand) would be read
    as a dense pool of that many distinct slices: refuse it."""
    for d in (0, 1):
        if t.shape[d] > 1 and t.stride(d) == 0:
            raise ValueError(f"{name} has stride 0 over dimension {d} (a broadcast view); "
                             "the cache needs one slice per (block, head)")


def check_debug_shapes(B: int, Hkv: int, MB: int, debug_gather_k=None, debug_trace=None,
                       debug_error_word=None):
    """The debug outputs must be exactly as large as the kernel writes them:
    debug_gather_k [B, Hkv, MB*16, 128], debug_trace [B, Hkv, MB, 2], and at
    least one error word."""
    if debug_gather_k is not None and tuple(debug_gather_k.shape) != (B, Hkv, MB * 16, 128):
        raise ValueError(f"debug_gather_k must be [{B}, {Hkv}, {MB * 16}, 128], got "
                         f"{list(debug_gather_k.shape)}")
    if debug_trace is not None and tuple(debug_trace.shape) != (B, Hkv, MB, 2):
        raise ValueError(f"debug_trace must be [{B}, {Hkv}, {MB}, 2], got "
                         f"{list(debug_trace.shape)}")
    if debug_error_word is not None and debug_error_word.numel() < 1:
        raise ValueError("debug_error_word must hold at least one int32")


def check_debug_timeline(debug_timeline, workgroups: int):
    """The timeline holds one int64 row of 4 per decode work-group of the plan."""
    if debug_timeline is None:
        return
    if debug_timeline.dtype != torch.int64 or tuple(debug_timeline.shape) != (workgroups, 4):
        raise ValueError(f"debug_timeline must be int64 [{workgroups}, 4] (the plan's "
                         f"work-groups), got {debug_timeline.dtype} {list(debug_timeline.shape)}")


def shape_of(q: torch.Tensor, k_cache: torch.Tensor, block_tables: torch.Tensor,
             v_cache: Optional[torch.Tensor] = None) -> nat.PaShape:
    """pa_shape of these tensors; K and V may be views into a larger pool
    (their strides over blocks and heads are passed on in bytes).  A one-byte
    K cache is E4M3."""
    B, Hq, D = q.shape
    NB, Hkv, G8, T, X = k_cache.shape
    _pool_strides_nonzero(k_cache, "k_cache")
    if v_cache is not None:
        _pool_strides_nonzero(v_cache, "v_cache")
    ek = k_cache.element_size()
    kw0 = dict(kv_dtype=nat.KV_E4M3 if ek == 1 else nat.KV_F16)
    kw = dict(k_block_stride=k_cache.stride(0) * ek, k_head_stride=k_cache.stride(1) * ek)
    if v_cache is not None:
        ev = v_cache.element_size()
        kw.update(v_block_stride=v_cache.stride(0) * ev, v_head_stride=v_cache.stride(1) * ev)
    return nat.make_shape(B, Hq, Hkv, block_tables.shape[1], NB, head_dim=G8 * X, block_size=T,
                          **kw0, **kw)


def options(prefetch: int = -1, partition_blocks: int = 0, waves_per_wg: int = 0,
            prefetch_distance: int = 0, seq_order: int = 0, structure: int = 0,
            debug_gather_k: Optional[torch.Tensor] = None,
            debug_trace: Optional[torch.Tensor] = None,
            debug_error_word: Optional[torch.Tensor] = None, *,
            min_context_hint: int = 0, max_resident_wgs: int = 0,
            debug_timeline: Optional[torch.Tensor] = None,
            even_split: int = 0) -> nat.PaOptions:
    """pa_options for these settings (any debug tensor selects the checked
    kernel variant).  min_context_hint: a lower bound on every context length
    (tokens) that the caller knows, 0 = none; it only steers the auto plan."""
    o = nat.default_options()
    o.prefetch = int(prefetch)
    o.partition_blocks = int(partition_blocks)
    o.waves_per_wg = int(waves_per_wg)
    o.prefetch_distance = int(prefetch_distance)
    o.seq_order = int(seq_order)
    o.structure = int(structure)
    o.min_context_hint = int(min_context_hint)
    o.max_resident_wgs = int(max_resident_wgs)
    o.even_split = int(even_split)
    if debug_gather_k is not None:
        _check(debug_gather_k, "debug_gather_k", torch.float16, 4)
        o.debug_gather_k = debug_gather_k.data_ptr()
    if debug_trace is not None:
        _check(debug_trace, "debug_trace", torch.int32, 4)
        o.debug_trace = debug_trace.data_ptr()
    if debug_error_word is not None:
        _check(debug_error_word, "debug_error_word", torch.int32, 1)
        o.debug_error_word = debug_error_word.data_ptr()
    if debug_timeline is not None:
        _check(debug_timeline, "debug_timeline", torch.int64, 2)
        o.debug_timeline = debug_timeline.data_ptr()
    return o


def plan(q, k_cache, block_tables, **kw) -> dict:
    return nat.plan(shape_of(q, k_cache, block_tables), options(**kw))


def new_workspace(q, k_cache, block_tables, **kw) -> torch.Tensor:
    """A workspace for this shape and these options (reusable by every later
    call with the same plan; calls must not overlap on it)."""
    n = workspace_bytes(q, k_cache, block_tables, **kw)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=q.device)


def workspace_bytes(q, k_cache, block_tables, **kw) -> int:
    sh = shape_of(q, k_cache, block_tables)
    return int(nat.lib().paged_attn_workspace_size(ctypes.byref(sh), ctypes.byref(options(**kw))))


def _check_kv(t: torch.Tensor, name: str, fp8: bool, ndim: int):
    """A cache: the right dtype and rank, each (block, head) slice contiguous
    (the pool itself may be a strided view)."""
    if fp8 and isinstance(t, torch.Tensor) and t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    want = torch.uint8 if fp8 else torch.float16
    if t.dtype != want:
        raise TypeError(f"{name} must be {want}, got {t.dtype}")
    if t.dim() != ndim or not _slice_contiguous(t):
        raise ValueError(f"{name} must be a {ndim}-d tensor whose (block, head) slices are "
                         "contiguous")


class DecodeCall:
    """One decode call, validated and marshalled once.

    Calling it runs the step again on the same tensors, whose contents may
    change between calls (their storage and shapes may not); it allocates
    nothing and costs one C call, about what a C caller of the library pays.
    The stream is the one given, or the device's current stream when the
    call was prepared.  Calls on one DecodeCall must not overlap (they share
    its workspace).  With noalloc, the call goes to paged_attn_decode_noalloc,
    whose partials live in the library's per-device scratch array: no
    workspace is allocated or taken, and calls that overlap on one GPU race."""

    def __init__(self, fp8: bool, q, k_cache, v_cache, block_tables, context_lens, scale,
                 k_scale, v_scale, out, prefetch, partition_blocks, waves_per_wg,
                 prefetch_distance, seq_order, structure, workspace, debug_gather_k,
                 debug_trace, debug_error_word, stream, noalloc: bool = False,
                 min_context_hint: int = 0, max_resident_wgs: int = 0,
                 debug_timeline: Optional[torch.Tensor] = None, even_split: int = 0):
        if noalloc and (fp8 or workspace is not None):
            raise ValueError("the no-allocation call takes an fp16 cache and no workspace")
        self.name = ("paged_attn_decode_noalloc" if noalloc else
                     "paged_attn_decode_fp8" if fp8 else "paged_attn_decode")
        _check(q, "q", torch.float16, 3)
        _check_kv(k_cache, "k_cache", fp8, 5)
        _check_kv(v_cache, "v_cache", fp8, 4)
        _check(block_tables, "block_tables", torch.int32, 2)
        _check(context_lens, "context_lens", torch.int32, 1)
        NB, Hkv, NG, T, X = k_cache.shape
        B, Hq, D = q.shape
        if tuple(v_cache.shape) != (NB, Hkv, T, NG * X) or NG * X != D or X != (16 if fp8 else 8):
            raise ValueError("k_cache must be [NB, Hkv, D/%d, T, %d] and v_cache [NB, Hkv, T, D]"
                             % ((16, 16) if fp8 else (8, 8)))
        if block_tables.shape[0] != B or context_lens.shape[0] != B:
            raise ValueError("inconsistent shapes")
        check_debug_shapes(B, Hkv, block_tables.shape[1], debug_gather_k, debug_trace,
                           debug_error_word)
        self.device = q.device
        self._index = q.get_device()
        _same_device(self._index, k_cache=k_cache, v_cache=v_cache, block_tables=block_tables,
                     context_lens=context_lens, out=out, workspace=workspace,
                     debug_gather_k=debug_gather_k, debug_trace=debug_trace,
                     debug_error_word=debug_error_word, debug_timeline=debug_timeline)
        if scale is None:
            scale = D ** -0.5
        if out is None:
            out = torch.empty_like(q)
        else:
            _check(out, "out", torch.float16, 3)
            if out.shape != q.shape:
                raise ValueError("out must have q's shape")
        self._shape = shape_of(q, k_cache, block_tables, v_cache)
        self._opts = options(prefetch, partition_blocks, waves_per_wg, prefetch_distance,
                             seq_order, structure, debug_gather_k, debug_trace,
                             debug_error_word, min_context_hint=min_context_hint,
                             max_resident_wgs=max_resident_wgs, debug_timeline=debug_timeline,
                      even_split=even_split)
        if debug_timeline is not None:
            check_debug_timeline(debug_timeline, nat.plan(self._shape, self._opts)["workgroups"])
        L = nat.lib()
        need = int(L.paged_attn_workspace_size(ctypes.byref(self._shape),
                                               ctypes.byref(self._opts)))
        if noalloc:
            if need > nat.NOALLOC_SCRATCH_BYTES:
                raise ValueError(f"{self.name}: the plan needs {need} bytes of partials, the "
                                 f"scratch array holds {nat.NOALLOC_SCRATCH_BYTES}")
        elif need:
            if workspace is None:
                workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
            elif not workspace.is_cuda or workspace.numel() * workspace.element_size() < need:
                raise ValueError(f"workspace needs {need} bytes")
            self._opts.workspace = workspace.data_ptr()
            self._opts.workspace_bytes = workspace.numel() * workspace.element_size()
        self.out, self.workspace = out, workspace
        # the tensors whose storage the call reads or writes stay alive with it
        self._keep = (q, k_cache, v_cache, block_tables, context_lens, debug_gather_k,
                      debug_trace, debug_error_word, debug_timeline)
        ptrs = [ctypes.c_void_p(t.data_ptr()) for t in (q, k_cache, v_cache, block_tables,
                                                          context_lens)]
        st = _stream_handle(stream, q.device)
        if fp8:
            self._fn = L.paged_attn_decode_fp8
            self._args = (*ptrs, ctypes.c_float(scale), ctypes.c_float(k_scale),
                          ctypes.c_float(v_scale), ctypes.c_void_p(out.data_ptr()),
                          ctypes.byref(self._shape), ctypes.byref(self._opts), st)
        else:
            self._fn = L.paged_attn_decode_noalloc if noalloc else L.paged_attn_decode
            self._args = (*ptrs, ctypes.c_float(scale), ctypes.c_void_p(out.data_ptr()),
                          ctypes.byref(self._shape), ctypes.byref(self._opts), st)

    def __call__(self) -> torch.Tensor:
        if torch.cuda.current_device() == self._index:
            rc = self._fn(*self._args)
        else:
            with torch.cuda.device(self._index):  # the library launches on the current device
                rc = self._fn(*self._args)
        if rc != nat.PA_OK:
            raise RuntimeError(f"{self.name}: {nat.error_string(rc)} ({rc})")
        return self.out


def prepare_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   block_tables: torch.Tensor, context_lens: torch.Tensor,
                   scale: Optional[float] = None, out: Optional[torch.Tensor] = None, *,
                   prefetch: int = -1, partition_blocks: int = 0, waves_per_wg: int = 0,
                   prefetch_distance: int = 0, seq_order: int = 0, structure: int = 0,
                   workspace: Optional[torch.Tensor] = None,
                   debug_gather_k: Optional[torch.Tensor] = None,
                   debug_trace: Optional[torch.Tensor] = None,
                   debug_error_word: Optional[torch.Tensor] = None,
                   stream: Optional[torch.cuda.Stream] = None, min_context_hint: int = 0,
                   max_resident_wgs: int = 0,
                   debug_timeline: Optional[torch.Tensor] = None,
                   even_split: int = 0) -> DecodeCall:
    """paged_attn_decode prepared for repeated calls on the same tensors."""
    return DecodeCall(False, q, k_cache, v_cache, block_tables, context_lens, scale, 1.0, 1.0,
                      out, prefetch, partition_blocks, waves_per_wg, prefetch_distance,
                      seq_order, structure, workspace, debug_gather_k, debug_trace,
                      debug_error_word, stream, min_context_hint=min_context_hint,
                      max_resident_wgs=max_resident_wgs, debug_timeline=debug_timeline,
                      even_split=even_split)


def prepare_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                           block_tables: torch.Tensor, context_lens: torch.Tensor,
                           scale: Optional[float] = None, out: Optional[torch.Tensor] = None, *,
                           prefetch: int = -1, partition_blocks: int = 0, waves_per_wg: int = 0,
                           prefetch_distance: int = 0, seq_order: int = 0, structure: int = 0,
                           debug_gather_k: Optional[torch.Tensor] = None,
                           debug_trace: Optional[torch.Tensor] = None,
                           debug_error_word: Optional[torch.Tensor] = None,
                           stream: Optional[torch.cuda.Stream] = None,
                           min_context_hint: int = 0, max_resident_wgs: int = 0,
                           debug_timeline: Optional[torch.Tensor] = None,
                           even_split: int = 0) -> DecodeCall:
    """paged_attn_decode_noalloc prepared for repeated calls; pass `out` to
    keep the calls free of allocation."""
    return DecodeCall(False, q, k_cache, v_cache, block_tables, context_lens, scale, 1.0, 1.0,
                      out, prefetch, partition_blocks, waves_per_wg, prefetch_distance,
                      seq_order, structure, None, debug_gather_k, debug_trace,
                      debug_error_word, stream, noalloc=True, min_context_hint=min_context_hint,
                      max_resident_wgs=max_resident_wgs, debug_timeline=debug_timeline,
                      even_split=even_split)


def paged_attn_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                              block_tables: torch.Tensor, context_lens: torch.Tensor,
                              scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                              **kw) -> torch.Tensor:
    """paged_attn_decode without a workspace: the partition partials go to the
    library's per-device scratch array (PA_NOALLOC_SCRATCH_BYTES), so with
    `out` given nothing is allocated.  Calls that overlap on one GPU race."""
    return prepare_decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, scale, out,
                                  **kw)()


def prepare_decode_fp8(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                       block_tables: torch.Tensor, context_lens: torch.Tensor,
                       scale: Optional[float] = None, k_scale: float = 1.0,
                       v_scale: float = 1.0, out: Optional[torch.Tensor] = None, *,
                       prefetch: int = -1, partition_blocks: int = 0, waves_per_wg: int = 0,
                       prefetch_distance: int = 0, seq_order: int = 0, structure: int = 0,
                       workspace: Optional[torch.Tensor] = None,
                       debug_gather_k: Optional[torch.Tensor] = None,
                       debug_trace: Optional[torch.Tensor] = None,
                       debug_error_word: Optional[torch.Tensor] = None,
                       stream: Optional[torch.cuda.Stream] = None, min_context_hint: int = 0,
                       max_resident_wgs: int = 0,
                       debug_timeline: Optional[torch.Tensor] = None,
                       even_split: int = 0) -> DecodeCall:
    """paged_attn_decode_fp8 prepared for repeated calls on the same tensors."""
    if k_cache.dtype == torch.float8_e4m3fn:
        k_cache = k_cache.view(torch.uint8)
    if v_cache.dtype == torch.float8_e4m3fn:
        v_cache = v_cache.view(torch.uint8)
    return DecodeCall(True, q, k_cache, v_cache, block_tables, context_lens, scale, k_scale,
                      v_scale, out, prefetch, partition_blocks, waves_per_wg, prefetch_distance,
                      seq_order, structure, workspace, debug_gather_k, debug_trace,
                      debug_error_word, stream, min_context_hint=min_context_hint,
                      max_resident_wgs=max_resident_wgs, debug_timeline=debug_timeline,
                      even_split=even_split)


def paged_attn_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      block_tables: torch.Tensor, context_lens: torch.Tensor,
                      scale: Optional[float] = None, out: Optional[torch.Tensor] = None, *,
                      prefetch: int = -1, partition_blocks: int = 0, waves_per_wg: int = 0,
                      prefetch_distance: int = 0, seq_order: int = 0, structure: int = 0,
                      workspace: Optional[torch.Tensor] = None,
                      debug_gather_k: Optional[torch.Tensor] = None,
                      debug_trace: Optional[torch.Tensor] = None,
                      debug_error_word: Optional[torch.Tensor] = None,
                      stream: Optional[torch.cuda.Stream] = None, min_context_hint: int = 0,
                      max_resident_wgs: int = 0,
                      debug_timeline: Optional[torch.Tensor] = None,
                      even_split: int = 0) -> torch.Tensor:
    """One decode step of paged attention; returns out (fp16 [B, Hq, 128]).

    q [B, Hq, 128] fp16; k_cache [NB, Hkv, 16, 16, 8] fp16 (dim group, token, 8
    dims); v_cache [NB, Hkv, 16, 128] fp16 (token, dim); block_tables [B, MB]
    int32; context_lens [B] int32; scale defaults to 1/sqrt(128).
    """
    return prepare_decode(q, k_cache, v_cache, block_tables, context_lens, scale, out,
                          prefetch=prefetch, partition_blocks=partition_blocks,
                          waves_per_wg=waves_per_wg, prefetch_distance=prefetch_distance,
                          seq_order=seq_order, structure=structure, workspace=workspace,
                          debug_gather_k=debug_gather_k, debug_trace=debug_trace,
                          debug_error_word=debug_error_word, stream=stream,
                          min_context_hint=min_context_hint,
                          max_resident_wgs=max_resident_wgs, debug_timeline=debug_timeline,
                      even_split=even_split)()


def paged_attn_decode_fp8(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                          block_tables: torch.Tensor, context_lens: torch.Tensor,
                          scale: Optional[float] = None, k_scale: float = 1.0,
                          v_scale: float = 1.0, out: Optional[torch.Tensor] = None, *,
                          prefetch: int = -1, partition_blocks: int = 0, waves_per_wg: int = 0,
                          prefetch_distance: int = 0, seq_order: int = 0,
                          structure: int = 0,
                          workspace: Optional[torch.Tensor] = None,
                          debug_gather_k: Optional[torch.Tensor] = None,
                          debug_trace: Optional[torch.Tensor] = None,
                          debug_error_word: Optional[torch.Tensor] = None,
                          stream: Optional[torch.cuda.Stream] = None,
                          min_context_hint: int = 0, max_resident_wgs: int = 0,
                          debug_timeline: Optional[torch.Tensor] = None,
                          even_split: int = 0) -> torch.Tensor:
    """Decode over an OCP E4M3 cache (uint8 or float8_e4m3fn); a cached value
    is decode(byte) * k_scale (K) or * v_scale (V).

    k_cache [NB, Hkv, 8, 16, 16] (16-dim group, token, 16 dims); v_cache
    [NB, Hkv, 16, 128] (token, dim); the rest as paged_attn_decode.
    debug_gather_k receives the widened K values before k_scale (fp16).
    """
    return prepare_decode_fp8(q, k_cache, v_cache, block_tables, context_lens, scale, k_scale,
                              v_scale, out, prefetch=prefetch,
                              partition_blocks=partition_blocks, waves_per_wg=waves_per_wg,
                              prefetch_distance=prefetch_distance, seq_order=seq_order,
                              structure=structure, workspace=workspace,
                              debug_gather_k=debug_gather_k, debug_trace=debug_trace,
                              debug_error_word=debug_error_word, stream=stream,
                              min_context_hint=min_context_hint,
                              max_resident_wgs=max_resident_wgs, debug_timeline=debug_timeline,
                      even_split=even_split)()


def pack_k(k_token_major: torch.Tensor, out: Optional[torch.Tensor] = None,
           stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """K from the token-major layout [NB, Hkv, 16, 128] (fp16, or E4M3 as
    uint8 / float8_e4m3fn) into the layout the decode calls read: fp16
    [NB, Hkv, 16, 16, 8], E4M3 [NB, Hkv, 8, 16, 16] (paged_attn_pack_k, on the
    device, bit for bit)."""
    k = k_token_major
    if k.dtype == torch.float8_e4m3fn:
        k = k.view(torch.uint8)
    if not isinstance(k, torch.Tensor) or not k.is_cuda or not k.is_contiguous():
        raise ValueError("k_token_major must be a contiguous device tensor")
    if k.dim() != 4 or tuple(k.shape[2:]) != (16, 128):
        raise ValueError("k_token_major must be [NB, Hkv, 16, 128]")
    if k.dtype not in (torch.float16, torch.uint8):
        raise TypeError(f"k_token_major must be fp16 or E4M3 bytes, got {k.dtype}")
    fp8 = k.dtype == torch.uint8
    NB, Hkv = k.shape[:2]
    shape = (NB, Hkv, 8, 16, 16) if fp8 else (NB, Hkv, 16, 16, 8)
    if out is None:
        out = torch.empty(shape, dtype=k.dtype, device=k.device)
    elif (tuple(out.shape) != shape or out.dtype != k.dtype or not out.is_contiguous() or
          out.device != k.device):
        raise ValueError(f"out must be a contiguous {k.dtype} tensor {list(shape)} on {k.device}")
    st = _stream_handle(stream, k.device)
    with torch.cuda.device(k.device):
        rc = nat.lib().paged_attn_pack_k(ctypes.c_void_p(k.data_ptr()),
                                         ctypes.c_void_p(out.data_ptr()), ctypes.c_int64(NB),
                                         ctypes.c_int32(Hkv),
                                         ctypes.c_int32(nat.KV_E4M3 if fp8 else nat.KV_F16), st)
    if rc != nat.PA_OK:
        raise RuntimeError(f"paged_attn_pack_k: {nat.error_string(rc)} ({rc})")
    return out


def stream_read(buf: torch.Tensor, sink: Optional[torch.Tensor] = None,
                stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Read every byte of buf once (the streaming-read ceiling kernel).
    Returns the sink: one 16-byte XOR per work-group."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    nbytes = buf.numel() * buf.element_size()
    sink_bytes = int(nat.lib().paged_attn_stream_read_sink_bytes(nbytes))
    if sink is None:
        sink = torch.zeros(sink_bytes // 4, dtype=torch.int32, device=buf.device)
    elif (not sink.is_contiguous() or sink.device != buf.device or
          sink.numel() * sink.element_size() < sink_bytes):
        raise ValueError(f"sink must be a contiguous tensor of at least {sink_bytes} bytes "
                         f"on {buf.device}")
    st = _stream_handle(stream, buf.device)
    with torch.cuda.device(buf.device):
        rc = nat.lib().paged_attn_stream_read(ctypes.c_void_p(buf.data_ptr()),
                                              ctypes.c_size_t(nbytes),
                                              ctypes.c_void_p(sink.data_ptr()), st)
    if rc != nat.PA_OK:
        raise RuntimeError(f"paged_attn_stream_read: {nat.error_string(rc)} ({rc})")
    return sink
