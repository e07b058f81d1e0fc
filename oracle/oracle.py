"""ctypes wrapper around liboracle.so (fp64 paged decode attention).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The functions take the same host arrays the GPU path receives: fp16 Q, fp16
K/V pools laid out [num_blocks][num_kv_heads][block_size][head_dim], int32
block tables [num_seqs][max_blocks_per_seq] and int32 context lengths.  They
return float64 results; nothing is rounded back to fp16.

What is computed is the plain paged softmax attention described by the
asynchronous-KV-prefetch review (sections 3.4 and 4.1: block-table lookup,
Q*K^T per block, logits times V) and the PagedAttention answer (section 3:
page table -> physical page -> attention -> output); see pa_oracle.c.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_ERRORS = {
    1: "invalid argument",
    2: "block-table entry outside the pool",
    3: "context length exceeds the block table",
    4: "out of host memory",
}

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB):
        _build.build()
    lib = ctypes.CDLL(_build.LIB)
    p = ctypes.c_void_p
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    lib.pao_decode_f64.argtypes = [p, p, p, p, p, ctypes.c_float, i32, i32, i32,
                                   i32, i32, i32, i64, p, i32]
    lib.pao_decode_f64.restype = ctypes.c_int
    lib.pao_decode_rows_f64.argtypes = [p, p, p, p, p, ctypes.c_float, i32, i32,
                                        i32, i32, i32, i32, i64, p, p, i64, p,
                                        i32]
    lib.pao_decode_rows_f64.restype = ctypes.c_int
    lib.pao_half_to_double.argtypes = [ctypes.c_uint16]
    lib.pao_half_to_double.restype = ctypes.c_double
    lib.pao_e4m3_to_double.argtypes = [ctypes.c_uint8]
    lib.pao_e4m3_to_double.restype = ctypes.c_double
    f = ctypes.c_float
    lib.pao_decode_fp8_f64.argtypes = [p, p, p, p, p, f, f, f, i32, i32, i32, i32, i32, i32,
                                       i64, p, i32]
    lib.pao_decode_fp8_f64.restype = ctypes.c_int
    lib.pao_decode_fp8_rows_f64.argtypes = [p, p, p, p, p, f, f, f, i32, i32, i32, i32, i32,
                                            i32, i64, p, p, i64, p, i32]
    lib.pao_decode_fp8_rows_f64.restype = ctypes.c_int
    lib.pao_max_threads.argtypes = []
    lib.pao_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def max_threads() -> int:
    """Threads OpenMP will use by default (OMP_NUM_THREADS or all cores)."""
    return int(_load().pao_max_threads())


def half_to_double(bits: int) -> float:
    """The oracle's own fp16 decoder, exposed so tests can pin it."""
    return float(_load().pao_half_to_double(int(bits) & 0xFFFF))


def e4m3_to_double(bits: int) -> float:
    """The oracle's own OCP FP8 E4M3 decoder, exposed so tests can pin it."""
    return float(_load().pao_e4m3_to_double(int(bits) & 0xFF))


def _prep(q, k_cache, v_cache, block_tables, context_lens, kv_dtype=np.float16):
    q = np.ascontiguousarray(q, dtype=np.float16)
    k_cache = np.ascontiguousarray(k_cache, dtype=kv_dtype)
    v_cache = np.ascontiguousarray(v_cache, dtype=kv_dtype)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    if q.ndim != 3 or k_cache.ndim != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [B,Hq,D]; k/v caches [NB,Hkv,T,D] of equal shape")
    B, Hq, D = q.shape
    NB, Hkv, T, Dk = k_cache.shape
    if Dk != D or bt.ndim != 2 or bt.shape[0] != B or ctx.shape != (B,):
        raise ValueError("inconsistent shapes")
    dims = (B, Hq, Hkv, D, T, bt.shape[1], NB)
    return q, k_cache, v_cache, bt, ctx, dims


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc):
    if rc != 0:
        raise RuntimeError(f"oracle error {rc}: {_ERRORS.get(rc, 'unknown')}")


def paged_attention_f64(q, k_cache, v_cache, block_tables, context_lens, scale,
                        threads: int = 0) -> np.ndarray:
    """All (b, h) rows; returns float64 [B, Hq, D]."""
    q, k, v, bt, ctx, (B, Hq, Hkv, D, T, MB, NB) = _prep(
        q, k_cache, v_cache, block_tables, context_lens)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    rc = _load().pao_decode_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(bt), _ptr(ctx),
                                float(np.float32(scale)), B, Hq, Hkv, D, T, MB,
                                NB, _ptr(out), int(threads))
    _check(rc)
    return out


def paged_attention_rows_f64(q, k_cache, v_cache, block_tables, context_lens,
                             scale, rows, threads: int = 0) -> np.ndarray:
    """Only the listed (b, h) rows; rows is an int array [n, 2].  Returns [n, D]."""
    q, k, v, bt, ctx, (B, Hq, Hkv, D, T, MB, NB) = _prep(
        q, k_cache, v_cache, block_tables, context_lens)
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 2)
    rb = np.ascontiguousarray(rows[:, 0], dtype=np.int32)
    rh = np.ascontiguousarray(rows[:, 1], dtype=np.int32)
    out = np.zeros((rows.shape[0], D), dtype=np.float64)
    rc = _load().pao_decode_rows_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(bt),
                                     _ptr(ctx), float(np.float32(scale)), B, Hq,
                                     Hkv, D, T, MB, NB, _ptr(rb), _ptr(rh),
                                     rows.shape[0], _ptr(out), int(threads))
    _check(rc)
    return out


def paged_attention_fp8_f64(q, k8, v8, block_tables, context_lens, scale, k_scale, v_scale,
                            threads: int = 0) -> np.ndarray:
    """E4M3 caches (uint8 [NB, Hkv, T, D], token-major), values byte * scale.
    All (b, h) rows; float64 [B, Hq, D]."""
    q, k, v, bt, ctx, (B, Hq, Hkv, D, T, MB, NB) = _prep(
        q, k8, v8, block_tables, context_lens, np.uint8)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    rc = _load().pao_decode_fp8_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(bt), _ptr(ctx),
                                    float(np.float32(scale)), float(np.float32(k_scale)),
                                    float(np.float32(v_scale)), B, Hq, Hkv, D, T, MB, NB,
                                    _ptr(out), int(threads))
    _check(rc)
    return out


def paged_attention_fp8_rows_f64(q, k8, v8, block_tables, context_lens, scale, k_scale,
                                 v_scale, rows, threads: int = 0) -> np.ndarray:
    """The listed (b, h) rows of paged_attention_fp8_f64; returns [n, D]."""
    q, k, v, bt, ctx, (B, Hq, Hkv, D, T, MB, NB) = _prep(
        q, k8, v8, block_tables, context_lens, np.uint8)
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 2)
    rb = np.ascontiguousarray(rows[:, 0], dtype=np.int32)
    rh = np.ascontiguousarray(rows[:, 1], dtype=np.int32)
    out = np.zeros((rows.shape[0], D), dtype=np.float64)
    rc = _load().pao_decode_fp8_rows_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(bt), _ptr(ctx),
                                         float(np.float32(scale)), float(np.float32(k_scale)),
                                         float(np.float32(v_scale)), B, Hq, Hkv, D, T, MB, NB,
                                         _ptr(rb), _ptr(rh), rows.shape[0], _ptr(out),
                                         int(threads))
    _check(rc)
    return out
