"""INT4 per-token-head paged KV cache on MI355X (gfx950): Python binding.

A thin ctypes layer over the C ABI of ``include/int4kv.h``.  It only marshals
arguments (device pointers, sizes, the current HIP stream); every step of the
write and the attention runs in the HIP kernels of ``libint4kv.so``.  If the
library is missing, every call raises: there is no CPU fallback.

Exports the C entry points under the same names:
    int4_kv_write(...)          quantize + pack K/V rows into the paged cache
    int4_paged_attention(...)   causal attention over the packed cache
    int4_decode_step(...)       both for a decode step, in one launch where it can
plus small helpers to size and allocate the buffers those calls take.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "int4_kv_write", "int4_paged_attention", "int4_paged_attention_noalloc", "int4_decode_step",
    "int4kv_decode_num_segments", "NOALLOC_SCRATCH_BYTES",
    "int4kv_cache_bytes", "int4kv_status_string",
    "int4kv_last_error", "Int4KVError", "cache_shape", "empty_cache", "segment_buffers",
    "library_path", "load_library", "int4kv_stream_rw", "int4kv_stream_blocks", "DecodeStepPlan",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libint4kv.so")
_lib = None

INT4KV_F16, INT4KV_BF16 = 0, 1
_STATUS = {0: "INT4KV_OK", 1: "INT4KV_ERR_INVALID_ARG", 2: "INT4KV_ERR_UNSUPPORTED",
           3: "INT4KV_ERR_WORKSPACE", 4: "INT4KV_ERR_LAUNCH"}


class Int4KVError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_STATUS.get(status, status)}: {detail}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libint4kv.so (built in-tree by build.py); raise if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"HIP library not built: {_LIB_PATH} is missing "
                           "(run python -m int4_quantized_paged_amd.build)")
    lib = ctypes.CDLL(_LIB_PATH)
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.int4kv_cache_bytes.argtypes = [i32, i32, i32, i32]
    lib.int4kv_cache_bytes.restype = i64
    lib.int4kv_status_string.argtypes = [ctypes.c_int]
    lib.int4kv_status_string.restype = ctypes.c_char_p
    lib.int4kv_last_error.argtypes = []
    lib.int4kv_last_error.restype = ctypes.c_char_p
    lib.int4_kv_write.argtypes = [P, i64, P, i64, ctypes.c_int, P, i32, P, i32, i32, i32, i32, P, P]
    lib.int4_kv_write.restype = ctypes.c_int
    lib.int4_paged_attention.argtypes = [P, i64, P, ctypes.c_int, P, i32, i32, i32, i32, i32, P, P,
                                         i32, i32, i32, P, i32, ctypes.c_float, i32,
                                         ctypes.c_float, P, i32, P, P, P, P]
    lib.int4_paged_attention.restype = ctypes.c_int
    lib.int4_paged_attention_noalloc.argtypes = [P, i64, P, ctypes.c_int, P, i32, i32, i32, i32,
                                                 i32, P, P, i32, i32, i32, P, i32, ctypes.c_float,
                                                 i32, ctypes.c_float, P, i32, P]
    lib.int4_paged_attention_noalloc.restype = ctypes.c_int
    lib.int4kv_stream_rw.argtypes = [P, i64, P, i64, P]
    lib.int4kv_stream_rw.restype = ctypes.c_int
    lib.int4kv_stream_blocks.argtypes = [P, i64, P, i64, i32, P]
    lib.int4kv_stream_blocks.restype = ctypes.c_int
    lib.int2_paged_attention.argtypes = lib.int4_paged_attention.argtypes
    lib.int2_paged_attention.restype = ctypes.c_int
    lib.int4_decode_step.argtypes = [P, i64, P, i64, P, P, i64, P, ctypes.c_int, P, i32, i32, i32,
                                     i32, i32, P, P, i32, i32, i32, P, i32, ctypes.c_float, i32,
                                     ctypes.c_float, P, i32, P, P, P, P]
    lib.int4_decode_step.restype = ctypes.c_int
    lib.int2kv_cache_bytes.argtypes = [i32, i32, i32, i32]
    lib.int2kv_cache_bytes.restype = i64
    lib.int2_kv_write.argtypes = [P, i64, P, i64, ctypes.c_int, P, i32, P, i32, i32, i32, i32, P,
                                  P]
    lib.int8kv_cache_bytes.argtypes = [i32, i32, i32, i32]
    lib.int8kv_cache_bytes.restype = i64
    lib.int8_kv_write.argtypes = [P, i64, P, i64, ctypes.c_int, P, i32, P, i32, i32, i32, i32, P]
    lib.int8_kv_write.restype = ctypes.c_int
    lib.int8_paged_attention.argtypes = [P, i64, P, ctypes.c_int, P, i32, i32, i32, i32, i32, P, P,
                                         i32, i32, i32, P, i32, ctypes.c_float, i32,
                                         ctypes.c_float, i32, P, P, P, P]
    lib.int8_paged_attention.restype = ctypes.c_int
    lib.int8kv_decode_num_segments.argtypes = [i32, i32, i32]
    lib.int8kv_decode_num_segments.restype = i32
    lib.int4kv_decode_num_segments.argtypes = [i32, i32, i32]
    lib.int4kv_decode_num_segments.restype = i32
    _lib = lib
    return lib


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float16:
        return INT4KV_F16
    if dt == torch.bfloat16:
        return INT4KV_BF16
    raise TypeError(f"unsupported dtype {dt}: float16 or bfloat16")


def _check(status: int):
    if status != 0:
        raise Int4KVError(status, load_library().int4kv_last_error().decode())


def int4kv_cache_bytes(num_blocks: int, block_size: int, num_kv_heads: int, head_size: int) -> int:
    return int(load_library().int4kv_cache_bytes(num_blocks, block_size, num_kv_heads, head_size))


def int4kv_status_string(status: int) -> str:
    return load_library().int4kv_status_string(status).decode()


def int4kv_last_error() -> str:
    return load_library().int4kv_last_error().decode()


def int4kv_decode_num_segments(num_seqs: int, num_kv_heads: int, max_seqlen_k: int) -> int:
    """The library's split-K segment count for a decode batch (host only)."""
    return int(load_library().int4kv_decode_num_segments(num_seqs, num_kv_heads, max_seqlen_k))


def int8kv_decode_num_segments(num_seqs: int, num_kv_heads: int, max_seqlen_k: int) -> int:
    """The library's split-K segment count for an INT8 decode batch (host only)."""
    return int(load_library().int8kv_decode_num_segments(num_seqs, num_kv_heads, max_seqlen_k))


def cache_shape(num_blocks: int, num_kv_heads: int, head_size: int, block_size: int = 16):
    """[num_blocks, 2, block_size, num_kv_heads, head_size/2 + 4] uint8."""
    return (num_blocks, 2, block_size, num_kv_heads, head_size // 2 + 4)


def empty_cache(num_blocks: int, num_kv_heads: int, head_size: int, device="cuda",
                block_size: int = 16) -> torch.Tensor:
    return torch.empty(cache_shape(num_blocks, num_kv_heads, head_size, block_size),
                       dtype=torch.uint8, device=device)


def segment_buffers(num_seqs: int, num_q_heads: int, num_segments: int, head_size: int,
                    device="cuda"):
    """Split-K scratch: (output [S, Hq, NS, d], max [S, Hq, NS], expsum [S, Hq, NS]) fp32."""
    o = torch.empty((num_seqs, num_q_heads, num_segments, head_size), dtype=torch.float32,
                    device=device)
    m = torch.empty((num_seqs, num_q_heads, num_segments), dtype=torch.float32, device=device)
    s = torch.empty((num_seqs, num_q_heads, num_segments), dtype=torch.float32, device=device)
    return o, m, s


def int8kv_cache_bytes(num_blocks: int, block_size: int, num_kv_heads: int,
                       head_size: int) -> int:
    return int(load_library().int8kv_cache_bytes(num_blocks, block_size, num_kv_heads, head_size))


def cache_shape_int8(num_blocks: int, num_kv_heads: int, head_size: int, block_size: int = 16):
    """INT8 per-token-head cache: [num_blocks, 2, block_size, num_kv_heads, head_size + 4] uint8."""
    return (num_blocks, 2, block_size, num_kv_heads, head_size + 4)


def empty_cache_int8(num_blocks: int, num_kv_heads: int, head_size: int, device="cuda",
                     block_size: int = 16) -> torch.Tensor:
    return torch.empty(cache_shape_int8(num_blocks, num_kv_heads, head_size, block_size),
                       dtype=torch.uint8, device=device)


def int8_kv_write(key: torch.Tensor, value: torch.Tensor, slot_mapping: torch.Tensor,
                  kv_cache: torch.Tensor) -> None:
    """INT8 per-token-head write of ``key``/``value`` [T, Hkv, d] at ``slot_mapping``
    into ``kv_cache`` uint8 [NB, 2, B, Hkv, d + 4].  Enqueued on the current stream."""
    lib = load_library()
    T = key.shape[0]
    if key.dim() != 3 or value.shape != key.shape or key.dtype != value.dtype:
        raise ValueError("key and value must both be [T, Hkv, d] of one dtype")
    if key.stride(2) != 1 or key.stride(1) != key.shape[2] or value.stride(2) != 1 or \
            value.stride(1) != value.shape[2]:
        raise ValueError("key/value heads must be contiguous ([T, Hkv, d] with a token stride)")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be int64 [T]")
    if kv_cache.dtype != torch.uint8 or kv_cache.dim() != 5 or not kv_cache.is_contiguous() or \
            kv_cache.shape[4] != key.shape[2] + 4:
        raise ValueError("kv_cache must be a contiguous uint8 [NB, 2, B, Hkv, d+4] tensor")
    nb, two, bs, hkv, _ = kv_cache.shape
    _check(lib.int8_kv_write(_ptr(key), key.stride(0), _ptr(value), value.stride(0),
                             _dtype_code(key.dtype), _ptr(slot_mapping.contiguous()), T,
                             _ptr(kv_cache), nb, bs, hkv, key.shape[2], _stream(key.device)))


def int2kv_cache_bytes(num_blocks: int, block_size: int, num_kv_heads: int,
                       head_size: int) -> int:
    return int(load_library().int2kv_cache_bytes(num_blocks, block_size, num_kv_heads, head_size))


def cache_shape_int2(num_blocks: int, num_kv_heads: int, head_size: int, block_size: int = 16):
    """INT2 Lloyd-Max cache: [num_blocks, 2, block_size, num_kv_heads, head_size/4 + 4] uint8."""
    return (num_blocks, 2, block_size, num_kv_heads, head_size // 4 + 4)


def empty_cache_int2(num_blocks: int, num_kv_heads: int, head_size: int, device="cuda",
                     block_size: int = 16) -> torch.Tensor:
    return torch.empty(cache_shape_int2(num_blocks, num_kv_heads, head_size, block_size),
                       dtype=torch.uint8, device=device)


def int2_kv_write(key: torch.Tensor, value: torch.Tensor, slot_mapping: torch.Tensor,
                  kv_cache: torch.Tensor, rht_signs: torch.Tensor) -> None:
    """INT2 Lloyd-Max write of ``key``/``value`` [T, Hkv, d] at ``slot_mapping`` into
    ``kv_cache`` uint8 [NB, 2, B, Hkv, d/4 + 4], rotated with ``rht_signs`` (fp32 [d]).
    Enqueued on the current stream."""
    lib = load_library()
    T = key.shape[0]
    if key.dim() != 3 or value.shape != key.shape or key.dtype != value.dtype:
        raise ValueError("key and value must both be [T, Hkv, d] of one dtype")
    if key.stride(2) != 1 or key.stride(1) != key.shape[2] or value.stride(2) != 1 or \
            value.stride(1) != value.shape[2]:
        raise ValueError("key/value heads must be contiguous ([T, Hkv, d] with a token stride)")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be int64 [T]")
    if kv_cache.dtype != torch.uint8 or kv_cache.dim() != 5 or not kv_cache.is_contiguous() or \
            kv_cache.shape[4] != key.shape[2] // 4 + 4:
        raise ValueError("kv_cache must be a contiguous uint8 [NB, 2, B, Hkv, d/4+4] tensor")
    if rht_signs.dtype != torch.float32 or rht_signs.shape != (key.shape[2],):
        raise ValueError("rht_signs must be float32 [d]")
    nb, two, bs, hkv, _ = kv_cache.shape
    _check(lib.int2_kv_write(_ptr(key), key.stride(0), _ptr(value), value.stride(0),
                             _dtype_code(key.dtype), _ptr(slot_mapping.contiguous()), T,
                             _ptr(kv_cache), nb, bs, hkv, key.shape[2],
                             _ptr(rht_signs.contiguous()), _stream(key.device)))


def int8_paged_attention(q: torch.Tensor, kv_cache: torch.Tensor, cu_seqlens_q: torch.Tensor,
                         seqused_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int,
                         block_table: torch.Tensor, softmax_scale: float,
                         out: torch.Tensor | None = None, num_segments: int = 1,
                         segm_output: torch.Tensor | None = None,
                         segm_max: torch.Tensor | None = None,
                         segm_expsum: torch.Tensor | None = None,
                         sliding_window: int = 0, softcap: float = 0.0) -> torch.Tensor:
    """Causal attention of ``q`` [Tq, Hq, d] (decode or prefill / mixed batches)
    over the INT8 per-token-head cache (uint8 [NB, 2, B, Hkv, d + 4]); returns ``out``."""
    lib = load_library()
    if q.dim() != 3 or q.stride(2) != 1 or q.stride(1) != q.shape[2]:
        raise ValueError("q must be [Tq, Hq, d] with contiguous heads")
    Tq, hq, d = q.shape
    if out is None:
        out = torch.empty((Tq, hq, d), dtype=q.dtype, device=q.device)
    if not out.is_contiguous() or out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must be contiguous with q's shape and dtype")
    if kv_cache.dtype != torch.uint8 or kv_cache.dim() != 5 or kv_cache.shape[4] != d + 4:
        raise ValueError("kv_cache must be a uint8 [NB, 2, B, Hkv, d+4] tensor")
    nb, two, bs, hkv, _ = kv_cache.shape
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("seqused_k", seqused_k),
                    ("block_table", block_table)):
        if t.dtype != torch.int32:
            raise ValueError(f"{name} must be int32")
    if block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("block_table must be [S, max_blocks] with unit column stride")
    S = seqused_k.shape[0]
    _check(lib.int8_paged_attention(
        _ptr(q), q.stride(0), _ptr(out), _dtype_code(q.dtype), _ptr(kv_cache), nb, bs, hkv, d, hq,
        _ptr(cu_seqlens_q.contiguous()), _ptr(seqused_k.contiguous()), S, int(max_seqlen_q),
        int(max_seqlen_k), _ptr(block_table), block_table.stride(0), float(softmax_scale),
        int(sliding_window), float(softcap), int(num_segments), _ptr(segm_output),
        _ptr(segm_max), _ptr(segm_expsum), _stream(q.device)))
    return out


def int4_paged_attention_noalloc(q: torch.Tensor, kv_cache: torch.Tensor,
                                 cu_seqlens_q: torch.Tensor, seqused_k: torch.Tensor,
                                 max_seqlen_q: int, max_seqlen_k: int, block_table: torch.Tensor,
                                 softmax_scale: float, rht_signs: torch.Tensor,
                                 out: torch.Tensor, num_segments: int = 1,
                                 sliding_window: int = 0, softcap: float = 0.0) -> torch.Tensor:
    """int4_paged_attention with the split-K partials in the library's fixed device
    buffer (NOALLOC_SCRATCH_BYTES per GPU): nothing is allocated, ``out`` included."""
    lib = load_library()
    if q.dim() != 3 or q.stride(2) != 1 or q.stride(1) != q.shape[2]:
        raise ValueError("q must be [Tq, Hq, d] with contiguous heads")
    Tq, hq, d = q.shape
    if not out.is_contiguous() or out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must be contiguous with q's shape and dtype")
    nb, two, bs, hkv, _ = kv_cache.shape
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("seqused_k", seqused_k),
                    ("block_table", block_table)):
        if t.dtype != torch.int32 or not t.is_contiguous() and t is not block_table:
            raise ValueError(f"{name} must be contiguous int32")
    if block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("block_table must be [S, max_blocks] with unit column stride")
    if not rht_signs.is_contiguous():
        raise ValueError("rht_signs must be contiguous")
    S = seqused_k.shape[0]
    _check(lib.int4_paged_attention_noalloc(
        _ptr(q), q.stride(0), _ptr(out), _dtype_code(q.dtype), _ptr(kv_cache), nb, bs, hkv, d, hq,
        _ptr(cu_seqlens_q), _ptr(seqused_k), S, int(max_seqlen_q), int(max_seqlen_k),
        _ptr(block_table), block_table.stride(0), float(softmax_scale), int(sliding_window),
        float(softcap), _ptr(rht_signs), int(num_segments), _stream(q.device)))
    return out


NOALLOC_SCRATCH_BYTES = 16 * 1024 * 1024  # INT4KV_NOALLOC_SCRATCH_BYTES of include/int4kv.h


def int4kv_stream_rw(src: torch.Tensor, read_bytes: int, dst: torch.Tensor, write_bytes: int):
    """Plain streaming pass (calibration of the write path's attainable bandwidth):
    reads ``read_bytes`` of ``src``, writes ``write_bytes`` of ``dst``."""
    lib = load_library()
    if read_bytes > src.numel() * src.element_size() or \
            write_bytes > dst.numel() * dst.element_size():
        raise ValueError("byte counts exceed the buffers")
    _check(lib.int4kv_stream_rw(_ptr(src), int(read_bytes), _ptr(dst), int(write_bytes),
                                _stream(src.device)))


def int4kv_stream_blocks(cache: torch.Tensor, block_bytes: int, block_ids: torch.Tensor,
                         num_workgroups: int):
    """The decode path's block gather on its own (calibration): copies the cache
    blocks listed in ``block_ids`` (int32, contiguous, on the cache's device)
    into LDS as the decode kernel does, computing and writing nothing.  Every
    id must lie in [0, cache bytes / block_bytes) (not checked: reading the
    ids back would synchronise the stream)."""
    lib = load_library()
    if block_ids.dtype != torch.int32 or not block_ids.is_contiguous() or \
            block_ids.device != cache.device:
        raise ValueError("block_ids must be a contiguous int32 tensor on the cache's device")
    _check(lib.int4kv_stream_blocks(_ptr(cache), int(block_bytes), _ptr(block_ids),
                                    int(block_ids.numel()), int(num_workgroups),
                                    _stream(cache.device)))


def int4_kv_write(key: torch.Tensor, value: torch.Tensor, slot_mapping: torch.Tensor,
                  kv_cache: torch.Tensor, rht_signs: torch.Tensor) -> None:
    """Quantize and store ``key``/``value`` [T, Hkv, d] at ``slot_mapping`` (int64 [T]).

    ``kv_cache`` is uint8 [num_blocks, 2, block_size, Hkv, d/2 + 4] on the same
    device; ``rht_signs`` fp32 [d] of +-1.  Enqueued on the current stream."""
    lib = load_library()
    T = key.shape[0]
    if key.dim() != 3 or value.shape != key.shape or key.dtype != value.dtype:
        raise ValueError("key and value must both be [T, Hkv, d] of one dtype")
    if key.stride(2) != 1 or key.stride(1) != key.shape[2] or value.stride(2) != 1 or \
            value.stride(1) != value.shape[2]:
        raise ValueError("key/value heads must be contiguous ([T, Hkv, d] with a token stride)")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be int64 [T]")
    if kv_cache.dtype != torch.uint8 or kv_cache.dim() != 5 or not kv_cache.is_contiguous():
        raise ValueError("kv_cache must be a contiguous uint8 [NB, 2, B, Hkv, d/2+4] tensor")
    nb, two, bs, hkv, _ = kv_cache.shape
    signs = rht_signs.contiguous()
    _check(lib.int4_kv_write(_ptr(key), key.stride(0), _ptr(value), value.stride(0),
                             _dtype_code(key.dtype), _ptr(slot_mapping.contiguous()), T,
                             _ptr(kv_cache), nb, bs, hkv, key.shape[2], _ptr(signs),
                             _stream(key.device)))


def int4_paged_attention(q: torch.Tensor, kv_cache: torch.Tensor, cu_seqlens_q: torch.Tensor,
                         seqused_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int,
                         block_table: torch.Tensor, softmax_scale: float,
                         rht_signs: torch.Tensor, out: torch.Tensor | None = None,
                         num_segments: int = 1, segm_output: torch.Tensor | None = None,
                         segm_max: torch.Tensor | None = None,
                         segm_expsum: torch.Tensor | None = None,
                         sliding_window: int = 0, softcap: float = 0.0) -> torch.Tensor:
    """Causal attention of ``q`` [Tq, Hq, d] over the packed cache; returns ``out``.
    ``sliding_window`` W > 0: a query at position pos sees keys [pos - W + 1, pos].
    ``softcap`` c > 0: scores z become c * tanh(z / c) before the softmax."""
    lib = load_library()
    if q.dim() != 3 or q.stride(2) != 1 or q.stride(1) != q.shape[2]:
        raise ValueError("q must be [Tq, Hq, d] with contiguous heads")
    Tq, hq, d = q.shape
    if out is None:
        out = torch.empty((Tq, hq, d), dtype=q.dtype, device=q.device)
    if not out.is_contiguous() or out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must be contiguous with q's shape and dtype")
    nb, two, bs, hkv, _ = kv_cache.shape
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("seqused_k", seqused_k),
                    ("block_table", block_table)):
        if t.dtype != torch.int32:
            raise ValueError(f"{name} must be int32")
    if block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("block_table must be [S, max_blocks] with unit column stride")
    S = seqused_k.shape[0]
    _check(lib.int4_paged_attention(
        _ptr(q), q.stride(0), _ptr(out), _dtype_code(q.dtype), _ptr(kv_cache), nb, bs, hkv, d, hq,
        _ptr(cu_seqlens_q.contiguous()), _ptr(seqused_k.contiguous()), S, int(max_seqlen_q),
        int(max_seqlen_k), _ptr(block_table), block_table.stride(0), float(softmax_scale),
        int(sliding_window), float(softcap), _ptr(rht_signs.contiguous()), int(num_segments),
        _ptr(segm_output),
        _ptr(segm_max), _ptr(segm_expsum), _stream(q.device)))
    return out


def int2_paged_attention(q: torch.Tensor, kv_cache: torch.Tensor, cu_seqlens_q: torch.Tensor,
                         seqused_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int,
                         block_table: torch.Tensor, softmax_scale: float,
                         rht_signs: torch.Tensor, out: torch.Tensor | None = None,
                         num_segments: int = 1, segm_output: torch.Tensor | None = None,
                         segm_max: torch.Tensor | None = None,
                         segm_expsum: torch.Tensor | None = None,
                         sliding_window: int = 0, softcap: float = 0.0) -> torch.Tensor:
    """Causal attention of ``q`` [Tq, Hq, d] (decode or prefill / mixed batches) over
    the INT2 Lloyd-Max cache (uint8 [NB, 2, B, Hkv, d/4 + 4]); returns ``out``."""
    lib = load_library()
    if q.dim() != 3 or q.stride(2) != 1 or q.stride(1) != q.shape[2]:
        raise ValueError("q must be [Tq, Hq, d] with contiguous heads")
    Tq, hq, d = q.shape
    if out is None:
        out = torch.empty((Tq, hq, d), dtype=q.dtype, device=q.device)
    if not out.is_contiguous() or out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must be contiguous with q's shape and dtype")
    if kv_cache.dtype != torch.uint8 or kv_cache.dim() != 5 or kv_cache.shape[4] != d // 4 + 4:
        raise ValueError("kv_cache must be uint8 [NB, 2, B, Hkv, d/4+4]")
    nb, two, bs, hkv, _ = kv_cache.shape
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("seqused_k", seqused_k),
                    ("block_table", block_table)):
        if t.dtype != torch.int32:
            raise ValueError(f"{name} must be int32")
    if block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("block_table must be [S, max_blocks] with unit column stride")
    S = seqused_k.shape[0]
    _check(lib.int2_paged_attention(
        _ptr(q), q.stride(0), _ptr(out), _dtype_code(q.dtype), _ptr(kv_cache), nb, bs, hkv, d, hq,
        _ptr(cu_seqlens_q.contiguous()), _ptr(seqused_k.contiguous()), S, int(max_seqlen_q),
        int(max_seqlen_k), _ptr(block_table), block_table.stride(0), float(softmax_scale),
        int(sliding_window), float(softcap), _ptr(rht_signs.contiguous()), int(num_segments),
        _ptr(segm_output), _ptr(segm_max), _ptr(segm_expsum), _stream(q.device)))
    return out


def _decode_step_args(key_new, value_new, slot_mapping, q, kv_cache, cu_seqlens_q, seqused_k,
                      max_seqlen_q, max_seqlen_k, block_table, softmax_scale, rht_signs,
                      out=None, num_segments=1, segm_output=None, segm_max=None,
                      segm_expsum=None, sliding_window=0, softcap=0.0):
    """Checks int4_decode_step's arguments; returns the C call's arguments
    without the stream, and ``out``."""
    S = seqused_k.shape[0]
    if key_new.dim() != 3 or value_new.shape != key_new.shape or key_new.shape[0] != S:
        raise ValueError("key_new and value_new must both be [S, Hkv, d], one token per sequence")
    if key_new.dtype != q.dtype or value_new.dtype != q.dtype:
        raise ValueError("key_new, value_new and q must share one dtype")
    for t in (key_new, value_new):
        if t.stride(2) != 1 or t.stride(1) != t.shape[2]:
            raise ValueError("key_new/value_new heads must be contiguous")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (S,):
        raise ValueError("slot_mapping must be int64 [S]")
    if q.dim() != 3 or q.stride(2) != 1 or q.stride(1) != q.shape[2]:
        raise ValueError("q must be [Tq, Hq, d] with contiguous heads")
    Tq, hq, d = q.shape
    if out is None:
        out = torch.empty((Tq, hq, d), dtype=q.dtype, device=q.device)
    if not out.is_contiguous() or out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must be contiguous with q's shape and dtype")
    if kv_cache.dtype != torch.uint8 or kv_cache.dim() != 5 or not kv_cache.is_contiguous():
        raise ValueError("kv_cache must be a contiguous uint8 [NB, 2, B, Hkv, d/2+4] tensor")
    nb, two, bs, hkv, _ = kv_cache.shape
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("seqused_k", seqused_k),
                    ("block_table", block_table)):
        if t.dtype != torch.int32:
            raise ValueError(f"{name} must be int32")
    if block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("block_table must be [S, max_blocks] with unit column stride")
    args = (_ptr(key_new), key_new.stride(0), _ptr(value_new), value_new.stride(0),
            _ptr(slot_mapping.contiguous()), _ptr(q), q.stride(0), _ptr(out),
            _dtype_code(q.dtype), _ptr(kv_cache), nb, bs, hkv, d, hq,
            _ptr(cu_seqlens_q.contiguous()), _ptr(seqused_k.contiguous()), S, int(max_seqlen_q),
            int(max_seqlen_k), _ptr(block_table), block_table.stride(0), float(softmax_scale),
            int(sliding_window), float(softcap), _ptr(rht_signs.contiguous()), int(num_segments),
            _ptr(segm_output), _ptr(segm_max), _ptr(segm_expsum))
    return args, out


def int4_decode_step(key_new: torch.Tensor, value_new: torch.Tensor, slot_mapping: torch.Tensor,
                     q: torch.Tensor, kv_cache: torch.Tensor, cu_seqlens_q: torch.Tensor,
                     seqused_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int,
                     block_table: torch.Tensor, softmax_scale: float, rht_signs: torch.Tensor,
                     out: torch.Tensor | None = None, num_segments: int = 1,
                     segm_output: torch.Tensor | None = None,
                     segm_max: torch.Tensor | None = None,
                     segm_expsum: torch.Tensor | None = None,
                     sliding_window: int = 0, softcap: float = 0.0) -> torch.Tensor:
    """``int4_kv_write`` of one new token per sequence (``key_new``/``value_new``
    [S, Hkv, d], token b is sequence b's last key, at ``slot_mapping[b]``), then
    ``int4_paged_attention``; one launch on the decode path.  Returns ``out``."""
    args, out = _decode_step_args(key_new, value_new, slot_mapping, q, kv_cache, cu_seqlens_q,
                                  seqused_k, max_seqlen_q, max_seqlen_k, block_table,
                                  softmax_scale, rht_signs, out, num_segments, segm_output,
                                  segm_max, segm_expsum, sliding_window, softcap)
    _check(load_library().int4_decode_step(*args, _stream(q.device)))
    return out


class DecodeStepPlan:
    """``int4_decode_step`` with its arguments checked and converted once, for
    a loop that runs the same step on the same buffers again and again (their
    contents change between calls; their storage, shapes and the other
    arguments do not).  Calling the plan launches the step on the current
    stream of the query's device and returns ``out``; the result is the plain
    call's, bit for bit.  The plan keeps its tensors alive."""

    def __init__(self, key_new, value_new, slot_mapping, q, kv_cache, cu_seqlens_q, seqused_k,
                 max_seqlen_q, max_seqlen_k, block_table, softmax_scale, rht_signs, out=None,
                 num_segments=1, segm_output=None, segm_max=None, segm_expsum=None,
                 sliding_window=0, softcap=0.0):
        slot_mapping, cu_seqlens_q, seqused_k, rht_signs = (
            t.contiguous() for t in (slot_mapping, cu_seqlens_q, seqused_k, rht_signs))
        args, out = _decode_step_args(key_new, value_new, slot_mapping, q, kv_cache,
                                      cu_seqlens_q, seqused_k, max_seqlen_q, max_seqlen_k,
                                      block_table, softmax_scale, rht_signs, out, num_segments,
                                      segm_output, segm_max, segm_expsum, sliding_window,
                                      softcap)
        self._fn = load_library().int4_decode_step
        self._args = tuple(ty(v) for ty, v in zip(self._fn.argtypes, args))
        self._keep = (key_new, value_new, slot_mapping, q, kv_cache, cu_seqlens_q, seqused_k,
                      block_table, rht_signs, segm_output, segm_max, segm_expsum)
        self._device = q.device
        self.out = out

    def __call__(self) -> torch.Tensor:
        _check(self._fn(*self._args, torch.cuda.current_stream(self._device).cuda_stream))
        return self.out
