"""CPU oracle for the INT4 (and INT8) per-token-head paged KV cache: TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg
may import this package.  The product path (``int4_quantized_paged_amd``) never
imports it, and it never imports the product path: they share no code.

Thin ctypes wrapper over ``int4kv_oracle.c`` (plain C, fp32 encoding steps,
fp64 attention).  Arrays are numpy; 16-bit inputs are passed as their raw bit
patterns (``uint16``) together with a dtype tag ("f16" or "bf16").

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, textbook constructions, brute force or hand-worked
examples.  Agreement with the pages' own Triton kernels is not pinnable (the
pages print no INT4 output values and no sign generator).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_SANITIZED=1 loads the AddressSanitizer/UBSan build (liboracle_san.so;
# the process must preload the ASan runtime)
_SANITIZED = os.environ.get("ORACLE_SANITIZED") == "1"
_LIB_PATH = os.path.join(_HERE, "liboracle_san.so" if _SANITIZED else "liboracle.so")
_lib = None

_DT = {"f16": 0, "bf16": 1}


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b  # compile on first use (gcc is everywhere)
        _b.build(sanitized=_SANITIZED)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.oracle_rht_forward_f32.argtypes = [P, i32, P]
    lib.oracle_rht_inverse_f64.argtypes = [P, i32, P]
    lib.oracle_pack_nibbles.argtypes = [P, i32, P]
    lib.oracle_unpack_nibbles.argtypes = [P, i32, P]
    lib.oracle_stego_encode.argtypes = [ctypes.c_float, i32]
    lib.oracle_stego_encode.restype = ctypes.c_uint32
    lib.oracle_stego_decode.argtypes = [ctypes.c_uint32, P, P]
    lib.oracle_quantize_row.argtypes = [P, i32, P, P]
    lib.oracle_kv_write.argtypes = [P, i64, P, i64, i32, P, i32, P, i32, i32, i32, i32, P]
    lib.oracle_decode_row.argtypes = [P, i32, P, P]
    lib.oracle_attention_plain.argtypes = [P, i64, i32, P, i32, i32, i32, i32, i32,
                                           P, P, i32, P, i32, f64, P, i32, f64, P]
    lib.oracle_attention_method.argtypes = [P, i64, i32, P, i32, i32, i32, i32, i32,
                                            P, P, i32, P, i32, f64, P, i32, i32, f64, P]
    lib.oracle_quantize_row_int8.argtypes = [P, i32, P, P]
    lib.oracle_kv_write_int8.argtypes = [P, i64, P, i64, i32, P, i32, P, i32, i32, i32, i32]
    lib.oracle_decode_row_int8.argtypes = [P, i32, P]
    lib.oracle_attention_plain_int8.argtypes = [P, i64, i32, P, i32, i32, i32, i32, i32,
                                                P, P, i32, P, i32, f64, i32, f64, P]
    lib.oracle_lloyd_max4.argtypes = [P, P, P]
    lib.oracle_quantize_row_int2.argtypes = [P, i32, P, P]
    lib.oracle_kv_write_int2.argtypes = [P, i64, P, i64, i32, P, i32, P, i32, i32, i32, i32, P]
    lib.oracle_decode_row_int2.argtypes = [P, i32, P, P]
    lib.oracle_attention_plain_int2.argtypes = [P, i64, i32, P, i32, i32, i32, i32, i32,
                                                P, P, i32, P, i32, f64, P, i32, f64, P]
    lib.oracle_set_num_threads.argtypes = [i32]
    lib.oracle_max_threads.restype = i32
    _lib = lib
    return lib


def set_num_threads(n: int) -> None:
    """OpenMP threads of the write and plain-attention loops (timing only: the
    results do not depend on it)."""
    _load().oracle_set_num_threads(int(n))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def row_bytes(head_size: int) -> int:
    """Packed row: head_size/2 code bytes + 4 scale bytes."""
    return head_size // 2 + 4


def rht_forward_f32(x: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """fp32 forward rotation y = H (D x) of each row of ``x`` [..., d]."""
    x = _c(x, np.float32).copy()
    s = _c(signs, np.float32)
    d = x.shape[-1]
    flat = x.reshape(-1, d)
    lib = _load()
    for r in range(flat.shape[0]):
        row = flat[r]
        lib.oracle_rht_forward_f32(_p(row), d, _p(s))
    return flat.reshape(x.shape)


def rht_inverse_f64(y: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """fp64 inverse rotation x = D (H y) / d of each row of ``y``."""
    y = _c(y, np.float64).copy()
    s = _c(signs, np.float32)
    d = y.shape[-1]
    flat = y.reshape(-1, d)
    lib = _load()
    for r in range(flat.shape[0]):
        row = flat[r]
        lib.oracle_rht_inverse_f64(_p(row), d, _p(s))
    return flat.reshape(y.shape)


def pack_nibbles(q: np.ndarray) -> np.ndarray:
    q = _c(q, np.uint8)
    out = np.zeros(q.size // 2, dtype=np.uint8)
    _load().oracle_pack_nibbles(_p(q), q.size, _p(out))
    return out


def unpack_nibbles(b: np.ndarray) -> np.ndarray:
    b = _c(b, np.uint8)
    out = np.zeros(b.size * 2, dtype=np.uint8)
    _load().oracle_unpack_nibbles(_p(b), b.size * 2, _p(out))
    return out


def stego_encode(s: float, zp: int) -> int:
    return int(_load().oracle_stego_encode(ctypes.c_float(s), int(zp)))


def stego_decode(word: int) -> tuple[float, int]:
    st = np.zeros(1, np.float32)
    zp = np.zeros(1, np.int32)
    _load().oracle_stego_decode(ctypes.c_uint32(word), _p(st), _p(zp))
    return float(st[0]), int(zp[0])


def quantize_row(y: np.ndarray) -> tuple[np.ndarray, int]:
    """Quantize one rotated fp32 row: (packed code bytes, scale word)."""
    y = _c(y, np.float32)
    b = np.zeros(y.size // 2, dtype=np.uint8)
    w = np.zeros(1, dtype=np.uint32)
    _load().oracle_quantize_row(_p(y), y.size, _p(b), _p(w))
    return b, int(w[0])


def cache_shape(num_blocks: int, block_size: int, num_kv_heads: int, head_size: int):
    return (num_blocks, 2, block_size, num_kv_heads, row_bytes(head_size))


def kv_write(key_bits: np.ndarray, value_bits: np.ndarray, dtype: str,
             slot_mapping: np.ndarray, cache: np.ndarray, signs: np.ndarray) -> None:
    """Write tokens into ``cache`` (uint8 [NB, 2, B, Hkv, d/2+4]) in place.

    key_bits/value_bits: uint16 [T, Hkv, d] raw 16-bit patterns.
    """
    assert cache.dtype == np.uint8 and cache.flags.c_contiguous and cache.ndim == 5
    nb, two, bs, hkv, r = cache.shape
    k = _c(key_bits, np.uint16)
    v = _c(value_bits, np.uint16)
    T, hk, d = k.shape
    assert two == 2 and hk == hkv and r == row_bytes(d) and v.shape == k.shape
    sm = _c(slot_mapping, np.int64)
    assert sm.shape == (T,)
    s = _c(signs, np.float32)
    _load().oracle_kv_write(_p(k), hkv * d, _p(v), hkv * d, _DT[dtype], _p(sm), T,
                            _p(cache), nb, bs, hkv, d, _p(s))


def decode_row(row: np.ndarray, head_size: int, signs: np.ndarray) -> np.ndarray:
    """Original-domain fp64 values of one packed row."""
    row = _c(row, np.uint8)
    out = np.zeros(head_size, np.float64)
    _load().oracle_decode_row(_p(row), head_size, _p(_c(signs, np.float32)), _p(out))
    return out


def _attn_args(q_bits, dtype, cache, cu_seqlens_q, seqused_k, block_table, num_q_heads):
    q = _c(q_bits, np.uint16)
    nb, two, bs, hkv, r = cache.shape
    assert bs <= 1024
    d = (r - 4) * 2
    Tq = q.shape[0]
    assert q.shape == (Tq, num_q_heads, d)
    cu = _c(cu_seqlens_q, np.int32)
    su = _c(seqused_k, np.int32)
    bt = _c(block_table, np.int32)
    assert bt.ndim == 2 and cu.shape == (su.shape[0] + 1,)
    return q, nb, bs, hkv, d, Tq, cu, su, bt


def attention_plain(q_bits, dtype, cache, cu_seqlens_q, seqused_k, block_table,
                    softmax_scale, signs, num_q_heads, window: int = 0,
                    softcap: float = 0.0) -> np.ndarray:
    """Causal softmax attention over the decoded cache, fp64 [Tq, Hq, d].
    window > 0: the query at position pos sees keys [pos - window + 1, pos].
    softcap > 0: scores z become softcap * tanh(z / softcap) before the softmax."""
    q, nb, bs, hkv, d, Tq, cu, su, bt = _attn_args(q_bits, dtype, cache, cu_seqlens_q,
                                                   seqused_k, block_table, num_q_heads)
    out = np.zeros((Tq, num_q_heads, d), np.float64)
    cache = _c(cache, np.uint8)
    _load().oracle_attention_plain(_p(q), num_q_heads * d, _DT[dtype], _p(cache), nb, bs, hkv,
                                   d, num_q_heads, _p(cu), _p(su), su.shape[0], _p(bt),
                                   bt.shape[1], float(softmax_scale),
                                   _p(_c(signs, np.float32)), int(window), float(softcap),
                                   _p(out))
    return out


def attention_method(q_bits, dtype, cache, cu_seqlens_q, seqused_k, block_table,
                     softmax_scale, signs, num_q_heads, num_segments=1,
                     window: int = 0, softcap: float = 0.0) -> np.ndarray:
    """Same result as attention_plain, computed the way the packed read path does."""
    q, nb, bs, hkv, d, Tq, cu, su, bt = _attn_args(q_bits, dtype, cache, cu_seqlens_q,
                                                   seqused_k, block_table, num_q_heads)
    out = np.zeros((Tq, num_q_heads, d), np.float64)
    cache = _c(cache, np.uint8)
    _load().oracle_attention_method(_p(q), num_q_heads * d, _DT[dtype], _p(cache), nb, bs, hkv,
                                    d, num_q_heads, _p(cu), _p(su), su.shape[0], _p(bt),
                                    bt.shape[1], float(softmax_scale),
                                    _p(_c(signs, np.float32)), int(num_segments),
                                    int(window), float(softcap), _p(out))
    return out


# ---- INT8 per-token-head mode: rows of d int8 codes + an fp32 scale, no rotation


def cache_shape_int8(num_blocks: int, block_size: int, num_kv_heads: int, head_size: int):
    return (num_blocks, 2, block_size, num_kv_heads, head_size + 4)


def quantize_row_int8(x: np.ndarray) -> tuple[np.ndarray, float]:
    """Quantize one fp32 row: (int8 codes, fp32 scale)."""
    x = _c(x, np.float32)
    codes = np.zeros(x.size, dtype=np.int8)
    s = np.zeros(1, dtype=np.float32)
    _load().oracle_quantize_row_int8(_p(x), x.size, _p(codes), _p(s))
    return codes, float(s[0])


def kv_write_int8(key_bits: np.ndarray, value_bits: np.ndarray, dtype: str,
                  slot_mapping: np.ndarray, cache: np.ndarray) -> None:
    """Write tokens into ``cache`` (uint8 [NB, 2, B, Hkv, d+4]) in place."""
    assert cache.dtype == np.uint8 and cache.flags.c_contiguous and cache.ndim == 5
    nb, two, bs, hkv, r = cache.shape
    k = _c(key_bits, np.uint16)
    v = _c(value_bits, np.uint16)
    T, hk, d = k.shape
    assert two == 2 and hk == hkv and r == d + 4 and v.shape == k.shape
    sm = _c(slot_mapping, np.int64)
    assert sm.shape == (T,)
    _load().oracle_kv_write_int8(_p(k), hkv * d, _p(v), hkv * d, _DT[dtype], _p(sm), T,
                                 _p(cache), nb, bs, hkv, d)


def decode_row_int8(row: np.ndarray, head_size: int) -> np.ndarray:
    row = _c(row, np.uint8)
    out = np.zeros(head_size, np.float64)
    _load().oracle_decode_row_int8(_p(row), head_size, _p(out))
    return out


def attention_plain_int8(q_bits, dtype, cache, cu_seqlens_q, seqused_k, block_table,
                         softmax_scale, num_q_heads, window: int = 0,
                         softcap: float = 0.0) -> np.ndarray:
    """Causal softmax attention over the dequantised INT8 cache, fp64 [Tq, Hq, d]."""
    q = _c(q_bits, np.uint16)
    nb, two, bs, hkv, r = cache.shape
    d = r - 4
    Tq = q.shape[0]
    assert q.shape == (Tq, num_q_heads, d)
    cu = _c(cu_seqlens_q, np.int32)
    su = _c(seqused_k, np.int32)
    bt = _c(block_table, np.int32)
    out = np.zeros((Tq, num_q_heads, d), np.float64)
    cache = _c(cache, np.uint8)
    _load().oracle_attention_plain_int8(_p(q), num_q_heads * d, _DT[dtype], _p(cache), nb, bs,
                                        hkv, d, num_q_heads, _p(cu), _p(su), su.shape[0],
                                        _p(bt), bt.shape[1], float(softmax_scale), int(window),
                                        float(softcap), _p(out))
    return out


# ---- INT2 Lloyd-Max mode: rows of d/4 code bytes (4 codes each) + an fp32 scale,
# over the same rotation as the INT4 mode


def lloyd_max4() -> tuple[float, float, float]:
    """The 4-level Lloyd-Max quantizer of N(0, 1): levels (a, b) and threshold t
    (levels -b, -a, a, b; thresholds -t, 0, t)."""
    v = np.zeros(3, np.float64)
    _load().oracle_lloyd_max4(_p(v[0:1]), _p(v[1:2]), _p(v[2:3]))
    return float(v[0]), float(v[1]), float(v[2])


def cache_shape_int2(num_blocks: int, block_size: int, num_kv_heads: int, head_size: int):
    return (num_blocks, 2, block_size, num_kv_heads, head_size // 4 + 4)


def quantize_row_int2(y: np.ndarray) -> tuple[np.ndarray, float]:
    """Quantize one rotated fp32 row: (d/4 code bytes, fp32 scale)."""
    y = _c(y, np.float32)
    b = np.zeros(y.size // 4, dtype=np.uint8)
    s = np.zeros(1, dtype=np.float32)
    _load().oracle_quantize_row_int2(_p(y), y.size, _p(b), _p(s))
    return b, float(s[0])


def kv_write_int2(key_bits: np.ndarray, value_bits: np.ndarray, dtype: str,
                  slot_mapping: np.ndarray, cache: np.ndarray, signs: np.ndarray) -> None:
    """Write tokens into ``cache`` (uint8 [NB, 2, B, Hkv, d/4+4]) in place."""
    assert cache.dtype == np.uint8 and cache.flags.c_contiguous and cache.ndim == 5
    nb, two, bs, hkv, r = cache.shape
    k = _c(key_bits, np.uint16)
    v = _c(value_bits, np.uint16)
    T, hk, d = k.shape
    assert two == 2 and hk == hkv and r == d // 4 + 4 and v.shape == k.shape
    sm = _c(slot_mapping, np.int64)
    sg = _c(signs, np.float32)
    assert sm.shape == (T,) and sg.shape == (d,)
    _load().oracle_kv_write_int2(_p(k), hkv * d, _p(v), hkv * d, _DT[dtype], _p(sm), T,
                                 _p(cache), nb, bs, hkv, d, _p(sg))


def decode_row_int2(row: np.ndarray, head_size: int, signs: np.ndarray) -> np.ndarray:
    row = _c(row, np.uint8)
    sg = _c(signs, np.float32)
    out = np.zeros(head_size, np.float64)
    _load().oracle_decode_row_int2(_p(row), head_size, _p(sg), _p(out))
    return out


def attention_plain_int2(q_bits, dtype, cache, cu_seqlens_q, seqused_k, block_table,
                         softmax_scale, signs, num_q_heads, window: int = 0,
                         softcap: float = 0.0) -> np.ndarray:
    """Causal softmax attention over the dequantised INT2 cache, fp64 [Tq, Hq, d]."""
    q = _c(q_bits, np.uint16)
    nb, two, bs, hkv, r = cache.shape
    d = (r - 4) * 4
    Tq = q.shape[0]
    assert q.shape == (Tq, num_q_heads, d)
    cu = _c(cu_seqlens_q, np.int32)
    su = _c(seqused_k, np.int32)
    bt = _c(block_table, np.int32)
    sg = _c(signs, np.float32)
    out = np.zeros((Tq, num_q_heads, d), np.float64)
    cache = _c(cache, np.uint8)
    _load().oracle_attention_plain_int2(_p(q), num_q_heads * d, _DT[dtype], _p(cache), nb, bs,
                                        hkv, d, num_q_heads, _p(cu), _p(su), su.shape[0],
                                        _p(bt), bt.shape[1], float(softmax_scale), _p(sg),
                                        int(window), float(softcap), _p(out))
    return out
