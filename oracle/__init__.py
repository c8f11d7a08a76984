"""CPU oracle for the paged quantized KV-cache data path (ctypes binding).

TEST INFRASTRUCTURE ONLY.  This package says what the right bytes are; it is
not part of the product.  Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import it.  It shares no code with
the HIP library (``paged_quantized_kv_amd``) and never imports it.

The arithmetic lives in ``pkv_oracle.c`` (plain C, binary32 IEEE, one thread);
this module only marshals numpy arrays.  Every function cites the page it
follows in the C source.  ``build()`` compiles ``liboracle.so`` next to this
file; loading builds it only when no library is there yet.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pkv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

# IEEE binary32 step by step: no fast-math, no contraction of a*b+c.
CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
          "-fPIC", "-shared", "-Wall", "-Wextra"]


def build() -> str:
    """Compile liboracle.so from pkv_oracle.c (always recompiles)."""
    tmp = _LIB_PATH + ".tmp"
    subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, f32, u8, u16 = (ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                              ctypes.c_uint8, ctypes.c_uint16)
    lib.oracle_bf16_to_f32.argtypes = [u16]
    lib.oracle_bf16_to_f32.restype = f32
    lib.oracle_f16_to_f32.argtypes = [u16]
    lib.oracle_f16_to_f32.restype = f32
    lib.oracle_e4m3_encode.argtypes = [f32]
    lib.oracle_e4m3_encode.restype = u8
    lib.oracle_e4m3_decode.argtypes = [u8]
    lib.oracle_e4m3_decode.restype = f32
    lib.oracle_e2m1_encode.argtypes = [f32]
    lib.oracle_e2m1_encode.restype = u8
    lib.oracle_e2m1_decode.argtypes = [u8]
    lib.oracle_e2m1_decode.restype = f32
    lib.oracle_e4m3_encode_array.argtypes = [P, P, i64]
    lib.oracle_e4m3_encode_array.restype = None
    lib.oracle_e2m1_encode_array.argtypes = [P, P, i64]
    lib.oracle_e2m1_encode_array.restype = None
    lib.oracle_swizzle_offset.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.oracle_swizzle_offset.restype = ctypes.c_int
    lib.oracle_gather_indexer_k_fp8.argtypes = [P, P, P, P, P, i32, i32, i64, i64,
                                                i64, i32, i32]
    lib.oracle_gather_indexer_k_fp8.restype = None
    lib.oracle_store_indexer_k_fp8.argtypes = [P, i64, i32, P, i64, P, i64, i64, i32, i32]
    lib.oracle_store_indexer_k_fp8.restype = None
    lib.oracle_store_kv_fp4.argtypes = [P, i64, P, i64, i32, P, P, P, i64, i32, i32, i32,
                                        i64, i64, i32, f32, f32]
    lib.oracle_store_kv_fp4.restype = None
    lib.oracle_f32_to_bf16.argtypes = [f32]
    lib.oracle_f32_to_bf16.restype = u16
    lib.oracle_f32_to_f16.argtypes = [f32]
    lib.oracle_f32_to_f16.restype = u16
    lib.oracle_f32_to_bf16_array.argtypes = [P, P, i64]
    lib.oracle_f32_to_bf16_array.restype = None
    lib.oracle_f32_to_f16_array.argtypes = [P, P, i64]
    lib.oracle_f32_to_f16_array.restype = None
    lib.oracle_gather_indexer_k_dequant.argtypes = [P, P, i64, i32, P, P, i32, i32, i64, i64,
                                                    i64, i32, i32]
    lib.oracle_gather_indexer_k_dequant.restype = None
    lib.oracle_gather_kv_fp4_dequant.argtypes = [P, P, P, i64, P, i64, i32, P, P, i32, i32,
                                                 i64, i32, i32, i32, i64, i64, i32, f32, f32]
    lib.oracle_gather_kv_fp4_dequant.restype = None
    lib.oracle_fp8_mqa_logits.argtypes = [P, P, P, P, P, P, P, i64, i64, i32, i32, i64, i32]
    lib.oracle_fp8_mqa_logits.restype = None
    lib.oracle_paged_attention_decode.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32,
                                                  i32, i64, ctypes.c_double, f32, f32]
    lib.oracle_paged_attention_decode.restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray, offset: int = 0) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle buffers must be C-contiguous"
    return a.ctypes.data + offset


def _need(a, dtype, name):
    if not isinstance(a, np.ndarray) or a.dtype != dtype:
        raise TypeError(f"{name} must be a numpy {np.dtype(dtype).name} array")


# ----------------------------------------------------------------- codecs
def e4m3_encode(y) -> np.ndarray:
    """OCP E4M3FN round-to-nearest-even, saturating; elementwise."""
    y = np.ascontiguousarray(np.asarray(y, dtype=np.float32))
    out = np.empty(y.shape, dtype=np.uint8)
    _load().oracle_e4m3_encode_array(_ptr(y), _ptr(out), y.size)
    return out


def e4m3_decode(codes) -> np.ndarray:
    lib = _load()
    codes = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.oracle_e4m3_decode(int(c)) for c in codes.ravel()],
                    dtype=np.float32).reshape(codes.shape)


def e2m1_encode(y) -> np.ndarray:
    """E2M1 round-to-nearest-even (ties to even code), saturating; elementwise."""
    y = np.ascontiguousarray(np.asarray(y, dtype=np.float32))
    out = np.empty(y.shape, dtype=np.uint8)
    _load().oracle_e2m1_encode_array(_ptr(y), _ptr(out), y.size)
    return out


def e2m1_decode(codes) -> np.ndarray:
    lib = _load()
    codes = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.oracle_e2m1_decode(int(c)) for c in codes.ravel()],
                    dtype=np.float32).reshape(codes.shape)


def swizzle_offset(t: int, s: int, S: int) -> int:
    return _load().oracle_swizzle_offset(t, s, S)


# ----------------------------------------------------------------- the ops
def gather_indexer_k_fp8(kv_cache, k_fp8, k_scale, block_table, cu_seq_lens,
                         block_size, head_dim):
    """Gather codes and scale bytes into k_fp8 [T, D] / k_scale [T, 4] (in place).

    kv_cache: uint8 [num_blocks, page_stride]; block_table: int32 [R, maxb];
    cu_seq_lens: int32 [R + 1].
    """
    _need(kv_cache, np.uint8, "kv_cache")
    _need(k_fp8, np.uint8, "k_fp8")
    _need(k_scale, np.uint8, "k_scale")
    _need(block_table, np.int32, "block_table")
    _need(cu_seq_lens, np.int32, "cu_seq_lens")
    num_reqs, maxb = block_table.shape
    assert cu_seq_lens.shape == (num_reqs + 1,)
    assert k_fp8.shape[1] == head_dim and k_scale.shape[1] == 4
    assert k_fp8.shape[0] == k_scale.shape[0]
    _load().oracle_gather_indexer_k_fp8(
        _ptr(kv_cache), _ptr(k_fp8), _ptr(k_scale), _ptr(block_table),
        _ptr(cu_seq_lens), num_reqs, maxb, k_fp8.shape[0], kv_cache.shape[0],
        kv_cache.shape[1], block_size, head_dim)


SRC_DTYPES = {"bf16": 0, "f16": 1}


def f16_to_f32(bits) -> np.ndarray:
    lib = _load()
    bits = np.asarray(bits, dtype=np.uint16)
    return np.array([lib.oracle_f16_to_f32(int(b)) for b in bits.ravel()],
                    dtype=np.float32).reshape(bits.shape)


def store_indexer_k_fp8(k_bits, slot_mapping, kv_cache, block_size, head_dim, dtype="bf16"):
    """Quantize 16-bit float rows (uint16 bit patterns [T, >=D], bf16 or f16)
    into kv_cache (in place)."""
    _need(k_bits, np.uint16, "k_bits")
    _need(slot_mapping, np.int64, "slot_mapping")
    _need(kv_cache, np.uint8, "kv_cache")
    assert k_bits.ndim == 2 and k_bits.shape[1] >= head_dim
    assert slot_mapping.shape == (k_bits.shape[0],)
    _load().oracle_store_indexer_k_fp8(
        _ptr(k_bits), k_bits.shape[1], SRC_DTYPES[dtype], _ptr(slot_mapping), k_bits.shape[0],
        _ptr(kv_cache), kv_cache.shape[0], kv_cache.shape[1], block_size, head_dim)


LAYOUT_HND = 0
LAYOUT_NHD = 1


def store_kv_fp4(key_bits, value_bits, kv_cache, slot_mapping, num_heads, head_size,
                 block_size, layout, k_scale, v_scale, dtype="bf16"):
    """NVFP4 store of bf16 or f16 K/V (uint16 patterns [T, H*D]) into kv_cache (in place).

    kv_cache: uint8 [num_blocks, 2, side_bytes]; side 0 holds K, side 1 holds V.
    """
    _need(key_bits, np.uint16, "key_bits")
    _need(value_bits, np.uint16, "value_bits")
    _need(kv_cache, np.uint8, "kv_cache")
    _need(slot_mapping, np.int64, "slot_mapping")
    assert kv_cache.ndim == 3 and kv_cache.shape[1] == 2
    T = slot_mapping.shape[0]
    assert key_bits.shape[0] == T and value_bits.shape[0] == T
    assert key_bits.shape[1] >= num_heads * head_size
    side_bytes = kv_cache.shape[2]
    page_stride = 2 * side_bytes
    _load().oracle_store_kv_fp4(
        _ptr(key_bits), key_bits.shape[1], _ptr(value_bits), value_bits.shape[1],
        SRC_DTYPES[dtype], _ptr(kv_cache), _ptr(kv_cache, side_bytes), _ptr(slot_mapping), T,
        num_heads, head_size, block_size, kv_cache.shape[0], page_stride, layout,
        float(k_scale), float(v_scale))


# ----------------------------------------------------------------- reader side
OUT_DTYPES = {"bf16": 0, "f16": 1}


def f32_to_bf16(x) -> np.ndarray:
    """binary32 -> bf16 bit patterns, round to nearest even; elementwise."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_f32_to_bf16_array(_ptr(x), _ptr(out), x.size)
    return out


def f32_to_f16(x) -> np.ndarray:
    """binary32 -> binary16 bit patterns, round to nearest even; elementwise."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_f32_to_f16_array(_ptr(x), _ptr(out), x.size)
    return out


def gather_indexer_k_dequant(kv_cache, out, block_table, cu_seq_lens, block_size, head_dim,
                             dtype="bf16"):
    """Gather and dequantise into out (uint16 patterns [T, >=D], bf16 or f16; in place)."""
    _need(kv_cache, np.uint8, "kv_cache")
    _need(out, np.uint16, "out")
    _need(block_table, np.int32, "block_table")
    _need(cu_seq_lens, np.int32, "cu_seq_lens")
    num_reqs, maxb = block_table.shape
    assert cu_seq_lens.shape == (num_reqs + 1,)
    assert out.ndim == 2 and out.shape[1] >= head_dim
    _load().oracle_gather_indexer_k_dequant(
        _ptr(kv_cache), _ptr(out), out.shape[1], OUT_DTYPES[dtype], _ptr(block_table),
        _ptr(cu_seq_lens), num_reqs, maxb, out.shape[0], kv_cache.shape[0], kv_cache.shape[1],
        block_size, head_dim)


def gather_kv_fp4_dequant(kv_cache, key_out, value_out, block_table, cu_seq_lens, num_heads,
                          head_size, block_size, layout, k_scale, v_scale, dtype="bf16"):
    """NVFP4 pages back to bf16 or f16 K/V rows (uint16 patterns [T, >=H*D]; in place).

    kv_cache: uint8 [num_blocks, 2, side_bytes]; side 0 holds K, side 1 holds V.
    """
    _need(kv_cache, np.uint8, "kv_cache")
    _need(key_out, np.uint16, "key_out")
    _need(value_out, np.uint16, "value_out")
    _need(block_table, np.int32, "block_table")
    _need(cu_seq_lens, np.int32, "cu_seq_lens")
    assert kv_cache.ndim == 3 and kv_cache.shape[1] == 2
    num_reqs, maxb = block_table.shape
    assert cu_seq_lens.shape == (num_reqs + 1,)
    T = key_out.shape[0]
    assert value_out.shape[0] == T
    assert key_out.shape[1] >= num_heads * head_size and value_out.shape[1] >= num_heads * head_size
    side_bytes = kv_cache.shape[2]
    _load().oracle_gather_kv_fp4_dequant(
        _ptr(kv_cache), _ptr(kv_cache, side_bytes), _ptr(key_out), key_out.shape[1],
        _ptr(value_out), value_out.shape[1], OUT_DTYPES[dtype], _ptr(block_table),
        _ptr(cu_seq_lens), num_reqs, maxb, T, num_heads, head_size, block_size,
        kv_cache.shape[0], 2 * side_bytes, layout, float(k_scale), float(v_scale))


# ----------------------------------------------------------------- indexer logits
def fp8_mqa_logits(q_codes, k_codes, k_scale, weights, ks, ke, logits):
    """Indexer scores in binary64 (in place into logits, float64 [M, row_cols]).

    q_codes uint8 [M, H, D]; k_codes uint8 [N, D]; k_scale float32 [N];
    weights float32 [M, H]; ks, ke int32 [M].  Row i, column j - ks[i] gets
    sum_h weights[i,h] * relu(k_scale[j] * q[i,h] . k[j]) for j in [ks, ke).
    """
    _need(q_codes, np.uint8, "q_codes")
    _need(k_codes, np.uint8, "k_codes")
    _need(k_scale, np.float32, "k_scale")
    _need(weights, np.float32, "weights")
    _need(ks, np.int32, "ks")
    _need(ke, np.int32, "ke")
    _need(logits, np.float64, "logits")
    M, H, D = q_codes.shape
    N = k_codes.shape[0]
    assert k_codes.shape == (N, D) and k_scale.shape == (N,) and weights.shape == (M, H)
    assert ks.shape == (M,) and ke.shape == (M,) and logits.shape[0] == M
    _load().oracle_fp8_mqa_logits(_ptr(q_codes), _ptr(k_codes), _ptr(k_scale), _ptr(weights),
                                  _ptr(ks), _ptr(ke), _ptr(logits), logits.shape[1],
                                  logits.shape[1], M, H, N, D)


# ----------------------------------------------------------------- paged decode attention
def paged_attention_decode(query_bits, key_cache, value_cache, block_tables, context_lens,
                           num_kv_heads, scale, k_scale, v_scale):
    """Decode attention over fp8 pages in binary64; returns out float64 [S, H, D].

    query_bits uint16 bf16 patterns [S, H, D]; key_cache uint8
    [num_blocks, KVH, D/16, B, 16]; value_cache uint8 [num_blocks, KVH, D, B];
    block_tables int32 [S, maxb]; context_lens int32 [S].
    """
    _need(query_bits, np.uint16, "query_bits")
    _need(key_cache, np.uint8, "key_cache")
    _need(value_cache, np.uint8, "value_cache")
    _need(block_tables, np.int32, "block_tables")
    _need(context_lens, np.int32, "context_lens")
    S, H, D = query_bits.shape
    nb, kvh, d16, B, x = key_cache.shape
    assert kvh == num_kv_heads and d16 * 16 == D and x == 16
    assert value_cache.shape == (nb, kvh, D, B)
    assert block_tables.shape[0] == S and context_lens.shape == (S,)
    out = np.zeros((S, H, D), np.float64)
    _load().oracle_paged_attention_decode(
        _ptr(out), _ptr(query_bits), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        _ptr(context_lens), S, H, num_kv_heads, D, B, block_tables.shape[1], nb, float(scale),
        float(k_scale), float(v_scale))
    return out
