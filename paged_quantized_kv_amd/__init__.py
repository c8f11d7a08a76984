"""Python binding of libpkv (include/pkv.h): argument marshalling only.

Every function takes torch tensors, checks dtypes and shapes, derives the
sizes the C ABI needs from tensor shapes and strides, and calls the
identically named C entry point on torch's current HIP stream.  All
arithmetic runs in libpkv's gfx950 kernels; there is no fallback.  If
libpkv.so is missing, importing this package raises.

torch is imported before libpkv.so is loaded so that the library binds to
the HIP runtime torch already holds (one runtime per process).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "pkv_gather_indexer_k_fp8", "pkv_store_indexer_k_fp8", "pkv_store_kv_fp4",
    "pkv_gather_indexer_k_dequant", "pkv_gather_kv_fp4_dequant", "pkv_fp8_mqa_logits",
    "pkv_paged_attention_decode", "paged_attention_workspace", "pkv_attention_balanced_units",
    "pkv_paged_attention_decode_noalloc", "ATTENTION_SCRATCH_BYTES",
    "pkv_diag_narrow",
    "pkv_diag_encode_e4m3", "pkv_diag_encode_e2m1", "PkvError", "LAYOUT_HND", "LAYOUT_NHD",
    "library_path", "abi_version",
]

LAYOUT_HND = 0
LAYOUT_NHD = 1
DTYPE_BF16 = 0
DTYPE_F16 = 1
SCALE_BYTES = 4
ATTENTION_SCRATCH_BYTES = 32 << 20   # PKV_ATTENTION_SCRATCH_BYTES

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv.so")


class PkvError(RuntimeError):
    """A libpkv entry point returned a non-zero status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def _hip_runtimes_loaded():
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    paths.add(os.path.realpath(line.split()[-1]))
    except OSError:
        pass
    return paths


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"libpkv.so not found at {_LIB_PATH}; build it with __graft_entry__.build() "
            "or python -m paged_quantized_kv_amd.build")
    lib = ctypes.CDLL(_LIB_PATH)
    runtimes = _hip_runtimes_loaded()
    if len(runtimes) > 1:
        raise ImportError(f"more than one HIP runtime is loaded: {sorted(runtimes)}")
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.pkv_abi_version.restype = ctypes.c_int
    lib.pkv_last_error.restype = ctypes.c_char_p
    lib.pkv_gather_indexer_k_fp8.argtypes = [P, P, P, P, P, i32, i32, i64, i64, i64, i32, i32, P]
    lib.pkv_store_indexer_k_fp8.argtypes = [P, i64, i32, P, i64, P, i64, i64, i32, i32, P]
    lib.pkv_store_kv_fp4.argtypes = [P, i64, P, i64, i32, P, P, P, i64, i32, i32, i32, i64, i64,
                                     i32, P, P, P]
    lib.pkv_gather_indexer_k_dequant.argtypes = [P, P, i64, i32, P, P, i32, i32, i64, i64,
                                                 i64, i32, i32, P]
    lib.pkv_gather_kv_fp4_dequant.argtypes = [P, P, P, i64, P, i64, i32, P, P, i32, i32, i64,
                                              i32, i32, i32, i64, i64, i32, P, P, P]
    lib.pkv_diag_encode_e4m3.argtypes = [P, P, i64, P]
    lib.pkv_diag_narrow.argtypes = [P, P, i64, i32, P]
    lib.pkv_fp8_mqa_logits.argtypes = [P, i64, P, P, P, P, P, P, i64, i64, i32, i32, i64, i32, P]
    lib.pkv_diag_encode_e2m1.argtypes = [P, P, i64, P]
    f32 = ctypes.c_float
    lib.pkv_paged_attention_decode.argtypes = [P, P, P, P, P, P, P, P, P, i32, i32, i32, i32, i32,
                                               i32, i32, i64, f32, f32, f32, i32, P]
    lib.pkv_paged_attention_decode_noalloc.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32,
                                                       i32, i32, i32, i64, f32, f32, f32, i32, P]
    lib.pkv_attention_balanced_units.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.pkv_attention_balanced_units.restype = i64
    for name in ("pkv_gather_indexer_k_fp8", "pkv_store_indexer_k_fp8", "pkv_store_kv_fp4",
                 "pkv_gather_indexer_k_dequant", "pkv_gather_kv_fp4_dequant",
                 "pkv_diag_encode_e4m3", "pkv_diag_encode_e2m1", "pkv_diag_narrow",
                 "pkv_fp8_mqa_logits", "pkv_paged_attention_decode",
                 "pkv_paged_attention_decode_noalloc"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


_lib = _load()


def abi_version() -> int:
    return _lib.pkv_abi_version()


def _check(status: int):
    if status != 0:
        raise PkvError(status, _lib.pkv_last_error().decode(errors="replace"))


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dev(t: torch.Tensor, name: str, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device (cuda/HIP) tensor, got {t.device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _row_stride(t: torch.Tensor, natural: int) -> int:
    """stride(0) of a row-major view; an empty tensor's strides carry no
    layout (torch and numpy give empty arrays arbitrary strides), so it gets
    the natural one."""
    return t.stride(0) if t.numel() else natural


def _src_dtype(t: torch.Tensor, name: str) -> int:
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float16:
        return DTYPE_F16
    raise TypeError(f"{name} must be bfloat16 or float16, got {t.dtype}")


def _contig(t: torch.Tensor, name: str):
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def pkv_gather_indexer_k_fp8(kv_cache, k_fp8, k_scale, block_table, cu_seq_lens,
                             block_size: int | None = None, stream=None):
    """Gather fp8 key rows and their scales (vLLM cp_gather_indexer_k_quant_cache).

    kv_cache:   uint8, first dim num_blocks, page = [B*D codes | B*4 scale bytes]
                contiguous within a page (stride(0) = page stride in bytes).
                A 3-D [num_blocks, B, D+4] view supplies block_size itself.
    k_fp8:      uint8 (or float8_e4m3fn) [num_tokens, D], written.
    k_scale:    uint8 [num_tokens, 4] or float32 [num_tokens] / [num_tokens, 1], written.
    block_table int32 [num_reqs, max_blocks_per_req], cu_seq_lens int32 [num_reqs + 1].
    """
    _dev(kv_cache, "kv_cache", torch.uint8)
    _dev(k_fp8, "k_fp8")
    if k_fp8.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise TypeError("k_fp8 must be uint8 or float8_e4m3fn")
    _dev(k_scale, "k_scale")
    _dev(block_table, "block_table", torch.int32)
    _dev(cu_seq_lens, "cu_seq_lens", torch.int32)
    for t, n in ((k_fp8, "k_fp8"), (k_scale, "k_scale"), (block_table, "block_table"),
                 (cu_seq_lens, "cu_seq_lens")):
        _contig(t, n)
    if k_fp8.dim() != 2:
        raise ValueError("k_fp8 must be [num_tokens, head_dim]")
    num_tokens, head_dim = k_fp8.shape
    if k_scale.dtype == torch.uint8:
        ok = k_scale.dim() == 2 and tuple(k_scale.shape) == (num_tokens, SCALE_BYTES)
    elif k_scale.dtype == torch.float32:
        ok = k_scale.numel() == num_tokens
    else:
        ok = False
    if not ok:
        raise ValueError("k_scale must be uint8 [num_tokens, 4] or float32 [num_tokens]")
    if block_table.dim() != 2 or cu_seq_lens.dim() != 1:
        raise ValueError("block_table must be 2-D and cu_seq_lens 1-D")
    num_reqs, max_blocks = block_table.shape
    if cu_seq_lens.numel() != num_reqs + 1:
        raise ValueError(f"cu_seq_lens must have num_reqs + 1 = {num_reqs + 1} entries")
    if block_size is None:
        if kv_cache.dim() != 3:
            raise ValueError("pass block_size, or kv_cache as [num_blocks, block_size, D + 4]")
        block_size = kv_cache.shape[1]
    if kv_cache.dim() >= 2 and kv_cache.stride(-1) != 1:
        raise ValueError("kv_cache pages must be contiguous")
    _check(_lib.pkv_gather_indexer_k_fp8(
        kv_cache.data_ptr(), k_fp8.data_ptr(), k_scale.data_ptr(), block_table.data_ptr(),
        cu_seq_lens.data_ptr(), num_reqs, max_blocks, num_tokens,
        kv_cache.shape[0], kv_cache.stride(0), block_size, head_dim, _stream(stream)))


def pkv_store_indexer_k_fp8(k, slot_mapping, kv_cache, block_size: int | None = None,
                            stream=None):
    """fp8 per-token quantize of bf16/fp16 k [num_tokens, D] and scatter into kv_cache."""
    _dev(k, "k")
    k_dtype = _src_dtype(k, "k")
    _dev(slot_mapping, "slot_mapping", torch.int64)
    _dev(kv_cache, "kv_cache", torch.uint8)
    _contig(slot_mapping, "slot_mapping")
    if k.dim() != 2 or (k.numel() and k.stride(1) != 1):
        raise ValueError("k must be [num_tokens, head_dim] with unit element stride")
    num_tokens, head_dim = k.shape
    if slot_mapping.numel() != num_tokens:
        raise ValueError("slot_mapping must have num_tokens entries")
    if block_size is None:
        if kv_cache.dim() != 3:
            raise ValueError("pass block_size, or kv_cache as [num_blocks, block_size, D + 4]")
        block_size = kv_cache.shape[1]
    if kv_cache.stride(-1) != 1:
        raise ValueError("kv_cache pages must be contiguous")
    _check(_lib.pkv_store_indexer_k_fp8(
        k.data_ptr(), _row_stride(k, head_dim), k_dtype, slot_mapping.data_ptr(), num_tokens,
        kv_cache.data_ptr(),
        kv_cache.shape[0], kv_cache.stride(0), block_size, head_dim, _stream(stream)))


def pkv_store_kv_fp4(key, value, key_cache, value_cache, slot_mapping, k_scale, v_scale,
                     block_size: int | None = None, layout: int | None = None, stream=None):
    """NVFP4 store of bf16/fp16 key/value [num_tokens, H, D] into kv_cache[:,0] / kv_cache[:,1].

    key_cache / value_cache: uint8 views of the two page sides.  A 4-D
    [num_blocks, block_size, num_heads, D/2 + D/16] view supplies block_size
    and the layout from its strides (HND when stride(2) > stride(1)), as the
    page's dispatcher does; a 2-D [num_blocks, side_bytes] view needs both
    passed explicitly.  k_scale / v_scale: float32 device scalars.
    """
    _dev(key, "key")
    _dev(value, "value")
    src_dtype = _src_dtype(key, "key")
    if value.dtype != key.dtype:
        raise TypeError("key and value must have the same dtype")
    _dev(key_cache, "key_cache", torch.uint8)
    _dev(value_cache, "value_cache", torch.uint8)
    _dev(slot_mapping, "slot_mapping", torch.int64)
    _dev(k_scale, "k_scale", torch.float32)
    _dev(v_scale, "v_scale", torch.float32)
    _contig(slot_mapping, "slot_mapping")
    if key.dim() != 3 or value.shape != key.shape:
        raise ValueError("key and value must both be [num_tokens, num_heads, head_size]")
    num_tokens, num_heads, head_size = key.shape
    for t, n in ((key, "key"), (value, "value")):
        if t.numel() and (t.stride(2) != 1 or t.stride(1) != head_size):
            raise ValueError(f"{n}: heads and elements must be contiguous (only stride(0) is free)")
    if slot_mapping.numel() != num_tokens:
        raise ValueError("slot_mapping must have num_tokens entries")
    if k_scale.numel() != 1 or v_scale.numel() != 1:
        raise ValueError("k_scale and v_scale must be scalars")
    if key_cache.dim() == 4:
        full_dim = head_size // 2 + head_size // 16
        if key_cache.shape[3] != full_dim or key_cache.shape[2] != num_heads:
            raise ValueError(f"key_cache must be [num_blocks, block_size, {num_heads}, {full_dim}]")
        if block_size is None:
            block_size = key_cache.shape[1]
        if layout is None:
            layout = LAYOUT_HND if key_cache.stride(2) > key_cache.stride(1) else LAYOUT_NHD
    elif block_size is None or layout is None:
        raise ValueError("pass block_size and layout, or 4-D cache views")
    if key_cache.stride(0) != value_cache.stride(0) or key_cache.shape[0] != value_cache.shape[0]:
        raise ValueError("key_cache and value_cache must share num_blocks and page stride")
    _check(_lib.pkv_store_kv_fp4(
        key.data_ptr(), _row_stride(key, num_heads * head_size), value.data_ptr(),
        _row_stride(value, num_heads * head_size), src_dtype,
        key_cache.data_ptr(),
        value_cache.data_ptr(), slot_mapping.data_ptr(), num_tokens, num_heads, head_size,
        block_size, key_cache.shape[0], key_cache.stride(0), layout, k_scale.data_ptr(),
        v_scale.data_ptr(), _stream(stream)))


def _table_args(block_table, cu_seq_lens):
    _dev(block_table, "block_table", torch.int32)
    _dev(cu_seq_lens, "cu_seq_lens", torch.int32)
    _contig(block_table, "block_table")
    _contig(cu_seq_lens, "cu_seq_lens")
    if block_table.dim() != 2 or cu_seq_lens.dim() != 1:
        raise ValueError("block_table must be 2-D and cu_seq_lens 1-D")
    num_reqs, max_blocks = block_table.shape
    if cu_seq_lens.numel() != num_reqs + 1:
        raise ValueError(f"cu_seq_lens must have num_reqs + 1 = {num_reqs + 1} entries")
    return num_reqs, max_blocks


def pkv_gather_indexer_k_dequant(kv_cache, out, block_table, cu_seq_lens,
                                 block_size: int | None = None, stream=None):
    """Gather the indexer keys of every request and dequantise them into out.

    kv_cache:   uint8 indexer pages, as for pkv_gather_indexer_k_fp8.
    out:        bfloat16 or float16 [num_tokens, head_dim] (row stride free), written:
                out[row, d] = round(E4M3 decode(code) * scale).
    block_table int32 [num_reqs, max_blocks_per_req], cu_seq_lens int32 [num_reqs + 1].
    """
    _dev(kv_cache, "kv_cache", torch.uint8)
    _dev(out, "out")
    out_dtype = _src_dtype(out, "out")
    if out.dim() != 2 or (out.numel() and out.stride(1) != 1):
        raise ValueError("out must be [num_tokens, head_dim] with contiguous rows")
    num_tokens, head_dim = out.shape
    num_reqs, max_blocks = _table_args(block_table, cu_seq_lens)
    if block_size is None:
        if kv_cache.dim() != 3:
            raise ValueError("pass block_size, or kv_cache as [num_blocks, block_size, D + 4]")
        block_size = kv_cache.shape[1]
    if kv_cache.dim() >= 2 and kv_cache.stride(-1) != 1:
        raise ValueError("kv_cache pages must be contiguous")
    _check(_lib.pkv_gather_indexer_k_dequant(
        kv_cache.data_ptr(), out.data_ptr(), _row_stride(out, head_dim), out_dtype,
        block_table.data_ptr(),
        cu_seq_lens.data_ptr(), num_reqs, max_blocks, num_tokens, kv_cache.shape[0],
        kv_cache.stride(0), block_size, head_dim, _stream(stream)))


def pkv_gather_kv_fp4_dequant(key_cache, value_cache, key_out, value_out, block_table,
                              cu_seq_lens, k_scale, v_scale, block_size: int | None = None,
                              layout: int | None = None, stream=None):
    """Read NVFP4 K/V pages back into bfloat16 or float16 rows.

    key_cache / value_cache: uint8 views of the two page sides, as for
    pkv_store_kv_fp4 (a 4-D [num_blocks, block_size, num_heads, D/2 + D/16]
    view supplies block_size and the layout).  key_out / value_out: bf16 or
    fp16 [num_tokens, num_heads, head_size] (only stride(0) free), written:
    element = round(E2M1 decode(code) * block scale * k_scale (v_scale)).
    """
    _dev(key_out, "key_out")
    _dev(value_out, "value_out")
    out_dtype = _src_dtype(key_out, "key_out")
    if value_out.dtype != key_out.dtype:
        raise TypeError("key_out and value_out must have the same dtype")
    _dev(key_cache, "key_cache", torch.uint8)
    _dev(value_cache, "value_cache", torch.uint8)
    _dev(k_scale, "k_scale", torch.float32)
    _dev(v_scale, "v_scale", torch.float32)
    if key_out.dim() != 3 or value_out.shape != key_out.shape:
        raise ValueError("key_out and value_out must both be [num_tokens, num_heads, head_size]")
    num_tokens, num_heads, head_size = key_out.shape
    for t, n in ((key_out, "key_out"), (value_out, "value_out")):
        if t.numel() and (t.stride(2) != 1 or t.stride(1) != head_size):
            raise ValueError(f"{n}: heads and elements must be contiguous (only stride(0) is free)")
    if k_scale.numel() != 1 or v_scale.numel() != 1:
        raise ValueError("k_scale and v_scale must be scalars")
    num_reqs, max_blocks = _table_args(block_table, cu_seq_lens)
    if key_cache.dim() == 4:
        full_dim = head_size // 2 + head_size // 16
        if key_cache.shape[3] != full_dim or key_cache.shape[2] != num_heads:
            raise ValueError(f"key_cache must be [num_blocks, block_size, {num_heads}, {full_dim}]")
        if block_size is None:
            block_size = key_cache.shape[1]
        if layout is None:
            layout = LAYOUT_HND if key_cache.stride(2) > key_cache.stride(1) else LAYOUT_NHD
    elif block_size is None or layout is None:
        raise ValueError("pass block_size and layout, or 4-D cache views")
    if key_cache.stride(0) != value_cache.stride(0) or key_cache.shape[0] != value_cache.shape[0]:
        raise ValueError("key_cache and value_cache must share num_blocks and page stride")
    _check(_lib.pkv_gather_kv_fp4_dequant(
        key_cache.data_ptr(), value_cache.data_ptr(), key_out.data_ptr(),
        _row_stride(key_out, num_heads * head_size), value_out.data_ptr(),
        _row_stride(value_out, num_heads * head_size), out_dtype, block_table.data_ptr(),
        cu_seq_lens.data_ptr(), num_reqs, max_blocks, num_tokens, num_heads, head_size,
        block_size, key_cache.shape[0], key_cache.stride(0), layout, k_scale.data_ptr(),
        v_scale.data_ptr(), _stream(stream)))


def pkv_diag_encode_e4m3(y, out, stream=None):
    """out[i] = device E4M3 code of y[i] (defined for |y| < 464)."""
    _contig(_dev(y, "y", torch.float32), "y")
    _contig(_dev(out, "out", torch.uint8), "out")
    if out.numel() != y.numel():
        raise ValueError("out must have y.numel() bytes")
    _check(_lib.pkv_diag_encode_e4m3(y.data_ptr(), out.data_ptr(), y.numel(), _stream(stream)))


def pkv_diag_encode_e2m1(y, out, stream=None):
    """out[i] = device E2M1 code of y[i] in the low nibble (every non-NaN y)."""
    _contig(_dev(y, "y", torch.float32), "y")
    _contig(_dev(out, "out", torch.uint8), "out")
    if out.numel() != y.numel():
        raise ValueError("out must have y.numel() bytes")
    _check(_lib.pkv_diag_encode_e2m1(y.data_ptr(), out.data_ptr(), y.numel(), _stream(stream)))


def pkv_diag_narrow(x, out, stream=None):
    """out[i] = device bf16 / fp16 rounding of x[i] (the dequantising gathers' output step)."""
    _contig(_dev(x, "x", torch.float32), "x")
    _contig(_dev(out, "out"), "out")
    dt = _src_dtype(out, "out")
    if out.numel() != x.numel():
        raise ValueError("out must have x.numel() elements")
    _check(_lib.pkv_diag_narrow(x.data_ptr(), out.data_ptr(), x.numel(), dt, _stream(stream)))


def pkv_fp8_mqa_logits(q, k, k_scale, weights, ks, ke, logits, stream=None):
    """Indexer scores of query tokens against the gathered keys.

    q:        float8_e4m3fn or uint8 [num_q, num_heads, 128] (heads and elements
              contiguous, token stride free).
    k:        float8_e4m3fn or uint8 [num_k, 128] contiguous (the gather's k_fp8).
    k_scale:  float32 [num_k] (or the gather's uint8 [num_k, 4] scale bytes).
    weights:  float32 [num_q, num_heads] contiguous.
    ks, ke:   int32 [num_q]: key range of each query token.
    logits:   float32 [num_q, row_cols] (row stride free), written at column
              j - ks[i] for j in [ks[i], ke[i]).
    """
    for t, n in ((q, "q"), (k, "k")):
        _dev(t, n)
        if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise TypeError(f"{n} must be uint8 or float8_e4m3fn")
    _dev(k_scale, "k_scale")
    _dev(weights, "weights", torch.float32)
    _dev(ks, "ks", torch.int32)
    _dev(ke, "ke", torch.int32)
    _dev(logits, "logits", torch.float32)
    for t, n in ((k, "k"), (k_scale, "k_scale"), (weights, "weights"), (ks, "ks"), (ke, "ke")):
        _contig(t, n)
    if q.dim() != 3 or (q.numel() and (q.stride(2) != 1 or q.stride(1) != q.shape[2])):
        raise ValueError("q must be [num_q, num_heads, head_dim] with contiguous heads")
    num_q, num_heads, head_dim = q.shape
    if k.dim() != 2 or k.shape[1] != head_dim:
        raise ValueError("k must be [num_k, head_dim]")
    num_k = k.shape[0]
    if k_scale.dtype == torch.uint8:
        ok = tuple(k_scale.shape) == (num_k, SCALE_BYTES)
    else:
        ok = k_scale.dtype == torch.float32 and k_scale.numel() == num_k
    if not ok:
        raise ValueError("k_scale must be float32 [num_k] or uint8 [num_k, 4]")
    if tuple(weights.shape) != (num_q, num_heads):
        raise ValueError("weights must be [num_q, num_heads]")
    if ks.numel() != num_q or ke.numel() != num_q:
        raise ValueError("ks and ke must have num_q entries")
    if logits.dim() != 2 or logits.shape[0] != num_q or (logits.numel() and logits.stride(1) != 1):
        raise ValueError("logits must be [num_q, row_cols] with contiguous rows")
    _check(_lib.pkv_fp8_mqa_logits(
        q.data_ptr(), _row_stride(q, num_heads * head_dim) * q.element_size(), k.data_ptr(),
        k_scale.data_ptr(), weights.data_ptr(), ks.data_ptr(), ke.data_ptr(), logits.data_ptr(),
        _row_stride(logits, logits.shape[1]),
        logits.shape[1], num_q, num_heads, num_k, head_dim, _stream(stream)))


def paged_attention_workspace(num_seqs: int, num_heads: int, max_context_len: int,
                              partition_size: int = 256, head_size: int = 128, device="cuda"):
    """The caller-owned workspace of pkv_paged_attention_decode: exp_sums and
    max_logits float32 [S, H, P], tmp_out float32 [S, H, P, head_size], with
    P = ceil(max_context_len / partition_size) (at least 1)."""
    parts = max(1, -(-int(max_context_len) // int(partition_size)))
    exp_sums = torch.empty((num_seqs, num_heads, parts), dtype=torch.float32, device=device)
    max_logits = torch.empty_like(exp_sums)
    tmp_out = torch.empty((num_seqs, num_heads, parts, head_size), dtype=torch.float32,
                          device=device)
    return exp_sums, max_logits, tmp_out


def _attention_shapes(out, query, key_cache, value_cache, num_kv_heads, block_tables,
                      context_lens, block_size):
    """Checks the decode-attention tensors; returns (num_seqs, num_heads,
    head_size, num_blocks)."""
    _dev(out, "out", torch.bfloat16)
    _dev(query, "query", torch.bfloat16)
    for t, n in ((key_cache, "key_cache"), (value_cache, "value_cache")):
        _dev(t, n)
        if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise TypeError(f"{n} must be uint8 or float8_e4m3fn")
    _dev(block_tables, "block_tables", torch.int32)
    _dev(context_lens, "context_lens", torch.int32)
    for t, n in ((out, "out"), (query, "query"), (key_cache, "key_cache"),
                 (value_cache, "value_cache"), (block_tables, "block_tables"),
                 (context_lens, "context_lens")):
        _contig(t, n)
    if query.dim() != 3:
        raise ValueError("query must be [num_seqs, num_heads, head_size]")
    num_seqs, num_heads, head_size = query.shape
    if tuple(out.shape) != tuple(query.shape):
        raise ValueError("out must have the shape of query")
    if key_cache.dim() != 5 or value_cache.dim() != 4:
        raise ValueError("key_cache must be [nb, KVH, D/16, B, 16] and value_cache [nb, KVH, D, B]")
    num_blocks = key_cache.shape[0]
    if (tuple(key_cache.shape) != (num_blocks, num_kv_heads, head_size // 16, block_size, 16) or
            tuple(value_cache.shape) != (num_blocks, num_kv_heads, head_size, block_size)):
        raise ValueError("key_cache / value_cache shapes do not match num_kv_heads, head_size "
                         "and block_size")
    if block_tables.dim() != 2 or block_tables.shape[0] != num_seqs:
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq]")
    if context_lens.numel() != num_seqs:
        raise ValueError("context_lens must have num_seqs entries")
    return num_seqs, num_heads, head_size, num_blocks


def pkv_paged_attention_decode(out, exp_sums, max_logits, tmp_out, query, key_cache,
                               value_cache, num_kv_heads: int, scale: float, block_tables,
                               context_lens, block_size: int, max_context_len: int,
                               k_scale: float = 1.0, v_scale: float = 1.0,
                               partition_size: int = 256, stream=None):
    """Decode attention over fp8 KV pages with per-tensor scales.

    out:          bfloat16 [num_seqs, num_heads, 128], contiguous.
    exp_sums, max_logits: float32 [num_seqs, num_heads, P] workspace,
                  tmp_out float32 [num_seqs, num_heads, P, 128], with
                  P = ceil(max_context_len / partition_size)
                  (paged_attention_workspace makes them).
    query:        bfloat16 [num_seqs, num_heads, 128], contiguous.
    key_cache:    uint8 / float8_e4m3fn [num_blocks, num_kv_heads, 8, block_size, 16].
    value_cache:  uint8 / float8_e4m3fn [num_blocks, num_kv_heads, 128, block_size].
    block_tables: int32 [num_seqs, max_blocks_per_seq]; context_lens int32 [num_seqs].
    scale, k_scale, v_scale: host floats.
    """
    num_seqs, num_heads, head_size, num_blocks = _attention_shapes(
        out, query, key_cache, value_cache, num_kv_heads, block_tables, context_lens, block_size)
    for t, n in ((exp_sums, "exp_sums"), (max_logits, "max_logits"), (tmp_out, "tmp_out")):
        _dev(t, n, torch.float32)
        _contig(t, n)
    parts = -(-int(max_context_len) // int(partition_size)) if partition_size > 0 else 0
    if exp_sums.dim() != 3 or tuple(exp_sums.shape[:2]) != (num_seqs, num_heads) or \
            tuple(max_logits.shape) != tuple(exp_sums.shape) or \
            tuple(tmp_out.shape) != (*exp_sums.shape, head_size):
        raise ValueError("workspace shapes do not match [num_seqs, num_heads, P(, head_size)]")
    if exp_sums.shape[2] != max(parts, 1) and exp_sums.shape[2] != parts:
        raise ValueError(f"workspace holds {exp_sums.shape[2]} partitions, the call needs {parts}")
    _check(_lib.pkv_paged_attention_decode(
        out.data_ptr(), exp_sums.data_ptr(), max_logits.data_ptr(), tmp_out.data_ptr(),
        query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(), block_tables.data_ptr(),
        context_lens.data_ptr(), num_seqs, num_heads, num_kv_heads, head_size, block_size,
        block_tables.shape[1], max_context_len, num_blocks, scale, k_scale, v_scale,
        partition_size, _stream(stream)))


def pkv_paged_attention_decode_noalloc(out, query, key_cache, value_cache, num_kv_heads: int,
                                       scale: float, block_tables, context_lens,
                                       block_size: int, max_context_len: int,
                                       k_scale: float = 1.0, v_scale: float = 1.0,
                                       partition_size: int = 256, stream=None):
    """pkv_paged_attention_decode with the library's built-in workspace (no
    allocation by the call, ATTENTION_SCRATCH_BYTES per GPU, shared by every
    call on that GPU: calls that may overlap on one GPU race).  Arguments as
    there, without the three workspace tensors."""
    num_seqs, num_heads, head_size, num_blocks = _attention_shapes(
        out, query, key_cache, value_cache, num_kv_heads, block_tables, context_lens, block_size)
    _check(_lib.pkv_paged_attention_decode_noalloc(
        out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
        block_tables.data_ptr(), context_lens.data_ptr(), num_seqs, num_heads, num_kv_heads,
        head_size, block_size, block_tables.shape[1], max_context_len, num_blocks, scale,
        k_scale, v_scale, partition_size, _stream(stream)))


def pkv_attention_balanced_units(num_seqs: int, num_heads: int, num_kv_heads: int,
                                 max_context_len: int, partition_size: int,
                                 wave_slots: int) -> int:
    """Work units of pkv_paged_attention_decode's balanced split for these
    sizes on a device holding wave_slots partition-kernel waves at once (12
    per compute unit), or 0 for the fixed split.  Host only; no GPU work."""
    return int(_lib.pkv_attention_balanced_units(num_seqs, num_heads, num_kv_heads,
                                                 max_context_len, partition_size, wave_slots))
