"""Seeded synthetic inputs for the paged quantized KV-cache data path.

This module serves both the CPU oracle and the HIP library, and therefore
holds none of the method's arithmetic: only random numbers (numpy PCG64 with
a fixed seed per workload), index tables (block tables, cumulative sequence
lengths, slot maps), random sentinel bytes for every buffer an op writes, and
the binary32 -> bf16 input cast (round-to-nearest-even, done by torch on the
CPU).

Shapes follow the pages' workloads: the DeepSeek-V3.2 indexer K cache of the
gather PRs (one 128-wide fp8 key row plus a 4-byte scale per token, 64-token
pages) and the NVFP4 K/V store of vLLM's nvfp4 KV-cache kernel source (bf16
[tokens, heads, head_size], 16-token pages).  The serving benchmark on the
integration PR used 256 requests x 1000 prompt tokens; that shape is the
prefill batch here.  No dataset item is reproduced; values are N(0, 1).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

INDEXER_SCALE_BYTES = 4  # one binary32 scale per token


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


_CHUNK = 1 << 22


def normal_f32(g: np.random.Generator, shape) -> np.ndarray:
    """N(0, 1) binary32 array.  Large arrays are drawn in fixed 4 Mi-element
    chunks, chunk i from PCG64(SeedSequence([base, i])) with base drawn from
    g, on a thread pool; the values do not depend on the thread count."""
    n = int(np.prod(shape))
    if n <= _CHUNK:
        return g.standard_normal(shape, dtype=np.float32)
    base = int(g.integers(0, 2 ** 63))
    out = np.empty(n, dtype=np.float32)
    starts = range(0, n, _CHUNK)

    def fill(i_start):
        i, start = i_start
        gen = np.random.Generator(np.random.PCG64(np.random.SeedSequence([base, i])))
        gen.standard_normal(min(_CHUNK, n - start), dtype=np.float32,
                            out=out[start:start + _CHUNK])

    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(fill, enumerate(starts)))
    return out.reshape(shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """binary32 -> bf16 (RNE) as uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def f16_bits(x: np.ndarray) -> np.ndarray:
    """binary32 -> binary16 (RNE, numpy) as uint16 bit patterns."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def half_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    return f16_bits(x) if dtype == "f16" else bf16_bits(x)


def random_bytes(g: np.random.Generator, shape) -> np.ndarray:
    return g.integers(0, 256, size=shape, dtype=np.uint8)


def slots_from_table(table: np.ndarray, lens, block_size: int) -> np.ndarray:
    """Slot of token i of request r = table[r][i // B] * B + i % B, in token order."""
    out = []
    for r, n in enumerate(lens):
        i = np.arange(n, dtype=np.int64)
        out.append(table[r, i // block_size].astype(np.int64) * block_size + i % block_size)
    return np.concatenate(out) if out else np.zeros(0, np.int64)


def _pages_table(g, lens, block_size, num_blocks, width=None, poison=None):
    """Distinct pages for every request from one seeded permutation; unused
    entries hold `poison` (a page id that no request owns) or 0."""
    need = [(-(-n // block_size)) for n in lens]
    width = width if width is not None else max(need + [1])
    perm = g.permutation(num_blocks).astype(np.int32)
    assert sum(need) <= num_blocks - (1 if poison is not None else 0)
    fill = -1 if poison is None else poison
    table = np.full((len(lens), width), fill, dtype=np.int32)
    pos = 0
    for r, n in enumerate(need):
        table[r, :n] = perm[pos:pos + n]
        pos += n
    if poison is None:
        # pad with a page that exists; the gather never reads past the
        # request's own columns, so any in-range id is fine
        table[table < 0] = perm[-1]
    return table, perm


@dataclass
class IndexerWorkload:
    """Indexer K cache workload: fp8 store of K, then gather back."""
    name: str
    block_size: int
    head_dim: int
    num_blocks: int
    lens: list
    cu_seq_lens: np.ndarray          # int32 [R+1]
    block_table: np.ndarray          # int32 [R, maxb]
    k_bits: np.ndarray               # uint16 [T, D] bf16 patterns, token order
    slot_mapping: np.ndarray         # int64 [T]
    cache_init: np.ndarray           # uint8 [num_blocks, page_bytes] sentinel bytes
    k_fp8_init: np.ndarray           # uint8 [T + guard, D] sentinel bytes
    k_scale_init: np.ndarray         # uint8 [T + guard, 4] sentinel bytes
    notes: dict = field(default_factory=dict)
    dtype: str = "bf16"              # source element type of k_bits: "bf16" or "f16"

    @property
    def page_bytes(self) -> int:
        return self.block_size * (self.head_dim + INDEXER_SCALE_BYTES)

    @property
    def num_tokens(self) -> int:
        return int(self.cu_seq_lens[-1] - self.cu_seq_lens[0])


def _indexer(name, seed, lens, block_size, head_dim, num_blocks, width=None,
             poison=False, outlier_frac=0.0, outlier_mult=20.0, guard=3,
             drop_frac=0.0, k_override=None, dtype="bf16"):
    g = rng(seed)
    lens = [int(x) for x in lens]
    poison_id = None
    if poison:
        poison_id = int(num_blocks - 1)
    if poison_id is not None:
        # keep the poison page out of the permutation's assigned prefix
        table, _ = _pages_table(g, lens, block_size, num_blocks - 1, width, poison_id)
    else:
        table, _ = _pages_table(g, lens, block_size, num_blocks, width)
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens, dtype=np.int64).astype(np.int32)
    T = int(cu[-1])
    if k_override is not None:
        kf = k_override
    else:
        kf = normal_f32(g, (T, head_dim))
        if outlier_frac > 0:
            n_out = int(round(outlier_frac * T))
            rows = g.choice(T, size=n_out, replace=False)
            kf[rows] *= np.float32(outlier_mult)
    k_bits = half_bits(kf, dtype)
    slots = slots_from_table(table, lens, block_size)
    if drop_frac > 0:
        n_drop = int(np.floor(drop_frac * T))
        slots[g.choice(T, size=n_drop, replace=False)] = -1
    page_bytes = block_size * (head_dim + INDEXER_SCALE_BYTES)
    cache = random_bytes(g, (num_blocks, page_bytes))
    k_fp8 = random_bytes(g, (T + guard, head_dim))
    k_scale = random_bytes(g, (T + guard, INDEXER_SCALE_BYTES))
    return IndexerWorkload(name, block_size, head_dim, num_blocks, lens, cu, table,
                           k_bits, slots, cache, k_fp8, k_scale,
                           notes={"poison_page": poison_id, "seed": seed}, dtype=dtype)


def c1_tiny_gather() -> IndexerWorkload:
    """2 requests (17 and 40 tokens), B=64, D=128, 8 pages."""
    return _indexer("tiny_gather_2req", 1000, [17, 40], 64, 128, 8, width=4)


def c2_prefill_256x1000() -> IndexerWorkload:
    """256 requests x 1000 tokens, B=64, D=128, 4096 pages, 1% outlier rows x20."""
    return _indexer("prefill_256x1000", 1001, [1000] * 256, 64, 128, 4096, width=16,
                    outlier_frac=0.01)


def c3_long_ragged() -> IndexerWorkload:
    """8 requests, lengths uniform in [1, 32768], 8192 pages, block table width 512,
    unused block-table entries hold a poison page id."""
    lens = rng(2002).integers(1, 32769, size=8)
    return _indexer("long_ragged_8req", 1002, lens, 64, 128, 8192, width=512,
                    poison=True)


def c4_roundtrip(dtype="bf16") -> IndexerWorkload:
    """16 requests x 512 tokens stored into a 256-page cache (5% of slots = -1),
    then gathered back."""
    return _indexer("roundtrip_16x512", 1003, [512] * 16, 64, 128, 256, width=8,
                    drop_frac=0.05, dtype=dtype)


def small_indexer(seed, lens, block_size=64, head_dim=128, num_blocks=None, width=None,
                  drop_frac=0.0, poison=False, dtype="bf16"):
    """Small random case for the property tests."""
    need = sum(-(-int(n) // block_size) for n in lens)
    if num_blocks is None:
        num_blocks = max(need + 2, 4)
    return _indexer(f"small_{seed}", seed, lens, block_size, head_dim, num_blocks,
                    width=width, drop_frac=drop_frac, poison=poison, dtype=dtype)


@dataclass
class Fp4Workload:
    """NVFP4 K/V store workload."""
    name: str
    num_heads: int
    head_size: int
    block_size: int
    num_blocks: int
    layout: int                      # 0 = HND, 1 = NHD
    key_bits: np.ndarray             # uint16 [T, H*D]
    value_bits: np.ndarray           # uint16 [T, H*D]
    slot_mapping: np.ndarray         # int64 [T]
    k_scale: float
    v_scale: float
    cache_init: np.ndarray           # uint8 [num_blocks, 2, side_bytes]
    dtype: str = "bf16"              # source element type: "bf16" or "f16"
    # when the slots come from request lengths: the pages each request owns
    # and the token offsets of the requests (for reading the pages back)
    block_table: np.ndarray = None   # int32 [R, maxb]
    cu_seq_lens: np.ndarray = None   # int32 [R+1]

    @property
    def side_bytes(self) -> int:
        return self.num_heads * self.block_size * (self.head_size // 2 + self.head_size // 16)

    @property
    def num_tokens(self) -> int:
        return int(self.slot_mapping.shape[0])


def _fp4(name, seed, T, H, D, B, num_blocks, layout=0, slots=None, drop_frac=0.05,
         lens=None, dtype="bf16"):
    g = rng(seed)
    table = cu = None
    if lens is not None:
        table, _ = _pages_table(g, lens, B, num_blocks)
        slot_mapping = slots_from_table(table, lens, B)
        T = slot_mapping.shape[0]
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    elif slots is None:
        slot_mapping = g.permutation(num_blocks * B)[:T].astype(np.int64)
    else:
        slot_mapping = np.asarray(slots, np.int64)
    if drop_frac > 0:
        n_drop = int(np.floor(drop_frac * T))
        slot_mapping[g.choice(T, size=n_drop, replace=False)] = -1
    kf = normal_f32(g, (T, H * D))
    vf = normal_f32(g, (T, H * D))
    k_scale, v_scale = (float(np.float32(v)) for v in g.uniform(0.5, 2.0, size=2))
    side = H * B * (D // 2 + D // 16)
    cache = random_bytes(g, (num_blocks, 2, side))
    return Fp4Workload(name, H, D, B, num_blocks, layout, half_bits(kf, dtype),
                       half_bits(vf, dtype), slot_mapping, k_scale, v_scale, cache, dtype,
                       table, cu)


def c5_nvfp4_store(layout=0, dtype="bf16") -> Fp4Workload:
    """K and V [4096, 8, 128], B=16, 512 pages, 5% of slots = -1, scales in [0.5, 2]."""
    return _fp4("nvfp4_4096x8x128", 1004, 4096, 8, 128, 16, 512, layout=layout, dtype=dtype)


def small_fp4(seed, T, H=2, D=64, B=8, num_blocks=None, layout=0, drop_frac=0.1,
              dtype="bf16"):
    if num_blocks is None:
        num_blocks = max(-(-T // B) + 2, 2)
    return _fp4(f"small_fp4_{seed}", seed, T, H, D, B, num_blocks, layout=layout,
                drop_frac=drop_frac, dtype=dtype)


def paged_fp4(seed, lens, H=2, D=128, B=16, layout=0, drop_frac=0.05, dtype="bf16",
              spare_pages=3) -> Fp4Workload:
    """NVFP4 store inputs whose slots fill pages the way a prefill does: each
    request (token counts `lens`, in order) owns whole pages from a seeded
    shuffle, token i of a request in slot page*B + i%B; then a fraction
    `drop_frac` of the slots is set to -1."""
    need = sum(-(-n // B) for n in lens)
    return _fp4(f"paged_fp4_{seed}", seed, None, H, D, B, need + spare_pages, layout=layout,
                lens=list(lens), drop_frac=drop_frac, dtype=dtype)


def prefill_fp4(num_reqs=256, req_len=1000, H=8, D=128, B=16, seed=1005) -> Fp4Workload:
    """The 256 x 1000-token prefill batch through the NVFP4 K/V store
    (H=8, D=128, B=16); every request owns whole pages from a seeded shuffle."""
    need = num_reqs * (-(-req_len // B))
    num_blocks = 1 << int(np.ceil(np.log2(need)))
    return _fp4(f"prefill_fp4_{num_reqs}x{req_len}", seed, None, H, D, B, num_blocks,
                lens=[req_len] * num_reqs, drop_frac=0.0)


@dataclass
class MqaLogitsCase:
    """Inputs of the indexer logits: fp8 query rows against fp8 keys."""
    q: np.ndarray          # uint8 E4M3 codes [M, H, 128]
    k: np.ndarray          # uint8 E4M3 codes [N, 128]
    k_scale: np.ndarray    # float32 [N]
    weights: np.ndarray    # float32 [M, H]
    ks: np.ndarray         # int32 [M]
    ke: np.ndarray         # int32 [M]


def _e4m3_codes(x: np.ndarray) -> np.ndarray:
    """Codes of float32 values already inside the E4M3 range (torch's cast)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).clamp(-448, 448)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def mqa_logits_case(seed, num_q, num_heads, num_k, causal_lens=None, head_dim=128):
    """Query codes from N(0,1)*8, key codes from N(0,1)*64 (so both span most
    E4M3 binades), key scales uniform in [0.001, 0.01] (the size amax/448 has
    for unit-normal keys), weights N(0,1)/8.  With causal_lens the queries
    and keys are the tokens of those requests in order and token i of a
    request sees keys [request start, i]; otherwise each query gets a random
    range inside [0, num_k)."""
    g = rng(seed)
    if causal_lens is not None:
        lens = [int(n) for n in causal_lens]
        num_q = num_k = sum(lens)
        ks = np.concatenate([np.full(n, s) for n, s in zip(lens, np.cumsum([0] + lens[:-1]))]
                            ).astype(np.int32) if num_q else np.zeros(0, np.int32)
        ke = (ks + np.concatenate([np.arange(1, n + 1) for n in lens])).astype(np.int32) \
            if num_q else np.zeros(0, np.int32)
    else:
        a = g.integers(0, num_k + 1, size=num_q)
        b = g.integers(0, num_k + 1, size=num_q)
        ks, ke = np.minimum(a, b).astype(np.int32), np.maximum(a, b).astype(np.int32)
    q = _e4m3_codes(normal_f32(g, (num_q, num_heads, head_dim)) * np.float32(8))
    k = _e4m3_codes(normal_f32(g, (num_k, head_dim)) * np.float32(64))
    k_scale = g.uniform(0.001, 0.01, size=num_k).astype(np.float32)
    weights = (normal_f32(g, (num_q, num_heads)) / np.float32(8)).astype(np.float32)
    return MqaLogitsCase(q, k, k_scale, weights, ks, ke)


@dataclass
class PagedAttentionCase:
    """Decode attention over fp8 KV pages in vLLM's layouts."""
    query: np.ndarray          # uint16 bf16 patterns [S, H, D]
    key_cache: np.ndarray      # uint8 E4M3 codes [num_blocks, KVH, D/16, B, 16]
    value_cache: np.ndarray    # uint8 E4M3 codes [num_blocks, KVH, D, B]
    block_tables: np.ndarray   # int32 [S, maxb]
    context_lens: np.ndarray   # int32 [S]
    num_kv_heads: int
    scale: float
    k_scale: float
    v_scale: float


def paged_attention_case(seed, num_seqs, num_heads, num_kv_heads, block_size=16, head_size=128,
                         max_context=2048, min_context=1, lens=None, spare_pages=3):
    """Context lengths uniform in [min_context, max_context] (or `lens`); each
    sequence owns whole pages from one seeded shuffle.  Cache codes are the
    E4M3 codes of N(0,1)*32 (torch's cast), queries N(0,1) in bf16, scale
    1/sqrt(head_size), k_scale and v_scale uniform in [0.02, 0.05] (the size
    amax/448 has for unit-normal K and V)."""
    g = rng(seed)
    if lens is None:
        lens = g.integers(min_context, max_context + 1, size=num_seqs)
    lens = [int(n) for n in lens]
    need = [-(-n // block_size) for n in lens]
    num_blocks = sum(need) + spare_pages
    table, _ = _pages_table(g, lens, block_size, num_blocks)
    D = head_size
    q = bf16_bits(normal_f32(g, (num_seqs, num_heads, D)))
    kc = normal_f32(g, (num_blocks, num_kv_heads, D // 16, block_size, 16))
    kc *= np.float32(32)
    kc = _e4m3_codes(kc)
    vc = normal_f32(g, (num_blocks, num_kv_heads, D, block_size))
    vc *= np.float32(32)
    vc = _e4m3_codes(vc)
    k_scale, v_scale = (float(np.float32(x)) for x in g.uniform(0.02, 0.05, size=2))
    return PagedAttentionCase(q, kc, vc, table.astype(np.int32), np.array(lens, np.int32),
                              num_kv_heads, float(np.float32(1.0 / np.sqrt(D))), k_scale, v_scale)


DECODE_SEQS = 200
DECODE_HEADS, DECODE_KV_HEADS, DECODE_HEAD_SIZE, DECODE_BLOCK = 64, 8, 128, 16
DECODE_MIN_CONTEXT, DECODE_MAX_CONTEXT = 128, 2560
# Tokens per partition of the decode batch's attention calls.  The page's
# kernel uses 256; the value only splits the work (results differ by rounding
# within the error bound), and 1024 is the fastest split for this batch here.
DECODE_PARTITION = 1024


def decode_batch(seed=2024):
    """One decode step of the fp8-KV serving runs on the Custom Paged Attention
    page: Llama-3.1-70B attention shapes (64 query heads, 8 KV heads, head
    size 128), 16-token pages, 200 requests (the page's prompt count) whose
    contexts are uniform in [128, 2560] (its 128- and 512-token inputs plus up
    to 2048 generated tokens)."""
    return paged_attention_case(seed, DECODE_SEQS, DECODE_HEADS, DECODE_KV_HEADS,
                                block_size=DECODE_BLOCK, head_size=DECODE_HEAD_SIZE,
                                max_context=DECODE_MAX_CONTEXT, min_context=DECODE_MIN_CONTEXT)
