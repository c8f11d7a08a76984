"""GPU parity: libpkv's gfx950 kernels, called through the C ABI (via the
Python binding), against the CPU oracle on the same seeded inputs.

Every comparison is bit-exact and covers whole buffers: caches (so bytes a
kernel must not touch are checked too) and outputs with guard rows.  Sizes
span several tiles with ragged tails; the 256 x 1000-token prefill batch is
compared in full for the fp8 store and the gather; the NVFP4 store at that
scale is compared on sampled tokens the oracle recomputes one by one.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import paged_quantized_kv_amd as pkv

DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bf16_dev(bits, shape=None, dtype="bf16"):
    t = dev(bits.view(np.int16)).view(torch.float16 if dtype == "f16" else torch.bfloat16)
    return t if shape is None else t.view(*shape)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def banner(name):
    print(f"\n[case] {name}", flush=True)


# ---------------------------------------------------------------- gather
def run_gather(w, cache_np, block_table=None, cu=None, k_rows=None):
    bt = w.block_table if block_table is None else block_table
    cu = w.cu_seq_lens if cu is None else cu
    kf0 = w.k_fp8_init if k_rows is None else w.k_fp8_init[:k_rows]
    ks0 = w.k_scale_init if k_rows is None else w.k_scale_init[:k_rows]
    ref_f, ref_s = kf0.copy(), ks0.copy()
    oracle.gather_indexer_k_fp8(cache_np, ref_f, ref_s, bt, cu, w.block_size, w.head_dim)
    kf, ks = dev(kf0), dev(ks0)
    pkv.pkv_gather_indexer_k_fp8(dev(cache_np), kf, ks, dev(bt), dev(cu),
                                 block_size=w.block_size)
    np.testing.assert_array_equal(host(kf), ref_f)
    np.testing.assert_array_equal(host(ks), ref_s)


@pytest.mark.parametrize("name", ["c1", "c3"])
def test_gather_configs_random_pages(name):
    w = {"c1": workloads.c1_tiny_gather, "c3": workloads.c3_long_ragged}[name]()
    banner(f"gather {w.name} lens={w.lens[:8]}")
    run_gather(w, w.cache_init)


def test_gather_prefill_256x1000_full():
    w = workloads.c2_prefill_256x1000()
    banner(f"gather {w.name}")
    run_gather(w, w.cache_init)


@pytest.mark.parametrize("lens,bs,hd", [
    ([0, 1, 63, 64, 65, 0, 200, 129], 64, 128),
    ([5, 9, 31, 16, 17], 16, 64),
    ([130, 1, 255], 32, 256),
    ([300, 7], 48, 128),          # block size that is not a power of two
    ([1000], 64, 1024),
    ([1] * 700, 64, 128),         # many short requests: several prefix tiles per thread
])
def test_gather_ragged(lens, bs, hd):
    banner(f"gather ragged lens={lens[:6]}.. B={bs} D={hd}")
    width = max(1, max(-(-n // bs) for n in lens)) + 3
    w = workloads.small_indexer(len(lens) * 7 + bs + hd, lens, block_size=bs, head_dim=hd,
                                poison=True, width=width)
    run_gather(w, w.cache_init)


def test_gather_skip_rules_and_offsets():
    banner("gather skip rules")
    w = workloads.small_indexer(77, [100, 30, 70, 5], width=3)
    bt = w.block_table.copy()
    bt[0, 1] = w.num_blocks + 3      # page past the cache
    bt[1, 0] = -1                    # negative page
    bt[2, 1] = w.num_blocks          # first invalid id
    run_gather(w, w.cache_init, block_table=bt)
    # cu_seq_lens not starting at 0, and rows beyond num_tokens (clipped)
    cu = w.cu_seq_lens.copy() + 5
    run_gather(w, w.cache_init, cu=cu, k_rows=150)
    # a request longer than the table is wide
    cu2 = np.array([0, 250, 250, 260, 300], np.int32)
    run_gather(w, w.cache_init, cu=cu2, k_rows=w.k_fp8_init.shape[0])


def test_gather_many_requests_chunked_launch():
    lens = [1 + (i % 3) for i in range(17000)]   # more requests than one launch stages
    banner("gather 17000 requests")
    w = workloads.small_indexer(99, lens, block_size=16, head_dim=64, width=1)
    run_gather(w, w.cache_init)


def test_gather_empty():
    banner("gather empty")
    w = workloads.c1_tiny_gather()
    cu = np.zeros(3, np.int32)
    run_gather(w, w.cache_init, cu=cu)
    kf = dev(w.k_fp8_init[:0])
    pkv.pkv_gather_indexer_k_fp8(dev(w.cache_init), kf, dev(w.k_scale_init[:0]),
                                 dev(w.block_table), dev(w.cu_seq_lens), block_size=64)


def test_empty_inputs_of_every_store_and_read_back():
    """Zero tokens, in tensors whose strides are those numpy and torch give
    empty arrays (here all zero): every entry point accepts them, launches
    nothing and leaves the caches as they were."""
    banner("empty inputs, zero strides")
    w = workloads.c1_tiny_gather()
    cache = dev(w.cache_init)
    empty_k = torch.from_numpy(np.zeros((0, 128), np.int16)).to(DEV).view(torch.bfloat16)
    empty_k = empty_k.as_strided((0, 128), (0, 0))
    pkv.pkv_store_indexer_k_fp8(empty_k, dev(np.zeros(0, np.int64)), cache, block_size=64)
    out = torch.zeros((0, 128), dtype=torch.bfloat16, device=DEV).as_strided((0, 128), (0, 0))
    pkv.pkv_gather_indexer_k_dequant(cache, out, dev(w.block_table), dev(w.cu_seq_lens),
                                     block_size=64)
    f = workloads.small_fp4(11, 8, H=2, D=128, B=16)
    c4 = dev(f.cache_init)
    e3 = torch.zeros((0, 2, 128), dtype=torch.bfloat16, device=DEV).as_strided((0, 2, 128),
                                                                               (0, 0, 0))
    one = torch.ones(1, dtype=torch.float32, device=DEV)
    pkv.pkv_store_kv_fp4(e3, e3, c4[:, 0], c4[:, 1], dev(np.zeros(0, np.int64)), one, one,
                         block_size=16, layout=0)
    pkv.pkv_gather_kv_fp4_dequant(c4[:, 0], c4[:, 1], e3, e3, dev(np.zeros((1, 1), np.int32)),
                                  dev(np.zeros(2, np.int32)), one, one, block_size=16, layout=0)
    np.testing.assert_array_equal(host(cache), w.cache_init)
    np.testing.assert_array_equal(host(c4), f.cache_init)


# ---------------------------------------------------------------- fp8 store
def run_store8(w, k_bits=None, slots=None, cache_np=None, row_pad=0):
    kb = w.k_bits if k_bits is None else k_bits
    sl = w.slot_mapping if slots is None else slots
    c0 = w.cache_init if cache_np is None else cache_np
    ref = c0.copy()
    if row_pad:
        kb = np.concatenate([kb, np.full((kb.shape[0], row_pad), 0x7F80, np.uint16)], axis=1)
    oracle.store_indexer_k_fp8(np.ascontiguousarray(kb), sl, ref, w.block_size, w.head_dim,
                               dtype=w.dtype)
    cache = dev(c0)
    k = bf16_dev(np.ascontiguousarray(kb), dtype=w.dtype)[:, :w.head_dim]
    pkv.pkv_store_indexer_k_fp8(k, dev(sl), cache, block_size=w.block_size)
    got = host(cache)
    np.testing.assert_array_equal(got, ref)
    return got


@pytest.mark.parametrize("name", ["c1", "c4"])
def test_store_fp8_configs(name):
    w = {"c1": workloads.c1_tiny_gather, "c4": workloads.c4_roundtrip}[name]()
    banner(f"store fp8 {w.name}")
    run_store8(w)


def test_store_fp8_prefill_256x1000_full():
    w = workloads.c2_prefill_256x1000()
    banner(f"store fp8 {w.name}")
    run_store8(w)


@pytest.mark.parametrize("lens,bs,hd", [
    ([37, 64, 1], 64, 16), ([100, 3], 16, 32), ([65, 70], 32, 64), ([200], 64, 256),
    ([50, 51], 64, 512), ([20], 8, 1024), ([90, 33], 48, 128), ([10, 11], 64, 96),
])
def test_store_fp8_shapes(lens, bs, hd):
    banner(f"store fp8 lens={lens} B={bs} D={hd}")
    w = workloads.small_indexer(sum(lens) + hd, lens, block_size=bs, head_dim=hd, drop_frac=0.1)
    run_store8(w)


def test_store_fp8_row_stride_and_skips():
    banner("store fp8 padded rows, -1 and out-of-range slots")
    w = workloads.small_indexer(5, [300, 77], drop_frac=0.2)
    sl = w.slot_mapping.copy()
    sl[4] = w.num_blocks * w.block_size          # first slot past the cache
    sl[9] = w.num_blocks * w.block_size + 1000
    run_store8(w, slots=sl, row_pad=24)
    run_store8(w, slots=np.full_like(sl, -1))


def test_stores_confine_non_finite_tokens_to_their_own_bytes():
    """Non-finite source values are outside the contract (their codes are
    unspecified), but memory access is not: tokens with NaN or infinite
    elements may write only their own code row and scale bytes (fp8 store)
    or their own data and block-scale bytes (NVFP4 store); every other byte
    must be the oracle's.  The bytes a token owns are found by storing the
    non-finite tokens alone into a cache and into its bitwise complement:
    a byte they write differs from at least one of the two."""
    banner("stores with non-finite tokens")
    g = workloads.rng(321)
    bad_tok = np.array([0, 5, 63, 64, 200, 511])

    # fp8 indexer store
    w = workloads.small_indexer(31, [512], drop_frac=0.0)
    x = g.standard_normal((512, 128)).astype(np.float32)
    x[0, 3] = np.nan
    x[5, :] = np.inf
    x[63, 100] = -np.inf
    x[64, ::7] = np.nan
    x[200, 0] = np.inf
    x[511] = np.nan
    kb = workloads.bf16_bits(x)
    ref = w.cache_init.copy()
    oracle.store_indexer_k_fp8(kb, w.slot_mapping, ref, 64, 128)
    cache = dev(w.cache_init)
    pkv.pkv_store_indexer_k_fp8(bf16_dev(kb), dev(w.slot_mapping), cache, block_size=64)
    got = host(cache)
    only = np.full(512, -1, np.int64)
    only[bad_tok] = w.slot_mapping[bad_tok]
    owned = np.zeros(w.cache_init.shape, bool)
    for init in (w.cache_init, ~w.cache_init):
        o = init.copy()
        oracle.store_indexer_k_fp8(kb, only, o, 64, 128)
        owned |= o != init
    assert owned.sum() == len(bad_tok) * (128 + 4)
    np.testing.assert_array_equal(got[~owned], ref[~owned])

    # NVFP4 store: NaN / inf in some 16-element blocks of some tokens
    f = workloads.paged_fp4(33, [100, 37, 64], H=4, D=128, B=16, drop_frac=0.0)
    T = f.num_tokens
    kf = f.key_bits.copy()
    vf = f.value_bits.copy()
    bad4 = np.array([0, 17, 99, 100, 136, T - 1])
    kf[bad4[:3], 5] = 0x7FC0                         # NaN in one block
    vf[bad4[3:], :] = 0x7F80                         # +inf everywhere
    ref4 = f.cache_init.copy()
    oracle.store_kv_fp4(kf, vf, ref4, f.slot_mapping, 4, 128, 16, 0, f.k_scale, f.v_scale)
    c4 = dev(f.cache_init)
    shape = (T, 4, 128)
    pkv.pkv_store_kv_fp4(bf16_dev(kf, shape), bf16_dev(vf, shape), c4[:, 0], c4[:, 1],
                         dev(f.slot_mapping),
                         torch.tensor([f.k_scale], dtype=torch.float32, device=DEV),
                         torch.tensor([f.v_scale], dtype=torch.float32, device=DEV),
                         block_size=16, layout=0)
    got4 = host(c4)
    only4 = np.full(T, -1, np.int64)
    only4[bad4] = f.slot_mapping[bad4]
    owned4 = np.zeros(f.cache_init.shape, bool)
    for init in (f.cache_init, ~f.cache_init):
        o = init.copy()
        oracle.store_kv_fp4(kf, vf, o, only4, 4, 128, 16, 0, f.k_scale, f.v_scale)
        owned4 |= o != init
    assert owned4.sum() == len(bad4) * 2 * 4 * (64 + 8)
    np.testing.assert_array_equal(got4[~owned4], ref4[~owned4])


def test_store_fp8_value_edge_cases():
    """Zero, tiny (IEEE-division path), subnormal, huge and tie-making tokens."""
    banner("store fp8 value edge cases")
    g = workloads.rng(123)
    T, D = 512, 128
    x = g.standard_normal((T, D)).astype(np.float32)
    x[0] = 0.0
    x[1, ::2] = -0.0
    x[1, 1::2] = 0.0
    x[2] *= np.float32(2.0 ** -70)             # amax < 2^-60: division path
    x[3] = np.float32(2.0 ** -133)             # smallest bf16 subnormal everywhere
    x[3, ::3] *= -1
    x[4] *= np.float32(2.0 ** -126)            # subnormal bf16 values
    x[5] *= np.float32(1e37)                   # large magnitudes, still finite
    x[6] = np.float32(3.3895314e38)
    x[7, :] = 1.953125 * 2.0 ** -16            # W8-style ties
    x[7, 0] = 1.953125
    x[8:64] *= np.exp2(g.integers(-60, 60, size=(56, 1))).astype(np.float32)
    x[64:128] *= np.float32(2.0 ** -60)        # right at the path boundary
    # every bf16 significand as amax, paired with every bf16 significand below it
    sig = (np.arange(128, dtype=np.uint32) | 0x3F80) << 16
    sigf = sig.view(np.float32)
    for i in range(128, 256):
        row = np.tile(sigf, 1)[:D] * np.float32(2.0 ** -((i % 20)))
        row[0] = sigf[i - 128] * np.float32(2.0 ** 3)
        x[i] = row
    kb = workloads.bf16_bits(x)
    w = workloads.small_indexer(3, [T], drop_frac=0.0)
    run_store8(w, k_bits=kb)


def test_store_then_gather_roundtrip_c4():
    w = workloads.c4_roundtrip()
    banner(f"round trip {w.name}")
    cache_ref = w.cache_init.copy()
    oracle.store_indexer_k_fp8(w.k_bits, w.slot_mapping, cache_ref, w.block_size, w.head_dim)
    kf_ref, ks_ref = w.k_fp8_init.copy(), w.k_scale_init.copy()
    oracle.gather_indexer_k_fp8(cache_ref, kf_ref, ks_ref, w.block_table, w.cu_seq_lens,
                                w.block_size, w.head_dim)
    cache = dev(w.cache_init)
    kf, ks = dev(w.k_fp8_init), dev(w.k_scale_init)
    pkv.pkv_store_indexer_k_fp8(bf16_dev(w.k_bits), dev(w.slot_mapping), cache, block_size=64)
    pkv.pkv_gather_indexer_k_fp8(cache, kf, ks, dev(w.block_table), dev(w.cu_seq_lens),
                                 block_size=64)
    np.testing.assert_array_equal(host(cache), cache_ref)
    np.testing.assert_array_equal(host(kf), kf_ref)
    np.testing.assert_array_equal(host(ks), ks_ref)


def test_store_gather_on_side_stream():
    banner("side stream")
    w = workloads.c1_tiny_gather()
    s = torch.cuda.Stream()
    cache_ref = w.cache_init.copy()
    oracle.store_indexer_k_fp8(w.k_bits, w.slot_mapping, cache_ref, 64, 128)
    cache = dev(w.cache_init)
    k, sl = bf16_dev(w.k_bits), dev(w.slot_mapping)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        pkv.pkv_store_indexer_k_fp8(k, sl, cache, block_size=64)
    s.synchronize()
    np.testing.assert_array_equal(cache.cpu().numpy(), cache_ref)


# ---------------------------------------------------------------- NVFP4 store
def run_store4(f, slots=None, layout=None, key_bits=None):
    layout = f.layout if layout is None else layout
    sl = f.slot_mapping if slots is None else slots
    kb = f.key_bits if key_bits is None else key_bits
    ref = f.cache_init.copy()
    oracle.store_kv_fp4(kb, f.value_bits, ref, sl, f.num_heads, f.head_size, f.block_size,
                        layout, f.k_scale, f.v_scale, dtype=f.dtype)
    c = dev(f.cache_init)
    T = sl.shape[0]
    shape = (T, f.num_heads, f.head_size)
    pkv.pkv_store_kv_fp4(bf16_dev(kb, shape, f.dtype), bf16_dev(f.value_bits, shape, f.dtype),
                         c[:, 0], c[:, 1],
                         dev(sl), torch.tensor([f.k_scale], dtype=torch.float32, device=DEV),
                         torch.tensor([f.v_scale], dtype=torch.float32, device=DEV),
                         block_size=f.block_size, layout=layout)
    np.testing.assert_array_equal(host(c), ref)


@pytest.mark.parametrize("layout", [0, 1])
def test_store_fp4_c5(layout):
    f = workloads.c5_nvfp4_store(layout)
    banner(f"nvfp4 {f.name} layout={layout}")
    run_store4(f)


@pytest.mark.parametrize("T,H,D,B,layout", [
    (37, 1, 64, 4, 0), (100, 2, 128, 8, 1), (64, 3, 192, 12, 0), (50, 5, 256, 16, 1),
    (130, 8, 128, 32, 0), (9, 16, 64, 64, 1), (33, 7, 128, 20, 0),
])
def test_store_fp4_shapes(T, H, D, B, layout):
    banner(f"nvfp4 T={T} H={H} D={D} B={B} layout={layout}")
    f = workloads.small_fp4(T * 13 + H, T, H=H, D=D, B=B, layout=layout)
    run_store4(f)


def test_store_fp4_value_edge_cases():
    banner("nvfp4 value edge cases")
    f = workloads.small_fp4(5, 64, H=2, D=128, B=16, drop_frac=0.0)
    x = (f.key_bits.astype(np.uint32) << 16).view(np.float32).reshape(64, 2, 8, 16).copy()
    x[0] = 0.0
    x[1, :, :, ::2] = -0.0
    x[2] *= np.float32(2.0 ** -120)          # block scale underflows E4M3
    x[3] *= np.float32(2.0 ** -8)            # subnormal E4M3 block scales
    x[4] *= np.float32(1e30)                 # block scale saturates at 448
    x[5, :, :, 0] = 6.0                      # exact ties on the E2M1 grid
    x[5, :, :, 1:] = np.array([2.5, .25, .75, 5, 1.25, 1.75, -.5, 3.5, 4, 1, 2, 3, .5, 1.5, -6],
                              np.float32)
    x[6:] *= np.exp2(np.random.default_rng(1).integers(-30, 30, size=(58, 1, 1, 1))).astype(np.float32)
    kb = workloads.bf16_bits(x.reshape(64, -1))
    run_store4(f, key_bits=kb)
    run_store4(f, slots=np.full_like(f.slot_mapping, -1))


def test_store_fp4_prefill_sampled():
    """256 x 1000-token prefill batch, H=8, D=128, B=16 (the benchmark's shape):
    full GPU run; the oracle recomputes 3000 sampled tokens and every byte those
    tokens own is compared: their code bytes and their K and V scale bytes.
    The owned bytes are found without any layout formula: the oracle runs
    twice, over the sentinel cache and over its bitwise complement, and the
    bytes that come out equal in both runs are the ones the tokens write."""
    f = workloads.prefill_fp4()
    banner(f"nvfp4 {f.name} sampled")
    c = dev(f.cache_init)
    T = f.num_tokens
    shape = (T, f.num_heads, f.head_size)
    pkv.pkv_store_kv_fp4(bf16_dev(f.key_bits, shape), bf16_dev(f.value_bits, shape), c[:, 0],
                         c[:, 1], dev(f.slot_mapping),
                         torch.tensor([f.k_scale], dtype=torch.float32, device=DEV),
                         torch.tensor([f.v_scale], dtype=torch.float32, device=DEV),
                         block_size=f.block_size, layout=f.layout)
    got = host(c)
    pick = np.sort(workloads.rng(5).choice(T, size=3000, replace=False))
    refs = []
    for init in (f.cache_init, ~f.cache_init):
        ref = init.copy()
        oracle.store_kv_fp4(np.ascontiguousarray(f.key_bits[pick]),
                            np.ascontiguousarray(f.value_bits[pick]), ref,
                            np.ascontiguousarray(f.slot_mapping[pick]), f.num_heads,
                            f.head_size, f.block_size, f.layout, f.k_scale, f.v_scale)
        refs.append(ref)
    owned = refs[0] == refs[1]
    H, D = f.num_heads, f.head_size
    kept = int((f.slot_mapping[pick] >= 0).sum())
    # per token: H*D/2 code bytes and H*D/16 scale bytes on each of two sides
    assert owned.sum() == kept * 2 * H * (D // 2 + D // 16)
    np.testing.assert_array_equal(got[owned], refs[0][owned])


@pytest.mark.parametrize("k_scale,v_scale", [(2.0 ** -126, 3.4028234663852886e38),
                                             (3.4028234663852886e38, 2.0 ** -126)])
def test_store_fp4_global_scale_domain_ends(k_scale, v_scale):
    """The two ends of the scales the boundary accepts (positive normal
    binary32): 2^-126 gives the global scale 2^126, FLT_MAX a subnormal one.
    Blocks span every bf16 binade, with zero and negative-zero blocks, so the
    products amax * gs overflow, underflow and land in between."""
    banner(f"nvfp4 k_scale = {k_scale:g}, v_scale = {v_scale:g}")
    g = workloads.rng(29)
    T, H, D, B = 48, 2, 128, 16

    def src():
        x = g.standard_normal((T, H, D // 16, 16)).astype(np.float32)
        x *= np.exp2(g.integers(-140, 126, size=(T, H, D // 16, 1))).astype(np.float32)
        x[:, :, 0] = 0.0                    # all-zero blocks
        x[:, 0, 1] = -0.0                   # negative-zero blocks
        return x.reshape(T, H, D)

    f = _fp4_custom(src(), src(), B, k_scale, v_scale)
    run_store4(f)


# ---------------------------------------------------------------- codecs
def _sweep(encode, lo_bits, hi_bits, oracle_fn, chunk=1 << 26):
    """Compare the device codec with the oracle on every binary32 pattern in
    [lo_bits, hi_bits) (unsigned bit order)."""
    from concurrent.futures import ThreadPoolExecutor
    pool = ThreadPoolExecutor(16)
    start = lo_bits
    while start < hi_bits:
        n = min(chunk, hi_bits - start)
        n16 = (n + 15) // 16 * 16
        b = torch.arange(start, start + n16, dtype=torch.int64, device=DEV)
        b = torch.where(b < hi_bits, b, torch.full_like(b, lo_bits))
        b = torch.where(b >= 2 ** 31, b - 2 ** 32, b).to(torch.int32)
        y32 = b.view(torch.float32)
        out = torch.empty(n16, dtype=torch.uint8, device=DEV)
        encode(y32.contiguous(), out)
        got = out.cpu().numpy()
        ybits = np.arange(start, start + n16, dtype=np.int64)
        ybits = np.where(ybits < hi_bits, ybits, lo_bits).astype(np.uint32)
        yf = ybits.view(np.float32)
        parts = np.array_split(np.arange(n16), 16)
        ref = np.empty(n16, np.uint8)

        def work(ix):
            ref[ix] = oracle_fn(yf[ix])
        list(pool.map(work, parts))
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, (f"{bad.size} mismatches, first y=0x{ybits[bad[0]]:08x} "
                               f"got {got[bad[0]]:#x} want {ref[bad[0]]:#x}")
        start += n
    pool.shutdown()


def test_device_e4m3_codec_exhaustive_below_464():
    banner("e4m3 codec sweep")
    lim = int(np.array([464.0], np.float32).view(np.uint32)[0])
    _sweep(pkv.pkv_diag_encode_e4m3, 0, lim, oracle.e4m3_encode)
    _sweep(pkv.pkv_diag_encode_e4m3, 0x80000000, 0x80000000 + lim, oracle.e4m3_encode)


def test_device_e2m1_codec_exhaustive():
    banner("e2m1 codec sweep")
    # every non-NaN pattern: [0, +inf] and [-0, -inf]
    _sweep(pkv.pkv_diag_encode_e2m1, 0, 0x7F800001, oracle.e2m1_encode)
    _sweep(pkv.pkv_diag_encode_e2m1, 0x80000000, 0xFF800001, oracle.e2m1_encode)


def _fp4_custom(x_key, x_val, B, k_scale, v_scale, seed=9):
    """NVFP4 workload around caller-chosen K/V values [T, H, D] (one page per 4 tokens)."""
    T, H, D = x_key.shape
    g = workloads.rng(seed)
    nb = -(-T // B) + 1
    f = workloads.Fp4Workload(
        "custom", H, D, B, nb, 0, workloads.bf16_bits(x_key.reshape(T, -1)),
        workloads.bf16_bits(x_val.reshape(T, -1)), np.arange(T, dtype=np.int64),
        float(np.float32(k_scale)), float(np.float32(v_scale)),
        workloads.random_bytes(g, (nb, 2, H * B * (D // 2 + D // 16))))
    return f


def test_store_fp4_every_block_scale_code():
    """k_scale = v_scale = 1 and block amax = 6 * decode(c): the block scale is
    exactly decode(c), so every E4M3 code 0..126 appears as a block scale (and
    every entry of the reciprocal table with every exponent is used)."""
    banner("nvfp4 every block-scale code")
    codes = np.arange(127, dtype=np.uint8)
    dec = oracle.e4m3_decode(codes).astype(np.float32)
    H, D, B = 2, 64, 4                      # 4 blocks per head, 16 blocks per token
    nblk = 2 * H * (D // 16)
    T = -(-len(codes) // nblk) + 1
    g = workloads.rng(17)
    blocks = np.zeros((T * nblk, 16), np.float32)
    for i, c in enumerate(codes):
        amax = np.float32(6.0) * dec[c]
        frac = g.uniform(-1, 1, 15).astype(np.float32)
        blocks[i, 0] = amax if i % 2 else -amax
        blocks[i, 1:] = frac * amax
    x = blocks.reshape(T, 2, H, D)
    f = _fp4_custom(x[:, 0].copy(), x[:, 1].copy(), B, 1.0, 1.0)
    run_store4(f)


@pytest.mark.parametrize("scale", [2.0 ** 110, 2.0 ** -110])
def test_store_fp4_global_scale_outside_table_range(scale):
    banner(f"nvfp4 k_scale = {scale:g}")
    g = workloads.rng(23)
    T, H, D, B = 24, 2, 128, 8
    mag = np.float32(2.0 ** 100 if scale > 1 else 2.0 ** -100)
    x = (g.standard_normal((T, H, D)) * mag).astype(np.float32)
    y = g.standard_normal((T, H, D)).astype(np.float32)
    f = _fp4_custom(x, y, B, scale, 1.0)
    run_store4(f)


# ---------------------------------------------------------------- fp16 sources
def test_store_fp8_f16_roundtrip_and_shapes():
    banner("store fp8 f16 sources")
    w = workloads.c4_roundtrip(dtype="f16")
    run_store8(w)
    for lens, bs, hd in (([37, 64, 1], 64, 16), ([65, 70], 32, 64), ([200], 64, 256),
                         ([20], 8, 1024), ([90, 33], 48, 128)):
        run_store8(workloads.small_indexer(sum(lens) + hd + 7, lens, block_size=bs,
                                           head_dim=hd, drop_frac=0.1, dtype="f16"))


def test_store_fp8_f16_value_edge_cases():
    banner("store fp8 f16 value edge cases")
    g = workloads.rng(321)
    T, D = 256, 128
    x = g.standard_normal((T, D)).astype(np.float32)
    x[0] = 0.0
    x[1, ::2] = -0.0
    x[2] = np.float32(2.0 ** -24)                  # smallest fp16 subnormal
    x[2, ::3] *= -1
    x[3] *= np.float32(2.0 ** -16)                 # fp16 subnormal values
    x[4] = np.float32(65504.0)                     # fp16 maximum
    x[4, 1::2] = -1.0
    x[5:64] *= np.exp2(g.integers(-20, 14, size=(59, 1))).astype(np.float32)
    # every fp16 significand as amax
    sig = ((np.arange(1024, dtype=np.uint32) << 13) | 0x3F800000).view(np.float32)
    for i in range(64, 192):
        row = sig[(i * 8) % 1024:(i * 8) % 1024 + D] if (i * 8) % 1024 + D <= 1024 else sig[:D]
        x[i] = row * np.float32(2.0 ** -(i % 9))
        x[i, 0] = sig[(i * 37) % 1024] * np.float32(4.0)
    x = np.clip(x, -65504, 65504)
    w = workloads.small_indexer(3, [T], drop_frac=0.0, dtype="f16")
    run_store8(w, k_bits=workloads.f16_bits(x))


@pytest.mark.parametrize("layout", [0, 1])
def test_store_fp4_c5_f16(layout):
    f = workloads.c5_nvfp4_store(layout, dtype="f16")
    banner(f"nvfp4 {f.name} f16 layout={layout}")
    run_store4(f)


def test_store_fp4_f16_shapes_and_edges():
    banner("nvfp4 f16 shapes and edges")
    for T, H, D, B, layout in ((37, 1, 64, 4, 0), (64, 3, 192, 12, 1), (33, 7, 128, 20, 0)):
        run_store4(workloads.small_fp4(T * 17 + H, T, H=H, D=D, B=B, layout=layout,
                                       dtype="f16"))
    f = workloads.small_fp4(77, 48, H=2, D=128, B=16, drop_frac=0.0, dtype="f16")
    x = f.key_bits.view(np.float16).astype(np.float32).reshape(48, 2, 8, 16).copy()
    x[0] = 0.0
    x[1] = np.float32(2.0 ** -24)
    x[2] *= np.float32(2.0 ** -14)
    x[3] = np.float32(65504.0)
    x[3, :, :, 1::2] = -3.0
    run_store4(f, key_bits=workloads.f16_bits(x.reshape(48, -1)))


# Slots that fill pages as a prefill does: runs of consecutive slots, so the
# NVFP4 store writes whole page lines and whole 4-token V-scale tiles; the
# request lengths (not multiples of 4 or 16) and dropped slots make tiles
# that straddle pages, partial swizzle tiles and ragged tails.
@pytest.mark.parametrize("lens,H,D,B,layout,drop,dtype", [
    ([37, 5, 16, 100, 1, 64], 2, 128, 16, 0, 0.0, "bf16"),
    ([37, 5, 16, 100, 1, 64], 2, 128, 16, 1, 0.05, "bf16"),
    ([40, 24, 3, 96], 3, 64, 8, 0, 0.1, "f16"),
    ([200, 17, 33], 1, 256, 32, 0, 0.02, "bf16"),
    ([200, 17, 33], 2, 256, 32, 1, 0.0, "f16"),
    ([48, 48, 13, 50], 4, 128, 12, 0, 0.05, "bf16"),
    ([1000, 1000, 1000], 8, 128, 16, 0, 0.0, "bf16"),
])
def test_store_fp4_paged_slots(lens, H, D, B, layout, drop, dtype):
    banner(f"nvfp4 paged slots lens={lens} H={H} D={D} B={B} layout={layout} drop={drop} {dtype}")
    f = workloads.paged_fp4(sum(lens) + H + D + B, lens, H=H, D=D, B=B, layout=layout,
                            drop_frac=drop, dtype=dtype)
    run_store4(f)


@pytest.mark.parametrize("D,layout", [(128, 0), (128, 1), (64, 0), (256, 1)])
def test_store_fp4_sides_8_byte_aligned(D, layout):
    """Page sides that are 8- but not 16-byte aligned (page stride = two sides
    + 8 bytes, buffer offset 8): the store still writes exactly the oracle's
    bytes and leaves the 8 padding bytes of every page untouched."""
    banner(f"nvfp4 8-byte aligned sides D={D} layout={layout}")
    H, B = 2, 16
    f = workloads.paged_fp4(77 + D + layout, [45, 19, 64], H=H, D=D, B=B, layout=layout)
    nb, side = f.cache_init.shape[0], f.cache_init.shape[2]
    stride = 2 * side + 8
    rng = np.random.default_rng(5)
    flat = rng.integers(0, 256, size=8 + nb * stride, dtype=np.uint8)
    pages = flat[8:].reshape(nb, stride)
    pages[:, :2 * side] = f.cache_init.reshape(nb, 2 * side)
    ref_pages = pages.copy()
    ref = f.cache_init.copy()
    oracle.store_kv_fp4(f.key_bits, f.value_bits, ref, f.slot_mapping, H, D, B, layout,
                        f.k_scale, f.v_scale, dtype=f.dtype)
    ref_pages[:, :2 * side] = ref.reshape(nb, 2 * side)
    buf = dev(flat)
    view = buf[8:].view(nb, stride)
    T = f.slot_mapping.shape[0]
    shape = (T, H, D)
    pkv.pkv_store_kv_fp4(bf16_dev(f.key_bits, shape, f.dtype), bf16_dev(f.value_bits, shape, f.dtype),
                         view[:, :side], view[:, side:2 * side], dev(f.slot_mapping),
                         torch.tensor([f.k_scale], dtype=torch.float32, device=DEV),
                         torch.tensor([f.v_scale], dtype=torch.float32, device=DEV),
                         block_size=B, layout=layout)
    out = host(buf)
    np.testing.assert_array_equal(out[:8], flat[:8])
    np.testing.assert_array_equal(out[8:].reshape(nb, stride), ref_pages)
