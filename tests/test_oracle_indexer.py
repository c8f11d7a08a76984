"""Pins for the oracle's fp8 indexer store and gather.

Store: hand-worked cases W1, W2, W3, W8 (golden files); the dequantisation
error bound |x - q*s| <= (h(y) + |y|*2^-24)*s with h = half an E4M3 step;
the invariant that every token's largest element codes to magnitude 0x7E;
slot = -1 and out-of-cache slots leave pages untouched.
Gather: hand-worked W7; an independent numpy fancy-index reading on ragged
cases; guard rows, poison pages and skip rules; and the store -> gather
round trip, which must equal a per-token quantisation with no paging at all.
"""
import numpy as np
import pytest

import oracle
import workloads
from conftest import load_golden

B, D = 64, 128


def bits_of(x):
    return workloads.bf16_bits(np.asarray(x, np.float32))


def store_one_token(x_row, block_size=4, head_dim=128, slot=1, num_blocks=2, seed=0):
    """Quantise one token into a small sentinel-filled cache; return (cache, before)."""
    g = workloads.rng(seed)
    page = block_size * (head_dim + 4)
    cache = workloads.random_bytes(g, (num_blocks, page))
    before = cache.copy()
    k = bits_of(np.asarray(x_row, np.float32).reshape(1, head_dim))
    oracle.store_indexer_k_fp8(k, np.array([slot], np.int64), cache, block_size, head_dim)
    return cache, before


def unpack_token(cache, slot, block_size, head_dim):
    p, off = divmod(slot, block_size)
    codes = cache[p, off * head_dim:(off + 1) * head_dim]
    sb = cache[p, block_size * head_dim + off * 4: block_size * head_dim + off * 4 + 4]
    return codes, sb


@pytest.mark.parametrize("name", ["w1_fp8_exact_scale.json", "w3_fp8_inexact_scale.json",
                                  "w8_fp8_division_tie.json"])
def test_store_golden(name):
    gd = load_golden(name)
    hd = gd["head_dim"]
    x = np.zeros(hd, np.float32)
    x[:len(gd["x"])] = gd["x"]
    assert np.array_equal(np.asarray(bits_of(x), np.uint32) << 16,
                          x.view(np.uint32)), "golden x must be exact bf16 values"
    cache, before = store_one_token(x, head_dim=hd, slot=5, num_blocks=3)
    codes, sb = unpack_token(cache, 5, 4, hd)
    want = [int(c, 16) for c in gd["codes"]] + [int(gd["pad_code"], 16)] * (hd - len(gd["codes"]))
    np.testing.assert_array_equal(codes, want)
    if "scale_bytes_le" in gd:
        np.testing.assert_array_equal(sb, [int(c, 16) for c in gd["scale_bytes_le"]])
    if "scale_bits" in gd:
        assert sb.view("<u4")[0] == int(gd["scale_bits"], 16)
    # nothing else in the cache changed
    mask = np.ones_like(cache, bool)
    p, off = divmod(5, 4)
    mask[p, off * hd:(off + 1) * hd] = False
    mask[p, 4 * hd + off * 4: 4 * hd + off * 4 + 4] = False
    np.testing.assert_array_equal(cache[mask], before[mask])


def test_store_zero_token_w2():
    gd = load_golden("w2_fp8_zero_token.json")
    x = np.zeros(128, np.float32)
    x[1::2] = -0.0
    cache, _ = store_one_token(x, slot=0)
    codes, sb = unpack_token(cache, 0, 4, 128)
    want = np.tile([int(c, 16) for c in gd["codes_pattern"]], 64)
    np.testing.assert_array_equal(codes, want)
    np.testing.assert_array_equal(sb, [0, 0, 0, 0])


def quantize_tokens(k_bits, head_dim=D):
    """Store every token into its own slot of an identity-mapped cache
    (one token per page) and return (codes [T, D], scales fp32 [T])."""
    T = k_bits.shape[0]
    cache = np.zeros((T, 1 * (head_dim + 4)), np.uint8)
    oracle.store_indexer_k_fp8(k_bits, np.arange(T, dtype=np.int64), cache, 1, head_dim)
    return cache[:, :head_dim], cache[:, head_dim:].copy().view("<f4")[:, 0]


def e4m3_half_step(y):
    a = np.abs(y.astype(np.float64))
    h = np.where(a >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 4),
                 2.0 ** -10)
    return h


def test_store_error_bound_and_max_code():
    g = workloads.rng(11)
    x = g.standard_normal((4000, D)).astype(np.float32)
    x[::97] *= 20                                          # outlier rows
    x[5::131] *= np.float32(2.0 ** -60)                    # tiny tokens
    x[7::113] *= np.float32(2.0 ** 30)                     # huge tokens
    kb = bits_of(x)
    xf = (kb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    codes, s = quantize_tokens(kb)
    q = oracle.e4m3_decode(codes.ravel()).reshape(codes.shape).astype(np.float64)
    s64 = s.astype(np.float64)[:, None]
    y = xf / s64
    bound = (e4m3_half_step(y) + np.abs(y) * 2.0 ** -24) * s64
    err = np.abs(xf - q * s64)
    assert (err <= bound).all(), float((err - bound).max())
    # amax element codes to +-448 (0x7E) for every token with a normal scale
    amax_code = (codes & 0x7F).max(axis=1)
    assert (amax_code == 0x7E).all()
    assert not np.isin(codes, [0x7F, 0xFF]).any()
    # scale is amax/448 within binary32 rounding
    amax = np.abs(xf).max(axis=1)
    np.testing.assert_allclose(s.astype(np.float64), amax / 448, rtol=2 ** -24)


def test_store_skips_negative_and_out_of_range_slots():
    w = workloads.small_indexer(21, [50, 70], drop_frac=0.2)
    cache = w.cache_init.copy()
    slots = w.slot_mapping.copy()
    slots[3] = w.num_blocks * w.block_size + 5  # past the cache: skipped
    oracle.store_indexer_k_fp8(w.k_bits, slots, cache, w.block_size, w.head_dim)
    touched = np.zeros_like(cache, bool)
    for s in slots:
        if 0 <= s < w.num_blocks * w.block_size:
            p, off = divmod(int(s), w.block_size)
            touched[p, off * D:(off + 1) * D] = True
            touched[p, B * D + off * 4: B * D + off * 4 + 4] = True
    np.testing.assert_array_equal(cache[~touched], w.cache_init[~touched])
    assert (cache[touched] != w.cache_init[touched]).mean() > 0.9


def test_gather_golden_w7():
    gd = load_golden("w7_gather_tiny.json")
    b, d = gd["block_size"], gd["head_dim"]
    g = workloads.rng(3)
    cache = workloads.random_bytes(g, (10, b * (d + 4)))
    k_fp8 = workloads.random_bytes(g, (7, d))
    k_scale = workloads.random_bytes(g, (7, 4))
    kf0, ks0 = k_fp8.copy(), k_scale.copy()
    oracle.gather_indexer_k_fp8(cache, k_fp8, k_scale, np.array(gd["block_table"], np.int32),
                                np.array(gd["cu_seq_lens"], np.int32), b, d)
    for row, (p, off) in enumerate(gd["rows"]):
        np.testing.assert_array_equal(k_fp8[row], cache[p, off * d:(off + 1) * d])
        np.testing.assert_array_equal(k_scale[row], cache[p, b * d + off * 4: b * d + off * 4 + 4])
    np.testing.assert_array_equal(k_fp8[5:], kf0[5:])
    np.testing.assert_array_equal(k_scale[5:], ks0[5:])


def numpy_gather(w, cache, k_fp8, k_scale):
    """Independent reading: build a (page, offset) pair per output row."""
    out_c, out_s = k_fp8.copy(), k_scale.copy()
    R, maxb = w.block_table.shape
    for r in range(R):
        n = int(w.cu_seq_lens[r + 1] - w.cu_seq_lens[r])
        i = np.arange(n)
        i = i[i // w.block_size < maxb]
        pages = w.block_table[r, i // w.block_size]
        ok = (pages >= 0) & (pages < cache.shape[0])
        i, pages = i[ok], pages[ok]
        rows = w.cu_seq_lens[r] + i
        ok = (rows >= 0) & (rows < k_fp8.shape[0])
        i, pages, rows = i[ok], pages[ok], rows[ok]
        offs = i % w.block_size
        col = offs[:, None] * w.head_dim + np.arange(w.head_dim)[None, :]
        out_c[rows] = cache[pages[:, None], col]
        scol = w.block_size * w.head_dim + offs[:, None] * 4 + np.arange(4)[None, :]
        out_s[rows] = cache[pages[:, None], scol]
    return out_c, out_s


@pytest.mark.parametrize("lens,bs,hd", [([17, 40], 64, 128), ([0, 1, 63, 64, 65, 0, 200], 64, 128),
                                        ([5, 9, 31], 16, 64), ([130, 1], 32, 256)])
def test_gather_matches_numpy_reading(lens, bs, hd):
    w = workloads.small_indexer(sum(lens) + bs, lens, block_size=bs, head_dim=hd, poison=True,
                                width=max(1, max(-(-n // bs) for n in lens)) + 2)
    kf, ks = w.k_fp8_init.copy(), w.k_scale_init.copy()
    oracle.gather_indexer_k_fp8(w.cache_init, kf, ks, w.block_table, w.cu_seq_lens, bs, hd)
    ref_c, ref_s = numpy_gather(w, w.cache_init, w.k_fp8_init, w.k_scale_init)
    np.testing.assert_array_equal(kf, ref_c)
    np.testing.assert_array_equal(ks, ref_s)
    T = w.num_tokens
    np.testing.assert_array_equal(kf[T:], w.k_fp8_init[T:])  # guard rows untouched


def test_gather_skip_rules():
    w = workloads.small_indexer(5, [100, 30], width=2)
    bt = w.block_table.copy()
    bt[0, 1] = w.num_blocks + 3     # page past the cache -> rows 64..99 skipped
    bt[1, 0] = -1                   # negative page -> request 1 skipped
    cu = w.cu_seq_lens.copy()
    kf, ks = w.k_fp8_init.copy(), w.k_scale_init.copy()
    oracle.gather_indexer_k_fp8(w.cache_init, kf, ks, bt, cu, B, D)
    np.testing.assert_array_equal(kf[64:], w.k_fp8_init[64:])
    np.testing.assert_array_equal(ks[64:], w.k_scale_init[64:])
    np.testing.assert_array_equal(kf[:64], w.cache_init[bt[0, 0], :64 * D].reshape(64, D))
    # request longer than the block table is wide: columns past it are skipped
    cu2 = np.array([0, 200], np.int32)
    bt2 = w.block_table[:1, :2].copy()
    out = np.zeros((200, D), np.uint8)
    outs = np.zeros((200, 4), np.uint8)
    oracle.gather_indexer_k_fp8(w.cache_init, out, outs, bt2, cu2, B, D)
    assert (out[128:] == 0).all() and (outs[128:] == 0).all()
    # rows past num_tokens are skipped
    out3 = np.zeros((70, D), np.uint8)
    outs3 = np.zeros((70, 4), np.uint8)
    oracle.gather_indexer_k_fp8(w.cache_init, out3, outs3, bt2, cu2, B, D)
    np.testing.assert_array_equal(out3[64:70], w.cache_init[bt2[0, 1], :6 * D].reshape(6, D))


def test_store_gather_roundtrip_equals_unpaged_quantisation():
    w = workloads.c4_roundtrip()
    cache = w.cache_init.copy()
    oracle.store_indexer_k_fp8(w.k_bits, w.slot_mapping, cache, w.block_size, w.head_dim)
    kf, ks = w.k_fp8_init.copy(), w.k_scale_init.copy()
    oracle.gather_indexer_k_fp8(cache, kf, ks, w.block_table, w.cu_seq_lens, w.block_size,
                                w.head_dim)
    codes, s = quantize_tokens(w.k_bits)
    kept = w.slot_mapping >= 0
    T = w.num_tokens
    np.testing.assert_array_equal(kf[:T][kept], codes[kept])
    np.testing.assert_array_equal(ks[:T][kept].view("<f4")[:, 0].view(np.uint32),
                                  s[kept].view(np.uint32))
    # dropped tokens read back the page's untouched sentinel bytes
    for t in np.nonzero(~kept)[0][:50]:
        p, off = divmod(int(w.block_table[t // 512, (t % 512) // 64]) * 64 + t % 64, 64)
        np.testing.assert_array_equal(kf[t], w.cache_init[p, off * D:(off + 1) * D])
    np.testing.assert_array_equal(kf[T:], w.k_fp8_init[T:])
