"""Pins for the oracle's reader side: binary32 -> bf16 / fp16 rounding, the
dequantising gather of the indexer K cache, and the NVFP4 page read-back.

Each oracle function is checked against something other than itself: exact
rational arithmetic on the rounding definition, library conversions (torch's
CPU bf16 cast, numpy's float16 cast), hand-worked pages (tests/golden), an
independent numpy reading of the page layouts, and the round-trip error
bounds of the stores they invert.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def hexes(v):
    return np.array([int(h, 16) for h in v])


# ------------------------------------------------------------- rounding
def _structured_f32(rng, n_random=200_000):
    """binary32 patterns that exercise every rounding case of a 16-bit
    target: each binade (subnormal to the largest), low halves at the tie,
    just below / above it, zero and all-ones, plus random patterns."""
    exps = np.arange(0, 255, dtype=np.uint32)
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000],
                    dtype=np.uint32)
    hi_frac = rng.integers(0, 1 << 7, size=16, dtype=np.uint32)
    hi_frac = np.concatenate([hi_frac, np.array([0, 1, 0x7E, 0x7F], np.uint32)])
    e, lo, hf = np.meshgrid(exps, lows, hi_frac, indexing="ij")
    bits = (e << 23) | (hf << 16) | lo
    bits = np.concatenate([bits.ravel(), rng.integers(0, 0x7F800000, size=n_random,
                                                      dtype=np.uint32)])
    bits = np.concatenate([bits, bits | 0x80000000])
    return bits.view(np.float32)


def _nearest_even(value: Fraction, grid_lo: Fraction, grid_hi: Fraction, lo_even: bool):
    d_lo, d_hi = value - grid_lo, grid_hi - value
    if d_lo < d_hi:
        return grid_lo
    if d_hi < d_lo:
        return grid_hi
    return grid_lo if lo_even else grid_hi


def test_bf16_rounding_matches_torch_cpu_cast():
    # Library special case: torch's CPU float32 -> bfloat16 cast rounds to
    # nearest even and overflows to infinity.
    x = _structured_f32(np.random.default_rng(1))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f32_to_bf16(x)
    np.testing.assert_array_equal(got, ref)


def test_f16_rounding_matches_numpy_cast():
    # Library special case: numpy's float32 -> float16 cast (IEEE round to
    # nearest even, subnormals kept, overflow to infinity).
    rng = np.random.default_rng(2)
    x = _structured_f32(rng)
    # every fp16 value, the midpoints to its neighbour, and one binary32 ulp
    # either side of each midpoint
    h = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (h[:-1] + h[1:]) / 2
    m32 = mids.astype(np.float32)
    extra = np.concatenate([m32, np.nextafter(m32, np.float32(np.inf)),
                            np.nextafter(m32, np.float32(0)), h.astype(np.float32),
                            np.array([65504, 65519.996, 65520, 65536, 1e30], np.float32)])
    x = np.concatenate([x, extra, -extra])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    got = oracle.f32_to_f16(x)
    np.testing.assert_array_equal(got, ref)


def test_bf16_rounding_exact_rationals():
    # Brute force on the definition: the nearer of the two bf16 neighbours,
    # ties to the even last bit, computed with exact rationals.
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 0x7F800000, size=3000, dtype=np.uint32)
    bits[:8] = [0x3F808000, 0x3F818000, 0x00008000, 0x00018000, 0x7F7F8000, 0x7F7F7FFF,
                0x00000001, 0x3F80FFFF]
    for b in bits:
        x = np.array([b], np.uint32).view(np.float32)[0]
        lo_bits = int(b) & 0xFFFF0000
        hi_bits = lo_bits + 0x10000
        lo = Fraction(float(np.array([lo_bits], np.uint32).view(np.float32)[0]))
        if hi_bits >= 0x7F800000:
            hi = Fraction(2) ** 128     # the step past the largest finite bf16
        else:
            hi = Fraction(float(np.array([hi_bits], np.uint32).view(np.float32)[0]))
        pick = _nearest_even(Fraction(float(x)), lo, hi, ((lo_bits >> 16) & 1) == 0)
        want = 0x7F80 if pick == Fraction(2) ** 128 else (
            (lo_bits if pick == lo else hi_bits) >> 16)
        assert int(oracle.f32_to_bf16(np.array([x], np.float32))[0]) == want, hex(int(b))


def test_rounding_special_values():
    vals = np.array([0.0, -0.0, np.inf, -np.inf, 1.0, -1.0], np.float32)
    np.testing.assert_array_equal(oracle.f32_to_bf16(vals),
                                  [0x0000, 0x8000, 0x7F80, 0xFF80, 0x3F80, 0xBF80])
    np.testing.assert_array_equal(oracle.f32_to_f16(vals),
                                  [0x0000, 0x8000, 0x7C00, 0xFC00, 0x3C00, 0xBC00])
    nan = oracle.f32_to_bf16(np.array([np.nan], np.float32))[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0


# ------------------------------------------------------------- indexer dequant gather
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_w10_fp8_dequant_hand_worked(dtype):
    g = golden("w10_fp8_dequant.json")
    D = g["head_dim"]
    page = np.zeros((1, D + 4), np.uint8)
    page[0, :D] = hexes(g["codes"])
    page[0, D:] = hexes(g["scale_bytes"])
    out = np.full((1, D), 0xABCD, np.uint16)
    oracle.gather_indexer_k_dequant(page, out, np.zeros((1, 1), np.int32),
                                    np.array([0, 1], np.int32), 1, D, dtype=dtype)
    np.testing.assert_array_equal(out[0], hexes(g[dtype]))


def _numpy_dequant_gather(cache, block_table, cu, B, D, T, dtype):
    """Independent reading: fancy-indexed gather, torch's CPU float8_e4m3fn
    decode, a binary32 product, torch's bf16 / numpy's float16 cast."""
    out = np.full((T, D), 0x5A5A, np.uint16)
    codes = cache[:, :B * D].reshape(-1, B, D)
    scales = cache[:, B * D:B * D + 4 * B].copy().view(np.float32).reshape(-1, B)
    for r in range(block_table.shape[0]):
        n = int(cu[r + 1] - cu[r])
        i = np.arange(n)
        pages = block_table[r, i // B]
        q = codes[pages, i % B]
        dec = torch.from_numpy(q.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy()
        v = (dec * scales[pages, i % B][:, None]).astype(np.float32)
        if dtype == "bf16":
            o = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        else:
            o = v.astype(np.float16).view(np.uint16)
        out[cu[r]:cu[r] + n] = o
    return out


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_dequant_gather_matches_numpy_reading(dtype):
    w = workloads.c1_tiny_gather()
    cache = w.cache_init.copy()
    oracle.store_indexer_k_fp8(w.k_bits, w.slot_mapping, cache, w.block_size, w.head_dim)
    T = int(w.cu_seq_lens[-1])
    got = np.full((T, w.head_dim), 0x5A5A, np.uint16)
    oracle.gather_indexer_k_dequant(cache, got, w.block_table, w.cu_seq_lens, w.block_size,
                                    w.head_dim, dtype=dtype)
    ref = _numpy_dequant_gather(cache, w.block_table, w.cu_seq_lens, w.block_size, w.head_dim,
                                T, dtype)
    np.testing.assert_array_equal(got, ref)


def test_dequant_gather_round_trip_bound():
    # store -> dequantising gather returns x within the fp8 bound of the
    # store, |x - q*s| <= (h(y) + |y|*2^-24)*s, plus the binary32 product's
    # and the bf16 result's half ulps.
    w = workloads.c4_roundtrip()
    cache = w.cache_init.copy()
    slots = w.slot_mapping
    oracle.store_indexer_k_fp8(w.k_bits, slots, cache, w.block_size, w.head_dim)
    T = int(w.cu_seq_lens[-1])
    out = np.zeros((T, w.head_dim), np.uint16)
    oracle.gather_indexer_k_dequant(cache, out, w.block_table, w.cu_seq_lens, w.block_size,
                                    w.head_dim)
    x = (w.k_bits[:T].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    deq = (out.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    keep = slots[:T] >= 0
    amax = np.abs(x).max(axis=1, keepdims=True)
    s = (amax.astype(np.float32) / np.float32(448)).astype(np.float64)
    y = np.where(s > 0, x / np.where(s > 0, s, 1), 0)
    ay = np.abs(y)
    half_step = np.where(ay >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(ay, 2.0 ** -6))) - 4),
                         2.0 ** -10)
    bound = (half_step + ay * 2.0 ** -24) * s + np.abs(deq) * (2.0 ** -24 + 2.0 ** -8)
    err = np.abs(x - deq)
    assert np.all(err[keep] <= bound[keep] * (1 + 1e-12))


def test_dequant_gather_skips_and_untouched_rows():
    g = golden("w7_gather_tiny.json")
    B, D = g["block_size"], g["head_dim"]
    rng = np.random.default_rng(7)
    cache = rng.integers(0, 256, size=(10, B * (D + 4)), dtype=np.uint8)
    cache[:, B * D:] = 0x3C  # scale 2^-7-ish patterns (0x3C3C3C3C), finite
    bt = np.array(g["block_table"], np.int32)
    cu = np.array(g["cu_seq_lens"], np.int32)
    T = int(cu[-1])
    out = np.full((T + 2, D), 0x1234, np.uint16)
    bt_bad = bt.copy()
    bt_bad[1, 0] = 99  # page out of range: request 1's first run is skipped
    oracle.gather_indexer_k_dequant(cache, out, bt_bad, cu, B, D)
    ref = _numpy_dequant_gather(cache, bt, cu, B, D, T, "bf16")
    n0 = int(cu[1])
    np.testing.assert_array_equal(out[:n0], ref[:n0])
    np.testing.assert_array_equal(out[n0:n0 + B], 0x1234)       # skipped rows
    np.testing.assert_array_equal(out[n0 + B:T], ref[n0 + B:T])
    np.testing.assert_array_equal(out[T:], 0x1234)               # guard rows


# ------------------------------------------------------------- NVFP4 read-back
def test_w11_nvfp4_dequant_hand_worked():
    g = golden("w11_nvfp4_dequant.json")
    H, D, B = g["num_heads"], g["head_size"], g["block_size"]
    S = D // 16
    side = H * B * (D // 2 + S)
    cache = np.zeros((1, 2, side), np.uint8)
    data_k = g["k_token"] * (D // 2) + g["k_block"] * 8
    cache[0, 0, data_k:data_k + 8] = hexes(g["k_data"])
    cache[0, 0, H * B * D // 2 + g["k_scale_pos"]] = int(g["k_scale_byte"], 16)
    data_v = g["v_token"] * (D // 2) + g["v_block"] * 8
    cache[0, 1, data_v:data_v + 8] = hexes(g["v_data"])
    assert oracle.swizzle_offset(g["v_token"], g["v_block"], S) == g["v_scale_pos"]
    cache[0, 1, H * B * D // 2 + g["v_scale_pos"]] = int(g["v_scale_byte"], 16)
    ko = np.full((2, H * D), 0x7777, np.uint16)
    vo = np.full((2, H * D), 0x7777, np.uint16)
    oracle.gather_kv_fp4_dequant(cache, ko, vo, np.zeros((1, 1), np.int32),
                                 np.array([0, 2], np.int32), H, D, B, g["layout"],
                                 g["k_scale"], g["v_scale"])
    want_k = np.zeros((2, H * D), np.uint16)
    kb = g["k_block"] * 16
    want_k[g["k_token"], kb:kb + 16] = hexes(g["k_bf16"])
    want_v = np.zeros((2, H * D), np.uint16)
    vb = g["v_block"] * 16
    want_v[g["v_token"], vb:vb + 16] = hexes(g["v_bf16"])
    np.testing.assert_array_equal(ko, want_k)
    np.testing.assert_array_equal(vo, want_v)


E2M1_GRID = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float64)


def _numpy_fp4_readback(cache, block_table, cu, H, D, B, layout, k_scale, v_scale, T, dtype):
    """Independent reading of the NVFP4 pages: nibbles by numpy shifts, the
    E2M1 grid by table, V scales un-swizzled with the reshape/transpose form
    of the layout, products in binary32, torch's bf16 / numpy's fp16 cast."""
    S = D // 16
    nb = cache.shape[0]
    outs = []
    for kv, ts in ((0, k_scale), (1, v_scale)):
        side = cache[:, kv]
        data = side[:, :H * B * D // 2]
        sc = side[:, H * B * D // 2:H * B * D // 2 + H * B * S]
        if layout == 0:
            data = data.reshape(nb, H, B, D // 2).transpose(0, 2, 1, 3)
            sc = sc.reshape(nb, H, B, S)
        else:
            data = data.reshape(nb, B, H, D // 2)
            sc = sc.reshape(nb, B, H, S).transpose(0, 2, 1, 3)
        if kv == 1:   # stored order [B/4, 4, 4, S/4] -> (0, 2, 3, 1); invert it
            st = sc.reshape(nb, H, B // 4, 4, S // 4, 4)      # [p, h, tile, s/(S/4), s%(S/4), t%4]
            sc = st.transpose(0, 1, 2, 5, 3, 4).reshape(nb, H, B, S)
        sc = sc.transpose(0, 2, 1, 3)                         # [p, B, H, S]
        lo, hi = data & 0xF, data >> 4
        codes = np.stack([lo, hi], axis=-1).reshape(nb, B, H, D)
        mag = E2M1_GRID[codes & 7]
        val = np.where(codes & 8, -mag, mag)
        sfd = torch.from_numpy(sc.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy()
        v = (val.astype(np.float32) * np.repeat(sfd, 16, axis=-1)).astype(np.float32)
        v = (v * np.float32(ts)).astype(np.float32)
        if dtype == "bf16":
            o = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        else:
            o = v.astype(np.float16).view(np.uint16)
        o = o.reshape(nb, B, H * D)
        out = np.full((T, H * D), 0x5A5A, np.uint16)
        for r in range(block_table.shape[0]):
            n = int(cu[r + 1] - cu[r])
            i = np.arange(n)
            out[cu[r]:cu[r] + n] = o[block_table[r, i // B], i % B]
        outs.append(out)
    return outs


@pytest.mark.parametrize("layout,dtype", [(0, "bf16"), (1, "bf16"), (0, "f16")])
def test_nvfp4_readback_matches_numpy_reading(layout, dtype):
    lens = [37, 5, 16, 23]
    f = workloads.paged_fp4(41 + layout, lens, H=2, D=128, B=8, layout=layout, drop_frac=0.0,
                            dtype=dtype)
    cache = f.cache_init.copy()
    oracle.store_kv_fp4(f.key_bits, f.value_bits, cache, f.slot_mapping, f.num_heads,
                        f.head_size, f.block_size, layout, f.k_scale, f.v_scale, dtype=dtype)
    bt, cu = f.block_table, f.cu_seq_lens
    T = int(cu[-1])
    ko = np.full((T, 2 * 128), 0x5A5A, np.uint16)
    vo = np.full((T, 2 * 128), 0x5A5A, np.uint16)
    oracle.gather_kv_fp4_dequant(cache, ko, vo, bt, cu, 2, 128, 8, layout, f.k_scale, f.v_scale,
                                 dtype=dtype)
    rk, rv = _numpy_fp4_readback(cache, bt, cu, 2, 128, 8, layout, f.k_scale, f.v_scale, T,
                                 dtype)
    np.testing.assert_array_equal(ko, rk)
    np.testing.assert_array_equal(vo, rv)


def test_nvfp4_round_trip_bound():
    # store -> read back returns x within the E2M1 half step of the block:
    # |x - deq| <= h4(y) * sfd/gs (1 + 2^-22) + |deq| * 2^-8, h4 = 0.25 below
    # |y| = 2, 0.5 below 4, 1 above (saturated y <= 6.4 stays within 1).
    lens = [64, 33, 100]
    f = workloads.paged_fp4(5, lens, H=2, D=64, B=16, layout=0, drop_frac=0.0)
    cache = f.cache_init.copy()
    oracle.store_kv_fp4(f.key_bits, f.value_bits, cache, f.slot_mapping, 2, 64, 16, 0,
                        f.k_scale, f.v_scale)
    T = int(f.cu_seq_lens[-1])
    ko = np.zeros((T, 128), np.uint16)
    vo = np.zeros((T, 128), np.uint16)
    oracle.gather_kv_fp4_dequant(cache, ko, vo, f.block_table, f.cu_seq_lens, 2, 64, 16, 0,
                                 f.k_scale, f.v_scale)
    for bits, out, ts in ((f.key_bits, ko, f.k_scale), (f.value_bits, vo, f.v_scale)):
        x = (bits[:T].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        deq = (out.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        gs = float(np.float32(1) / np.float32(ts))
        xb = x.reshape(T, -1, 16)
        amax = np.abs(xb).max(axis=2, keepdims=True)
        sf = (amax * gs / 6).astype(np.float32)
        sfd = torch.from_numpy(sf).to(torch.float8_e4m3fn).to(torch.float64).numpy()
        y = np.abs(xb) * gs / np.where(sfd > 0, sfd, 1)
        h4 = np.where(y < 2, 0.25, np.where(y < 4, 0.5, 1.0))
        bound = h4 * sfd / gs * (1 + 2.0 ** -22) + np.abs(deq.reshape(xb.shape)) * 2.0 ** -8
        err = np.abs(xb - deq.reshape(xb.shape))
        assert np.all(err <= bound + 1e-300)
