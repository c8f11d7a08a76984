"""Pins for the oracle's NVFP4 K/V store (vLLM nvfp4 KV-cache kernel source).

Hand-worked W4, W5 (codes, nibble order, block scale), W6 (swizzle closed
form), W9 (a whole page: data region, K scales linear, V scales swizzled);
the swizzle equals numpy's reshape(T/4,4,4,S/4).transpose(0,2,3,1), a
library routine, and is a bijection on every 4-token tile; the decoded block
scale tracks amax*gs/6 within half an E4M3 step; the dequantisation bound
|x - c*sfd/gs| <= (h4(y) + |y|*2^-23)*sfd/gs; every group with a normal
block scale has a code of magnitude 7; HND and NHD place the same bytes;
skipped slots leave pages untouched; page size is 2*H*B*(D/2 + D/16).
"""
import numpy as np
import pytest

import oracle
import workloads
from conftest import load_golden


def bits_of(x):
    return workloads.bf16_bits(np.asarray(x, np.float32))


def store(key_f, val_f, slots, H, D, B, num_blocks, layout, ks, vs, seed=0):
    T = len(slots)
    side = H * B * (D // 2 + D // 16)
    cache = workloads.random_bytes(workloads.rng(seed), (num_blocks, 2, side))
    before = cache.copy()
    oracle.store_kv_fp4(bits_of(np.asarray(key_f).reshape(T, H * D)),
                        bits_of(np.asarray(val_f).reshape(T, H * D)), cache,
                        np.asarray(slots, np.int64), H, D, B, layout, ks, vs)
    return cache, before


@pytest.mark.parametrize("name", ["w4_nvfp4_unit_scale.json", "w5_nvfp4_scale2.json"])
@pytest.mark.parametrize("side", [0, 1])
def test_group_golden(name, side):
    gd = load_golden(name)
    H, D, B = 1, 64, 4
    x = np.zeros((1, H * D), np.float32)
    x[0, :16] = gd["x"]
    assert np.array_equal(bits_of(x).astype(np.uint32) << 16, x.view(np.uint32))
    other = np.zeros_like(x)
    key, val = (x, other) if side == 0 else (other, x)
    ks = gd["scale"] if side == 0 else 1.0
    vs = gd["scale"] if side == 1 else 1.0
    cache, _ = store(key, val, [6], H, D, B, 2, 0, ks, vs)
    p, off = divmod(6, B)
    sidebuf = cache[p, side]
    data = sidebuf[off * (D // 2): off * (D // 2) + 8]
    np.testing.assert_array_equal(data, [int(c, 16) for c in gd["data_bytes"]])
    S = D // 16
    scale_region = sidebuf[H * B * D // 2:]
    pos = off * S + 0 if side == 0 else oracle.swizzle_offset(off, 0, S)
    assert scale_region[pos] == int(gd["scale_byte"], 16)


def test_swizzle_golden_w6():
    gd = load_golden("w6_swizzle.json")
    for t, s, want in gd["cases"]:
        assert oracle.swizzle_offset(t, s, gd["S"]) == want


@pytest.mark.parametrize("T,S", [(16, 8), (4, 4), (64, 16), (8, 12), (32, 4)])
def test_swizzle_equals_reshape_permute(T, S):
    lin = np.arange(T * S).reshape(T, S)
    swz = lin.reshape(T // 4, 4, 4, S // 4).transpose(0, 2, 3, 1).reshape(T, S)
    pos = np.empty(T * S, np.int64)
    for t in range(T):
        for s in range(S):
            pos[oracle.swizzle_offset(t, s, S)] = lin[t, s]
    np.testing.assert_array_equal(pos.reshape(T, S), swz)
    # bijection inside each 4-token tile
    for tile in range(T // 4):
        got = sorted(oracle.swizzle_offset(t, s, S) for t in range(4 * tile, 4 * tile + 4)
                     for s in range(S))
        assert got == list(range(4 * tile * S, 4 * tile * S + 4 * S))


def test_page_layout_golden_w9():
    gd = load_golden("w9_nvfp4_page_layout.json")
    H, D, B = gd["num_heads"], gd["head_size"], gd["block_size"]
    S = D // 16
    x = np.zeros((4, H * D), np.float32)
    for t in range(4):
        for g in range(S):
            x[t, g * 16] = 6.0 * 2.0 ** (4 * t + g - 8)
    cache, _ = store(x, x, [0, 1, 2, 3], H, D, B, 1, 0, 1.0, 1.0)
    assert cache.shape[2] == gd["side_bytes"]
    grp = [int(c, 16) for c in gd["data_group_bytes"]]
    for side in (0, 1):
        np.testing.assert_array_equal(cache[0, side, :H * B * D // 2], np.tile(grp, B * S))
    np.testing.assert_array_equal(cache[0, 0, H * B * D // 2:],
                                  [int(c, 16) for c in gd["k_scale_region"]])
    np.testing.assert_array_equal(cache[0, 1, H * B * D // 2:],
                                  [int(c, 16) for c in gd["v_scale_region"]])


def test_layout_algebra_c5():
    w = workloads.c5_nvfp4_store()
    assert w.side_bytes == 8 * 16 * (64 + 8) == 9216
    assert w.cache_init.shape == (512, 2, 9216)  # page = 18432 bytes


def decode_store(cache, w, layout):
    """Read back (codes[T,2,H,D], sf8[T,2,H,S]) of every stored token."""
    H, D, B = w.num_heads, w.head_size, w.block_size
    S, dd = D // 16, D // 2
    T = w.num_tokens
    codes = np.zeros((T, 2, H, D), np.uint8)
    sf8 = np.zeros((T, 2, H, S), np.uint8)
    for t, slot in enumerate(w.slot_mapping):
        if slot < 0:
            continue
        p, off = divmod(int(slot), B)
        for kv in range(2):
            side = cache[p, kv]
            for h in range(H):
                base = (h * B + off) * dd if layout == 0 else (off * H + h) * dd
                byts = side[base: base + dd]
                codes[t, kv, h, 0::2] = byts & 0xF
                codes[t, kv, h, 1::2] = byts >> 4
                for g in range(S):
                    if kv == 0:
                        row, col = off, g
                    else:
                        row, col = divmod(oracle.swizzle_offset(off, g, S), S)
                    so = (h * B + row) * S + col if layout == 0 else (row * H + h) * S + col
                    sf8[t, kv, h, g] = side[H * B * dd + so]
    return codes, sf8


@pytest.mark.parametrize("layout", [0, 1])
def test_bounds_invariants_and_skips(layout):
    w = workloads.small_fp4(31, 200, H=2, D=64, B=8, layout=layout, drop_frac=0.1)
    cache = w.cache_init.copy()
    oracle.store_kv_fp4(w.key_bits, w.value_bits, cache, w.slot_mapping, w.num_heads,
                        w.head_size, w.block_size, layout, w.k_scale, w.v_scale)
    codes, sf8 = decode_store(cache, w, layout)
    H, D = w.num_heads, w.head_size
    kept = w.slot_mapping >= 0
    for kv, bits, scale in ((0, w.key_bits, w.k_scale), (1, w.value_bits, w.v_scale)):
        x = (bits.astype(np.uint32) << 16).view(np.float32).reshape(-1, H, D // 16, 16)[kept]
        gs = np.float32(np.float32(1.0) / np.float32(scale)).astype(np.float64)
        sfd = oracle.e4m3_decode(sf8[kept, kv].ravel()).reshape(x.shape[:3]).astype(np.float64)
        amax = np.abs(x.astype(np.float64)).max(axis=-1)
        # decoded block scale is amax*gs/6 to within half an E4M3 step (+ fp32 rounding)
        target = amax * gs / 6
        rel = np.abs(sfd - target) / target
        assert (rel <= 2.0 ** -4 * (1 + 2.0 ** -20)).all(), rel.max()
        c = codes[kept, kv].reshape(x.shape)
        cv = oracle.e2m1_decode(c.ravel()).reshape(c.shape).astype(np.float64)
        y = x.astype(np.float64) * (gs / sfd)[..., None]
        h4 = np.where(np.abs(y) < 2, 0.25, np.where(np.abs(y) < 4, 0.5, 1.0))
        deq = cv * (sfd / gs)[..., None]
        err = np.abs(x - deq)
        bound = (h4 + np.abs(y) * 2.0 ** -23) * (sfd / gs)[..., None]
        assert (err <= bound).all()
        assert ((c & 7).max(axis=-1) == 7).all()
    # bytes of dropped / untouched slots are unchanged
    touched = np.zeros(cache.shape, bool)
    H, D, B = w.num_heads, w.head_size, w.block_size
    S, dd = D // 16, D // 2
    for slot in w.slot_mapping[kept]:
        p, off = divmod(int(slot), B)
        for kv in range(2):
            for h in range(H):
                base = (h * B + off) * dd if layout == 0 else (off * H + h) * dd
                touched[p, kv, base:base + dd] = True
                for g in range(S):
                    row, col = (off, g) if kv == 0 else divmod(oracle.swizzle_offset(off, g, S), S)
                    so = (h * B + row) * S + col if layout == 0 else (row * H + h) * S + col
                    touched[p, kv, H * B * dd + so] = True
    np.testing.assert_array_equal(cache[~touched], w.cache_init[~touched])


def test_hnd_and_nhd_hold_the_same_bytes():
    a = workloads.small_fp4(41, 64, H=4, D=128, B=16, layout=0)
    b = workloads.small_fp4(41, 64, H=4, D=128, B=16, layout=1)
    ca, cb = a.cache_init.copy(), b.cache_init.copy()
    for w, c in ((a, ca), (b, cb)):
        oracle.store_kv_fp4(w.key_bits, w.value_bits, c, w.slot_mapping, w.num_heads,
                            w.head_size, w.block_size, w.layout, w.k_scale, w.v_scale)
    A, sa = decode_store(ca, a, 0)
    Bc, sb = decode_store(cb, b, 1)
    np.testing.assert_array_equal(A, Bc)
    np.testing.assert_array_equal(sa, sb)


def test_zero_and_tiny_groups():
    H, D, B = 1, 64, 4
    x = np.zeros((2, 64), np.float32)
    x[0, 1::2] = -0.0
    x[1, :16] = 2.0 ** -133                       # smallest bf16 subnormal
    cache, _ = store(x, x, [0, 1], H, D, B, 1, 0, 1.0, 1.0)
    # token 0: sf = 0 -> scale byte 0, codes signed zeros (nibble 8 for -0)
    np.testing.assert_array_equal(cache[0, 0, 0:8], [0x80] * 8)
    assert cache[0, 0, H * B * D // 2 + 0] == 0
    # token 1: amax*gs/6 underflows E4M3 -> sfd = 0 -> r = 0 -> all codes +0
    np.testing.assert_array_equal(cache[0, 0, 32:40], [0] * 8)
    assert cache[0, 0, H * B * D // 2 + 4] == 0
