"""Pins for the oracle's fp16 source path (the NVFP4 dispatcher on the vLLM
page covers both 16-bit float types).

The widening is checked against numpy's binary16 -> binary32 conversion on
all 65536 patterns (a library routine); the hand-worked fp8 and NVFP4 cases
use values that are exact in both 16-bit formats, so the fp16 path must give
the same bytes as the bf16 path; the error bounds and invariants hold on
random fp16 inputs, including subnormals and values near the fp16 maximum.
"""
import numpy as np
import pytest

import oracle
import workloads
from conftest import load_golden


def test_f16_widening_matches_numpy_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = oracle.f16_to_f32(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def store_one(x, dtype, head_dim=128, block_size=4, slot=5):
    cache = np.zeros((3, block_size * (head_dim + 4)), np.uint8)
    kb = workloads.half_bits(np.asarray(x, np.float32).reshape(1, head_dim), dtype)
    oracle.store_indexer_k_fp8(kb, np.array([slot], np.int64), cache, block_size, head_dim,
                               dtype=dtype)
    p, off = divmod(slot, block_size)
    return (cache[p, off * head_dim:(off + 1) * head_dim],
            cache[p, block_size * head_dim + off * 4: block_size * head_dim + off * 4 + 4])


@pytest.mark.parametrize("name", ["w1_fp8_exact_scale.json", "w3_fp8_inexact_scale.json"])
def test_fp8_golden_through_f16(name):
    gd = load_golden(name)
    x = np.zeros(128, np.float32)
    x[:len(gd["x"])] = gd["x"]
    assert np.array_equal(x.astype(np.float16).astype(np.float32), x)  # exact in fp16
    codes, sb = store_one(x, "f16")
    want = [int(c, 16) for c in gd["codes"]] + [0] * (128 - len(gd["codes"]))
    np.testing.assert_array_equal(codes, want)
    np.testing.assert_array_equal(sb, [int(c, 16) for c in gd["scale_bytes_le"]])


def test_fp8_bound_and_invariants_f16():
    g = workloads.rng(12)
    x = g.standard_normal((3000, 128)).astype(np.float32)
    x[::50] *= np.float32(2.0 ** -16)          # fp16 subnormal territory
    x[7::97] *= np.float32(3000.0)             # near the fp16 maximum
    x = np.clip(x, -65504, 65504)
    kb = workloads.f16_bits(x)
    xf = kb.view(np.float16).astype(np.float64)
    T = x.shape[0]
    cache = np.zeros((T, 132), np.uint8)
    oracle.store_indexer_k_fp8(kb, np.arange(T, dtype=np.int64), cache, 1, 128, dtype="f16")
    codes, s = cache[:, :128], cache[:, 128:].copy().view("<f4")[:, 0].astype(np.float64)
    q = oracle.e4m3_decode(codes.ravel()).reshape(codes.shape).astype(np.float64)
    y = xf / s[:, None]
    a = np.abs(y)
    h = np.where(a >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 4), 2.0 ** -10)
    assert (np.abs(xf - q * s[:, None]) <= (h + a * 2.0 ** -24) * s[:, None]).all()
    assert ((codes & 0x7F).max(axis=1) == 0x7E).all()
    np.testing.assert_allclose(s, np.abs(xf).max(axis=1) / 448, rtol=2 ** -24)


@pytest.mark.parametrize("name", ["w4_nvfp4_unit_scale.json", "w5_nvfp4_scale2.json"])
def test_nvfp4_golden_through_f16(name):
    gd = load_golden(name)
    H, D, B = 1, 64, 4
    x = np.zeros((1, 64), np.float32)
    x[0, :16] = gd["x"]
    assert np.array_equal(x.astype(np.float16).astype(np.float32), x)
    side = H * B * (D // 2 + D // 16)
    cache = np.zeros((2, 2, side), np.uint8)
    kb = workloads.f16_bits(x)
    oracle.store_kv_fp4(kb, kb, cache, np.array([6], np.int64), H, D, B, 0, gd["scale"],
                        gd["scale"], dtype="f16")
    p, off = divmod(6, B)
    for kv in (0, 1):
        np.testing.assert_array_equal(cache[p, kv, off * 32: off * 32 + 8],
                                      [int(c, 16) for c in gd["data_bytes"]])
    assert cache[p, 0, H * B * D // 2 + off * 4] == int(gd["scale_byte"], 16)


def test_nvfp4_f16_matches_bf16_on_common_values():
    """Inputs exact in both formats give identical pages through both paths."""
    g = workloads.rng(31)
    T, H, D, B = 40, 2, 128, 8
    # values with at most 8 significant bits and exponents inside fp16's range
    x = (g.integers(-255, 256, size=(2, T, H * D)) * 2.0 ** g.integers(-14, 6, size=(2, T, 1)))
    x = x.astype(np.float32)
    assert np.array_equal(x.astype(np.float16).astype(np.float32), x)
    assert np.array_equal(workloads.bf16_bits(x).astype(np.uint32) << 16, x.view(np.uint32))
    slots = g.permutation(8 * B)[:T].astype(np.int64)
    side = H * B * (D // 2 + D // 16)
    pages = []
    for dt in ("bf16", "f16"):
        cache = np.zeros((8, 2, side), np.uint8)
        oracle.store_kv_fp4(workloads.half_bits(x[0], dt), workloads.half_bits(x[1], dt), cache,
                            slots, H, D, B, 0, 0.75, 1.5, dtype=dt)
        pages.append(cache)
    np.testing.assert_array_equal(pages[0], pages[1])
