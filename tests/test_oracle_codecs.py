"""Pins for the oracle's E4M3 and E2M1 codecs.

Each codec is checked against (1) a brute-force nearest-grid-value search in
numpy float64 with ties to the even code, over every bf16 pattern and a
structured set that walks every binade with every kept-bit pattern and the
round/sticky cases; (2) decode -> encode identity on every code; (3) every
midpoint between adjacent codes going to the even neighbour; (4) for E4M3,
torch's CPU float8_e4m3fn cast, a library special case, where it saturates
the same way (|y| < 464).
"""
import numpy as np
import pytest
import torch

import oracle

E4M3_POS = np.array([oracle.e4m3_decode(np.array([c], np.uint8))[0] for c in range(0x7F)],
                    dtype=np.float64)  # codes 0x00..0x7E
E2M1_POS = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)


def test_e4m3_decode_table_closed_form():
    # E4M3FN: subnormal m*2^-9, normal (1+m/8)*2^(e-7); closed form per code
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        want = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        assert E4M3_POS[c] == want
    assert E4M3_POS[0x7E] == 448.0
    assert np.isnan(oracle.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()


def brute_nearest(a, grid, chunk=8192):
    """Index of the nearest grid value; ties go to the even index; above the top
    value saturates.  Every grid value is compared (in row chunks)."""
    a = np.asarray(a, np.float64)
    if a.size > chunk:
        return np.concatenate([brute_nearest(a[i:i + chunk], grid, chunk)
                               for i in range(0, a.size, chunk)])
    a = a[:, None]
    d = np.abs(a - grid[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    n = grid.size
    idx = np.where(cand, np.arange(n)[None, :], n + 1)
    even = np.where(cand & (np.arange(n)[None, :] % 2 == 0), np.arange(n)[None, :], n + 1)
    one = idx.min(axis=1)
    ev = even.min(axis=1)
    n_cand = cand.sum(axis=1)
    out = np.where(n_cand > 1, ev, one)
    out = np.where(a[:, 0] >= grid[-1], n - 1, out)
    return out.astype(np.uint8)


def brute_e4m3(y):
    y = np.asarray(y, np.float32)
    code = brute_nearest(np.abs(y.astype(np.float64)), E4M3_POS)
    return code | np.where(np.signbit(y), 0x80, 0).astype(np.uint8)


def brute_e2m1(y):
    y = np.asarray(y, np.float32)
    code = brute_nearest(np.abs(y.astype(np.float64)), E2M1_POS)
    return code | np.where(np.signbit(y), 0x8, 0).astype(np.uint8)


def all_bf16_finite():
    b = np.arange(1 << 16, dtype=np.uint32) << 16
    f = b.view(np.float32)
    return f[np.isfinite(f)]


def structured_f32(exp_lo, exp_hi, top_bits=11):
    """Every binade in [2^exp_lo, 2^exp_hi), every pattern of the top `top_bits`
    fraction bits, low bits in {0, 1, half-1, half, half+1, all ones}, both signs."""
    lows = np.array([0, 1, (1 << (22 - top_bits)) - 1, 1 << (22 - top_bits),
                     (1 << (22 - top_bits)) + 1, (1 << (23 - top_bits)) - 1], np.uint32)
    tops = np.arange(1 << top_bits, dtype=np.uint32) << (23 - top_bits)
    out = []
    for e in range(exp_lo, exp_hi):
        base = np.uint32((e + 127) << 23)
        out.append((base | tops[:, None] | lows[None, :]).ravel())
    bits = np.concatenate(out)
    bits = np.concatenate([bits, bits | np.uint32(0x80000000)])
    return bits.view(np.float32)


@pytest.mark.parametrize("chunk", range(4))
def test_e4m3_matches_bruteforce_structured(chunk):
    y = structured_f32(-20 + 8 * chunk, -12 + 8 * chunk)  # binades 2^-20 .. 2^12
    got = oracle.e4m3_encode(y)
    np.testing.assert_array_equal(got, brute_e4m3(y))


def test_e4m3_matches_bruteforce_all_bf16_and_specials():
    y = np.concatenate([all_bf16_finite(),
                        np.array([0.0, -0.0, np.inf, -np.inf, 1e-45, -1e-45, 463.99997,
                                  464.0, 464.00003, 3.4e38], np.float32)])
    np.testing.assert_array_equal(oracle.e4m3_encode(y), brute_e4m3(y))


def test_e4m3_matches_torch_cast_below_464():
    g = np.random.Generator(np.random.PCG64(7))
    y = (g.standard_normal(1 << 20) * np.exp(g.uniform(-14, 6.1, 1 << 20))).astype(np.float32)
    y = y[np.abs(y) < 464]
    y = np.concatenate([y, all_bf16_finite()])
    y = y[np.abs(y) < 464]
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.e4m3_encode(y), ref)


def test_e4m3_roundtrip_every_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = oracle.e4m3_decode(codes)
    np.testing.assert_array_equal(oracle.e4m3_encode(vals), codes)


def test_e4m3_midpoints_go_to_even_code():
    for c in range(0x7E):
        lo, hi = E4M3_POS[c], E4M3_POS[c + 1]
        mid = np.float32((lo + hi) / 2)
        assert float(mid) == (lo + hi) / 2  # exactly representable
        want = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_encode(np.array([mid]))[0] == want
        assert oracle.e4m3_encode(np.array([-mid]))[0] == want | 0x80
        # one binary32 ulp either side decides by distance
        below = np.nextafter(mid, np.float32(0))
        above = np.nextafter(mid, np.float32(1e9))
        assert oracle.e4m3_encode(np.array([below]))[0] == c
        assert oracle.e4m3_encode(np.array([above]))[0] == c + 1


def test_e4m3_saturates():
    y = np.array([448, 463.9, 464, 1e6, np.inf, -np.inf, -500], np.float32)
    np.testing.assert_array_equal(oracle.e4m3_encode(y),
                                  [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE])


def test_e2m1_matches_bruteforce():
    y = np.concatenate([all_bf16_finite(), structured_f32(-6, 5, top_bits=8)])
    np.testing.assert_array_equal(oracle.e2m1_encode(y), brute_e2m1(y))


def test_e2m1_roundtrip_and_midpoints():
    codes = np.arange(16, dtype=np.uint8)
    vals = oracle.e2m1_decode(codes)
    np.testing.assert_array_equal(vals[:8], E2M1_POS.astype(np.float32))
    np.testing.assert_array_equal(vals[8:], -E2M1_POS.astype(np.float32))
    np.testing.assert_array_equal(oracle.e2m1_encode(vals), codes)
    for c in range(7):
        mid = np.float32((E2M1_POS[c] + E2M1_POS[c + 1]) / 2)
        want = c if c % 2 == 0 else c + 1
        assert oracle.e2m1_encode(np.array([mid]))[0] == want
        assert oracle.e2m1_encode(np.array([np.nextafter(mid, np.float32(0))]))[0] == c
        assert oracle.e2m1_encode(np.array([np.nextafter(mid, np.float32(9))]))[0] == c + 1
    np.testing.assert_array_equal(
        oracle.e2m1_encode(np.array([6.0, 7.0, 1e30, np.inf, -8.0], np.float32)),
        [7, 7, 7, 7, 15])


def test_bf16_widening_exact():
    lib = oracle._load()
    for b in [0x0000, 0x8000, 0x3F80, 0xBF80, 0x0001, 0x7F7F, 0x3DCD]:
        want = np.array([b << 16], np.uint32).view(np.float32)[0]
        assert lib.oracle_bf16_to_f32(b) == want
