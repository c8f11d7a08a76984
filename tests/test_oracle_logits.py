"""Pins for the oracle's indexer logits (the scores fp8_mqa_logits computes on
the gathered keys): a hand-worked case, an independent numpy reading (torch's
float8_e4m3fn decode, a float64 matmul), exactness of the dot products, and
the invariants of the formula (linearity in the weights, ReLU, scale zero,
range and column clipping)."""
import json
import os

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def dec(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()


def finite_codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38
    return c


def numpy_logits(q, k, k_scale, w, ks, ke, cols, fill=np.nan):
    M, H, D = q.shape
    out = np.full((M, cols), fill)
    qd, kd = dec(q), dec(k)
    for i in range(M):
        lo, hi = max(int(ks[i]), 0), min(int(ke[i]), k.shape[0])
        for j in range(lo, hi):
            if j - ks[i] >= cols:
                continue
            s = k_scale[j].astype(np.float64) * (qd[i] @ kd[j])      # [H]
            out[i, j - ks[i]] = np.sum(w[i].astype(np.float64) * np.maximum(s, 0.0))
    return out


def run_oracle(q, k, k_scale, w, ks, ke, cols, fill=np.nan):
    out = np.full((q.shape[0], cols), fill)
    oracle.fp8_mqa_logits(q, k, k_scale, w, ks, ke, out)
    return out


def test_w12_hand_worked():
    with open(os.path.join(GOLDEN, "w12_mqa_logits.json")) as f:
        g = json.load(f)
    h = lambda a: np.array([[int(x, 16) for x in row] for row in a], np.uint8)
    q = np.stack([h(t) for t in g["q"]])
    k = h(g["k"])
    out = run_oracle(q, k, np.array(g["k_scale"], np.float32), np.array(g["weights"], np.float32),
                     np.array(g["ks"], np.int32), np.array(g["ke"], np.int32), 3)
    np.testing.assert_array_equal(out, np.array(g["logits"]))


def test_matches_numpy_reading():
    rng = np.random.default_rng(1)
    M, H, D, N = 6, 8, 128, 40
    q, k = finite_codes(rng, (M, H, D)), finite_codes(rng, (N, D))
    k_scale = rng.uniform(0, 2, N).astype(np.float32)
    w = rng.normal(size=(M, H)).astype(np.float32)
    ks = np.array([0, 3, 10, 0, 39, 5], np.int32)
    ke = np.array([40, 17, 11, 1, 40, 5], np.int32)
    got = run_oracle(q, k, k_scale, w, ks, ke, 40)
    ref = numpy_logits(q, k, k_scale, w, ks, ke, 40)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    m = ~np.isnan(ref)
    np.testing.assert_allclose(got[m], ref[m], rtol=1e-13, atol=1e-300)


def test_dot_products_are_exact():
    # one head, weight 1, scale 1: the logit is relu(q.k) exactly (compare
    # with exact rationals)
    from fractions import Fraction
    rng = np.random.default_rng(2)
    q, k = finite_codes(rng, (3, 1, 128)), finite_codes(rng, (5, 128))
    out = run_oracle(q, k, np.ones(5, np.float32), np.ones((3, 1), np.float32),
                     np.zeros(3, np.int32), np.full(3, 5, np.int32), 5)
    qd, kd = dec(q), dec(k)
    for i in range(3):
        for j in range(5):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(qd[i, 0], kd[j]))
            assert out[i, j] == float(max(exact, 0)), (i, j)


def test_invariants():
    rng = np.random.default_rng(3)
    M, H, D, N = 4, 16, 128, 24
    q, k = finite_codes(rng, (M, H, D)), finite_codes(rng, (N, D))
    k_scale = rng.uniform(0.1, 2, N).astype(np.float32)
    w = rng.normal(size=(M, H)).astype(np.float32)
    ks, ke = np.zeros(M, np.int32), np.full(M, N, np.int32)
    base = run_oracle(q, k, k_scale, w, ks, ke, N)
    # linear in the weights (scaling by 2 is exact)
    np.testing.assert_array_equal(run_oracle(q, k, k_scale, (w * 2).astype(np.float32), ks, ke, N),
                                  2 * base)
    # a zero key scale gives zero
    np.testing.assert_array_equal(run_oracle(q, k, np.zeros(N, np.float32), w, ks, ke, N), 0.0)
    # ReLU: with q negated, each head contributes where its dot was negative
    qneg = q ^ 0x80
    pos = run_oracle(q, k, k_scale, np.abs(w), ks, ke, N)
    neg = run_oracle(qneg, k, k_scale, np.abs(w), ks, ke, N)
    both = run_oracle(q, k, k_scale, np.abs(w), ks, ke, N) + neg
    full = np.zeros((M, N))
    qd, kd = dec(q), dec(k)
    for i in range(M):
        full[i] = (np.abs(w[i]).astype(np.float64)[:, None] *
                   np.abs(k_scale.astype(np.float64)[None, :] * (qd[i] @ kd.T))).sum(0)
    np.testing.assert_allclose(both, full, rtol=1e-13)
    assert np.all(pos >= 0) and np.all(neg >= 0)


def test_ranges_and_clipping_leave_the_rest_untouched():
    rng = np.random.default_rng(4)
    M, H, D, N = 5, 4, 128, 16
    q, k = finite_codes(rng, (M, H, D)), finite_codes(rng, (N, D))
    k_scale = rng.uniform(0.1, 2, N).astype(np.float32)
    w = rng.normal(size=(M, H)).astype(np.float32)
    ks = np.array([-3, 4, 10, 2, 7], np.int32)     # a negative start is clipped to 0
    ke = np.array([5, 4, 30, 16, 8], np.int32)     # an end past N is clipped; ks == ke is empty
    cols = 6                                      # columns past 6 are not written
    got = run_oracle(q, k, k_scale, w, ks, ke, cols, fill=-7.0)
    ref = numpy_logits(q, k, k_scale, w, ks, ke, cols, fill=-7.0)
    np.testing.assert_allclose(got, ref, rtol=1e-13)
    assert np.all(got[1] == -7.0)                  # empty range
    assert np.all(got[0, :3] == -7.0)              # columns j - ks < 3 have j < 0
    assert np.all(got[2] != -7.0)                  # row 2: j in [10, 16) fills columns 0..5
    assert np.all(got[4, 1:] == -7.0)              # row 4: only j = 7, column 0
