"""GPU parity of the indexer logits (pkv_fp8_mqa_logits) against the CPU
oracle (binary64, exact dot products), within a bound derived from the
arithmetic; elements outside each row's range must be left untouched.

The bound.  The kernel's dot products run on v_mfma_f32_16x16x128_f8f6f4:
every fp8 x fp8 product is exact, but the unit adds each group of 8
consecutive products aligned to the group's largest and keeps about 13 bits
below it (measured on this GPU: with 2^16 and seven 2^q in one group, the
seven are dropped for q <= 2), then adds the group sums in binary32.  Per
head h, with p_k = q[h,k]*k[k]:
    |dot~ - dot| <= E_h = 2^-9 * sum_groups max|p| + 20 * 2^-24 * sum|p|
(over 2x the measured truncation; the test bounds max|p| over a group by
max|q| * max|k| over it).  ReLU is 1-Lipschitz; the sum over 64
heads and the final product with k_scale are binary32 operations:
    |L~ - L| <= k_scale * (sum_h |w_h| E_h + 80 * 2^-24 * sum_h |w_h| (|dot_h| + E_h))
                + 2^-23 |L|.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skip(reason="pkv_fp8_mqa_logits is switched off: a GPU run of the causal-range "
                            "case did not finish and its cause is not found yet"),
]

if torch.cuda.is_available():
    import paged_quantized_kv_amd as pkv

DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def banner(name):
    print(f"\n[case] {name}", flush=True)


def dec(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()


def bound(q, k, k_scale, w, ks, ke, cols, ref):
    """Per-element error bound (float64) for rows' valid entries; NaN elsewhere."""
    M, H, D = q.shape
    qd, kd = dec(q), dec(k)
    out = np.full((M, cols), np.nan)
    for i in range(M):
        lo, hi = max(int(ks[i]), 0), min(int(ke[i]), k.shape[0], int(ks[i]) + cols)
        if hi <= lo:
            continue
        qa, ka = np.abs(qd[i]), np.abs(kd[lo:hi])                   # [H, D], [n, D]
        # sum over groups of max|q_k k_k| <= sum over groups of max|q| * max|k|
        gmax = qa.reshape(H, D // 8, 8).max(2) @ ka.reshape(hi - lo, D // 8, 8).max(2).T
        E = 2.0 ** -9 * gmax + 20 * 2.0 ** -24 * (qa @ ka.T)       # [H, n]
        dots = np.abs(qd[i] @ kd[lo:hi].T)                            # [H, n]
        aw = np.abs(w[i].astype(np.float64))[:, None]
        b = k_scale[lo:hi].astype(np.float64) * ((aw * E).sum(0) +
                                                 80 * 2.0 ** -24 * (aw * (dots + E)).sum(0))
        out[i, lo - ks[i]:hi - ks[i]] = b + 2.0 ** -23 * np.abs(ref[i, lo - ks[i]:hi - ks[i]])
    return out


def check(q, k, k_scale, w, ks, ke, cols, stride_pad=0):
    M = q.shape[0]
    sentinel = np.float32(-1234.5)
    ref = np.full((M, cols), np.nan)
    oracle.fp8_mqa_logits(q, k, k_scale, w, ks, ke, ref)
    buf = torch.full((M, cols + stride_pad), float(sentinel), dtype=torch.float32, device=DEV)
    pkv.pkv_fp8_mqa_logits(dev(q).view(torch.float8_e4m3fn), dev(k), dev(k_scale), dev(w),
                           dev(ks), dev(ke), buf[:, :cols])
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    assert np.all(got[:, cols:] == sentinel)          # padding columns untouched
    got = got[:, :cols].astype(np.float64)
    valid = ~np.isnan(ref)
    assert np.all(got[~valid] == sentinel)            # outside the ranges: untouched
    b = bound(q, k, k_scale, w, ks, ke, cols, ref)
    err = np.abs(got[valid] - ref[valid])
    worst = np.max(err / b[valid]) if err.size else 0.0
    assert np.all(err <= b[valid]), f"max err/bound = {worst:.3g}"
    return worst


@pytest.mark.parametrize("H", [16, 32, 48, 64])
def test_logits_random_ranges(H):
    banner(f"mqa logits random ranges H={H}")
    g = workloads.mqa_logits_case(100 + H, num_q=37, num_heads=H, num_k=300)
    ks = g.ks.copy()
    ke = g.ke.copy()
    ks[:4] = [-5, 0, 290, 100]     # negative start, full range, short tail, empty
    ke[:4] = [20, 300, 350, 100]   # end past num_k
    worst = check(g.q, g.k, g.k_scale, g.weights, ks, ke, 200)
    print(f"max err / bound = {worst:.3g}")


def test_logits_causal_requests_and_padding():
    banner("mqa logits causal requests")
    g = workloads.mqa_logits_case(7, num_q=0, num_heads=64, num_k=0, causal_lens=[1, 70, 129, 5])
    check(g.q, g.k, g.k_scale, g.weights, g.ks, g.ke, int(max(g.ke - g.ks)), stride_pad=12)


def test_logits_from_the_gathered_keys():
    """Keys and scales as the path produces them: the fp8 store of bf16 K, then
    the gather back (k_scale read as float32)."""
    banner("mqa logits on gathered keys")
    w = workloads.c4_roundtrip()
    cache = w.cache_init.copy()
    oracle.store_indexer_k_fp8(w.k_bits, w.slot_mapping, cache, w.block_size, w.head_dim)
    T = int(w.cu_seq_lens[-1])
    kf = np.zeros((T, 128), np.uint8)
    ksb = np.zeros((T, 4), np.uint8)
    oracle.gather_indexer_k_fp8(cache, kf, ksb, w.block_table, w.cu_seq_lens, w.block_size, 128)
    k_scale = ksb.view(np.float32).reshape(T)
    keep = w.slot_mapping[:T] >= 0    # dropped slots hold stale bytes; use the stored tokens
    g = workloads.mqa_logits_case(11, num_q=0, num_heads=64, num_k=0,
                                  causal_lens=list(np.diff(w.cu_seq_lens)))
    kf[~keep] = 0
    k_scale = np.where(keep, k_scale, 0).astype(np.float32)
    worst = check(g.q[:T], kf, k_scale, g.weights[:T], g.ks[:T], g.ke[:T], 512)
    print(f"max err / bound = {worst:.3g}")


def test_logits_zero_and_extreme_codes():
    banner("mqa logits extreme codes")
    g = workloads.mqa_logits_case(13, num_q=16, num_heads=64, num_k=80)
    q, k = g.q.copy(), g.k.copy()
    q[0] = 0x7E                   # every q at +448
    q[1] = 0xFE                   # every q at -448: all dots negative where k > 0
    k[:8] = 0x7E
    k[8:16] = 0x01                # the smallest subnormal
    q[2, :, ::8] = 0x7E           # one large product per group of 8
    check(q, k, g.k_scale, g.weights, g.ks, g.ke, 80)
