"""GPU parity of calls that the C ABI splits into several launches.

The fp8 store and the dense-table gather size their grids from the input,
so calls of more than 2^22 tokens (store) or block-table entries (gather)
are enqueued as several launches over token or request ranges.  These
cases cross that boundary -- a second launch of 777 tokens, and a second
launch of 3 requests -- and compare the whole cache and the whole outputs,
guard rows included, byte for byte with the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import paged_quantized_kv_amd as pkv

DEV = "cuda:0"
PER_LAUNCH = 1 << 22   # tokens per store launch, table entries per gather launch


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def test_store_fp8_split_over_two_launches():
    T, D, B = PER_LAUNCH + 777, 128, 64
    print(f"\n[case] fp8 store split launch: {T} tokens, D={D}, B={B}", flush=True)
    g = workloads.rng(3101)
    num_blocks = -(-T // B) + 16
    distinct = g.permutation(num_blocks * B)[:T].astype(np.int64)
    slots = distinct.copy()
    slots[g.choice(T, size=T // 20, replace=False)] = -1
    edge = slice(PER_LAUNCH - 3, PER_LAUNCH + 3)                  # around the split
    slots[edge] = distinct[edge]
    k_bits = workloads.bf16_bits(workloads.normal_f32(g, (T, D)))
    cache0 = workloads.random_bytes(g, (num_blocks, B * (D + 4)))
    ref = cache0.copy()
    oracle.store_indexer_k_fp8(k_bits, slots, ref, B, D)
    cache = dev(cache0)
    pkv.pkv_store_indexer_k_fp8(dev(k_bits.view(np.int16)).view(torch.bfloat16), dev(slots),
                                cache, block_size=B)
    torch.cuda.synchronize()
    got = cache.cpu().numpy()
    np.testing.assert_array_equal(got, ref)


def test_gather_split_over_two_launches():
    R, maxb, B, D, pages = 2 * (PER_LAUNCH // 4) + 3, 2, 64, 128, 4096
    print(f"\n[case] gather split launch: {R} requests x {maxb} table columns", flush=True)
    assert R * maxb > PER_LAUNCH
    g = workloads.rng(3102)
    lens = g.integers(0, 4, size=R).astype(np.int64)
    long_reqs = g.choice(R, size=200, replace=False)
    lens[long_reqs] = g.integers(65, 129, size=200)                # both table columns
    lens[PER_LAUNCH // maxb - 2:PER_LAUNCH // maxb + 3] = [100, 7, 128, 1, 70]  # around the split
    cu = np.zeros(R + 1, np.int64)
    cu[1:] = np.cumsum(lens)
    cu = cu.astype(np.int32)
    T = int(cu[-1])
    table = g.integers(0, pages, size=(R, maxb)).astype(np.int32)  # pages may be shared
    bad = g.choice(R * maxb, size=1000, replace=False)
    table.reshape(-1)[bad[:500]] = -1
    table.reshape(-1)[bad[500:]] = pages + 7
    cache = workloads.random_bytes(g, (pages, B * (D + 4)))
    kf0 = workloads.random_bytes(g, (T + 3, D))
    ks0 = workloads.random_bytes(g, (T + 3, 4))
    ref_f, ref_s = kf0.copy(), ks0.copy()
    oracle.gather_indexer_k_fp8(cache, ref_f, ref_s, table, cu, B, D)
    kf, ks = dev(kf0), dev(ks0)
    pkv.pkv_gather_indexer_k_fp8(dev(cache), kf, ks, dev(table), dev(cu), block_size=B)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(kf.cpu().numpy(), ref_f)
    np.testing.assert_array_equal(ks.cpu().numpy(), ref_s)
