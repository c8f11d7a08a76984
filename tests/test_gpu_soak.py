"""Repeatability under varied timing: thousands of decode-attention calls,
interleaved with the stores and the gather on other buffers and with the
partition size alternating, must each give the bit-identical output of the
first call (the kernels are deterministic: any difference would be a
timing-dependent error, such as an MFMA register read before it is
written); the stores and the gather, repeated over the same inputs, must
keep giving the oracle's bytes."""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import paged_quantized_kv_amd as pkv

DEV = "cuda:0"
CALLS = 10000


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def test_repeated_calls_are_bit_identical():
    print(f"\n[case] soak: {CALLS} decode-attention calls interleaved with the stores", flush=True)
    c = workloads.decode_batch()
    S, H, D = c.query.shape
    B = c.key_cache.shape[3]
    maxc = int(c.context_lens.max())
    q = dev(c.query.view(np.int16)).view(torch.bfloat16)
    kc, vc, bt, cl = dev(c.key_cache), dev(c.value_cache), dev(c.block_tables), dev(c.context_lens)
    outs, wss, refs = {}, {}, {}
    for P in (1024, 256):
        outs[P] = torch.empty((S, H, D), dtype=torch.bfloat16, device=DEV)
        wss[P] = pkv.paged_attention_workspace(S, H, maxc, P, device=DEV)

    def attend(P):
        pkv.pkv_paged_attention_decode(outs[P], *wss[P], q, kc, vc, c.num_kv_heads, c.scale, bt,
                                       cl, B, maxc, c.k_scale, c.v_scale, partition_size=P)

    for P in (1024, 256):
        attend(P)
        torch.cuda.synchronize()
        refs[P] = outs[P].clone()

    # stores and gather of a round-trip batch, with their oracle bytes
    w = workloads.c4_roundtrip()
    cache_ref = w.cache_init.copy()
    oracle.store_indexer_k_fp8(w.k_bits, w.slot_mapping, cache_ref, 64, 128)
    kf_ref, ks_ref = w.k_fp8_init.copy(), w.k_scale_init.copy()
    oracle.gather_indexer_k_fp8(cache_ref, kf_ref, ks_ref, w.block_table, w.cu_seq_lens, 64, 128)
    f = workloads.c5_nvfp4_store()
    c4_ref = f.cache_init.copy()
    oracle.store_kv_fp4(f.key_bits, f.value_bits, c4_ref, f.slot_mapping, 8, 128, 16, 0,
                        f.k_scale, f.v_scale)
    k = dev(w.k_bits.view(np.int16)).view(torch.bfloat16)
    sl, cache, kf, ks = dev(w.slot_mapping), dev(w.cache_init), dev(w.k_fp8_init), dev(w.k_scale_init)
    btw, cuw = dev(w.block_table), dev(w.cu_seq_lens)
    T4 = f.num_tokens
    key = dev(f.key_bits.view(np.int16)).view(torch.bfloat16).view(T4, 8, 128)
    val = dev(f.value_bits.view(np.int16)).view(torch.bfloat16).view(T4, 8, 128)
    sl4, c4 = dev(f.slot_mapping), dev(f.cache_init)
    k4s = torch.tensor([f.k_scale], dtype=torch.float32, device=DEV)
    v4s = torch.tensor([f.v_scale], dtype=torch.float32, device=DEV)

    bad = torch.zeros((), dtype=torch.int64, device=DEV)
    for i in range(CALLS):
        P = 1024 if i % 3 else 256
        attend(P)
        bad += (outs[P].view(torch.int16) != refs[P].view(torch.int16)).any().to(torch.int64)
        if i % 4 == 0:
            pkv.pkv_store_indexer_k_fp8(k, sl, cache, block_size=64)
            pkv.pkv_gather_indexer_k_fp8(cache, kf, ks, btw, cuw, block_size=64)
        if i % 7 == 0:
            pkv.pkv_store_kv_fp4(key, val, c4[:, 0], c4[:, 1], sl4, k4s, v4s, block_size=16,
                                 layout=0)
        if i % 2000 == 1999:
            torch.cuda.synchronize()
            assert int(bad) == 0, f"attention output changed within the first {i + 1} calls"
            np.testing.assert_array_equal(cache.cpu().numpy(), cache_ref)
            np.testing.assert_array_equal(kf.cpu().numpy(), kf_ref)
            np.testing.assert_array_equal(ks.cpu().numpy(), ks_ref)
            np.testing.assert_array_equal(c4.cpu().numpy(), c4_ref)
            print(f"{i + 1} calls: identical", flush=True)
    torch.cuda.synchronize()
    assert int(bad) == 0


def test_bench_step_repeats_bit_identically():
    """The benchmark's step -- fp8 store, NVFP4 store, gather over the 256 x
    1000-token batch -- repeated 500 times over one buffer set gives the
    same bytes every time (the first step's, which the parity tests compare
    with the oracle)."""
    print("\n[case] soak: 500 steps of the 256 x 1000-token batch", flush=True)
    w = workloads.c2_prefill_256x1000()
    f = workloads.prefill_fp4()
    T = w.num_tokens
    k = dev(w.k_bits.view(np.int16)).view(torch.bfloat16)
    sl, cache = dev(w.slot_mapping), dev(w.cache_init)
    kf, ks = dev(w.k_fp8_init[:T]), dev(w.k_scale_init[:T])
    bt, cu = dev(w.block_table), dev(w.cu_seq_lens)
    key = dev(f.key_bits.view(np.int16)).view(torch.bfloat16).view(T, 8, 128)
    val = dev(f.value_bits.view(np.int16)).view(torch.bfloat16).view(T, 8, 128)
    sl4, c4 = dev(f.slot_mapping), dev(f.cache_init)
    k4s = torch.tensor([f.k_scale], dtype=torch.float32, device=DEV)
    v4s = torch.tensor([f.v_scale], dtype=torch.float32, device=DEV)

    def step():
        pkv.pkv_store_indexer_k_fp8(k, sl, cache, block_size=64)
        pkv.pkv_store_kv_fp4(key, val, c4[:, 0], c4[:, 1], sl4, k4s, v4s, block_size=16,
                             layout=0)
        pkv.pkv_gather_indexer_k_fp8(cache, kf, ks, bt, cu, block_size=64)

    step()
    torch.cuda.synchronize()
    refs = [t.clone() for t in (cache, c4, kf, ks)]
    bad = torch.zeros((), dtype=torch.int64, device=DEV)
    for i in range(500):
        # the outputs are rewritten with the same bytes: clear the gather's
        # outputs first so that a skipped write would show
        kf.zero_()
        ks.zero_()
        step()
        for t, r in zip((cache, c4, kf, ks), refs):
            bad += (t != r).any().to(torch.int64)
    torch.cuda.synchronize()
    assert int(bad) == 0
