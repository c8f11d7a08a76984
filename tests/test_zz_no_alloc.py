"""The allocation-free decode attention (pkv_paged_attention_decode_noalloc,
its workspace in the library's built-in per-GPU scratch array) against the
entry point with a caller workspace (pkv_paged_attention_decode): the same
kernels on the same inputs, so the outputs must be identical bit for bit;
both are also held to the oracle's bound.  Two calls in a row, the second
smaller, so the second runs over the first call's leftovers in the scratch.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle.attention_bound import attention_bound

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import paged_quantized_kv_amd as pkv

DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def both(c, P):
    """Outputs of the caller-workspace and the allocation-free entry point."""
    S, H, D = c.query.shape
    B = c.key_cache.shape[3]
    maxc = int(c.context_lens.max(initial=0))
    q = dev(c.query.view(np.int16)).view(torch.bfloat16)
    kc, vc, bt, cl = dev(c.key_cache), dev(c.value_cache), dev(c.block_tables), dev(c.context_lens)
    outs = []
    for noalloc in (False, True):
        out = torch.full((S, H, D), float("nan"), dtype=torch.bfloat16, device=DEV)
        if noalloc:
            pkv.pkv_paged_attention_decode_noalloc(out, q, kc, vc, c.num_kv_heads, c.scale, bt,
                                                   cl, B, maxc, c.k_scale, c.v_scale,
                                                   partition_size=P)
        else:
            ws = pkv.paged_attention_workspace(S, H, maxc, P, device=DEV)
            pkv.pkv_paged_attention_decode(out, *ws, q, kc, vc, c.num_kv_heads, c.scale, bt, cl,
                                           B, maxc, c.k_scale, c.v_scale, partition_size=P)
        torch.cuda.synchronize()
        outs.append(out.view(torch.int16).cpu().numpy())
    return outs


def within_bound(c, got_bits):
    ref = oracle.paged_attention_decode(c.query, c.key_cache, c.value_cache, c.block_tables,
                                        c.context_lens, c.num_kv_heads, c.scale, c.k_scale,
                                        c.v_scale)
    b = attention_bound(c.query, c.key_cache, c.value_cache, c.block_tables, c.context_lens,
                        c.num_kv_heads, c.scale, c.k_scale, c.v_scale)
    got = torch.from_numpy(got_bits).view(torch.bfloat16).to(torch.float64).numpy()
    assert not np.isnan(got).any()
    assert np.all(got[b == 0] == 0)
    assert np.all(np.abs(got - ref) <= b)


def test_noalloc_matches_the_caller_workspace_entry_point_twice():
    # call 1: 24 sequences with Llama-3.1-70B heads, mixed contexts (balanced split)
    lens1 = workloads.rng(71).integers(128, 2561, size=24).tolist()
    c1 = workloads.paged_attention_case(71, len(lens1), 64, 8, lens=lens1)
    print(f"\n[case] noalloc call 1: 24 seqs, H=64, KVH=8, P=1024", flush=True)
    ref1, got1 = both(c1, 1024)
    np.testing.assert_array_equal(got1, ref1)
    within_bound(c1, got1)
    # call 2, smaller: 5 sequences, an empty one, 4 query heads per KV head (fixed split)
    lens2 = [1, 40, 300, 0, 1000]
    c2 = workloads.paged_attention_case(72, len(lens2), 8, 2, lens=lens2)
    print("[case] noalloc call 2: 5 seqs, H=8, KVH=2, P=256", flush=True)
    ref2, got2 = both(c2, 256)
    np.testing.assert_array_equal(got2, ref2)
    within_bound(c2, got2)


def test_noalloc_rejects_a_workspace_larger_than_the_scratch():
    """Checked on the host before any HIP call: nothing is enqueued."""
    c = workloads.paged_attention_case(73, 2, 8, 2, lens=[10, 20])
    S, H, D = c.query.shape
    out = torch.zeros((S, H, D), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(pkv.PkvError, match="built-in scratch"):
        # 2 x 8 heads x 2^30 / 64 partitions: 2^31 bytes of partial rows
        pkv.pkv_paged_attention_decode_noalloc(
            out, dev(c.query.view(np.int16)).view(torch.bfloat16), dev(c.key_cache),
            dev(c.value_cache), c.num_kv_heads, c.scale, dev(c.block_tables),
            dev(c.context_lens), c.key_cache.shape[3], 1 << 30, c.k_scale, c.v_scale,
            partition_size=64)
