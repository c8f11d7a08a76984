"""The whole path captured in one HIP graph (torch.cuda.CUDAGraph): the fp8
indexer store, the gather, the indexer read-back, the NVFP4 store and its
read-back, and the decode attention.  The library allocates nothing, never
synchronizes and records no memset, so the captured launches are the eager
ones; every replay, with eager work and synchronizations between replays,
must reproduce the eager results bit for bit."""
import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import paged_quantized_kv_amd as pkv

DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bits(t):
    return t.view(torch.uint8).clone() if t.dtype != torch.uint8 else t.clone()


def test_path_captured_in_a_hip_graph():
    print("\n[case] whole path in one HIP graph, three replays", flush=True)
    w = workloads.c4_roundtrip()
    fp = workloads.paged_fp4(71, [40, 16, 7, 33], H=2, D=128, B=16)
    c = workloads.paged_attention_case(72, 6, 64, 8, lens=[900, 1, 513, 64, 2000, 100])
    T = int(w.cu_seq_lens[-1])
    T4 = fp.num_tokens
    S, H, D = c.query.shape
    maxc = int(c.context_lens.max())

    k = dev(w.k_bits.view(np.int16)).view(torch.bfloat16)
    slots = dev(w.slot_mapping)
    cache0 = dev(w.cache_init)
    cache = cache0.clone()
    bt, cu = dev(w.block_table), dev(w.cu_seq_lens)
    kf0, ks0 = dev(w.k_fp8_init[:T]), dev(w.k_scale_init[:T])
    kf, ks = kf0.clone(), ks0.clone()
    deq = torch.empty((T, w.head_dim), dtype=torch.bfloat16, device=DEV)

    shape4 = (T4, fp.num_heads, fp.head_size)
    key4 = dev(fp.key_bits.view(np.int16)).view(torch.bfloat16).view(shape4)
    val4 = dev(fp.value_bits.view(np.int16)).view(torch.bfloat16).view(shape4)
    slot4 = dev(fp.slot_mapping)
    c40 = dev(fp.cache_init)
    c4 = c40.clone()
    k4s = torch.tensor([fp.k_scale], dtype=torch.float32, device=DEV)
    v4s = torch.tensor([fp.v_scale], dtype=torch.float32, device=DEV)
    bt4, cu4 = dev(fp.block_table), dev(fp.cu_seq_lens)
    R4 = int(fp.cu_seq_lens[-1])
    ko = torch.empty((R4, fp.num_heads, fp.head_size), dtype=torch.bfloat16, device=DEV)
    vo = torch.empty_like(ko)

    q = dev(c.query.view(np.int16)).view(torch.bfloat16)
    kc, vc = dev(c.key_cache), dev(c.value_cache)
    abt, acl = dev(c.block_tables), dev(c.context_lens)
    out = torch.empty((S, H, D), dtype=torch.bfloat16, device=DEV)
    ws = pkv.paged_attention_workspace(S, H, maxc, 256, device=DEV)

    outputs = [cache, kf, ks, deq, c4, ko, vo, out]

    def reset():
        cache.copy_(cache0)
        kf.copy_(kf0)
        ks.copy_(ks0)
        c4.copy_(c40)
        for t in (deq, ko, vo, out):
            t.view(torch.int16).fill_(0x7FC1)   # a NaN pattern nothing writes

    def step():
        pkv.pkv_store_indexer_k_fp8(k, slots, cache, block_size=w.block_size)
        pkv.pkv_gather_indexer_k_fp8(cache, kf, ks, bt, cu, block_size=w.block_size)
        pkv.pkv_gather_indexer_k_dequant(cache, deq, bt, cu, block_size=w.block_size)
        pkv.pkv_store_kv_fp4(key4, val4, c4[:, 0], c4[:, 1], slot4, k4s, v4s,
                             block_size=fp.block_size, layout=fp.layout)
        pkv.pkv_gather_kv_fp4_dequant(c4[:, 0], c4[:, 1], ko, vo, bt4, cu4, k4s, v4s,
                                      block_size=fp.block_size, layout=fp.layout)
        pkv.pkv_paged_attention_decode(out, *ws, q, kc, vc, c.num_kv_heads, c.scale, abt, acl, 16,
                                       maxc, c.k_scale, c.v_scale, partition_size=256)

    reset()
    step()
    torch.cuda.synchronize()
    eager = [bits(t) for t in outputs]

    g = torch.cuda.CUDAGraph()
    reset()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    side = torch.empty_like(deq)
    for rep in range(3):
        reset()
        # eager work of the program between replays
        pkv.pkv_gather_indexer_k_dequant(cache0, side, bt, cu, block_size=w.block_size)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (t, e) in enumerate(zip(outputs, eager)):
            assert torch.equal(bits(t), e), f"replay {rep}: output {i} differs from the eager run"


def test_allocation_free_attention_captured_in_a_hip_graph():
    """The allocation-free attention (its workspace the library's own device
    array) captured in a graph; between replays an eager call of the same
    entry point on another batch rewrites that array.  Every replay must
    reproduce the eager result bit for bit."""
    print("\n[case] allocation-free attention in a HIP graph, three replays", flush=True)
    c = workloads.paged_attention_case(73, 8, 64, 8, lens=[700, 1, 2100, 64, 0, 333, 1024, 5])
    o = workloads.paged_attention_case(74, 5, 32, 4, lens=[1500, 3, 800, 64, 900])
    args = []
    for case in (c, o):
        S, H, D = case.query.shape
        args.append(dict(
            out=torch.empty((S, H, D), dtype=torch.bfloat16, device=DEV),
            query=dev(case.query.view(np.int16)).view(torch.bfloat16),
            key_cache=dev(case.key_cache), value_cache=dev(case.value_cache),
            num_kv_heads=case.num_kv_heads, scale=case.scale,
            block_tables=dev(case.block_tables), context_lens=dev(case.context_lens),
            block_size=16, max_context_len=int(case.context_lens.max()),
            k_scale=case.k_scale, v_scale=case.v_scale, partition_size=256))

    def call(a):
        pkv.pkv_paged_attention_decode_noalloc(**a)

    call(args[0])
    torch.cuda.synchronize()
    eager = bits(args[0]["out"])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(args[0])
    torch.cuda.synchronize()
    for rep in range(3):
        args[0]["out"].view(torch.int16).fill_(0x7FC1)
        call(args[1])                      # another batch through the same array
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(args[0]["out"]), eager), f"replay {rep} differs from the eager run"
