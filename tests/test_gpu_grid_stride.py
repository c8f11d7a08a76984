"""GPU parity where the grid-stride kernels take more than one pass.

The NVFP4 store, the gather's wide-table kernel and both read-backs cap
their grids at 65536 workgroups and loop over the rest of the work; the
other parity cases fit in one pass.  Each case here needs a second pass
and is compared whole, byte for byte, with the oracle:
- the NVFP4 tile kernel over 80000 logical workgroups (H=64, D=64);
- its pages read back through a block table of 4000 columns per request
  (320000 wave items for the NVFP4 read-back);
- the indexer read-back and the gather through a table of 268800 entries;
- the gather's wide-table kernel over about 300000 page runs (B = 1,
  pages at a stride of 144 bytes).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from test_gpu_reader import assert_same16

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import paged_quantized_kv_amd as pkv

DEV = "cuda:0"
MAX_WORKGROUPS = 65536
WAVES_PER_WORKGROUP = 4


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bf16(bits):
    return dev(bits.view(np.int16)).view(torch.bfloat16)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def widen(table, width, fill):
    out = np.full((table.shape[0], width), fill, np.int32)
    out[:, :table.shape[1]] = table
    return out


def fp4_read_back(f, cache, bt, seed):
    """Read f's pages back through block table bt; compare with the oracle."""
    H, D, B, T = f.num_heads, f.head_size, f.block_size, f.num_tokens
    g = workloads.rng(seed)
    k_init = workloads.random_bytes(g, (T + 2, H * D * 2)).view(np.uint16) & 0xBFFF
    v_init = workloads.random_bytes(g, (T + 2, H * D * 2)).view(np.uint16) & 0xBFFF
    k_ref, v_ref = k_init.copy(), v_init.copy()
    oracle.gather_kv_fp4_dequant(cache, k_ref[:T], v_ref[:T], bt, f.cu_seq_lens, H, D, B,
                                 f.layout, f.k_scale, f.v_scale)
    c = dev(cache)
    ko, vo = dev(k_init.view(np.int16)), dev(v_init.view(np.int16))
    pkv.pkv_gather_kv_fp4_dequant(c[:, 0], c[:, 1], ko.view(torch.bfloat16)[:T].view(T, H, D),
                                  vo.view(torch.bfloat16)[:T].view(T, H, D), dev(bt),
                                  dev(f.cu_seq_lens),
                                  torch.tensor([f.k_scale], dtype=torch.float32, device=DEV),
                                  torch.tensor([f.v_scale], dtype=torch.float32, device=DEV),
                                  block_size=B, layout=f.layout)
    # dropped tokens leave random page bytes, whose NaN block scales read back
    # as NaN with unspecified sign and payload
    assert_same16(host(ko).view(np.uint16), k_ref, "bf16")
    assert_same16(host(vo).view(np.uint16), v_ref, "bf16")


def test_nvfp4_store_in_several_passes_and_direct_read_back():
    H, D, B = 64, 64, 16
    f = workloads.paged_fp4(3201, [1000] * 40, H=H, D=D, B=B)
    T = f.num_tokens
    items = -(-T // 16) * 2 * H                       # (16-token tile, side, head) per wave
    assert items // WAVES_PER_WORKGROUP > MAX_WORKGROUPS
    print(f"\n[case] NVFP4 store, {T} tokens H={H} D={D}: {items} wave items", flush=True)
    cache_ref = f.cache_init.copy()
    oracle.store_kv_fp4(f.key_bits, f.value_bits, cache_ref, f.slot_mapping, H, D, B, f.layout,
                        f.k_scale, f.v_scale)
    c = dev(f.cache_init)
    k4s = torch.tensor([f.k_scale], dtype=torch.float32, device=DEV)
    v4s = torch.tensor([f.v_scale], dtype=torch.float32, device=DEV)
    pkv.pkv_store_kv_fp4(bf16(f.key_bits).view(T, H, D), bf16(f.value_bits).view(T, H, D),
                         c[:, 0], c[:, 1], dev(f.slot_mapping), k4s, v4s, block_size=B,
                         layout=f.layout)
    np.testing.assert_array_equal(host(c), cache_ref)
    # page sides of 36 KB: the read-back's direct kernel; 2 x 40 x 4000 wave items
    bt = widen(f.block_table, 4000, f.num_blocks + 5)
    assert 2 * bt.size > MAX_WORKGROUPS * WAVES_PER_WORKGROUP
    print(f"[case] NVFP4 read-back (direct kernel), {bt.size} table entries", flush=True)
    fp4_read_back(f, cache_ref, bt, 3202)


def test_nvfp4_staged_read_back_through_a_wide_table():
    f = workloads.paged_fp4(3207, [1000, 999, 1, 1000], H=8, D=128, B=16)
    cache = f.cache_init.copy()
    oracle.store_kv_fp4(f.key_bits, f.value_bits, cache, f.slot_mapping, 8, 128, 16, f.layout,
                        f.k_scale, f.v_scale)
    bt = widen(f.block_table, 40000, -1)              # page sides of 9 KB: the staged kernel
    assert 2 * bt.size > MAX_WORKGROUPS * WAVES_PER_WORKGROUP
    print(f"\n[case] NVFP4 read-back (staged kernel), {bt.size} table entries", flush=True)
    fp4_read_back(f, cache, bt, 3208)


def test_indexer_read_back_and_gather_through_a_wide_table():
    w = workloads.small_indexer(3203, [1000] * 63 + [517], width=4200)
    T, B, D = w.num_tokens, w.block_size, w.head_dim
    assert w.block_table.size > MAX_WORKGROUPS * WAVES_PER_WORKGROUP
    print(f"\n[case] indexer read-back and gather, {w.block_table.size} table entries",
          flush=True)
    cache = w.cache_init.copy()
    oracle.store_indexer_k_fp8(w.k_bits, w.slot_mapping, cache, B, D)
    g = workloads.rng(3204)
    out0 = workloads.random_bytes(g, (T + 3, 2 * D)).view(np.uint16) & 0xBFFF
    ref = out0.copy()
    oracle.gather_indexer_k_dequant(cache, ref[:T], w.block_table, w.cu_seq_lens, B, D)
    out = dev(out0.view(np.int16))
    cd, bt, cu = dev(cache), dev(w.block_table), dev(w.cu_seq_lens)
    pkv.pkv_gather_indexer_k_dequant(cd, out.view(torch.bfloat16)[:T], bt, cu, block_size=B)
    np.testing.assert_array_equal(host(out).view(np.uint16), ref)

    ref_f, ref_s = w.k_fp8_init.copy(), w.k_scale_init.copy()
    oracle.gather_indexer_k_fp8(cache, ref_f, ref_s, w.block_table, w.cu_seq_lens, B, D)
    kf, ks = dev(w.k_fp8_init), dev(w.k_scale_init)
    pkv.pkv_gather_indexer_k_fp8(cd, kf, ks, bt, cu, block_size=B)
    np.testing.assert_array_equal(host(kf), ref_f)
    np.testing.assert_array_equal(host(ks), ref_s)


def test_gather_wide_table_kernel_over_many_runs():
    lens = list(workloads.rng(3205).integers(2500, 3500, size=100))
    w = workloads.small_indexer(3206, lens, block_size=1, width=7000)
    runs = w.num_tokens                                # one token per page
    assert runs > MAX_WORKGROUPS * WAVES_PER_WORKGROUP
    assert w.block_table.size > 2 * (runs + len(lens))  # the wide-table kernel
    print(f"\n[case] gather, {runs} page runs of one token", flush=True)
    # one-token pages of 132 bytes, at a stride of 144 (a multiple of 16)
    cache = workloads.random_bytes(workloads.rng(3209), (w.num_blocks, 144))
    oracle.store_indexer_k_fp8(w.k_bits, w.slot_mapping, cache, 1, w.head_dim)
    ref_f, ref_s = w.k_fp8_init.copy(), w.k_scale_init.copy()
    oracle.gather_indexer_k_fp8(cache, ref_f, ref_s, w.block_table, w.cu_seq_lens, 1,
                                w.head_dim)
    kf, ks = dev(w.k_fp8_init), dev(w.k_scale_init)
    pkv.pkv_gather_indexer_k_fp8(dev(cache), kf, ks, dev(w.block_table), dev(w.cu_seq_lens),
                                 block_size=1)
    np.testing.assert_array_equal(host(kf), ref_f)
    np.testing.assert_array_equal(host(ks), ref_s)
