"""Seeded random sweep over the configuration space of the store / gather /
read-back entry points, every case compared byte for byte with the oracle.

The targeted parity cases list shapes one by one; here block size, head
size, heads, layout, source and output types, row and page strides (padded
or not, 8- or 16-byte aligned page sides), request lengths, table width,
invalid table entries and dropped slots are drawn together from one seed per
case, so that combinations no list names are exercised too.  Each indexer
case runs the fp8 store, the gather of what it stored and the read-back into
bf16 or fp16; each NVFP4 case runs the store and, for page-filling slots,
the read-back.  Whole caches and whole outputs (guard rows, padding bytes
and columns included) are compared.
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
N_INDEXER = 256
N_FP4 = 256
TORCH_DT = {"bf16": torch.bfloat16, "f16": torch.float16}


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def half_dev(bits, dtype):
    return dev(bits.view(np.int16)).view(TORCH_DT[dtype])


def indexer_case(i):
    g = workloads.rng(4000 + i)
    B = int(g.choice([1, 2, 3, 4, 5, 8, 12, 16, 24, 32, 48, 64, 96, 128]))
    D = int(g.choice([16, 32, 48, 64, 112, 128, 128, 128, 144, 256, 384, 512, 1024]))
    R = int(g.integers(1, 13))
    lens = [int(x) for x in g.integers(0, 4 * B + 40, size=R)]
    lens[int(g.integers(0, R))] = int(g.choice([0, 1, B, B + 1, 3 * B - 1]))
    need = [-(-n // B) for n in lens]
    width = max(need + [1]) + int(g.integers(0, 4))
    num_blocks = sum(need) + int(g.integers(1, 6))
    page = B * (D + 4)
    stride = -(-page // 16) * 16 + 16 * int(g.choice([0, 0, 1, 3]))
    src_dtype = str(g.choice(["bf16", "f16"]))
    out_dtype = str(g.choice(["bf16", "f16"]))
    k_pad = 8 * int(g.choice([0, 0, 1, 3]))
    out_pad = 8 * int(g.choice([0, 0, 2]))
    cu0 = int(g.choice([0, 0, 5]))
    return dict(B=B, D=D, lens=lens, width=width, num_blocks=num_blocks, stride=stride,
                src_dtype=src_dtype, out_dtype=out_dtype, k_pad=k_pad, out_pad=out_pad,
                cu0=cu0, g=g)


@pytest.mark.parametrize("i", range(N_INDEXER))
def test_indexer_store_gather_read_back(i):
    c = indexer_case(i)
    g, B, D, lens = c.pop("g"), c["B"], c["D"], c["lens"]
    print(f"\n[case] indexer sweep {i}: {c}", flush=True)
    R, nb, stride = len(lens), c["num_blocks"], c["stride"]
    perm = g.permutation(nb).astype(np.int32)
    table = np.empty((R, c["width"]), np.int32)
    pos = 0
    for r, n in enumerate(lens):
        k = -(-n // B)
        table[r, :k] = perm[pos:pos + k]
        pos += k
        rest = c["width"] - k           # columns past the request: any id, also invalid
        table[r, k:] = g.choice([-1, nb, nb + 7, int(perm[0])], size=rest)
    bad = g.random(table.shape) < 0.03  # a few invalid ids inside requests too
    table[bad] = g.choice([-1, nb + 3], size=int(bad.sum()))
    cu = (c["cu0"] + np.concatenate([[0], np.cumsum(lens)])).astype(np.int32)
    T = int(cu[-1])                     # output rows (rows below cu[0] stay untouched)
    # token i of request r: slot page*B + i%B with page = table[r][i/B], or -1
    # where that entry is not a valid page id; then a fraction dropped
    r_of = np.repeat(np.arange(R), lens)
    i_of = np.concatenate([np.arange(n) for n in lens]).astype(np.int64) if sum(lens) else \
        np.zeros(0, np.int64)
    pg = table[r_of, i_of // B].astype(np.int64)
    slots = np.where((pg >= 0) & (pg < nb), pg * B + i_of % B, -1).astype(np.int64)
    slots[g.random(slots.shape) < float(g.choice([0.0, 0.1]))] = -1
    Tk = slots.shape[0]
    x = workloads.normal_f32(g, (Tk, D + c["k_pad"]))
    x[g.random(Tk) < 0.05] *= np.float32(100.0)
    k_bits = workloads.half_bits(x, c["src_dtype"])
    cache0 = workloads.random_bytes(g, (nb, stride))

    # fp8 store of every token (rows of k padded by k_pad elements)
    ref = cache0.copy()
    oracle.store_indexer_k_fp8(k_bits, slots, ref, B, D, dtype=c["src_dtype"])
    cache = dev(cache0)
    k_dev = half_dev(k_bits, c["src_dtype"])[:, :D]
    pkv.pkv_store_indexer_k_fp8(k_dev, dev(slots), cache, block_size=B)
    np.testing.assert_array_equal(host(cache), ref)

    # gather of what was stored (guard rows after the last one)
    kf0 = workloads.random_bytes(g, (T + 3, D))
    ks0 = workloads.random_bytes(g, (T + 3, 4))
    ref_f, ref_s = kf0.copy(), ks0.copy()
    oracle.gather_indexer_k_fp8(ref, ref_f, ref_s, table, cu, B, D)
    kf, ks = dev(kf0), dev(ks0)
    bt_d, cu_d = dev(table), dev(cu)
    pkv.pkv_gather_indexer_k_fp8(cache, kf, ks, bt_d, cu_d, block_size=B)
    np.testing.assert_array_equal(host(kf), ref_f)
    np.testing.assert_array_equal(host(ks), ref_s)

    # read-back into bf16 / fp16 rows (padded columns untouched)
    od = c["out_dtype"]
    out0 = workloads.random_bytes(g, (T + 3, 2 * (D + c["out_pad"]))).view(np.uint16) & 0xBFFF
    out_ref = out0.copy()
    oracle.gather_indexer_k_dequant(ref, out_ref[:T], table, cu, B, D, dtype=od)
    out = half_dev(out0, od)
    pkv.pkv_gather_indexer_k_dequant(cache, out[:T, :D], bt_d, cu_d, block_size=B)
    assert_same16(host(out.view(torch.int16)).view(np.uint16), out_ref, od)


def fp4_case(i):
    g = workloads.rng(5000 + i)
    H = int(g.integers(1, 17))
    D = int(g.choice([64, 128, 128, 192, 256, 320, 512]))
    B = int(g.choice([4, 8, 12, 16, 16, 20, 32]))
    layout = int(g.integers(0, 2))
    dtype = str(g.choice(["bf16", "f16"]))
    gap = int(g.choice([0, 0, 8, 16]))          # bytes after the two sides of a page
    paged = bool(g.random() < 0.6)
    return dict(H=H, D=D, B=B, layout=layout, dtype=dtype, gap=gap, paged=paged, g=g)


@pytest.mark.parametrize("i", range(N_FP4))
def test_nvfp4_store_and_read_back(i):
    c = fp4_case(i)
    g, H, D, B, layout, gap = c.pop("g"), c["H"], c["D"], c["B"], c["layout"], c["gap"]
    if c["paged"]:
        lens = [int(x) for x in g.integers(1, 3 * B + 20, size=int(g.integers(1, 6)))]
        f = workloads.paged_fp4(6000 + i, lens, H=H, D=D, B=B, layout=layout,
                                drop_frac=float(g.choice([0.0, 0.05])), dtype=c["dtype"])
    else:
        T = int(g.integers(1, 600))
        f = workloads.small_fp4(6000 + i, T, H=H, D=D, B=B, layout=layout, dtype=c["dtype"])
    print(f"\n[case] nvfp4 sweep {i}: {c} T={f.num_tokens}", flush=True)
    nb, side = f.cache_init.shape[0], f.cache_init.shape[2]
    stride = 2 * side + gap
    # pages at `stride` bytes, the buffer offset by 8 when the gap is 8 (sides
    # 8-byte aligned only); padding bytes must stay as they were
    off = 8 if gap == 8 else 0
    flat = workloads.random_bytes(g, (off + nb * stride,))
    pages = flat[off:].reshape(nb, stride)
    pages[:, :2 * side] = f.cache_init.reshape(nb, 2 * side)
    ref = f.cache_init.copy()
    oracle.store_kv_fp4(f.key_bits, f.value_bits, ref, f.slot_mapping, H, D, B, layout,
                        f.k_scale, f.v_scale, dtype=c["dtype"])
    ref_flat = flat.copy()
    ref_flat[off:].reshape(nb, stride)[:, :2 * side] = ref.reshape(nb, 2 * side)
    buf = dev(flat)
    view = buf[off:].view(nb, stride)
    T = f.num_tokens
    shape = (T, H, D)
    k4s = torch.tensor([f.k_scale], dtype=torch.float32, device=DEV)
    v4s = torch.tensor([f.v_scale], dtype=torch.float32, device=DEV)
    pkv.pkv_store_kv_fp4(half_dev(f.key_bits, c["dtype"]).view(shape),
                         half_dev(f.value_bits, c["dtype"]).view(shape),
                         view[:, :side], view[:, side:2 * side], dev(f.slot_mapping), k4s, v4s,
                         block_size=B, layout=layout)
    np.testing.assert_array_equal(host(buf), ref_flat)
    if not c["paged"] or gap == 8:
        return                                  # the read-back needs 16-byte aligned sides
    od = str(g.choice(["bf16", "f16"]))
    Tr = int(f.cu_seq_lens[-1])
    k0 = workloads.random_bytes(g, (Tr + 2, 2 * H * D)).view(np.uint16) & 0xBFFF
    v0 = workloads.random_bytes(g, (Tr + 2, 2 * H * D)).view(np.uint16) & 0xBFFF
    k_ref, v_ref = k0.copy(), v0.copy()
    oracle.gather_kv_fp4_dequant(ref, k_ref[:Tr], v_ref[:Tr], f.block_table, f.cu_seq_lens, H,
                                 D, B, layout, f.k_scale, f.v_scale, dtype=od)
    ko, vo = half_dev(k0, od), half_dev(v0, od)
    pkv.pkv_gather_kv_fp4_dequant(view[:, :side], view[:, side:2 * side],
                                  ko[:Tr].view(Tr, H, D), vo[:Tr].view(Tr, H, D),
                                  dev(f.block_table), dev(f.cu_seq_lens), k4s, v4s,
                                  block_size=B, layout=layout)
    assert_same16(host(ko.view(torch.int16)).view(np.uint16), k_ref, od)
    assert_same16(host(vo.view(torch.int16)).view(np.uint16), v_ref, od)
