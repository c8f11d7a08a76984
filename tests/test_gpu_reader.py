"""GPU parity of the reader side: the dequantising gathers of the indexer K
cache and of the NVFP4 K/V pages, called through the C ABI (via the Python
binding), against the CPU oracle on the same seeded inputs.

Outputs are compared bit for bit over whole buffers, including padding
columns and guard rows that must stay untouched.  Pages the stores never
wrote (random sentinel bytes, read through dropped slots or random tables)
may hold NaN codes or scales; there both sides must give NaN, whatever its
bits.  The device rounding to bf16 / fp16 is swept over every binary32.
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
TORCH_DT = {"bf16": torch.bfloat16, "f16": torch.float16}


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def half_dev(bits, shape, dtype):
    return dev(bits.view(np.int16)).view(TORCH_DT[dtype]).view(*shape)


def host16(t):
    torch.cuda.synchronize()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def banner(name):
    print(f"\n[case] {name}", flush=True)


def is_nan16(bits, dtype):
    bits = bits.astype(np.uint32)
    if dtype == "bf16":
        return ((bits & 0x7F80) == 0x7F80) & ((bits & 0x7F) != 0)
    return ((bits & 0x7C00) == 0x7C00) & ((bits & 0x3FF) != 0)


def assert_same16(got, ref, dtype):
    """Bit-exact, except that a NaN on the oracle's side needs only a NaN."""
    nan_ref = is_nan16(ref, dtype)
    np.testing.assert_array_equal(is_nan16(got, dtype), nan_ref)
    np.testing.assert_array_equal(np.where(nan_ref, 0, got), np.where(nan_ref, 0, ref))


# ------------------------------------------------------------- indexer K
def run_dequant(cache_np, bt, cu, B, D, T, dtype, pad=0, guard=3, seed=0):
    rows = T + guard
    init = np.random.default_rng(seed).integers(0, 1 << 16, size=(rows, D + pad),
                                                dtype=np.uint16)
    init &= 0xBFFF  # keep sentinels finite-looking; any bits are fine
    ref = init.copy()
    oracle.gather_indexer_k_dequant(cache_np, ref[:T], bt, cu, B, D, dtype=dtype)
    out = dev(init.view(np.int16)).view(TORCH_DT[dtype])
    pkv.pkv_gather_indexer_k_dequant(dev(cache_np), out[:T, :D] if pad else out[:T], dev(bt),
                                     dev(cu), block_size=B)
    assert_same16(host16(out), ref, dtype)


@pytest.mark.parametrize("name", ["c1", "c3", "c4"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_indexer_dequant_configs(name, dtype):
    w = {"c1": workloads.c1_tiny_gather, "c3": workloads.c3_long_ragged,
         "c4": workloads.c4_roundtrip}[name]()
    banner(f"indexer dequant {w.name} {dtype}")
    cache = w.cache_init.copy()
    oracle.store_indexer_k_fp8(w.k_bits, w.slot_mapping, cache, w.block_size, w.head_dim)
    run_dequant(cache, w.block_table, w.cu_seq_lens, w.block_size, w.head_dim,
                int(w.cu_seq_lens[-1]), dtype)


def test_indexer_dequant_prefill_256x1000_full():
    w = workloads.c2_prefill_256x1000()
    banner(f"indexer dequant {w.name}")
    cache = w.cache_init.copy()
    oracle.store_indexer_k_fp8(w.k_bits, w.slot_mapping, cache, w.block_size, w.head_dim)
    run_dequant(cache, w.block_table, w.cu_seq_lens, w.block_size, w.head_dim,
                int(w.cu_seq_lens[-1]), "bf16")


@pytest.mark.parametrize("lens,B,D,pad", [
    ([1], 64, 128, 0), ([65, 1, 130, 64], 64, 128, 8), ([33, 17], 12, 16, 0),
    ([300, 7], 48, 1024, 16), ([5, 0, 9], 4, 64, 0), ([129], 128, 256, 0),
])
def test_indexer_dequant_ragged_shapes(lens, B, D, pad):
    banner(f"indexer dequant lens={lens} B={B} D={D} pad={pad}")
    w = workloads.small_indexer(sum(lens) + B + D, lens, block_size=B, head_dim=D)
    cache = w.cache_init.copy()
    oracle.store_indexer_k_fp8(w.k_bits, w.slot_mapping, cache, B, D)
    run_dequant(cache, w.block_table, w.cu_seq_lens, B, D, int(w.cu_seq_lens[-1]), "bf16",
                pad=pad)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_indexer_dequant_random_pages(dtype):
    """Pages of random bytes: every code (NaN codes included) times scales of
    every exponent, subnormal and infinite ones included."""
    banner(f"indexer dequant random pages {dtype}")
    B, D, nb = 16, 128, 40
    rng = np.random.default_rng(11)
    cache = rng.integers(0, 256, size=(nb, B * (D + 4)), dtype=np.uint8)
    lens = [B * 10, 37, B * 20 - 3]
    maxb = 20
    bt = rng.integers(0, nb, size=(3, maxb)).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    run_dequant(cache, bt, cu, B, D, int(cu[-1]), dtype)


def test_indexer_dequant_skip_rules_and_offsets():
    banner("indexer dequant skip rules")
    w = workloads.small_indexer(9, [70, 20, 64], block_size=32, head_dim=128)
    cache = w.cache_init.copy()
    oracle.store_indexer_k_fp8(w.k_bits, w.slot_mapping, cache, 32, 128)
    bt = w.block_table.copy()
    bt[0, 1] = -1                    # invalid page id: skipped
    bt[2, 0] = w.num_blocks + 5      # past the cache: skipped
    cu = w.cu_seq_lens.copy() + 3    # cu[0] need not be 0
    T = int(cu[-1]) - 10             # the last rows fall outside the output: skipped
    run_dequant(cache, bt, cu, 32, 128, T, "bf16")


# ------------------------------------------------------------- NVFP4 K/V
def run_fp4_readback(f, cache_np, bt, cu, dtype="bf16", pad=0, guard=2, k_scale=None,
                     v_scale=None, layout=None):
    H, D, B = f.num_heads, f.head_size, f.block_size
    layout = f.layout if layout is None else layout
    ks = f.k_scale if k_scale is None else k_scale
    vs = f.v_scale if v_scale is None else v_scale
    T = int(cu[-1])
    rows = T + guard
    rng = np.random.default_rng(3)
    k_init = rng.integers(0, 1 << 16, size=(rows, H * D + pad), dtype=np.uint16) & 0xBFFF
    v_init = rng.integers(0, 1 << 16, size=(rows, H * D + pad), dtype=np.uint16) & 0xBFFF
    k_ref, v_ref = k_init.copy(), v_init.copy()
    oracle.gather_kv_fp4_dequant(cache_np, k_ref[:T], v_ref[:T], bt, cu, H, D, B, layout, ks,
                                 vs, dtype=dtype)
    ko = dev(k_init.view(np.int16)).view(TORCH_DT[dtype])
    vo = dev(v_init.view(np.int16)).view(TORCH_DT[dtype])
    c = dev(cache_np)
    kview = ko[:T, :H * D].view(T, H, D) if not pad else ko[:T].as_strided((T, H, D), (H * D + pad, D, 1))
    vview = vo[:T, :H * D].view(T, H, D) if not pad else vo[:T].as_strided((T, H, D), (H * D + pad, D, 1))
    pkv.pkv_gather_kv_fp4_dequant(c[:, 0], c[:, 1], kview, vview, dev(bt), dev(cu),
                                  torch.tensor([ks], dtype=torch.float32, device=DEV),
                                  torch.tensor([vs], dtype=torch.float32, device=DEV),
                                  block_size=B, layout=layout)
    assert_same16(host16(ko), k_ref, dtype)
    assert_same16(host16(vo), v_ref, dtype)


@pytest.mark.parametrize("lens,H,D,B,layout,dtype,pad", [
    ([37, 5, 16, 100, 1, 64], 2, 128, 16, 0, "bf16", 0),
    ([37, 5, 16, 100, 1, 64], 2, 128, 16, 1, "bf16", 8),
    ([40, 24, 3, 96], 3, 64, 8, 0, "f16", 0),
    ([200, 17, 33], 1, 256, 32, 1, "bf16", 0),
    ([48, 48, 13, 50], 4, 128, 12, 0, "f16", 16),
    ([300], 2, 512, 4, 0, "bf16", 0),
    # page sides of 4608 and 16128 bytes (8 and 16 staged loads per lane),
    # and two shapes the staged kernel leaves to the direct one: a side of
    # 18432 bytes (over 16 KB) and head_size 192
    ([33, 64], 4, 128, 16, 0, "bf16", 8),
    ([70, 16, 5], 14, 128, 16, 1, "f16", 0),
    ([70, 16, 5], 16, 128, 16, 0, "bf16", 0),
    ([20, 9], 3, 192, 8, 1, "bf16", 0),
])
def test_fp4_readback_paged(lens, H, D, B, layout, dtype, pad):
    banner(f"nvfp4 readback lens={lens} H={H} D={D} B={B} layout={layout} {dtype} pad={pad}")
    f = workloads.paged_fp4(sum(lens) * 3 + H + D, lens, H=H, D=D, B=B, layout=layout,
                            drop_frac=0.05, dtype=dtype)
    cache = f.cache_init.copy()
    oracle.store_kv_fp4(f.key_bits, f.value_bits, cache, f.slot_mapping, H, D, B, layout,
                        f.k_scale, f.v_scale, dtype=dtype)
    run_fp4_readback(f, cache, f.block_table, f.cu_seq_lens, dtype=dtype, pad=pad)


@pytest.mark.parametrize("dtype,layout", [("bf16", 0), ("f16", 1)])
def test_fp4_readback_random_pages(dtype, layout):
    """Random page bytes: every E2M1 code and every E4M3 scale byte (NaN
    ones included), random tables, tensor scales far from 1."""
    banner(f"nvfp4 readback random pages {dtype} layout={layout}")
    f = workloads.paged_fp4(77, [50, 3, 64], H=2, D=128, B=16, layout=layout, dtype=dtype)
    rng = np.random.default_rng(21)
    cache = rng.integers(0, 256, size=f.cache_init.shape, dtype=np.uint8)
    nb = cache.shape[0]
    bt = rng.integers(-1, nb + 1, size=f.block_table.shape).astype(np.int32)
    for ks, vs in ((f.k_scale, f.v_scale), (2.0 ** 100, 2.0 ** -120), (3e38, 1e-45)):
        run_fp4_readback(f, cache, bt, f.cu_seq_lens, dtype=dtype, k_scale=ks, v_scale=vs)


def test_fp4_readback_prefill_sampled():
    """The 256 x 1000-token prefill batch (H=8, D=128, B=16): stored by the
    GPU store, read back on the GPU, and compared with the oracle's read-back
    of the same pages for a sample of requests."""
    f = workloads.prefill_fp4()
    banner(f"nvfp4 readback {f.name} sampled")
    T, H, D = f.num_tokens, f.num_heads, f.head_size
    c = dev(f.cache_init)
    k_scale = torch.tensor([f.k_scale], dtype=torch.float32, device=DEV)
    v_scale = torch.tensor([f.v_scale], dtype=torch.float32, device=DEV)
    pkv.pkv_store_kv_fp4(half_dev(f.key_bits, (T, H, D), "bf16"),
                         half_dev(f.value_bits, (T, H, D), "bf16"), c[:, 0], c[:, 1],
                         dev(f.slot_mapping), k_scale, v_scale, block_size=f.block_size,
                         layout=f.layout)
    ko = torch.empty((T, H, D), dtype=torch.bfloat16, device=DEV)
    vo = torch.empty((T, H, D), dtype=torch.bfloat16, device=DEV)
    pkv.pkv_gather_kv_fp4_dequant(c[:, 0], c[:, 1], ko, vo, dev(f.block_table),
                                  dev(f.cu_seq_lens), k_scale, v_scale,
                                  block_size=f.block_size, layout=f.layout)
    cache_np = c.cpu().numpy()
    got_k, got_v = host16(ko).reshape(T, -1), host16(vo).reshape(T, -1)
    cu = f.cu_seq_lens
    for r in (0, 1, 127, 255):
        n = int(cu[r + 1] - cu[r])
        kr = np.zeros((n, H * D), np.uint16)
        vr = np.zeros((n, H * D), np.uint16)
        oracle.gather_kv_fp4_dequant(cache_np, kr, vr, f.block_table[r:r + 1].copy(),
                                     np.array([0, n], np.int32), H, D, f.block_size, f.layout,
                                     f.k_scale, f.v_scale)
        np.testing.assert_array_equal(got_k[cu[r]:cu[r] + n], kr)
        np.testing.assert_array_equal(got_v[cu[r]:cu[r] + n], vr)


# ------------------------------------------------------------- rounding sweep
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_device_narrow_exhaustive(dtype):
    """Every binary32 pattern through the device rounding, against the oracle."""
    banner(f"narrow sweep {dtype}")
    from concurrent.futures import ThreadPoolExecutor
    fn = oracle.f32_to_bf16 if dtype == "bf16" else oracle.f32_to_f16
    pool = ThreadPoolExecutor(16)
    chunk = 1 << 26
    for start in range(0, 1 << 32, chunk):
        b = torch.arange(start, start + chunk, dtype=torch.int64, device=DEV)
        b = torch.where(b >= 2 ** 31, b - 2 ** 32, b).to(torch.int32)
        out = torch.empty(chunk, dtype=TORCH_DT[dtype], device=DEV)
        pkv.pkv_diag_narrow(b.view(torch.float32), out)
        got = host16(out)
        x = np.arange(start, start + chunk, dtype=np.uint64).astype(np.uint32).view(np.float32)
        ref = np.empty(chunk, np.uint16)
        parts = np.array_split(np.arange(chunk), 16)

        def work(ix):
            ref[ix] = fn(x[ix])
        list(pool.map(work, parts))
        nan_ref = is_nan16(ref, dtype)
        ok = (got == ref) | (nan_ref & is_nan16(got, dtype))
        bad = np.nonzero(~ok)[0]
        assert bad.size == 0, (f"{bad.size} mismatches, first x=0x{start + bad[0]:08x} "
                               f"got {got[bad[0]]:#06x} want {ref[bad[0]]:#06x}")
    pool.shutdown()
