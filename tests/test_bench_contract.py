"""CPU checks of bench.py's contract: the algorithmic bytes it divides by are
the per-unit figures of the path (gather 2(D+4) B per token plus metadata,
fp8 store 2D + 8 + D + 4, NVFP4 store K and V bf16 + slot + 2 H (D/2 + D/16)
per token, the read-backs, decode attention 2 D KVH per context token plus
queries, outputs and metadata), it refuses more than one GPU, and it ignores
a counter summary taken on other kernel source."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_step_bytes_of_the_prefill_batch():
    # 256 requests x 1000 tokens, D = 128, 16 table columns; NVFP4 H = 8, D = 128
    b = bench.algorithmic_bytes(T=256000, D=128, H4=8, D4=128, R=256, maxb=16)
    assert b["gather_indexer_k_fp8"] == 256000 * 264 + 256 * 16 * 4 + 257 * 4 == 67601412
    assert b["store_indexer_k_fp8"] == 256000 * 396 == 101376000
    assert b["store_kv_fp4"] == 256000 * (4096 + 8 + 2 * 8 * 72) + 8 == 1345536008


def test_reader_bytes_of_the_prefill_batch():
    # NVFP4 read-back tables: 256 requests x 63 pages of 16 tokens
    r = bench.reader_bytes(T=256000, D=128, H4=8, D4=128, R=256, maxb=16, R4=256, maxb4=63)
    assert r["gather_indexer_k_dequant"] == 256000 * 388 + 256 * 16 * 4 + 257 * 4 == 99345412
    assert r["gather_kv_fp4_dequant"] == (256000 * 2 * 8 * (64 + 8 + 256) + 256 * 63 * 4
                                         + 257 * 4 + 8) == 1343553548


class _Case:
    def __init__(self, S, H, D, KVH, B, lens):
        self.query = np.zeros((S, H, D), np.uint16)
        self.key_cache = np.zeros((1, KVH, D // 16, B, 16), np.uint8)
        self.context_lens = np.asarray(lens, np.int32)
        self.num_kv_heads = KVH


def test_decode_attention_bytes():
    c = _Case(S=3, H=8, D=128, KVH=2, B=16, lens=[1, 16, 17])
    # K and V codes of 34 context tokens for 2 kv heads, bf16 q and out, 1+1+2 table
    # entries, 3 context lengths
    assert bench.decode_attention_bytes(c) == 34 * 2 * 2 * 128 + 2 * 3 * 8 * 128 * 2 + 4 * 4 + 12


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_counter_summary_needs_the_current_kernel_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    path = tmp_path / "gather_indexer_k_fp8_prefill_256x1000_pmc.md"
    assert bench.measured_traffic("gather_indexer_k_fp8") is None          # no summary
    path.write_text("traffic_bytes_per_launch: 12345\nsource_sha256: 0123456789abcdef\n")
    assert bench.measured_traffic("gather_indexer_k_fp8") is None          # other source
    path.write_text("traffic_bytes_per_launch: 12345\nsource_sha256: "
                    f"{bench.source_hash('gather_indexer_k_fp8')}\n")
    assert bench.measured_traffic("gather_indexer_k_fp8") == 12345.0


def test_cpu_baseline_split_writes_what_one_thread_writes():
    """The CPU baseline runs the oracle's functions over disjoint token or
    request ranges on several threads; the bytes they write must be exactly
    those of one call over everything."""
    from concurrent.futures import ThreadPoolExecutor

    import workloads
    w = workloads.c4_roundtrip()
    f = workloads.c5_nvfp4_store(0)
    one = bench.oracle_ops(w, f, 600)
    many = bench.oracle_ops(w, f, 600)
    with ThreadPoolExecutor(3) as pool:
        for name in ("store_indexer_k_fp8", "store_kv_fp4", "gather_indexer_k_fp8"):
            fn1, n, *_, out1 = one[name]
            fn3, _, *_, out3 = many[name]
            bench.run_split(pool, fn1, n, 1)
            bench.run_split(pool, fn3, n, 3)
            for a, b in zip(out1, out3):
                np.testing.assert_array_equal(a, b)
    # the ops wrote something: the stores changed their caches, the gather its rows
    assert (one["store_indexer_k_fp8"][-1][0] != w.cache_init).any()
    assert (one["store_kv_fp4"][-1][0] != f.cache_init).any()
    assert (one["gather_indexer_k_fp8"][-1][0] != w.k_fp8_init).any()
