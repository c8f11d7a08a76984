"""The C ABI from C++ without PyTorch: tests/c_client/pkv_hip_client.cpp
allocates with hipMalloc, creates its own HIP stream, runs the fp8 store and
the gather of what it stored through libpkv, and writes the results back;
they must equal the oracle's bytes (the round-trip workload: 16 x 512 tokens
into 256 pages, 5% of the slots -1)."""
import subprocess

import numpy as np
import pytest

import oracle
import workloads
from test_abi import build_hip_client

pytestmark = pytest.mark.gpu


def test_hip_client_store_then_gather(tmp_path):
    print("\n[case] C++ HIP client: fp8 store + gather, round-trip workload", flush=True)
    exe = build_hip_client(tmp_path)
    w = workloads.c4_roundtrip()
    T, D, B = w.slot_mapping.shape[0], w.head_dim, w.block_size
    nb, stride = w.cache_init.shape
    R, maxb = w.block_table.shape
    rows = int(w.cu_seq_lens[-1]) + 3
    kf0, ks0 = w.k_fp8_init[:rows], w.k_scale_init[:rows]
    inp, out = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(np.array([T, D, B, nb, stride, R, maxb], np.int64).tobytes())
        for a in (w.k_bits, w.slot_mapping, w.cache_init, w.block_table, w.cu_seq_lens, kf0, ks0):
            f.write(np.ascontiguousarray(a).tobytes())
    r = subprocess.run([str(exe), str(inp), str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "hip client ok" in r.stdout, (r.returncode, r.stderr[-2000:])
    got = np.fromfile(out, np.uint8)
    cache_ref = w.cache_init.copy()
    oracle.store_indexer_k_fp8(w.k_bits, w.slot_mapping, cache_ref, B, D)
    kf_ref, ks_ref = kf0.copy(), ks0.copy()
    oracle.gather_indexer_k_fp8(cache_ref, kf_ref, ks_ref, w.block_table, w.cu_seq_lens, B, D)
    n_c, n_f = cache_ref.size, kf_ref.size
    np.testing.assert_array_equal(got[:n_c].reshape(cache_ref.shape), cache_ref)
    np.testing.assert_array_equal(got[n_c:n_c + n_f].reshape(kf_ref.shape), kf_ref)
    np.testing.assert_array_equal(got[n_c + n_f:].reshape(ks_ref.shape), ks_ref)
