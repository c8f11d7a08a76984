"""Several host threads drive the library at once, each on its own stream and
buffers: the fp8 store, the gather of what it stored, the NVFP4 store and a
decode-attention call, many times over.  Every thread's results must equal
the oracle's bytes (stores, gather) or the single-threaded result of the same
call (attention), on every round: the host side keeps no shared state that
concurrent calls could corrupt, and launches go to the caller's stream."""
import threading

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import paged_quantized_kv_amd as pkv

DEV = "cuda:0"
THREADS = 4
ROUNDS = 12


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bf16(bits, shape=None):
    t = dev(bits.view(np.int16)).view(torch.bfloat16)
    return t if shape is None else t.view(*shape)


class Job:
    """One thread's inputs, buffers and expected results."""

    def __init__(self, i):
        self.w = workloads.small_indexer(500 + i, [300 + 37 * i, 65, 1, 640], drop_frac=0.05)
        w = self.w
        self.cache_ref = w.cache_init.copy()
        oracle.store_indexer_k_fp8(w.k_bits, w.slot_mapping, self.cache_ref, w.block_size,
                                   w.head_dim)
        self.kf_ref, self.ks_ref = w.k_fp8_init.copy(), w.k_scale_init.copy()
        oracle.gather_indexer_k_fp8(self.cache_ref, self.kf_ref, self.ks_ref, w.block_table,
                                    w.cu_seq_lens, w.block_size, w.head_dim)
        self.f = workloads.small_fp4(600 + i, 96 + 16 * i, H=4, D=128, B=16)
        f = self.f
        self.c4_ref = f.cache_init.copy()
        oracle.store_kv_fp4(f.key_bits, f.value_bits, self.c4_ref, f.slot_mapping, f.num_heads,
                            f.head_size, f.block_size, f.layout, f.k_scale, f.v_scale)
        self.pa = workloads.paged_attention_case(700 + i, 6, 16, 2,
                                                 lens=[1, 200, 513, 64 + i, 0, 1500])
        # device buffers
        self.k, self.slots = bf16(w.k_bits), dev(w.slot_mapping)
        self.cache = dev(w.cache_init)
        self.kf, self.ks = dev(w.k_fp8_init), dev(w.k_scale_init)
        self.bt, self.cu = dev(w.block_table), dev(w.cu_seq_lens)
        T4 = f.slot_mapping.shape[0]
        shape = (T4, f.num_heads, f.head_size)
        self.key, self.val = bf16(f.key_bits, shape), bf16(f.value_bits, shape)
        self.slot4, self.c4 = dev(f.slot_mapping), dev(f.cache_init)
        self.k4s = torch.tensor([f.k_scale], dtype=torch.float32, device=DEV)
        self.v4s = torch.tensor([f.v_scale], dtype=torch.float32, device=DEV)
        c = self.pa
        S, H, D = c.query.shape
        self.maxc = int(c.context_lens.max())
        self.q = bf16(c.query)
        self.kc, self.vc = dev(c.key_cache), dev(c.value_cache)
        self.pbt, self.pcl = dev(c.block_tables), dev(c.context_lens)
        self.out = torch.empty((S, H, D), dtype=torch.bfloat16, device=DEV)
        self.ws = pkv.paged_attention_workspace(S, H, self.maxc, 256, device=DEV)

    def attention(self):
        c = self.pa
        pkv.pkv_paged_attention_decode(self.out, *self.ws, self.q, self.kc, self.vc,
                                       c.num_kv_heads, c.scale, self.pbt, self.pcl,
                                       c.key_cache.shape[3], self.maxc, c.k_scale, c.v_scale,
                                       partition_size=256)

    def round(self):
        """One round on the current stream; the caches start from their
        initial bytes so every round must give the same results."""
        w, f = self.w, self.f
        self.cache.copy_(dev(w.cache_init), non_blocking=False)
        self.c4.copy_(dev(f.cache_init), non_blocking=False)
        pkv.pkv_store_indexer_k_fp8(self.k, self.slots, self.cache, block_size=w.block_size)
        pkv.pkv_gather_indexer_k_fp8(self.cache, self.kf, self.ks, self.bt, self.cu,
                                     block_size=w.block_size)
        pkv.pkv_store_kv_fp4(self.key, self.val, self.c4[:, 0], self.c4[:, 1], self.slot4,
                             self.k4s, self.v4s, block_size=f.block_size, layout=f.layout)
        self.attention()


def test_threads_on_their_own_streams():
    print("\n[case] 4 threads x 12 rounds: store, gather, NVFP4 store, attention", flush=True)
    torch.cuda.set_device(0)
    jobs = [Job(i) for i in range(THREADS)]
    # single-threaded attention results, the reference for the threaded ones
    att_ref = []
    for j in jobs:
        j.attention()
        torch.cuda.synchronize()
        att_ref.append(j.out.clone())
    errors = []
    start = threading.Barrier(THREADS)

    def work(i):
        try:
            torch.cuda.set_device(0)
            j = jobs[i]
            s = torch.cuda.Stream()
            start.wait()
            with torch.cuda.stream(s):
                for r in range(ROUNDS):
                    j.round()
                    s.synchronize()
                    if not (np.array_equal(j.cache.cpu().numpy(), j.cache_ref)
                            and np.array_equal(j.kf.cpu().numpy(), j.kf_ref)
                            and np.array_equal(j.ks.cpu().numpy(), j.ks_ref)
                            and np.array_equal(j.c4.cpu().numpy(), j.c4_ref)
                            and torch.equal(j.out, att_ref[i])):
                        errors.append((i, r))
                        return
        except Exception as e:  # reported below, with the thread that raised it
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=work, args=(i,)) for i in range(THREADS)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=240)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
