#!/usr/bin/env python3
"""Throughput of the paged quantized KV-cache data path on one MI355X.

One step is one pass of the whole path over the prefill batch of 256 requests
x 1000 tokens (the shape of the serving benchmark on the vLLM integration PR
"[Deepseek-V3.2][Kernel] Integrate cuda indexer k cache gather"):

  1. pkv_store_indexer_k_fp8  bf16 K [256000, 128] -> fp8 codes + binary32 scales
                              into 4096 indexer pages of 64 tokens (slots from
                              each request's block-table row);
  2. pkv_store_kv_fp4         bf16 K and V [256000, 8, 128] -> NVFP4 pages of 16
                              tokens, [K_data|K_scale|V_data|V_scale], HND;
  3. pkv_gather_indexer_k_fp8 the indexer pages back into contiguous k_fp8
                              [256000, 128] and k_scale [256000, 4], driven by
                              block_table and cu_seq_lens.

Inputs are synthetic (seeded N(0,1), 1% outlier rows x20 for the indexer K)
and resident in HBM before timing starts.  The indexer buffers rotate over
eight sets (~1.1 GB) and the gather of step i reads the pages that the fp8
store wrote at step i - 4, so no kernel reads data that the 256 MB Infinity
Cache still holds from a recent write; the NVFP4 store reads 1 GB of K/V and
writes 0.3 GB of pages per step.

Timing, in this order:
  - pre-roll: steps launched for a fixed 0.5 s of wall clock (reported as
    `preroll`, not counted in `warmup`), so that the clocks have left their
    idle state before anything is timed;
  - `warmup` untimed steps, then `steps` steps timed by wall clock between
    two synchronizations, nothing recorded between the launches:
    `ms_per_step` and `value`;
  - each of the step's three kernels alone: 32 launches back to back (the
    same rotating buffers) between one pair of HIP events on the launch
    stream, three times, median of the three averages: `kernels`; each run
    starts behind three NVFP4 stores (0.7 ms of GPU work), so all 32
    launches are queued before the first event and the GPU never waits for
    the host between the events;
    `roofline` describes the kernel with the longest duration;
  - reported workloads (not part of `value`): the gather on 8 long ragged
    requests, the 16 x 512-token store-then-gather round trip, the NVFP4
    store of [4096, 8, 128] K and V, and the step's NVFP4 store with its
    tokens stored to pages in order, each timed the same way;
  - the reader side (pkv_gather_indexer_k_dequant, pkv_gather_kv_fp4_dequant)
    on the prefill batch and the decode consumer (pkv_paged_attention_decode,
    200 requests with Llama-3.1-70B attention shapes) on its own batch, timed
    the same way;
  - `d2d_copy_same_bytes`: the runtime's device-to-device copy moving the
    step's bytes (a reference point for a plain stream of that size);
  - `cpu_baseline`: the CPU oracle on bounded samples of the same batch, per
    op, on one thread and on every thread used (the oracle's functions called
    on disjoint token or request ranges), median of 5 after one warm-up.
Events are created with hipEventDisableSystemFence (recording one then does
not write back and invalidate the caches).  Printed: one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, 8 TB/s
METRIC = "gather/store HBM GB/s and % of MI355X peak; Mtokens/s at 256×1000 tok"
PREROLL_S = 0.5                 # fixed pre-roll of step launches before any timing
B2B_LAUNCHES = 32               # back-to-back launches per timed kernel run
B2B_RUNS = 3                    # runs per kernel; the median is reported

CSRC = os.path.join(ROOT, "paged_quantized_kv_amd", "csrc")
BUILD_PY = os.path.join(ROOT, "paged_quantized_kv_amd", "build.py")
KERNEL_SOURCES = {
    "store_indexer_k_fp8": ["store_indexer_k_fp8.hip", "device_common.h"],
    "store_kv_fp4": ["store_kv_fp4.hip", "device_common.h"],
    "gather_indexer_k_fp8": ["gather_indexer_k_fp8.hip", "device_common.h"],
    "gather_indexer_k_dequant": ["gather_dequant.hip", "device_common.h"],
    "gather_kv_fp4_dequant": ["gather_dequant.hip", "device_common.h"],
    "paged_attention_decode": ["paged_attention.hip", "device_common.h"],
}
PROFILES = os.path.join(ROOT, "profiles")


def source_hash(kernel: str) -> str:
    """Hash of the kernel's source files and of the build script (its flags
    shape the compiled kernel too)."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    with open(BUILD_PY, "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str = "prefill_256x1000"):
    """HBM bytes per launch from a committed counter summary, if it was taken
    on the current source of the kernel; else None."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_t = re.search(r"^traffic_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    m_h = re.search(r"^source_sha256:\s*([0-9a-f]+)", text, re.M)
    if not m_t or not m_h or m_h.group(1) != source_hash(kernel):
        return None
    return float(m_t.group(1))


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--sets", type=int, default=8, help="rotating indexer buffer sets")
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip the CPU oracle timing (profiling runs)")
    p.add_argument("--no-extras", action="store_true",
                   help="time only the step and its three kernels (short profiling runs)")
    p.add_argument("--calibration-copy", action="store_true",
                   help="run a plain fp32 copy-like kernel (torch.neg) over 16 MiB to 1 GiB "
                        "before the timed steps, for scaling hardware byte counters")
    return p.parse_args()


class HipTimingEvents:
    """HIP events for timing only, on the HIP runtime torch has loaded.

    They are created with hipEventDisableSystemFence: recording one then does
    not write back and invalidate the caches, which torch's events do and
    which would add that cost to the kernels around it."""

    DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence

    def __init__(self, lead=None):
        # lead(): enqueues at least half a millisecond of GPU work; run before
        # the first event of a back-to-back run, it keeps the GPU busy while
        # the host enqueues the timed launches (a Python launch call takes
        # about 10 us, as long as the shorter kernels), so that every timed
        # launch is already queued when the GPU reaches it
        self.lead = lead
        import ctypes
        paths = set()
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    paths.add(os.path.realpath(line.split()[-1]))
        if len(paths) != 1:
            raise RuntimeError(f"expected one loaded HIP runtime, found {sorted(paths)}")
        self._ct = ctypes
        hip = ctypes.CDLL(paths.pop())
        P = ctypes.c_void_p
        hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(P), ctypes.c_uint]
        hip.hipEventRecord.argtypes = [P, P]
        hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), P, P]
        hip.hipEventDestroy.argtypes = [P]
        for fn in ("hipEventCreateWithFlags", "hipEventRecord", "hipEventElapsedTime",
                   "hipEventDestroy"):
            getattr(hip, fn).restype = ctypes.c_int
        self._hip = hip

    def _ok(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def create(self):
        ev = self._ct.c_void_p()
        self._ok(self._hip.hipEventCreateWithFlags(self._ct.byref(ev), self.DISABLE_SYSTEM_FENCE),
                 "hipEventCreateWithFlags")
        return ev

    def record(self, ev, stream_handle):
        self._ok(self._hip.hipEventRecord(ev, self._ct.c_void_p(stream_handle)), "hipEventRecord")

    def elapsed_ms(self, a, b):
        ms = self._ct.c_float()
        self._ok(self._hip.hipEventElapsedTime(self._ct.byref(ms), a, b), "hipEventElapsedTime")
        return ms.value

    def destroy(self, *events):
        for ev in events:
            self._hip.hipEventDestroy(ev)


def time_back_to_back(torch, timing, stream, launch, n=B2B_LAUNCHES, runs=B2B_RUNS, warm=4):
    """Median over `runs` of the average duration (ms) of `n` launches issued
    back to back between one pair of events on the launch stream; launch(i)
    enqueues the i-th launch.  Each run starts behind timing.lead (when set),
    so the GPU never waits for the host between the two events."""
    e0, e1 = timing.create(), timing.create()
    for i in range(warm):
        launch(i)
    torch.cuda.synchronize()
    avgs = []
    for r in range(runs):
        if timing.lead is not None:
            timing.lead()
        timing.record(e0, stream)
        for i in range(n):
            launch(r * n + i)
        timing.record(e1, stream)
        torch.cuda.synchronize()
        avgs.append(timing.elapsed_ms(e0, e1) / n)
    timing.destroy(e0, e1)
    return statistics.median(avgs)


def rate(nbytes, tokens, ms):
    """GB/s, fraction of the HBM peak and Mtokens/s of `nbytes` and `tokens` per `ms`."""
    gbps = nbytes / (ms * 1e-3) / 1e9
    out = {"us": round(ms * 1e3, 2), "alg_bytes": int(nbytes), "GBps": round(gbps, 1),
           "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
    if tokens is not None:
        out["mtokens_per_s"] = round(tokens / (ms * 1e-3) / 1e6, 1)
    return out


def algorithmic_bytes(T, D, H4, D4, R, maxb):
    """Bytes each op must move at minimum (read + write), per step."""
    store8 = T * (2 * D + 8 + D + 4)                     # bf16 K + slot -> codes + scale
    gather = T * 2 * (D + 4) + R * maxb * 4 + (R + 1) * 4  # pages -> k_fp8/k_scale, metadata
    fp4 = T * (2 * H4 * D4 * 2 + 8 + 2 * H4 * (D4 // 2 + D4 // 16)) + 8  # K,V,slot -> pages
    return {"store_indexer_k_fp8": store8, "store_kv_fp4": fp4, "gather_indexer_k_fp8": gather}


def gather_bytes(w):
    """Gather bytes of an indexer workload: 2 (D + 4) per token, table and cu_seq_lens."""
    R, maxb = w.block_table.shape
    return w.num_tokens * 2 * (w.head_dim + 4) + R * maxb * 4 + (R + 1) * 4


def store8_bytes(w):
    """fp8 store bytes of an indexer workload: bf16 row and slot read, codes and
    scale written for every token with a slot."""
    T, D = w.k_bits.shape[0], w.head_dim
    kept = int((w.slot_mapping >= 0).sum())
    return T * (2 * D + 8) + kept * (D + 4)


def fp4_bytes(f):
    """NVFP4 store bytes: K and V 16-bit rows and the slot read for every token,
    code and scale bytes of both sides written for every token with a slot."""
    T = f.slot_mapping.shape[0]
    H, D = f.num_heads, f.head_size
    kept = int((f.slot_mapping >= 0).sum())
    return T * (2 * H * D * 2 + 8) + kept * 2 * H * (D // 2 + D // 16) + 8


def reader_bytes(T, D, H4, D4, R, maxb, R4, maxb4):
    """Bytes the reader-side gathers must move (read + write) over the batch."""
    idx = T * (D + 4 + 2 * D) + R * maxb * 4 + (R + 1) * 4      # codes + scale -> bf16 row
    fp4 = T * 2 * H4 * (D4 // 2 + D4 // 16 + 2 * D4) + R4 * maxb4 * 4 + (R4 + 1) * 4 + 8
    return {"gather_indexer_k_dequant": idx, "gather_kv_fp4_dequant": fp4}


def decode_attention_bytes(c):
    """Bytes decode attention must move: the K and V codes of every token of
    every sequence (each read once), the bf16 queries and outputs, and the
    block-table entries and context lengths it reads."""
    S, H, D = c.query.shape
    B = c.key_cache.shape[3]
    L = c.context_lens.astype(int)
    kv = int(L.sum()) * c.num_kv_heads * 2 * D
    return kv + 2 * (S * H * D * 2) + 4 * int(sum(-(-n // B) for n in L)) + 4 * S


def rotation_sets(footprint_bytes, cap=8):
    """Buffer sets to rotate so that the sets together exceed twice the 256 MB
    Infinity Cache (at least one)."""
    return max(1, min(cap, -(-(512 << 20) // max(1, footprint_bytes))))


# ---------------------------------------------------------------- CPU baseline
def cpu_threads():
    """Threads the CPU baseline uses: every host CPU, but no more than the
    OMP_NUM_THREADS share when that is set."""
    n = os.cpu_count() or 1
    share = os.environ.get("OMP_NUM_THREADS")
    if share and share.isdigit() and int(share) > 0:
        n = min(n, int(share))
    return n


def _split(n, parts):
    step = -(-n // parts)
    return [(a, min(a + step, n)) for a in range(0, n, step)]


def oracle_ops(w, f, fp4_sample_tokens):
    """The oracle's three step ops on fresh copies of the sentinel buffers,
    each as (fn(a, b), n, algorithmic bytes, tokens, sample, outputs): fn runs
    the oracle on items [a, b) (tokens for the stores, requests for the
    gather), so calls on disjoint ranges write disjoint bytes."""
    import oracle
    T, D = w.num_tokens, w.head_dim
    R = w.block_table.shape[0]
    n4 = min(fp4_sample_tokens, f.slot_mapping.shape[0])
    H4, D4 = f.num_heads, f.head_size
    cache8 = w.cache_init.copy()
    kf, ks = w.k_fp8_init.copy(), w.k_scale_init.copy()
    c4 = f.cache_init.copy()

    def store8(a, b):
        oracle.store_indexer_k_fp8(w.k_bits[a:b], w.slot_mapping[a:b], cache8, w.block_size, D,
                                   dtype=w.dtype)

    def gather(a, b):
        oracle.gather_indexer_k_fp8(cache8, kf, ks, w.block_table[a:b], w.cu_seq_lens[a:b + 1],
                                    w.block_size, D)

    def store4(a, b):
        oracle.store_kv_fp4(f.key_bits[a:b], f.value_bits[a:b], c4, f.slot_mapping[a:b],
                            f.num_heads, f.head_size, f.block_size, f.layout, f.k_scale,
                            f.v_scale, dtype=f.dtype)

    return {
        "store_indexer_k_fp8": (store8, T, T * (2 * D + 8 + D + 4), T,
                                f"{T} tokens (the whole batch)", [cache8]),
        "store_kv_fp4": (store4, n4, n4 * (2 * H4 * D4 * 2 + 8 + 2 * H4 * (D4 // 2 + D4 // 16)),
                         n4, f"the first {n4} tokens", [c4]),
        "gather_indexer_k_fp8": (gather, R, T * 2 * (D + 4) + w.block_table.size * 4 + (R + 1) * 4,
                                 T, f"{T} tokens (the whole batch)", [kf, ks]),
    }


def run_split(pool, fn, n, threads):
    """fn over [0, n) on one thread, or over `threads` disjoint ranges on the pool."""
    if threads == 1:
        fn(0, n)
    else:
        list(pool.map(lambda ab: fn(*ab), _split(n, threads)))


def cpu_baseline(w, f, fp4_sample_tokens=16000, runs=5):
    """The oracle as it stands, on bounded samples of the prefill batch: every
    op on one thread and on `cpu_threads()` threads (disjoint token ranges for
    the stores, disjoint request ranges for the gather; ctypes releases the
    GIL during each call), median of `runs` after one warm-up."""
    from concurrent.futures import ThreadPoolExecutor
    nthreads = cpu_threads()
    pool = ThreadPoolExecutor(nthreads)
    ops = oracle_ops(w, f, fp4_sample_tokens)

    def timed(fn, n, threads):
        t0 = time.perf_counter()
        run_split(pool, fn, n, threads)
        return time.perf_counter() - t0

    out = {}
    total_bytes = 0
    total_s_all = 0.0
    for name, (fn, n, nbytes, tokens, what, _) in ops.items():
        entry = {"sample": what}
        for label, threads in (("one_thread", 1), ("all_threads", nthreads)):
            timed(fn, n, threads)                        # warm-up
            s = statistics.median(timed(fn, n, threads) for _ in range(runs))
            entry[label] = {"threads": threads, "seconds": round(s, 4),
                            "GBps": round(nbytes / s / 1e9, 4),
                            "mtokens_per_s": round(tokens / s / 1e6, 4)}
        out[name] = entry
        total_bytes += nbytes
        total_s_all += entry["all_threads"]["seconds"]
    pool.shutdown()
    n4 = ops["store_kv_fp4"][1]
    return {"value": round(total_bytes / total_s_all / 1e9, 4), "unit": "GB/s",
            "cores": nthreads, "host_cpu_count": os.cpu_count(), "kind": "oracle",
            "sample": (f"per op: fp8 store and gather on the whole 256 x 1000-token batch, "
                       f"NVFP4 store on its first {n4} tokens; value = the samples' algorithmic "
                       f"bytes over their summed times on {nthreads} threads (median of "
                       f"{runs} after one warm-up)"),
            "ops": out}


# ---------------------------------------------------------------- reported workloads
def time_reported(torch, np, pkv, workloads, timing, stream):
    """The long ragged gather, the round-trip store + gather and the NVFP4
    store of [4096, 8, 128] K and V, each launched back to back."""
    def to(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")

    out = {}
    # long ragged gather: 8 requests of up to 32768 tokens, 8192 pages
    w = workloads.c3_long_ragged()
    T = w.num_tokens
    nsets = rotation_sets(w.cache_init.nbytes + T * (w.head_dim + 4))
    sets = [(to(w.cache_init), to(w.k_fp8_init), to(w.k_scale_init)) for _ in range(nsets)]
    bt, cu = to(w.block_table), to(w.cu_seq_lens)

    def g3(i):
        c, kf, ks = sets[i % nsets]
        pkv.pkv_gather_indexer_k_fp8(c, kf, ks, bt, cu, block_size=w.block_size)

    ms = time_back_to_back(torch, timing, stream, g3)
    out["gather_long_ragged"] = dict(rate(gather_bytes(w), T, ms), rotating_sets=nsets,
                                     workload=f"8 requests, {T} tokens (lengths "
                                              f"{[int(x) for x in w.lens]}), B=64, D=128, "
                                              "8192 pages")
    del sets
    # round trip: fp8 store of 8192 tokens (5% slots -1), then gather of 16 x 512
    w = workloads.c4_roundtrip()
    T = w.num_tokens
    nsets = rotation_sets(w.cache_init.nbytes + T * (w.head_dim * 3 + 4))
    sets = [(to(w.k_bits.view(np.int16)).view(torch.bfloat16), to(w.cache_init),
             to(w.k_fp8_init), to(w.k_scale_init)) for _ in range(nsets)]
    slots, bt, cu = to(w.slot_mapping), to(w.block_table), to(w.cu_seq_lens)

    def s4(i):
        k, c, _, _ = sets[i % nsets]
        pkv.pkv_store_indexer_k_fp8(k, slots, c, block_size=w.block_size)

    def g4(i):
        _, c, kf, ks = sets[i % nsets]
        pkv.pkv_gather_indexer_k_fp8(c, kf, ks, bt, cu, block_size=w.block_size)

    ms_s, ms_g = (time_back_to_back(torch, timing, stream, fn) for fn in (s4, g4))
    out["roundtrip_store"] = dict(rate(store8_bytes(w), T, ms_s), rotating_sets=nsets,
                                  workload="16 x 512 tokens, D=128, 256 pages of 64, "
                                           "5% of slots -1")
    out["roundtrip_gather"] = dict(rate(gather_bytes(w), T, ms_g), rotating_sets=nsets,
                                   workload="the same pages gathered back, 16 x 512 tokens")
    del sets
    # NVFP4 store: K and V [4096, 8, 128], B=16, 512 pages, 5% of slots -1, HND
    f = workloads.c5_nvfp4_store(0)
    T = f.slot_mapping.shape[0]
    nsets = rotation_sets(f.cache_init.nbytes + f.key_bits.nbytes * 2)
    shape = (T, f.num_heads, f.head_size)
    sets = [(to(f.key_bits.view(np.int16)).view(torch.bfloat16).view(shape),
             to(f.value_bits.view(np.int16)).view(torch.bfloat16).view(shape),
             to(f.cache_init)) for _ in range(nsets)]
    sl = to(f.slot_mapping)
    ksc = torch.tensor([f.k_scale], dtype=torch.float32, device="cuda")
    vsc = torch.tensor([f.v_scale], dtype=torch.float32, device="cuda")

    def s5(i):
        k, v, c = sets[i % nsets]
        pkv.pkv_store_kv_fp4(k, v, c[:, 0], c[:, 1], sl, ksc, vsc, block_size=f.block_size,
                             layout=0)

    ms = time_back_to_back(torch, timing, stream, s5)
    out["nvfp4_store_4096x8x128"] = dict(rate(fp4_bytes(f), T, ms), rotating_sets=nsets,
                                         workload="K and V [4096, 8, 128] bf16, B=16, 512 pages, "
                                                  "HND, 5% of slots -1")
    del sets
    return out


def time_reader(torch, np, pkv, timing, stream, sets, w, f, bt, cu, c4, k4s, v4s):
    """Durations (ms) of the two reader-side gathers over the batch, each
    launched back to back.  The indexer read-back cycles over the rotating
    page sets; the NVFP4 read-back reads the pages of the step's NVFP4 store
    (0.3 GB, larger than the Infinity Cache)."""
    T = w.num_tokens
    H4, D4 = f.num_heads, f.head_size
    outs = [torch.empty((T, w.head_dim), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    ko = torch.empty((T, H4, D4), dtype=torch.bfloat16, device="cuda")
    vo = torch.empty((T, H4, D4), dtype=torch.bfloat16, device="cuda")
    bt4, cu4 = (torch.from_numpy(a).to("cuda") for a in (f.block_table, f.cu_seq_lens))

    def idx(i):
        pkv.pkv_gather_indexer_k_dequant(sets[i % len(sets)]["cache"], outs[i % 2], bt, cu,
                                         block_size=w.block_size)

    def fp4(i):
        pkv.pkv_gather_kv_fp4_dequant(c4[:, 0], c4[:, 1], ko, vo, bt4, cu4, k4s, v4s,
                                      block_size=f.block_size, layout=f.layout)

    ms = {"gather_indexer_k_dequant": time_back_to_back(torch, timing, stream, idx),
          "gather_kv_fp4_dequant": time_back_to_back(torch, timing, stream, fp4)}
    del outs, ko, vo
    return ms


def time_decode_attention(torch, np, pkv, workloads, timing, stream):
    """Duration of one pkv_paged_attention_decode call (partition and reduce
    kernels) over the decode batch, launched back to back.  Its 0.5 GB of K/V
    codes is larger than the Infinity Cache, so each call reads them from
    HBM."""
    c = workloads.decode_batch()
    S, H, D = c.query.shape
    B = c.key_cache.shape[3]
    maxc = int(c.context_lens.max())

    def to(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")

    q = to(c.query.view(np.int16)).view(torch.bfloat16)
    kc, vc, bt, cl = to(c.key_cache), to(c.value_cache), to(c.block_tables), to(c.context_lens)
    out = torch.empty((S, H, D), dtype=torch.bfloat16, device="cuda")
    P = workloads.DECODE_PARTITION
    ws = pkv.paged_attention_workspace(S, H, maxc, P, device="cuda")

    def call(i):
        pkv.pkv_paged_attention_decode(out, *ws, q, kc, vc, c.num_kv_heads, c.scale, bt, cl, B,
                                       maxc, c.k_scale, c.v_scale, partition_size=P)

    ms = time_back_to_back(torch, timing, stream, call)
    nbytes = decode_attention_bytes(c)
    res = rate(nbytes, None, ms)
    res.update({"seqs_per_s": round(S / (ms * 1e-3), 1),
                "context_tokens": int(c.context_lens.sum()),
                "workload": "decode step: 200 req, H=64, KVH=8, D=128, B=16, contexts "
                            f"U[128, 2560], fp8 E4M3 K/V, partitions of {P}",
                "traffic": measured_traffic("paged_attention_decode", "decode_200req")})
    return res


def time_d2d_copy(torch, timing, stream, nbytes):
    """A device-to-device copy (torch's copy_, the runtime's copy kernel)
    moving nbytes in all (half read, half written), over rotating buffers."""
    half = (nbytes // 2 + 255) // 256 * 256
    nsets = rotation_sets(2 * half, cap=4)
    bufs = [(torch.empty(half, dtype=torch.uint8, device="cuda"),
             torch.empty(half, dtype=torch.uint8, device="cuda")) for _ in range(nsets)]

    def cp(i):
        src, dst = bufs[i % nsets]
        dst.copy_(src)

    ms = time_back_to_back(torch, timing, stream, cp, n=12)
    del bufs
    res = rate(2 * half, None, ms)
    res["what"] = ("torch copy_ of half the step's algorithmic bytes (read + write = the step's "
                   "bytes), back to back over rotating buffers")
    return res


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (the path has "
              "no cross-GPU step; requests and tokens shard across GPUs with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_quantized_kv_amd as pkv
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    t_gen = time.perf_counter()
    w = workloads.c2_prefill_256x1000()
    f = workloads.prefill_fp4()
    T, D = w.num_tokens, w.head_dim
    R, maxb = w.block_table.shape
    H4, D4 = f.num_heads, f.head_size
    assert f.num_tokens == T
    t_gen = time.perf_counter() - t_gen

    def to(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    sets = []
    for _ in range(args.sets):
        sets.append({
            "k": to(w.k_bits.view(np.int16)).view(torch.bfloat16),
            "slot": to(w.slot_mapping),
            "cache": to(w.cache_init),
            "kf": to(w.k_fp8_init[:T]),
            "ks": to(w.k_scale_init[:T]),
        })
    bt, cu = to(w.block_table), to(w.cu_seq_lens)
    key = to(f.key_bits.view(np.int16)).view(torch.bfloat16).view(T, H4, D4)
    val = to(f.value_bits.view(np.int16)).view(torch.bfloat16).view(T, H4, D4)
    slot4 = to(f.slot_mapping)
    c4 = to(f.cache_init)
    k4s = torch.tensor([f.k_scale], dtype=torch.float32, device=dev)
    v4s = torch.tensor([f.v_scale], dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    names = ["store_indexer_k_fp8", "store_kv_fp4", "gather_indexer_k_fp8"]
    lag = len(sets) // 2  # the gather reads pages stored `lag` steps earlier

    stream = torch.cuda.current_stream().cuda_stream  # every launch goes to this stream

    def store8(i):
        s = sets[i % len(sets)]
        pkv.pkv_store_indexer_k_fp8(s["k"], s["slot"], s["cache"], block_size=w.block_size)

    def store4(i):
        pkv.pkv_store_kv_fp4(key, val, c4[:, 0], c4[:, 1], slot4, k4s, v4s,
                             block_size=f.block_size, layout=f.layout)

    def gather(i):
        sg = sets[(i - lag) % len(sets)]
        pkv.pkv_gather_indexer_k_fp8(sg["cache"], sg["kf"], sg["ks"], bt, cu,
                                     block_size=w.block_size)

    def step(i):
        store8(i)
        store4(i)
        gather(i)

    def lead():
        for k in range(3):          # about 0.7 ms of NVFP4 stores
            store4(k)

    timing = HipTimingEvents(lead=lead)

    if args.calibration_copy:
        # 16 MiB, 64 MiB, 256 MiB and 1 GiB of fp32 each way, three times each:
        # the counters' scale factors at several sizes
        for mib in (16, 64, 256, 1024):
            src = torch.randn(mib << 18, device=dev)
            dst = torch.empty_like(src)
            for _ in range(3):
                torch.neg(src, out=dst)
            torch.cuda.synchronize()
            del src, dst

    # fixed pre-roll: steps for PREROLL_S of wall clock, in batches of 20
    t_pre = time.perf_counter()
    preroll_steps = 0
    while time.perf_counter() - t_pre < PREROLL_S:
        for _ in range(20):
            step(preroll_steps)
            preroll_steps += 1
        torch.cuda.synchronize()
    preroll_s = time.perf_counter() - t_pre

    for i in range(args.warmup):
        step(preroll_steps + i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    base = preroll_steps + args.warmup
    for i in range(args.steps):
        step(base + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # each step kernel alone, back to back
    per_kernel_ms = {"store_indexer_k_fp8": time_back_to_back(torch, timing, stream, store8),
                     "store_kv_fp4": time_back_to_back(torch, timing, stream, store4),
                     "gather_indexer_k_fp8": time_back_to_back(torch, timing, stream, gather)}

    alg = algorithmic_bytes(T, D, H4, D4, R, maxb)
    step_bytes = sum(alg.values())
    kernels = {n: dict(rate(alg[n], T, per_kernel_ms[n]), traffic=measured_traffic(n))
               for n in names}
    dom = max(names, key=lambda n: per_kernel_ms[n])
    roofline = {"kernel": dom, "bound": "hbm", "achieved": kernels[dom]["GBps"],
                "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(kernels[dom]["GBps"] / HBM_PEAK_GBPS, 4),
                "traffic": measured_traffic(dom), "alg_bytes_per_launch": alg[dom]}
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "preroll": {"steps": preroll_steps, "seconds": round(preroll_s, 3),
                    "what": f"steps launched for a fixed {PREROLL_S} s before the warmup, "
                            "so that no timed launch meets the clocks' idle state"},
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "prefill batch 256 req x 1000 tok: indexer K fp8 store + gather "
                        "(D=128, B=64, 4096 pages) and NVFP4 K/V store (H=8, D=128, B=16, HND)",
            "tokens": T,
            "requests": R,
            "parallelism": "single GPU",
        },
        "frac_hbm_peak": round(value / HBM_PEAK_GBPS, 4),
        "mtokens_per_s": round(T / (ms_per_step * 1e-3) / 1e6, 2),
        "kernels": kernels,
        "kernel_timing": (f"each kernel alone: {B2B_LAUNCHES} launches back to back between "
                          f"one pair of HIP events, median of {B2B_RUNS} runs; each run starts "
                          "behind 0.7 ms of queued GPU work (three NVFP4 stores), so the GPU "
                          "never waits for the host between the events"),
        "roofline": roofline,
        "input_gen_s": round(t_gen, 1),
    }
    if not args.no_extras:
        out["reported"] = time_reported(torch, np, pkv, workloads, timing, stream)
        reader = time_reader(torch, np, pkv, timing, stream, sets, w, f, bt, cu, c4, k4s, v4s)
        R4, maxb4 = f.block_table.shape
        rb = reader_bytes(T, D, H4, D4, R, maxb, R4, maxb4)
        out["reader_side"] = {n: dict(rate(rb[n], T, reader[n]), traffic=measured_traffic(n))
                              for n in rb}
        out["decode_attention"] = time_decode_attention(torch, np, pkv, workloads, timing,
                                                        stream)
        # the step's NVFP4 store with the same tokens stored to pages in order
        # (slot = token index): the kernel when the placement of the pages does
        # not scatter its writes (after the reader side, which reads the pages
        # the workload's slots wrote)
        assert c4.shape[0] * f.block_size >= T
        slot_in_order = torch.arange(T, dtype=torch.int64, device=dev)

        def store4_in_order(i):
            pkv.pkv_store_kv_fp4(key, val, c4[:, 0], c4[:, 1], slot_in_order, k4s, v4s,
                                 block_size=f.block_size, layout=f.layout)

        # 64 untimed launches first: after the stores into shuffled pages the
        # in-order store takes about 40 launches to settle (trace: 245-288 us
        # at first, then 212-218 us)
        ms = time_back_to_back(torch, timing, stream, store4_in_order, warm=64)
        out["reported"]["nvfp4_store_256x1000_pages_in_order"] = dict(
            rate(alg["store_kv_fp4"], T, ms),
            workload="the step's NVFP4 store (256 x 1000 tokens, H=8, D=128, B=16, HND) with "
                     "slot = token index instead of the workload's shuffled pages")
        del sets
        torch.cuda.empty_cache()
        out["d2d_copy_same_bytes"] = time_d2d_copy(torch, timing, stream, step_bytes)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, f)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
