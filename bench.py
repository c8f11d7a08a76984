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

After the timed steps, the reader side is timed on the same batch (not part
of `value`): pkv_gather_indexer_k_dequant (indexer pages -> bf16 rows) and
pkv_gather_kv_fp4_dequant (NVFP4 pages -> bf16 K and V rows), reported under
`reader_side`.

Then the decode consumer of fp8 KV pages is timed on its own batch (not
part of `value` either): pkv_paged_attention_decode over one decode step of
200 requests with Llama-3.1-70B attention shapes (64 query heads, 8 KV heads,
head size 128, 16-token pages, contexts uniform in [128, 2560]: 0.5 GB of K/V
codes), reported under `decode_attention`.

Printed: one JSON line.  `value` = algorithmic bytes of one step / measured
step time (GB/s), the wall clock of K steps with nothing between the
launches; the per-kernel durations come from the K steps that follow, with
HIP events recorded on the launch stream around each launch (timing-only
events, without the cache write-back a default event performs), and
`ms_per_step_with_events` is those steps' wall clock; `roofline` describes
the kernel with the longest average duration; `d2d_copy_same_bytes` times a
device-to-device copy moving the step's bytes (the practical ceiling);
`store_kv_fp4_alone` times the NVFP4 store back to back with the
workload's slots and with the same tokens stored to pages in order;
`cpu_baseline` times the CPU oracle on the same batch (one thread).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, 8 TB/s
METRIC = "gather/store HBM GB/s and % of MI355X peak; Mtokens/s at 256×1000 tok"

CSRC = os.path.join(ROOT, "paged_quantized_kv_amd", "csrc")
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
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
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
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--sets", type=int, default=8, help="rotating indexer buffer sets")
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip the CPU oracle timing (profiling runs)")
    p.add_argument("--reader-steps", type=int, default=50,
                   help="timed iterations of the reader-side gathers (0: skip them)")
    p.add_argument("--decode-steps", type=int, default=50,
                   help="timed calls of the paged decode attention (0: skip them)")
    p.add_argument("--calibration-copy", action="store_true",
                   help="run a plain 256 MiB fp32 copy-like kernel (torch.neg) before the "
                        "timed steps, for scaling hardware byte counters")
    return p.parse_args()


class HipTimingEvents:
    """HIP events for timing only, on the HIP runtime torch has loaded.

    They are created with hipEventDisableSystemFence: recording one then does
    not write back and invalidate the caches, which torch's events do and
    which would add that cost to the kernel timed before it and to the one
    after it.  A timed step therefore runs like an untimed one."""

    DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence

    def __init__(self):
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
        self._events = []

    def _ok(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def create(self):
        ev = self._ct.c_void_p()
        self._ok(self._hip.hipEventCreateWithFlags(self._ct.byref(ev), self.DISABLE_SYSTEM_FENCE),
                 "hipEventCreateWithFlags")
        self._events.append(ev)
        return ev

    def record(self, ev, stream_handle):
        self._ok(self._hip.hipEventRecord(ev, self._ct.c_void_p(stream_handle)), "hipEventRecord")

    def elapsed_ms(self, a, b):
        ms = self._ct.c_float()
        self._ok(self._hip.hipEventElapsedTime(self._ct.byref(ms), a, b), "hipEventElapsedTime")
        return ms.value

    def destroy_all(self):
        for ev in self._events:
            self._hip.hipEventDestroy(ev)
        self._events = []


def algorithmic_bytes(T, D, H4, D4, R, maxb):
    """Bytes each op must move at minimum (read + write), per step."""
    store8 = T * (2 * D + 8 + D + 4)                     # bf16 K + slot -> codes + scale
    gather = T * 2 * (D + 4) + R * maxb * 4 + (R + 1) * 4  # pages -> k_fp8/k_scale, metadata
    fp4 = T * (2 * H4 * D4 * 2 + 8 + 2 * H4 * (D4 // 2 + D4 // 16)) + 8  # K,V,slot -> pages
    return {"store_indexer_k_fp8": store8, "store_kv_fp4": fp4, "gather_indexer_k_fp8": gather}


def reader_bytes(T, D, H4, D4, R, maxb, R4, maxb4):
    """Bytes the reader-side gathers must move (read + write) over the batch."""
    idx = T * (D + 4 + 2 * D) + R * maxb * 4 + (R + 1) * 4      # codes + scale -> bf16 row
    fp4 = T * 2 * H4 * (D4 // 2 + D4 // 16 + 2 * D4) + R4 * maxb4 * 4 + (R4 + 1) * 4 + 8
    return {"gather_indexer_k_dequant": idx, "gather_kv_fp4_dequant": fp4}


def cpu_baseline(w, f, step_bytes):
    import numpy as np

    import oracle
    cache = w.cache_init.copy()
    kf, ks = w.k_fp8_init.copy(), w.k_scale_init.copy()
    c4 = f.cache_init.copy()
    t0 = time.perf_counter()
    oracle.store_indexer_k_fp8(w.k_bits, w.slot_mapping, cache, w.block_size, w.head_dim)
    oracle.store_kv_fp4(f.key_bits, f.value_bits, c4, f.slot_mapping, f.num_heads, f.head_size,
                        f.block_size, f.layout, f.k_scale, f.v_scale)
    oracle.gather_indexer_k_fp8(cache, kf, ks, w.block_table, w.cu_seq_lens, w.block_size,
                                w.head_dim)
    dt = time.perf_counter() - t0
    del np
    return {"value": round(step_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "seconds": round(dt, 3),
            "mtokens_per_s": round(w.num_tokens / dt / 1e6, 4),
            "sample": "one full step (256 req x 1000 tok through fp8 store, NVFP4 store and "
                      "gather), plain C oracle, one thread"}


def time_reader(args, pkv, torch, timing, stream, sets, w, f, bt, cu, c4, k4s, v4s):
    """Average durations (ms) of the two reader-side gathers over the batch,
    timed like the step's kernels.  The indexer read-back cycles over the
    rotating page sets; the NVFP4 read-back reads the pages the last step
    stored (0.3 GB, larger than the Infinity Cache)."""
    T = w.num_tokens
    H4, D4 = f.num_heads, f.head_size
    outs = [torch.empty((T, w.head_dim), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    ko = torch.empty((T, H4, D4), dtype=torch.bfloat16, device="cuda")
    vo = torch.empty((T, H4, D4), dtype=torch.bfloat16, device="cuda")
    bt4, cu4 = (torch.from_numpy(a).to("cuda") for a in (f.block_table, f.cu_seq_lens))
    names = ["gather_indexer_k_dequant", "gather_kv_fp4_dequant"]

    def it(i, ev=None):
        s = sets[i % len(sets)]
        if ev is not None:
            timing.record(ev[0], stream)
        pkv.pkv_gather_indexer_k_dequant(s["cache"], outs[i % 2], bt, cu, block_size=w.block_size)
        if ev is not None:
            timing.record(ev[1], stream)
        pkv.pkv_gather_kv_fp4_dequant(c4[:, 0], c4[:, 1], ko, vo, bt4, cu4, k4s, v4s,
                                      block_size=f.block_size, layout=f.layout)
        if ev is not None:
            timing.record(ev[2], stream)

    evs = [[timing.create() for _ in range(3)] for _ in range(args.reader_steps)]
    for i in range(min(args.warmup, 20)):
        it(i)
    torch.cuda.synchronize()
    for i in range(args.reader_steps):
        it(i, evs[i])
    torch.cuda.synchronize()
    ms = {n: sum(timing.elapsed_ms(e[j], e[j + 1]) for e in evs) / args.reader_steps
          for j, n in enumerate(names)}
    del outs, ko, vo
    timing.destroy_all()
    return ms


def time_d2d_copy(torch, timing, stream, nbytes, reps=20):
    """A device-to-device copy (torch's copy_, the runtime's copy kernel)
    moving nbytes in all (half read, half written): the practical ceiling
    the step's kernels are set against."""
    half = (nbytes // 2 + 255) // 256 * 256
    src = torch.empty(half, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = timing.create(), timing.create()
    timing.record(e0, stream)
    for _ in range(reps):
        dst.copy_(src)
    timing.record(e1, stream)
    torch.cuda.synchronize()
    ms = timing.elapsed_ms(e0, e1) / reps
    timing.destroy_all()
    del src, dst
    gbps = 2 * half / (ms * 1e-3) / 1e9
    return {"bytes": 2 * half, "us": round(ms * 1e3, 2), "GBps": round(gbps, 1),
            "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
            "what": "torch copy_ of half the step's algorithmic bytes (read + write = the step's bytes)"}


def decode_attention_bytes(c):
    """Bytes decode attention must move: the K and V codes of every token of
    every sequence (each read once), the bf16 queries and outputs, and the
    block-table entries and context lengths it reads."""
    S, H, D = c.query.shape
    B = c.key_cache.shape[3]
    L = c.context_lens.astype(int)
    kv = int(L.sum()) * c.num_kv_heads * 2 * D
    return kv + 2 * (S * H * D * 2) + 4 * int(sum(-(-n // B) for n in L)) + 4 * S


def time_decode_attention(args, pkv, torch, timing, stream, workloads, np):
    """Average duration (ms) of one pkv_paged_attention_decode call (partition
    and reduce kernels) over the decode batch, timed like the step's kernels.
    Its 0.5 GB of K/V codes is larger than the Infinity Cache, so each call
    reads them from HBM."""
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

    def call():
        pkv.pkv_paged_attention_decode(out, *ws, q, kc, vc, c.num_kv_heads, c.scale, bt, cl, B,
                                       maxc, c.k_scale, c.v_scale, partition_size=P)

    evs = [[timing.create() for _ in range(2)] for _ in range(args.decode_steps)]
    for _ in range(min(args.warmup, 20)):
        call()
    torch.cuda.synchronize()
    for e in evs:
        timing.record(e[0], stream)
        call()
        timing.record(e[1], stream)
    torch.cuda.synchronize()
    ms = sum(timing.elapsed_ms(e[0], e[1]) for e in evs) / args.decode_steps
    timing.destroy_all()
    nbytes = decode_attention_bytes(c)
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"us": round(ms * 1e3, 2), "alg_bytes": nbytes, "GBps": round(gbps, 1),
            "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
            "seqs_per_s": round(S / (ms * 1e-3), 1),
            "context_tokens": int(c.context_lens.sum()),
            "workload": "decode step: 200 req, H=64, KVH=8, D=128, B=16, contexts U[128, 2560], "
                        f"fp8 E4M3 K/V, partitions of {P}",
            "traffic": measured_traffic("paged_attention_decode", "decode_200req")}


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

    timing = HipTimingEvents()
    stream = torch.cuda.current_stream().cuda_stream  # every launch goes to this stream

    def mark(ev, j):
        if ev is not None:
            timing.record(ev[j], stream)

    def step(i, ev=None):
        s = sets[i % len(sets)]
        sg = sets[(i - lag) % len(sets)]
        mark(ev, 0)
        pkv.pkv_store_indexer_k_fp8(s["k"], s["slot"], s["cache"], block_size=w.block_size)
        mark(ev, 1)
        pkv.pkv_store_kv_fp4(key, val, c4[:, 0], c4[:, 1], slot4, k4s, v4s,
                             block_size=f.block_size, layout=f.layout)
        mark(ev, 2)
        pkv.pkv_gather_indexer_k_fp8(sg["cache"], sg["kf"], sg["ks"], bt, cu,
                                     block_size=w.block_size)
        mark(ev, 3)

    if args.calibration_copy:
        src = torch.randn(64 << 20, device=dev)          # 256 MiB fp32
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # Events are created before the warmup so that no host-side pause separates
    # the warmup from the timed steps (an idle GPU lowers its clocks).  The
    # default warmup (~30 ms of steps) runs past the clock transient that the
    # first few dozen launches of the step show, so the timed steps measure the
    # sustained rate.
    # The step's wall clock is taken over K steps with no event between
    # launches (each recorded event is one more packet the command processor
    # waits on, about 2 us per event here); the per-kernel durations come
    # from the next K steps, with events around every launch.
    events = [[timing.create() for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t1 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + args.steps + i, events[i])
    torch.cuda.synchronize()
    wall_events = time.perf_counter() - t1

    per_kernel_ms = {n: 0.0 for n in names}
    for ev in events:
        for j, n in enumerate(names):
            per_kernel_ms[n] += timing.elapsed_ms(ev[j], ev[j + 1])
    per_kernel_ms = {n: v / args.steps for n, v in per_kernel_ms.items()}
    timing.destroy_all()
    ms_per_step = wall * 1e3 / args.steps

    reader = None
    if args.reader_steps > 0:
        reader = time_reader(args, pkv, torch, timing, stream, sets, w, f, bt, cu, c4, k4s, v4s)
        R4, maxb4 = f.block_table.shape
        rb = reader_bytes(T, D, H4, D4, R, maxb, R4, maxb4)
        reader = {n: {"us": round(reader[n] * 1e3, 2), "alg_bytes": rb[n],
                      "GBps": round(rb[n] / (reader[n] * 1e-3) / 1e9, 1),
                      "frac_hbm_peak": round(rb[n] / (reader[n] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                      "mtokens_per_s": round(T / (reader[n] * 1e-3) / 1e6, 1),
                      "traffic": measured_traffic(n)}
                  for n in rb}

    decode = None
    if args.decode_steps > 0:
        decode = time_decode_attention(args, pkv, torch, timing, stream, workloads, np)

    alg = algorithmic_bytes(T, D, H4, D4, R, maxb)
    step_bytes = sum(alg.values())

    # The NVFP4 store alone, back to back, with the workload's slots and with
    # the same tokens' slots in page order (same bytes, pages written in
    # order rather than in the workload's shuffled order).
    def store_alone(slots):
        ev = [timing.create(), timing.create()]
        for _ in range(3):
            pkv.pkv_store_kv_fp4(key, val, c4[:, 0], c4[:, 1], slots, k4s, v4s,
                                 block_size=f.block_size, layout=f.layout)
        torch.cuda.synchronize()
        timing.record(ev[0], stream)
        for _ in range(10):
            pkv.pkv_store_kv_fp4(key, val, c4[:, 0], c4[:, 1], slots, k4s, v4s,
                                 block_size=f.block_size, layout=f.layout)
        timing.record(ev[1], stream)
        torch.cuda.synchronize()
        ms = timing.elapsed_ms(ev[0], ev[1]) / 10
        timing.destroy_all()
        return ms

    slot_in_order = torch.arange(T, dtype=torch.int64, device=dev)
    alone = {"workload_slots": [], "pages_in_order": []}
    for _ in range(3):  # interleaved, medians reported
        alone["workload_slots"].append(store_alone(slot4))
        alone["pages_in_order"].append(store_alone(slot_in_order))
    store_alone_runs = {}
    for name, v in alone.items():
        ms = sorted(v)[len(v) // 2]
        gbps = alg["store_kv_fp4"] / (ms * 1e-3) / 1e9
        store_alone_runs[name] = {"us": round(ms * 1e3, 2), "GBps": round(gbps, 1),
                                  "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
    store_alone_runs["what"] = ("store_kv_fp4 alone, back-to-back launches (median of three "
                                "interleaved runs of 10): the workload's slots, and slots 0..T-1 "
                                "(the same tokens into pages in order)")
    copy_ceiling = time_d2d_copy(torch, timing, stream, step_bytes)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    kernels = {}
    for n in names:
        ms = per_kernel_ms[n]
        gbps = alg[n] / (ms * 1e-3) / 1e9
        kernels[n] = {"us": round(ms * 1e3, 2), "alg_bytes": alg[n], "GBps": round(gbps, 1),
                      "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
                      "mtokens_per_s": round(T / (ms * 1e-3) / 1e6, 1)}
    dom = max(names, key=lambda n: per_kernel_ms[n])
    dom_gbps = kernels[dom]["GBps"]
    roofline = {"kernel": dom, "bound": "hbm", "achieved": dom_gbps, "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(dom_gbps / HBM_PEAK_GBPS, 4),
                "traffic": measured_traffic(dom),
                "alg_bytes_per_launch": alg[dom]}

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
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
        "event_ms_per_step": round(sum(per_kernel_ms.values()), 4),
        "ms_per_step_with_events": round(wall_events * 1e3 / args.steps, 4),
        "kernels": kernels,
        "roofline": roofline,
        "d2d_copy_same_bytes": copy_ceiling,
        "store_kv_fp4_alone": store_alone_runs,
        "input_gen_s": round(t_gen, 1),
    }
    if reader is not None:
        out["reader_side"] = reader
    if decode is not None:
        out["decode_attention"] = decode
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, f, step_bytes)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
