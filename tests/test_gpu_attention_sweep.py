"""Seeded random sweep of decode attention against the binary64 oracle,
within the per-element bound attention_bound derives from the kernels'
arithmetic.

Each case draws the query group size (1-16), the number of KV heads (1-8,
including counts that leave a workgroup's four KV-head slots partly empty),
the page size, the partition size (64-2048), the number of sequences, their
context lengths (0, 1, page-edge lengths and up to 2000 tokens), invalid
page ids inside a context, NaN codes in the unused slots of a context's last
page and a max_context_len above the longest context; every other case runs
the allocation-free entry point.  The targeted cases in test_gpu_attention
list these one at a time.
"""
import numpy as np
import pytest
import torch

import workloads
from test_gpu_attention import check, reference, run

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import paged_quantized_kv_amd as pkv

DEV = "cuda:0"
N_CASES = 64


def draw(i):
    g = workloads.rng(7000 + i)
    G = int(g.choice([1, 2, 4, 8, 8, 16]))
    KVH = int(g.choice([1, 2, 3, 4, 5, 8]))
    if G * KVH > 64:
        KVH = max(1, 64 // G)
    B = int(g.choice([16, 16, 32, 48, 64]))
    P = int(g.choice([64, 128, 256, 256, 512, 1024, 2048]))
    S = int(g.integers(1, 11))
    lens = [int(x) for x in g.integers(0, 2001, size=S)]
    lens[int(g.integers(0, S))] = int(g.choice([0, 1, B, B + 1, 2 * B - 1]))
    extra = int(g.choice([0, 0, 1, 300]))
    noalloc = i % 2 == 1
    return g, dict(G=G, KVH=KVH, B=B, P=P, lens=lens, extra=extra, noalloc=noalloc)


@pytest.mark.parametrize("i", range(N_CASES))
def test_attention_random_case(i):
    g, c = draw(i)
    print(f"\n[case] attention sweep {i}: {c}", flush=True)
    H, KVH, B, lens = c["G"] * c["KVH"], c["KVH"], c["B"], c["lens"]
    case = workloads.paged_attention_case(7500 + i, len(lens), H, KVH, block_size=B, lens=lens)
    nb = case.key_cache.shape[0]
    for s, n in enumerate(lens):
        pages = -(-n // B)
        if pages > 1 and g.random() < 0.3:              # an invalid id inside the context
            case.block_tables[s, int(g.integers(0, pages))] = int(g.choice([-1, nb, nb + 9]))
        if n % B and g.random() < 0.5:                  # NaN codes past the context's end
            p = case.block_tables[s, n // B]
            if 0 <= p < nb:
                case.key_cache[p, :, :, n % B:, :] = 0x7F
                case.value_cache[p, :, :, n % B:] = 0xFF
    maxc = max(lens + [0]) + c["extra"]
    ref, b = reference(case)
    if c["noalloc"]:
        S, _, D = case.query.shape
        q = torch.from_numpy(np.ascontiguousarray(case.query.view(np.int16))).to(DEV)
        out = torch.full((S, H, D), float("nan"), dtype=torch.bfloat16, device=DEV)
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
        pkv.pkv_paged_attention_decode_noalloc(
            out, q.view(torch.bfloat16), dev(case.key_cache), dev(case.value_cache), KVH,
            case.scale, dev(case.block_tables), dev(case.context_lens), B, maxc, case.k_scale,
            case.v_scale, partition_size=c["P"])
        torch.cuda.synchronize()
        got = out.to(torch.float64).cpu().numpy()
    else:
        got = run(case, c["P"], max_context_len=maxc)
    worst = check(got, ref, b)
    print(f"max err / bound = {worst:.3g}", flush=True)
