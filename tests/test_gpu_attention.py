"""GPU parity of paged decode attention (pkv_paged_attention_decode) against
the binary64 oracle on the same seeded inputs, within the per-element bound
that attention_bound derives from the kernels' arithmetic.  Rows without a
valid token must be exactly zero; page bytes past a context's end (here NaN
codes) must not reach the result."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle.attention_bound import attention_bound
from test_attention_split import balanced_units

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import paged_quantized_kv_amd as pkv

DEV = "cuda:0"


def banner(name):
    print(f"\n[case] {name}", flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def run(c, partition_size=256, max_context_len=None, stream=None, ws=None):
    S, H, D = c.query.shape
    B = c.key_cache.shape[3]
    maxc = int(c.context_lens.max(initial=0)) if max_context_len is None else max_context_len
    q = dev(c.query.view(np.int16)).view(torch.bfloat16)
    out = torch.full((S, H, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    if ws is None:
        ws = pkv.paged_attention_workspace(S, H, maxc, partition_size, device=DEV)
    pkv.pkv_paged_attention_decode(out, *ws, q, dev(c.key_cache), dev(c.value_cache),
                                   c.num_kv_heads, c.scale, dev(c.block_tables),
                                   dev(c.context_lens), B, maxc, c.k_scale, c.v_scale,
                                   partition_size=partition_size, stream=stream)
    torch.cuda.synchronize()
    return out.to(torch.float64).cpu().numpy()


def reference(c, rows=None):
    sel = np.arange(c.query.shape[0]) if rows is None else np.asarray(rows)
    ref = oracle.paged_attention_decode(
        np.ascontiguousarray(c.query[sel]), c.key_cache, c.value_cache,
        np.ascontiguousarray(c.block_tables[sel]), np.ascontiguousarray(c.context_lens[sel]),
        c.num_kv_heads, c.scale, c.k_scale, c.v_scale)
    b = attention_bound(c.query, c.key_cache, c.value_cache, c.block_tables, c.context_lens,
                        c.num_kv_heads, c.scale, c.k_scale, c.v_scale, rows=sel)
    return ref, b


def check(got, ref, b):
    assert not np.isnan(got).any(), "NaN in the output"
    err = np.abs(got - ref)
    worst = float(np.max(err / np.maximum(b, 1e-300))) if err.size else 0.0
    zero = b == 0
    assert np.all(got[zero] == 0), "rows without a valid token must be zero"
    assert np.all(err <= b), f"max err/bound = {worst:.3g}"
    return worst


@pytest.mark.parametrize("H,KVH,B,P", [
    (8, 1, 16, 256),     # 8 query heads per KV head
    (32, 2, 16, 64),     # 16 per KV head (the largest group)
    (4, 4, 32, 64),      # no grouping, 32-token pages, smallest partition
    (14, 2, 16, 128),    # a group of 7
    (64, 8, 16, 256),    # Llama-3.1-70B heads
    (16, 1, 64, 256),    # 64-token pages
    (24, 2, 16, 512),    # a group of 12, the largest partition
])
def test_shapes(H, KVH, B, P):
    banner(f"paged attention H={H} KVH={KVH} B={B} P={P}")
    lens = [1, 15, 16, 17, 31, 255, 256, 257, 600, 1029]
    c = workloads.paged_attention_case(40 + H + B + P, len(lens), H, KVH, block_size=B, lens=lens)
    ref, b = reference(c)
    worst = check(run(c, P), ref, b)
    print(f"max err / bound = {worst:.3g}", flush=True)


def test_long_contexts_many_partitions():
    banner("paged attention long contexts, P=64 to 2048")
    lens = [4100, 3000, 2049]
    c = workloads.paged_attention_case(9, len(lens), 16, 2, lens=lens)
    ref, b = reference(c)
    for P in (64, 512, 1024, 2048):
        check(run(c, P), ref, b)


def test_edges_empty_invalid_pages_and_stale_bytes():
    """Context 0; a sequence whose only pages are invalid ids (-1 and
    >= num_blocks); invalid pages in the middle of a context; a context that
    ends inside a page whose later slots hold NaN codes; max_context_len
    larger than every context."""
    banner("paged attention edges")
    lens = [0, 40, 300, 77, 1]
    c = workloads.paged_attention_case(21, len(lens), 8, 2, lens=lens)
    nb = c.key_cache.shape[0]
    c.block_tables[1, :3] = [-1, nb, nb + 7]            # no valid page at all
    c.block_tables[2, 3] = -5                           # a hole in the middle
    c.block_tables[2, 7] = nb + 1
    p = c.block_tables[3, 77 // 16]                     # the page where seq 3 ends
    c.key_cache[p, :, :, 77 % 16:, :] = 0x7F            # NaN codes past the end
    c.value_cache[p, :, :, 77 % 16:] = 0xFF
    ref, b = reference(c)
    assert np.all(ref[0] == 0) and np.all(ref[1] == 0)
    check(run(c, 256), ref, b)
    check(run(c, 64, max_context_len=1000), ref, b)


def test_repeated_calls_share_a_workspace_on_a_side_stream():
    banner("paged attention workspace reuse, side stream")
    c1 = workloads.paged_attention_case(31, 6, 64, 8, lens=[900, 1, 513, 64, 2000, 100])
    c2 = workloads.paged_attention_case(32, 6, 64, 8, lens=[5, 1999, 17, 256, 1, 700])
    ws = pkv.paged_attention_workspace(6, 64, 2000, 256, device=DEV)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g1 = run(c1, 256, max_context_len=2000, stream=s, ws=ws)
        g2 = run(c2, 256, max_context_len=2000, stream=s, ws=ws)
    check(g1, *reference(c1))
    check(g2, *reference(c2))


@pytest.mark.parametrize("P,B,balanced", [(2048, 16, False), (2048, 32, False), (512, 16, True),
                                          (64, 16, True), (256, 32, True)])
def test_both_work_splits_on_a_mixed_batch(P, B, balanced):
    """Contexts from one token to 4000 (whole-partition and ragged ends, a
    sequence inside one unit and sequences across many), through the fixed
    split (one partition per 2048 tokens) and the balanced one, with the
    16-token page build and the generic one."""
    lens = [1, 64, 65, 700, 2048, 1500, 4000, 3, 129, 2047, 999, 0, 64, 3333]
    H, KVH = 32, 4
    assert (balanced_units(len(lens), H, KVH, max(lens), P, 3072) > 0) == balanced
    banner(f"paged attention work split P={P} B={B} balanced={balanced}")
    c = workloads.paged_attention_case(50 + P + B, len(lens), H, KVH, block_size=B, lens=lens)
    ref, b = reference(c)
    worst = check(run(c, P), ref, b)
    print(f"max err / bound = {worst:.3g}", flush=True)


@pytest.mark.parametrize("P,balanced", [(256, True), (1024, False)])
def test_tokens_past_the_workspace_are_not_read(P, balanced):
    """Only tokens below ceil(max_context_len / P) * P are read, under either
    split: a context longer than that attends its first tokens only (the
    caller broke the max_context_len contract; nothing past it is touched)."""
    lens = [3000, 100, 700]
    maxc = 1000
    cap = -(-maxc // P) * P
    assert (balanced_units(len(lens), 16, 2, maxc, P, 3072) > 0) == balanced
    banner(f"paged attention contexts past max_context_len, P={P}")
    c = workloads.paged_attention_case(80 + P, len(lens), 16, 2, lens=lens)
    got = run(c, P, max_context_len=maxc)
    capped = workloads.PagedAttentionCase(c.query, c.key_cache, c.value_cache, c.block_tables,
                                          np.minimum(c.context_lens, cap).astype(np.int32),
                                          c.num_kv_heads, c.scale, c.k_scale, c.v_scale)
    ref, b = reference(capped)
    check(got, ref, b)


def test_one_long_context_across_many_units():
    """A 16K-token context beside a short one: the balanced split spreads the
    long sequence over about 86 units, and the reduce combines that many
    partials per head, four at a time."""
    lens = [16384, 300]
    assert balanced_units(2, 64, 8, max(lens), 256, 3072) > 100
    banner("paged attention one 16K-token context")
    c = workloads.paged_attention_case(91, len(lens), 64, 8, lens=lens)
    ref, b = reference(c)
    worst = check(run(c, 256), ref, b)
    print(f"max err / bound = {worst:.3g}", flush=True)


def test_one_64k_context_both_splits():
    """A 64K-token context beside a short and a one-token one.  At P=256 the
    balanced split spreads the long sequence over about 340 units (the reduce
    combines that many partials per head); at P=2048 the fixed split gives it
    32 partitions."""
    lens = [65536, 777, 1]
    assert balanced_units(3, 64, 8, max(lens), 256, 3072) > 300
    assert balanced_units(3, 64, 8, max(lens), 2048, 3072) == 0
    banner("paged attention one 64K-token context, P=256 and P=2048")
    c = workloads.paged_attention_case(93, len(lens), 64, 8, lens=lens)
    ref, b = reference(c)
    for P in (256, 2048):
        worst = check(run(c, P), ref, b)
        print(f"P={P}: max err / bound = {worst:.3g}", flush=True)


@pytest.mark.parametrize("S,balanced", [(4096, True), (4100, False)])
def test_many_sequences(S, balanced):
    """The most sequences the balanced split takes (their block counts fill
    one lane's range each), and just past it (the fixed split)."""
    lens = workloads.rng(60 + S).integers(0, 300, size=S).tolist()
    lens[5] = 300
    assert (balanced_units(S, 8, 1, 300, 64, 3072) > 0) == balanced
    banner(f"paged attention {S} sequences, balanced={balanced}")
    c = workloads.paged_attention_case(60 + S, S, 8, 1, lens=lens)
    got = run(c, 64, max_context_len=300)
    rows = sorted({5, *range(0, S, 97), S - 1})
    ref, b = reference(c, rows)
    worst = check(got[rows], ref, b)
    print(f"rows sampled: max err / bound = {worst:.3g}", flush=True)


def test_decode_batch_sampled():
    """The decode batch at its full size, in the launch configuration that is
    timed (200 sequences, Llama-3.1-70B heads, 16-token pages, the bench's
    partition size); the oracle checks a sample of sequences that includes the longest
    and the shortest."""
    banner("paged attention decode batch, sampled rows")
    c = workloads.decode_batch()
    got = run(c, workloads.DECODE_PARTITION)
    L = c.context_lens
    rows = sorted({int(np.argmax(L)), int(np.argmin(L)), *range(0, len(L), 23)})
    ref, b = reference(c, rows)
    worst = check(got[rows], ref, b)
    print(f"rows {rows}: max err / bound = {worst:.3g}", flush=True)
