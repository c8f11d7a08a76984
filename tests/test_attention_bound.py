"""CPU checks of the paged-attention error bound used by the GPU parity tests:
it holds for a binary32 model of the kernels' arithmetic, and it is tight
enough that plausible mistakes (a dropped token, a wrong scale, a wrong
query-to-KV-head map, a shifted page offset, softmax without the scale)
break it somewhere."""
import numpy as np
import pytest

import oracle
import workloads
from oracle.attention_bound import attention_bound, emulate_f32


def case(seed=3, lens=(1, 17, 300, 1000), H=8, KVH=2, B=16):
    return workloads.paged_attention_case(seed, len(lens), H, KVH, block_size=B, lens=list(lens))


def ref_of(c, **over):
    a = dict(query_bits=c.query, key_cache=c.key_cache, value_cache=c.value_cache,
             block_tables=c.block_tables, context_lens=c.context_lens,
             num_kv_heads=c.num_kv_heads, scale=c.scale, k_scale=c.k_scale, v_scale=c.v_scale)
    a.update(over)
    return oracle.paged_attention_decode(**a)


def bound_of(c):
    return attention_bound(c.query, c.key_cache, c.value_cache, c.block_tables, c.context_lens,
                           c.num_kv_heads, c.scale, c.k_scale, c.v_scale)


@pytest.mark.parametrize("P", [64, 512, 2048])
def test_bound_holds_for_a_binary32_model(P):
    c = case()
    ref, b = ref_of(c), bound_of(c)
    emu = emulate_f32(c.query, c.key_cache, c.value_cache, c.block_tables, c.context_lens,
                      c.num_kv_heads, c.scale, c.k_scale, c.v_scale, partition_size=P)
    err = np.abs(emu - ref)
    assert np.all(err <= b), f"max err/bound {np.max(err / np.maximum(b, 1e-300)):.3g}"
    # the bound is not vacuous: it is within a few bf16 ulps of the values
    assert np.all(b <= 2.0 ** -6 * np.abs(ref) + 1e-3)


def test_bound_catches_planted_mistakes():
    c = case()
    ref, b = ref_of(c), bound_of(c)
    G = c.query.shape[1] // c.num_kv_heads

    def broken(name, got):
        viol = np.abs(got - ref) > b
        assert viol.any(), f"the bound does not catch: {name}"

    lens = c.context_lens.copy()
    lens[lens > 1] -= 1
    broken("last token dropped", ref_of(c, context_lens=lens))
    broken("v_scale replaced by k_scale", ref_of(c, v_scale=c.k_scale))
    broken("scale left out", ref_of(c, scale=1.0))
    # query head h read against KV head h % KVH instead of h // G
    H = c.query.shape[1]
    perm = np.array([(h % c.num_kv_heads) * G + h // c.num_kv_heads for h in range(H)])
    q2 = c.query.copy()
    q2[:, perm] = c.query
    broken("GQA head map", ref_of(c, query_bits=np.ascontiguousarray(q2)))
    # every page read one row later (wrong offset inside the page)
    kc = np.roll(c.key_cache, 1, axis=3)
    vc = np.roll(c.value_cache, 1, axis=3)
    broken("page offset shifted", ref_of(c, key_cache=np.ascontiguousarray(kc),
                                         value_cache=np.ascontiguousarray(vc)))


def test_empty_rows_have_zero_bound():
    c = case(lens=(0, 5))
    c.block_tables[1, 0] = -1
    b = bound_of(c)
    assert np.all(b == 0)
    assert np.all(ref_of(c) == 0)
