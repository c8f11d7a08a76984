"""Pins for the oracle's paged decode attention over fp8 pages: a hand-worked
case (W13), an independent numpy reading (pages unpacked with reshapes,
torch's float8_e4m3fn decode, a float64 softmax), and the invariants of
attention (uniform weights for equal keys, page placement, GQA sharing,
linearity in v_scale, dropped tokens, empty sequences)."""
import json
import math
import os

import numpy as np
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def dec(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()


def numpy_attention(qbits, kc, vc, bt, cl, kvh, scale, ks, vs):
    S, H, D = qbits.shape
    nb, _, _, B, _ = kc.shape
    q = (qbits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    K = dec(kc).transpose(0, 1, 3, 2, 4).reshape(nb, kvh, B, D) * np.float64(np.float32(ks))
    V = dec(vc).transpose(0, 1, 3, 2) * np.float64(np.float32(vs))       # [nb, kvh, B, D]
    out = np.zeros((S, H, D))
    g = H // kvh
    for s in range(S):
        toks = [t for t in range(int(cl[s])) if t // B < bt.shape[1] and 0 <= bt[s, t // B] < nb]
        if not toks:
            continue
        pages = np.array([bt[s, t // B] for t in toks])
        offs = np.array([t % B for t in toks])
        for h in range(H):
            k = K[pages, h // g, offs]                    # [n, D]
            v = V[pages, h // g, offs]
            lg = scale * (k @ q[s, h])
            w = np.exp(lg - lg.max())
            out[s, h] = (w @ v) / w.sum()
    return out


def test_w13_hand_worked():
    with open(os.path.join(GOLDEN, "w13_paged_attention.json")) as f:
        g = json.load(f)
    H, KVH, D, B, NB = g["num_heads"], g["num_kv_heads"], g["head_size"], g["block_size"], g["num_blocks"]
    kc = np.zeros((NB, KVH, D // 16, B, 16), np.uint8)
    for d, code in g["key_token1"].items():
        d = int(d)
        kc[1, 0, d // 16, 1, d % 16] = int(code, 16)
    vc = np.zeros((NB, KVH, D, B), np.uint8)
    vc[1, 0, :, 0] = int(g["value_codes"][0], 16)
    vc[1, 0, :, 1] = int(g["value_codes"][1], 16)
    q = np.zeros((1, H, D), np.uint16)
    q[0, 0, 0] = 0x3F80
    q[0, 1, 1] = 0x3F80
    out = oracle.paged_attention_decode(q, kc, vc, np.array(g["block_table"], np.int32),
                                        np.array([g["context_len"]], np.int32), KVH, math.log(3),
                                        g["k_scale"], g["v_scale"])
    np.testing.assert_allclose(out[0, 0], g["out_head0"], rtol=1e-14)
    np.testing.assert_allclose(out[0, 1], g["out_head1"], rtol=1e-14)


def test_matches_numpy_reading():
    c = workloads.paged_attention_case(3, num_seqs=5, num_heads=8, num_kv_heads=2, block_size=16,
                                       max_context=100)
    out = oracle.paged_attention_decode(c.query, c.key_cache, c.value_cache, c.block_tables,
                                        c.context_lens, c.num_kv_heads, c.scale, c.k_scale,
                                        c.v_scale)
    ref = numpy_attention(c.query, c.key_cache, c.value_cache, c.block_tables, c.context_lens,
                          c.num_kv_heads, c.scale, c.k_scale, c.v_scale)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-13)


def test_invariants():
    c = workloads.paged_attention_case(4, num_seqs=3, num_heads=4, num_kv_heads=2, block_size=16,
                                       max_context=64)
    run = lambda **kw: oracle.paged_attention_decode(
        kw.get("q", c.query), kw.get("kc", c.key_cache), kw.get("vc", c.value_cache),
        kw.get("bt", c.block_tables), kw.get("cl", c.context_lens), c.num_kv_heads, c.scale,
        c.k_scale, kw.get("vs", c.v_scale))
    base = run()
    # equal keys everywhere: uniform weights, the plain mean of the values
    kc_eq = np.full_like(c.key_cache, 0x38)
    out = run(kc=kc_eq)
    ref = numpy_attention(c.query, kc_eq, c.value_cache, c.block_tables, c.context_lens,
                          c.num_kv_heads, c.scale, c.k_scale, c.v_scale)
    np.testing.assert_allclose(out, ref, rtol=1e-12)
    # doubling v_scale doubles the output exactly
    np.testing.assert_array_equal(run(vs=2 * c.v_scale), 2 * base)
    # moving the pages (and the block table with them) changes nothing
    nb = c.key_cache.shape[0]
    perm = np.random.default_rng(0).permutation(nb)
    inv = np.argsort(perm)
    bt2 = np.where((c.block_tables >= 0) & (c.block_tables < nb), inv[np.clip(c.block_tables, 0, nb - 1)],
                   c.block_tables).astype(np.int32)
    np.testing.assert_array_equal(run(kc=c.key_cache[perm].copy(), vc=c.value_cache[perm].copy(),
                                      bt=bt2), base)
    # GQA: two heads of one kv group with the same query get the same output
    q2 = c.query.copy()
    q2[:, 1] = q2[:, 0]
    o2 = run(q=q2)
    np.testing.assert_array_equal(o2[:, 0], o2[:, 1])
    # an empty sequence gets a zero row; a dropped page drops its tokens
    cl = c.context_lens.copy()
    cl[0] = 0
    np.testing.assert_array_equal(run(cl=cl)[0], 0.0)
    bt3 = c.block_tables.copy()
    bt3[1, 0] = -1
    out3 = run(bt=bt3)
    ref3 = numpy_attention(c.query, c.key_cache, c.value_cache, bt3, c.context_lens,
                           c.num_kv_heads, c.scale, c.k_scale, c.v_scale)
    np.testing.assert_allclose(out3, ref3, rtol=1e-11, atol=1e-13)
