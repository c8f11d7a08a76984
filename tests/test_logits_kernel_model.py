"""A lane-level host model of the indexer-logits kernel (mqa_logits.hip), run
on the CPU over the inputs of its GPU tests, the causal-range case among them.

The kernel is switched off because a GPU run of the causal-range case did not
finish.  This model executes the kernel's work map step by step for every
workgroup, wave and lane -- the per-token ranges, the cross-lane union of the
workgroup's key range (each ds_bpermute source lane), the tile loop's trip
count, every barrier, every global load and store address, every LDS write
and read of the double-buffered key tile -- and checks that
  * every loop ends and every wave of a workgroup reaches the same barriers;
  * every cross-lane source is a lane of the wave (0..63), all lanes active;
  * every global access is inside its buffer, every LDS access inside the
    tile (rows of 144 bytes, 64 rows, two buffers);
  * no LDS buffer is written while another wave may still read it (reads of
    tile n and the write of tile n+1 into the other buffer are separated by
    a barrier), and each read sees the tile the loop index says;
  * every logits element inside a row's range is written exactly once, and
    nothing outside the ranges (or in the padding columns) is written;
  * the values it computes from the key bytes it moved through the model LDS
    agree with the oracle (binary64 dot products in both, so only summation
    order differs).
It is a model of the indexing, not of the arithmetic units: the dot products
are exact binary64 here, where the matrix unit truncates (the GPU test bounds
that).  It proves nothing about the hardware; it shows that the kernel's own
logic on these inputs has no out-of-bounds access, unbounded loop or
mismatched barrier.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

WAVE = 64
THREADS = 256
WAVES = THREADS // WAVE
TOK_PER_WAVE = 2
TOKENS = WAVES * TOK_PER_WAVE     # query tokens per workgroup
TILE = 64                         # keys per LDS tile
D = 128
ROW = D + 16                      # padded LDS row, bytes
LDS_BYTES = TILE * ROW


def e4m3(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()


class Violation(AssertionError):
    pass


def need(cond, what):
    if not np.all(cond):
        raise Violation(what)


def run_model(q, k, k_scale, w, ks, ke, row_cols, row_stride, max_trips=1 << 20, mistake=None):
    """Executes the kernel's work map; returns (logits float64 [M, row_stride]
    with NaN where nothing was written, write counts, per-workgroup trips).
    `mistake` plants one indexing error in the model (to show the checks bite)."""
    M, H, _ = q.shape
    N = k.shape[0]
    kHB = H // 16
    q_token_stride = H * D
    qd, kd = e4m3(q), e4m3(k)
    out = np.full((M, row_stride), np.nan)
    writes = np.zeros((M, row_stride), np.int64)
    lane = np.arange(WAVE)
    col, grp = lane & 15, lane >> 4
    trips = []
    for b in range((M + TOKENS - 1) // TOKENS):
        i0 = b * TOKENS
        barriers = []
        # ---- per-wave token state (every wave computes the union itself)
        lo_w, hi_w = [], []
        for wave in range(WAVES):
            for t in range(TOK_PER_WAVE):
                i = i0 + wave * TOK_PER_WAVE + t
                if i < M:
                    for hb in range(kHB):
                        off = i * q_token_stride + (hb * 16 + col) * D + grp * 32
                        need((off >= 0) & (off + 32 <= M * q_token_stride), "q load out of bounds")
                        widx = i * H + hb * 16 + grp[:, None] * 4 + np.arange(4)
                        need((widx >= 0) & (widx < M * H), "weights load out of bounds")
            # union over lanes 0..7 (butterfly of ds_bpermute over lane ^ d)
            i_l = i0 + (lane & (TOKENS - 1))
            act = (lane < TOKENS) & (i_l < M)
            need((i_l[act] >= 0) & (i_l[act] < M), "ks/ke load out of bounds")
            s = np.where(act, ks[np.minimum(i_l, M - 1)].astype(np.int64), 0)
            e = np.where(act, ke[np.minimum(i_l, M - 1)].astype(np.int64), 0)
            ll = np.maximum(s, 0)
            hh = np.minimum(np.minimum(e, N), s + row_cols)
            has = act & (hh > ll)
            l = np.where(has, ll, np.iinfo(np.int64).max)
            h = np.where(has, hh, 0)
            d = 1
            while d < TOKENS:
                src = lane ^ d
                need((src >= 0) & (src < WAVE), "cross-lane source outside the wave")
                l, h = np.minimum(l, l[src]), np.maximum(h, h[src])
                d <<= 1
            lo_w.append(int(l[0]))
            hi_w.append(int(h[0]))
        need(len(set(lo_w)) == 1 and len(set(hi_w)) == 1, "waves disagree on the union")
        lo, hi = lo_w[0], hi_w[0]
        if hi <= lo:
            trips.append(0)
            continue                                  # every wave returns before any barrier
        ntiles = (hi - lo + TILE - 1) // TILE
        need(0 < ntiles <= max_trips and ntiles <= (N + TILE - 1) // TILE + 1,
             "tile loop trip count out of range")
        trips.append(ntiles)

        # ---- model LDS: bytes and, per buffer, which tile it holds
        lds = np.zeros((2, LDS_BYTES), np.uint8)
        lds_scale = np.zeros((2, TILE), np.float32)
        holds = [-1, -1]
        readers_since_barrier = [set(), set()]

        def load_tile(n):
            j0 = lo + n * TILE
            stage = []
            for u in range(2):
                c = np.arange(THREADS) + u * THREADS
                j = j0 + c // 8
                ok = j < hi if mistake != "no_key_guard" else np.ones_like(j, bool)
                off = j * D + (c % 8) * 16
                need((off[ok] >= 0) & (off[ok] + 16 <= N * D), "key load out of bounds")
                data = np.zeros((THREADS, 16), np.uint8)
                flat = k.reshape(-1)
                for x in np.nonzero(ok)[0]:
                    data[x] = flat[off[x]:off[x] + 16]
                stage.append(data)
            tid = np.arange(TILE)
            j = j0 + tid
            ok = j < hi
            need((j[ok] >= 0) & (j[ok] < N), "k_scale load out of bounds")
            sc = np.where(ok, k_scale[np.minimum(j, N - 1)], np.float32(0))
            return stage, sc

        def store_tile(buf, staged, n):
            need(not readers_since_barrier[buf], "LDS buffer written while it may still be read")
            stage, sc = staged
            for u in range(2):
                c = np.arange(THREADS) + u * THREADS
                off = (c // 8) * ROW + (c % 8) * 16
                need((off >= 0) & (off + 16 <= LDS_BYTES), "LDS tile write out of bounds")
                for x in range(THREADS):
                    lds[buf, off[x]:off[x] + 16] = stage[u][x]
            lds_scale[buf] = sc
            holds[buf] = n

        def barrier():
            barriers.append(1)
            readers_since_barrier[0].clear()
            readers_since_barrier[1].clear()

        store_tile(0, load_tile(0), 0)
        barrier()
        for n in range(ntiles):
            buf = n & 1
            staged = load_tile(n + 1) if n + 1 < ntiles else None
            need(holds[buf] == n, "a wave reads a tile the loop index does not name")
            j0 = lo + n * TILE
            for wave in range(WAVES):
                readers_since_barrier[buf].add(wave)
                for s16 in range(TILE // 16):
                    brow = (s16 * 16 + col) * ROW + grp * 32
                    need((brow >= 0) & (brow + 32 <= LDS_BYTES), "LDS key read out of bounds")
                    need((s16 * 16 + col < TILE), "LDS scale read out of bounds")
                    keys = np.stack([lds[buf, brow[x]:brow[x] + 32] for x in range(16)])  # lanes 0..15
                    # the 16 keys of this subtile, rebuilt from the four lane groups' 32-byte quarters
                    full = np.zeros((16, D), np.uint8)
                    for g in range(4):
                        rows = (s16 * 16 + np.arange(16)) * ROW + g * 32
                        for x in range(16):
                            full[x, g * 32:(g + 1) * 32] = lds[buf, rows[x]:rows[x] + 32]
                    need(np.array_equal(keys, full[:, :32]), "lane-group layout mismatch")
                    sc = lds_scale[buf, s16 * 16 + np.arange(16)].astype(np.float64)
                    j = j0 + s16 * 16 + np.arange(16)
                    for t in range(TOK_PER_WAVE):
                        i = i0 + wave * TOK_PER_WAVE + t
                        for src_d in (16, 32):
                            need(((lane ^ src_d) >= 0) & ((lane ^ src_d) < WAVE),
                                 "shuffle source outside the wave")
                        if i >= M:
                            continue
                        s_t = int(ks[i])
                        lo_t = max(s_t, 0)
                        hi_t = max(min(int(ke[i]), N, s_t + row_cols), lo_t)
                        dots = qd[i] @ e4m3(full).T                     # [H, 16]
                        part = (w[i].astype(np.float64)[:, None] * np.maximum(dots, 0)).sum(0)
                        for x in np.nonzero((j >= lo_t) & (j < hi_t))[0]:
                            cidx = int(j[x]) - (s_t if mistake != "column_from_union" else lo)
                            need(0 <= cidx < row_cols, "logits store outside the row's columns")
                            out[i, cidx] = sc[x] * part[x]
                            writes[i, cidx] += 1
            if n + 1 < ntiles:
                store_tile(buf if mistake == "one_buffer" else buf ^ 1, staged, n + 1)
            barrier()
        need(len(barriers) == ntiles + 1, "barrier count differs from the trip count")
    return out, writes, trips


def check_case(q, k, k_scale, w, ks, ke, row_cols, pad=0):
    M = q.shape[0]
    N = k.shape[0]
    out, writes, trips = run_model(q, k, k_scale, w, ks, ke, row_cols, row_cols + pad)
    ref = np.full((M, row_cols), np.nan)
    oracle.fp8_mqa_logits(q, k, k_scale, w, ks, ke, ref)
    valid = ~np.isnan(ref)
    assert np.all(writes[:, row_cols:] == 0), "padding columns written"
    assert np.all(writes[:, :row_cols][valid] == 1), "an element in range not written exactly once"
    assert np.all(writes[:, :row_cols][~valid] == 0), "an element outside the ranges written"
    got = out[:, :row_cols][valid]
    # binary64 on both sides in different summation orders: agreement to 1e-12
    # of the largest magnitude (the sums cancel, so a purely relative test is too tight)
    assert np.allclose(got, ref[valid], rtol=1e-12, atol=1e-12 * np.abs(ref[valid]).max())
    return trips


def test_model_on_the_causal_request_case():
    """The GPU case that did not finish: causal ranges of requests of 1, 70,
    129 and 5 tokens, H = 64, a row stride 12 columns wider than the rows."""
    g = workloads.mqa_logits_case(7, num_q=0, num_heads=64, num_k=0, causal_lens=[1, 70, 129, 5])
    cols = int(max(g.ke - g.ks))
    trips = check_case(g.q, g.k, g.k_scale, g.weights, g.ks, g.ke, cols, pad=12)
    assert len(trips) == 26 and max(trips) == 3 and min(trips) >= 1


@pytest.mark.parametrize("H", [16, 64])
def test_model_on_random_ranges(H):
    """The GPU cases that passed (negative start, full range, tail past the
    keys, an empty range)."""
    g = workloads.mqa_logits_case(100 + H, num_q=37, num_heads=H, num_k=300)
    ks, ke = g.ks.copy(), g.ke.copy()
    ks[:4] = [-5, 0, 290, 100]
    ke[:4] = [20, 300, 350, 100]
    check_case(g.q, g.k, g.k_scale, g.weights, ks, ke, 200)


@pytest.mark.parametrize("mistake", ["column_from_union", "one_buffer", "no_key_guard"])
def test_model_catches_planted_mistakes(mistake):
    """Each planted indexing error fails a check on the causal case: the store
    column taken from the workgroup's union start instead of the token's own
    range start; the next tile staged into the buffer being read; key loads
    without the range guard (the last tile runs past the keys)."""
    g = workloads.mqa_logits_case(7, num_q=0, num_heads=16, num_k=0, causal_lens=[1, 70, 129, 5])
    cols = int(max(g.ke - g.ks))
    with pytest.raises(AssertionError):
        out, writes, _ = run_model(g.q, g.k, g.k_scale, g.weights, g.ks, g.ke, cols, cols,
                                   mistake=mistake)
        ref = np.full((g.q.shape[0], cols), np.nan)
        oracle.fp8_mqa_logits(g.q, g.k, g.k_scale, g.weights, g.ks, g.ke, ref)
        valid = ~np.isnan(ref)
        assert np.all(writes[:, :cols][valid] == 1) and np.all(writes[:, :cols][~valid] == 0)
        assert np.allclose(out[:, :cols][valid], ref[valid], rtol=1e-12,
                           atol=1e-12 * np.abs(ref[valid]).max())


def test_model_on_the_gathered_keys_case():
    """The GPU case on keys the path produced: the fp8 store of bf16 K, then
    the gather back; 16 requests of 512 tokens with causal ranges."""
    w = workloads.c4_roundtrip()
    cache = w.cache_init.copy()
    oracle.store_indexer_k_fp8(w.k_bits, w.slot_mapping, cache, w.block_size, w.head_dim)
    T = int(w.cu_seq_lens[-1])
    kf = np.zeros((T, 128), np.uint8)
    ksb = np.zeros((T, 4), np.uint8)
    oracle.gather_indexer_k_fp8(cache, kf, ksb, w.block_table, w.cu_seq_lens, w.block_size, 128)
    k_scale = ksb.view(np.float32).reshape(T)
    keep = w.slot_mapping[:T] >= 0
    g = workloads.mqa_logits_case(11, num_q=0, num_heads=64, num_k=0,
                                  causal_lens=list(np.diff(w.cu_seq_lens)))
    kf[~keep] = 0
    k_scale = np.where(keep, k_scale, 0).astype(np.float32)
    # the first request (512 query tokens) keeps the model's run short
    n = 512
    check_case(np.ascontiguousarray(g.q[:n]), kf, k_scale, np.ascontiguousarray(g.weights[:n]),
               np.ascontiguousarray(g.ks[:n]), np.ascontiguousarray(g.ke[:n]), 512)


def test_model_on_the_extreme_codes_case():
    g = workloads.mqa_logits_case(13, num_q=16, num_heads=64, num_k=80)
    q, k = g.q.copy(), g.k.copy()
    q[0] = 0x7E
    q[1] = 0xFE
    k[:8] = 0x7E
    k[8:16] = 0x01
    q[2, :, ::8] = 0x7E
    check_case(q, k, g.k_scale, g.weights, g.ks, g.ke, 80)
