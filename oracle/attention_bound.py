"""Per-element error bound of the paged decode attention kernels against the
exact (binary64) result, derived from their arithmetic.

TEST INFRASTRUCTURE, like the rest of this package: the tests and
``__graft_entry__.smoke()`` use it to check the GPU result; the product
never imports it.

With w_t = exp(l_t - M) the exact softmax weights of the valid tokens,
W = sum_t w_t, o = sum_t w_t v_t / W:

1. Logits.  q (bf16) and the key codes (E4M3, exact in bf16) meet in
   v_mfma_f32_16x16x32_bf16: products exact, binary32 accumulation over 128
   of them (4 instructions), error <= 128 * 2^-24 * sum_d |q_d c_d|; then
   one multiply by fl(scale * k_scale): two more roundings.  We take
       delta_t = 2^-15 * s * sum_d |q_d c_d| + 2^-21 * |l_t|,  s = scale*k_scale
   (4x the accumulation bound).
2. Exponentials.  Logits are scaled by log2(e) (in binary32) and each
   weight is a product of hardware exp2 values: the token's own (against a
   reference point that trails the running maximum by at most 2^8), one
   rescale factor per later move of the reference point (a move raises it
   by more than 8 in log2 units, so there are at most R log2(e) / 8 of
   them, R the logit range of the row, however many blocks a partition
   has), the partial's weight in the final combination, and one rescale
   factor per later group of four partials that raises the combination's
   running maximum (at most ceil(n_p / 4) for n_p partials).  A row has at
   most n_p = ceil(L / 64) + 1 partials under either work split (a segment
   is at least one 64-token block; the balanced split adds at most one
   segment per sequence).  Each factor has relative error <= 2^-23 +
   2^-24 |x| for an argument x of natural size; the |x| along one product
   sum to at most 3 (R + 8 ln 2) + R.  So the product of (2 + R/5 +
   ceil(n_p/4)) factors is within
       rho = (2 + R/5 + ceil(n_p/4)) 2^-23 + (4 R + 17) 2^-24.
   Together with 1., the device weights are w_t (1 + g_t) with
   |g_t| <= gamma = max_t expm1(2 delta_t) + 2 rho (the factor 2 on delta
   covers the shifted reference, the one on rho is margin).
   Perturbing the weights moves the result by at most
       gamma / (1 - gamma) * C,   C = sum_t w_t |v_t - o| / W.
3. The P.V product and the sums.  A partition covers at most 2048 tokens.
   Probabilities enter the bf16 MFMA as a hi + lo pair (relative error
   <= 2^-17) and accumulate in binary32 over at most 2048 tokens x 2 terms,
   each addition rounded (<= 2^12 * 2^-24 = 2^-12 of sum w|v|); they are
   normalised by the partition's exp-sum.  The exp-sum takes at most 2048
   terms in per-lane sums of 16 per block (<= 32 * 17 + 2 roundings), the
   normalisation 3 more and the combination of n_p partials at most 3 n_p
   + 2 (the weighted sums, their rescalings and the final reciprocal): at
   most (551 + 3 n_p) 2^-24 relative to the denominator.  With alpha =
   2^-11 (2x margin) and beta = (551 + 3 n_p) 2^-23 (2x margin):
       E = gamma C / (1 - gamma) + (alpha A (1 + gamma) + beta (|o| + gamma C)) / (1 - beta),
       A = sum_t w_t |v_t| / W.
4. The bf16 output rounds to nearest (8 significant bits): + 2^-8 (|o| + E).

A row without a valid token must be exactly zero (bound 0).
"""
import numpy as np
import torch


def e4m3_decode(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()


def bf16_decode(bits):
    return (np.ascontiguousarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def row_tokens(block_tables, context_lens, s, block_size, num_blocks):
    """(pages, offsets) of the valid tokens of sequence s, in token order."""
    L = int(context_lens[s])
    if L <= 0:
        return np.zeros(0, np.int64), np.zeros(0, np.int64)
    t = np.arange(L)
    j = t // block_size
    ok = j < block_tables.shape[1]
    pages = np.full(L, -1, np.int64)
    pages[ok] = block_tables[s, j[ok]]
    ok &= (pages >= 0) & (pages < num_blocks)
    return pages[ok], (t % block_size)[ok]


def attention_bound(query_bits, key_cache, value_cache, block_tables, context_lens,
                    num_kv_heads, scale, k_scale, v_scale, rows=None):
    """bound float64 [len(rows), H, D] for the selected sequences (all by default)."""
    S, H, D = query_bits.shape
    nb, _, _, B, _ = key_cache.shape
    G = H // num_kv_heads
    rows = range(S) if rows is None else rows
    q_all = bf16_decode(query_bits)
    out = []
    for s in rows:
        pages, offs = row_tokens(block_tables, context_lens, s, B, nb)
        bnd = np.zeros((H, D))
        if pages.size:
            kc = e4m3_decode(key_cache[pages, :, :, offs, :]).reshape(pages.size, num_kv_heads, D)
            vv = e4m3_decode(value_cache[pages, :, :, offs]) * v_scale      # [n, KVH, D]
            sk = float(scale) * float(k_scale)
            n_p = -(-int(context_lens[s]) // 64) + 1
            for kvh in range(num_kv_heads):
                qh = q_all[s, kvh * G:(kvh + 1) * G]                         # [G, D]
                l = sk * (qh @ kc[:, kvh].T)                                 # [G, n]
                absdot = sk * (np.abs(qh) @ np.abs(kc[:, kvh]).T)
                M = l.max(1, keepdims=True)
                w = np.exp(l - M)
                W = w.sum(1, keepdims=True)
                Vh = vv[:, kvh]                                              # [n, D]
                o = (w @ Vh) / W                                             # [G, D]
                A = (w @ np.abs(Vh)) / W
                C = np.einsum("gt,gtd->gd", w, np.abs(Vh[None, :, :] - o[:, None, :])) / W
                delta = 2.0 ** -15 * absdot + 2.0 ** -21 * np.abs(l)
                R = l.max(1) - l.min(1)
                rho = (2 + R / 5 + -(-n_p // 4)) * 2.0 ** -23 + (4 * R + 17) * 2.0 ** -24
                gamma = (np.expm1(2 * delta).max(1) + 2 * rho)[:, None]
                alpha, beta = 2.0 ** -11, (551 + 3 * n_p) * 2.0 ** -23
                E = gamma * C / (1 - gamma) + (alpha * A * (1 + gamma) +
                                               beta * (np.abs(o) + gamma * C)) / (1 - beta)
                bnd[kvh * G:(kvh + 1) * G] = E + 2.0 ** -8 * (np.abs(o) + E)
        out.append(bnd)
    return np.stack(out) if out else np.zeros((0, H, D))


def emulate_f32(query_bits, key_cache, value_cache, block_tables, context_lens, num_kv_heads,
                scale, k_scale, v_scale, partition_size=256):
    """A binary32 model of the kernels' arithmetic (partitions, exp-sums,
    combination, bf16 output) for checking the bound on the CPU; returns the
    bf16 results widened to float64."""
    S, H, D = query_bits.shape
    nb, _, _, B, _ = key_cache.shape
    G = H // num_kv_heads
    f = np.float32
    q_all = bf16_decode(query_bits).astype(f)
    sk = f(f(scale) * f(k_scale))
    res = np.zeros((S, H, D))
    for s in range(S):
        L = int(context_lens[s])
        if L <= 0:
            continue
        t = np.arange(L)
        j = t // B
        pages = np.full(L, -1, np.int64)
        ok = j < block_tables.shape[1]
        pages[ok] = block_tables[s, j[ok]]
        ok &= (pages >= 0) & (pages < nb)
        for kvh in range(num_kv_heads):
            acc_num = np.zeros((G, D), f)
            parts = []
            for p0 in range(0, L, partition_size):
                sel = np.arange(p0, min(p0 + partition_size, L))
                sel = sel[ok[sel]]
                if sel.size == 0:
                    continue
                kc = e4m3_decode(key_cache[pages[sel], kvh, :, sel % B, :]).reshape(
                    sel.size, D).astype(f)
                vc = e4m3_decode(value_cache[pages[sel], kvh, :, sel % B]).astype(f)
                qh = q_all[s, kvh * G:(kvh + 1) * G]
                l = (qh @ kc.T).astype(f) * sk
                m = l.max(1, keepdims=True)
                p = np.exp((l - m).astype(f)).astype(f)
                lsum = p.sum(1, dtype=f, keepdims=True)
                hi = (p.view(np.uint32) + 0x7FFF + ((p.view(np.uint32) >> 16) & 1)) & 0xFFFF0000
                hi = hi.view(f)
                num = (hi @ vc).astype(f) + ((p - hi).astype(f) @ vc).astype(f)
                parts.append((lsum, m, (num * f(f(v_scale) / lsum)).astype(f)))
            if not parts:
                continue
            M = np.max(np.concatenate([m for _, m, _ in parts], 1), 1, keepdims=True)
            Wsum = np.zeros((G, 1), f)
            for lsum, m, o in parts:
                w = (lsum * np.exp((m - M).astype(f))).astype(f)
                acc_num = (acc_num + w * o).astype(f)
                Wsum = (Wsum + w).astype(f)
            o = (acc_num * (f(1) / Wsum)).astype(f)
            res[s, kvh * G:(kvh + 1) * G] = torch.from_numpy(o).to(torch.bfloat16).to(
                torch.float64).numpy()
    return res
