"""The balanced work split of the paged decode attention, modelled on the
CPU: unit u of U takes the flattened 64-token blocks [u W, (u + 1) W) of all
sequences (W = ceil(N / U)); its segments must cover every readable token of
every sequence exactly once, stay within 2048 tokens, write distinct
workspace rows u + s inside the caller's [num_seqs * max_parts] rows, and the
reduce must read back exactly the rows written for each sequence, from the
per-sequence record (first row, count) that the wave attending the
sequence's first block leaves after the rows.  The model
follows the kernels' index arithmetic step by step, including the lane-range
search the partition kernel uses to find a unit's first sequence."""
import math

import numpy as np
import pytest

WAVE = 64
WAVE_TOKENS = 64


def balanced_units(S, H, KVH, maxc, P, wave_slots):
    """The host's choice (0 = fixed split)."""
    max_parts = -(-maxc // P)
    if max_parts < 2 or S < 1 or S > WAVE * WAVE:
        return 0
    n_max = S * (max_parts * P // WAVE_TOKENS)
    if n_max >= 2 ** 31 - 1:
        return 0
    u_min = -(-n_max // 32)
    u_cap = S * (max_parts - 1) - -(-2 * S // H)
    if u_cap < u_min:
        return 0
    groups = -(-KVH // 4)
    active = min(KVH, 4)
    u = -(-wave_slots // (groups * active))
    return min(max(u, u_min), u_cap)


def seq_blocks(L, cap):
    n = min(L, cap)
    return -(-n // WAVE_TOKENS) if n > 0 else 0


def lane_prefix(lens, cap):
    S = len(lens)
    per = -(-S // WAVE)
    mine = [sum(seq_blocks(int(lens[i * per + k]), cap) for k in range(per) if i * per + k < S)
            for i in range(WAVE)]
    base = np.concatenate([[0], np.cumsum(mine)[:-1]]).astype(int)
    return per, base, int(sum(mine))


def first_sequence(lens, cap, per, base, N, b0):
    """The partition kernel's search: the lane range whose end exceeds b0,
    then the first sequence inside it whose blocks end past b0."""
    S = len(lens)
    end = [int(base[i + 1]) if i < WAVE - 1 else N for i in range(WAVE)]
    r = next(i for i in range(WAVE) if end[i] > b0)
    rbase = int(base[r])
    nb = [seq_blocks(int(lens[r * per + k]), cap) if k < per and r * per + k < S else 0
          for k in range(WAVE)]
    incl = np.cumsum(nb)
    k = next(i for i in range(WAVE) if i < per and rbase + incl[i] > b0)
    return r * per + k, rbase + int(incl[k]) - nb[k]


def seq_cum(lens, cap, per, base, s):
    c = s // per
    return int(base[c]) + sum(seq_blocks(int(lens[c * per + k]), cap)
                              for k in range(WAVE) if c * per + k < s)


def run_split(lens, H, KVH, maxc, P, slots):
    S = len(lens)
    U = balanced_units(S, H, KVH, maxc, P, slots)
    if U == 0:
        return None
    max_parts = -(-maxc // P)
    cap = max_parts * P
    per, base, N = lane_prefix(lens, cap)
    segs = []          # (u, s, t_begin, t_end, row, direct)
    meta = {}          # s -> (first row, count), as the partition kernel records it
    if N == 0:
        return U, segs, {s: [] for s in range(S)}
    W = -(-N // U)
    assert W <= 32
    for u in range(U):
        b0 = u * W
        if b0 >= N:
            continue
        b1 = min(b0 + W, N)
        s, cum = first_sequence(lens, cap, per, base, N, b0)
        assert cum == seq_cum(lens, cap, per, base, s)
        while cum < b1 and s < S:
            lo = b0 - cum if b0 > cum else 0
            L = min(int(lens[s]), cap)
            nb = seq_blocks(L, cap)
            if nb > 0:
                hi = min(b1 - cum, nb)
                t_begin, t_end = lo * WAVE_TOKENS, min(hi * WAVE_TOKENS, L)
                first = cum // W
                count = (cum + nb - 1) // W - first + 1
                if lo == 0:
                    assert s not in meta
                    meta[s] = (first + s, count)
                segs.append((u, s, t_begin, t_end, u + s, count == 1))
            cum += nb
            s += 1
    # the reduce kernel's view of each sequence: its record, read only for
    # a sequence with blocks
    reads = {}
    for s in range(S):
        if seq_blocks(int(lens[s]), cap) == 0:
            reads[s] = []
            continue
        r0, count = meta[s]
        assert r0 >= 0 and count >= 1 and r0 + count <= U + S
        reads[s] = [r0 + p for p in range(count)]
    # the records sit after the rows and inside the workspace
    assert (U + S) * H + 2 * S <= S * max_parts * H
    return U, segs, reads


def check_split(lens, KVH, maxc, P, slots=3072, H=None):
    H = 8 * KVH if H is None else H
    out = run_split(lens, H, KVH, maxc, P, slots)
    if out is None:
        return False
    U, segs, reads = out
    S = len(lens)
    max_parts = -(-maxc // P)
    cap = max_parts * P
    covered = {s: np.zeros(max(min(int(lens[s]), cap), 0), int) for s in range(S)}
    rows = set()
    by_seq = {}
    for u, s, t0, t1, row, direct in segs:
        assert t0 % WAVE_TOKENS == 0 and 0 <= t0 < t1 <= min(int(lens[s]), cap)
        assert t1 - t0 <= 2048
        covered[s][t0:t1] += 1
        assert 0 <= row < S * max_parts and row not in rows
        rows.add(row)
        by_seq.setdefault(s, []).append((t0, row, direct))
    for s in range(S):
        assert np.all(covered[s] == 1), f"sequence {s} not covered once"
        mine = sorted(by_seq.get(s, []))
        if not mine:
            assert reads[s] == []
            continue
        if len(mine) == 1:
            assert mine[0][2], "a one-segment sequence is written directly"
            assert len(reads[s]) == 1
        else:
            assert not any(d for _, _, d in mine)
            assert reads[s] == [r for _, r, _ in mine], f"reduce rows of sequence {s}"
    return True


def test_decode_batch_shape_uses_the_balanced_split():
    rng = np.random.default_rng(1)
    lens = rng.integers(128, 2561, size=200)
    assert balanced_units(200, 64, 8, 2560, 1024, 3072) == 384
    assert check_split(lens, 8, int(lens.max()), 1024, H=64)


@pytest.mark.parametrize("seed", range(12))
def test_random_batches(seed):
    rng = np.random.default_rng(100 + seed)
    S = int(rng.integers(1, 300))
    maxc = int(rng.integers(1, 9000))
    lens = rng.integers(0, maxc + 1, size=S)
    lens[rng.random(S) < 0.1] = 0
    if S > 2:
        lens[rng.integers(0, S)] = maxc
    P = int(2 ** rng.integers(6, 12))
    KVH = int(rng.choice([1, 2, 4, 8, 16]))
    G = int(rng.choice([1, 3, 8, 16]))
    slots = int(rng.choice([64, 3072, 7000]))
    check_split(lens, KVH, maxc, P, slots, H=G * KVH)


def test_edge_batches():
    # all empty, one long sequence, contexts past max_context_len (capped),
    # many one-block sequences in one unit, the most sequences the split takes
    assert check_split(np.zeros(10, int), 8, 5000, 256)
    assert check_split(np.array([100000]), 8, 100000, 2048) is False   # no room for units
    assert check_split(np.array([100000]), 8, 100000, 1024)
    assert check_split(np.array([3000, 9000, 5]), 8, 3000, 512)
    assert check_split(np.ones(1000, int) * 3, 8, 3000, 1024, slots=64)
    rng = np.random.default_rng(7)
    assert check_split(rng.integers(0, 200, size=4096), 8, 200, 64)
    assert balanced_units(4097, 64, 8, 4096, 64, 3072) == 0
    assert balanced_units(10, 64, 8, 1024, 1024, 3072) == 0              # one partition
    # one head: the records take whole rows, so short workspaces keep the fixed split
    assert check_split(np.array([500, 700]), 1, 700, 256, H=1) is False
    assert check_split(np.array([500, 2000]), 1, 2000, 256, H=1)


def test_units_fit_the_workspace_and_the_table_slice():
    for S in (1, 7, 200, 4096):
        for maxc in (65, 1000, 2560, 65536):
            for P in (64, 256, 1024, 2048):
                U = balanced_units(S, 64, 8, maxc, P, 3072)
                if U == 0:
                    continue
                max_parts = -(-maxc // P)
                assert (U + S) * 64 + 2 * S <= S * max_parts * 64
                assert math.ceil(S * (max_parts * P // 64) / U) <= 32


def test_library_sizes_the_split_like_the_model():
    """The library's host-side choice (pkv_attention_balanced_units, no GPU
    work) agrees with the model above on random and edge sizes, so the
    coverage and workspace properties checked here hold for what it launches."""
    import paged_quantized_kv_amd as pkv
    rng = np.random.default_rng(5)
    cases = [(200, 64, 8, 2560, 1024, 3072), (1, 8, 1, 1, 64, 3072), (4096, 64, 8, 4096, 64, 3072),
             (4097, 64, 8, 4096, 64, 3072), (2, 1, 1, 700, 256, 3072), (2, 1, 1, 2000, 256, 3072),
             (3, 16, 2, 1 << 30, 2048, 3072), (0, 8, 1, 100, 64, 3072), (10, 64, 8, 1024, 1024, 3072)]
    for _ in range(3000):
        kvh = int(rng.choice([1, 2, 4, 8, 16]))
        cases.append((int(rng.integers(0, 5000)), kvh * int(rng.integers(1, 17)), kvh,
                      int(rng.integers(0, 200000)), int(2 ** rng.integers(6, 12)),
                      int(rng.choice([64, 1024, 3072, 7000]))))
    for S, H, KVH, maxc, P, slots in cases:
        want = balanced_units(S, H, KVH, maxc, P, slots) if S > 0 else 0
        got = pkv.pkv_attention_balanced_units(S, H, KVH, maxc, P, slots)
        assert got == want, (S, H, KVH, maxc, P, slots, got, want)
