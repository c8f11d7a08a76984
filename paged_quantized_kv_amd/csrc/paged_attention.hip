// Paged decode attention over fp8 pages (vLLM PR "[ROCm] Faster Custom Paged
// Attention kernels": the op paged_attention(out, exp_sums, max_logits,
// tmp_out, query, key_cache, value_cache, num_kv_heads, scale, block_tables,
// context_lens, block_size, max_context_len, ..., kv_cache_dtype, k_scale,
// v_scale, ..., partition_size) for fp8 caches with per-tensor scales).
// The page's kernel is built on 16x16x16 MFMA for MI300X; this is a gfx950
// design of the same contract:
//
//   out[s, h] = sum_t softmax_t(scale * q[s,h] . k_t) v_t,
//   k_t = E4M3dec(key_cache[page][kvh][d/16][t%B][d%16]) * k_scale,
//   v_t = E4M3dec(value_cache[page][kvh][d][t%B]) * v_scale,
//   page = block_tables[s][t/B], kvh = h / (num_heads / num_kv_heads).
//
// Partition kernel: one wave per (sequence, kv head, partition of
// partition_size tokens); a workgroup holds the waves of four consecutive kv
// heads of one (sequence, partition).  The G = num_heads/num_kv_heads query
// heads of the kv head are the 16 rows of v_mfma_f32_16x16x32_bf16 operands
// (rows >= G are zero); fp8 keys and values become bf16 exactly (4
// significant bits fit in 8).  The wave walks its partition in blocks of 64
// tokens: per block each lane issues two 16-byte key rows and eight 16-byte
// value rows (16 KB per wave), and the next block's keys are requested as
// soon as the logits are formed, its values as soon as the P.V product has
// consumed the current ones, so one block is always in flight.  The
// contractions run in the order those loads deliver: over d, chunk c takes
// d = 16 (grp + 4 (c/2)) + 8 (c%2) + e (the query operand is loaded in the
// same order); over tokens, the k index 8 grp + e of MFMA h is token
// 16 grp + 8 h + e.  Per 16-token tile (inside one page: block_size is a
// multiple of 16) 4 MFMAs give the 16 x 16 logits; a running softmax (row
// maxima and sums by DPP within 16-lane rows, exponentials as exp2 of logits
// kept in log2(e) units, a reference point that moves only when a block
// exceeds it by more than 2^8) turns them into weights, which go through a
// wave-private LDS slice (to operand order) as a bf16 high part plus the
// bf16 of the exact remainder (16 significant bits); 4 MFMAs per 16 values
// of d give the 16 x 128 partial output.  The wave writes the partition's
// normalised output, exp-sum and maximum to the caller's workspace
// (exp_sums, max_logits, tmp_out), as the page's schema does.
//
// Reduce kernel: one wave per (sequence, head) combines the partitions:
//   out = sum_p l_p e^(m_p - M) o_p / sum_p l_p e^(m_p - M)
// and rounds to bf16.  A sequence without a valid token gets a zero row;
// tokens whose page id is outside [0, num_blocks) are left out.
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "pkv.h"

namespace pkv {

namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kPaThreads = 256;
constexpr int kPaWaves = kPaThreads / kWave;
constexpr int kPaD = 128;        // head_size
constexpr int kPaWaveTokens = 64;  // tokens per wave in the partition kernel
constexpr int kPaTiles = kPaWaveTokens / 16;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLazy = 8.0f;  // log2 of the largest weight before a rescale

__device__ __forceinline__ v4f mfma_bf16(const v8bf a, const v8bf b, const v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 8 E4M3 codes (little-endian in two dwords) -> 8 bf16, exact: the gfx950
// scaled converter with unit scale, two codes per instruction (every E4M3
// value has at most 4 significant bits and lies in bf16's range).
__device__ __forceinline__ v8bf fp8x8_to_bf16(u32x2 w) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, true);
  return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Lane exchange inside rows of 16 lanes by DPP (no LDS round trip).
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}
// Max / sum over the 16 lanes of each row: swap neighbours, swap pairs
// (quad permutations), then the mirrored lane of the half row and of the
// row, which pairs up the quads and then the halves.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
constexpr int kDppMirror = 0x140;     // row_mirror
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp<kDppXor1>(v));
  v = fmaxf(v, dpp<kDppXor2>(v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v));
  return fmaxf(v, dpp<kDppMirror>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  return v + dpp<kDppMirror>(v);
}

__device__ __forceinline__ uint16_t bf16_rn(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// Pages of the four 16-token tiles of the 64-token block starting at token
// tb: table entries read without branches (column clamped into the row), so
// that the four scalar reads are in flight together.
struct BlockTable {
  int32_t e[kPaTiles];
};

__device__ __forceinline__ BlockTable read_block_table(const int32_t* trow, int32_t max_blocks,
                                                       const FastDiv& bdiv, int32_t tb) {
  BlockTable t;
  const int32_t jmax = max_blocks > 0 ? max_blocks - 1 : 0;
#pragma unroll
  for (int tt = 0; tt < kPaTiles; ++tt) {
    const int32_t j = (int32_t)bdiv.div((uint32_t)(tb + tt * 16));
    t.e[tt] = max_blocks > 0 ? trow[j < jmax ? j : jmax] : -1;
  }
  return t;
}

// Valid page id of each tile, or -1 (tile past the context, column past the
// row, id outside [0, num_blocks)).
__device__ __forceinline__ void block_pages(const BlockTable& t, int32_t tb, int32_t t_end,
                                            int32_t max_blocks, const FastDiv& bdiv,
                                            int64_t num_blocks, int32_t (&page)[kPaTiles]) {
#pragma unroll
  for (int tt = 0; tt < kPaTiles; ++tt) {
    const int32_t t0 = tb + tt * 16;
    const int32_t j = (int32_t)bdiv.div((uint32_t)t0);
    const int32_t pg = t.e[tt];
    page[tt] = (t0 < t_end && j < max_blocks && pg >= 0 && pg < num_blocks) ? pg : -1;
  }
}

// One wave per (sequence, kv head, partition); a workgroup holds the waves of
// four consecutive kv heads of one (sequence, partition), so that all of
// them have work or none has.  There is no barrier: waves only share the
// workgroup's LDS through disjoint slices.
__global__ __launch_bounds__(kPaThreads) void paged_attention_partition_kernel(
    float* __restrict__ exp_sums, float* __restrict__ max_logits, float* __restrict__ tmp_out,
    const uint16_t* __restrict__ query, const uint8_t* __restrict__ key_cache,
    const uint8_t* __restrict__ value_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t block_size, FastDiv bdiv, int32_t max_blocks, int32_t max_parts,
    int32_t partition_size, int64_t num_blocks, float scale, float k_scale, float v_scale) {
  constexpr int kPRow = kPaWaveTokens + 8;  // u16 per probability row
  __shared__ __align__(16) uint16_t p_lds[kPaWaves][2][16][kPRow];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform per wave
  const int col = lane & 15;  // operand row / result column
  const int grp = lane >> 4;  // K quarter / result row quarter
  // 32-bit index arithmetic: the host bounds the grid and every token index
  // below 2^31.  Partition-major order: the workgroups of all sequences'
  // first partitions come first.
  const uint32_t groups = ((uint32_t)num_kv_heads + kPaWaves - 1) / kPaWaves;
  const uint32_t unit = blockIdx.x;
  const uint32_t kvh = (unit % groups) * kPaWaves + wave;
  const uint32_t sp = unit / groups;
  const uint32_t s = sp % (uint32_t)num_seqs;
  const uint32_t part = sp / (uint32_t)num_seqs;
  if (kvh >= (uint32_t)num_kv_heads || part >= (uint32_t)max_parts) return;
  const int32_t L = context_lens[s];
  const int32_t t_begin = (int32_t)part * partition_size;
  if (t_begin >= L) return;
  const int32_t t_end = (L - t_begin > partition_size) ? t_begin + partition_size : L;
  const int32_t nblk = (t_end - t_begin + kPaWaveTokens - 1) / kPaWaveTokens;
  const int32_t G = num_heads / num_kv_heads;
  const int32_t* trow = block_tables + (int64_t)s * max_blocks;
  const int64_t kv_head_keys = (int64_t)(kPaD / 16) * block_size * 16;  // bytes per (page, kv head)
  const int64_t kv_head_vals = (int64_t)kPaD * block_size;
  const uint8_t* kbase = key_cache + (int64_t)kvh * kv_head_keys;
  const uint8_t* vbase = value_cache + (int64_t)kvh * kv_head_vals;
  const int64_t kpage = (int64_t)num_kv_heads * kv_head_keys;  // bytes per page, all kv heads
  const int64_t vpage = (int64_t)num_kv_heads * kv_head_vals;

  // ---- query rows: chunk c of the contraction takes d = 16 (grp + 4 (c/2)) +
  // 8 (c%2) + e, the order in which one 16-byte key row feeds it.  Rows past
  // the group read the group's last head and are zeroed when used.
  const uint16_t* qrow =
      query + ((int64_t)s * num_heads + (int64_t)kvh * G + (col < G ? col : G - 1)) * kPaD;
  u32x4 qv[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
    qv[c] = *reinterpret_cast<const u32x4*>(qrow + 16 * (grp + 4 * (c >> 1)) + 8 * (c & 1));

  // Loads of one 64-token block.  Keys: lane (col, grp) holds rows grp and
  // grp + 4 of token col of each tile.  Values: the 16 tokens of tile grp for
  // d = 16n + col.  Tiles without a valid page read page 0 (in bounds) and
  // are masked when used.
  u32x4 kw[kPaTiles][2];
  u32x4 vw[8];
  auto issue_keys = [&](const int32_t (&pg)[kPaTiles], int32_t tb) {
#pragma unroll
    for (int tt = 0; tt < kPaTiles; ++tt) {
      const uint32_t t0 = (uint32_t)(tb + tt * 16);
      const int32_t off0 = (int32_t)(t0 - bdiv.div(t0) * (uint32_t)block_size);
      const uint8_t* kp = kbase + (int64_t)(pg[tt] >= 0 ? pg[tt] : 0) * kpage;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        kw[tt][h] = *reinterpret_cast<const u32x4*>(
            kp + ((int64_t)(grp + 4 * h) * block_size + off0 + col) * 16);
    }
  };
  // page of tile grp, by masks: a select chain on grp would be turned into an
  // indexed (scratch) access to the array
  const uint32_t sel0 = 0u - (uint32_t)(grp == 0), sel1 = 0u - (uint32_t)(grp == 1);
  const uint32_t sel2 = 0u - (uint32_t)(grp == 2), sel3 = 0u - (uint32_t)(grp == 3);
  auto lane_page = [&](const int32_t (&pg)[kPaTiles]) {
    return (int32_t)(((uint32_t)pg[0] & sel0) | ((uint32_t)pg[1] & sel1) |
                     ((uint32_t)pg[2] & sel2) | ((uint32_t)pg[3] & sel3));
  };
  auto issue_values = [&](const int32_t (&pg)[kPaTiles], int32_t tb) {
    const int32_t pv = lane_page(pg);
    const uint32_t t0 = (uint32_t)(tb + grp * 16);
    const uint8_t* vp = vbase + (int64_t)(pv >= 0 ? pv : 0) * vpage +
                        (t0 - bdiv.div(t0) * (uint32_t)block_size);
#pragma unroll
    for (int n = 0; n < 8; ++n)
      vw[n] = *reinterpret_cast<const u32x4*>(vp + (int64_t)(16 * n + col) * block_size);
  };

  // ---- prologue: block 0's pages and loads; block 1's table entries
  int32_t page[kPaTiles];
  {
    const BlockTable t0 = read_block_table(trow, max_blocks, bdiv, t_begin);
    block_pages(t0, t_begin, t_end, max_blocks, bdiv, num_blocks, page);
  }
  issue_keys(page, t_begin);
  issue_values(page, t_begin);
  BlockTable next_tbl = read_block_table(trow, max_blocks, bdiv, t_begin + kPaWaveTokens);
  __builtin_amdgcn_sched_barrier(0);  // block 0 is requested before anything waits

  v8bf aq[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    aq[c] = __builtin_bit_cast(v8bf, col < G ? qv[c] : zero);
  }

  // logits in units of log2(e), so that each weight is one hardware exp2
  const float qk_scale = (scale * k_scale) * kLog2e;
  const float neg_inf = -__builtin_inff();
  float m_run[4] = {neg_inf, neg_inf, neg_inf, neg_inf};
  float l_run[4] = {0.f, 0.f, 0.f, 0.f};
  v4f o[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) o[n] = v4f{0.f, 0.f, 0.f, 0.f};

  // One block: logits, running softmax, P.V.  With kPrefetch the next
  // block's keys are requested as soon as the key registers are free and its
  // values as soon as the value registers are; the last block is peeled off
  // so that every iteration of the loop issues the same loads (the waits
  // then keep exactly the newest block in flight).
  auto block = [&](int32_t b, auto prefetch) {
    constexpr bool kPrefetch = decltype(prefetch)::value;
    const int32_t tb = t_begin + b * kPaWaveTokens;
    BlockTable tbl2;
    if constexpr (kPrefetch)  // table entries two blocks ahead
      tbl2 = read_block_table(trow, max_blocks, bdiv, tb + 2 * kPaWaveTokens);

    // ---- logits of the block: lane holds token col of each tile, heads 4*grp + r
    float lg[kPaTiles][4];
#pragma unroll
    for (int tt = 0; tt < kPaTiles; ++tt) {
      v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x4 w = kw[tt][c >> 1];
        const u32x2 half = (c & 1) ? u32x2{w.z, w.w} : u32x2{w.x, w.y};
        acc = mfma_bf16(aq[c], fp8x8_to_bf16(half), acc);
      }
      const bool valid = page[tt] >= 0 && tb + tt * 16 + col < t_end;
      lg[tt][0] = valid ? acc.x * qk_scale : neg_inf;
      lg[tt][1] = valid ? acc.y * qk_scale : neg_inf;
      lg[tt][2] = valid ? acc.z * qk_scale : neg_inf;
      lg[tt][3] = valid ? acc.w * qk_scale : neg_inf;
    }
    int32_t next_page[kPaTiles];
    if constexpr (kPrefetch) {
      block_pages(next_tbl, tb + kPaWaveTokens, t_end, max_blocks, bdiv, num_blocks, next_page);
      issue_keys(next_page, tb + kPaWaveTokens);
    }

    // ---- softmax reference point per head.  It only moves when the block's
    // maximum exceeds it by more than 2^kLazy (weights stay <= 2^kLazy), so
    // the output and exp-sum so far are rarely rescaled; the result is the
    // same sum with other intermediate scalings.
    float m_blk[4];
    bool move = false;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v = neg_inf;
#pragma unroll
      for (int tt = 0; tt < kPaTiles; ++tt) v = fmaxf(v, lg[tt][r]);
      m_blk[r] = row16_max(v);
      move |= m_blk[r] > m_run[r] + kLazy;
    }
    if (__builtin_amdgcn_ballot_w64(move) != 0) {  // uniform over the wave
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float m_new = m_blk[r] > m_run[r] + kLazy ? m_blk[r] : m_run[r];
        const float alpha =
            (m_run[r] == neg_inf) ? 0.0f : __builtin_amdgcn_exp2f(m_run[r] - m_new);
        l_run[r] *= alpha;
        m_run[r] = m_new;
#pragma unroll
        for (int n = 0; n < 8; ++n) o[n][r] *= alpha;
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float e = 0.0f;
#pragma unroll
      for (int tt = 0; tt < kPaTiles; ++tt) {
        const float p = (m_run[r] == neg_inf) ? 0.0f : __builtin_amdgcn_exp2f(lg[tt][r] - m_run[r]);
        lg[tt][r] = p;
        e += p;
      }
      l_run[r] += row16_sum(e);
    }

    // ---- probabilities to operand order through the wave's LDS slice, as a
    // bf16 high part and the bf16 of the (exact) remainder
#pragma unroll
    for (int tt = 0; tt < kPaTiles; ++tt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = lg[tt][r];
        const uint16_t hi = bf16_rn(p);
        p_lds[wave][0][4 * grp + r][16 * tt + col] = hi;
        p_lds[wave][1][4 * grp + r][16 * tt + col] =
            bf16_rn(p - __uint_as_float((uint32_t)hi << 16));
      }
    }
    wave_sync();
    // MFMA h of a d block takes K index 8*grp + e as token 16*grp + 8*h + e:
    // probabilities from LDS, values from byte 8*h + e of the lane's 16.
    v8bf ap[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int x = 0; x < 2; ++x)
        ap[h][x] = __builtin_bit_cast(
            v8bf, *reinterpret_cast<const u32x4*>(&p_lds[wave][x][col][16 * grp + 8 * h]));
    wave_sync();  // the next block rewrites the slice

    // value bytes of tokens without a valid page or past the context: zero
    const int32_t live = lane_page(page) >= 0 ? t_end - (tb + grp * 16) : 0;
    u32x4 keep;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int32_t n_live = live - 4 * q;
      keep[q] = n_live >= 4 ? 0xFFFFFFFFu : n_live <= 0 ? 0u : (0xFFFFFFFFu >> (8 * (4 - n_live)));
    }
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const u32x4 w = vw[n] & keep;
      const v8bf b0 = fp8x8_to_bf16(u32x2{w.x, w.y});
      const v8bf b1 = fp8x8_to_bf16(u32x2{w.z, w.w});
      o[n] = mfma_bf16(ap[0][0], b0, o[n]);
      o[n] = mfma_bf16(ap[0][1], b0, o[n]);
      o[n] = mfma_bf16(ap[1][0], b1, o[n]);
      o[n] = mfma_bf16(ap[1][1], b1, o[n]);
    }
    if constexpr (kPrefetch) {
      __builtin_amdgcn_sched_barrier(0);  // the values are used before they are replaced
      issue_values(next_page, tb + kPaWaveTokens);
#pragma unroll
      for (int tt = 0; tt < kPaTiles; ++tt) page[tt] = next_page[tt];
      next_tbl = tbl2;
    }
  };
  for (int32_t b = 0; b + 1 < nblk; ++b) block(b, std::true_type{});
  block(nblk - 1, std::false_type{});

  // ---- normalised partial output, exp-sum and maximum of each real head
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * grp + r;
    if (row >= G) continue;
    const int64_t sh = (int64_t)s * num_heads + (int64_t)kvh * G + row;
    const float inv = l_run[r] > 0.0f ? v_scale / l_run[r] : 0.0f;
    float* dst = tmp_out + (sh * max_parts + part) * kPaD;
#pragma unroll
    for (int n = 0; n < 8; ++n) dst[16 * n + col] = o[n][r] * inv;
    if (col == 0) {
      exp_sums[sh * max_parts + part] = l_run[r];
      max_logits[sh * max_parts + part] = m_run[r];
    }
  }
}

// One wave per (sequence, head): lanes take the partitions' exp-sums and
// maxima in parallel, then the weighted partial outputs (two d per lane).
__global__ __launch_bounds__(kPaThreads) void paged_attention_reduce_kernel(
    uint16_t* __restrict__ out, const float* __restrict__ exp_sums,
    const float* __restrict__ max_logits, const float* __restrict__ tmp_out,
    const int32_t* __restrict__ context_lens, int32_t num_seqs, int32_t num_heads,
    int32_t max_parts, int32_t partition_size) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t sh = blockIdx.x * kPaWaves + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  if (sh >= (uint32_t)num_seqs * (uint32_t)num_heads) return;
  const uint32_t s = sh / (uint32_t)num_heads;
  const int32_t L = context_lens[s];
  int32_t nparts = L > 0 ? (L - 1) / partition_size + 1 : 0;
  if (nparts > max_parts) nparts = max_parts;
  const float* es = exp_sums + (int64_t)sh * max_parts;
  const float* ml = max_logits + (int64_t)sh * max_parts;
  const float neg_inf = -__builtin_inff();
  float M = neg_inf;
  for (int32_t b = 0; b < nparts; b += kWave) {
    const int32_t p = b + lane;
    if (p < nparts && es[p] > 0.0f) M = fmaxf(M, ml[p]);
  }
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) M = fmaxf(M, __shfl_xor(M, d));
  float W = 0.0f, a0 = 0.0f, a1 = 0.0f;
  const float* o = tmp_out + (int64_t)sh * max_parts * kPaD + 2 * lane;
  for (int32_t b = 0; b < nparts; b += kWave) {
    const int32_t p = b + lane;
    float wl = 0.0f;
    if (p < nparts && es[p] > 0.0f) wl = es[p] * __builtin_amdgcn_exp2f(ml[p] - M);
    W += wl;
    const int cnt = nparts - b < kWave ? nparts - b : kWave;
    // every partition row below nparts was written by this call, with
    // finite values, so rows of weight 0 add exactly 0
    int i = 0;
    for (; i + 8 <= cnt; i += 8) {  // eight rows in flight
      f32x2 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const f32x2*>(o + (int64_t)(b + i + u) * kPaD);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float w = __shfl(wl, i + u);
        a0 = __builtin_fmaf(w, v[u].x, a0);
        a1 = __builtin_fmaf(w, v[u].y, a1);
      }
    }
    for (; i < cnt; ++i) {
      const float w = __shfl(wl, i);
      const f32x2 v = *reinterpret_cast<const f32x2*>(o + (int64_t)(b + i) * kPaD);
      a0 = __builtin_fmaf(w, v.x, a0);
      a1 = __builtin_fmaf(w, v.y, a1);
    }
  }
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) W += __shfl_xor(W, d);
  const float inv = W > 0.0f ? 1.0f / W : 0.0f;
  const uint32_t packed = (uint32_t)bf16_rn(a0 * inv) | ((uint32_t)bf16_rn(a1 * inv) << 16);
  *reinterpret_cast<uint32_t*>(out + (int64_t)sh * kPaD + 2 * lane) = packed;
}

}  // namespace

int launch_paged_attention_decode(const PagedAttentionArgs& a, hipStream_t stream) {
  const int32_t P = a.partition_size;
  const int32_t max_parts = (a.max_context_len + P - 1) / P;
  const int64_t groups = (a.num_kv_heads + kPaWaves - 1) / kPaWaves;
  const int64_t units = (int64_t)a.num_seqs * max_parts * groups;
  if (units > 0) {
    hipLaunchKernelGGL(paged_attention_partition_kernel, dim3((unsigned)units), dim3(kPaThreads), 0,
                       stream, a.exp_sums, a.max_logits, a.tmp_out, a.query, a.key_cache,
                       a.value_cache, a.block_tables, a.context_lens, a.num_seqs, a.num_heads,
                       a.num_kv_heads, a.block_size, FastDiv::make((uint32_t)a.block_size),
                       a.max_blocks_per_seq, max_parts, P, a.num_blocks, a.scale, a.k_scale,
                       a.v_scale);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
  }
  const int64_t rows = (int64_t)a.num_seqs * a.num_heads;
  hipLaunchKernelGGL(paged_attention_reduce_kernel, dim3((unsigned)((rows + kPaWaves - 1) / kPaWaves)),
                     dim3(kPaThreads), 0, stream, a.out, a.exp_sums, a.max_logits, a.tmp_out,
                     a.context_lens, a.num_seqs, a.num_heads, max_parts, P);
  return (int)hipGetLastError();
}

}  // namespace pkv
