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
// Partition kernel: one wave per (kv head, segment), a segment being a run
// of whole 64-token blocks of one sequence; a workgroup holds the waves of
// four consecutive kv heads.  The balanced split numbers the blocks of all
// sequences in order and gives every unit of work the same count (so mixed
// context lengths leave no wave with much more to do than the others); the
// fixed split, as on the page, makes one segment per partition of
// partition_size tokens and serves the batches the balanced one cannot
// (one partition of workspace per sequence, very many sequences).  Both
// products are computed
// transposed, S^T = K Q^T and O^T = V^T P^T, on v_mfma_f32_16x16x32_bf16:
// the 16 tokens of an MFMA's rows are chosen so that the logits a lane holds
// afterwards are exactly the probabilities its B operand needs in P.V, so
// the probabilities never leave registers, and each lane owns one query
// head (the G = num_heads/num_kv_heads heads of the kv head are the 16
// columns; columns >= G are zero).  fp8 keys and values become bf16 exactly
// (4 significant bits fit in 8).  The wave walks its partition in blocks of
// 64 tokens: per block each lane issues eight 16-byte key rows (whole-line
// loads, rearranged for the MFMA by DPP row rotations) and eight 16-byte
// value rows (16 KB per wave), and the next block's keys are
// requested as soon as the logits are formed, its values as soon as the P.V
// product has consumed the current ones.  A running softmax per head (the
// maximum reduced over the four lane groups with the gfx950 lane-swap
// instructions, exponentials as exp2 of logits kept in log2(e) units, a
// reference point that moves only when a block exceeds it by more than 2^8)
// turns logits into weights, which enter P.V as a bf16 high part plus the
// bf16 of the exact remainder (16 significant bits).  The segment's
// block-table entries are read once per wave into two registers and looked
// up with v_readlane, so the loop issues no scalar loads.  The wave writes
// the segment's normalised output, exp-sum and maximum to the caller's
// workspace (exp_sums, max_logits, tmp_out), the buffers of the page's
// schema.
//
// A sequence whose context is a single segment gets its output row from the
// partition kernel directly (normalised, rounded to bf16).
//
// Reduce kernel: each (sequence, head) row of the other sequences combines
// its segments' partials:
//   out = sum_p l_p e^(m_p - M) o_p / sum_p l_p e^(m_p - M)
// and rounds to bf16.  A sequence without a valid token gets a zero row;
// tokens whose page id is outside [0, num_blocks) are left out.
#include <atomic>
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

// An MFMA, then a gap: nothing is scheduled across the two barriers,
// and the s_nop between them is 8 wait states, so no later instruction can
// rewrite the MFMA's source or accumulator registers, or read its result,
// sooner than 8 wait states after it issued.  Without the gap the compiler
// lets a key conversion overwrite the chain's previous accumulator register
// 3 wait states after the MFMA that reads it as SrcC (the logits chains
// alternate dst and SrcC between two register quads), the closest its hazard
// model allows for this 4-pass instruction; a build whose K steps were
// interleaved across tiles had the same pattern and gave wrong results that
// depended on timing.  8 wait states is more than twice that distance.  The
// P.V pairs (high then low probability half into one output) alternate the
// same way; there the register the first MFMA frees is the second one's
// destination, so one gap after the pair suffices.
__device__ __forceinline__ void mfma_gap() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7");
  __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ v4f mfma_bf16_gap(const v8bf a, const v8bf b, const v4f c) {
  const v4f d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  mfma_gap();
  return d;
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

__device__ __forceinline__ uint16_t bf16_rn(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// The block-table entries a partition can touch, two per lane: entry
// j0 + lane in .lo and j0 + 64 + lane in .hi, -1 where the column is past the
// row or the page id is outside [0, num_blocks).  A partition of at most 2048
// tokens in pages of at least 16 spans at most 128 entries.  Loaded once per
// wave with vector loads, so that the block loop issues no scalar loads.
struct TableSlice {
  int32_t lo, hi;
};
__device__ __forceinline__ int32_t table_entry(const int32_t* trow, int32_t j,
                                               int32_t max_blocks, int64_t num_blocks) {
  const int32_t pg = j < max_blocks ? trow[j] : -1;
  return (pg >= 0 && pg < num_blocks) ? pg : -1;
}
__device__ __forceinline__ TableSlice load_table_slice(const int32_t* trow, int32_t j0,
                                                       int32_t max_blocks, int64_t num_blocks,
                                                       int lane) {
  return TableSlice{table_entry(trow, j0 + lane, max_blocks, num_blocks),
                    table_entry(trow, j0 + kWave + lane, max_blocks, num_blocks)};
}

// Valid page id of each 16-token tile of the 64-token block starting at
// token tb, or -1 (tile past the context, column past the row, invalid id).
__device__ __forceinline__ void block_pages(const TableSlice& slice, int32_t j0, int32_t tb,
                                            int32_t t_end, const FastDiv& bdiv,
                                            int32_t (&page)[kPaTiles]) {
#pragma unroll
  for (int tt = 0; tt < kPaTiles; ++tt) {
    const int32_t t0 = tb + tt * 16;
    const int32_t j = (int32_t)bdiv.div((uint32_t)(t0 < t_end ? t0 : tb)) - j0;
    const int32_t pg = j < kWave ? __builtin_amdgcn_readlane(slice.lo, j)
                                 : __builtin_amdgcn_readlane(slice.hi, j - kWave);
    page[tt] = t0 < t_end ? pg : -1;
  }
}

// Max over lanes l, l ^ 16, l ^ 32 and l ^ 48 (the four lane groups), by the
// gfx950 lane-swap instructions: after a swap of the odd and even 16-lane rows
// (then of the two halves) between two copies of v, each lane holds its own
// value and its partner's.
__device__ __forceinline__ float group4_max(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = fmaxf(v, fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1])));
  const uint32_t w = __float_as_uint(v);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(v, fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1])));
}

// 8 floats -> bf16 high parts (round to nearest even) and the bf16 of the
// exact remainders, as MFMA operands; element k keeps position k.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ void split_bf16x8(const float (&p)[8], v8bf& hi, v8bf& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    h[k] = pack_bf16x2(p[2 * k], p[2 * k + 1]);
    // p - hi is exact in binary32 (at most 16 significant bits remain)
    l[k] = pack_bf16x2(p[2 * k] - __uint_as_float(h[k] << 16),
                       p[2 * k + 1] - __uint_as_float(h[k] & 0xffff0000u));
  }
  hi = __builtin_bit_cast(v8bf, u32x4{h[0], h[1], h[2], h[3]});
  lo = __builtin_bit_cast(v8bf, u32x4{l[0], l[1], l[2], l[3]});
}

// Key operand of logits MFMA M from whole-line key loads.  kw[tt][h] holds,
// in lane (c, g), the 16-byte key row of token c of tile tt at d/16 = g + 4h;
// MFMA M needs in lane (col, grp) the row of token 4 M + col%4 of tile col/4
// at the same d/16, i.e. lane (4 M + col%4, grp) of kw[col/4][h]: within each
// 16-lane row, bank col/4 (lanes 4 (col/4) .. + 3) rotated by 4 (col/4 - M)
// lanes.  One DPP row rotation per other tile, each writing its own bank.
template <int kTile, int kM>
__device__ __forceinline__ uint32_t bank_from_tile(uint32_t acc, uint32_t src) {
  constexpr int n = (4 * (kTile - kM)) & 15;  // row_ror:n -- lane i takes lane (i - n) mod 16
  return (uint32_t)__builtin_amdgcn_update_dpp((int)acc, (int)src, 0x120 + n, 0xF, 1 << kTile,
                                               false);
}
template <int kM, int kH>
__device__ __forceinline__ uint32_t key_operand_dword(const u32x4 (&kw)[kPaTiles][2], int d) {
  uint32_t x = kw[kM][kH][d];  // bank kM: no rotation
  if constexpr (kM != 0) x = bank_from_tile<0, kM>(x, kw[0][kH][d]);
  if constexpr (kM != 1) x = bank_from_tile<1, kM>(x, kw[1][kH][d]);
  if constexpr (kM != 2) x = bank_from_tile<2, kM>(x, kw[2][kH][d]);
  if constexpr (kM != 3) x = bank_from_tile<3, kM>(x, kw[3][kH][d]);
  return x;
}
template <int kM, int kH>
__device__ __forceinline__ u32x4 key_operand(const u32x4 (&kw)[kPaTiles][2]) {
  return u32x4{key_operand_dword<kM, kH>(kw, 0), key_operand_dword<kM, kH>(kw, 1),
               key_operand_dword<kM, kH>(kw, 2), key_operand_dword<kM, kH>(kw, 3)};
}

// One of four uniform values, chosen by a per-lane index in [0, 4): a select
// chain on the values as scalars (readfirstlane makes them opaque, so the
// selects cannot become an indexed access to the array, which would put the
// array and everything around it in scratch memory).
__device__ __forceinline__ int32_t pick4(const int32_t (&v)[kPaTiles], int idx) {
  const int32_t v0 = __builtin_amdgcn_readfirstlane(v[0]);
  const int32_t v1 = __builtin_amdgcn_readfirstlane(v[1]);
  const int32_t v2 = __builtin_amdgcn_readfirstlane(v[2]);
  const int32_t v3 = __builtin_amdgcn_readfirstlane(v[3]);
  const int32_t lo = (idx & 1) ? v1 : v0;
  const int32_t hi = (idx & 1) ? v3 : v2;
  return (idx & 2) ? hi : lo;
}

// One wave attends one kv head of one sequence over one segment of its
// context: a run of whole 64-token blocks (the last one ragged), at most 2048
// tokens, given by the work split (below).  Waves share nothing: there is
// no barrier and no LDS.
//
// Both products are computed transposed, S^T = K Q^T and O^T = V^T P^T, with
// lane (col, grp) = (lane % 16, lane / 16):
//  - logits, MFMA m of a 64-token block (m = 0..3): A row i is token
//    16 (i/4) + 4m + i%4 (tile i/4 of the block), B column j is query head j
//    of the group; the result gives lane (col, grp) the logits of head col for
//    tokens 16 grp + 4m + r, r = 0..3 -- all in tile grp;
//  - P.V, step s of a block (s = 0, 1): the K index 8 grp + e is token
//    16 grp + 8s + e, so the B operand of lane (col, grp) is exactly the 8
//    probabilities it holds from logits MFMAs 2s and 2s+1, and the A operand
//    (values of d = 16n + col) is bytes 8s..8s+7 of tile grp's row d, one
//    half of the 16-byte row the lane loads;
//  - the result gives lane (col, grp) head col at d = 16n + 4 grp + r.
// Each lane therefore owns one head: its running maximum is a scalar
// (reduced over the four lane groups once per block) and its exp-sum a
// per-lane partial, reduced at the end.
// kB: the page size when it is fixed at compile time (all load offsets are
// then immediates, which keeps the two stages within the register budget of
// two waves per SIMD), 0 for any multiple of 16 given at run time.
template <int kB>
__device__ __forceinline__ void attend_segment(
    uint32_t s, uint32_t kvh, int32_t t_begin, int32_t t_end, const TableSlice& slice, int32_t j0,
    int64_t row, bool direct, uint16_t* __restrict__ out, float* __restrict__ exp_sums,
    float* __restrict__ max_logits, float* __restrict__ tmp_out, const uint16_t* __restrict__ query,
    const uint8_t* __restrict__ key_cache, const uint8_t* __restrict__ value_cache,
    int32_t num_heads, int32_t num_kv_heads, int32_t block_size_arg, FastDiv bdiv, float scale,
    float k_scale, float v_scale) {
  const int32_t block_size = kB ? kB : block_size_arg;
  const int lane = threadIdx.x & (kWave - 1);
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int32_t nblk = (t_end - t_begin + kPaWaveTokens - 1) / kPaWaveTokens;
  const int32_t G = num_heads / num_kv_heads;
  const int64_t kv_head_keys = (int64_t)(kPaD / 16) * block_size * 16;  // bytes per (page, kv head)
  const int64_t kv_head_vals = (int64_t)kPaD * block_size;
  const uint8_t* kbase = key_cache + (int64_t)kvh * kv_head_keys;
  const uint8_t* vbase = value_cache + (int64_t)kvh * kv_head_vals;
  const int64_t kpage = (int64_t)num_kv_heads * kv_head_keys;  // bytes per page, all kv heads
  const int64_t vpage = (int64_t)num_kv_heads * kv_head_vals;

  // ---- query operand (B of the logits): lane (col, grp) holds head col at
  // d = 16 (grp + 4 (c/2)) + 8 (c%2) + e for K step c, the order in which one
  // 16-byte key row feeds it.  Columns past the group read the group's last
  // head and are zeroed.
  const uint16_t* qrow =
      query + ((int64_t)s * num_heads + (int64_t)kvh * G + (col < G ? col : G - 1)) * kPaD;
  u32x4 qv[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
    qv[c] = *reinterpret_cast<const u32x4*>(qrow + 16 * (grp + 4 * (c >> 1)) + 8 * (c & 1));

  // Loads of one 64-token block.  Keys: kw[tt][h] holds in lane (col, grp)
  // the 16-byte key row of token col of tile tt at d/16 = grp + 4h (whole
  // lines; key_operand rearranges them per MFMA).  Values: the 16 tokens of
  // tile grp at d = 16n + col.  Tiles without a valid page read page 0 (in
  // bounds) and are masked when used.
  u32x4 kw[kPaTiles][2];
  u32x4 vw[8];
  auto issue_keys = [&](const int32_t (&pg)[kPaTiles], int32_t tb) {
#pragma unroll
    for (int tt = 0; tt < kPaTiles; ++tt) {
      const int32_t p = pg[tt];
      const uint32_t t0 = (uint32_t)(tb + tt * 16);
      const uint32_t off0 = t0 - bdiv.div(t0) * (uint32_t)block_size;
      const uint8_t* kp = kbase + (int64_t)(p >= 0 ? p : 0) * kpage +
                          ((int64_t)grp * block_size + off0 + col) * 16;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        kw[tt][h] = *reinterpret_cast<const u32x4*>(kp + (int64_t)4 * h * block_size * 16);
    }
  };
  auto issue_values = [&](const int32_t (&pg)[kPaTiles], int32_t tb) {
    const int32_t p = pick4(pg, grp);
    const uint32_t t0 = (uint32_t)(tb + grp * 16);
    const uint8_t* vp = vbase + (int64_t)(p >= 0 ? p : 0) * vpage +
                        (t0 - bdiv.div(t0) * (uint32_t)block_size) + (int64_t)col * block_size;
#pragma unroll
    for (int n = 0; n < 8; ++n)
      vw[n] = *reinterpret_cast<const u32x4*>(vp + (int64_t)16 * n * block_size);
  };

  // ---- prologue: block 0's pages and loads
  int32_t page[kPaTiles];
  block_pages(slice, j0, t_begin, t_end, bdiv, page);
  issue_keys(page, t_begin);
  issue_values(page, t_begin);
  __builtin_amdgcn_sched_barrier(0);  // block 0 is requested before anything waits

  v8bf bq[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    bq[c] = __builtin_bit_cast(v8bf, col < G ? qv[c] : zero);
  }

  // logits in units of log2(e), so that each weight is one hardware exp2
  const float qk_scale = (scale * k_scale) * kLog2e;
  const float neg_inf = -__builtin_inff();
  float m_run = neg_inf;  // reference point of head col
  float l_part = 0.0f;    // exp-sum of head col over this lane's tokens
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
    // every token of the block is inside the context and has a valid page
    const bool full = tb + kPaWaveTokens <= t_end && page[0] >= 0 && page[1] >= 0 &&
                      page[2] >= 0 && page[3] >= 0;

    // ---- logits: lg[m][r] is head col at token 16 grp + 4m + r.  Each
    // tile's four K steps run back to back on one accumulator.  (With the K
    // step as the outer loop, the same arithmetic gave wrong results that
    // depended on timing; the cause was not found, so that order is not used.)
    v4f acc[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[m] = v4f{0.f, 0.f, 0.f, 0.f};
    auto tile_logits = [&](auto mc) {
      constexpr int m = decltype(mc)::value;
      const u32x4 w0 = key_operand<m, 0>(kw);
      acc[m] = mfma_bf16_gap(fp8x8_to_bf16(u32x2{w0.x, w0.y}), bq[0], acc[m]);
      acc[m] = mfma_bf16_gap(fp8x8_to_bf16(u32x2{w0.z, w0.w}), bq[1], acc[m]);
      const u32x4 w1 = key_operand<m, 1>(kw);
      acc[m] = mfma_bf16_gap(fp8x8_to_bf16(u32x2{w1.x, w1.y}), bq[2], acc[m]);
      acc[m] = mfma_bf16_gap(fp8x8_to_bf16(u32x2{w1.z, w1.w}), bq[3], acc[m]);
    };
    tile_logits(std::integral_constant<int, 0>{});
    tile_logits(std::integral_constant<int, 1>{});
    tile_logits(std::integral_constant<int, 2>{});
    tile_logits(std::integral_constant<int, 3>{});
    float lg[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      lg[m][0] = acc[m].x * qk_scale;
      lg[m][1] = acc[m].y * qk_scale;
      lg[m][2] = acc[m].z * qk_scale;
      lg[m][3] = acc[m].w * qk_scale;
    }
    const int32_t live = full ? kPaWaveTokens
                              : (pick4(page, grp) >= 0 ? t_end - (tb + grp * 16) : 0);
    if (!full) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * m + r >= live) lg[m][r] = neg_inf;
    }
    int32_t next_page[kPaTiles];
    if constexpr (kPrefetch) {
      block_pages(slice, j0, tb + kPaWaveTokens, t_end, bdiv, next_page);
      issue_keys(next_page, tb + kPaWaveTokens);
    }

    // ---- softmax reference point of head col.  It only moves when the
    // block's maximum exceeds it by more than 2^kLazy (weights stay <=
    // 2^kLazy), so the output and exp-sum so far are rarely rescaled; the
    // result is the same sum with other intermediate scalings.
    float mx = neg_inf;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      mx = fmaxf(fmaxf(mx, fmaxf(lg[m][0], lg[m][1])), fmaxf(lg[m][2], lg[m][3]));
    mx = group4_max(mx);
    const bool move = mx > m_run + kLazy;
    if (__builtin_amdgcn_ballot_w64(move) != 0) {  // uniform over the wave
      const float m_new = move ? mx : m_run;
      const float alpha = (m_run == neg_inf) ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_part *= alpha;
      m_run = m_new;
#pragma unroll
      for (int n = 0; n < 8; ++n) o[n] *= alpha;
    }
    float e = 0.0f;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = (m_run == neg_inf) ? 0.0f : __builtin_amdgcn_exp2f(lg[m][r] - m_run);
        lg[m][r] = p;
        e += p;
      }
    l_part += e;

    // ---- P.V: value bytes of tokens without a valid page or past the
    // context are zeroed (the page may hold anything there)
    if (!full) {
      u32x4 keep;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int32_t n_live = live - 4 * q;
        keep[q] = n_live >= 4 ? 0xFFFFFFFFu : n_live <= 0 ? 0u : (0xFFFFFFFFu >> (8 * (4 - n_live)));
      }
#pragma unroll
      for (int n = 0; n < 8; ++n) vw[n] &= keep;
    }
#pragma unroll
    for (int sp2 = 0; sp2 < 2; ++sp2) {
      const float p8[8] = {lg[2 * sp2][0],     lg[2 * sp2][1],     lg[2 * sp2][2],
                           lg[2 * sp2][3],     lg[2 * sp2 + 1][0], lg[2 * sp2 + 1][1],
                           lg[2 * sp2 + 1][2], lg[2 * sp2 + 1][3]};
      v8bf bhi, blo;
      split_bf16x8(p8, bhi, blo);
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const u32x4 w = vw[n];
        const v8bf a = fp8x8_to_bf16(sp2 ? u32x2{w.z, w.w} : u32x2{w.x, w.y});
        o[n] = mfma_bf16(a, bhi, o[n]);
        o[n] = mfma_bf16(a, blo, o[n]);
        mfma_gap();
      }
    }
    if constexpr (kPrefetch) {
      __builtin_amdgcn_sched_barrier(0);  // the values are used before they are replaced
      issue_values(next_page, tb + kPaWaveTokens);
#pragma unroll
      for (int tt = 0; tt < kPaTiles; ++tt) page[tt] = next_page[tt];
    }
  };
  for (int32_t b = 0; b + 1 < nblk; ++b) block(b, std::true_type{});
  block(nblk - 1, std::false_type{});

  // ---- normalised output of each real head: the output row itself when the
  // segment is the sequence's whole context, else the segment's partial
  // output, exp-sum and maximum for the reduce kernel
  float l_run = l_part;
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (col < G) {
    const int64_t h = (int64_t)kvh * G + col;
    const float inv = l_run > 0.0f ? v_scale / l_run : 0.0f;
    if (direct) {
      uint16_t* dst = out + ((int64_t)s * num_heads + h) * kPaD + 4 * grp;
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const v4f v = o[n] * inv;
        const u32x2 w = {(uint32_t)bf16_rn(v.x) | ((uint32_t)bf16_rn(v.y) << 16),
                         (uint32_t)bf16_rn(v.z) | ((uint32_t)bf16_rn(v.w) << 16)};
        *reinterpret_cast<u32x2*>(dst + 16 * n) = w;
      }
    } else {
      const int64_t e = row * num_heads + h;
      float* dst = tmp_out + e * kPaD + 4 * grp;
#pragma unroll
      for (int n = 0; n < 8; ++n) *reinterpret_cast<v4f*>(dst + 16 * n) = o[n] * inv;
      if (grp == 0) {
        exp_sums[e] = l_run;
        max_logits[e] = m_run;
      }
    }
  }
}

// ---- Work split.
//
// Fixed split (as on the page): one workgroup per (sequence, partition of
// partition_size tokens, four consecutive kv heads); partition p of
// sequence s has workspace row s * max_parts + p.
template <int kB>
__global__ __launch_bounds__(kPaThreads, 3) void paged_attention_partition_kernel(
    uint32_t num_units, uint16_t* __restrict__ out, float* __restrict__ exp_sums,
    float* __restrict__ max_logits, float* __restrict__ tmp_out, const uint16_t* __restrict__ query,
    const uint8_t* __restrict__ key_cache, const uint8_t* __restrict__ value_cache,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t block_size_arg,
    FastDiv bdiv, int32_t max_blocks, int32_t max_parts, int32_t partition_size,
    int64_t num_blocks, float scale, float k_scale, float v_scale) {
  if (blockIdx.x >= num_units) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform per wave
  // 32-bit index arithmetic: the host bounds the unit count and every token
  // index below 2^31.  Partition-major order: the units of all sequences'
  // first partitions come first.
  const uint32_t groups = ((uint32_t)num_kv_heads + kPaWaves - 1) / kPaWaves;
  const uint32_t kvh = (blockIdx.x % groups) * kPaWaves + wave;
  const uint32_t sp = blockIdx.x / groups;
  const uint32_t s = sp % (uint32_t)num_seqs;
  const uint32_t part = sp / (uint32_t)num_seqs;
  if (kvh >= (uint32_t)num_kv_heads || part >= (uint32_t)max_parts) return;
  const int32_t t_begin = (int32_t)part * partition_size;
  // the table slice does not depend on the context length: both are in
  // flight together
  const int32_t j0 = (int32_t)bdiv.div((uint32_t)t_begin);
  const TableSlice slice =
      load_table_slice(block_tables + (int64_t)s * max_blocks, j0, max_blocks, num_blocks, lane);
  const int32_t L = context_lens[s];
  if (t_begin >= L) return;
  const int32_t nparts = (L - 1) / partition_size + 1 < max_parts ? (L - 1) / partition_size + 1
                                                                   : max_parts;
  const int32_t t_end = (L - t_begin > partition_size) ? t_begin + partition_size : L;
  attend_segment<kB>(s, kvh, t_begin, t_end, slice, j0, (int64_t)s * max_parts + part,
                     nparts == 1, out, exp_sums, max_logits, tmp_out, query, key_cache,
                     value_cache, num_heads, num_kv_heads, block_size_arg, bdiv, scale, k_scale,
                     v_scale);
}

// Balanced split.  With one partition per fixed number of tokens, a batch of
// mixed context lengths gives some waves many more blocks than others, and
// the call lasts as long as the longest.  Here the 64-token blocks of all
// sequences are numbered in sequence order, block j of sequence s being
// number cum(s) + j with cum(s) = sum over s' < s of blocks(s'), N in all,
// and unit u of num_units takes numbers [u W, (u + 1) W), W = ceil(N /
// num_units): every wave gets the same number of blocks, in one or more
// segments (one per sequence its range touches).  Sequence s then has
// partials from units first(s) = floor(cum(s) / W) through last(s) =
// floor((cum(s) + blocks(s) - 1) / W); the partial of unit u goes to
// workspace row u + s, which no other (unit, sequence) pair uses, since
// last(s) <= first(s') for s < s', and rows stay below num_units +
// num_seqs.  The wave of kv head 0 that attends the first block of a
// sequence also records (first(s) + s, last(s) - first(s) + 1) for the
// reduce kernel, as two int32 at exp_sums entries (num_units + num_seqs) *
// num_heads + 2 s and + 1.  The host bounds num_units so that all of it fits
// the caller's [num_seqs, num_heads, max_parts] workspace, and makes W at
// most 32 blocks (2048 tokens, the table slice).  Tokens past token_cap =
// max_parts * partition_size are not read, as in the fixed split.

// 64-token blocks of a context of L tokens of which at most `cap` are read.
__device__ __forceinline__ int32_t seq_blocks(int32_t L, int32_t cap) {
  const int32_t n = L < cap ? L : cap;
  return n > 0 ? (n + kPaWaveTokens - 1) / kPaWaveTokens : 0;
}

// Lane i sums the blocks of sequences [i per, (i + 1) per), per =
// ceil(num_seqs / 64); base is the lane's exclusive prefix of those sums and
// total (uniform) is N.  All lanes must be active.
struct SeqPrefix {
  int32_t per, base, total;
};
__device__ __forceinline__ SeqPrefix seq_prefix(const int32_t* __restrict__ context_lens,
                                                int32_t num_seqs, int32_t cap, int lane) {
  const int32_t per = (num_seqs + kWave - 1) / kWave;
  const int32_t first = lane * per;
  int32_t mine = 0;
  for (int32_t k0 = 0; k0 < per; k0 += 8) {  // eight loads in flight per lane
    int32_t L[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int32_t k = k0 + i;
      L[i] = (k < per && first + k < num_seqs) ? context_lens[first + k] : 0;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) mine += seq_blocks(L[i], cap);
  }
  const int32_t incl = wave_inclusive_scan(mine);
  return SeqPrefix{per, incl - mine, __builtin_amdgcn_readlane(incl, kWave - 1)};
}

// A workgroup per (unit, four consecutive kv heads).
template <int kB>
__global__ __launch_bounds__(kPaThreads, 3) void paged_attention_balanced_kernel(
    uint32_t num_units, uint16_t* __restrict__ out, float* __restrict__ exp_sums,
    float* __restrict__ max_logits, float* __restrict__ tmp_out, const uint16_t* __restrict__ query,
    const uint8_t* __restrict__ key_cache, const uint8_t* __restrict__ value_cache,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t block_size_arg,
    FastDiv bdiv, int32_t max_blocks, int32_t token_cap, int64_t num_blocks, float scale,
    float k_scale, float v_scale) {
  const uint32_t groups = ((uint32_t)num_kv_heads + kPaWaves - 1) / kPaWaves;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform per wave
  const uint32_t u = blockIdx.x / groups;
  const uint32_t kvh = (blockIdx.x % groups) * kPaWaves + wave;
  if (u >= num_units || kvh >= (uint32_t)num_kv_heads) return;
  const SeqPrefix pre = seq_prefix(context_lens, num_seqs, token_cap, lane);
  const int32_t N = pre.total;
  if (N == 0) return;
  const int32_t W = (int32_t)(((int64_t)N + num_units - 1) / num_units);
  const int64_t b0l = (int64_t)u * W;
  if (b0l >= N) return;
  const int32_t b0 = (int32_t)b0l;
  const int32_t b1 = N - b0 > W ? b0 + W : N;

  // first sequence with cum(s) + blocks(s) > b0: the lane range that holds
  // it, then the sequence inside that range
  int32_t s = 0, cum = 0;
  {
    // lane i's range ends at base_i + mine_i; mine_i = base_{i+1} - base_i
    const int32_t end_i = __shfl_down(pre.base, 1);
    const int32_t end = lane == kWave - 1 ? N : end_i;
    const uint64_t m = __builtin_amdgcn_ballot_w64(end > b0);
    const int32_t r = (int32_t)__builtin_ctzll(m);
    const int32_t rbase = __builtin_amdgcn_readlane(pre.base, r);
    const int32_t sq = r * pre.per + lane;
    const int32_t nb = lane < pre.per && sq < num_seqs ? seq_blocks(context_lens[sq], token_cap) : 0;
    const int32_t incl = wave_inclusive_scan(nb);
    const int32_t k = (int32_t)__builtin_ctzll(
        __builtin_amdgcn_ballot_w64(lane < pre.per && rbase + incl > b0));
    s = r * pre.per + k;
    cum = rbase + __builtin_amdgcn_readlane(incl, k) - __builtin_amdgcn_readlane(nb, k);
  }

  // the segments: sequences s, s + 1, ... while their blocks start below b1
  while (cum < b1 && s < num_seqs) {
    const int32_t lo = b0 > cum ? b0 - cum : 0;  // first block of the segment in s
    const int32_t t_begin = lo * kPaWaveTokens;
    const int32_t j0 = (int32_t)bdiv.div((uint32_t)t_begin);
    const TableSlice slice =
        load_table_slice(block_tables + (int64_t)s * max_blocks, j0, max_blocks, num_blocks, lane);
    const int32_t Lraw = context_lens[s];
    const int32_t L = Lraw < token_cap ? Lraw : token_cap;
    const int32_t nb = seq_blocks(L, token_cap);
    if (nb > 0) {
      const int32_t hi = b1 - cum < nb ? b1 - cum : nb;  // end block of the segment in s
      const int32_t t_end = hi * kPaWaveTokens < L ? hi * kPaWaveTokens : L;
      const int32_t first = cum / W;
      const int32_t count = (cum + nb - 1) / W - first + 1;
      if (lo == 0 && kvh == 0 && lane == 0) {
        int32_t* meta = reinterpret_cast<int32_t*>(exp_sums) +
                        ((int64_t)num_units + num_seqs) * num_heads + 2 * (int64_t)s;
        meta[0] = first + s;
        meta[1] = count;
      }
      const bool direct = count == 1;
      attend_segment<kB>(s, kvh, t_begin, t_end, slice, j0, (int64_t)u + s, direct, out,
                         exp_sums, max_logits, tmp_out, query, key_cache, value_cache, num_heads,
                         num_kv_heads, block_size_arg, bdiv, scale, k_scale, v_scale);
    }
    cum += nb;
    ++s;
  }
}

// ---- Reduce: one wave per (sequence, eight heads); lane l takes head
// 8 g + l/8 and the 16 values d = 16 (l%8) + i of it, and walks the head's
// partials itself, four at a time (their exp-sums, maxima and outputs all
// loaded at once), so the combination needs no lane exchange.  Rows of one partial
// (the partition kernel wrote them) are skipped; rows with no valid token
// become zero.  num_units = 0 selects the fixed split.
__global__ __launch_bounds__(kPaThreads) void paged_attention_reduce_kernel(
    uint16_t* __restrict__ out, const float* __restrict__ exp_sums,
    const float* __restrict__ max_logits, const float* __restrict__ tmp_out,
    const int32_t* __restrict__ context_lens, int32_t num_seqs, int32_t num_heads,
    int32_t max_parts, int32_t partition_size, uint32_t num_units, int32_t token_cap) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t hg = ((uint32_t)num_heads + 7) / 8;
  const uint32_t w = blockIdx.x * kPaWaves + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  if (w >= (uint32_t)num_seqs * hg) return;
  const int32_t s = (int32_t)(w / hg);
  const int32_t h = (int32_t)(w % hg) * 8 + (lane >> 3);
  const int sub = lane & 7;
  int64_t r0 = 0;
  int32_t count = 0;
  if (num_units == 0) {
    const int32_t L = context_lens[s];
    count = L > 0 ? (L - 1) / partition_size + 1 : 0;
    if (count > max_parts) count = max_parts;
    r0 = (int64_t)s * max_parts;
  } else {
    // the partition kernel recorded the sequence's rows (only for a
    // sequence with blocks; anything else there is stale)
    const int32_t* meta = reinterpret_cast<const int32_t*>(exp_sums) +
                          ((int64_t)num_units + num_seqs) * num_heads + 2 * (int64_t)s;
    const int32_t m0 = meta[0], m1 = meta[1];
    if (seq_blocks(context_lens[s], token_cap) > 0 && m0 >= 0 && m1 >= 0 &&
        (int64_t)m0 + m1 <= (int64_t)num_units + num_seqs) {
      r0 = m0;
      count = m1;
    }
  }
  if (count == 1) return;  // the partition kernel wrote this row
  if (h >= num_heads) return;
  // four partials at a time, all their loads in flight together; the
  // running maximum M and the sums are rescaled when a group raises M
  const float neg_inf = -__builtin_inff();
  float M = neg_inf;
  float Wsum = 0.0f;
  v4f acc[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f},
                {0.f, 0.f, 0.f, 0.f}};
  for (int32_t p0 = 0; p0 < count; p0 += 4) {
    float es[4], ml[4];
    v4f v[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool in = p0 + j < count;
      const int64_t e = (r0 + (in ? p0 + j : 0)) * num_heads + h;
      const v4f* row = reinterpret_cast<const v4f*>(tmp_out + e * kPaD + 16 * sub);
      es[j] = in ? exp_sums[e] : 0.0f;
      ml[j] = in ? max_logits[e] : neg_inf;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[j][i] = in ? row[i] : v4f{0.f, 0.f, 0.f, 0.f};
    }
    // every partial row read here was written by this call with finite
    // values, so a partial of weight 0 adds exactly 0
    float mg = M;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (es[j] > 0.0f) mg = fmaxf(mg, ml[j]);
    if (mg > M) {
      const float alpha = M == neg_inf ? 0.0f : __builtin_amdgcn_exp2f(M - mg);
      Wsum *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] *= alpha;
      M = mg;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float wp = es[j] > 0.0f ? es[j] * __builtin_amdgcn_exp2f(ml[j] - M) : 0.0f;
      Wsum += wp;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i].x = __builtin_fmaf(wp, v[j][i].x, acc[i].x);
        acc[i].y = __builtin_fmaf(wp, v[j][i].y, acc[i].y);
        acc[i].z = __builtin_fmaf(wp, v[j][i].z, acc[i].z);
        acc[i].w = __builtin_fmaf(wp, v[j][i].w, acc[i].w);
      }
    }
  }
  const float inv = Wsum > 0.0f ? 1.0f / Wsum : 0.0f;
  uint32_t packed[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const v4f v = acc[i] * inv;
    packed[2 * i] = (uint32_t)bf16_rn(v.x) | ((uint32_t)bf16_rn(v.y) << 16);
    packed[2 * i + 1] = (uint32_t)bf16_rn(v.z) | ((uint32_t)bf16_rn(v.w) << 16);
  }
  u32x4* dst = reinterpret_cast<u32x4*>(out + ((int64_t)s * num_heads + h) * kPaD + 16 * sub);
  dst[0] = u32x4{packed[0], packed[1], packed[2], packed[3]};
  dst[1] = u32x4{packed[4], packed[5], packed[6], packed[7]};
}

// Workspace of the allocation-free entry point: one array per GPU, loaded
// with the code object and held until the process ends.  Host code never
// uses its name as an address (on the host it is only a stand-in); the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[PKV_ATTENTION_SCRATCH_BYTES];

// Wave slots of the device for the partition kernels (three waves per SIMD,
// four SIMDs per compute unit), cached per device (threads that race on the
// first call store the same value).
int partition_wave_slots() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256 * 12;
  int slots = cached[dev].load(std::memory_order_relaxed);
  if (slots == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    slots = cus * 12;
    cached[dev].store(slots, std::memory_order_relaxed);
  }
  return slots;
}

}  // namespace

// Device address of this GPU's scratch array (the current device's), looked
// up on the first call on each device and cached; threads that race on the
// first call store the same value.  Returns 0 or a HIP error code.
int attention_scratch(void** ptr) {
  static std::atomic<void*> per_device[64];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= 64) return (int)hipErrorInvalidDevice;
  void* p = per_device[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (p == nullptr) return (int)hipErrorInvalidSymbol;
    per_device[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return 0;
}

// Units of the balanced split, or 0 for the fixed split: the balanced one
// needs more than one partition of workspace per sequence, at most 64 * 64
// sequences (the prefix of their block counts is one lane's range each),
// and room in the workspace for num_units + num_seqs rows and the
// per-sequence records with units of at most 32 blocks.  It aims at one
// wave per wave slot.
static int64_t paged_attention_balanced_units(int32_t num_seqs, int32_t num_heads,
                                              int32_t num_kv_heads, int32_t max_context_len,
                                              int32_t partition_size, int wave_slots) {
  const int64_t max_parts = ((int64_t)max_context_len + partition_size - 1) / partition_size;
  if (max_parts < 2 || num_seqs < 1 || num_seqs > kWave * kWave) return 0;
  const int64_t cap_blocks = max_parts * partition_size / kPaWaveTokens;
  const int64_t n_max = (int64_t)num_seqs * cap_blocks;
  if (n_max >= INT32_MAX) return 0;
  const int64_t u_min = (n_max + 31) / 32;
  // rows num_units + num_seqs, then two int32 per sequence
  const int64_t u_cap = (int64_t)num_seqs * (max_parts - 1) -
                        (2 * (int64_t)num_seqs + num_heads - 1) / num_heads;
  if (u_cap < u_min) return 0;
  const int64_t groups = (num_kv_heads + kPaWaves - 1) / kPaWaves;
  const int64_t active = num_kv_heads < kPaWaves ? num_kv_heads : kPaWaves;
  int64_t u = (wave_slots + groups * active - 1) / (groups * active);
  if (u < u_min) u = u_min;
  if (u > u_cap) u = u_cap;
  if (u * groups >= INT32_MAX) return 0;
  return u;
}

int64_t attention_balanced_units(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t max_context_len, int32_t partition_size,
                                 int32_t wave_slots) {
  return paged_attention_balanced_units(num_seqs, num_heads, num_kv_heads, max_context_len,
                                        partition_size, wave_slots);
}

int launch_paged_attention_decode(const PagedAttentionArgs& a, hipStream_t stream) {
  const int32_t P = a.partition_size;
  const int32_t max_parts = (a.max_context_len + P - 1) / P;
  const int32_t token_cap = max_parts * P;
  const int64_t groups = (a.num_kv_heads + kPaWaves - 1) / kPaWaves;
  const int64_t bal = paged_attention_balanced_units(a.num_seqs, a.num_heads, a.num_kv_heads,
                                                     a.max_context_len, P, partition_wave_slots());
  const FastDiv bdiv = FastDiv::make((uint32_t)a.block_size);
  if (bal > 0) {
    auto kernel = a.block_size == 16 ? paged_attention_balanced_kernel<16>
                                     : paged_attention_balanced_kernel<0>;
    hipLaunchKernelGGL(kernel, dim3((unsigned)(bal * groups)), dim3(kPaThreads), 0, stream,
                       (uint32_t)bal, a.out, a.exp_sums, a.max_logits, a.tmp_out, a.query,
                       a.key_cache, a.value_cache, a.block_tables, a.context_lens, a.num_seqs,
                       a.num_heads, a.num_kv_heads, a.block_size, bdiv, a.max_blocks_per_seq,
                       token_cap, a.num_blocks, a.scale, a.k_scale, a.v_scale);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
  } else {
    const int64_t units = (int64_t)a.num_seqs * max_parts * groups;
    if (units > 0) {
      auto kernel = a.block_size == 16 ? paged_attention_partition_kernel<16>
                                       : paged_attention_partition_kernel<0>;
      hipLaunchKernelGGL(kernel, dim3((unsigned)units), dim3(kPaThreads), 0, stream,
                         (uint32_t)units, a.out, a.exp_sums, a.max_logits, a.tmp_out, a.query,
                         a.key_cache, a.value_cache, a.block_tables, a.context_lens, a.num_seqs,
                         a.num_heads, a.num_kv_heads, a.block_size, bdiv, a.max_blocks_per_seq,
                         max_parts, P, a.num_blocks, a.scale, a.k_scale, a.v_scale);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return (int)e;
    }
  }
  const int64_t waves = (int64_t)a.num_seqs * ((a.num_heads + 7) / 8);
  hipLaunchKernelGGL(paged_attention_reduce_kernel, dim3((unsigned)((waves + kPaWaves - 1) / kPaWaves)),
                     dim3(kPaThreads), 0, stream, a.out, a.exp_sums, a.max_logits, a.tmp_out,
                     a.context_lens, a.num_seqs, a.num_heads, max_parts, P, (uint32_t)bal,
                     token_cap);
  return (int)hipGetLastError();
}

}  // namespace pkv
