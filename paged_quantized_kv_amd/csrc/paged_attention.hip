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
// Partition kernel: one workgroup per (sequence, kv head, partition of
// partition_size tokens), partition_size / 64 waves of 64 tokens each.  The
// G = num_heads/num_kv_heads query heads of the kv head are the 16 rows of
// v_mfma_f32_16x16x32_bf16 operands (rows >= G are zero); fp8 keys and values
// become bf16 exactly (4 significant bits fit in 8).  A wave first issues
// every load it needs -- two 16-byte key rows and eight 16-byte value rows
// per lane, 16 KB per wave -- so that its whole share of the pages is in
// flight at once, then computes.  The contractions run in the order those
// loads deliver: over d, chunk c takes d = 16 (grp + 4 (c/2)) + 8 (c%2) + e
// (the query operand is loaded in the same order); over tokens, the k index
// 8 grp + e of MFMA h is token 16 grp + 8 h + e.  Per 16-token tile (inside
// one page: block_size is a multiple of 16) 4 MFMAs give the 16 x 16 logits;
// after the wave's max and exp-sum per head, the probabilities go through a
// wave-private LDS slice (to operand order) as a bf16 high part plus the bf16
// of the exact remainder (16 significant bits), and 4 MFMAs per 16 values of
// d give the 16 x 128 partial output.  The waves then meet in LDS: common
// maximum, rescaled exp-sums, summed outputs; the workgroup writes the
// partition's normalised output, exp-sum and maximum to the caller's
// workspace (exp_sums, max_logits, tmp_out), as the page's schema does.
//
// Reduce kernel: one wave per (sequence, head) combines the partitions:
//   out = sum_p l_p e^(m_p - M) o_p / sum_p l_p e^(m_p - M)
// and rounds to bf16.  A sequence without a valid token gets a zero row;
// tokens whose page id is outside [0, num_blocks) are left out.
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

__device__ __forceinline__ v4f mfma_bf16(const v8bf a, const v8bf b, const v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 8 E4M3 codes (little-endian in two dwords) -> 8 bf16, exact.
__device__ __forceinline__ v8bf fp8x8_to_bf16(u32x2 w) {
  const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, false);
  const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, true);
  const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, false);
  const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, true);
  // a binary32 value with at most 8 significant bits is its own top half
  v8bf r;
  r[0] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(a.x) >> 16));
  r[1] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(a.y) >> 16));
  r[2] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(b.x) >> 16));
  r[3] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(b.y) >> 16));
  r[4] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(c.x) >> 16));
  r[5] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(c.y) >> 16));
  r[6] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(d.x) >> 16));
  r[7] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(d.y) >> 16));
  return r;
}

// Max / sum over the 16 lanes of each lane row (lanes 16g .. 16g+15).
__device__ __forceinline__ float row16_max(float v) {
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) v = fmaxf(v, __shfl_xor(v, d));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) v += __shfl_xor(v, d);
  return v;
}

__device__ __forceinline__ uint16_t bf16_rn(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

template <int kWaves>  // partition_size / 64
__global__ __launch_bounds__(kWaves * kWave) void paged_attention_partition_kernel(
    float* __restrict__ exp_sums, float* __restrict__ max_logits, float* __restrict__ tmp_out,
    const uint16_t* __restrict__ query, const uint8_t* __restrict__ key_cache,
    const uint8_t* __restrict__ value_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t block_size, int32_t max_blocks, int32_t max_parts,
    int64_t num_blocks, float scale, float k_scale, float v_scale) {
  constexpr int P = kWaves * kPaWaveTokens;
  constexpr int kPRow = kPaWaveTokens + 8;                // u16 per probability row
  constexpr int kPBytes = kWaves * 2 * 16 * kPRow * 2;    // hi and lo, per wave
  constexpr int kORow = kPaD + 4;                         // floats per output row
  constexpr int kOBytes = kWaves * 16 * kORow * 4;        // partial outputs, per wave
  // The probability slices are dead once the P.V products are done; the
  // partial outputs reuse the same bytes after the first barrier.
  __shared__ __align__(16) unsigned char lds[kPBytes > kOBytes ? kPBytes : kOBytes];
  __shared__ float m_lds[kWaves][16], l_lds[kWaves][16];
  uint16_t(*p_lds)[2][16][kPRow] = reinterpret_cast<uint16_t(*)[2][16][kPRow]>(lds);
  float(*o_lds)[16][kORow] = reinterpret_cast<float(*)[16][kORow]>(lds);

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform per wave
  const int col = lane & 15;  // operand row / result column
  const int grp = lane >> 4;  // K quarter / result row quarter
  // 32-bit index arithmetic: the host bounds the grid and every token index
  // below 2^31.
  const uint32_t unit = blockIdx.x;
  const uint32_t part = unit % (uint32_t)max_parts;
  const uint32_t kvh = (unit / (uint32_t)max_parts) % (uint32_t)num_kv_heads;
  const uint32_t s = unit / ((uint32_t)max_parts * (uint32_t)num_kv_heads);
  if (s >= (uint32_t)num_seqs) return;
  const int32_t L = context_lens[s];
  const int32_t t_begin = (int32_t)part * P;
  if (t_begin >= L) return;  // uniform over the workgroup: no barrier is skipped by some waves only
  const int32_t t_end = (L - t_begin > P) ? t_begin + P : L;
  const int32_t G = num_heads / num_kv_heads;
  const int32_t tw = t_begin + wave * kPaWaveTokens;  // this wave's first token

  // ---- query operands.  The contraction over d runs in the order that one
  // 16-byte key row feeds: chunk c takes d = 16 (grp + 4 (c/2)) + 8 (c%2) + e.
  // Rows past the group read the group's last head and are zeroed after.
  const uint16_t* qrow =
      query + ((int64_t)s * num_heads + (int64_t)kvh * G + (col < G ? col : G - 1)) * kPaD;
  u32x4 qv[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
    qv[c] = *reinterpret_cast<const u32x4*>(qrow + 16 * (grp + 4 * (c >> 1)) + 8 * (c & 1));

  // ---- page of each of the wave's tiles (-1: no valid token in it).  The
  // table entries are read without branches (column clamped into the row)
  // so that the four reads are in flight together.
  int32_t page[kPaTiles];  // table entries are int32: valid ids fit
  int32_t tbl[kPaTiles];
  const int32_t* trow = block_tables + (int64_t)s * max_blocks;
  const int32_t jmax = max_blocks > 0 ? max_blocks - 1 : 0;
#pragma unroll
  for (int tt = 0; tt < kPaTiles; ++tt) {
    const int32_t j = (int32_t)((uint32_t)(tw + tt * 16) / (uint32_t)block_size);
    tbl[tt] = max_blocks > 0 ? trow[j < jmax ? j : jmax] : -1;
  }
#pragma unroll
  for (int tt = 0; tt < kPaTiles; ++tt) {
    const int32_t t0 = tw + tt * 16;
    const int32_t j = (int32_t)((uint32_t)t0 / (uint32_t)block_size);
    const int32_t pg = tbl[tt];
    page[tt] = (t0 < t_end && j < max_blocks && pg >= 0 && pg < num_blocks) ? pg : -1;
  }

  // ---- every K and V load of the wave, issued before any of them is used.
  // Tiles without a valid page read page 0 (in bounds) and are masked below.
  const int64_t kv_head_keys = (int64_t)(kPaD / 16) * block_size * 16;  // bytes per (page, kv head)
  const int64_t kv_head_vals = (int64_t)kPaD * block_size;
  u32x4 kw[kPaTiles][2];  // tile tt: lane (col, grp) holds rows grp and grp + 4 of token col
#pragma unroll
  for (int tt = 0; tt < kPaTiles; ++tt) {
    const int64_t pg = page[tt] >= 0 ? page[tt] : 0;
    const int32_t off0 = (int32_t)((uint32_t)(tw + tt * 16) % (uint32_t)block_size);
    const uint8_t* kp = key_cache + (pg * num_kv_heads + kvh) * kv_head_keys;
#pragma unroll
    for (int h = 0; h < 2; ++h)
      kw[tt][h] = *reinterpret_cast<const u32x4*>(
          kp + ((int64_t)(grp + 4 * h) * block_size + off0 + col) * 16);
  }
  // values: lane (col, grp) holds the 16 tokens of tile grp for d = 16n + col
  int32_t page_v = page[0];
  page_v = grp == 1 ? page[1] : page_v;
  page_v = grp == 2 ? page[2] : page_v;
  page_v = grp == 3 ? page[3] : page_v;
  const int32_t tv = tw + grp * 16;
  const uint8_t* vp = value_cache + ((int64_t)(page_v >= 0 ? page_v : 0) * num_kv_heads + kvh) * kv_head_vals +
                      (uint32_t)tv % (uint32_t)block_size;
  u32x4 vw[8];
#pragma unroll
  for (int n = 0; n < 8; ++n)
    vw[n] = *reinterpret_cast<const u32x4*>(vp + (int64_t)(16 * n + col) * block_size);
  // keep the scheduler from holding any of these loads back behind a use of
  // an earlier one: the wave's whole share is requested before it waits
  __builtin_amdgcn_sched_barrier(0);

  v8bf aq[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    aq[c] = __builtin_bit_cast(v8bf, col < G ? qv[c] : zero);
  }

  // ---- logits: lane holds token col of each tile for heads 4*grp + r
  const float qk_scale = scale * k_scale;
  const float neg_inf = -__builtin_inff();
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
    const bool valid = page[tt] >= 0 && tw + tt * 16 + col < t_end;
    lg[tt][0] = valid ? acc.x * qk_scale : neg_inf;
    lg[tt][1] = valid ? acc.y * qk_scale : neg_inf;
    lg[tt][2] = valid ? acc.z * qk_scale : neg_inf;
    lg[tt][3] = valid ? acc.w * qk_scale : neg_inf;
  }

  // ---- per-head maximum and exp-sum over the wave's tokens
  float m[4], sum[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float v = neg_inf;
#pragma unroll
    for (int tt = 0; tt < kPaTiles; ++tt) v = fmaxf(v, lg[tt][r]);
    m[r] = row16_max(v);
    float e = 0.0f;
#pragma unroll
    for (int tt = 0; tt < kPaTiles; ++tt) {
      const float p = (m[r] == neg_inf) ? 0.0f : __expf(lg[tt][r] - m[r]);
      lg[tt][r] = p;
      e += p;
    }
    sum[r] = row16_sum(e);
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
      p_lds[wave][1][4 * grp + r][16 * tt + col] = bf16_rn(p - __uint_as_float((uint32_t)hi << 16));
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

  // value bytes of tokens without a valid page or past the context: zero
  const int32_t live = page_v >= 0 ? t_end - tv : 0;
  u32x4 keep;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int32_t n_live = live - 4 * q;
    keep[q] = n_live >= 4 ? 0xFFFFFFFFu : n_live <= 0 ? 0u : (0xFFFFFFFFu >> (8 * (4 - n_live)));
  }
  v4f o[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const u32x4 w = vw[n] & keep;
    const v8bf b0 = fp8x8_to_bf16(u32x2{w.x, w.y});
    const v8bf b1 = fp8x8_to_bf16(u32x2{w.z, w.w});
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    acc = mfma_bf16(ap[0][0], b0, acc);
    acc = mfma_bf16(ap[0][1], b0, acc);
    acc = mfma_bf16(ap[1][0], b1, acc);
    acc = mfma_bf16(ap[1][1], b1, acc);
    o[n] = acc;
  }

  // ---- combine the waves: common maximum, rescaled exp-sums and outputs
  if (col == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      m_lds[wave][4 * grp + r] = m[r];
      l_lds[wave][4 * grp + r] = sum[r];
    }
  }
  __syncthreads();  // also ends every read of the probability slices
  float M[4], Lsum[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float mx = neg_inf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, m_lds[w][4 * grp + r]);
    float l = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = m_lds[w][4 * grp + r];
      if (mw != neg_inf) l += l_lds[w][4 * grp + r] * __expf(mw - mx);
    }
    M[r] = mx;
    Lsum[r] = l;
    const float f = (m[r] == neg_inf) ? 0.0f : __expf(m[r] - mx);
#pragma unroll
    for (int n = 0; n < 8; ++n) o_lds[wave][4 * grp + r][16 * n + col] = o[n][r] * f;
  }
  __syncthreads();
  constexpr int kNPerWave = 8 / kWaves;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * grp + r;
    if (row >= G) continue;
    const int64_t sh = (int64_t)s * num_heads + (int64_t)kvh * G + row;
    const float inv = Lsum[r] > 0.0f ? v_scale / Lsum[r] : 0.0f;
    float* dst = tmp_out + (sh * max_parts + part) * kPaD;
#pragma unroll
    for (int i = 0; i < kNPerWave; ++i) {
      const int n = wave * kNPerWave + i;
      float x = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) x += o_lds[w][row][16 * n + col];
      dst[16 * n + col] = x * inv;
    }
    if (wave == 0 && col == 0) {
      exp_sums[sh * max_parts + part] = Lsum[r];
      max_logits[sh * max_parts + part] = M[r];
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
    if (p < nparts && es[p] > 0.0f) wl = es[p] * __expf(ml[p] - M);
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
  const int64_t units = (int64_t)a.num_seqs * a.num_kv_heads * max_parts;
  if (units > 0) {
    const dim3 grid((unsigned)units);
    switch (P) {
      case 64:
        hipLaunchKernelGGL(paged_attention_partition_kernel<1>, grid, dim3(kWave), 0, stream,
                           a.exp_sums, a.max_logits, a.tmp_out, a.query, a.key_cache,
                           a.value_cache, a.block_tables, a.context_lens, a.num_seqs, a.num_heads,
                           a.num_kv_heads, a.block_size, a.max_blocks_per_seq, max_parts,
                           a.num_blocks, a.scale, a.k_scale, a.v_scale);
        break;
      case 128:
        hipLaunchKernelGGL(paged_attention_partition_kernel<2>, grid, dim3(2 * kWave), 0, stream,
                           a.exp_sums, a.max_logits, a.tmp_out, a.query, a.key_cache,
                           a.value_cache, a.block_tables, a.context_lens, a.num_seqs, a.num_heads,
                           a.num_kv_heads, a.block_size, a.max_blocks_per_seq, max_parts,
                           a.num_blocks, a.scale, a.k_scale, a.v_scale);
        break;
      case 256:
        hipLaunchKernelGGL(paged_attention_partition_kernel<4>, grid, dim3(4 * kWave), 0, stream,
                           a.exp_sums, a.max_logits, a.tmp_out, a.query, a.key_cache,
                           a.value_cache, a.block_tables, a.context_lens, a.num_seqs, a.num_heads,
                           a.num_kv_heads, a.block_size, a.max_blocks_per_seq, max_parts,
                           a.num_blocks, a.scale, a.k_scale, a.v_scale);
        break;
      default:
        hipLaunchKernelGGL(paged_attention_partition_kernel<8>, grid, dim3(8 * kWave), 0, stream,
                           a.exp_sums, a.max_logits, a.tmp_out, a.query, a.key_cache,
                           a.value_cache, a.block_tables, a.context_lens, a.num_seqs, a.num_heads,
                           a.num_kv_heads, a.block_size, a.max_blocks_per_seq, max_parts,
                           a.num_blocks, a.scale, a.k_scale, a.v_scale);
        break;
    }
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
