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
// partition_size tokens); no LDS is shared between waves and there is no
// barrier.  The wave's G = num_heads/num_kv_heads query heads are the 16 rows
// of v_mfma_f32_16x16x32_bf16 operands (rows >= G are zero); fp8 keys and
// values become bf16 exactly (4 significant bits fit in 8).  Per 16-token
// tile (one page, block_size a multiple of 16): 4 MFMAs give the 16 x 16
// logits.  After the partition's max and exp-sum per head, the probabilities
// go through a wave-private LDS slice (transposed to operand order) as bf16
// hi + lo parts (16 significant bits), and 2 x 8 MFMAs per 32 tokens give
// the 16 x 128 partial output.  The partition writes its normalised partial
// output, exp-sum and max to the caller's workspace (exp_sums, max_logits,
// tmp_out), as the page's schema does.
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
constexpr int kPaMaxPart = 256;  // largest partition_size (logit registers)
constexpr int kPaChunk = 32;     // tokens per PV step (one MFMA K)

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

template <int kTiles>  // partition_size / 16
__global__ __launch_bounds__(kPaThreads) void paged_attention_partition_kernel(
    float* __restrict__ exp_sums, float* __restrict__ max_logits, float* __restrict__ tmp_out,
    const uint16_t* __restrict__ query, const uint8_t* __restrict__ key_cache,
    const uint8_t* __restrict__ value_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t block_size, int32_t max_blocks, int32_t max_parts,
    int64_t num_blocks, float scale, float k_scale, float v_scale) {
  constexpr int P = kTiles * 16;
  // per wave: probabilities of one 32-token chunk, [16 heads][32 tokens], hi and lo
  __shared__ __align__(16) uint16_t p_lds[kPaWaves][2][16][kPaChunk + 8];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int col = lane & 15;  // operand row / result column
  const int grp = lane >> 4;  // K quarter / result row quarter
  const int64_t unit = (int64_t)blockIdx.x * kPaWaves + wave;
  if (unit >= (int64_t)num_seqs * num_kv_heads * max_parts) return;
  const int32_t part = (int32_t)(unit % max_parts);
  const int32_t kvh = (int32_t)((unit / max_parts) % num_kv_heads);
  const int32_t s = (int32_t)(unit / ((int64_t)max_parts * num_kv_heads));
  const int64_t L = context_lens[s];
  const int64_t t_begin = (int64_t)part * P;
  if (t_begin >= L) return;  // this partition holds no token
  const int64_t t_end = (t_begin + P < L) ? t_begin + P : L;
  const int32_t G = num_heads / num_kv_heads;

  // ---- query operands: row = head kvh*G + col (zero past G), K = d
  v8bf aq[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (col < G)
      v = *reinterpret_cast<const u32x4*>(
          query + ((int64_t)s * num_heads + kvh * G + col) * kPaD + c * 32 + grp * 8);
    aq[c] = __builtin_bit_cast(v8bf, v);
  }

  // ---- logits of every tile: lane holds token col, heads 4*grp + r
  const float qk_scale = scale * k_scale;
  const float neg_inf = -__builtin_inff();
  const int64_t kv_head_keys = (int64_t)(kPaD / 16) * block_size * 16;  // bytes per (page, kv head)
  float lg[kTiles][4];
  int64_t tile_page[kTiles];
#pragma unroll
  for (int tt = 0; tt < kTiles; ++tt) {
    const int64_t t0 = t_begin + tt * 16;
    int64_t page = -1;
    if (t0 < t_end) {
      const int64_t j = t0 / block_size;
      if (j < max_blocks) page = block_tables[(int64_t)s * max_blocks + j];
      if (page >= num_blocks) page = -1;
    }
    tile_page[tt] = page;
    const int64_t off0 = t0 % block_size;
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    if (page >= 0) {  // uniform over the wave
      const uint8_t* kp = key_cache + (page * num_kv_heads + kvh) * kv_head_keys;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        // d = 32c + 8*grp + e -> row d/16 = 2c + grp/2, column d%16 = 8*(grp%2) + e
        const u32x2 w = *reinterpret_cast<const u32x2*>(
            kp + ((int64_t)(2 * c + (grp >> 1)) * block_size + off0 + col) * 16 + 8 * (grp & 1));
        acc = mfma_bf16(aq[c], fp8x8_to_bf16(w), acc);
      }
    }
    const bool valid = page >= 0 && t0 + col < t_end;
    lg[tt][0] = valid ? acc.x * qk_scale : neg_inf;
    lg[tt][1] = valid ? acc.y * qk_scale : neg_inf;
    lg[tt][2] = valid ? acc.z * qk_scale : neg_inf;
    lg[tt][3] = valid ? acc.w * qk_scale : neg_inf;
  }

  // ---- per-head max and exp-sum over the partition
  float m[4], sum[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float v = neg_inf;
#pragma unroll
    for (int tt = 0; tt < kTiles; ++tt) v = fmaxf(v, lg[tt][r]);
    m[r] = row16_max(v);
    float e = 0.0f;
#pragma unroll
    for (int tt = 0; tt < kTiles; ++tt) {
      const float p = (m[r] == neg_inf) ? 0.0f : __expf(lg[tt][r] - m[r]);
      lg[tt][r] = p;
      e += p;
    }
    sum[r] = row16_sum(e);
  }

  // ---- partial output: 32 tokens per step, probabilities as bf16 hi + lo
  v4f o[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) o[n] = v4f{0.f, 0.f, 0.f, 0.f};
  const int64_t kv_head_vals = (int64_t)kPaD * block_size;  // bytes per (page, kv head)
#pragma unroll
  for (int k = 0; k < kTiles / 2; ++k) {
    // transpose the chunk's probabilities to operand order through LDS
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int tt = 2 * k + half;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = lg[tt][r];
        const uint16_t hi = bf16_rn(p);
        const float rem = p - __uint_as_float((uint32_t)hi << 16);  // exact
        p_lds[wave][0][4 * grp + r][16 * half + col] = hi;
        p_lds[wave][1][4 * grp + r][16 * half + col] = bf16_rn(rem);
      }
    }
    wave_sync();
    const v8bf ap_hi = __builtin_bit_cast(v8bf, *reinterpret_cast<const u32x4*>(&p_lds[wave][0][col][8 * grp]));
    const v8bf ap_lo = __builtin_bit_cast(v8bf, *reinterpret_cast<const u32x4*>(&p_lds[wave][1][col][8 * grp]));
    // values: tokens 8*grp .. +8 of the chunk lie in tile 2k + grp/2, offsets 8*(grp%2) ..
    const int tt = 2 * k + (grp >> 1);
    const int64_t page = tile_page[tt];
    const int64_t t0 = t_begin + tt * 16 + 8 * (grp & 1);  // first token of this lane's 8
    const int64_t off = t0 % block_size;
    // tokens past the context may hold any bytes: zero their value codes
    const int64_t n_live = t_end - t0;
    uint32_t keep_lo = 0u, keep_hi = 0u;  // byte masks
    if (page >= 0 && n_live > 0) {
      keep_lo = n_live >= 4 ? 0xFFFFFFFFu : (0xFFFFFFFFu >> (8 * (4 - n_live)));
      keep_hi = n_live >= 8 ? 0xFFFFFFFFu : (n_live <= 4 ? 0u : (0xFFFFFFFFu >> (8 * (8 - n_live))));
    }
    const uint8_t* vp = value_cache + (page >= 0 ? (page * num_kv_heads + kvh) * kv_head_vals : 0);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      u32x2 w = {0u, 0u};
      if (keep_lo) w = *reinterpret_cast<const u32x2*>(vp + (int64_t)(16 * n + col) * block_size + off);
      w.x &= keep_lo;
      w.y &= keep_hi;
      const v8bf bv = fp8x8_to_bf16(w);
      o[n] = mfma_bf16(ap_hi, bv, o[n]);
      o[n] = mfma_bf16(ap_lo, bv, o[n]);
    }
    wave_sync();  // the next chunk rewrites this wave's LDS slice
  }

  // ---- normalised partial output, exp-sum and max of each real head
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * grp + r;
    if (row >= G) continue;
    const int64_t h = (int64_t)kvh * G + row;
    const int64_t sh = (int64_t)s * num_heads + h;
    const float inv = sum[r] > 0.0f ? v_scale / sum[r] : 0.0f;
    float* dst = tmp_out + (sh * max_parts + part) * kPaD;
#pragma unroll
    for (int n = 0; n < 8; ++n) dst[16 * n + col] = o[n][r] * inv;
    if (col == 0) {
      exp_sums[sh * max_parts + part] = sum[r];
      max_logits[sh * max_parts + part] = m[r];
    }
  }
}

__global__ __launch_bounds__(kPaThreads) void paged_attention_reduce_kernel(
    uint16_t* __restrict__ out, const float* __restrict__ exp_sums,
    const float* __restrict__ max_logits, const float* __restrict__ tmp_out,
    const int32_t* __restrict__ context_lens, int32_t num_seqs, int32_t num_heads,
    int32_t max_parts, int32_t partition_size) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t sh = (int64_t)blockIdx.x * kPaWaves + threadIdx.x / kWave;
  if (sh >= (int64_t)num_seqs * num_heads) return;
  const int32_t s = (int32_t)(sh / num_heads);
  const int64_t L = context_lens[s];
  int64_t nparts = L > 0 ? (L + partition_size - 1) / partition_size : 0;
  if (nparts > max_parts) nparts = max_parts;
  const float* es = exp_sums + sh * max_parts;
  const float* ml = max_logits + sh * max_parts;
  float M = -__builtin_inff();
  for (int64_t p = 0; p < nparts; ++p)
    if (es[p] > 0.0f) M = fmaxf(M, ml[p]);
  float a0 = 0.0f, a1 = 0.0f, W = 0.0f;
  for (int64_t p = 0; p < nparts; ++p) {
    if (!(es[p] > 0.0f)) continue;
    const float w = es[p] * __expf(ml[p] - M);
    const float* o = tmp_out + (sh * max_parts + p) * kPaD;
    a0 = __builtin_fmaf(w, o[lane], a0);
    a1 = __builtin_fmaf(w, o[lane + 64], a1);
    W += w;
  }
  const float inv = W > 0.0f ? 1.0f / W : 0.0f;
  out[sh * kPaD + lane] = bf16_rn(a0 * inv);
  out[sh * kPaD + lane + 64] = bf16_rn(a1 * inv);
}

}  // namespace

int launch_paged_attention_decode(const PagedAttentionArgs& a, hipStream_t stream) {
  const int32_t P = a.partition_size;
  const int32_t max_parts = (a.max_context_len + P - 1) / P;
  const int64_t units = (int64_t)a.num_seqs * a.num_kv_heads * max_parts;
  const int64_t blocks = (units + kPaWaves - 1) / kPaWaves;
  auto kernel = paged_attention_partition_kernel<16>;
  switch (P / 16) {
    case 2: kernel = paged_attention_partition_kernel<2>; break;
    case 4: kernel = paged_attention_partition_kernel<4>; break;
    case 8: kernel = paged_attention_partition_kernel<8>; break;
    default: break;
  }
  if (blocks > 0) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kPaThreads), 0, stream, a.exp_sums,
                       a.max_logits, a.tmp_out, a.query, a.key_cache, a.value_cache,
                       a.block_tables, a.context_lens, a.num_seqs, a.num_heads, a.num_kv_heads,
                       a.block_size, a.max_blocks_per_seq, max_parts, a.num_blocks, a.scale,
                       a.k_scale, a.v_scale);
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
