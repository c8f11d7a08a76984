// Indexer logits on the gathered keys: the op the integration PR ("[Deepseek-
// V3.2][Kernel] Integrate cuda indexer k cache gather") hands k_fp8 and
// k_scale.view(float32) to, fp8_mqa_logits.  Its body is not on the pages;
// the reading is the lightning-indexer score
//     logits[i, j - ks[i]] = k_scale[j] * sum_h w[i,h] * relu(q[i,h,:] . k[j,:])
// for j in [ks[i], ke[i]), q and k OCP E4M3 codes (k_scale >= 0, so it may
// leave the ReLU).
//
// The dot products are a dense contraction over head_dim = 128 for every
// (query token, head) row and key column: v_mfma_f32_16x16x128_f8f6f4, one
// instruction per 16 heads x 16 keys.  Operand layout (gfx950): lane l holds
// row (or column) l % 16 and bytes [32*(l/16), +32) of K; the 16x16 result
// gives lane l column l % 16 and rows 4*(l/16) + r, r = 0..3.
//
// A workgroup of 4 waves owns 8 consecutive query tokens (2 per wave, their
// 64-head q rows held as MFMA operands in registers, with their weights).
// It walks the union of their key ranges in tiles of 64 keys, staged in LDS
// (double-buffered, rows padded to 144 bytes) so that all 8 tokens share each
// key load.  Per 16-key subtile a wave issues 2 tokens x 4 head blocks of
// MFMA; the epilogue takes relu, multiplies by the head weight and sums over
// heads -- 16 terms in registers, then across the 4 lane groups -- and
// lanes 0..15 store the 16 logits of each token that fall in its range.
#include "device_common.h"
#include "launch.h"
#include "pkv.h"

namespace pkv {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kLgThreads = 256;
constexpr int kLgWaves = kLgThreads / kWave;
constexpr int kLgTokPerWave = 2;
constexpr int kLgTokens = kLgWaves * kLgTokPerWave;  // query tokens per workgroup
constexpr int kLgTile = 64;                           // keys per LDS tile
constexpr int kLgD = 128;                             // head_dim (one MFMA K)
constexpr int kLgRow = kLgD + 16;                     // padded LDS row, bytes

__device__ __forceinline__ v4f mfma_fp8(const v8i a, const v8i b) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  // format 0 (E4M3) for both operands, no block scaling
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

template <int kHB>  // head blocks of 16: num_heads = 16 * kHB
__global__ __launch_bounds__(kLgThreads) void fp8_mqa_logits_kernel(
    const uint8_t* __restrict__ q, int64_t q_token_stride, const uint8_t* __restrict__ k,
    const float* __restrict__ k_scale, const float* __restrict__ weights,
    const int32_t* __restrict__ ks, const int32_t* __restrict__ ke, float* __restrict__ logits,
    int64_t row_stride, int64_t row_cols, int32_t num_q, int64_t num_k) {
  constexpr int H = 16 * kHB;
  __shared__ __align__(16) uint8_t tile[2][kLgTile * kLgRow];
  __shared__ float tile_scale[2][kLgTile];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int col = lane & 15;   // MFMA row/column within a 16-block
  const int grp = lane >> 4;   // K quarter (operands) / row quarter (result)
  const int64_t i0 = (int64_t)blockIdx.x * kLgTokens;

  // ---- this wave's tokens: ranges, q operands, weights
  int64_t lo_t[kLgTokPerWave], hi_t[kLgTokPerWave], ks_t[kLgTokPerWave];
  v8i a[kLgTokPerWave][kHB];
  float w[kLgTokPerWave][kHB][4];
#pragma unroll
  for (int t = 0; t < kLgTokPerWave; ++t) {
    const int64_t i = i0 + wave * kLgTokPerWave + t;
    lo_t[t] = 0;
    hi_t[t] = 0;
    ks_t[t] = 0;
    if (i < num_q) {
      const int64_t s = ks[i], e = ke[i];
      ks_t[t] = s;
      lo_t[t] = s > 0 ? s : 0;
      int64_t hi = e < num_k ? e : num_k;
      if (hi > s + row_cols) hi = s + row_cols;
      hi_t[t] = hi > lo_t[t] ? hi : lo_t[t];
    }
#pragma unroll
    for (int hb = 0; hb < kHB; ++hb) {
      a[t][hb] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
      if (i < num_q) {
        const u32x4* src = reinterpret_cast<const u32x4*>(
            q + i * q_token_stride + (int64_t)(hb * 16 + col) * kLgD + grp * 32);
        const u32x4 x0 = src[0], x1 = src[1];
        a[t][hb] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                       (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
        w[t][hb][r] = i < num_q ? weights[i * H + hb * 16 + grp * 4 + r] : 0.0f;
    }
  }

  // ---- union of the workgroup's key ranges (every wave computes it)
  int64_t lo = INT64_MAX, hi = 0;
  {
    const int64_t i = i0 + (lane & (kLgTokens - 1));
    int64_t l = INT64_MAX, h = 0;
    if (lane < kLgTokens && i < num_q) {
      const int64_t s = ks[i], e = ke[i];
      const int64_t ll = s > 0 ? s : 0;
      int64_t hh = e < num_k ? e : num_k;
      if (hh > s + row_cols) hh = s + row_cols;
      if (hh > ll) {
        l = ll;
        h = hh;
      }
    }
#pragma unroll
    for (int d = 1; d < kLgTokens; d <<= 1) {
      const int64_t lo2 = lane_value(l, lane ^ d);
      const int64_t hi2 = lane_value(h, lane ^ d);
      l = lo2 < l ? lo2 : l;
      h = hi2 > h ? hi2 : h;
    }
    lo = lane_value(l, 0);
    hi = lane_value(h, 0);
  }
  if (hi <= lo) return;  // uniform over the workgroup: no barrier is skipped by some waves only
  const int64_t ntiles = (hi - lo + kLgTile - 1) / kLgTile;

  // ---- tile loads: 64 rows x 128 bytes = 512 chunks of 16 bytes, 2 per thread
  u32x4 stage[2];
  float stage_scale = 0.0f;
  auto load_tile = [&](int64_t n) {
    const int64_t j0 = lo + n * kLgTile;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = tid + u * kLgThreads;
      const int64_t j = j0 + c / 8;
      stage[u] = u32x4{0u, 0u, 0u, 0u};
      if (j < hi) stage[u] = *reinterpret_cast<const u32x4*>(k + j * kLgD + (c % 8) * 16);
    }
    if (tid < kLgTile) {
      const int64_t j = j0 + tid;
      stage_scale = j < hi ? k_scale[j] : 0.0f;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = tid + u * kLgThreads;
      *reinterpret_cast<u32x4*>(&tile[buf][(c / 8) * kLgRow + (c % 8) * 16]) = stage[u];
    }
    if (tid < kLgTile) tile_scale[buf][tid] = stage_scale;
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int64_t n = 0; n < ntiles; ++n) {
    const int buf = (int)(n & 1);
    if (n + 1 < ntiles) load_tile(n + 1);  // in flight during the MFMA work below
    const int64_t j0 = lo + n * kLgTile;
#pragma unroll
    for (int s = 0; s < kLgTile / 16; ++s) {
      const uint8_t* brow = &tile[buf][(s * 16 + col) * kLgRow + grp * 32];
      const u32x4 b0 = *reinterpret_cast<const u32x4*>(brow);
      const u32x4 b1 = *reinterpret_cast<const u32x4*>(brow + 16);
      const v8i b = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
                     (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
      const float sc = tile_scale[buf][s * 16 + col];
      const int64_t j = j0 + s * 16 + col;
#pragma unroll
      for (int t = 0; t < kLgTokPerWave; ++t) {
        float part = 0.0f;
#pragma unroll
        for (int hb = 0; hb < kHB; ++hb) {
          const v4f acc = mfma_fp8(a[t][hb], b);
          part = __builtin_fmaf(w[t][hb][0], fmaxf(acc.x, 0.0f), part);
          part = __builtin_fmaf(w[t][hb][1], fmaxf(acc.y, 0.0f), part);
          part = __builtin_fmaf(w[t][hb][2], fmaxf(acc.z, 0.0f), part);
          part = __builtin_fmaf(w[t][hb][3], fmaxf(acc.w, 0.0f), part);
        }
        part += __shfl_xor(part, 16);
        part += __shfl_xor(part, 32);
        if (grp == 0 && j >= lo_t[t] && j < hi_t[t]) {
          const int64_t i = i0 + wave * kLgTokPerWave + t;
          logits[i * row_stride + (j - ks_t[t])] = sc * part;
        }
      }
    }
    if (n + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }
}

}  // namespace

int launch_fp8_mqa_logits(const MqaLogitsArgs& a, hipStream_t stream) {
  const int64_t blocks = (a.num_q + kLgTokens - 1) / kLgTokens;
  auto kernel = fp8_mqa_logits_kernel<4>;
  switch (a.num_heads / 16) {
    case 1: kernel = fp8_mqa_logits_kernel<1>; break;
    case 2: kernel = fp8_mqa_logits_kernel<2>; break;
    case 3: kernel = fp8_mqa_logits_kernel<3>; break;
    default: break;
  }
  hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kLgThreads), 0, stream, a.q,
                     a.q_token_stride, a.k, a.k_scale, a.weights, a.ks, a.ke, a.logits,
                     a.row_stride, a.row_cols, a.num_q, a.num_k);
  return (int)hipGetLastError();
}

}  // namespace pkv
