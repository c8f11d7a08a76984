// NVFP4 K/V store (vLLM source nvfp4_kv_cache_kernels.cu: header comment,
// swizzle_scale_offset, reshape_and_cache_nvfp4_kernel,
// reshape_and_cache_nvfp4_dispatch).  Each 16-element block of a token's K
// or V head (bf16 or fp16, as the page's dispatcher instantiates it) becomes
// 8 bytes of packed E2M1 codes plus one E4M3 block scale;
// page sides are [data | scales], K scales linear, V scales in the 4x4-tile
// swizzled order.
//
// Mapping: two lanes per 16-element block, 8 bf16 (one 16-byte load) per
// lane.  Work items are half-blocks ordered (token, side, head, block,
// half), so a wave-wide load reads 1 KB of one token side contiguously; the
// block amax is a DPP swap between the two lanes, and each lane writes the
// 4 code bytes of its half.  K scales, which are linear, leave as one dword
// per 4 blocks (collected from neighbouring lanes with DPP row shifts); V
// scales are single bytes at their swizzled positions.  Each lane issues the
// loads of several items before it quantizes any of them, and the grid is
// numbered so that each XCD takes one contiguous range of tokens: the tokens
// that share a page then write its lines through one L2.
//
// Arithmetic per block, all binary32 with round-to-nearest-even:
//   amax = max|x|;  sf = (amax * gs) / 6;  sf8 = E4M3(min(sf, 448))
//   r = gs / decode(sf8) (0 if the decoded scale is 0);  c = E2M1(x * r)
// Both divisions are the IEEE quotients, obtained without a divide:
//  - t/6 by Markstein's correction of t * RN(1/6), exact for every binary32
//    t in the normal range (checked over all significands on the host); a
//    t small enough to leave that range gives sf8 = 0 either way, and an
//    infinite t saturates either way;
//  - decode(sf8) = M * 2^p with M in 1..15, so RN(gs/decode(sf8)) =
//    RN(gs/M) * 2^-p whenever gs lies in [2^-100, 2^100] (all results stay
//    normal); each workgroup divides gs by M = 1..15 once per side into LDS.
//    A gs outside that range takes the IEEE division per block.
// E4M3 and E2M1 use the gfx950 converters; the clamp at 448 gives the
// saturating E4M3 result for any sf >= 448.
#include "device_common.h"
#include "launch.h"
#include "pkv.h"

namespace pkv {

namespace {

constexpr int kFp4Threads = 256;

#ifndef PKV_FP4_UNROLL
#define PKV_FP4_UNROLL 2
#endif
constexpr int kFp4Unroll = PKV_FP4_UNROLL;  // half-blocks per lane in flight

struct Div {
  // n / d and n % d for a positive divisor that may or may not be a power of two
  int32_t d;
  int32_t log2d;
  __device__ __forceinline__ void split(uint32_t n, uint32_t& q, uint32_t& r) const {
    if (log2d >= 0) {
      q = n >> log2d;
      r = n & (uint32_t)(d - 1);
    } else {
      q = n / (uint32_t)d;
      r = n - q * (uint32_t)d;
    }
  }
};

// DPP row shift: lane i receives lane i + k of its 16-lane row (0 past the row end).
template <int k>
__device__ __forceinline__ uint32_t from_lane_above(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x100 + k, 0xF, 0xF, true);
}

template <bool kF16>
__global__ __launch_bounds__(kFp4Threads) void store_kv_fp4_kernel(
    const uint16_t* __restrict__ key, int64_t key_row_stride, const uint16_t* __restrict__ value,
    int64_t value_row_stride, uint8_t* __restrict__ key_cache, uint8_t* __restrict__ value_cache,
    const int64_t* __restrict__ slot_mapping, int64_t token0, uint32_t num_items,
    int32_t num_heads, int32_t head_size, int32_t block_size, int32_t log2_bs, int64_t num_blocks,
    int64_t page_stride, int32_t layout, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, Div halves, Div scale_dim, Div quarter_s) {
  __shared__ float gs_over_m[2][16];  // RN(gs / M), M = 1..15, per side
  const float gs_k = 1.0f / *k_scale;
  const float gs_v = 1.0f / *v_scale;
  if (threadIdx.x < 32) {
    const int side = threadIdx.x >> 4, mm = threadIdx.x & 15;
    gs_over_m[side][mm] = mm ? (side ? gs_v : gs_k) / (float)mm : 0.0f;
  }
  __syncthreads();
  const bool table_k = gs_k >= 0x1p-100f && gs_k <= 0x1p100f;
  const bool table_v = gs_v >= 0x1p-100f && gs_v <= 0x1p100f;
  constexpr float kSixth = 1.0f / 6.0f;  // RN(1/6)
  const int32_t S = scale_dim.d;
  const int64_t data_dim = head_size / 2;
  const int64_t data_per_side = (int64_t)num_heads * block_size * data_dim;

  // A workgroup's iteration covers kFp4Unroll * kFp4Threads consecutive
  // items; item k of a lane is base + k * kFp4Threads.  Item parity is lane
  // parity, so the two halves of a block always sit in lanes 2i and 2i+1,
  // and the 8 lanes of 4 consecutive blocks share one 16-lane DPP row.
  const uint32_t span = kFp4Unroll * kFp4Threads;
  const uint32_t stride = gridDim.x * span;
  const uint32_t block = xcd_contiguous_block();
  for (uint32_t base = block * span + threadIdx.x; base < num_items; base += stride) {
    u32x4 xv[kFp4Unroll];
    int64_t slot[kFp4Unroll];
    uint32_t tk[kFp4Unroll], hq[kFp4Unroll];
    // ---- issue every load first
#pragma unroll
    for (int k = 0; k < kFp4Unroll; ++k) {
      const uint32_t u = base + k * kFp4Threads;
      slot[k] = -1;
      xv[k] = u32x4{0u, 0u, 0u, 0u};
      tk[k] = 0;
      hq[k] = 0;
      if (u < num_items) {
        halves.split(u, tk[k], hq[k]);  // tk = 2*token + side, hq = 2*(h*S + g) + half
        const int64_t t = token0 + (tk[k] >> 1);
        slot[k] = slot_mapping[t];
        const uint16_t* src = (tk[k] & 1) ? value + t * value_row_stride
                                          : key + t * key_row_stride;
        xv[k] = load_stream(reinterpret_cast<const u32x4*>(src + (int64_t)hq[k] * 8));
      }
    }
    // ---- quantize and store (cross-lane steps run with every lane active)
#pragma unroll
    for (int k = 0; k < kFp4Unroll; ++k) {
      float x[8];
      unpack8_src<kF16>(xv[k], x);
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) m = max(m, abs_bits(x[i]));
      m = max(m, dpp<kQuadSwap1>(m));  // the other half of the block
      const int kv = tk[k] & 1;
      const float gs = kv ? gs_v : gs_k;
      const float amax = __uint_as_float(m);
      const float t6 = amax * gs;
      const float q6 = t6 * kSixth;
      const float sf = __builtin_fmaf(__builtin_fmaf(-q6, 6.0f, t6), kSixth, q6);  // = t6 / 6
      const uint32_t sf8 = e4m3_pack2<false>(fminf(sf, 448.0f), 0.0f, 0u) & 0xffu;
      // K: scale bytes of blocks g..g+3 (lanes +0, +2, +4, +6) in one dword
      const uint32_t sf_word = sf8 | (from_lane_above<2>(sf8) << 8) |
                               (from_lane_above<4>(sf8) << 16) | (from_lane_above<6>(sf8) << 24);
      if (slot[k] < 0) continue;
      int64_t page, off;
      split_slot(slot[k], block_size, log2_bs, page, off);
      if (page >= num_blocks) continue;

      // decode(sf8) = M * 2^p: normal codes M = 8 + mantissa, p = exponent - 10;
      // subnormal codes M = mantissa, p = -9
      const uint32_t ex = sf8 >> 3;
      const uint32_t mm = ex ? 8u + (sf8 & 7u) : (sf8 & 7u);
      const int p = ex ? (int)ex - 10 : -9;
      float r;
      if (kv ? table_v : table_k)
        r = sf8 ? __builtin_ldexpf(gs_over_m[kv][mm], -p) : 0.0f;
      else
        r = sf8 ? gs / e4m3_decode(sf8) : 0.0f;
      uint32_t packed = e2m1_pack2<0>(x[0] * r, x[1] * r, 0u);
      packed = e2m1_pack2<1>(x[2] * r, x[3] * r, packed);
      packed = e2m1_pack2<2>(x[4] * r, x[5] * r, packed);
      packed = e2m1_pack2<3>(x[6] * r, x[7] * r, packed);

      const uint32_t half = hq[k] & 1;
      uint32_t h, g;
      scale_dim.split(hq[k] >> 1, h, g);
      uint8_t* side = (kv ? value_cache : key_cache) + page * page_stride;
      int64_t data_off;
      if (layout == 0)  // HND
        data_off = ((int64_t)h * block_size + off) * data_dim + (int64_t)g * 8 + half * 4;
      else              // NHD
        data_off = (off * num_heads + h) * data_dim + (int64_t)g * 8 + half * 4;
      *reinterpret_cast<uint32_t*>(side + data_off) = packed;

      if (half) continue;
      uint8_t* scales = side + data_per_side;
      if (kv == 0) {
        if ((g & 3) == 0) {
          const int64_t row_off = layout == 0 ? ((int64_t)h * block_size + off) * S
                                              : (off * num_heads + h) * S;
          *reinterpret_cast<uint32_t*>(scales + row_off + g) = sf_word;
        }
      } else {  // V scales: 4x4-tile swizzle of the per-head [B, S] tile
        uint32_t gq, gr;
        quarter_s.split(g, gq, gr);  // g / (S/4), g % (S/4)
        const int64_t row = (off >> 2) * 4 + gq;
        const int64_t col = (int64_t)gr * 4 + (off & 3);
        const int64_t so = layout == 0 ? ((int64_t)h * block_size + row) * S + col
                                       : (row * num_heads + h) * S + col;
        scales[so] = (uint8_t)sf8;
      }
    }
  }
}

int32_t log2_exact(int64_t v) {
  if (v <= 0 || (v & (v - 1))) return -1;
  int32_t l = 0;
  while ((int64_t{1} << l) < v) ++l;
  return l;
}

}  // namespace

int launch_store_kv_fp4(const StoreFp4Args& a, hipStream_t stream) {
  const int32_t S = a.head_size / 16;
  const int64_t halves = 2 * (int64_t)a.num_heads * S;  // half-blocks per token side
  const Div halves_div{(int32_t)halves, log2_exact(halves)};
  const Div scale_dim{S, log2_exact(S)};
  const Div quarter_s{S / 4, log2_exact(S / 4)};
  // Items are indexed in 32 bits: split the tokens into launches of at most
  // 2^31 items each.
  const int64_t max_tokens = (int64_t{1} << 31) / (2 * halves);
  for (int64_t t0 = 0; t0 < a.num_tokens; t0 += max_tokens) {
    const int64_t nt = (a.num_tokens - t0) < max_tokens ? (a.num_tokens - t0) : max_tokens;
    const uint32_t items = (uint32_t)(nt * 2 * halves);
    int64_t blocks = ((int64_t)items + kFp4Unroll * kFp4Threads - 1) / (kFp4Unroll * kFp4Threads);
    if (blocks > kFp4MaxBlocks) blocks = kFp4MaxBlocks;
    blocks = (blocks + kNumXcd - 1) / kNumXcd * kNumXcd;  // whole XCD ranges
    auto kernel = a.src_dtype == PKV_DTYPE_F16 ? store_kv_fp4_kernel<true> : store_kv_fp4_kernel<false>;
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kFp4Threads), 0, stream,
                       a.key, a.key_row_stride, a.value, a.value_row_stride, a.key_cache,
                       a.value_cache, a.slot_mapping, t0, items, a.num_heads, a.head_size,
                       a.block_size, a.log2_block_size, a.num_blocks, a.page_stride, a.layout,
                       a.k_scale, a.v_scale, halves_div, scale_dim, quarter_s);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
  }
  return 0;
}

}  // namespace pkv
