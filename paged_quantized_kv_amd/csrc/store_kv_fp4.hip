// NVFP4 K/V store (vLLM source nvfp4_kv_cache_kernels.cu: header comment,
// swizzle_scale_offset, reshape_and_cache_nvfp4_kernel,
// reshape_and_cache_nvfp4_dispatch).  Each 16-element block of a token's K
// or V head becomes 8 bytes of packed E2M1 codes plus one E4M3 block scale;
// page sides are [data | scales], K scales linear, V scales in the 4x4-tile
// swizzled order.
//
// Mapping: one lane per 16-element block (32 bytes in, 8 + 1 bytes out).
// Work items are ordered (token, side, head, block), so for H*D = 1024 one
// wave reads one token side as 2 KB of contiguous bf16 and writes 64-byte
// head rows.  Lanes stride over items; the global scales 1/k_scale and
// 1/v_scale are computed once per lane.
//
// Arithmetic per block, all binary32 with round-to-nearest-even:
//   amax = max|x|;  sf = (amax * gs) / 6;  sf8 = E4M3(min(sf, 448))
//   r = gs / decode(sf8) (0 if the decoded scale is 0);  c = E2M1(x * r)
// Divisions are IEEE divisions.  E4M3 and E2M1 use the gfx950 converters;
// the clamp at 448 gives the saturating E4M3 result for any sf >= 448.
#include "device_common.h"
#include "launch.h"

namespace pkv {

namespace {

constexpr int kFp4Threads = 256;

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

__global__ __launch_bounds__(kFp4Threads) void store_kv_fp4_kernel(
    const uint16_t* __restrict__ key, int64_t key_row_stride, const uint16_t* __restrict__ value,
    int64_t value_row_stride, uint8_t* __restrict__ key_cache, uint8_t* __restrict__ value_cache,
    const int64_t* __restrict__ slot_mapping, int64_t token0, uint32_t num_items,
    int32_t num_heads, int32_t head_size, int32_t block_size, int32_t log2_bs, int64_t num_blocks,
    int64_t page_stride, int32_t layout, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, Div groups, Div scale_dim, Div quarter_s) {
  const float gs_k = 1.0f / *k_scale;
  const float gs_v = 1.0f / *v_scale;
  const int32_t S = scale_dim.d;
  const int64_t data_dim = head_size / 2;
  const int64_t data_per_side = (int64_t)num_heads * block_size * data_dim;

  const uint32_t stride = gridDim.x * kFp4Threads;
  for (uint32_t u = blockIdx.x * kFp4Threads + threadIdx.x; u < num_items; u += stride) {
    uint32_t tk, q;
    groups.split(u, tk, q);          // tk = 2*token + side, q = h*S + g
    const int64_t t = token0 + (tk >> 1);
    const int kv = tk & 1;
    const int64_t slot = slot_mapping[t];
    if (slot < 0) continue;
    int64_t page, off;
    split_slot(slot, block_size, log2_bs, page, off);
    if (page >= num_blocks) continue;
    uint32_t h, g;
    scale_dim.split(q, h, g);

    const uint16_t* src = kv ? value + t * value_row_stride : key + t * key_row_stride;
    const u32x4* p = reinterpret_cast<const u32x4*>(src + (int64_t)q * 16);
    float x[16];
    unpack8(load_stream(p), x);
    unpack8(load_stream(p + 1), x + 8);

    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = max(m, abs_bits(x[i]));
    const float amax = __uint_as_float(m);
    const float gs = kv ? gs_v : gs_k;
    const float sf = (amax * gs) / 6.0f;
    const uint32_t sf8 = e4m3_pack2<false>(fminf(sf, 448.0f), 0.0f, 0u) & 0xffu;
    const float sfd = e4m3_decode(sf8);
    const float r = (sfd == 0.0f) ? 0.0f : gs / sfd;

    u32x2 packed;
    packed.x = e2m1_pack2<0>(x[0] * r, x[1] * r, 0u);
    packed.x = e2m1_pack2<1>(x[2] * r, x[3] * r, packed.x);
    packed.x = e2m1_pack2<2>(x[4] * r, x[5] * r, packed.x);
    packed.x = e2m1_pack2<3>(x[6] * r, x[7] * r, packed.x);
    packed.y = e2m1_pack2<0>(x[8] * r, x[9] * r, 0u);
    packed.y = e2m1_pack2<1>(x[10] * r, x[11] * r, packed.y);
    packed.y = e2m1_pack2<2>(x[12] * r, x[13] * r, packed.y);
    packed.y = e2m1_pack2<3>(x[14] * r, x[15] * r, packed.y);

    uint8_t* side = (kv ? value_cache : key_cache) + page * page_stride;
    int64_t row = off, col = g;
    if (kv) {  // V scales: 4x4-tile swizzle of the per-head [B, S] tile
      uint32_t gq, gr;
      quarter_s.split(g, gq, gr);   // g / (S/4), g % (S/4)
      row = (off >> 2) * 4 + gq;
      col = (int64_t)gr * 4 + (off & 3);
    }
    int64_t data_off, scale_off;
    if (layout == 0) {  // HND
      data_off = ((int64_t)h * block_size + off) * data_dim + (int64_t)g * 8;
      scale_off = ((int64_t)h * block_size + row) * S + col;
    } else {            // NHD
      data_off = (off * num_heads + h) * data_dim + (int64_t)g * 8;
      scale_off = (row * num_heads + h) * S + col;
    }
    *reinterpret_cast<u32x2*>(side + data_off) = packed;
    side[data_per_side + scale_off] = (uint8_t)sf8;
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
  const int64_t G = (int64_t)a.num_heads * S;  // blocks per token side
  const Div groups{(int32_t)G, log2_exact(G)};
  const Div scale_dim{S, log2_exact(S)};
  const Div quarter_s{S / 4, log2_exact(S / 4)};
  // Items are indexed in 32 bits: split the tokens into launches of at most
  // 2^31 items each.
  const int64_t max_tokens = (int64_t{1} << 31) / (2 * G);
  for (int64_t t0 = 0; t0 < a.num_tokens; t0 += max_tokens) {
    const int64_t nt = (a.num_tokens - t0) < max_tokens ? (a.num_tokens - t0) : max_tokens;
    const uint32_t items = (uint32_t)(nt * 2 * G);
    int64_t blocks = ((int64_t)items + kFp4Threads - 1) / kFp4Threads;
    if (blocks > kFp4MaxBlocks) blocks = kFp4MaxBlocks;
    hipLaunchKernelGGL(store_kv_fp4_kernel, dim3((unsigned)blocks), dim3(kFp4Threads), 0, stream,
                       a.key, a.key_row_stride, a.value, a.value_row_stride, a.key_cache,
                       a.value_cache, a.slot_mapping, t0, items, a.num_heads, a.head_size,
                       a.block_size, a.log2_block_size, a.num_blocks, a.page_stride, a.layout,
                       a.k_scale, a.v_scale, groups, scale_dim, quarter_s);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
  }
  return 0;
}

}  // namespace pkv
