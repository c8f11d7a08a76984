// NVFP4 K/V store (vLLM source nvfp4_kv_cache_kernels.cu: header comment,
// swizzle_scale_offset, reshape_and_cache_nvfp4_kernel,
// reshape_and_cache_nvfp4_dispatch).  Each 16-element block of a token's K
// or V head (bf16 or fp16, as the page's dispatcher instantiates it) becomes
// 8 bytes of packed E2M1 codes plus one E4M3 block scale;
// page sides are [data | scales], K scales linear, V scales in the 4x4-tile
// swizzled order.
//
// Two kernels share the block quantizer below; both give the same bytes.
//
// Tile kernel (head_size 64, 128 or 256, 16-byte aligned page sides): one
// wave quantizes one (16-token tile, side, head).  Lane loads are 16 bytes
// and contiguous over the wave, two lanes per 16-element block.  The wave
// assembles the tile's code bytes and scale bytes in LDS in page order, then
// writes them out 16 bytes per lane for the codes and one dword per lane for
// the scales.  Every lane computes the address of what it writes from the
// slot of its own token, so any slot_mapping is handled; when the tile's
// tokens sit in consecutive slots of one page (as a prefill fills pages),
// a wave's code store covers tile * head_size/2 contiguous bytes and its
// scale store tile * head_size/16 contiguous bytes, whole cache lines.  A
// V-scale dword holds one block scale of 4 tokens of one swizzle tile, so it
// is written as a dword only when those 4 tokens are the 4 consecutive slots
// of a tile; otherwise byte by byte.
//
// Generic kernel (any head_size that is a multiple of 64): work items are
// half-blocks ordered (token, side, head, block, half), so a wave-wide load
// reads 1 KB of one token side contiguously; each lane writes the 4 code
// bytes of its half, K scales leave as one dword per 4 blocks (collected
// from neighbouring lanes with DPP row shifts) and V scales as single bytes
// at their swizzled positions.
//
// In both, workgroups are renumbered so that each XCD takes one contiguous
// range of tokens: the tokens that share a page then write its lines
// through one L2.
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
constexpr int kFp4Waves = kFp4Threads / kWave;

constexpr int kFp4Unroll = 2;  // half-blocks per lane in flight (generic kernel)

constexpr int kFp4Tile = 16;  // tokens per wave item (tile kernel)
// Items per wave whose loads are in flight together; 2 or 4 cut occupancy
// more than they added bytes in flight.
constexpr int kFp4Items = 1;


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

// Per-side global scales gs = 1/k_scale, 1/v_scale, and RN(gs / M) for
// M = 1..15 in LDS.  Called by every thread of the workgroup (barrier).
struct GlobalScales {
  float gs_k, gs_v;
  bool table_k, table_v;  // gs in [2^-100, 2^100]: the LDS quotients are exact
  __device__ __forceinline__ float gs(int kv) const { return kv ? gs_v : gs_k; }
  __device__ __forceinline__ bool table(int kv) const { return kv ? table_v : table_k; }
};
__device__ __forceinline__ GlobalScales load_global_scales(const float* k_scale,
                                                           const float* v_scale,
                                                           float (*gs_over_m)[16]) {
  GlobalScales g;
  g.gs_k = 1.0f / *k_scale;
  g.gs_v = 1.0f / *v_scale;
  if (threadIdx.x < 32) {
    const int side = threadIdx.x >> 4, mm = threadIdx.x & 15;
    gs_over_m[side][mm] = mm ? g.gs(side) / (float)mm : 0.0f;
  }
  __syncthreads();
  g.table_k = g.gs_k >= 0x1p-100f && g.gs_k <= 0x1p100f;
  g.table_v = g.gs_v >= 0x1p-100f && g.gs_v <= 0x1p100f;
  return g;
}

// Quantizes the 8 elements this lane holds, one half of a 16-element block
// whose other half is in lane l ^ 1.  Returns the 4 code bytes (element 2m in
// the low nibble of byte m) and the block's E4M3 scale in sf8.  Every lane of
// the wave must call it (the block amax is a DPP swap).
__device__ __forceinline__ uint32_t nvfp4_half_block(const float (&x)[8], float gs, bool table,
                                                     const float* gs_over_m, uint32_t& sf8) {
  constexpr float kSixth = 1.0f / 6.0f;  // RN(1/6)
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = max(m, abs_bits(x[i]));
  m = max(m, dpp<kQuadSwap1>(m));  // the other half of the block
  const float amax = __uint_as_float(m);
  const float t6 = amax * gs;
  const float q6 = t6 * kSixth;
  const float sf = __builtin_fmaf(__builtin_fmaf(-q6, 6.0f, t6), kSixth, q6);  // = t6 / 6
  sf8 = e4m3_pack2<false>(fminf(sf, 448.0f), 0.0f, 0u) & 0xffu;
  // decode(sf8) = M * 2^p: normal codes M = 8 + mantissa, p = exponent - 10;
  // subnormal codes M = mantissa, p = -9
  const uint32_t ex = sf8 >> 3;
  const uint32_t mm = ex ? 8u + (sf8 & 7u) : (sf8 & 7u);
  const int p = ex ? (int)ex - 10 : -9;
  float r;
  if (table)
    r = sf8 ? __builtin_ldexpf(gs_over_m[mm], -p) : 0.0f;
  else
    r = sf8 ? gs / e4m3_decode(sf8) : 0.0f;
  uint32_t packed = e2m1_pack2<0>(x[0] * r, x[1] * r, 0u);
  packed = e2m1_pack2<1>(x[2] * r, x[3] * r, packed);
  packed = e2m1_pack2<2>(x[4] * r, x[5] * r, packed);
  packed = e2m1_pack2<3>(x[6] * r, x[7] * r, packed);
  return packed;
}

// K/V rows are read once: nontemporal loads.
__device__ __forceinline__ u32x4 load_src(const u32x4* p) { return load_stream(p); }

// Code chunks fill whole lines: nontemporal stores (about 7% faster here than
// write-back ones, and they leave the next kernel fewer dirty lines).
__device__ __forceinline__ void store_codes16(uint8_t* p, u32x4 v) {
  store_stream(reinterpret_cast<u32x4*>(p), v);
}

// Scale dwords cover parts of lines that other waves complete: plain stores,
// merged in L2 (nontemporal ones measured slower).
__device__ __forceinline__ void store_scale4(uint8_t* p, uint32_t v) {
  *reinterpret_cast<uint32_t*>(p) = v;
}

// Byte offset of V scale (off, g) inside its page side's scale region:
// 4x4-tile swizzle of the per-head [B, S] tile, (t', s') =
// ((off/4)*4 + g/(S/4), (g % (S/4))*4 + off%4).
__device__ __forceinline__ int64_t v_scale_offset(int64_t off, int32_t g, int32_t S, int32_t h,
                                                  int32_t num_heads, int32_t block_size,
                                                  int32_t layout) {
  const int32_t q4 = S / 4;
  const int64_t row = (off >> 2) * 4 + g / q4;
  const int64_t col = (int64_t)(g % q4) * 4 + (off & 3);
  return layout == PKV_LAYOUT_HND ? ((int64_t)h * block_size + row) * S + col
                                  : (row * num_heads + h) * S + col;
}

// ------------------------------------------------------------------ tile kernel
template <int kD, bool kF16>
__global__ __launch_bounds__(kFp4Threads) void store_kv_fp4_tile_kernel(
    const uint16_t* __restrict__ key, int64_t key_row_stride, const uint16_t* __restrict__ value,
    int64_t value_row_stride, uint8_t* __restrict__ key_cache, uint8_t* __restrict__ value_cache,
    const int64_t* __restrict__ slot_mapping, int64_t num_tokens, int64_t num_items,
    int64_t num_logical_blocks, int32_t num_heads, int32_t block_size, int32_t log2_bs,
    int64_t num_blocks, int64_t page_stride, int32_t layout, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale) {
  constexpr int kC = kD / 8;                       // 16-byte source chunks per token head
  constexpr int kS = kD / 16;                      // blocks (scale bytes) per token head
  constexpr int kTokPerLoad = kWave / kC;          // tokens one wave-wide load covers
  constexpr int kLoads = kFp4Tile / kTokPerLoad;   // loads per lane per item
  constexpr int kDataBytes = kFp4Tile * kD / 2;    // code bytes of one item
  constexpr int kDataChunks = kDataBytes / 16;     // 16-byte code chunks of one item
  constexpr int kChunksPerTok = kD / 32;           // 16-byte code chunks per token head
  constexpr int kScaleWords = kFp4Tile * kS / 4;   // scale dwords of one item
  static_assert(kC % 2 == 0 && kWave % kC == 0 && kFp4Tile % kTokPerLoad == 0, "tile shape");
  static_assert(kDataChunks % kWave == 0 || kDataChunks < kWave, "code chunks per lane");
  static_assert(kScaleWords <= kWave && kS % 4 == 0, "scale words per lane");

  __shared__ float gs_over_m[2][16];
  __shared__ __align__(16) uint32_t data_img[kFp4Waves][kFp4Items][kDataBytes / 4];
  __shared__ __align__(16) uint32_t scale_img[kFp4Waves][kFp4Items][kScaleWords];
  const GlobalScales G = load_global_scales(k_scale, v_scale, gs_over_m);

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int c = lane % kC;  // source chunk this lane loads, in every load
  const int64_t data_per_side = (int64_t)num_heads * block_size * (kD / 2);
  const int32_t sides_heads = 2 * num_heads;

  for (int64_t lb = xcd_contiguous_block(); lb < num_logical_blocks; lb += gridDim.x) {
    // this wave's kFp4Items consecutive items, each a (tile, side, head)
    int64_t t0[kFp4Items], my_slot[kFp4Items];
    int kv[kFp4Items];
    int32_t h[kFp4Items];
    bool valid[kFp4Items];
    u32x4 xv[kFp4Items][kLoads];
#pragma unroll
    for (int u = 0; u < kFp4Items; ++u) {
      const int64_t item = (lb * kFp4Waves + wave) * kFp4Items + u;
      valid[u] = item < num_items;  // wave-uniform
      const int64_t tile = item / sides_heads;
      const int32_t sh = (int32_t)(item - tile * sides_heads);
      kv[u] = sh >= num_heads;
      h[u] = kv[u] ? sh - num_heads : sh;
      t0[u] = tile * kFp4Tile;
      // slot of token t0 + (lane % 16); tokens past the end have slot -1
      const int64_t my_t = t0[u] + (lane & (kFp4Tile - 1));
      my_slot[u] = valid[u] && my_t < num_tokens ? slot_mapping[my_t] : -1;
      // loads: lane holds chunk c of token k * kTokPerLoad + lane / kC
      const uint16_t* src = kv[u] ? value : key;
      const int64_t row_stride = kv[u] ? value_row_stride : key_row_stride;
#pragma unroll
      for (int k = 0; k < kLoads; ++k) {
        const int64_t t = t0[u] + k * kTokPerLoad + lane / kC;
        xv[u][k] = u32x4{0u, 0u, 0u, 0u};
        if (valid[u] && t < num_tokens)
          xv[u][k] = load_src(
              reinterpret_cast<const u32x4*>(src + t * row_stride + (int64_t)h[u] * kD) + c);
      }
    }

#pragma unroll
    for (int u = 0; u < kFp4Items; ++u) {
      if (!valid[u]) continue;
      uint32_t* dimg = data_img[wave][u];
      uint32_t* simg = scale_img[wave][u];
      uint8_t* simg8 = reinterpret_cast<uint8_t*>(simg);
      // ---- quantize into the LDS images (codes [tok][kD/2]; K scales
      // [tok][kS]; V scales [tok/4][g][tok%4], i.e. the swizzled order)
      const float gs = G.gs(kv[u]);
      const bool table = G.table(kv[u]);
#pragma unroll
      for (int k = 0; k < kLoads; ++k) {
        const int tk = k * kTokPerLoad + lane / kC;
        float x[8];
        unpack8_src<kF16>(xv[u][k], x);
        uint32_t sf8;
        const uint32_t packed = nvfp4_half_block(x, gs, table, gs_over_m[kv[u]], sf8);
        dimg[tk * kC + c] = packed;  // byte offset tk*kD/2 + 4c
        if ((c & 1) == 0) {
          const int g = c >> 1;
          const int pos = kv[u] ? (tk >> 2) * 4 * kS + g * 4 + (tk & 3) : tk * kS + g;
          simg8[pos] = (uint8_t)sf8;
        }
      }
      wave_sync();

      // ---- code bytes: 16 bytes per lane, address from the chunk's token slot
#pragma unroll
      for (int q0 = 0; q0 < kDataChunks; q0 += kWave) {
        const int q = q0 + lane;
        const int tok = (q < kDataChunks ? q : 0) / kChunksPerTok;
        const int64_t slot = lane_value(my_slot[u], tok);
        if (q < kDataChunks && slot >= 0) {
          int64_t page, off;
          split_slot(slot, block_size, log2_bs, page, off);
          if (page < num_blocks) {
            uint8_t* side = (kv[u] ? value_cache : key_cache) + page * page_stride;
            const int64_t row = layout == PKV_LAYOUT_HND ? (int64_t)h[u] * block_size + off
                                                         : off * num_heads + h[u];
            const u32x4 v = *reinterpret_cast<const u32x4*>(dimg + 4 * q);
            store_codes16(side + row * (kD / 2) + (q % kChunksPerTok) * 16, v);
          }
        }
      }

      // ---- scale bytes: one dword per lane
      const int sw = lane < kScaleWords ? lane : 0;
      const uint32_t word = simg[sw];
      if (kv[u] == 0) {
        const int tok = (4 * sw) / kS;
        const int64_t slot = lane_value(my_slot[u], tok);
        if (lane < kScaleWords && slot >= 0) {
          int64_t page, off;
          split_slot(slot, block_size, log2_bs, page, off);
          if (page < num_blocks) {
            uint8_t* scales = key_cache + page * page_stride + data_per_side;
            const int64_t row = layout == PKV_LAYOUT_HND ? (int64_t)h[u] * block_size + off
                                                         : off * num_heads + h[u];
            store_scale4(scales + row * kS + (4 * sw) % kS, word);
          }
        }
      } else {
        // dword sw = block g of the 4 tokens 4*quad .. 4*quad+3
        const int quad = sw / kS, g = sw % kS;
        int64_t s4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) s4[i] = lane_value(my_slot[u], 4 * quad + i);
        if (lane < kScaleWords) {
          const bool whole = s4[0] >= 0 && (s4[0] & 3) == 0 && s4[1] == s4[0] + 1 &&
                             s4[2] == s4[0] + 2 && s4[3] == s4[0] + 3;
          if (whole) {
            // 4 consecutive slots starting at a multiple of 4: one page (block
            // sizes are multiples of 4), one swizzle tile, one dword
            int64_t page, off;
            split_slot(s4[0], block_size, log2_bs, page, off);
            if (page < num_blocks) {
              uint8_t* scales = value_cache + page * page_stride + data_per_side;
              store_scale4(
                  scales + v_scale_offset(off, g, kS, h[u], num_heads, block_size, layout), word);
            }
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if (s4[i] < 0) continue;
              int64_t page, off;
              split_slot(s4[i], block_size, log2_bs, page, off);
              if (page >= num_blocks) continue;
              uint8_t* scales = value_cache + page * page_stride + data_per_side;
              scales[v_scale_offset(off, g, kS, h[u], num_heads, block_size, layout)] =
                  (uint8_t)(word >> (8 * i));
            }
          }
        }
      }
    }
    wave_sync();  // the next iteration rewrites this wave's LDS images
  }
}

// --------------------------------------------------------------- generic kernel
template <bool kF16>
__global__ __launch_bounds__(kFp4Threads) void store_kv_fp4_kernel(
    const uint16_t* __restrict__ key, int64_t key_row_stride, const uint16_t* __restrict__ value,
    int64_t value_row_stride, uint8_t* __restrict__ key_cache, uint8_t* __restrict__ value_cache,
    const int64_t* __restrict__ slot_mapping, int64_t token0, uint32_t num_items,
    int32_t num_heads, int32_t head_size, int32_t block_size, int32_t log2_bs, int64_t num_blocks,
    int64_t page_stride, int32_t layout, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, Div halves, Div scale_dim) {
  __shared__ float gs_over_m[2][16];  // RN(gs / M), M = 1..15, per side
  const GlobalScales G = load_global_scales(k_scale, v_scale, gs_over_m);
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
        xv[k] = load_src(reinterpret_cast<const u32x4*>(src + (int64_t)hq[k] * 8));
      }
    }
    // ---- quantize and store (cross-lane steps run with every lane active)
#pragma unroll
    for (int k = 0; k < kFp4Unroll; ++k) {
      float x[8];
      unpack8_src<kF16>(xv[k], x);
      const int kv = tk[k] & 1;
      uint32_t sf8;
      const uint32_t packed = nvfp4_half_block(x, G.gs(kv), G.table(kv), gs_over_m[kv], sf8);
      // K: scale bytes of blocks g..g+3 (lanes +0, +2, +4, +6) in one dword
      const uint32_t sf_word = sf8 | (from_lane_above<2>(sf8) << 8) |
                               (from_lane_above<4>(sf8) << 16) | (from_lane_above<6>(sf8) << 24);
      if (slot[k] < 0) continue;
      int64_t page, off;
      split_slot(slot[k], block_size, log2_bs, page, off);
      if (page >= num_blocks) continue;

      const uint32_t half = hq[k] & 1;
      uint32_t h, g;
      scale_dim.split(hq[k] >> 1, h, g);
      uint8_t* side = (kv ? value_cache : key_cache) + page * page_stride;
      int64_t data_off;
      if (layout == PKV_LAYOUT_HND)
        data_off = ((int64_t)h * block_size + off) * data_dim + (int64_t)g * 8 + half * 4;
      else
        data_off = (off * num_heads + h) * data_dim + (int64_t)g * 8 + half * 4;
      *reinterpret_cast<uint32_t*>(side + data_off) = packed;

      if (half) continue;
      uint8_t* scales = side + data_per_side;
      if (kv == 0) {
        if ((g & 3) == 0) {
          const int64_t row_off = layout == PKV_LAYOUT_HND ? ((int64_t)h * block_size + off) * S
                                                           : (off * num_heads + h) * S;
          *reinterpret_cast<uint32_t*>(scales + row_off + g) = sf_word;
        }
      } else {  // V scales: 4x4-tile swizzle of the per-head [B, S] tile
        scales[v_scale_offset(off, (int32_t)g, S, (int32_t)h, num_heads, block_size, layout)] =
            (uint8_t)sf8;
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

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <int kD>
int launch_tile(const StoreFp4Args& a, hipStream_t stream) {
  const int64_t tiles = (a.num_tokens + kFp4Tile - 1) / kFp4Tile;
  const int64_t items = tiles * 2 * a.num_heads;
  const int64_t logical = (items + kFp4Waves * kFp4Items - 1) / (kFp4Waves * kFp4Items);
  int64_t blocks = logical < kFp4MaxBlocks ? logical : kFp4MaxBlocks;
  blocks = (blocks + kNumXcd - 1) / kNumXcd * kNumXcd;  // whole XCD ranges
  auto kernel = a.src_dtype == PKV_DTYPE_F16 ? store_kv_fp4_tile_kernel<kD, true>
                                             : store_kv_fp4_tile_kernel<kD, false>;
  hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kFp4Threads), 0, stream, a.key,
                     a.key_row_stride, a.value, a.value_row_stride, a.key_cache, a.value_cache,
                     a.slot_mapping, a.num_tokens, items, logical, a.num_heads, a.block_size,
                     a.log2_block_size, a.num_blocks, a.page_stride, a.layout, a.k_scale,
                     a.v_scale);
  return (int)hipGetLastError();
}

int launch_generic(const StoreFp4Args& a, hipStream_t stream) {
  const int32_t S = a.head_size / 16;
  const int64_t halves = 2 * (int64_t)a.num_heads * S;  // half-blocks per token side
  const Div halves_div{(int32_t)halves, log2_exact(halves)};
  const Div scale_dim{S, log2_exact(S)};
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
                       a.k_scale, a.v_scale, halves_div, scale_dim);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
  }
  return 0;
}

}  // namespace


int launch_store_kv_fp4(const StoreFp4Args& a, hipStream_t stream) {
  const bool sides16 = aligned16(a.key_cache) && aligned16(a.value_cache) && a.page_stride % 16 == 0;
  if (sides16) {  // the tile kernel where it applies
    if (a.head_size == 64) return launch_tile<64>(a, stream);
    if (a.head_size == 128) return launch_tile<128>(a, stream);
    if (a.head_size == 256) return launch_tile<256>(a, stream);
  }
  return launch_generic(a, stream);
}

}  // namespace pkv
