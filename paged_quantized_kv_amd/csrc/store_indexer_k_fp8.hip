// fp8 per-token quantize-and-scatter into the paged indexer K cache: the
// producer of the pages that the gather of vLLM PR "Add
// gather_indexer_k_quant_cache kernel" reads.  For every token with a
// non-negative slot: s = amax/448 in binary32, codes E4M3(x/s) (OCP E4M3FN,
// round to nearest even), 4 scale bytes after the page's code region.
//
// Mapping: kLanes lanes per token, 16 bf16 elements (two 16-byte loads) per
// lane, so a wave covers 64/kLanes tokens (8 for head_dim 128).  The token
// amax is a DPP max over the kLanes lanes.  Each lane writes its 16 codes as
// one 16-byte store, so a token's 128-byte code row is one cache line.
//
// Division: x/s must be the correctly rounded binary32 quotient (it decides
// ties of the E4M3 rounding).  For amax >= 2^-60 every step of the
// Markstein-corrected product stays in the normal range, so one correctly
// rounded reciprocal per token plus three operations per element give the
// IEEE quotient; tokens with a smaller amax (subnormal scales) take the
// IEEE division directly.  E4M3 encoding uses the hardware converter, exact
// for |y| < 464; here |y| <= 448 * (1 + 2^-8) even for subnormal scales.
#include "device_common.h"
#include "launch.h"

namespace pkv {

namespace {

constexpr int kStoreThreads = 256;

template <int kLanes>
__global__ __launch_bounds__(kStoreThreads) void store_indexer_k_fp8_kernel(
    const uint16_t* __restrict__ k, int64_t k_row_stride,
    const int64_t* __restrict__ slot_mapping, int64_t num_tokens, uint8_t* __restrict__ kv_cache,
    int64_t num_blocks, int64_t page_stride, int32_t block_size, int32_t log2_bs,
    int32_t head_dim) {
  constexpr int kTokensPerWave = kWave / kLanes;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave_id = ((int64_t)blockIdx.x * kStoreThreads + threadIdx.x) / kWave;
  const int64_t t = wave_id * kTokensPerWave + lane / kLanes;
  const int part = lane % kLanes;
  const bool in_token = t < num_tokens;
  const bool active = in_token && part * 16 < head_dim;

  u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
  int64_t slot = -1;
  if (in_token) slot = slot_mapping[t];
  if (active) {
    const u32x4* src = reinterpret_cast<const u32x4*>(k + t * k_row_stride + part * 16);
    lo = load_stream(src);
    hi = load_stream(src + 1);
  }
  float x[16];
  unpack8(lo, x);
  unpack8(hi, x + 8);
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = max(m, abs_bits(x[i]));
  m = group_max<kLanes>(m);  // all 64 lanes take part
  if (!active || slot < 0) return;
  int64_t page, off;
  split_slot(slot, block_size, log2_bs, page, off);
  if (page >= num_blocks) return;

  const float amax = __uint_as_float(m);
  const float s = amax / 448.0f;
  float y[16];
  if (amax >= 0x1p-60f) {
    const float rs = 1.0f / s;
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = div_by_scale(x[i], s, rs);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = (s == 0.0f) ? x[i] : x[i] / s;
  }
  u32x4 codes;
  codes.x = e4m3_pack4(y[0], y[1], y[2], y[3]);
  codes.y = e4m3_pack4(y[4], y[5], y[6], y[7]);
  codes.z = e4m3_pack4(y[8], y[9], y[10], y[11]);
  codes.w = e4m3_pack4(y[12], y[13], y[14], y[15]);

  uint8_t* page_base = kv_cache + page * page_stride;
  store_stream(reinterpret_cast<u32x4*>(page_base + off * head_dim + part * 16), codes);
  if (part == 0)
    *reinterpret_cast<float*>(page_base + (int64_t)block_size * head_dim + off * 4) = s;
}

template <int kLanes>
int launch_lanes(const StoreFp8Args& a, hipStream_t stream) {
  constexpr int64_t kTokensPerBlock = (kStoreThreads / kWave) * (kWave / kLanes);
  const int64_t blocks = (a.num_tokens + kTokensPerBlock - 1) / kTokensPerBlock;
  hipLaunchKernelGGL(store_indexer_k_fp8_kernel<kLanes>, dim3((unsigned)blocks),
                     dim3(kStoreThreads), 0, stream, a.k, a.k_row_stride, a.slot_mapping,
                     a.num_tokens, a.kv_cache, a.num_blocks, a.cache_block_stride, a.block_size,
                     a.log2_block_size, a.head_dim);
  return (int)hipGetLastError();
}

}  // namespace

int launch_store_indexer_k_fp8(const StoreFp8Args& a, hipStream_t stream) {
  const int parts = a.head_dim / 16;  // 16 elements per lane
  if (parts <= 1) return launch_lanes<1>(a, stream);
  if (parts <= 2) return launch_lanes<2>(a, stream);
  if (parts <= 4) return launch_lanes<4>(a, stream);
  if (parts <= 8) return launch_lanes<8>(a, stream);
  if (parts <= 16) return launch_lanes<16>(a, stream);
  if (parts <= 32) return launch_lanes<32>(a, stream);
  return launch_lanes<64>(a, stream);
}

}  // namespace pkv
