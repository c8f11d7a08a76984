// fp8 per-token quantize-and-scatter into the paged indexer K cache: the
// producer of the pages that the gather of vLLM PR "Add
// gather_indexer_k_quant_cache kernel" reads.  For every token with a
// non-negative slot: s = amax/448 in binary32, codes E4M3(x/s) (OCP E4M3FN,
// round to nearest even), 4 scale bytes after the page's code region.
// Source elements are bf16 or fp16, widened exactly.
//
// Mapping: kLanes lanes per token, 8 bf16 elements (one 16-byte load) per
// lane and chunk, so the lanes of a token read its row with contiguous
// loads and a wave covers 64/kLanes tokens (4 for head_dim 128).  The token
// amax is a DPP max over the kLanes lanes.  Each lane writes its 8 codes as
// one 8-byte store, so the 16 lanes of a 128-wide token fill its 128-byte
// code row, one cache line.
//
// Division: x/s must be the correctly rounded binary32 quotient (it decides
// ties of the E4M3 rounding).  Per token, s = amax/448 and rs = RN(1/s) are
// correctly rounded divisions; per element, Markstein's correction turns
// x * rs into the IEEE quotient x/s in three operations (for amax >= 2^-60
// every step stays in the normal range; checked over every significand
// pair on the host).  Tokens with a smaller amax (subnormal scales) take
// the IEEE division per element.  E4M3 encoding uses the hardware converter, exact for |y| < 464;
// here |y| <= 448 * (1 + 2^-8) even for subnormal scales.
#include "device_common.h"
#include "launch.h"
#include "pkv.h"

namespace pkv {

namespace {

constexpr int kStoreThreads = 256;

constexpr int kStoreUnroll = 2;  // token groups per wave in flight

// kLanes lanes per token (a power of two), each holding kChunks runs of 8
// elements: lane l of a token takes elements [8*(l + c*kLanes), +8), so the
// lanes of a token read its row with contiguous 16-byte loads.
template <int kLanes, int kChunks, bool kF16>
__global__ __launch_bounds__(kStoreThreads) void store_indexer_k_fp8_kernel(
    const uint16_t* __restrict__ k, int64_t k_row_stride,
    const int64_t* __restrict__ slot_mapping, int64_t num_tokens, uint8_t* __restrict__ kv_cache,
    int64_t num_blocks, int64_t page_stride, int32_t block_size, int32_t log2_bs,
    int32_t head_dim) {
  constexpr int kTokensPerWave = kWave / kLanes;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave_id = ((int64_t)blockIdx.x * kStoreThreads + threadIdx.x) / kWave;
  const int part = lane % kLanes;
  const int64_t last_token = num_tokens - 1;
  const int last_chunk = head_dim / 8 - 1;

  // ---- every group's loads, unconditional (rows past the end re-read the
  // last row, chunks past head_dim the last chunk; neither is stored)
  u32x4 xv[kStoreUnroll][kChunks];
  int64_t slot[kStoreUnroll];
#pragma unroll
  for (int u = 0; u < kStoreUnroll; ++u) {
    const int64_t t = (wave_id * kStoreUnroll + u) * kTokensPerWave + lane / kLanes;
    const int64_t tc = t < num_tokens ? t : last_token;
    slot[u] = slot_mapping[tc];
    if (t >= num_tokens) slot[u] = -1;
    const u32x4* src = reinterpret_cast<const u32x4*>(k + tc * k_row_stride);
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int ch = part + c * kLanes;
      xv[u][c] = load_stream(src + (ch < last_chunk ? ch : last_chunk));
    }
  }

  // ---- quantize group by group (each waits only for its own loads); the
  // stores follow once every group is done, so no store is outstanding while
  // a later group's loads are awaited
  u32x2 codes[kStoreUnroll][kChunks];
  float sv[kStoreUnroll];
  uint8_t* base[kStoreUnroll];
  int64_t offv[kStoreUnroll];
  bool keep[kStoreUnroll];
#pragma unroll
  for (int u = 0; u < kStoreUnroll; ++u) {
    float x[kChunks][8];
    uint32_t m = 0;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      unpack8_src<kF16>(xv[u][c], x[c]);
      const bool in = (part + c * kLanes) * 8 < head_dim;
#pragma unroll
      for (int i = 0; i < 8; ++i) m = max(m, in ? abs_bits(x[c][i]) : 0u);
    }
    m = group_max<kLanes>(m);  // all 64 lanes take part
    int64_t page = 0, off = 0;
    if (slot[u] >= 0) split_slot(slot[u], block_size, log2_bs, page, off);
    keep[u] = slot[u] >= 0 && page < num_blocks;
    const float amax = __uint_as_float(m);
    const bool fast = amax >= 0x1p-60f;
    const float s = amax / 448.0f;
    const float rs = fast ? 1.0f / s : 0.0f;
    sv[u] = s;
    base[u] = kv_cache + page * page_stride;
    offv[u] = off;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      float y[8];
      if (fast) {
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = div_by_scale(x[c][i], s, rs);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = (s == 0.0f) ? x[c][i] : x[c][i] / s;
      }
      codes[u][c].x = e4m3_pack4(y[0], y[1], y[2], y[3]);
      codes[u][c].y = e4m3_pack4(y[4], y[5], y[6], y[7]);
    }
  }
#pragma unroll
  for (int u = 0; u < kStoreUnroll; ++u) {
    if (!keep[u]) continue;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int e0 = (part + c * kLanes) * 8;
      if (e0 < head_dim)
        *reinterpret_cast<u32x2*>(base[u] + offv[u] * head_dim + e0) = codes[u][c];
    }
    if (part == 0)
      *reinterpret_cast<float*>(base[u] + (int64_t)block_size * head_dim + offv[u] * 4) = sv[u];
  }
}

template <int kLanes, int kChunks, bool kF16>
int launch_lanes_t(const StoreFp8Args& a, hipStream_t stream) {
  constexpr int64_t kTokensPerBlock = (kStoreThreads / kWave) * (kWave / kLanes) * kStoreUnroll;
  const int64_t blocks = (a.num_tokens + kTokensPerBlock - 1) / kTokensPerBlock;
  hipLaunchKernelGGL((store_indexer_k_fp8_kernel<kLanes, kChunks, kF16>), dim3((unsigned)blocks),
                     dim3(kStoreThreads), 0, stream, a.k, a.k_row_stride, a.slot_mapping,
                     a.num_tokens, a.kv_cache, a.num_blocks, a.cache_block_stride, a.block_size,
                     a.log2_block_size, a.head_dim);
  return (int)hipGetLastError();
}

template <int kLanes, int kChunks>
int launch_lanes(const StoreFp8Args& a, hipStream_t stream) {
  return a.k_dtype == PKV_DTYPE_F16 ? launch_lanes_t<kLanes, kChunks, true>(a, stream)
                                    : launch_lanes_t<kLanes, kChunks, false>(a, stream);
}

}  // namespace

int launch_store_indexer_k_fp8(const StoreFp8Args& a, hipStream_t stream) {
  const int runs = a.head_dim / 8;  // 8 elements per lane and chunk
  if (runs <= 2) return launch_lanes<2, 1>(a, stream);
  if (runs <= 4) return launch_lanes<4, 1>(a, stream);
  if (runs <= 8) return launch_lanes<8, 1>(a, stream);
  if (runs <= 16) return launch_lanes<16, 1>(a, stream);
  if (runs <= 32) return launch_lanes<32, 1>(a, stream);
  if (runs <= 64) return launch_lanes<64, 1>(a, stream);
  return launch_lanes<64, 2>(a, stream);  // head_dim <= 1024
}

}  // namespace pkv
