// Reader side of the paged quantized caches: gathers that hand a consumer
// without fp8 or fp4 inputs contiguous bf16 or fp16 rows.
//
// Indexer K (vLLM PR "Add gather_indexer_k_quant_cache kernel": the gather
// of quantized keys and their scales, driven by block_table and
// cu_seq_lens; the integration PR reads the scale bytes back as float32):
// row cu_seq_lens[r] + i gets token i of request r, each element
// E4M3 decode(code) * scale in binary32, then rounded to the output type.
//
// NVFP4 K/V (vLLM source nvfp4_kv_cache_kernels.cu: page layout
// [K_data|K_scale|V_data|V_scale], 16-element blocks, K scales linear, V
// scales at swizzle_scale_offset; the store's global scale is 1/k_scale):
// each element E2M1 decode(code) * E4M3 decode(block scale), which is exact,
// times k_scale (v_scale for V) in binary32, then rounded to the output type.
//
// Both walk the block table directly: one wave per (table entry, ...) unit,
// exiting at once when the entry holds no tokens of its request, with a
// grid-stride loop so the grid never decides coverage.  A wave's loads
// (16-byte code chunks, contiguous over the wave) are all issued before it
// converts any of them; every 16-byte chunk of codes becomes 32 (fp8) or 64
// (fp4) bytes of output, stored 16 bytes per lane.
//
// Conversions are the gfx950 ones: v_cvt_pk_f32_fp8 (exact E4M3 decode),
// v_cvt_scalef32_pk_f32_fp4 with unit scale (exact E2M1 decode),
// v_cvt_pk_bf16_f32 and v_cvt_f16_f32 (round to nearest even).  NaN codes
// (0x7F, 0xFF) and non-finite scales lie outside what the stores write; they
// give NaN or infinity, with unspecified NaN bits.
#include "device_common.h"
#include "launch.h"
#include "pkv.h"

namespace pkv {

namespace {

constexpr int kDqThreads = 256;
constexpr int kDqWaves = kDqThreads / kWave;
constexpr int kDqUnroll = 4;  // 16-byte code chunks per lane in flight

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Two binary32 values rounded to nearest even into one dword of bf16 or fp16
// (first value in the low half).
template <bool kF16>
__device__ __forceinline__ uint32_t narrow2(float a, float b) {
  const f32x2 v = {a, b};
  if constexpr (kF16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// 16 E4M3 codes times s -> 16 narrowed outputs (32 bytes, element order).
template <bool kF16>
__device__ __forceinline__ void dequant16_fp8(const u32x4 codes, float s, u32x4& lo, u32x4& hi) {
  uint32_t w[8];
  const uint32_t c[4] = {codes.x, codes.y, codes.z, codes.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[q], false);  // bytes 0, 1
    const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[q], true);   // bytes 2, 3
    w[2 * q] = narrow2<kF16>(a.x * s, a.y * s);
    w[2 * q + 1] = narrow2<kF16>(b.x * s, b.y * s);
  }
  lo = u32x4{w[0], w[1], w[2], w[3]};
  hi = u32x4{w[4], w[5], w[6], w[7]};
}

// The two E2M1 codes of byte kByte of `word` (low nibble first) times the
// block scale sfd (exact) times the tensor scale ts (one binary32 rounding),
// narrowed into one dword.
template <int kByte, bool kF16>
__device__ __forceinline__ uint32_t fp4_pair(uint32_t word, float sfd, float ts) {
  const f32x2 d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, kByte);
  const float p0 = d.x * sfd, p1 = d.y * sfd;
  return narrow2<kF16>(p0 * ts, p1 * ts);
}

// Tokens [j*B, min((j+1)*B, len)) of request r, clipped to [0, num_tokens)
// rows; returns false when the entry holds nothing to copy.
struct Run {
  int64_t page;   // page id
  int64_t first;  // first page offset copied
  int64_t row;    // output row of that offset
  int64_t rows;   // rows copied
};
__device__ __forceinline__ bool table_entry_run(const int32_t* __restrict__ block_table,
                                                const int32_t* __restrict__ cu_seq_lens,
                                                int64_t e, int32_t max_blocks,
                                                int64_t num_tokens, int64_t num_blocks,
                                                int32_t block_size, Run& run) {
  const int32_t r = (int32_t)(e / max_blocks);
  const int32_t j = (int32_t)(e - (int64_t)r * max_blocks);
  const int64_t start = cu_seq_lens[r];
  const int64_t len = (int64_t)cu_seq_lens[r + 1] - start;
  const int64_t page = block_table[e];
  if (page < 0 || page >= num_blocks) return false;
  const int64_t i0 = (int64_t)j * block_size;
  if (i0 >= len) return false;
  const int64_t n = (len - i0 < block_size) ? (len - i0) : block_size;
  const int64_t row0 = start + i0;
  const int64_t rb = row0 > 0 ? row0 : 0;
  const int64_t re = (row0 + n < num_tokens) ? row0 + n : num_tokens;
  if (rb >= re) return false;
  run.page = page;
  run.first = rb - row0;
  run.row = rb;
  run.rows = re - rb;
  return true;
}

// ------------------------------------------------------------- indexer K
template <bool kF16>
__global__ __launch_bounds__(kDqThreads) void gather_indexer_k_dequant_kernel(
    const uint8_t* __restrict__ kv_cache, uint16_t* __restrict__ out, int64_t out_row_stride,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ cu_seq_lens,
    int32_t num_reqs, int32_t max_blocks, int64_t num_tokens, int64_t num_blocks,
    int64_t page_stride, int32_t block_size, int32_t head_dim) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t entries = (int64_t)num_reqs * max_blocks;
  const int64_t stride = (int64_t)gridDim.x * kDqWaves;
  const int32_t cpt = head_dim / 16;  // 16-byte code chunks per token
  for (int64_t e = (int64_t)blockIdx.x * kDqWaves + threadIdx.x / kWave; e < entries;
       e += stride) {
    Run run;
    if (!table_entry_run(block_table, cu_seq_lens, e, max_blocks, num_tokens, num_blocks,
                         block_size, run))
      continue;
    const uint8_t* page = kv_cache + run.page * page_stride;
    const u32x4* csrc = reinterpret_cast<const u32x4*>(page + run.first * head_dim);
    const float* ssrc =
        reinterpret_cast<const float*>(page + (int64_t)block_size * head_dim) + run.first;
    const int64_t chunks = run.rows * cpt;
    for (int64_t c0 = 0; c0 < chunks; c0 += kWave * kDqUnroll) {
      u32x4 v[kDqUnroll];
      float s[kDqUnroll];
#pragma unroll
      for (int u = 0; u < kDqUnroll; ++u) {
        const int64_t c = c0 + u * kWave + lane;
        v[u] = u32x4{0u, 0u, 0u, 0u};
        s[u] = 0.0f;
        if (c < chunks) {
          v[u] = load_stream(csrc + c);
          s[u] = ssrc[c / cpt];
        }
      }
#pragma unroll
      for (int u = 0; u < kDqUnroll; ++u) {
        const int64_t c = c0 + u * kWave + lane;
        if (c >= chunks) continue;
        const int64_t t = c / cpt;
        u32x4 lo, hi;
        dequant16_fp8<kF16>(v[u], s[u], lo, hi);
        u32x4* dst = reinterpret_cast<u32x4*>(out + (run.row + t) * out_row_stride +
                                              (c - t * cpt) * 16);
        store_stream(dst, lo);
        store_stream(dst + 1, hi);
      }
    }
  }
}

// ------------------------------------------------------------- NVFP4 K/V
// Unit = (table entry, side, head).  A 16-byte chunk holds the codes of two
// consecutive blocks of one token head (32 elements -> 64 output bytes).
template <bool kF16>
__global__ __launch_bounds__(kDqThreads) void gather_kv_fp4_dequant_kernel(
    const uint8_t* __restrict__ key_cache, const uint8_t* __restrict__ value_cache,
    uint16_t* __restrict__ key_out, int64_t key_row_stride, uint16_t* __restrict__ value_out,
    int64_t value_row_stride, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ cu_seq_lens, int32_t num_reqs, int32_t max_blocks,
    int64_t num_tokens, int32_t num_heads, int32_t head_size, int32_t block_size,
    int64_t num_blocks, int64_t page_stride, int32_t layout, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale) {
  const int lane = threadIdx.x & (kWave - 1);
  const float ts_k = *k_scale, ts_v = *v_scale;
  const int32_t S = head_size / 16;
  const int32_t q4 = S / 4;
  const int32_t cpt = head_size / 32;  // 16-byte code chunks per token head
  const int64_t data_dim = head_size / 2;
  const int64_t data_per_side = (int64_t)num_heads * block_size * data_dim;
  const int64_t units = (int64_t)num_reqs * max_blocks * 2 * num_heads;
  const int64_t stride = (int64_t)gridDim.x * kDqWaves;
  for (int64_t w = (int64_t)blockIdx.x * kDqWaves + threadIdx.x / kWave; w < units;
       w += stride) {
    const int64_t e = w / (2 * num_heads);
    const int32_t sh = (int32_t)(w - e * 2 * num_heads);
    const int kv = sh >= num_heads;
    const int32_t h = kv ? sh - num_heads : sh;
    Run run;
    if (!table_entry_run(block_table, cu_seq_lens, e, max_blocks, num_tokens, num_blocks,
                         block_size, run))
      continue;
    const uint8_t* side = (kv ? value_cache : key_cache) + run.page * page_stride;
    const uint8_t* scales = side + data_per_side;
    uint16_t* out = kv ? value_out : key_out;
    const int64_t out_stride = kv ? value_row_stride : key_row_stride;
    const float ts = kv ? ts_v : ts_k;
    const int64_t chunks = run.rows * cpt;
    for (int64_t c0 = 0; c0 < chunks; c0 += kWave * kDqUnroll) {
      u32x4 v[kDqUnroll];
      uint32_t sc[kDqUnroll];  // the two block-scale bytes, low byte first
#pragma unroll
      for (int u = 0; u < kDqUnroll; ++u) {
        const int64_t c = c0 + u * kWave + lane;
        v[u] = u32x4{0u, 0u, 0u, 0u};
        sc[u] = 0u;
        if (c < chunks) {
          const int64_t t = c / cpt;
          const int32_t wc = (int32_t)(c - t * cpt);
          const int64_t off = run.first + t;
          const int64_t row = layout == PKV_LAYOUT_HND ? (int64_t)h * block_size + off
                                                       : off * num_heads + h;
          v[u] = load_stream(reinterpret_cast<const u32x4*>(side + row * data_dim) + wc);
          const int32_t g0 = 2 * wc;
          if (kv == 0) {
            sc[u] = *reinterpret_cast<const uint16_t*>(scales + row * S + g0);
          } else {
            // swizzled: (t', s') = ((off/4)*4 + g/(S/4), (g % (S/4))*4 + off%4)
            const int64_t srow = (off >> 2) * 4 + g0 / q4;
            const int64_t col = (int64_t)(g0 % q4) * 4 + (off & 3);
            const int64_t base = layout == PKV_LAYOUT_HND ? ((int64_t)h * block_size + srow) * S
                                                          : (srow * num_heads + h) * S;
            const int32_t g1 = g0 + 1;
            const int64_t srow1 = (off >> 2) * 4 + g1 / q4;
            const int64_t col1 = (int64_t)(g1 % q4) * 4 + (off & 3);
            const int64_t base1 = layout == PKV_LAYOUT_HND
                                      ? ((int64_t)h * block_size + srow1) * S
                                      : (srow1 * num_heads + h) * S;
            sc[u] = (uint32_t)scales[base + col] | ((uint32_t)scales[base1 + col1] << 8);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kDqUnroll; ++u) {
        const int64_t c = c0 + u * kWave + lane;
        if (c >= chunks) continue;
        const int64_t t = c / cpt;
        const int32_t wc = (int32_t)(c - t * cpt);
        const float sfd0 = __builtin_amdgcn_cvt_f32_fp8((int)sc[u], 0);
        const float sfd1 = __builtin_amdgcn_cvt_f32_fp8((int)sc[u], 1);
        const uint32_t cw[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
        uint32_t o[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float sfd = q < 2 ? sfd0 : sfd1;  // dwords 0-1: block g0, 2-3: block g0+1
          // byte b of the dword holds elements 2b (low nibble) and 2b+1
          o[q * 4 + 0] = fp4_pair<0, kF16>(cw[q], sfd, ts);
          o[q * 4 + 1] = fp4_pair<1, kF16>(cw[q], sfd, ts);
          o[q * 4 + 2] = fp4_pair<2, kF16>(cw[q], sfd, ts);
          o[q * 4 + 3] = fp4_pair<3, kF16>(cw[q], sfd, ts);
        }
        u32x4* dst = reinterpret_cast<u32x4*>(out + (run.row + t) * out_stride +
                                              (int64_t)h * head_size + (int64_t)wc * 32);
#pragma unroll
        for (int k = 0; k < 4; ++k)
          store_stream(dst + k, u32x4{o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]});
      }
    }
  }
}

// Diagnostic: the output rounding of both gathers applied elementwise.
template <bool kF16>
__global__ __launch_bounds__(kDqThreads) void diag_narrow_kernel(const float* __restrict__ x,
                                                                  uint16_t* __restrict__ out,
                                                                  int64_t n8) {
  const int64_t stride = (int64_t)gridDim.x * kDqThreads;
  for (int64_t i = (int64_t)blockIdx.x * kDqThreads + threadIdx.x; i < n8; i += stride) {
    const u32x4* p = reinterpret_cast<const u32x4*>(x + i * 8);
    const u32x4 a = p[0], b = p[1];
    const u32x4 o = {narrow2<kF16>(__uint_as_float(a.x), __uint_as_float(a.y)),
                     narrow2<kF16>(__uint_as_float(a.z), __uint_as_float(a.w)),
                     narrow2<kF16>(__uint_as_float(b.x), __uint_as_float(b.y)),
                     narrow2<kF16>(__uint_as_float(b.z), __uint_as_float(b.w))};
    *reinterpret_cast<u32x4*>(out + i * 8) = o;
  }
}

int64_t dq_blocks(int64_t units) {
  int64_t b = (units + kDqWaves - 1) / kDqWaves;
  if (b > kGatherMaxBlocks) b = kGatherMaxBlocks;
  return b < 1 ? 1 : b;
}

}  // namespace

int launch_gather_indexer_k_dequant(const GatherDequantArgs& a, hipStream_t stream) {
  const int64_t entries = (int64_t)a.num_reqs * a.max_blocks_per_req;
  auto kernel = a.out_dtype == PKV_DTYPE_F16 ? gather_indexer_k_dequant_kernel<true>
                                             : gather_indexer_k_dequant_kernel<false>;
  hipLaunchKernelGGL(kernel, dim3((unsigned)dq_blocks(entries)), dim3(kDqThreads), 0, stream,
                     a.kv_cache, a.out, a.out_row_stride, a.block_table, a.cu_seq_lens,
                     a.num_reqs, a.max_blocks_per_req, a.num_tokens, a.num_blocks,
                     a.cache_block_stride, a.block_size, a.head_dim);
  return (int)hipGetLastError();
}

int launch_gather_kv_fp4_dequant(const GatherFp4DequantArgs& a, hipStream_t stream) {
  const int64_t units = (int64_t)a.num_reqs * a.max_blocks_per_req * 2 * a.num_heads;
  auto kernel = a.out_dtype == PKV_DTYPE_F16 ? gather_kv_fp4_dequant_kernel<true>
                                             : gather_kv_fp4_dequant_kernel<false>;
  hipLaunchKernelGGL(kernel, dim3((unsigned)dq_blocks(units)), dim3(kDqThreads), 0, stream,
                     a.key_cache, a.value_cache, a.key_out, a.key_row_stride, a.value_out,
                     a.value_row_stride, a.block_table, a.cu_seq_lens, a.num_reqs,
                     a.max_blocks_per_req, a.num_tokens, a.num_heads, a.head_size, a.block_size,
                     a.num_blocks, a.page_stride, a.layout, a.k_scale, a.v_scale);
  return (int)hipGetLastError();
}

int launch_diag_narrow(const float* x, uint16_t* out, int64_t n, int32_t out_dtype,
                       hipStream_t stream) {
  const int64_t n8 = n / 8;
  int64_t blocks = (n8 + kDqThreads - 1) / kDqThreads;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  auto kernel = out_dtype == PKV_DTYPE_F16 ? diag_narrow_kernel<true> : diag_narrow_kernel<false>;
  hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kDqThreads), 0, stream, x, out, n8);
  return (int)hipGetLastError();
}

}  // namespace pkv
