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
// Both walk the block table directly: one wave per table entry (and side,
// for NVFP4), exiting at once when the entry holds no tokens of its request,
// with a grid-stride loop so the grid never decides coverage.  A lane's unit
// is 8 elements of output: 8 fp8 codes (8 bytes) or one half-block of fp4
// codes (4 bytes) become one 16-byte store; units run in output order, so
// every wave store covers 1 KB of contiguous rows.  A wave issues the loads
// of several units before it converts any of them.
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
constexpr int kIdxUnroll = 4;   // lane units (8 elements each) in flight, indexer
constexpr int kFp4Unroll = 32;  // lane units in flight, NVFP4 (direct kernel)

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
// Work of a wave: one table entry's run of tokens.  Lane unit = 8 codes of
// one token (an 8-byte load) -> 8 outputs (one 16-byte store), so every wave
// load covers 512 contiguous code bytes and every wave store 1 KB of rows.
template <bool kF16>
__global__ __launch_bounds__(kDqThreads) void gather_indexer_k_dequant_kernel(
    const uint8_t* __restrict__ kv_cache, uint16_t* __restrict__ out, int64_t out_row_stride,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ cu_seq_lens,
    int32_t num_reqs, int32_t max_blocks, int64_t num_tokens, int64_t num_blocks,
    int64_t page_stride, int32_t block_size, int32_t head_dim, FastDiv upt_div) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t entries = (int64_t)num_reqs * max_blocks;
  const int64_t stride = (int64_t)gridDim.x * kDqWaves;
  const int32_t upt = head_dim / 8;  // 8-code units per token (upt_div divides by it)
  for (int64_t e = (int64_t)blockIdx.x * kDqWaves + threadIdx.x / kWave; e < entries;
       e += stride) {
    Run run;
    if (!table_entry_run(block_table, cu_seq_lens, e, max_blocks, num_tokens, num_blocks,
                         block_size, run))
      continue;
    const uint8_t* page = kv_cache + run.page * page_stride;
    const u32x2* csrc = reinterpret_cast<const u32x2*>(page + run.first * head_dim);
    const float* ssrc =
        reinterpret_cast<const float*>(page + (int64_t)block_size * head_dim) + run.first;
    uint16_t* orow = out + run.row * out_row_stride;
    const int32_t units = (int32_t)run.rows * upt;  // <= block_size * head_dim / 8
    // runs of up to 64 tokens: lane l holds the scale of token l, and each
    // unit takes its token's scale across lanes; longer runs load per unit
    const bool lane_scales = run.rows <= kWave;
    float my_scale = 0.0f;
    if (lane_scales && lane < run.rows) my_scale = ssrc[lane];
    for (int32_t c0 = 0; c0 < units; c0 += kWave * kIdxUnroll) {
      u32x2 v[kIdxUnroll];
      float sc[kIdxUnroll];
#pragma unroll
      for (int u = 0; u < kIdxUnroll; ++u) {
        const int32_t c = c0 + u * kWave + lane;
        v[u] = u32x2{0u, 0u};
        sc[u] = 0.0f;
        if (c < units) {
          v[u] = __builtin_nontemporal_load(csrc + c);
          if (!lane_scales) sc[u] = ssrc[upt_div.div((uint32_t)c)];
        }
      }
      if (lane_scales) {
#pragma unroll
        for (int u = 0; u < kIdxUnroll; ++u) {  // every lane takes part
          const int32_t c = c0 + u * kWave + lane;
          const int32_t t = c < units ? (int32_t)upt_div.div((uint32_t)c) : 0;
          sc[u] = __uint_as_float(
              (uint32_t)__builtin_amdgcn_ds_bpermute(t << 2, (int)__float_as_uint(my_scale)));
        }
      }
#pragma unroll
      for (int u = 0; u < kIdxUnroll; ++u) {
        const int32_t c = c0 + u * kWave + lane;
        if (c >= units) continue;
        const int32_t t = (int32_t)upt_div.div((uint32_t)c);
        const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[u].x, false);
        const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[u].x, true);
        const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[u].y, false);
        const f32x2 g = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[u].y, true);
        const float x = sc[u];
        const u32x4 o = {narrow2<kF16>(a.x * x, a.y * x), narrow2<kF16>(b.x * x, b.y * x),
                         narrow2<kF16>(d.x * x, d.y * x), narrow2<kF16>(g.x * x, g.y * x)};
        store_stream(reinterpret_cast<u32x4*>(orow + (int64_t)t * out_row_stride +
                                              (int64_t)(c - t * upt) * 8),
                     o);
      }
    }
  }
}

// Staged variant (runs of at most 64 tokens whose code rows fit 8 KB): the
// wave first copies the run's code rows into its LDS slice with
// global_load_lds_dwordx4 (all of them in flight at once, no registers
// held), then produces the same units from LDS.  The direct kernel keeps a
// few units' loads in flight and waits for them before every group of
// stores.
constexpr int kIdxStageMax = 8192;  // code bytes of one run, at most
constexpr int kIdxStageChunks = kIdxStageMax / (16 * kWave);  // 16-byte loads per lane

template <bool kF16>
__global__ __launch_bounds__(kDqThreads) void gather_indexer_k_dequant_staged_kernel(
    const uint8_t* __restrict__ kv_cache, uint16_t* __restrict__ out, int64_t out_row_stride,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ cu_seq_lens,
    int32_t num_reqs, int32_t max_blocks, int64_t num_tokens, int64_t num_blocks,
    int64_t page_stride, int32_t block_size, int32_t head_dim, FastDiv upt_div) {
  __shared__ __align__(16) uint8_t stage_lds[kDqWaves][kIdxStageMax];
  const int lane = threadIdx.x & (kWave - 1);
  uint8_t* stage = stage_lds[threadIdx.x / kWave];
  const int64_t entries = (int64_t)num_reqs * max_blocks;
  const int64_t stride = (int64_t)gridDim.x * kDqWaves;
  const int32_t upt = head_dim / 8;  // 8-code units per token (upt_div divides by it)
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
    const int32_t chunks = (int32_t)run.rows * head_dim / 16;
    // the previous run's LDS reads have all returned (their values were stored)
    wave_sync();
#pragma unroll
    for (int i = 0; i < kIdxStageChunks; ++i) {
      const int q = lane + kWave * i;
      if (q < chunks)
        __builtin_amdgcn_global_load_lds(csrc + q, (__attribute__((address_space(3))) void*)(stage + i * kWave * 16), 16, 0, 0);
    }
    // lane l holds the scale of token l (runs have at most 64 tokens)
    const float my_scale = lane < run.rows ? ssrc[lane] : 0.0f;
    __builtin_amdgcn_s_waitcnt(0);  // every load of this wave has written LDS
    wave_sync();

    uint16_t* orow = out + run.row * out_row_stride;
    const int32_t units = (int32_t)run.rows * upt;
    for (int32_t c0 = 0; c0 < units; c0 += kWave * kIdxUnroll) {
      u32x2 v[kIdxUnroll];
      float sc[kIdxUnroll];
#pragma unroll
      for (int u = 0; u < kIdxUnroll; ++u) {  // every lane takes part (bpermute)
        const int32_t c = c0 + u * kWave + lane;
        const int32_t t = c < units ? (int32_t)upt_div.div((uint32_t)c) : 0;
        v[u] = c < units ? *reinterpret_cast<const u32x2*>(stage + c * 8) : u32x2{0u, 0u};
        sc[u] = __uint_as_float(
            (uint32_t)__builtin_amdgcn_ds_bpermute(t << 2, (int)__float_as_uint(my_scale)));
      }
#pragma unroll
      for (int u = 0; u < kIdxUnroll; ++u) {
        const int32_t c = c0 + u * kWave + lane;
        if (c >= units) continue;
        const int32_t t = (int32_t)upt_div.div((uint32_t)c);
        const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[u].x, false);
        const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[u].x, true);
        const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[u].y, false);
        const f32x2 g = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[u].y, true);
        const float x = sc[u];
        const u32x4 o = {narrow2<kF16>(a.x * x, a.y * x), narrow2<kF16>(b.x * x, b.y * x),
                         narrow2<kF16>(d.x * x, d.y * x), narrow2<kF16>(g.x * x, g.y * x)};
        store_stream(reinterpret_cast<u32x4*>(orow + (int64_t)t * out_row_stride +
                                              (int64_t)(c - t * upt) * 8),
                     o);
      }
    }
  }
}

// ------------------------------------------------------------- NVFP4 K/V
// Work of a wave: one (table entry, side) -- the run's tokens, every head.
// Lane unit = one half-block (4 code bytes, 8 elements of one token head) ->
// 8 outputs (one 16-byte store); units run in output order, so a token's row
// of H*D outputs is written by consecutive lanes and every wave store covers
// 1 KB of it.
template <int kD, bool kF16>
__global__ __launch_bounds__(kDqThreads) void gather_kv_fp4_dequant_kernel(
    const uint8_t* __restrict__ key_cache, const uint8_t* __restrict__ value_cache,
    uint16_t* __restrict__ key_out, int64_t key_row_stride, uint16_t* __restrict__ value_out,
    int64_t value_row_stride, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ cu_seq_lens, int32_t num_reqs, int32_t max_blocks,
    int64_t num_tokens, int32_t num_heads, int32_t head_size, int32_t block_size,
    int64_t num_blocks, int64_t page_stride, int32_t layout, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, FastDiv upt_div, FastDiv hpt_div, FastDiv q4_div) {
  const int lane = threadIdx.x & (kWave - 1);
  const float ts_k = *k_scale, ts_v = *v_scale;
  if constexpr (kD > 0) head_size = kD;
  const int32_t S = head_size / 16;
  const int32_t hpt = head_size / 8;       // half-blocks per token head
  const int32_t upt = num_heads * hpt;     // half-blocks per token (upt_div divides by it)
  const int64_t data_dim = head_size / 2;
  const int64_t data_per_side = (int64_t)num_heads * block_size * data_dim;
  const int64_t units_total = (int64_t)num_reqs * max_blocks * 2;
  const int64_t stride = (int64_t)gridDim.x * kDqWaves;
  for (int64_t w = (int64_t)blockIdx.x * kDqWaves + threadIdx.x / kWave; w < units_total;
       w += stride) {
    const int64_t e = w >> 1;
    const int kv = (int)(w & 1);
    Run run;
    if (!table_entry_run(block_table, cu_seq_lens, e, max_blocks, num_tokens, num_blocks,
                         block_size, run))
      continue;
    const uint8_t* side = (kv ? value_cache : key_cache) + run.page * page_stride;
    const uint8_t* scales = side + data_per_side;
    uint16_t* orow = (kv ? value_out : key_out) + run.row * (kv ? value_row_stride : key_row_stride);
    const int64_t out_stride = kv ? value_row_stride : key_row_stride;
    const float ts = kv ? ts_v : ts_k;
    const int32_t units = (int32_t)run.rows * upt;
    for (int32_t c0 = 0; c0 < units; c0 += kWave * kFp4Unroll) {
      uint32_t v[kFp4Unroll], sb[kFp4Unroll];
#pragma unroll
      for (int u = 0; u < kFp4Unroll; ++u) {
        const int32_t c = c0 + u * kWave + lane;
        v[u] = 0u;
        sb[u] = 0u;
        if (c < units) {
          const int32_t t = (int32_t)upt_div.div((uint32_t)c);
          const int32_t r = c - t * upt;
          const int32_t h = kD > 0 ? r / (kD / 8) : (int32_t)hpt_div.div((uint32_t)r);
          const int32_t hb = r - h * hpt;  // half-block within the head
          const int32_t g = hb >> 1;
          const int64_t off = run.first + t;
          const int64_t row = layout == PKV_LAYOUT_HND ? (int64_t)h * block_size + off
                                                       : off * num_heads + h;
          v[u] = __builtin_nontemporal_load(
              reinterpret_cast<const uint32_t*>(side + row * data_dim) + hb);
          int64_t so;
          if (kv == 0) {
            so = row * S + g;
          } else {
            // swizzled: (t', s') = ((off/4)*4 + g/(S/4), (g % (S/4))*4 + off%4)
            const int32_t gq = kD > 0 ? g / (kD / 64) : (int32_t)q4_div.div((uint32_t)g);
            const int32_t gr = g - gq * (S / 4);
            const int64_t srow = (off >> 2) * 4 + gq;
            const int64_t col = (int64_t)gr * 4 + (off & 3);
            so = (layout == PKV_LAYOUT_HND ? ((int64_t)h * block_size + srow) * S
                                           : (srow * num_heads + h) * S) + col;
          }
          sb[u] = scales[so];
        }
      }
#pragma unroll
      for (int u = 0; u < kFp4Unroll; ++u) {
        const int32_t c = c0 + u * kWave + lane;
        if (c >= units) continue;
        const int32_t t = (int32_t)upt_div.div((uint32_t)c);
        const float sfd = __builtin_amdgcn_cvt_f32_fp8((int)sb[u], 0);
        const u32x4 o = {fp4_pair<0, kF16>(v[u], sfd, ts), fp4_pair<1, kF16>(v[u], sfd, ts),
                         fp4_pair<2, kF16>(v[u], sfd, ts), fp4_pair<3, kF16>(v[u], sfd, ts)};
        store_stream(reinterpret_cast<u32x4*>(orow + (int64_t)t * out_stride +
                                              (int64_t)(c - t * upt) * 8),
                     o);
      }
    }
  }
}

// Staged variant (head_size 64, 128 or 256, page sides of at most 16 KB,
// 16-byte aligned): a wave first copies its whole page side -- every head's
// codes and block scales, H*B*(D/2 + D/16) contiguous bytes -- into its LDS
// slice with 16-byte loads that write LDS directly (global_load_lds_dwordx4:
// lane i's 16 bytes land at the instruction's LDS base + 16 i, no registers
// held), then produces the same units, reading each unit's code dword and
// scale byte from LDS.  The 4- and 1-byte global loads of the direct kernel
// become whole-line loads; bytes of the page past the run are read but not
// used.
constexpr int kFp4StageMax = 16384;  // bytes of one page side, at most
constexpr int kFp4EmitUnroll = 16;   // tokens per lane in flight while emitting

template <int kD, bool kF16, int kChunks>  // kChunks: 16-byte loads per lane, at most
__global__ __launch_bounds__(kDqThreads) void gather_kv_fp4_dequant_staged_kernel(
    const uint8_t* __restrict__ key_cache, const uint8_t* __restrict__ value_cache,
    uint16_t* __restrict__ key_out, int64_t key_row_stride, uint16_t* __restrict__ value_out,
    int64_t value_row_stride, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ cu_seq_lens, int32_t num_reqs, int32_t max_blocks,
    int64_t num_tokens, int32_t num_heads, int32_t block_size, int64_t num_blocks,
    int64_t page_stride, int32_t layout, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, int32_t side_bytes) {
  extern __shared__ __align__(16) uint8_t stage_lds[];  // [kDqWaves][side_bytes]
  constexpr int S = kD / 16;       // blocks (scale bytes) per token head
  constexpr int hpt = kD / 8;      // half-blocks per token head
  constexpr int data_dim = kD / 2;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  uint8_t* stage = stage_lds + (int64_t)wave * side_bytes;
  const float ts_k = *k_scale, ts_v = *v_scale;
  const int32_t upt = num_heads * hpt;  // half-blocks per token
  const int32_t data_per_side = num_heads * block_size * data_dim;
  const int32_t chunks = side_bytes / 16;
  const int64_t units_total = (int64_t)num_reqs * max_blocks * 2;
  const int64_t stride = (int64_t)gridDim.x * kDqWaves;
  for (int64_t w = (int64_t)blockIdx.x * kDqWaves + threadIdx.x / kWave; w < units_total;
       w += stride) {
    const int64_t e = w >> 1;
    const int kv = (int)(w & 1);
    Run run;
    if (!table_entry_run(block_table, cu_seq_lens, e, max_blocks, num_tokens, num_blocks,
                         block_size, run))
      continue;
    // ---- the page side into LDS: chunk q = lane + 64 i lands at stage + 16 q.
    // The previous unit's LDS reads have all returned (their values were
    // stored), so the slice can be overwritten.
    const u32x4* side =
        reinterpret_cast<const u32x4*>((kv ? value_cache : key_cache) + run.page * page_stride);
    wave_sync();
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int q = lane + kWave * i;
      if (q < chunks)
        __builtin_amdgcn_global_load_lds(side + q, (__attribute__((address_space(3))) void*)(stage + i * kWave * 16), 16, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);  // every load of this wave has written LDS
    wave_sync();

    // ---- units from LDS.  Lane slot r (= half-block hb of head h within a
    // token row of upt half-blocks) is fixed for a pass over the run's
    // tokens, so the code and scale offsets of token offset `off` are a base
    // plus a per-token step: codes at cbase + off * cstep, scales at
    // sbase + (off >> ssh) * sstep + (off & smask) (V scales are swizzled in
    // groups of four tokens).  Each pass stores 64 consecutive units of a
    // token row (1 KB) per instruction.
    const uint8_t* scales = stage + data_per_side;
    uint16_t* orow = (kv ? value_out : key_out) + run.row * (kv ? value_row_stride : key_row_stride);
    const int64_t out_stride = kv ? value_row_stride : key_row_stride;
    const float ts = kv ? ts_v : ts_k;
    const int32_t rows = (int32_t)run.rows;
    const bool hnd = layout == PKV_LAYOUT_HND;
    for (int32_t r0 = 0; r0 < upt; r0 += kWave) {
      const int32_t r = r0 + lane;
      const bool live = r < upt;
      const int32_t h = r / hpt;
      const int32_t hb = r - h * hpt;
      const int32_t g = hb >> 1;
      const int32_t cbase = (hnd ? h * block_size : h) * data_dim + hb * 4;
      const int32_t cstep = hnd ? data_dim : num_heads * data_dim;
      int32_t sbase, sstep, ssh, smask;
      if (kv == 0) {
        sbase = (hnd ? h * block_size : h) * S + g;
        sstep = hnd ? S : num_heads * S;
        ssh = 0;
        smask = 0;
      } else {
        // swizzled: token offset off, block g -> row (off/4)*4 + g/(S/4), column (g % (S/4))*4 + off%4
        const int32_t gq = g / (S / 4);
        const int32_t gr = g - gq * (S / 4);
        sbase = (hnd ? (h * block_size + gq) * S : (gq * num_heads + h) * S) + gr * 4;
        sstep = hnd ? 4 * S : 4 * num_heads * S;
        ssh = 2;
        smask = 3;
      }
      uint16_t* obase = orow + (int64_t)r * 8;
      for (int32_t t0 = 0; t0 < rows; t0 += kFp4EmitUnroll) {
        uint32_t v[kFp4EmitUnroll], sb[kFp4EmitUnroll];
#pragma unroll
        for (int u = 0; u < kFp4EmitUnroll; ++u) {
          const int32_t off = (int32_t)run.first + t0 + u;
          const bool on = live && t0 + u < rows;
          v[u] = on ? *reinterpret_cast<const uint32_t*>(stage + cbase + off * cstep) : 0u;
          sb[u] = on ? scales[sbase + (off >> ssh) * sstep + (off & smask)] : 0u;
        }
#pragma unroll
        for (int u = 0; u < kFp4EmitUnroll; ++u) {
          if (!live || t0 + u >= rows) continue;
          const float sfd = __builtin_amdgcn_cvt_f32_fp8((int)sb[u], 0);
          const u32x4 o = {fp4_pair<0, kF16>(v[u], sfd, ts), fp4_pair<1, kF16>(v[u], sfd, ts),
                           fp4_pair<2, kF16>(v[u], sfd, ts), fp4_pair<3, kF16>(v[u], sfd, ts)};
          store_stream(reinterpret_cast<u32x4*>(obase + (int64_t)(t0 + u) * out_stride), o);
        }
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
  const bool f16 = a.out_dtype == PKV_DTYPE_F16;
  // staged kernel: runs of at most 64 tokens, code rows of at most 8 KB
  const bool staged = a.block_size <= kWave && (int64_t)a.block_size * a.head_dim <= kIdxStageMax;
  auto kernel = staged ? (f16 ? gather_indexer_k_dequant_staged_kernel<true>
                              : gather_indexer_k_dequant_staged_kernel<false>)
                       : (f16 ? gather_indexer_k_dequant_kernel<true>
                              : gather_indexer_k_dequant_kernel<false>);
  hipLaunchKernelGGL(kernel, dim3((unsigned)dq_blocks(entries)), dim3(kDqThreads), 0, stream,
                     a.kv_cache, a.out, a.out_row_stride, a.block_table, a.cu_seq_lens,
                     a.num_reqs, a.max_blocks_per_req, a.num_tokens, a.num_blocks,
                     a.cache_block_stride, a.block_size, a.head_dim,
                     FastDiv::make((uint32_t)(a.head_dim / 8)));
  return (int)hipGetLastError();
}

template <int kD, bool kF16>
int launch_fp4_staged(const GatherFp4DequantArgs& a, int64_t units, int32_t side_bytes,
                      hipStream_t stream) {
  const int chunks = (side_bytes / 16 + kWave - 1) / kWave;  // 16-byte loads per lane
  auto kernel = gather_kv_fp4_dequant_staged_kernel<kD, kF16, 16>;
  if (chunks <= 4) kernel = gather_kv_fp4_dequant_staged_kernel<kD, kF16, 4>;
  else if (chunks <= 8) kernel = gather_kv_fp4_dequant_staged_kernel<kD, kF16, 8>;
  else if (chunks <= 12) kernel = gather_kv_fp4_dequant_staged_kernel<kD, kF16, 12>;
  hipLaunchKernelGGL(kernel, dim3((unsigned)dq_blocks(units)), dim3(kDqThreads),
                     (size_t)kDqWaves * side_bytes, stream, a.key_cache, a.value_cache, a.key_out,
                     a.key_row_stride, a.value_out, a.value_row_stride, a.block_table,
                     a.cu_seq_lens, a.num_reqs, a.max_blocks_per_req, a.num_tokens, a.num_heads,
                     a.block_size, a.num_blocks, a.page_stride, a.layout, a.k_scale, a.v_scale,
                     side_bytes);
  return (int)hipGetLastError();
}

int launch_gather_kv_fp4_dequant(const GatherFp4DequantArgs& a, hipStream_t stream) {
  const int64_t units = (int64_t)a.num_reqs * a.max_blocks_per_req * 2;
  const bool f16 = a.out_dtype == PKV_DTYPE_F16;
  // staged kernel: whole page sides of at most kFp4StageMax bytes, 16-byte aligned
  const int64_t side_bytes =
      (int64_t)a.num_heads * a.block_size * (a.head_size / 2 + a.head_size / 16);
  const bool aligned16 = ((uintptr_t)a.key_cache % 16) == 0 && ((uintptr_t)a.value_cache % 16) == 0 &&
                         a.page_stride % 16 == 0 && side_bytes % 16 == 0;
  if (aligned16 && side_bytes <= kFp4StageMax) {
    switch (a.head_size) {
      case 64: return f16 ? launch_fp4_staged<64, true>(a, units, (int32_t)side_bytes, stream)
                          : launch_fp4_staged<64, false>(a, units, (int32_t)side_bytes, stream);
      case 128: return f16 ? launch_fp4_staged<128, true>(a, units, (int32_t)side_bytes, stream)
                           : launch_fp4_staged<128, false>(a, units, (int32_t)side_bytes, stream);
      case 256: return f16 ? launch_fp4_staged<256, true>(a, units, (int32_t)side_bytes, stream)
                           : launch_fp4_staged<256, false>(a, units, (int32_t)side_bytes, stream);
      default: break;
    }
  }
  auto kernel = f16 ? gather_kv_fp4_dequant_kernel<0, true> : gather_kv_fp4_dequant_kernel<0, false>;
  if (a.head_size == 64) kernel = f16 ? gather_kv_fp4_dequant_kernel<64, true> : gather_kv_fp4_dequant_kernel<64, false>;
  if (a.head_size == 128) kernel = f16 ? gather_kv_fp4_dequant_kernel<128, true> : gather_kv_fp4_dequant_kernel<128, false>;
  if (a.head_size == 256) kernel = f16 ? gather_kv_fp4_dequant_kernel<256, true> : gather_kv_fp4_dequant_kernel<256, false>;
  const uint32_t hpt = (uint32_t)(a.head_size / 8);
  hipLaunchKernelGGL(kernel, dim3((unsigned)dq_blocks(units)), dim3(kDqThreads), 0, stream,
                     a.key_cache, a.value_cache, a.key_out, a.key_row_stride, a.value_out,
                     a.value_row_stride, a.block_table, a.cu_seq_lens, a.num_reqs,
                     a.max_blocks_per_req, a.num_tokens, a.num_heads, a.head_size, a.block_size,
                     a.num_blocks, a.page_stride, a.layout, a.k_scale, a.v_scale,
                     FastDiv::make(hpt * (uint32_t)a.num_heads), FastDiv::make(hpt),
                     FastDiv::make((uint32_t)(a.head_size / 64)));
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
