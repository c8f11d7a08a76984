// Gather of fp8 indexer keys and their per-token scales out of the paged
// indexer K cache (vLLM PR "Add gather_indexer_k_quant_cache kernel": the op
// is called with kv_cache, k_fp8, k_scale, block_table, cu_seq_lens; the
// review of that PR notes a launch-grid bug that gathered long sequences
// wrongly, which is why nothing here sizes a grid from a sequence length).
//
// Work unit: a page run, i.e. the <= block_size consecutive tokens of one
// request that live in one page.  A run starts at page offset 0, so its
// code bytes are one contiguous span of the page and one contiguous span of
// k_fp8; likewise for its scale dwords.  One wavefront copies one run with
// 16-byte loads and stores (8 per lane for a 64 x 128-byte run), then the
// scale dwords, one per lane.
//
// Which wave copies which run:
//  - dense tables (at most about twice as many entries as page runs): wave w
//    takes block-table entry (w / max_blocks, w % max_blocks) and exits at
//    once if that column holds no tokens;
//  - otherwise every workgroup builds the exclusive prefix sum of runs per
//    request, min(ceil(len_r / block_size), max_blocks_per_req), in LDS from
//    cu_seq_lens, and each wave finds its request by binary search.
// In both, waves stride over the work until all of it is done, so the grid
// size only sets parallelism, never coverage.
#include "device_common.h"
#include "launch.h"

namespace pkv {

namespace {

constexpr int kGatherThreads = 256;
constexpr int kGatherWaves = kGatherThreads / kWave;
constexpr int kGatherUnroll = 8;  // 16-byte chunks per lane in flight

// Copy tokens [j*B + o_lo, j*B + o_hi) of a request whose rows are
// [start, end) of the output, clipped to the request: page offsets
// [o_lo, o_hi) of page `page`.  Rows outside [0, num_tokens) and pages
// outside [0, num_blocks) are skipped.  Executed by one whole wave.
__device__ __forceinline__ void copy_run(const uint8_t* __restrict__ kv_cache,
                                         uint8_t* __restrict__ k_fp8,
                                         uint8_t* __restrict__ k_scale, int64_t start,
                                         int64_t end, int64_t page, int32_t j, int32_t o_lo,
                                         int32_t o_hi, int64_t num_tokens, int64_t num_blocks,
                                         int64_t page_stride, int32_t block_size,
                                         int32_t head_dim, int lane) {
  const int64_t len = end - start;
  if (page < 0 || page >= num_blocks) return;
  const int64_t i0 = (int64_t)j * block_size + o_lo;
  if (i0 >= len) return;
  const int64_t n = (len - i0 < o_hi - o_lo) ? (len - i0) : (o_hi - o_lo);
  const int64_t row0 = start + i0;
  const int64_t rb = row0 > 0 ? row0 : 0;
  const int64_t re = (row0 + n < num_tokens) ? row0 + n : num_tokens;
  if (rb >= re) return;

  const uint8_t* src = kv_cache + page * page_stride;
  const int64_t first = o_lo + (rb - row0);  // first page offset copied
  const int64_t rows = re - rb;

  // scale dwords (issued first; at most block_size of them)
  const uint32_t* ssrc =
      reinterpret_cast<const uint32_t*>(src + (int64_t)block_size * head_dim) + first;
  uint32_t* sdst = reinterpret_cast<uint32_t*>(k_scale) + rb;
  uint32_t sv = 0;
  const bool has_scale = lane < rows;
  if (has_scale) sv = ssrc[lane];

  // code rows: one contiguous span of rows*head_dim bytes
  const u32x4* csrc = reinterpret_cast<const u32x4*>(src + first * head_dim);
  u32x4* cdst = reinterpret_cast<u32x4*>(k_fp8 + rb * head_dim);
  const int64_t chunks = rows * head_dim / 16;
  for (int64_t c0 = 0; c0 < chunks; c0 += kWave * kGatherUnroll) {
    u32x4 v[kGatherUnroll];
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) {
      const int64_t c = c0 + u * kWave + lane;
      if (c < chunks) v[u] = load_stream(csrc + c);
    }
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) {
      const int64_t c = c0 + u * kWave + lane;
      if (c < chunks) store_stream(cdst + c, v[u]);
    }
  }
  if (has_scale) sdst[lane] = sv;
  for (int64_t c = lane + kWave; c < rows; c += kWave) sdst[c] = ssrc[c];
}

// Dense tables: wave w copies block-table entry (r, j) = (w / max_blocks,
// w % max_blocks) when that column holds tokens of request r.  The three
// metadata loads are independent, so a wave reaches its data after one
// round trip.  Used when the table has at most about twice as many entries
// as there can be page runs.
__global__ __launch_bounds__(kGatherThreads) void gather_indexer_k_fp8_direct_kernel(
    const uint8_t* __restrict__ kv_cache, uint8_t* __restrict__ k_fp8,
    uint8_t* __restrict__ k_scale, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ cu_seq_lens, int32_t num_reqs, int32_t max_blocks,
    int64_t num_tokens, int64_t num_blocks, int64_t page_stride, int32_t block_size,
    int32_t head_dim) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t entries = (int64_t)num_reqs * max_blocks;
  const int64_t stride = (int64_t)gridDim.x * kGatherWaves;
  for (int64_t e = (int64_t)blockIdx.x * kGatherWaves + threadIdx.x / kWave; e < entries;
       e += stride) {
    const int32_t r = (int32_t)(e / max_blocks);
    const int32_t j = (int32_t)(e - (int64_t)r * max_blocks);
    copy_run(kv_cache, k_fp8, k_scale, cu_seq_lens[r], cu_seq_lens[r + 1], block_table[e], j,
             0, block_size, num_tokens, num_blocks, page_stride, block_size, head_dim, lane);
  }
}

__global__ __launch_bounds__(kGatherThreads) void gather_indexer_k_fp8_kernel(
    const uint8_t* __restrict__ kv_cache, uint8_t* __restrict__ k_fp8,
    uint8_t* __restrict__ k_scale, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ cu_seq_lens, int32_t num_reqs, int32_t max_blocks,
    int64_t num_tokens, int64_t num_blocks, int64_t page_stride, int32_t block_size,
    int32_t head_dim) {
  extern __shared__ int32_t run_start[];  // [num_reqs + 1]
  __shared__ int32_t wave_total[kGatherWaves];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;

  // ---- exclusive prefix sum of page runs per request, in place in LDS.
  // Stage cu_seq_lens[0..R] (coalesced), then thread tid owns the
  // contiguous slice [r_begin, r_end) of requests.
  for (int32_t i = tid; i <= num_reqs; i += kGatherThreads) run_start[i] = cu_seq_lens[i];
  __syncthreads();
  const int32_t per = (num_reqs + kGatherThreads - 1) / kGatherThreads;
  const int32_t r_begin = min(tid * per, num_reqs);
  const int32_t r_end = min(r_begin + per, num_reqs);
  const int64_t boundary = run_start[r_end];  // read before any slice is overwritten
  __syncthreads();
  int32_t local = 0;
  for (int32_t r = r_begin; r < r_end; ++r) {
    const int64_t next = (r + 1 < r_end) ? (int64_t)run_start[r + 1] : boundary;
    const int64_t len = next - (int64_t)run_start[r];
    int32_t runs = 0;
    if (len > 0) {
      const int64_t n = (len + block_size - 1) / block_size;
      runs = (int32_t)(n < max_blocks ? n : max_blocks);
    }
    run_start[r] = local;  // slice-local exclusive prefix
    local += runs;
  }
  const int32_t incl = wave_inclusive_scan(local);
  if (lane == kWave - 1) wave_total[wave] = incl;
  __syncthreads();
  int32_t before = incl - local, total_runs = 0;
#pragma unroll
  for (int w = 0; w < kGatherWaves; ++w) {
    before += (w < wave) ? wave_total[w] : 0;
    total_runs += wave_total[w];
  }
  for (int32_t r = r_begin; r < r_end; ++r) run_start[r] += before;
  if (tid == 0) run_start[num_reqs] = total_runs;
  __syncthreads();

  // ---- copy runs
  const int64_t stride = (int64_t)gridDim.x * kGatherWaves;
  for (int64_t run64 = (int64_t)blockIdx.x * kGatherWaves + wave; run64 < total_runs;
       run64 += stride) {
    const int32_t run = (int32_t)run64;
    // request r: run_start[r] <= run < run_start[r + 1]
    int32_t lo = 0, hi = num_reqs;
    while (hi - lo > 1) {
      const int32_t mid = (lo + hi) >> 1;
      if (run_start[mid] <= run) lo = mid; else hi = mid;
    }
    const int32_t r = lo;
    const int32_t j = run - run_start[r];

    copy_run(kv_cache, k_fp8, k_scale, cu_seq_lens[r], cu_seq_lens[r + 1],
             block_table[(int64_t)r * max_blocks + j], j, 0, block_size, num_tokens, num_blocks,
             page_stride, block_size, head_dim, lane);
  }
}

}  // namespace

#ifndef PKV_GATHER_MODE
#define PKV_GATHER_MODE 0  // 0: choose per call, 1: always prefix scan, 2: always direct
#endif

int launch_gather_indexer_k_fp8(const GatherArgs& a, hipStream_t stream) {
  // Upper bound on page runs when the rows fit num_tokens: sum(len)/B + R.
  const int64_t table = (int64_t)a.num_reqs * a.max_blocks_per_req;
  const int64_t run_bound = (a.num_tokens + a.block_size - 1) / a.block_size + a.num_reqs;
  const bool direct = PKV_GATHER_MODE == 2 || (PKV_GATHER_MODE == 0 && table <= 2 * run_bound);
  if (direct) {
    int64_t blocks = (table + kGatherWaves - 1) / kGatherWaves;
    if (blocks > kGatherMaxBlocks) blocks = kGatherMaxBlocks;
    hipLaunchKernelGGL(gather_indexer_k_fp8_direct_kernel, dim3((unsigned)blocks),
                       dim3(kGatherThreads), 0, stream, a.kv_cache, a.k_fp8, a.k_scale,
                       a.block_table, a.cu_seq_lens, a.num_reqs, a.max_blocks_per_req,
                       a.num_tokens, a.num_blocks, a.cache_block_stride, a.block_size,
                       a.head_dim);
    return (int)hipGetLastError();
  }
  // Requests are independent, so a table with more requests than one
  // workgroup's LDS prefix array can hold is processed in request chunks.
  const int64_t max_chunk = kGatherMaxReqsPerLaunch;
  for (int64_t r0 = 0; r0 < a.num_reqs; r0 += max_chunk) {
    const int32_t R = (int32_t)((a.num_reqs - r0) < max_chunk ? (a.num_reqs - r0) : max_chunk);
    // More runs than this bound are still all copied (grid-stride loop).
    int64_t bound = (a.num_tokens + a.block_size - 1) / a.block_size + R;
    const int64_t chunk_table = (int64_t)R * a.max_blocks_per_req;
    if (chunk_table < bound) bound = chunk_table;
    int64_t blocks = (bound + kGatherWaves - 1) / kGatherWaves;
    if (blocks < 1) blocks = 1;
    if (blocks > kGatherMaxBlocks) blocks = kGatherMaxBlocks;
    const size_t lds = sizeof(int32_t) * ((size_t)R + 1);
    hipLaunchKernelGGL(gather_indexer_k_fp8_kernel, dim3((unsigned)blocks), dim3(kGatherThreads),
                       lds, stream, a.kv_cache, a.k_fp8, a.k_scale,
                       a.block_table + r0 * a.max_blocks_per_req, a.cu_seq_lens + r0, R,
                       a.max_blocks_per_req, a.num_tokens, a.num_blocks, a.cache_block_stride,
                       a.block_size, a.head_dim);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
  }
  return 0;
}

}  // namespace pkv
