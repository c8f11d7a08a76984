// Gather of fp8 indexer keys and their per-token scales out of the paged
// indexer K cache (vLLM PR "Add gather_indexer_k_quant_cache kernel": the op
// is called with kv_cache, k_fp8, k_scale, block_table, cu_seq_lens; the
// review of that PR notes a launch-grid bug that gathered long sequences
// wrongly, which is why nothing here sizes a grid from a sequence length).
//
// Work unit: a page run, i.e. the <= block_size consecutive tokens of one
// request that live in one page.  A run starts at page offset 0, so its
// code bytes are one contiguous span of the page and one contiguous span of
// k_fp8; likewise for its scale dwords.
//
// Which wave copies which runs:
//  - dense tables (at most about twice as many entries as page runs): one
//    wave per group of consecutive block-table entries (entry e is request
//    e / max_blocks, column e % max_blocks; a column holding no tokens copies
//    nothing).  The grid is sized from the table's entry count, which the
//    host knows.  For page shapes whose run is a whole number of wave-wide
//    16-byte loads (kU per lane) and at most 64 tokens, a group is kK runs
//    with kK * kU = 16 loads per lane, all in flight before the first store:
//    16 KB per wave for 64 x 128-byte runs.  On the 256 x 1000-token batch
//    (interleaved runs on one GPU, kernel trace) one 8 KB run per wave took
//    12.3 us, two per wave 11.0-11.5 us, four per wave 12.7 us, and two per
//    wave copied one after the other 14.0 us.  Other shapes: one run per
//    wave, a generic loop;
//  - otherwise every workgroup builds the exclusive prefix sum of runs per
//    request, min(ceil(len_r / block_size), max_blocks_per_req), in LDS from
//    cu_seq_lens; its waves stride over the runs, one at a time, each
//    finding its request by binary search, until all are done.
#include "device_common.h"
#include "launch.h"

namespace pkv {

namespace {

constexpr int kGatherThreads = 256;
constexpr int kGatherWaves = kGatherThreads / kWave;

// One page run, as the copy needs it (wave-uniform): `rows` tokens whose
// code bytes start at `codes` in the page and whose scale dwords start at
// `scales`, going to output rows [row, row + rows).  rows == 0: nothing.
struct Run {
  const uint8_t* codes;
  const uint32_t* scales;
  int32_t row;
  int32_t rows;
};

// Page run j of the request whose output rows are [start, end): tokens
// [j*B, min((j+1)*B, end - start)) in page `page`, clipped to output rows
// [0, num_tokens).  Pages outside [0, num_blocks) copy nothing.  Output rows
// are below 2^31: they are less than some cu_seq_lens value.
__device__ __forceinline__ Run describe_run(const uint8_t* kv_cache, int32_t start, int32_t end,
                                            int32_t page, int32_t j, int64_t num_tokens,
                                            int64_t num_blocks, int64_t page_stride,
                                            int32_t block_size, int32_t head_dim) {
  Run run{kv_cache, reinterpret_cast<const uint32_t*>(kv_cache), 0, 0};
  const int64_t len = (int64_t)end - start;
  const int64_t i0 = (int64_t)j * block_size;
  if (page >= 0 && page < num_blocks && i0 < len) {
    const int64_t n = (len - i0 < block_size) ? (len - i0) : block_size;
    const int64_t row0 = start + i0;
    const int64_t rb = row0 > 0 ? row0 : 0;
    const int64_t re = (row0 + n < num_tokens) ? row0 + n : num_tokens;
    if (rb < re) {
      const int64_t first = rb - row0;  // page offset of the first copied token
      const uint8_t* page_base = kv_cache + (int64_t)page * page_stride;
      run.codes = page_base + first * head_dim;
      run.scales = reinterpret_cast<const uint32_t*>(page_base + (int64_t)block_size * head_dim) + first;
      run.row = (int32_t)rb;
      run.rows = (int32_t)(re - rb);
    }
  }
  return run;
}

// Any run: a loop of wave-wide 16-byte chunks, eight per lane in flight,
// then the scale dwords.  Executed by one whole wave.
__device__ __forceinline__ void copy_run_any(const Run& run, uint8_t* __restrict__ k_fp8,
                                             uint32_t* __restrict__ k_scale, int32_t head_dim,
                                             int lane) {
  constexpr int kUnroll = 8;
  const int64_t chunks = (int64_t)run.rows * (head_dim / 16);
  const u32x4* src = reinterpret_cast<const u32x4*>(run.codes);
  u32x4* dst = reinterpret_cast<u32x4*>(k_fp8 + (int64_t)run.row * head_dim);
  for (int64_t c0 = 0; c0 < chunks; c0 += kWave * kUnroll) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t c = c0 + u * kWave + lane;
      if (c < chunks) v[u] = load_stream(src + c);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t c = c0 + u * kWave + lane;
      if (c < chunks) store_stream(dst + c, v[u]);
    }
  }
  for (int32_t c = lane; c < run.rows; c += kWave) k_scale[run.row + c] = run.scales[c];
}

__device__ __forceinline__ int32_t wave_id_uniform() {
  return __builtin_amdgcn_readfirstlane((int32_t)(blockIdx.x * kGatherWaves + threadIdx.x / kWave));
}

// Dense tables, fast shapes: one wave per group of kK consecutive
// block-table entries e = kK*w + k (request e / max_blocks by the
// multiply-shift division, column e % max_blocks; entries < 2^31,
// host-checked).  The host sizes the grid from the table's entry count
// (never from a sequence length), so no wave loops.  The arguments the
// metadata addresses depend on come first, so that they are among the
// kernel arguments preloaded into SGPRs.
//
// Written as one straight pass over the group: page ids and request bounds
// as scalar loads, then every load of every run, then every store.  Loads
// past a short run's end re-read its last chunk and empty runs re-read the
// first chunk of page 0; they are not stored.  Three details of this shape
// were each measured on the 256 x 1000-token batch (interleaved runs on one
// GPU): loads issued as flat instructions (the compiler emits them for the
// selected source pointers) ran 6-8% faster than the same loads as global
// instructions; waiting for every load before the first store beat storing
// each chunk as its load returned; and the same steps spread over helper
// structures with 64-bit run arithmetic compiled to a kernel 4-8% slower.
template <int kU, int kK>
__global__ __launch_bounds__(kGatherThreads) void gather_indexer_k_fp8_direct_fast_kernel(
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ cu_seq_lens,
    int32_t max_blocks, int32_t num_reqs, uint32_t div_m, uint32_t div_shift,
    const uint8_t* __restrict__ kv_cache, uint8_t* __restrict__ k_fp8,
    uint8_t* __restrict__ k_scale, int32_t num_tokens, int32_t num_blocks, int64_t page_stride,
    int32_t block_size, int32_t head_dim) {
  const int lane = threadIdx.x & (kWave - 1);
  const FastDiv rdiv{(uint32_t)max_blocks, div_m, div_shift};
  const int32_t entries = num_reqs * max_blocks;
  const int32_t w = wave_id_uniform();
  if ((int64_t)w * kK >= entries) return;
  int32_t n2[kK], row2[kK];
  const uint8_t* src2[kK];
  const uint8_t* ssrc2[kK];
#pragma unroll
  for (int k = 0; k < kK; ++k) {
    const int64_t id = (int64_t)w * kK + k;
    const int32_t e = __builtin_amdgcn_readfirstlane(id < entries ? (int32_t)id : entries - 1);
    const int32_t r = __builtin_amdgcn_readfirstlane((int32_t)rdiv.div((uint32_t)e));
    const int32_t j = e - r * max_blocks;
    const int32_t p = block_table[e], c0 = cu_seq_lens[r], c1 = cu_seq_lens[r + 1];
    const int64_t i0 = (int64_t)j * block_size, len = (int64_t)c1 - c0;
    n2[k] = 0;
    row2[k] = 0;
    src2[k] = kv_cache;
    ssrc2[k] = kv_cache;
    if (id < entries && p >= 0 && p < num_blocks && i0 < len) {
      // tokens [i0, i0 + n) of the request, clipped to rows [0, num_tokens)
      const int64_t n = len - i0 < block_size ? len - i0 : block_size;
      const int64_t row0 = c0 + i0;
      const int64_t rb = row0 > 0 ? row0 : 0;
      const int64_t re = row0 + n < num_tokens ? row0 + n : num_tokens;
      if (rb < re) {
        const uint8_t* page_base = kv_cache + (int64_t)p * page_stride;
        n2[k] = (int32_t)(re - rb);
        row2[k] = (int32_t)rb;
        src2[k] = page_base + (rb - row0) * head_dim;
        ssrc2[k] = page_base + (int64_t)block_size * head_dim + (rb - row0) * 4;
      }
    }
  }
  u32x4 v[kK][kU];
  uint32_t sv[kK];
  const int32_t cpr = head_dim / 16;
#pragma unroll
  for (int k = 0; k < kK; ++k) {
    const int32_t chunks = n2[k] * cpr;
    const int32_t last = chunks > 0 ? chunks - 1 : 0;
    const u32x4* cs = reinterpret_cast<const u32x4*>(src2[k]);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int32_t c = u * kWave + lane;
      v[k][u] = load_stream(cs + (c < last ? c : last));
    }
    const int32_t lr = n2[k] > 0 ? n2[k] - 1 : 0;
    sv[k] = reinterpret_cast<const uint32_t*>(ssrc2[k])[lane < lr ? lane : lr];
  }
#pragma unroll
  for (int k = 0; k < kK; ++k) {
    const int32_t chunks = n2[k] * cpr;
    u32x4* cd = reinterpret_cast<u32x4*>(k_fp8 + (int64_t)row2[k] * head_dim);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int32_t c = u * kWave + lane;
      if (c < chunks) store_stream(cd + c, v[k][u]);
    }
    if (lane < n2[k]) reinterpret_cast<uint32_t*>(k_scale)[row2[k] + lane] = sv[k];
  }
}

// Dense tables, any shape: one wave per table entry, the generic copy.
__global__ __launch_bounds__(kGatherThreads) void gather_indexer_k_fp8_direct_kernel(
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ cu_seq_lens,
    int32_t max_blocks, int32_t num_reqs, uint32_t div_m, uint32_t div_shift,
    const uint8_t* __restrict__ kv_cache, uint8_t* __restrict__ k_fp8,
    uint8_t* __restrict__ k_scale, int64_t num_tokens, int64_t num_blocks, int64_t page_stride,
    int32_t block_size, int32_t head_dim) {
  const int32_t entries = num_reqs * max_blocks;
  const int32_t e = wave_id_uniform();
  if (e >= entries) return;
  const int32_t r = (int32_t)FastDiv{(uint32_t)max_blocks, div_m, div_shift}.div((uint32_t)e);
  const Run run = describe_run(kv_cache, cu_seq_lens[r], cu_seq_lens[r + 1], block_table[e],
                               e - r * max_blocks, num_tokens, num_blocks, page_stride,
                               block_size, head_dim);
  if (run.rows > 0)
    copy_run_any(run, k_fp8, reinterpret_cast<uint32_t*>(k_scale), head_dim,
                 threadIdx.x & (kWave - 1));
}

// Wide tables: runs numbered through an LDS prefix over the requests; each
// wave copies runs w, w + (waves in the grid), ...
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
  for (int64_t id = wave_id_uniform(); id < total_runs; id += stride) {
    // request r: run_start[r] <= id < run_start[r + 1]
    int32_t lo = 0, hi = num_reqs;
    while (hi - lo > 1) {
      const int32_t mid = (lo + hi) >> 1;
      if (run_start[mid] <= id) lo = mid; else hi = mid;
    }
    const int32_t r = __builtin_amdgcn_readfirstlane(lo);
    const int32_t j = __builtin_amdgcn_readfirstlane((int32_t)id - run_start[r]);
    const Run run = describe_run(kv_cache, cu_seq_lens[r], cu_seq_lens[r + 1],
                                 block_table[(int64_t)r * max_blocks + j], j, num_tokens,
                                 num_blocks, page_stride, block_size, head_dim);
    if (run.rows > 0)
      copy_run_any(run, k_fp8, reinterpret_cast<uint32_t*>(k_scale), head_dim, lane);
  }
}

// Chunks per lane per run (kU) of the fast path for this page shape, or 0
// for the generic copy: a run's code span must be a whole number of
// wave-wide 16-byte loads dividing 16, and a page at most 64 tokens.
int fast_chunks_per_lane(int32_t block_size, int32_t head_dim) {
  const int64_t chunks = (int64_t)block_size * head_dim / 16;
  if (block_size > kWave || chunks % kWave != 0) return 0;
  const int64_t u = chunks / kWave;
  return (u == 1 || u == 2 || u == 4 || u == 8 || u == 16) ? (int)u : 0;
}

template <int kU, int kK>
int launch_direct(const GatherArgs& a, hipStream_t stream) {
  // One wave per group of kK table entries (kK = 1 for the generic copy):
  // at most 2^31 / 4 workgroups.
  const int64_t groups = ((int64_t)a.num_reqs * a.max_blocks_per_req + kK - 1) / kK;
  const int64_t blocks = (groups + kGatherWaves - 1) / kGatherWaves;
  const FastDiv rdiv = FastDiv::make((uint32_t)a.max_blocks_per_req);
  if constexpr (kU == 0) {
    hipLaunchKernelGGL(gather_indexer_k_fp8_direct_kernel, dim3((unsigned)blocks),
                       dim3(kGatherThreads), 0, stream, a.block_table, a.cu_seq_lens,
                       a.max_blocks_per_req, a.num_reqs, rdiv.m, rdiv.shift, a.kv_cache, a.k_fp8,
                       a.k_scale, a.num_tokens, a.num_blocks, a.cache_block_stride, a.block_size,
                       a.head_dim);
  } else {
    // Output rows and page ids are int32 values (rows are below some
    // cu_seq_lens entry), so clamping these two sizes to 2^31 - 1 changes
    // nothing.
    const int32_t num_tokens = (int32_t)(a.num_tokens < INT32_MAX ? a.num_tokens : INT32_MAX);
    const int32_t num_blocks = (int32_t)(a.num_blocks < INT32_MAX ? a.num_blocks : INT32_MAX);
    hipLaunchKernelGGL((gather_indexer_k_fp8_direct_fast_kernel<kU, kK>), dim3((unsigned)blocks),
                       dim3(kGatherThreads), 0, stream, a.block_table, a.cu_seq_lens,
                       a.max_blocks_per_req, a.num_reqs, rdiv.m, rdiv.shift, a.kv_cache, a.k_fp8,
                       a.k_scale, num_tokens, num_blocks, a.cache_block_stride, a.block_size,
                       a.head_dim);
  }
  return (int)hipGetLastError();
}

int launch_prefix(const GatherArgs& a, hipStream_t stream) {
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

}  // namespace


int launch_gather_indexer_k_fp8(const GatherArgs& a, hipStream_t stream) {
  // Upper bound on page runs when the rows fit num_tokens: sum(len)/B + R.
  const int64_t table = (int64_t)a.num_reqs * a.max_blocks_per_req;
  const int64_t run_bound = (a.num_tokens + a.block_size - 1) / a.block_size + a.num_reqs;
  const bool direct = table <= 2 * run_bound;
  if (!direct) return launch_prefix(a, stream);
  // kK * kU = 16 chunks per lane in flight (8 runs per wave at most).
  switch (fast_chunks_per_lane(a.block_size, a.head_dim)) {
    case 1: return launch_direct<1, 8>(a, stream);
    case 2: return launch_direct<2, 8>(a, stream);
    case 4: return launch_direct<4, 4>(a, stream);
    case 8: return launch_direct<8, 2>(a, stream);
    case 16: return launch_direct<16, 1>(a, stream);
    default: return launch_direct<0, 1>(a, stream);
  }
}

}  // namespace pkv
