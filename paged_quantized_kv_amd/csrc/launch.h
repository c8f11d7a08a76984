// Internal interface between the C ABI layer (api.cpp) and the kernel
// launchers.  Launchers assume validated arguments and return 0 or the HIP
// error code of the launch.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace pkv {

// One workgroup stages cu_seq_lens and the run prefix of up to this many
// requests in LDS (4 bytes each, under 64 KiB with the static scratch);
// larger tables are launched in request chunks.
constexpr int64_t kGatherMaxReqsPerLaunch = 16000;
// Grid caps of the grid-stride kernels (the gather's prefix kernel, the
// read-backs, the NVFP4 store): larger inputs loop.
constexpr int64_t kGatherMaxBlocks = 65536;
constexpr int64_t kFp4MaxBlocks = 65536;
// The fp8 store and the dense-table gather are one-pass kernels whose grid
// follows the input, and a launch must stay below 2^32 work-items: the C ABI
// splits larger calls into launches of at most this many tokens (store) or
// block-table entries (gather), enqueued in order on the caller's stream.
// Tokens and requests are independent, so the split changes no result.
constexpr int64_t kStoreFp8MaxTokensPerLaunch = int64_t{1} << 22;
constexpr int64_t kGatherMaxEntriesPerLaunch = int64_t{1} << 22;

struct GatherArgs {
  const uint8_t* kv_cache;
  uint8_t* k_fp8;
  uint8_t* k_scale;
  const int32_t* block_table;
  const int32_t* cu_seq_lens;
  int32_t num_reqs;
  int32_t max_blocks_per_req;
  int64_t num_tokens;
  int64_t num_blocks;
  int64_t cache_block_stride;
  int32_t block_size;
  int32_t head_dim;
};

struct StoreFp8Args {
  const uint16_t* k;
  int64_t k_row_stride;
  int32_t k_dtype;  // PKV_DTYPE_BF16 / PKV_DTYPE_F16
  const int64_t* slot_mapping;
  int64_t num_tokens;
  uint8_t* kv_cache;
  int64_t num_blocks;
  int64_t cache_block_stride;
  int32_t block_size;
  int32_t log2_block_size;  // -1 when block_size is not a power of two
  int32_t head_dim;
};

struct StoreFp4Args {
  const uint16_t* key;
  int64_t key_row_stride;
  const uint16_t* value;
  int64_t value_row_stride;
  int32_t src_dtype;  // PKV_DTYPE_BF16 / PKV_DTYPE_F16
  uint8_t* key_cache;
  uint8_t* value_cache;
  const int64_t* slot_mapping;
  int64_t num_tokens;
  int32_t num_heads;
  int32_t head_size;
  int32_t block_size;
  int32_t log2_block_size;
  int64_t num_blocks;
  int64_t page_stride;
  int32_t layout;
  const float* k_scale;
  const float* v_scale;
};

struct GatherDequantArgs {
  const uint8_t* kv_cache;
  uint16_t* out;
  int64_t out_row_stride;
  int32_t out_dtype;  // PKV_DTYPE_BF16 / PKV_DTYPE_F16
  const int32_t* block_table;
  const int32_t* cu_seq_lens;
  int32_t num_reqs;
  int32_t max_blocks_per_req;
  int64_t num_tokens;
  int64_t num_blocks;
  int64_t cache_block_stride;
  int32_t block_size;
  int32_t head_dim;
};

struct GatherFp4DequantArgs {
  const uint8_t* key_cache;
  const uint8_t* value_cache;
  uint16_t* key_out;
  int64_t key_row_stride;
  uint16_t* value_out;
  int64_t value_row_stride;
  int32_t out_dtype;
  const int32_t* block_table;
  const int32_t* cu_seq_lens;
  int32_t num_reqs;
  int32_t max_blocks_per_req;
  int64_t num_tokens;
  int32_t num_heads;
  int32_t head_size;
  int32_t block_size;
  int64_t num_blocks;
  int64_t page_stride;
  int32_t layout;
  const float* k_scale;
  const float* v_scale;
};

struct MqaLogitsArgs {
  const uint8_t* q;
  int64_t q_token_stride;  // bytes
  const uint8_t* k;
  const float* k_scale;
  const float* weights;
  const int32_t* ks;
  const int32_t* ke;
  float* logits;
  int64_t row_stride;  // elements
  int64_t row_cols;
  int32_t num_q;
  int32_t num_heads;
  int64_t num_k;
};

struct PagedAttentionArgs {
  uint16_t* out;
  float* exp_sums;
  float* max_logits;
  float* tmp_out;
  const uint16_t* query;
  const uint8_t* key_cache;
  const uint8_t* value_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int32_t num_seqs;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t max_blocks_per_seq;
  int32_t max_context_len;
  int64_t num_blocks;
  float scale;
  float k_scale;
  float v_scale;
  int32_t partition_size;
};

int launch_gather_indexer_k_fp8(const GatherArgs& a, hipStream_t stream);
int launch_fp8_mqa_logits(const MqaLogitsArgs& a, hipStream_t stream);
int launch_gather_indexer_k_dequant(const GatherDequantArgs& a, hipStream_t stream);
int launch_gather_kv_fp4_dequant(const GatherFp4DequantArgs& a, hipStream_t stream);
int launch_paged_attention_decode(const PagedAttentionArgs& a, hipStream_t stream);
// Device address of the current GPU's attention scratch array (0 or a HIP error).
int attention_scratch(void** ptr);
// Units of the decode attention's balanced split for these sizes (0: fixed split).
int64_t attention_balanced_units(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t max_context_len, int32_t partition_size,
                                 int32_t wave_slots);
int launch_store_indexer_k_fp8(const StoreFp8Args& a, hipStream_t stream);
int launch_store_kv_fp4(const StoreFp4Args& a, hipStream_t stream);
int launch_diag_e4m3(const float* y, uint8_t* out, int64_t n, hipStream_t stream);
int launch_diag_e2m1(const float* y, uint8_t* out, int64_t n, hipStream_t stream);
int launch_diag_narrow(const float* x, uint16_t* out, int64_t n, int32_t out_dtype,
                       hipStream_t stream);

}  // namespace pkv
