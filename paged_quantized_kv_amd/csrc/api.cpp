// C ABI of libpkv (include/pkv.h): argument validation on the host, then the
// kernel launchers.  Every check returns before any HIP call, so a rejected
// call enqueues nothing.  No C++ exception crosses the ABI.
#include "pkv.h"

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "launch.h"

namespace {

thread_local char g_error[512] = "";

// The indexer-logits kernel stays off until the cause of an unfinished GPU
// run is found (see pkv_fp8_mqa_logits).
constexpr bool kMqaLogitsEnabled = false;

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_error, sizeof g_error, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_error[0] = '\0';
  return PKV_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int32_t log2_or_neg(int64_t v) {
  if (v <= 0 || (v & (v - 1))) return -1;
  int32_t l = 0;
  while ((int64_t{1} << l) < v) ++l;
  return l;
}

int launched(int hip_status, const char* op) {
  if (hip_status != 0)
    return fail(PKV_ELAUNCH, "%s: kernel launch failed: %s", op,
                hipGetErrorString(static_cast<hipError_t>(hip_status)));
  return ok();
}

// Shared checks of the indexer page geometry.
int check_indexer_geometry(const char* op, int64_t num_blocks, int64_t stride,
                           int32_t block_size, int32_t head_dim) {
  if (num_blocks <= 0) return fail(PKV_EINVAL, "%s: num_blocks must be > 0, got %lld", op, (long long)num_blocks);
  if (block_size <= 0) return fail(PKV_EINVAL, "%s: block_size must be > 0, got %d", op, block_size);
  if (head_dim <= 0) return fail(PKV_EINVAL, "%s: head_dim must be > 0, got %d", op, head_dim);
  if (head_dim % 16 != 0)
    return fail(PKV_EUNSUPPORTED, "%s: head_dim must be a multiple of 16, got %d", op, head_dim);
  const int64_t page = (int64_t)block_size * (head_dim + 4);
  if (stride < page)
    return fail(PKV_EUNSUPPORTED,
                "%s: cache_block_stride %lld is smaller than the page, block_size*(head_dim+4) = %lld",
                op, (long long)stride, (long long)page);
  if (stride % 16 != 0)
    return fail(PKV_EALIGN, "%s: cache_block_stride must be a multiple of 16, got %lld", op, (long long)stride);
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_abi_version(void) { return PKV_ABI_VERSION; }

const char* pkv_last_error(void) { return g_error; }

int pkv_gather_indexer_k_fp8(const void* kv_cache, void* k_fp8, void* k_scale,
                             const int32_t* block_table, const int32_t* cu_seq_lens,
                             int32_t num_reqs, int32_t max_blocks_per_req, int64_t num_tokens,
                             int64_t num_blocks, int64_t cache_block_stride, int32_t block_size,
                             int32_t head_dim, void* stream) {
  static const char* op = "pkv_gather_indexer_k_fp8";
  if (num_reqs < 0) return fail(PKV_EINVAL, "%s: num_reqs must be >= 0, got %d", op, num_reqs);
  if (num_tokens < 0) return fail(PKV_EINVAL, "%s: num_tokens must be >= 0, got %lld", op, (long long)num_tokens);
  if (int rc = check_indexer_geometry(op, num_blocks, cache_block_stride, block_size, head_dim)) return rc;
  if (max_blocks_per_req < 0)
    return fail(PKV_EINVAL, "%s: max_blocks_per_req must be >= 0, got %d", op, max_blocks_per_req);
  // no requests, no output rows or no page columns: nothing can be written
  if (num_reqs == 0 || num_tokens == 0 || max_blocks_per_req == 0) return ok();
  if ((int64_t)num_reqs * max_blocks_per_req > INT32_MAX)
    return fail(PKV_EUNSUPPORTED, "%s: num_reqs * max_blocks_per_req exceeds 2^31-1", op);
  if (max_blocks_per_req > pkv::kGatherMaxEntriesPerLaunch)
    return fail(PKV_EUNSUPPORTED, "%s: max_blocks_per_req must be <= %lld, got %d", op,
                (long long)pkv::kGatherMaxEntriesPerLaunch, max_blocks_per_req);
  if (!kv_cache || !k_fp8 || !k_scale || !block_table || !cu_seq_lens)
    return fail(PKV_EINVAL, "%s: null buffer pointer", op);
  if (!aligned(kv_cache, 16) || !aligned(k_fp8, 16))
    return fail(PKV_EALIGN, "%s: kv_cache and k_fp8 must be 16-byte aligned", op);
  if (!aligned(k_scale, 4) || !aligned(block_table, 4) || !aligned(cu_seq_lens, 4))
    return fail(PKV_EALIGN, "%s: k_scale, block_table and cu_seq_lens must be 4-byte aligned", op);
  // request chunks of at most kGatherMaxEntriesPerLaunch table entries; the
  // rows a chunk writes come from its own cu_seq_lens entries
  const int64_t per_launch = pkv::kGatherMaxEntriesPerLaunch / max_blocks_per_req;
  for (int64_t r0 = 0; r0 < num_reqs; r0 += per_launch) {
    const int64_t left = num_reqs - r0;
    pkv::GatherArgs a{static_cast<const uint8_t*>(kv_cache), static_cast<uint8_t*>(k_fp8),
                      static_cast<uint8_t*>(k_scale), block_table + r0 * max_blocks_per_req,
                      cu_seq_lens + r0, (int32_t)(left < per_launch ? left : per_launch),
                      max_blocks_per_req, num_tokens, num_blocks, cache_block_stride,
                      block_size, head_dim};
    if (int e = pkv::launch_gather_indexer_k_fp8(a, static_cast<hipStream_t>(stream)))
      return launched(e, op);
  }
  return ok();
}

int pkv_store_indexer_k_fp8(const void* k, int64_t k_row_stride, int32_t k_dtype,
                            const int64_t* slot_mapping, int64_t num_tokens, void* kv_cache,
                            int64_t num_blocks,
                            int64_t cache_block_stride, int32_t block_size, int32_t head_dim,
                            void* stream) {
  static const char* op = "pkv_store_indexer_k_fp8";
  if (num_tokens < 0) return fail(PKV_EINVAL, "%s: num_tokens must be >= 0, got %lld", op, (long long)num_tokens);
  if (int rc = check_indexer_geometry(op, num_blocks, cache_block_stride, block_size, head_dim)) return rc;
  if (head_dim > 1024) return fail(PKV_EUNSUPPORTED, "%s: head_dim must be <= 1024, got %d", op, head_dim);
  if (k_dtype != PKV_DTYPE_BF16 && k_dtype != PKV_DTYPE_F16)
    return fail(PKV_EINVAL, "%s: k_dtype must be PKV_DTYPE_BF16 or PKV_DTYPE_F16, got %d", op, k_dtype);
  if (k_row_stride < head_dim)
    return fail(PKV_EINVAL, "%s: k_row_stride %lld < head_dim %d", op, (long long)k_row_stride, head_dim);
  if (k_row_stride % 8 != 0)
    return fail(PKV_EALIGN, "%s: k_row_stride must be a multiple of 8 elements, got %lld", op, (long long)k_row_stride);
  if (num_tokens == 0) return ok();
  if (!k || !slot_mapping || !kv_cache) return fail(PKV_EINVAL, "%s: null buffer pointer", op);
  if (!aligned(k, 16) || !aligned(kv_cache, 16))
    return fail(PKV_EALIGN, "%s: k and kv_cache must be 16-byte aligned", op);
  if (!aligned(slot_mapping, 8)) return fail(PKV_EALIGN, "%s: slot_mapping must be 8-byte aligned", op);
  if (num_tokens > ((int64_t)1 << 40)) return fail(PKV_EUNSUPPORTED, "%s: num_tokens too large", op);
  // token chunks of at most kStoreFp8MaxTokensPerLaunch
  const uint16_t* k16 = static_cast<const uint16_t*>(k);
  for (int64_t t0 = 0; t0 < num_tokens; t0 += pkv::kStoreFp8MaxTokensPerLaunch) {
    const int64_t left = num_tokens - t0;
    pkv::StoreFp8Args a{k16 + t0 * k_row_stride, k_row_stride, k_dtype, slot_mapping + t0,
                        left < pkv::kStoreFp8MaxTokensPerLaunch ? left
                                                                : pkv::kStoreFp8MaxTokensPerLaunch,
                        static_cast<uint8_t*>(kv_cache), num_blocks, cache_block_stride,
                        block_size, log2_or_neg(block_size), head_dim};
    if (int e = pkv::launch_store_indexer_k_fp8(a, static_cast<hipStream_t>(stream)))
      return launched(e, op);
  }
  return ok();
}

int pkv_store_kv_fp4(const void* key, int64_t key_row_stride, const void* value,
                     int64_t value_row_stride, int32_t src_dtype, void* key_cache,
                     void* value_cache,
                     const int64_t* slot_mapping, int64_t num_tokens, int32_t num_heads,
                     int32_t head_size, int32_t block_size, int64_t num_blocks, int64_t page_stride,
                     int32_t layout, const float* k_scale, const float* v_scale, void* stream) {
  static const char* op = "pkv_store_kv_fp4";
  if (num_tokens < 0) return fail(PKV_EINVAL, "%s: num_tokens must be >= 0, got %lld", op, (long long)num_tokens);
  if (num_heads <= 0) return fail(PKV_EINVAL, "%s: num_heads must be > 0, got %d", op, num_heads);
  if (head_size <= 0) return fail(PKV_EINVAL, "%s: head_size must be > 0, got %d", op, head_size);
  if (block_size <= 0) return fail(PKV_EINVAL, "%s: block_size must be > 0, got %d", op, block_size);
  if (num_blocks <= 0) return fail(PKV_EINVAL, "%s: num_blocks must be > 0, got %lld", op, (long long)num_blocks);
  // The page's own checks (head_size % 16, block_size % 4), plus head_size %
  // 64 so that every 4x4 swizzle tile of the V scales is complete.
  if (head_size % 16 != 0)
    return fail(PKV_EUNSUPPORTED, "%s: head_size %d is not a multiple of 16 (16-element scale blocks)", op, head_size);
  if (head_size % 64 != 0)
    return fail(PKV_EUNSUPPORTED, "%s: head_size %d is not a multiple of 64 (complete 4x4 V-scale swizzle tiles)", op, head_size);
  if (block_size % 4 != 0)
    return fail(PKV_EUNSUPPORTED, "%s: block_size %d is not a multiple of 4 (4-token swizzle tiles)", op, block_size);
  if (src_dtype != PKV_DTYPE_BF16 && src_dtype != PKV_DTYPE_F16)
    return fail(PKV_EINVAL, "%s: src_dtype must be PKV_DTYPE_BF16 or PKV_DTYPE_F16, got %d", op, src_dtype);
  if (layout != PKV_LAYOUT_HND && layout != PKV_LAYOUT_NHD)
    return fail(PKV_EINVAL, "%s: layout must be PKV_LAYOUT_HND or PKV_LAYOUT_NHD, got %d", op, layout);
  const int64_t hd = (int64_t)num_heads * head_size;
  if (hd > ((int64_t)1 << 24)) return fail(PKV_EUNSUPPORTED, "%s: num_heads*head_size too large", op);
  if (key_row_stride < hd || value_row_stride < hd)
    return fail(PKV_EINVAL, "%s: row strides must be >= num_heads*head_size = %lld", op, (long long)hd);
  if (key_row_stride % 8 != 0 || value_row_stride % 8 != 0)
    return fail(PKV_EALIGN, "%s: row strides must be multiples of 8 elements", op);
  const int64_t side = (int64_t)num_heads * block_size * (head_size / 2 + head_size / 16);
  if (page_stride < side)
    return fail(PKV_EUNSUPPORTED, "%s: page_stride %lld is smaller than one side, %lld bytes", op,
                (long long)page_stride, (long long)side);
  if (page_stride % 8 != 0) return fail(PKV_EALIGN, "%s: page_stride must be a multiple of 8", op);
  if (num_tokens == 0) return ok();
  if (!key || !value || !key_cache || !value_cache || !slot_mapping || !k_scale || !v_scale)
    return fail(PKV_EINVAL, "%s: null buffer pointer", op);
  if (!aligned(key, 16) || !aligned(value, 16))
    return fail(PKV_EALIGN, "%s: key and value must be 16-byte aligned", op);
  if (!aligned(key_cache, 8) || !aligned(value_cache, 8) || !aligned(slot_mapping, 8))
    return fail(PKV_EALIGN, "%s: caches and slot_mapping must be 8-byte aligned", op);
  if (!aligned(k_scale, 4) || !aligned(v_scale, 4))
    return fail(PKV_EALIGN, "%s: k_scale and v_scale must be 4-byte aligned", op);
  pkv::StoreFp4Args a{static_cast<const uint16_t*>(key), key_row_stride,
                      static_cast<const uint16_t*>(value), value_row_stride, src_dtype,
                      static_cast<uint8_t*>(key_cache), static_cast<uint8_t*>(value_cache),
                      slot_mapping, num_tokens, num_heads, head_size, block_size,
                      log2_or_neg(block_size), num_blocks, page_stride, layout, k_scale, v_scale};
  return launched(pkv::launch_store_kv_fp4(a, static_cast<hipStream_t>(stream)), op);
}

int pkv_gather_indexer_k_dequant(const void* kv_cache, void* out, int64_t out_row_stride,
                                 int32_t out_dtype, const int32_t* block_table,
                                 const int32_t* cu_seq_lens, int32_t num_reqs,
                                 int32_t max_blocks_per_req, int64_t num_tokens,
                                 int64_t num_blocks, int64_t cache_block_stride,
                                 int32_t block_size, int32_t head_dim, void* stream) {
  static const char* op = "pkv_gather_indexer_k_dequant";
  if (num_reqs < 0) return fail(PKV_EINVAL, "%s: num_reqs must be >= 0, got %d", op, num_reqs);
  if (num_tokens < 0) return fail(PKV_EINVAL, "%s: num_tokens must be >= 0, got %lld", op, (long long)num_tokens);
  if (int rc = check_indexer_geometry(op, num_blocks, cache_block_stride, block_size, head_dim)) return rc;
  if (max_blocks_per_req < 0)
    return fail(PKV_EINVAL, "%s: max_blocks_per_req must be >= 0, got %d", op, max_blocks_per_req);
  if (out_dtype != PKV_DTYPE_BF16 && out_dtype != PKV_DTYPE_F16)
    return fail(PKV_EINVAL, "%s: out_dtype must be PKV_DTYPE_BF16 or PKV_DTYPE_F16, got %d", op, out_dtype);
  if (out_row_stride < head_dim)
    return fail(PKV_EINVAL, "%s: out_row_stride %lld is smaller than head_dim %d", op, (long long)out_row_stride, head_dim);
  if (out_row_stride % 8 != 0)
    return fail(PKV_EALIGN, "%s: out_row_stride must be a multiple of 8 elements", op);
  if ((int64_t)block_size * head_dim / 8 > INT32_MAX)
    return fail(PKV_EUNSUPPORTED, "%s: block_size * head_dim / 8 exceeds 2^31-1", op);
  if (num_reqs == 0 || num_tokens == 0 || max_blocks_per_req == 0) return ok();
  if ((int64_t)num_reqs * max_blocks_per_req > INT32_MAX)
    return fail(PKV_EUNSUPPORTED, "%s: num_reqs * max_blocks_per_req exceeds 2^31-1", op);
  if (!kv_cache || !out || !block_table || !cu_seq_lens)
    return fail(PKV_EINVAL, "%s: null buffer pointer", op);
  if (!aligned(kv_cache, 16) || !aligned(out, 16))
    return fail(PKV_EALIGN, "%s: kv_cache and out must be 16-byte aligned", op);
  if (!aligned(block_table, 4) || !aligned(cu_seq_lens, 4))
    return fail(PKV_EALIGN, "%s: block_table and cu_seq_lens must be 4-byte aligned", op);
  pkv::GatherDequantArgs a{static_cast<const uint8_t*>(kv_cache), static_cast<uint16_t*>(out),
                           out_row_stride, out_dtype, block_table, cu_seq_lens, num_reqs,
                           max_blocks_per_req, num_tokens, num_blocks, cache_block_stride,
                           block_size, head_dim};
  return launched(pkv::launch_gather_indexer_k_dequant(a, static_cast<hipStream_t>(stream)), op);
}

int pkv_gather_kv_fp4_dequant(const void* key_cache, const void* value_cache, void* key_out,
                              int64_t key_row_stride, void* value_out, int64_t value_row_stride,
                              int32_t out_dtype, const int32_t* block_table,
                              const int32_t* cu_seq_lens, int32_t num_reqs,
                              int32_t max_blocks_per_req, int64_t num_tokens, int32_t num_heads,
                              int32_t head_size, int32_t block_size, int64_t num_blocks,
                              int64_t page_stride, int32_t layout, const float* k_scale,
                              const float* v_scale, void* stream) {
  static const char* op = "pkv_gather_kv_fp4_dequant";
  if (num_reqs < 0) return fail(PKV_EINVAL, "%s: num_reqs must be >= 0, got %d", op, num_reqs);
  if (num_tokens < 0) return fail(PKV_EINVAL, "%s: num_tokens must be >= 0, got %lld", op, (long long)num_tokens);
  if (max_blocks_per_req < 0)
    return fail(PKV_EINVAL, "%s: max_blocks_per_req must be >= 0, got %d", op, max_blocks_per_req);
  if (num_heads <= 0) return fail(PKV_EINVAL, "%s: num_heads must be > 0, got %d", op, num_heads);
  if (head_size <= 0) return fail(PKV_EINVAL, "%s: head_size must be > 0, got %d", op, head_size);
  if (block_size <= 0) return fail(PKV_EINVAL, "%s: block_size must be > 0, got %d", op, block_size);
  if (num_blocks <= 0) return fail(PKV_EINVAL, "%s: num_blocks must be > 0, got %lld", op, (long long)num_blocks);
  if (head_size % 64 != 0)
    return fail(PKV_EUNSUPPORTED, "%s: head_size must be a multiple of 64, got %d", op, head_size);
  if (block_size % 4 != 0)
    return fail(PKV_EUNSUPPORTED, "%s: block_size %d is not a multiple of 4 (4-token swizzle tiles)", op, block_size);
  if (out_dtype != PKV_DTYPE_BF16 && out_dtype != PKV_DTYPE_F16)
    return fail(PKV_EINVAL, "%s: out_dtype must be PKV_DTYPE_BF16 or PKV_DTYPE_F16, got %d", op, out_dtype);
  if (layout != PKV_LAYOUT_HND && layout != PKV_LAYOUT_NHD)
    return fail(PKV_EINVAL, "%s: layout must be PKV_LAYOUT_HND or PKV_LAYOUT_NHD, got %d", op, layout);
  const int64_t hd = (int64_t)num_heads * head_size;
  if (hd > ((int64_t)1 << 24)) return fail(PKV_EUNSUPPORTED, "%s: num_heads*head_size too large", op);
  if (key_row_stride < hd || value_row_stride < hd)
    return fail(PKV_EINVAL, "%s: row strides must be >= num_heads*head_size = %lld", op, (long long)hd);
  if (key_row_stride % 8 != 0 || value_row_stride % 8 != 0)
    return fail(PKV_EALIGN, "%s: row strides must be multiples of 8 elements", op);
  const int64_t side = (int64_t)num_heads * block_size * (head_size / 2 + head_size / 16);
  if (page_stride < side)
    return fail(PKV_EUNSUPPORTED, "%s: page_stride %lld is smaller than one side, %lld bytes", op,
                (long long)page_stride, (long long)side);
  if (page_stride % 16 != 0) return fail(PKV_EALIGN, "%s: page_stride must be a multiple of 16", op);
  if ((int64_t)block_size * hd / 8 > INT32_MAX)
    return fail(PKV_EUNSUPPORTED, "%s: block_size * num_heads * head_size / 8 exceeds 2^31-1", op);
  if (num_reqs == 0 || num_tokens == 0 || max_blocks_per_req == 0) return ok();
  if ((int64_t)num_reqs * max_blocks_per_req * 2 > INT32_MAX)
    return fail(PKV_EUNSUPPORTED, "%s: num_reqs * max_blocks_per_req * 2 exceeds 2^31-1", op);
  if (!key_cache || !value_cache || !key_out || !value_out || !block_table || !cu_seq_lens ||
      !k_scale || !v_scale)
    return fail(PKV_EINVAL, "%s: null buffer pointer", op);
  if (!aligned(key_cache, 16) || !aligned(value_cache, 16) || !aligned(key_out, 16) ||
      !aligned(value_out, 16))
    return fail(PKV_EALIGN, "%s: caches and outputs must be 16-byte aligned", op);
  if (!aligned(block_table, 4) || !aligned(cu_seq_lens, 4) || !aligned(k_scale, 4) ||
      !aligned(v_scale, 4))
    return fail(PKV_EALIGN, "%s: block_table, cu_seq_lens and the scales must be 4-byte aligned", op);
  pkv::GatherFp4DequantArgs a{static_cast<const uint8_t*>(key_cache),
                              static_cast<const uint8_t*>(value_cache),
                              static_cast<uint16_t*>(key_out), key_row_stride,
                              static_cast<uint16_t*>(value_out), value_row_stride, out_dtype,
                              block_table, cu_seq_lens, num_reqs, max_blocks_per_req, num_tokens,
                              num_heads, head_size, block_size, num_blocks, page_stride, layout,
                              k_scale, v_scale};
  return launched(pkv::launch_gather_kv_fp4_dequant(a, static_cast<hipStream_t>(stream)), op);
}

int pkv_fp8_mqa_logits(const void* q, int64_t q_token_stride, const void* k, const float* k_scale,
                       const float* weights, const int32_t* ks, const int32_t* ke, float* logits,
                       int64_t row_stride, int64_t row_cols, int32_t num_q, int32_t num_heads,
                       int64_t num_k, int32_t head_dim, void* stream) {
  static const char* op = "pkv_fp8_mqa_logits";
  if (num_q < 0) return fail(PKV_EINVAL, "%s: num_q must be >= 0, got %d", op, num_q);
  if (num_k < 0) return fail(PKV_EINVAL, "%s: num_k must be >= 0, got %lld", op, (long long)num_k);
  if (row_cols < 0) return fail(PKV_EINVAL, "%s: row_cols must be >= 0, got %lld", op, (long long)row_cols);
  if (row_stride < row_cols)
    return fail(PKV_EINVAL, "%s: row_stride %lld is smaller than row_cols %lld", op,
                (long long)row_stride, (long long)row_cols);
  if (head_dim != 128)
    return fail(PKV_EUNSUPPORTED, "%s: head_dim must be 128 (one MFMA K), got %d", op, head_dim);
  if (num_heads <= 0 || num_heads % 16 != 0 || num_heads > 64)
    return fail(PKV_EUNSUPPORTED, "%s: num_heads must be 16, 32, 48 or 64, got %d", op, num_heads);
  if (q_token_stride < (int64_t)num_heads * head_dim)
    return fail(PKV_EINVAL, "%s: q_token_stride must be >= num_heads*head_dim", op);
  if (q_token_stride % 16 != 0) return fail(PKV_EALIGN, "%s: q_token_stride must be a multiple of 16", op);
  if (num_q == 0 || num_k == 0 || row_cols == 0) return ok();
  if (!q || !k || !k_scale || !weights || !ks || !ke || !logits)
    return fail(PKV_EINVAL, "%s: null buffer pointer", op);
  if (!aligned(q, 16) || !aligned(k, 16)) return fail(PKV_EALIGN, "%s: q and k must be 16-byte aligned", op);
  if (!aligned(k_scale, 4) || !aligned(weights, 4) || !aligned(ks, 4) || !aligned(ke, 4) ||
      !aligned(logits, 4))
    return fail(PKV_EALIGN, "%s: k_scale, weights, ks, ke and logits must be 4-byte aligned", op);
  // Switched off: a GPU run on causal per-request ranges did not finish, and
  // no cause has been found in the kernel yet; nothing is launched.
  if (!kMqaLogitsEnabled)
    return fail(PKV_EUNSUPPORTED, "%s: not enabled (a causal-range run of its "
                "kernel did not finish; the cause is not found yet)", op);
  pkv::MqaLogitsArgs a{static_cast<const uint8_t*>(q), q_token_stride,
                       static_cast<const uint8_t*>(k), k_scale, weights, ks, ke, logits,
                       row_stride, row_cols, num_q, num_heads, num_k};
  return launched(pkv::launch_fp8_mqa_logits(a, static_cast<hipStream_t>(stream)), op);
}

}  // extern "C"

namespace {

// Checks shared by both decode-attention entry points (everything but the
// workspace buffers).
int check_attention(const char* op, const void* out, const void* query, const void* key_cache,
                    const void* value_cache, const int32_t* block_tables,
                    const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                    int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                    int32_t max_blocks_per_seq, int32_t max_context_len, int64_t num_blocks,
                    float scale, float k_scale, float v_scale, int32_t partition_size) {
  if (num_seqs < 0) return fail(PKV_EINVAL, "%s: num_seqs must be >= 0, got %d", op, num_seqs);
  if (num_heads <= 0 || num_kv_heads <= 0)
    return fail(PKV_EINVAL, "%s: num_heads and num_kv_heads must be > 0, got %d and %d", op,
                num_heads, num_kv_heads);
  if (num_heads % num_kv_heads != 0)
    return fail(PKV_EINVAL, "%s: num_heads %d is not a multiple of num_kv_heads %d", op,
                num_heads, num_kv_heads);
  if (num_heads / num_kv_heads > 16)
    return fail(PKV_EUNSUPPORTED, "%s: at most 16 query heads per KV head, got %d", op,
                num_heads / num_kv_heads);
  if (head_size != 128) return fail(PKV_EUNSUPPORTED, "%s: head_size must be 128, got %d", op, head_size);
  if (block_size <= 0 || block_size % 16 != 0)
    return fail(PKV_EUNSUPPORTED, "%s: block_size must be a positive multiple of 16, got %d", op,
                block_size);
  if (partition_size < 64 || partition_size > 2048 || (partition_size & (partition_size - 1)) != 0)
    return fail(PKV_EUNSUPPORTED, "%s: partition_size must be a power of two in [64, 2048], got %d",
                op, partition_size);
  if (max_blocks_per_seq < 0)
    return fail(PKV_EINVAL, "%s: max_blocks_per_seq must be >= 0, got %d", op, max_blocks_per_seq);
  if (max_context_len < 0)
    return fail(PKV_EINVAL, "%s: max_context_len must be >= 0, got %d", op, max_context_len);
  if (num_blocks <= 0) return fail(PKV_EINVAL, "%s: num_blocks must be > 0, got %lld", op, (long long)num_blocks);
  if (!std::isfinite(scale) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return fail(PKV_EINVAL, "%s: scale, k_scale and v_scale must be finite", op);
  if (max_context_len > (1 << 30))
    return fail(PKV_EUNSUPPORTED, "%s: max_context_len must be <= 2^30, got %d", op, max_context_len);
  const int64_t parts = ((int64_t)max_context_len + partition_size - 1) / partition_size;
  if ((int64_t)num_seqs * num_heads >= INT32_MAX || (int64_t)num_seqs * num_kv_heads * parts >= INT32_MAX)
    return fail(PKV_EUNSUPPORTED, "%s: num_seqs * num_heads and the partition count must stay below 2^31", op);
  if ((int64_t)num_seqs * max_blocks_per_seq > INT32_MAX)
    return fail(PKV_EUNSUPPORTED, "%s: num_seqs * max_blocks_per_seq exceeds 2^31-1", op);
  if (num_seqs == 0) return PKV_OK;
  if (!out || !query || !context_lens ||
      (max_context_len > 0 && (!key_cache || !value_cache || !block_tables)))
    return fail(PKV_EINVAL, "%s: null buffer pointer", op);
  if (!aligned(out, 16) || !aligned(query, 16) || !aligned(key_cache, 16) || !aligned(value_cache, 16))
    return fail(PKV_EALIGN, "%s: out, query, key_cache and value_cache must be 16-byte aligned", op);
  if (!aligned(block_tables, 4) || !aligned(context_lens, 4))
    return fail(PKV_EALIGN, "%s: block_tables and context_lens must be 4-byte aligned", op);
  return PKV_OK;
}

int64_t align256(int64_t n) { return (n + 255) / 256 * 256; }

}  // namespace

extern "C" {

int pkv_paged_attention_decode(void* out, float* exp_sums, float* max_logits, float* tmp_out,
                               const void* query, const void* key_cache, const void* value_cache,
                               const int32_t* block_tables, const int32_t* context_lens,
                               int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                               int32_t head_size, int32_t block_size, int32_t max_blocks_per_seq,
                               int32_t max_context_len, int64_t num_blocks, float scale,
                               float k_scale, float v_scale, int32_t partition_size,
                               void* stream) {
  static const char* op = "pkv_paged_attention_decode";
  if (int rc = check_attention(op, out, query, key_cache, value_cache, block_tables, context_lens,
                               num_seqs, num_heads, num_kv_heads, head_size, block_size,
                               max_blocks_per_seq, max_context_len, num_blocks, scale, k_scale,
                               v_scale, partition_size))
    return rc;
  if (num_seqs == 0) return ok();
  if (max_context_len > 0 && (!exp_sums || !max_logits || !tmp_out))
    return fail(PKV_EINVAL, "%s: null buffer pointer", op);
  if (!aligned(tmp_out, 16))
    return fail(PKV_EALIGN, "%s: tmp_out must be 16-byte aligned", op);
  if (!aligned(exp_sums, 4) || !aligned(max_logits, 4))
    return fail(PKV_EALIGN, "%s: exp_sums and max_logits must be 4-byte aligned", op);
  pkv::PagedAttentionArgs a{static_cast<uint16_t*>(out), exp_sums, max_logits, tmp_out,
                            static_cast<const uint16_t*>(query),
                            static_cast<const uint8_t*>(key_cache),
                            static_cast<const uint8_t*>(value_cache), block_tables, context_lens,
                            num_seqs, num_heads, num_kv_heads, block_size, max_blocks_per_seq,
                            max_context_len, num_blocks, scale, k_scale, v_scale, partition_size};
  return launched(pkv::launch_paged_attention_decode(a, static_cast<hipStream_t>(stream)), op);
}

int pkv_paged_attention_decode_noalloc(void* out, const void* query, const void* key_cache,
                                       const void* value_cache, const int32_t* block_tables,
                                       const int32_t* context_lens, int32_t num_seqs,
                                       int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                                       int32_t block_size, int32_t max_blocks_per_seq,
                                       int32_t max_context_len, int64_t num_blocks, float scale,
                                       float k_scale, float v_scale, int32_t partition_size,
                                       void* stream) {
  static const char* op = "pkv_paged_attention_decode_noalloc";
  if (int rc = check_attention(op, out, query, key_cache, value_cache, block_tables, context_lens,
                               num_seqs, num_heads, num_kv_heads, head_size, block_size,
                               max_blocks_per_seq, max_context_len, num_blocks, scale, k_scale,
                               v_scale, partition_size))
    return rc;
  if (num_seqs == 0) return ok();
  // workspace [exp_sums | max_logits | tmp_out] as pkv_paged_attention_decode's,
  // each region 256-byte aligned
  const int64_t parts = ((int64_t)max_context_len + partition_size - 1) / partition_size;
  const int64_t n = (int64_t)num_seqs * num_heads * (parts > 0 ? parts : 1);
  const int64_t sums = align256(4 * n);
  const int64_t need = 2 * sums + 4 * n * head_size;
  if (need > (int64_t)PKV_ATTENTION_SCRATCH_BYTES)
    return fail(PKV_EUNSUPPORTED,
                "%s: the call needs %lld bytes of workspace, more than the %lld-byte built-in "
                "scratch (use pkv_paged_attention_decode with a caller workspace)",
                op, (long long)need, (long long)PKV_ATTENTION_SCRATCH_BYTES);
  // the scratch address is looked up for the current device, so the stream
  // must belong to that device (host queries only: nothing is enqueued)
  int cur = -1, sdev = -1;
  if (hipGetDevice(&cur) != hipSuccess ||
      hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess)
    return fail(PKV_ELAUNCH, "%s: querying the current device or the stream's device failed", op);
  if (sdev != cur)
    return fail(PKV_EINVAL, "%s: the stream belongs to device %d but device %d is current", op,
                sdev, cur);
  void* base = nullptr;
  if (int e = pkv::attention_scratch(&base))
    return fail(PKV_ELAUNCH, "%s: looking up the scratch array failed: %s", op,
                hipGetErrorString(static_cast<hipError_t>(e)));
  uint8_t* b = static_cast<uint8_t*>(base);
  pkv::PagedAttentionArgs a{static_cast<uint16_t*>(out), reinterpret_cast<float*>(b),
                            reinterpret_cast<float*>(b + sums), reinterpret_cast<float*>(b + 2 * sums),
                            static_cast<const uint16_t*>(query),
                            static_cast<const uint8_t*>(key_cache),
                            static_cast<const uint8_t*>(value_cache), block_tables, context_lens,
                            num_seqs, num_heads, num_kv_heads, block_size, max_blocks_per_seq,
                            max_context_len, num_blocks, scale, k_scale, v_scale, partition_size};
  return launched(pkv::launch_paged_attention_decode(a, static_cast<hipStream_t>(stream)), op);
}

static int check_diag(const char* op, const float* y, const uint8_t* out, int64_t n) {
  if (n < 0 || n % 16 != 0) return fail(PKV_EINVAL, "%s: n must be a non-negative multiple of 16", op);
  if (n > 0 && (!y || !out)) return fail(PKV_EINVAL, "%s: null buffer pointer", op);
  if (!aligned(y, 16) || !aligned(out, 16)) return fail(PKV_EALIGN, "%s: buffers must be 16-byte aligned", op);
  return PKV_OK;
}

int pkv_diag_encode_e4m3(const float* y, uint8_t* out, int64_t n, void* stream) {
  static const char* op = "pkv_diag_encode_e4m3";
  if (int rc = check_diag(op, y, out, n)) return rc;
  if (n == 0) return ok();
  return launched(pkv::launch_diag_e4m3(y, out, n, static_cast<hipStream_t>(stream)), op);
}

int pkv_diag_encode_e2m1(const float* y, uint8_t* out, int64_t n, void* stream) {
  static const char* op = "pkv_diag_encode_e2m1";
  if (int rc = check_diag(op, y, out, n)) return rc;
  if (n == 0) return ok();
  return launched(pkv::launch_diag_e2m1(y, out, n, static_cast<hipStream_t>(stream)), op);
}

int pkv_diag_narrow(const float* x, uint16_t* out, int64_t n, int32_t out_dtype, void* stream) {
  static const char* op = "pkv_diag_narrow";
  if (out_dtype != PKV_DTYPE_BF16 && out_dtype != PKV_DTYPE_F16)
    return fail(PKV_EINVAL, "%s: out_dtype must be PKV_DTYPE_BF16 or PKV_DTYPE_F16, got %d", op, out_dtype);
  if (int rc = check_diag(op, x, reinterpret_cast<const uint8_t*>(out), n)) return rc;
  if (n == 0) return ok();
  return launched(pkv::launch_diag_narrow(x, out, n, out_dtype, static_cast<hipStream_t>(stream)), op);
}

int64_t pkv_attention_balanced_units(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                     int32_t max_context_len, int32_t partition_size,
                                     int32_t wave_slots) {
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0 ||
      max_context_len < 0 || max_context_len > (1 << 30) || partition_size < 64 ||
      partition_size > 2048 || (partition_size & (partition_size - 1)) != 0 || wave_slots <= 0)
    return 0;
  return pkv::attention_balanced_units(num_seqs, num_heads, num_kv_heads, max_context_len,
                                       partition_size, wave_slots);
}

}  // extern "C"
