/*
 * pkv.h -- C ABI of libpkv, the paged quantized KV-cache data path for
 * AMD Instinct MI355X (gfx950).
 *
 * Three operations, named after the pages that define them:
 *
 *   pkv_store_indexer_k_fp8   quantize bf16/fp16 keys per token to OCP fp8 E4M3
 *                             with a binary32 scale (amax/448) and scatter
 *                             codes and scale into indexer K cache pages by
 *                             slot_mapping.
 *   pkv_gather_indexer_k_fp8  copy the fp8 key rows and their 4 scale bytes
 *                             of every request's tokens out of the paged
 *                             indexer K cache into contiguous buffers, driven
 *                             by block_table and cu_seq_lens (vLLM PR "Add
 *                             gather_indexer_k_quant_cache kernel", call site
 *                             with kv_cache, k_fp8, k_scale, block_table,
 *                             cu_seq_lens; vLLM PR "[Deepseek-V3.2][Kernel]
 *                             Integrate cuda indexer k cache gather": k_scale
 *                             is a byte buffer viewed as float32).
 *   pkv_store_kv_fp4          NVFP4 K/V store: 16-element blocks quantized to
 *                             packed E2M1 plus one E4M3 block scale, written
 *                             into [K_data|K_scale|V_data|V_scale] pages (vLLM
 *                             source nvfp4_kv_cache_kernels.cu: header
 *                             comment, swizzle_scale_offset,
 *                             reshape_and_cache_nvfp4_kernel and
 *                             reshape_and_cache_nvfp4_dispatch).
 *
 * and, on the reader side, two gathers that return the cached keys (and
 * values) dequantised to bf16 or fp16 rows for consumers without fp8 / fp4
 * inputs:
 *
 *   pkv_gather_indexer_k_dequant  the gather above, each element then
 *                             E4M3 decode(code) * scale.
 *   pkv_gather_kv_fp4_dequant  NVFP4 pages back to K and V rows, each element
 *                             E2M1 decode(code) * block scale * k_scale
 *                             (v_scale for V).
 *
 * and the consumer the integration PR hands the gathered k_fp8 and
 * k_scale.view(float32) to:
 *
 *   pkv_fp8_mqa_logits        indexer scores of query tokens against the
 *                             gathered keys (fp8 MFMA contraction).
 *
 * and the decode consumer of fp8 K/V pages with per-tensor scales:
 *
 *   pkv_paged_attention_decode  one query token per sequence attends over
 *                             its paged fp8 keys and values (vLLM PR
 *                             "[ROCm] Faster Custom Paged Attention
 *                             kernels").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every buffer pointer is a DEVICE pointer owned by the caller.  The
 *    library allocates nothing, never synchronizes, and enqueues its kernels
 *    on `stream` (a hipStream_t passed as void*; NULL = the null stream).
 *  - Inputs are read-only (const); only the documented outputs are written.
 *  - Return value: PKV_OK (0) when the work was enqueued, or a negative
 *    PKV_E* code, in which case NOTHING was enqueued and pkv_last_error()
 *    returns a message (thread-local, valid until the next call on the same
 *    thread).  Argument checks run on the host before any HIP call.
 *  - Values that live in device memory (slots, page ids, cumulative lengths)
 *    cannot be checked on the host without a synchronization.  Out-of-range
 *    ones are skipped by the kernels, never dereferenced: a negative slot, a
 *    slot past num_blocks*block_size, a page id outside [0, num_blocks), a
 *    block-table column >= max_blocks_per_req, an output row outside
 *    [0, num_tokens).  Duplicate slots, or overlapping cu_seq_lens ranges,
 *    give unspecified (but in-bounds) results.
 *  - Numerics are defined for finite bf16/fp16 inputs; non-finite inputs give
 *    unspecified codes (memory access is unaffected).
 *  - Results are bit-exact and independent of the launch configuration.
 */
#ifndef PKV_H
#define PKV_H

#include <stdint.h>

/* Every entry point is exported; the library is built with hidden
 * visibility otherwise, so nothing else of it is. */
#define PKV_API __attribute__((visibility("default")))

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_OK 0
#define PKV_EINVAL (-1)        /* null pointer with non-zero work, bad size   */
#define PKV_EUNSUPPORTED (-2)  /* valid request outside what the kernels do  */
#define PKV_EALIGN (-3)        /* pointer or stride misaligned               */
#define PKV_ELAUNCH (-4)       /* the HIP launch itself reported an error    */

#define PKV_LAYOUT_HND 0       /* per page side: data [H][B][D/2], scales [H][B][D/16] */
#define PKV_LAYOUT_NHD 1       /* per page side: data [B][H][D/2], scales [B][H][D/16] */

/* Source element types of the stores (the NVFP4 store's dispatcher on the
 * vLLM page covers both 16-bit float types); both widen exactly to binary32.
 * The same two are the output types of the dequantising gathers. */
#define PKV_DTYPE_BF16 0
#define PKV_DTYPE_F16 1

/* ABI version of this header; bumped when a signature changes. */
#define PKV_ABI_VERSION 6
PKV_API int pkv_abi_version(void);

/* Message for the last non-zero status on this thread ("" if none). */
PKV_API const char *pkv_last_error(void);

/*
 * Gather (vLLM PR "Add gather_indexer_k_quant_cache kernel").
 *
 * For each request r in [0, num_reqs) and each token i in
 * [0, cu_seq_lens[r+1] - cu_seq_lens[r]):
 *     page = block_table[r * max_blocks_per_req + i / block_size]
 *     off  = i % block_size
 *     row  = cu_seq_lens[r] + i
 *     k_fp8[row, 0:head_dim] = page bytes [off*head_dim, (off+1)*head_dim)
 *     k_scale[row, 0:4]      = page bytes [block_size*head_dim + off*4, +4)
 * Bytes are copied verbatim; no other output byte is written.
 *
 *   kv_cache           [num_blocks, cache_block_stride] bytes; page p starts
 *                      at kv_cache + p*cache_block_stride and holds
 *                      [block_size*head_dim code bytes | block_size*4 scale
 *                      bytes].  16-byte aligned; stride a multiple of 16 and
 *                      >= block_size*(head_dim+4).
 *   k_fp8              [num_tokens, head_dim] bytes, written.  16-byte aligned.
 *   k_scale            [num_tokens, 4] bytes (binary32 little-endian), written.
 *                      4-byte aligned.
 *   block_table        int32 [num_reqs, max_blocks_per_req], row-major.
 *   cu_seq_lens        int32 [num_reqs + 1]; cu_seq_lens[0] need not be 0.
 *   head_dim           multiple of 16.
 * Errors: PKV_EINVAL for negative sizes or missing pointers, PKV_EALIGN,
 * PKV_EUNSUPPORTED when head_dim % 16 != 0, the stride is too small,
 * num_reqs * max_blocks_per_req exceeds 2^31 - 1 or max_blocks_per_req
 * exceeds 2^22.  Tables of more than 2^22 entries are gathered by several
 * launches (request ranges), in order on the stream.
 */
PKV_API int pkv_gather_indexer_k_fp8(const void *kv_cache, void *k_fp8, void *k_scale,
                                     const int32_t *block_table, const int32_t *cu_seq_lens,
                                     int32_t num_reqs, int32_t max_blocks_per_req,
                                     int64_t num_tokens, int64_t num_blocks,
                                     int64_t cache_block_stride, int32_t block_size,
                                     int32_t head_dim, void *stream);

/*
 * fp8 per-token store into the indexer K cache (the producer of the pages
 * the gather reads; page layout as above).
 *
 * For each token t with slot = slot_mapping[t] >= 0 and
 * page = slot / block_size < num_blocks, off = slot % block_size:
 *     x_i  = k[t*k_row_stride + i], i < head_dim, widened exactly
 *     s    = binary32(max_i |x_i| / 448)              (IEEE division, RNE)
 *     code = E4M3(binary32(x_i / s))   (x_i itself when s == 0; OCP E4M3FN,
 *                                       round to nearest even, saturating)
 *     page bytes [off*head_dim + i]            = code_i
 *     page bytes [block_size*head_dim + off*4, +4) = s, little-endian
 *
 *   k             bf16 or fp16 (k_dtype) [num_tokens, >= head_dim] with row
 *                 stride k_row_stride ELEMENTS (>= head_dim, multiple of 8);
 *                 16-byte aligned.
 *   k_dtype       PKV_DTYPE_BF16 or PKV_DTYPE_F16.
 *   slot_mapping  int64 [num_tokens]; 8-byte aligned.
 *   kv_cache      written; 16-byte aligned; stride as for the gather.
 *   head_dim      multiple of 16, at most 1024.
 * Calls of more than 2^22 tokens are stored by several launches (token
 * ranges), in order on the stream.
 */
PKV_API int pkv_store_indexer_k_fp8(const void *k, int64_t k_row_stride, int32_t k_dtype,
                                    const int64_t *slot_mapping, int64_t num_tokens,
                                    void *kv_cache, int64_t num_blocks,
                                    int64_t cache_block_stride, int32_t block_size,
                                    int32_t head_dim, void *stream);

/*
 * NVFP4 K/V store (vLLM nvfp4_kv_cache_kernels.cu).
 *
 * key_cache / value_cache are side 0 / side 1 of page 0 (kv_cache[:,0] and
 * kv_cache[:,1]); page p of a side starts page_stride bytes after page p-1.
 * Inside a side, data (H*B*D/2 bytes) is followed by scales (H*B*D/16
 * bytes), laid out per `layout` (PKV_LAYOUT_HND or PKV_LAYOUT_NHD).
 * For each token t with slot = slot_mapping[t] >= 0, page = slot / B <
 * num_blocks, off = slot % B; for K then V (global scale gs = 1/k_scale,
 * resp. 1/v_scale, binary32 division); for every head h and 16-element
 * group g (S = D/16 groups per head):
 *     amax = max |x|, sf = binary32(binary32(amax*gs)/6), sf8 = E4M3(sf),
 *     r = gs / decode(sf8)  (0 when decode(sf8) == 0),
 *     c_k = E2M1(binary32(x_k * r))  (round to nearest even, saturating at 6)
 *     data bytes m = 0..7 of the group: c_{2m} | c_{2m+1} << 4
 *     scale byte sf8 at (row off, column g) for K; for V at the swizzled
 *     (row (off/4)*4 + g/(S/4), column (g % (S/4))*4 + off%4).
 *
 *   key, value      bf16 or fp16 (src_dtype) [num_tokens, num_heads,
 *                   head_size]; heads and elements contiguous, token stride
 *                   *_row_stride ELEMENTS (>= H*D, multiple of 8); 16-byte
 *                   aligned.
 *   src_dtype       PKV_DTYPE_BF16 or PKV_DTYPE_F16.
 *   key_cache,
 *   value_cache     written; 8-byte aligned; page_stride multiple of 8 and
 *                   >= the side size H*B*(D/2 + D/16).
 *   slot_mapping    int64 [num_tokens].
 *   k_scale,
 *   v_scale         device binary32 scalars (the checkpoint scales), each a
 *                   positive normal value, 2^-126 <= scale <= FLT_MAX, so
 *                   that the global scale 1/scale is positive and finite.
 *                   Zero, negative, subnormal or non-finite scales are
 *                   outside the contract: the bytes written for them are
 *                   unspecified (the addresses written are not affected).
 *                   The value is read on the device, so it is not checked.
 *   head_size       multiple of 64 (so each 4x4 swizzle tile is complete);
 *   block_size      multiple of 4.
 */
PKV_API int pkv_store_kv_fp4(const void *key, int64_t key_row_stride, const void *value,
                             int64_t value_row_stride, int32_t src_dtype, void *key_cache,
                             void *value_cache,
                             const int64_t *slot_mapping, int64_t num_tokens,
                             int32_t num_heads, int32_t head_size, int32_t block_size,
                             int64_t num_blocks, int64_t page_stride, int32_t layout,
                             const float *k_scale, const float *v_scale, void *stream);

/*
 * Dequantising gather of the indexer K cache (the gather of vLLM PR "Add
 * gather_indexer_k_quant_cache kernel" followed by the dequantisation its
 * per-token scale stands for).
 *
 * For each request r and token i of it, with page, off and row as for
 * pkv_gather_indexer_k_fp8 and s the binary32 scale of the token (page bytes
 * [block_size*head_dim + off*4, +4), little-endian):
 *     out[row*out_row_stride + d] = ROUND(binary32(E4M3 decode(code_d) * s))
 * for d < head_dim, where ROUND is round to nearest even into bf16 or fp16
 * (out_dtype; overflow gives infinity).  The same skip rules as the gather;
 * no other output element is written.
 *
 *   kv_cache         as for the gather (16-byte aligned, stride a multiple
 *                    of 16 and >= block_size*(head_dim+4)).
 *   out              [num_tokens, >= head_dim] bf16 or fp16, row stride
 *                    out_row_stride ELEMENTS (>= head_dim, multiple of 8);
 *                    16-byte aligned; written.
 *   out_dtype        PKV_DTYPE_BF16 or PKV_DTYPE_F16.
 *   block_table, cu_seq_lens, sizes: as for the gather.
 * Codes 0x7F / 0xFF (NaN) and non-finite scales are never written by the
 * store; reading them gives NaN or infinity (NaN bits unspecified).
 * Errors: as for the gather, plus PKV_EINVAL for a bad out_dtype or row
 * stride and PKV_EALIGN for a row stride that is not a multiple of 8.
 */
PKV_API int pkv_gather_indexer_k_dequant(const void *kv_cache, void *out, int64_t out_row_stride,
                                         int32_t out_dtype, const int32_t *block_table,
                                         const int32_t *cu_seq_lens, int32_t num_reqs,
                                         int32_t max_blocks_per_req, int64_t num_tokens,
                                         int64_t num_blocks, int64_t cache_block_stride,
                                         int32_t block_size, int32_t head_dim, void *stream);

/*
 * NVFP4 K/V pages read back (the inverse of pkv_store_kv_fp4 up to its
 * quantisation; page layout, HND / NHD and the V-scale swizzle as there).
 *
 * For each request r and token i of it: page = block_table[r *
 * max_blocks_per_req + i / block_size], off = i % block_size, row =
 * cu_seq_lens[r] + i; for K then V, every head h and 16-element group g:
 * sfd = E4M3 decode of the group's scale byte, and for element k
 *     out[row*row_stride + h*head_size + 16g + k] =
 *         ROUND(binary32(E2M1 decode(code_k) * sfd * scale))
 * where E2M1 decode(code_k) * sfd is exact, scale = *k_scale for K and
 * *v_scale for V (the store's global scale is their reciprocal), and ROUND is
 * round to nearest even into bf16 or fp16 (out_dtype).  Skip rules as for the
 * gathers; no other output element is written.
 *
 *   key_cache,
 *   value_cache      side 0 / side 1 of page 0, as for the store; 16-byte
 *                    aligned; page_stride a multiple of 16 and >= the side
 *                    size H*B*(D/2 + D/16).
 *   key_out,
 *   value_out        [num_tokens, >= H*D] bf16 or fp16, row strides in
 *                    ELEMENTS (>= H*D, multiples of 8); 16-byte aligned;
 *                    written.
 *   block_table      int32 [num_reqs, max_blocks_per_req].
 *   cu_seq_lens      int32 [num_reqs + 1].
 *   k_scale,
 *   v_scale          device binary32 scalars.
 *   head_size        multiple of 64; block_size multiple of 4.
 * NaN scale bytes (0x7F / 0xFF) are never written by the store; reading them
 * gives NaN (bits unspecified).
 */
PKV_API int pkv_gather_kv_fp4_dequant(const void *key_cache, const void *value_cache, void *key_out,
                                      int64_t key_row_stride, void *value_out,
                                      int64_t value_row_stride, int32_t out_dtype,
                                      const int32_t *block_table, const int32_t *cu_seq_lens,
                                      int32_t num_reqs, int32_t max_blocks_per_req,
                                      int64_t num_tokens, int32_t num_heads, int32_t head_size,
                                      int32_t block_size, int64_t num_blocks, int64_t page_stride,
                                      int32_t layout, const float *k_scale, const float *v_scale,
                                      void *stream);

/*
 * Indexer logits on the gathered keys (vLLM PR "[Deepseek-V3.2][Kernel]
 * Integrate cuda indexer k cache gather": the gathered k_fp8 and
 * k_scale.view(float32) go to fp8_mqa_logits; the pages do not show that
 * op's body, and this is the lightning-indexer score).
 *
 * For query token i < num_q and key j in [max(ks[i], 0), min(ke[i], num_k))
 * with j - ks[i] < row_cols:
 *     logits[i*row_stride + (j - ks[i])] =
 *         k_scale[j] * sum_h weights[i*num_heads + h] * relu(q[i,h,:] . k[j,:])
 * where q and k are OCP E4M3 codes.  No other logits element is written.
 * The dot products run on fp8 MFMA (v_mfma_f32_16x16x128_f8f6f4) in binary32;
 * that unit adds each group of 8 consecutive products aligned to the
 * group's largest, dropping bits below about 2^-13 of it, so results agree
 * with the exact value within a bound (the tests state it), not bit for bit.
 * k_scale must be >= 0 (the gathered scales are).
 *
 *   q          E4M3 [num_q, num_heads, head_dim], heads and elements
 *              contiguous, token stride q_token_stride BYTES (>= H*D,
 *              multiple of 16); 16-byte aligned.
 *   k          E4M3 [num_k, head_dim] contiguous (the gather's k_fp8);
 *              16-byte aligned.
 *   k_scale    binary32 [num_k] (the gather's k_scale).
 *   weights    binary32 [num_q, num_heads].
 *   ks, ke     int32 [num_q]: the key range of each query token.
 *   logits     binary32, row i at logits + i*row_stride, columns
 *              [0, row_cols) of it are written (row_stride >= row_cols).
 *   head_dim   128; num_heads 16, 32, 48 or 64.
 * The entry point currently validates its arguments and then returns
 * PKV_EUNSUPPORTED without launching: a GPU run of its kernel on causal
 * per-request ranges did not finish, and the cause is not found yet.
 */
PKV_API int pkv_fp8_mqa_logits(const void *q, int64_t q_token_stride, const void *k,
                               const float *k_scale, const float *weights, const int32_t *ks,
                               const int32_t *ke, float *logits, int64_t row_stride, int64_t row_cols,
                               int32_t num_q, int32_t num_heads, int64_t num_k, int32_t head_dim,
                               void *stream);

/*
 * Paged decode attention over fp8 pages (vLLM PR "[ROCm] Faster Custom Paged
 * Attention kernels": the op paged_attention(out, exp_sums, max_logits,
 * tmp_out, query, key_cache, value_cache, num_kv_heads, scale, block_tables,
 * context_lens, block_size, max_context_len, ..., kv_cache_dtype, k_scale,
 * v_scale, ..., partition_size), with an fp8 cache and per-tensor scales;
 * the schema's optional ALiBi slopes and fp8 output scale are not taken:
 * no ALiBi, bf16 output).
 *
 * For sequence s < num_seqs and head h < num_heads, with
 * kvh = h / (num_heads / num_kv_heads) and tokens t < context_lens[s]:
 *     k_t[d] = E4M3dec(key_cache[page][kvh][d/16][t%B][d%16]) * k_scale
 *     v_t[d] = E4M3dec(value_cache[page][kvh][d][t%B]) * v_scale
 *     page   = block_tables[s*max_blocks_per_seq + t/B]
 *     out[s][h][:] = bf16( sum_t softmax_t(scale * q[s][h] . k_t) v_t )
 * Tokens whose page id is outside [0, num_blocks) are left out of the
 * softmax; a sequence with no token left (or context_lens[s] <= 0) gets a
 * zero row.  Only tokens t < ceil(max_context_len / partition_size) *
 * partition_size are read: max_context_len must be >= every context_lens[s].
 *
 * The work is split into segments: runs of whole 64-token blocks of one
 * sequence, at most 2048 tokens.  When the workspace has room, the blocks of
 * all sequences are dealt out in equal shares, one per wave the GPU holds at
 * once, so that mixed context lengths keep every wave equally busy; else
 * (or for more than 4096 sequences) each partition of partition_size tokens
 * is a segment, as on the page.  A first kernel writes each segment's
 * softmax denominator, maximum logit and normalised partial output to the
 * caller's workspace (a sequence that is a single segment gets its output
 * row directly), and a second combines them.  partition_size therefore
 * sizes the workspace and the fixed split; the result does not depend on it
 * beyond rounding.  The dot products run on bf16 MFMA
 * (v_mfma_f32_16x16x32_bf16; fp8 keys and values are exact in bf16, the
 * probabilities enter as a bf16 high + low pair) with binary32
 * accumulation, and the exponentials on the hardware exp2; results agree
 * with the exact value within a bound (the tests state it), not bit for bit.
 *
 *   out          bf16 [num_seqs, num_heads, head_size]; 16-byte aligned.
 *   exp_sums,    binary32 [num_seqs, num_heads, max_num_partitions] with
 *   max_logits   max_num_partitions = ceil(max_context_len/partition_size);
 *                workspace written and read by the call.
 *   tmp_out      binary32 [num_seqs, num_heads, max_num_partitions,
 *                head_size]; workspace.  16-byte aligned.
 *   query        bf16 [num_seqs, num_heads, head_size]; 16-byte aligned.
 *   key_cache    E4M3 [num_blocks, num_kv_heads, head_size/16, block_size,
 *                16]; 16-byte aligned.
 *   value_cache  E4M3 [num_blocks, num_kv_heads, head_size, block_size];
 *                16-byte aligned.
 *   block_tables int32 [num_seqs, max_blocks_per_seq].
 *   context_lens int32 [num_seqs].
 *   head_size 128; block_size a positive multiple of 16;
 *   num_heads a multiple of num_kv_heads with at most 16 query heads per KV
 *   head; partition_size a power of two in [64, 2048]; max_context_len <= 2^30;
 *   num_seqs*num_heads and num_seqs*num_kv_heads*max_num_partitions below
 *   2^31; scale, k_scale, v_scale finite host values.
 * The workspace is the caller's: the library allocates nothing.  Calls that
 * share a workspace must be ordered on one stream.
 */
PKV_API int pkv_paged_attention_decode(void *out, float *exp_sums, float *max_logits, float *tmp_out,
                                       const void *query, const void *key_cache,
                                       const void *value_cache, const int32_t *block_tables,
                                       const int32_t *context_lens, int32_t num_seqs, int32_t num_heads,
                                       int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                                       int32_t max_blocks_per_seq, int32_t max_context_len,
                                       int64_t num_blocks, float scale, float k_scale, float v_scale,
                                       int32_t partition_size, void *stream);

/*
 * Allocation-free variant of pkv_paged_attention_decode, for callers that
 * cannot allocate device memory: code being captured into a HIP graph, tight
 * serving loops, harnesses that forbid hipMalloc.  Arguments, results and
 * errors are those of pkv_paged_attention_decode without its three workspace
 * buffers: the workspace is carved out of a library-owned device array of
 * PKV_ATTENTION_SCRATCH_BYTES bytes, one per GPU, held until the process
 * ends (its address is looked up once per device, on the first call there).
 * The call allocates nothing.
 *
 * A call needs 2 * align256(4 n) + 512 n workspace bytes, n = num_seqs *
 * num_heads * ceil(max_context_len / partition_size) (head_size 128); one
 * that needs more than PKV_ATTENTION_SCRATCH_BYTES returns PKV_EUNSUPPORTED
 * and enqueues nothing (PKV_ELAUNCH if the array's address cannot be looked
 * up).  The array is the current device's, so `stream` must belong to the
 * current device (PKV_EINVAL otherwise).  Every workspace element a call reads was written earlier in the
 * same call, so nothing carries over from one call to the next.  All calls
 * on one GPU share its array: calls that may run at the same time on one
 * GPU (on different streams, or enqueued from different threads without
 * ordering) race and give undefined results; order them on one stream.
 */
#define PKV_ATTENTION_SCRATCH_BYTES (32u << 20)
PKV_API int pkv_paged_attention_decode_noalloc(void *out, const void *query,
                                               const void *key_cache, const void *value_cache,
                                               const int32_t *block_tables,
                                               const int32_t *context_lens, int32_t num_seqs,
                                               int32_t num_heads, int32_t num_kv_heads,
                                               int32_t head_size, int32_t block_size,
                                               int32_t max_blocks_per_seq,
                                               int32_t max_context_len, int64_t num_blocks,
                                               float scale, float k_scale, float v_scale,
                                               int32_t partition_size, void *stream);

/* Host-only query (no GPU work): the number of work units the balanced split
 * of pkv_paged_attention_decode uses for these sizes when the device holds
 * wave_slots partition-kernel waves at once (a compute unit holds 12), or 0
 * when the call takes the fixed split of partitions of partition_size
 * tokens.  Arguments as for pkv_paged_attention_decode; returns 0 for sizes
 * that call would reject. */
PKV_API int64_t pkv_attention_balanced_units(int32_t num_seqs, int32_t num_heads,
                                             int32_t num_kv_heads, int32_t max_context_len,
                                             int32_t partition_size, int32_t wave_slots);


/*
 * Diagnostics: the device codecs the store kernels use, exposed so that a
 * test can sweep them over every binary32 input.
 *   pkv_diag_encode_e4m3: out[i] = E4M3(y[i]); defined for |y[i]| < 464
 *                         (the store kernels never pass a larger magnitude).
 *   pkv_diag_encode_e2m1: out[i] = E2M1(y[i]) in the low nibble; defined for
 *                         every non-NaN y[i].
 * y: binary32 [n], 16-byte aligned; out: bytes [n]; n a multiple of 16.
 */
PKV_API int pkv_diag_encode_e4m3(const float *y, uint8_t *out, int64_t n, void *stream);
PKV_API int pkv_diag_encode_e2m1(const float *y, uint8_t *out, int64_t n, void *stream);

/*
 * Diagnostic: the output rounding of the dequantising gathers,
 * out[i] = ROUND(x[i]) into bf16 or fp16 (out_dtype), round to nearest even.
 * x: binary32 [n], 16-byte aligned; out: 16-bit [n], 16-byte aligned; n a
 * multiple of 16.  NaN inputs give NaN (bits unspecified).
 */
PKV_API int pkv_diag_narrow(const float *x, uint16_t *out, int64_t n, int32_t out_dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
