/*
 * pkv_oracle.c -- plain, slow, single-threaded CPU oracle for the paged
 * quantized KV-cache data path.
 *
 * TEST INFRASTRUCTURE ONLY.  This file decides what the right bytes are; it
 * is not part of the product.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it.  It shares no code, header,
 * table or constant with the HIP library, and neither side includes the
 * other.
 *
 * Build: gcc -O2 -std=c11 -fno-fast-math -ffp-contract=off -fPIC -shared
 * (IEEE binary32 arithmetic, round-to-nearest-even, subnormals honoured,
 * every float expression rounded to binary32 at each step; x86-64 SSE has
 * FLT_EVAL_METHOD == 0).
 *
 * Sources, cited by page and section:
 *   [P1] vLLM PR "Add gather_indexer_k_quant_cache kernel" -- the op that
 *        copies quantized keys and their scales out of the paged indexer K
 *        cache, and its call site (kv_cache, k_fp8, k_scale, block_table,
 *        cu_seq_lens).
 *   [P2] vLLM PR "[Deepseek-V3.2][Kernel] Integrate cuda indexer k cache
 *        gather" -- review note: k_scale is a byte buffer read back with
 *        .view(torch.float32).
 *   [P3] vLLM source "csrc/libtorch_stable/nvfp4_kv_cache_kernels.cu" --
 *        header comment (page layout [K_data|K_scale|V_data|V_scale]),
 *        swizzle_scale_offset, reshape_and_cache_nvfp4_kernel and
 *        reshape_and_cache_nvfp4_dispatch.
 *
 * Readings where the pages are silent (listed in full in the design notes):
 *   - fp8 is OCP E4M3FN (bias 7, max 448, NaN 0x7F, no infinity), rounding to
 *     nearest with ties to the even code, saturating at +-448; the sign of
 *     zero is kept.
 *   - indexer page = [block_size*head_dim code bytes | block_size*4 scale
 *     bytes]; the per-token scale is amax/448 in binary32, stored as 4
 *     little-endian bytes; codes are E4M3(x / scale) with a true division.
 *   - NVFP4 block: 16 elements, scale sf = (amax*gs)/6 rounded to E4M3,
 *     codes E2M1(x * (gs/sf)), element 2m in the low nibble of byte m.
 *   - Out-of-range indices (page ids, block-table columns, output rows,
 *     slots past the cache) are skipped, never dereferenced.
 *   - Inputs are finite bf16 or fp16; non-finite inputs are outside the contract
 *     (the oracle still returns deterministic bytes for them).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* bf16 -> binary32: bf16 is the top half of a binary32 pattern, so the  */
/* widening is exact.                                                   */
/* ------------------------------------------------------------------ */
float oracle_bf16_to_f32(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

/* binary16 -> binary32, from the format's definition: sign, 5-bit exponent
 * (bias 15), 10-bit fraction; exponent 0 is subnormal (m * 2^-24), 31 is
 * infinity / NaN.  Every value is exact in binary32. */
float oracle_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp(1024.0 + m, e - 25);
    return (float)(sign ? -v : v);
}

/* Source element widening.  The NVFP4 store's dispatcher on the vLLM page
 * instantiates the kernel for both 16-bit float types (fp16 and bf16). */
#define ORACLE_SRC_BF16 0
#define ORACLE_SRC_F16 1
static float widen(uint16_t h, int32_t src_dtype)
{
    return src_dtype == ORACLE_SRC_F16 ? oracle_f16_to_f32(h) : oracle_bf16_to_f32(h);
}

/* ------------------------------------------------------------------ */
/* OCP E4M3FN.                                                         */
/*   code = s eeee mmm; e == 0: value m * 2^-9 (subnormal);            */
/*   e > 0: (1 + m/8) * 2^(e-7); 0x7F / 0xFF are NaN; max is 0x7E = 448. */
/* ------------------------------------------------------------------ */
float oracle_e4m3_decode(uint8_t code)
{
    int sign = code & 0x80;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double v;
    if ((code & 0x7F) == 0x7F)
        return sign ? -NAN : NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(8.0 + m, e - 10);
    return (float)(sign ? -v : v);
}

/* Round a binary32 value to the nearest E4M3 value, ties to the even code,
 * saturating to +-448.  Worked in binary64, where every step below is
 * exact except rint(), which performs the single round-to-nearest-even. */
uint8_t oracle_e4m3_encode(float y)
{
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    double a;
    int e;
    double m;

    if (isnan(y))
        return sign | 0x7F;
    a = fabs((double)y);
    if (a >= 448.0)                 /* saturate; includes +-inf */
        return sign | 0x7E;
    if (a < 0x1p-6) {               /* subnormal range, spacing 2^-9 */
        /* 0..8; 8 lands on 0x08, the smallest normal (2^-6) */
        return sign | (uint8_t)rint(a * 512.0);
    }
    e = ilogb(a);                   /* a in [2^e, 2^(e+1)), -6 <= e <= 8 */
    m = rint(ldexp(a, 3 - e));      /* significand with 3 fraction bits: 8..16 */
    if (m == 16.0) {                /* rounded up into the next binade */
        m = 8.0;
        e += 1;
    }
    if (e > 8 || (e == 8 && m > 14.0))
        return sign | 0x7E;         /* unreachable for a < 448; kept as a guard */
    return sign | (uint8_t)(((e + 7) << 3) | ((int)m - 8));
}

/* ------------------------------------------------------------------ */
/* E2M1 (4-bit: s ee m): magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6} for      */
/* codes 0..7; the sign is bit 3.                                       */
/* ------------------------------------------------------------------ */
static const double e2m1_grid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

float oracle_e2m1_decode(uint8_t code)
{
    double v = e2m1_grid[code & 7];
    return (float)((code & 8) ? -v : v);
}

/* Nearest grid magnitude, ties to the even code, saturating at 6.
 * Written as the definition: scan the grid. */
uint8_t oracle_e2m1_encode(float y)
{
    uint8_t sign = signbit(y) ? 0x8 : 0x0;
    double a;
    int best = 0, k;
    double bestd;

    if (isnan(y))
        return sign | 0x7;          /* outside the contract; deterministic */
    a = fabs((double)y);
    if (a >= 6.0)
        return sign | 0x7;
    bestd = a;                      /* distance to code 0 */
    for (k = 1; k < 8; ++k) {
        double d = fabs(a - e2m1_grid[k]);
        if (d < bestd || (d == bestd && (k % 2) == 0)) {
            best = k;
            bestd = d;
        }
    }
    return sign | (uint8_t)best;
}

/* Array helpers so the test suite can sweep the codecs quickly. */
void oracle_e4m3_encode_array(const float *y, uint8_t *out, int64_t n)
{
    int64_t i;
    for (i = 0; i < n; ++i)
        out[i] = oracle_e4m3_encode(y[i]);
}

void oracle_e2m1_encode_array(const float *y, uint8_t *out, int64_t n)
{
    int64_t i;
    for (i = 0; i < n; ++i)
        out[i] = oracle_e2m1_encode(y[i]);
}

/* ------------------------------------------------------------------ */
/* [P3] swizzle_scale_offset: a per-head [T, S] scale tile (T = block    */
/* size, S = head_size/16) is stored as [T/4, 4, 4, S/4] permuted to     */
/* (0, 2, 3, 1).  Position (t, s) moves to row (t/4)*4 + s/(S/4), column */
/* (s % (S/4))*4 + t%4.  Returns row*S + column.                         */
/* ------------------------------------------------------------------ */
int oracle_swizzle_offset(int t, int s, int S)
{
    int q = S / 4;
    int row = (t / 4) * 4 + s / q;
    int col = (s % q) * 4 + t % 4;
    return row * S + col;
}

/* ------------------------------------------------------------------ */
/* [P1] gather: for each request r and each of its tokens i, copy the    */
/* code row and the 4 scale bytes of token i out of page                 */
/* block_table[r][i / B] at offset i % B into row cu_seq_lens[r] + i of   */
/* k_fp8 / k_scale.  Everything else is left untouched.                  */
/* Page layout: [B*D code bytes | B*4 scale bytes], page p at            */
/* kv_cache + p * cache_block_stride.                                    */
/* ------------------------------------------------------------------ */
void oracle_gather_indexer_k_fp8(const uint8_t *kv_cache, uint8_t *k_fp8,
                                 uint8_t *k_scale, const int32_t *block_table,
                                 const int32_t *cu_seq_lens, int32_t num_reqs,
                                 int32_t max_blocks_per_req, int64_t num_tokens,
                                 int64_t num_blocks, int64_t cache_block_stride,
                                 int32_t block_size, int32_t head_dim)
{
    int32_t r;
    for (r = 0; r < num_reqs; ++r) {
        int64_t start = cu_seq_lens[r];
        int64_t len = (int64_t)cu_seq_lens[r + 1] - start;
        int64_t i;
        for (i = 0; i < len; ++i) {
            int64_t row = start + i;
            int64_t j = i / block_size;
            int64_t off = i % block_size;
            int64_t page;
            const uint8_t *base;
            if (row < 0 || row >= num_tokens)
                continue;
            if (j >= max_blocks_per_req)
                continue;
            page = block_table[(int64_t)r * max_blocks_per_req + j];
            if (page < 0 || page >= num_blocks)
                continue;
            base = kv_cache + page * cache_block_stride;
            memcpy(k_fp8 + row * head_dim, base + off * head_dim, (size_t)head_dim);
            memcpy(k_scale + row * 4,
                   base + (int64_t)block_size * head_dim + off * 4, 4);
        }
    }
}

/* ------------------------------------------------------------------ */
/* fp8 per-token quantize and scatter into the indexer page.             */
/* For token t with slot >= 0: page = slot / B, off = slot % B;          */
/*   x_i = k[t, i] (bf16 or fp16, widened exactly);                       */
/*   amax = max |x_i|;  s = amax / 448 (binary32);                        */
/*   code_i = E4M3(x_i / s)  (x_i itself when s == 0);                   */
/*   page codes [off*D .. +D) = code, page scale bytes [B*D + off*4 .. +4) */
/*   = s, little-endian.  Slots < 0, and pages past the cache, skip.     */
/* ------------------------------------------------------------------ */
void oracle_store_indexer_k_fp8(const uint16_t *k, int64_t k_row_stride, int32_t src_dtype,
                                const int64_t *slot_mapping, int64_t num_tokens,
                                uint8_t *kv_cache, int64_t num_blocks,
                                int64_t cache_block_stride, int32_t block_size,
                                int32_t head_dim)
{
    int64_t t;
    for (t = 0; t < num_tokens; ++t) {
        int64_t slot = slot_mapping[t];
        int64_t page, off;
        const uint16_t *src = k + t * k_row_stride;
        uint8_t *base;
        float amax = 0.0f, s;
        int i;
        if (slot < 0)
            continue;
        page = slot / block_size;
        off = slot % block_size;
        if (page >= num_blocks)
            continue;
        for (i = 0; i < head_dim; ++i) {
            float a = fabsf(widen(src[i], src_dtype));
            if (a > amax)
                amax = a;
        }
        s = amax / 448.0f;
        base = kv_cache + page * cache_block_stride;
        for (i = 0; i < head_dim; ++i) {
            float x = widen(src[i], src_dtype);
            float y = (s == 0.0f) ? x : x / s;
            base[off * head_dim + i] = oracle_e4m3_encode(y);
        }
        {
            uint32_t sb;
            uint8_t le[4];
            memcpy(&sb, &s, 4);
            le[0] = (uint8_t)(sb & 0xFF);
            le[1] = (uint8_t)((sb >> 8) & 0xFF);
            le[2] = (uint8_t)((sb >> 16) & 0xFF);
            le[3] = (uint8_t)((sb >> 24) & 0xFF);
            memcpy(base + (int64_t)block_size * head_dim + off * 4, le, 4);
        }
    }
}

/* ------------------------------------------------------------------ */
/* [P3] NVFP4 K/V store.                                                 */
/* key_cache / value_cache point at side 0 / side 1 of page 0; page p of  */
/* a side starts page_stride bytes after page p-1.  Inside a side the    */
/* data region (H*B*D/2 bytes) is followed by the scale region           */
/* (H*B*D/16 bytes).  HND (layout 0): data [H][B][D/2], scales [H][B][S]; */
/* NHD (layout 1): data [B][H][D/2], scales [B][H][S]; S = D/16.          */
/* For each token with slot >= 0, for K then V, gs = 1/scale, and for    */
/* every head h and 16-element group g:                                  */
/*   amax = max|x|, sf = (amax*gs)/6, sf8 = E4M3(sf), sfd = decode(sf8),  */
/*   r = gs/sfd (0 when sfd == 0), code_k = E2M1(x_k * r);               */
/*   8 data bytes at group g (element 2m low nibble, 2m+1 high nibble),  */
/*   scale byte sf8 at (off, g) for K and at the swizzled position for V. */
/* ------------------------------------------------------------------ */
void oracle_store_kv_fp4(const uint16_t *key, int64_t key_row_stride,
                         const uint16_t *value, int64_t value_row_stride, int32_t src_dtype,
                         uint8_t *key_cache, uint8_t *value_cache,
                         const int64_t *slot_mapping, int64_t num_tokens,
                         int32_t num_heads, int32_t head_size, int32_t block_size,
                         int64_t num_blocks, int64_t page_stride, int32_t layout,
                         float k_scale, float v_scale)
{
    const int64_t data_dim = head_size / 2;
    const int64_t S = head_size / 16;
    const int64_t data_per_side = (int64_t)num_heads * block_size * data_dim;
    int64_t t;

    for (t = 0; t < num_tokens; ++t) {
        int64_t slot = slot_mapping[t];
        int64_t page, off;
        int kv;
        if (slot < 0)
            continue;
        page = slot / block_size;
        off = slot % block_size;
        if (page >= num_blocks)
            continue;
        for (kv = 0; kv < 2; ++kv) {
            const uint16_t *src = (kv == 0) ? key + t * key_row_stride
                                            : value + t * value_row_stride;
            uint8_t *side = ((kv == 0) ? key_cache : value_cache) + page * page_stride;
            uint8_t *scales = side + data_per_side;
            float gs = 1.0f / ((kv == 0) ? k_scale : v_scale);
            int32_t h;
            int64_t g;
            for (h = 0; h < num_heads; ++h) {
                for (g = 0; g < S; ++g) {
                    float x[16];
                    float amax = 0.0f, prod, sf, sfd, rs;
                    uint8_t sf8, codes[16];
                    int k2, m;
                    int64_t data_off, scale_off, row, col;
                    for (k2 = 0; k2 < 16; ++k2) {
                        float a;
                        x[k2] = widen(src[(int64_t)h * head_size + g * 16 + k2], src_dtype);
                        a = fabsf(x[k2]);
                        if (a > amax)
                            amax = a;
                    }
                    prod = amax * gs;
                    sf = prod / 6.0f;
                    sf8 = oracle_e4m3_encode(sf);
                    sfd = oracle_e4m3_decode(sf8);
                    rs = (sfd == 0.0f) ? 0.0f : gs / sfd;
                    for (k2 = 0; k2 < 16; ++k2)
                        codes[k2] = oracle_e2m1_encode(x[k2] * rs);

                    if (layout == 0)
                        data_off = ((int64_t)h * block_size + off) * data_dim + g * 8;
                    else
                        data_off = (off * num_heads + h) * data_dim + g * 8;
                    for (m = 0; m < 8; ++m)
                        side[data_off + m] =
                            (uint8_t)(codes[2 * m] | (codes[2 * m + 1] << 4));

                    if (kv == 0) {
                        row = off;
                        col = g;
                    } else {
                        int sw = oracle_swizzle_offset((int)off, (int)g, (int)S);
                        row = sw / S;
                        col = sw % S;
                    }
                    if (layout == 0)
                        scale_off = ((int64_t)h * block_size + row) * S + col;
                    else
                        scale_off = (row * num_heads + h) * S + col;
                    scales[scale_off] = sf8;
                }
            }
        }
    }
}

/* ================================================================== */
/* Reader side: dequantising gathers.                                   */
/* ================================================================== */

/* binary32 -> bf16, round to nearest, ties to even.  bf16 keeps the top  */
/* 16 bits of the binary32 pattern; the result is the nearer of the two   */
/* bf16 values around x (by magnitude), the one with an even last kept bit */
/* on a tie; values past the largest finite bf16 by half an ulp or more    */
/* become infinity.  NaN stays NaN (quiet, sign kept).  Worked in binary64 */
/* on the magnitude, where every step is exact except rint().              */
uint16_t oracle_f32_to_bf16(float x)
{
    uint32_t bits;
    uint16_t sign;
    double a, ulp, q;
    int e;
    memcpy(&bits, &x, 4);
    sign = (uint16_t)((bits >> 16) & 0x8000);
    if (isnan(x))
        return sign | 0x7FC0;
    a = fabs((double)x);
    if (isinf(x))
        return sign | 0x7F80;
    if (a == 0.0)
        return sign;
    /* bf16 has 8 significant bits and binary32's exponent range: the ulp */
    /* of a normal value in [2^e, 2^(e+1)) is 2^(e-7); subnormals (below   */
    /* 2^-126) have ulp 2^-133.                                            */
    e = ilogb(a);
    if (e < -126)
        e = -126;
    ulp = ldexp(1.0, e - 7);
    q = rint(a / ulp) * ulp;          /* nearest multiple of the ulp, ties even */
    if (q > 0x1.FEp127)               /* past the largest finite bf16, 0x7F7F */
        return sign | 0x7F80;
    {
        float qf = (float)q;         /* exact: q has at most 8 significant bits */
        uint32_t qb;
        memcpy(&qb, &qf, 4);
        return sign | (uint16_t)((qb >> 16) & 0x7FFF);
    }
}

/* binary32 -> binary16, round to nearest, ties to even, subnormals kept,  */
/* overflow to infinity (magnitudes >= 65520, the midpoint past 65504).    */
uint16_t oracle_f32_to_f16(float x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0x0000;
    double a;
    int e;
    double m;
    if (isnan(x))
        return sign | 0x7E00;
    a = fabs((double)x);
    if (a >= 65520.0)                /* includes infinity */
        return sign | 0x7C00;
    if (a < 0x1p-14)                 /* subnormal range, spacing 2^-24; 1024 is 0x0400 */
        return sign | (uint16_t)rint(a * 0x1p24);
    e = ilogb(a);                    /* -14 <= e <= 15 */
    m = rint(ldexp(a, 10 - e));      /* 1024 .. 2048 */
    if (m == 2048.0) {
        m = 1024.0;
        e += 1;
    }
    return sign | (uint16_t)(((e + 15) << 10) | ((int)m - 1024));
}

void oracle_f32_to_bf16_array(const float *x, uint16_t *out, int64_t n)
{
    int64_t i;
    for (i = 0; i < n; ++i)
        out[i] = oracle_f32_to_bf16(x[i]);
}

void oracle_f32_to_f16_array(const float *x, uint16_t *out, int64_t n)
{
    int64_t i;
    for (i = 0; i < n; ++i)
        out[i] = oracle_f32_to_f16(x[i]);
}

#define ORACLE_OUT_BF16 0
#define ORACLE_OUT_F16 1
static uint16_t narrow(float x, int32_t out_dtype)
{
    return out_dtype == ORACLE_OUT_F16 ? oracle_f32_to_f16(x) : oracle_f32_to_bf16(x);
}

/* ------------------------------------------------------------------ */
/* [P1] gather, followed by the dequantisation the stored scale stands  */
/* for: value = E4M3 decode(code) * scale in binary32 (the product       */
/* rounded once), then rounded to the output type (bf16 or fp16, to      */
/* nearest even).  Row cu_seq_lens[r] + i of out [num_tokens, D] gets    */
/* token i of request r, from page block_table[r][i / B], offset i % B.  */
/* The same skip rules as the gather; other rows are left untouched.     */
/* ------------------------------------------------------------------ */
void oracle_gather_indexer_k_dequant(const uint8_t *kv_cache, uint16_t *out,
                                     int64_t out_row_stride, int32_t out_dtype,
                                     const int32_t *block_table, const int32_t *cu_seq_lens,
                                     int32_t num_reqs, int32_t max_blocks_per_req,
                                     int64_t num_tokens, int64_t num_blocks,
                                     int64_t cache_block_stride, int32_t block_size,
                                     int32_t head_dim)
{
    int32_t r;
    for (r = 0; r < num_reqs; ++r) {
        int64_t start = cu_seq_lens[r];
        int64_t len = (int64_t)cu_seq_lens[r + 1] - start;
        int64_t i;
        for (i = 0; i < len; ++i) {
            int64_t row = start + i;
            int64_t j = i / block_size;
            int64_t off = i % block_size;
            int64_t page;
            const uint8_t *base;
            uint8_t le[4];
            uint32_t sb;
            float s;
            int d;
            if (row < 0 || row >= num_tokens)
                continue;
            if (j >= max_blocks_per_req)
                continue;
            page = block_table[(int64_t)r * max_blocks_per_req + j];
            if (page < 0 || page >= num_blocks)
                continue;
            base = kv_cache + page * cache_block_stride;
            memcpy(le, base + (int64_t)block_size * head_dim + off * 4, 4);
            sb = (uint32_t)le[0] | ((uint32_t)le[1] << 8) | ((uint32_t)le[2] << 16) |
                 ((uint32_t)le[3] << 24);
            memcpy(&s, &sb, 4);
            for (d = 0; d < head_dim; ++d) {
                float v = oracle_e4m3_decode(base[off * head_dim + d]) * s;
                out[row * out_row_stride + d] = narrow(v, out_dtype);
            }
        }
    }
}

/* ------------------------------------------------------------------ */
/* [P3] NVFP4 pages read back: for each request r and token i, from page */
/* block_table[r][i / B] at offset i % B, for K and V, every head h and  */
/* 16-element group g: the block scale byte (K at (off, g), V at its     */
/* swizzled position), sfd = E4M3 decode of it, and for element k the   */
/* value E2M1 decode(code_k) * sfd (exact in binary32: at most 6         */
/* significant bits) times the per-tensor scale (k_scale or v_scale, the */
/* store's global scale is its reciprocal), rounded once in binary32 and */
/* then to the output type.  Rows go to cu_seq_lens[r] + i of            */
/* key_out / value_out [num_tokens, H, D] (row strides in elements).     */
/* Same page layout, HND / NHD, and skip rules as the store and gather.  */
/* ------------------------------------------------------------------ */
void oracle_gather_kv_fp4_dequant(const uint8_t *key_cache, const uint8_t *value_cache,
                                  uint16_t *key_out, int64_t key_row_stride,
                                  uint16_t *value_out, int64_t value_row_stride,
                                  int32_t out_dtype, const int32_t *block_table,
                                  const int32_t *cu_seq_lens, int32_t num_reqs,
                                  int32_t max_blocks_per_req, int64_t num_tokens,
                                  int32_t num_heads, int32_t head_size, int32_t block_size,
                                  int64_t num_blocks, int64_t page_stride, int32_t layout,
                                  float k_scale, float v_scale)
{
    const int64_t data_dim = head_size / 2;
    const int64_t S = head_size / 16;
    const int64_t data_per_side = (int64_t)num_heads * block_size * data_dim;
    int32_t r;
    for (r = 0; r < num_reqs; ++r) {
        int64_t start = cu_seq_lens[r];
        int64_t len = (int64_t)cu_seq_lens[r + 1] - start;
        int64_t i;
        for (i = 0; i < len; ++i) {
            int64_t row = start + i;
            int64_t j = i / block_size;
            int64_t off = i % block_size;
            int64_t page;
            int kv;
            if (row < 0 || row >= num_tokens)
                continue;
            if (j >= max_blocks_per_req)
                continue;
            page = block_table[(int64_t)r * max_blocks_per_req + j];
            if (page < 0 || page >= num_blocks)
                continue;
            for (kv = 0; kv < 2; ++kv) {
                const uint8_t *side = ((kv == 0) ? key_cache : value_cache) + page * page_stride;
                const uint8_t *scales = side + data_per_side;
                uint16_t *dst = (kv == 0) ? key_out + row * key_row_stride
                                          : value_out + row * value_row_stride;
                float ts = (kv == 0) ? k_scale : v_scale;
                int32_t h;
                int64_t g;
                for (h = 0; h < num_heads; ++h) {
                    for (g = 0; g < S; ++g) {
                        int64_t data_off, scale_off, srow, scol;
                        float sfd;
                        int k2;
                        if (layout == 0)
                            data_off = ((int64_t)h * block_size + off) * data_dim + g * 8;
                        else
                            data_off = (off * num_heads + h) * data_dim + g * 8;
                        if (kv == 0) {
                            srow = off;
                            scol = g;
                        } else {
                            int sw = oracle_swizzle_offset((int)off, (int)g, (int)S);
                            srow = sw / S;
                            scol = sw % S;
                        }
                        if (layout == 0)
                            scale_off = ((int64_t)h * block_size + srow) * S + scol;
                        else
                            scale_off = (srow * num_heads + h) * S + scol;
                        sfd = oracle_e4m3_decode(scales[scale_off]);
                        for (k2 = 0; k2 < 16; ++k2) {
                            uint8_t byte = side[data_off + k2 / 2];
                            uint8_t code = (k2 % 2) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 0xF);
                            float v = oracle_e2m1_decode(code) * sfd;
                            v = v * ts;
                            dst[(int64_t)h * head_size + g * 16 + k2] = narrow(v, out_dtype);
                        }
                    }
                }
            }
        }
    }
}

/* ================================================================== */
/* Indexer logits on the gathered keys (the op the integration PR hands */
/* k_fp8 and k_scale.view(float32) to, fp8_mqa_logits; its body is not  */
/* on the pages -- the reading is the lightning-indexer score).         */
/* ================================================================== */

/* For query token i and key j in [ks[i], ke[i]) (clipped to [0, num_k)  */
/* and to the row's first `row_cols` columns):                           */
/*   logits[i*row_stride + (j - ks[i])] =                                 */
/*       sum_h weights[i*H + h] * max(0, k_scale[j] * sum_d q[i,h,d]*k[j,d]) */
/* with q and k E4M3 codes decoded exactly.  Worked in binary64: every   */
/* product of two E4M3 values is exact, and a 128-term dot product of   */
/* them spans under 53 bits, so the dot product is exact; the rest is   */
/* binary64 arithmetic (relative error ~2^-50).  Entries outside the    */
/* ranges are left untouched.                                           */
void oracle_fp8_mqa_logits(const uint8_t *q, const uint8_t *k, const float *k_scale,
                           const float *weights, const int32_t *ks, const int32_t *ke,
                           double *logits, int64_t row_stride, int64_t row_cols,
                           int32_t num_q, int32_t num_heads, int64_t num_k,
                           int32_t head_dim)
{
    int32_t i;
    for (i = 0; i < num_q; ++i) {
        int64_t j, lo = ks[i], hi = ke[i];
        if (lo < 0) lo = 0;
        if (hi > num_k) hi = num_k;
        for (j = lo; j < hi; ++j) {
            double acc = 0.0;
            int32_t h;
            if (j - ks[i] >= row_cols)
                continue;
            for (h = 0; h < num_heads; ++h) {
                const uint8_t *qh = q + ((int64_t)i * num_heads + h) * head_dim;
                const uint8_t *kj = k + j * head_dim;
                double dot = 0.0, s;
                int32_t d;
                for (d = 0; d < head_dim; ++d)
                    dot += (double)oracle_e4m3_decode(qh[d]) * (double)oracle_e4m3_decode(kj[d]);
                s = (double)k_scale[j] * dot;
                if (s > 0.0)
                    acc += (double)weights[(int64_t)i * num_heads + h] * s;
            }
            logits[(int64_t)i * row_stride + (j - ks[i])] = acc;
        }
    }
}

/* ================================================================== */
/* [P4] paged decode attention over fp8 pages (vLLM PR "[ROCm] Faster   */
/* Custom Paged Attention kernels": the op schema paged_attention(out,  */
/* exp_sums, max_logits, tmp_out, query, key_cache, value_cache,        */
/* num_kv_heads, scale, block_tables, context_lens, block_size, ...,    */
/* kv_cache_dtype, k_scale, v_scale, ..., partition_size)).             */
/* ================================================================== */

/* One decode query per sequence.  For sequence s and head h (kv head     */
/* kvh = h / (num_heads / num_kv_heads)), token t < context_lens[s] lives */
/* in page block_tables[s][t / B] at offset t % B; its key and value are  */
/*   k_t[d] = E4M3dec(key_cache[page][kvh][d/16][t%B][d%16]) * k_scale     */
/*   v_t[d] = E4M3dec(value_cache[page][kvh][d][t%B]) * v_scale           */
/* and out[s][h] = sum_t softmax_t(scale * q.k_t) * v_t, in binary64.     */
/* Tokens whose page id is outside [0, num_blocks) or whose block-table   */
/* column is >= max_blocks are left out of the softmax; a sequence with   */
/* no token left gets a zero row.  q is bf16 (widened exactly).           */
void oracle_paged_attention_decode(double *out, const uint16_t *query,
                                   const uint8_t *key_cache, const uint8_t *value_cache,
                                   const int32_t *block_tables, const int32_t *context_lens,
                                   int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                   int32_t head_size, int32_t block_size, int32_t max_blocks,
                                   int64_t num_blocks, double scale, float k_scale, float v_scale)
{
    const int32_t group = num_heads / num_kv_heads;
    int32_t s, h;
    for (s = 0; s < num_seqs; ++s) {
        const int64_t L = context_lens[s];
        for (h = 0; h < num_heads; ++h) {
            const int32_t kvh = h / group;
            const uint16_t *q = query + ((int64_t)s * num_heads + h) * head_size;
            double *o = out + ((int64_t)s * num_heads + h) * head_size;
            double m = -INFINITY, denom = 0.0;
            int64_t t;
            int32_t d;
            for (d = 0; d < head_size; ++d)
                o[d] = 0.0;
            /* pass 1: the largest logit */
            for (t = 0; t < L; ++t) {
                int64_t j = t / block_size, page;
                double dot = 0.0, logit;
                if (j >= max_blocks) continue;
                page = block_tables[(int64_t)s * max_blocks + j];
                if (page < 0 || page >= num_blocks) continue;
                for (d = 0; d < head_size; ++d) {
                    const uint8_t c = key_cache[(((page * num_kv_heads + kvh) * (head_size / 16) +
                                                  d / 16) * block_size + t % block_size) * 16 +
                                                d % 16];
                    dot += (double)oracle_bf16_to_f32(q[d]) *
                           ((double)oracle_e4m3_decode(c) * (double)k_scale);
                }
                logit = scale * dot;
                if (logit > m) m = logit;
            }
            if (m == -INFINITY)
                continue;           /* no token: zero row */
            /* pass 2: weights and the weighted sum of values */
            for (t = 0; t < L; ++t) {
                int64_t j = t / block_size, page;
                double dot = 0.0, w;
                if (j >= max_blocks) continue;
                page = block_tables[(int64_t)s * max_blocks + j];
                if (page < 0 || page >= num_blocks) continue;
                for (d = 0; d < head_size; ++d) {
                    const uint8_t c = key_cache[(((page * num_kv_heads + kvh) * (head_size / 16) +
                                                  d / 16) * block_size + t % block_size) * 16 +
                                                d % 16];
                    dot += (double)oracle_bf16_to_f32(q[d]) *
                           ((double)oracle_e4m3_decode(c) * (double)k_scale);
                }
                w = exp(scale * dot - m);
                denom += w;
                for (d = 0; d < head_size; ++d) {
                    const uint8_t c = value_cache[((page * num_kv_heads + kvh) * head_size + d) *
                                                  block_size + t % block_size];
                    o[d] += w * ((double)oracle_e4m3_decode(c) * (double)v_scale);
                }
            }
            for (d = 0; d < head_size; ++d)
                o[d] /= denom;
        }
    }
}
