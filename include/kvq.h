/*
 * kvq.h -- C ABI of libkvq: decode-step attention read directly from a low-bit,
 * group-wise, asymmetrically quantized KV cache, for AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages; cited by title and section):
 *   [BitDecoding] "Tensor Core加速的低比特KV缓存解码系统" (cyqw.cn)
 *   [InnerQ]      "KV缓存量化技术InnerQ：提升大模型推理效率" (jsqmd.com)
 *   [3-bit blog]  "3-bit KV缓存量化：大模型推理功耗与带宽优化核心技术" (yfxerp.com)
 *
 * Conventions for every call:
 *   - All data pointers are DEVICE pointers, owned by the caller. The library never
 *     allocates, frees or synchronizes; work is enqueued on `stream` and the call
 *     returns at once. A NULL stream is the default stream.
 *   - Arguments are validated on the host before anything is launched; on error nothing
 *     is enqueued and a negative kvq_status is returned. A launch the runtime rejects
 *     returns KVQ_ERR_LAUNCH. No C++ exception crosses this interface.
 *   - The library keeps no mutable global state: calls are thread-safe and re-entrant.
 *     Calls on one stream run in order; the caller orders calls across streams.
 *   - Device pointers must be 64-byte aligned (KVQ_ERR_ALIGN otherwise). [BitDecoding]
 *     sec. 5.1 asks for aligned KV pointers; [InnerQ] sec. 3.2 aligns parameters to 64 B.
 *   - Non-finite fp16 inputs (inf, NaN) give undefined results.
 *
 * ---------------------------------------------------------------------------------
 * Packed cache format ([InnerQ] sec. 2.1 groups along head_dim, sec. 3.2 layout)
 * ---------------------------------------------------------------------------------
 * A "row" is the K (or the V) cache of one (batch, kv-head). A row is a sequence of
 * blocks of 128 tokens; block j of row r starts at base + r*row_stride + j*block_bytes.
 * Inside a block (d = head_dim, G = 32, ng = d/G groups per token, b = bits):
 *
 *   codes  [128 tokens][ng groups][4*b bytes]   at offset 0
 *          The 32 codes of a group form one little-endian (32*b)-bit word: code i sits
 *          at bits [b*i, b*i + b) (LSB first; 3-bit codes 10 and 21 straddle 32-bit
 *          words). At 4 bits a group is one 128-bit word ([InnerQ] sec. 3.2); at 3 bits
 *          it is three uint32; at 2 bits two uint32.
 *   sz     [128 tokens][ng groups]{fp16 scale, fp16 zero}   at offset align64(codes)
 *          4 bytes per group: scale in the low half, zero in the high half.
 *   flags  [128*ng bits], bit (token*ng + group), 1 = asymmetric, 0 = symmetric;
 *          present only when fmt.hybrid != 0, at offset align64(sz end).
 *   block_bytes = align64(end of the last region). At d = 128: 4-bit 10240 B,
 *   3-bit 8192 B, 2-bit 6144 B (hybrid +64 B).
 *
 * A value decodes as  x = zero + code * scale  ([InnerQ] sec. 3.1) in both modes.
 *
 * Quantizer, per group x[0..31] (fp16), N = 2^b - 1, every step one IEEE binary32
 * operation rounded to nearest even ([BitDecoding] sec. 2.1 scale and round;
 * [3-bit blog] sec. 2.3 clip):
 *   mn = min(x) + 0, mx = max(x) + 0            (-0.0 taken as +0.0)
 *   scale = fp16((mx - mn) / N), zero = fp16(mn)  (zero is exact)
 *   code_i = 0 if scale == 0, else min(N, round_half_away((x_i - zero) / scale))
 *   (the stored fp16 scale is the one used to compute the codes).
 * Hybrid ([InnerQ] sec. 2.2): a symmetric candidate with s = fp16(max|x| / (2^(b-1)-1)),
 *   code_i = 2^(b-1) + clamp(round_half_away(x_i / s), -(2^(b-1)-1), 2^(b-1)-1)
 *   (2^(b-1) when s == 0) and zero = -2^(b-1) * s (not eligible if that overflows fp16);
 *   its error e_i = x_i - fma(code_i, scale, zero) is summed as e_i^2 in binary32 in a
 *   balanced pairwise tree over channel order; the symmetric candidate is kept only
 *   when its sum is strictly below the asymmetric one's; the flag records the choice.
 *
 * ---------------------------------------------------------------------------------
 * Residual / sink window ([BitDecoding] sec. 2.2; [InnerQ] sec. 2.3)
 * ---------------------------------------------------------------------------------
 * fp16 K and V buffers [B][Hkv][res_capacity][head_dim], token-major. Slots
 * 0..n_res-1 are attended in full precision next to the packed tokens. Slot order does
 * not matter to the result (no mask). When the window is full, the caller quantizes it
 * into the next packed block with kvq_quantize_pack and starts again at slot 0.
 *
 * ---------------------------------------------------------------------------------
 * Split-K partials
 * ---------------------------------------------------------------------------------
 * The token sequence of a (batch, kv-head) is packed tokens 0..n_packed-1 then the
 * residual slots 0..n_res-1. Packed tokens form 32-token tiles (NT = n_packed/32).
 * With num_splits S > 1 and n_res > 0, split S-1 holds exactly the residual and splits
 * 0..S-2 share the tiles; otherwise all S splits share the tiles and split S-1 also takes
 * the residual. Of the Sp tile-sharing splits, split s gets tiles [s*NT/Sp, (s+1)*NT/Sp)
 * (integer division). A split with no token has lse = -inf and o = 0.
 *   part_o  [B][Hq][S][head_dim] fp32: sum_t p_t v_t / sum_t p_t over the split's tokens
 *   part_lse[B][Hq][S] fp32: m + ln(sum_t e^(l_t - m)), l_t = sm_scale * q . k_t
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KVQ_OK = 0,
    KVQ_ERR_NULL = -1,        /* a required pointer is NULL */
    KVQ_ERR_SHAPE = -2,       /* sizes or strides out of range or inconsistent */
    KVQ_ERR_UNSUPPORTED = -3, /* valid request that this build does not implement */
    KVQ_ERR_ALIGN = -4,       /* pointer or stride not aligned as required */
    KVQ_ERR_LAUNCH = -5,      /* the HIP runtime rejected a launch */
    KVQ_ERR_TOO_LARGE = -6    /* the sizes need more scratch than the allocation-free call has */
} kvq_status;

/* Bytes of device scratch behind kvq_decode_attention_fused_noalloc (one array per GPU). */
#define KVQ_NOALLOC_SCRATCH_BYTES (8 << 20)

typedef struct {
    int32_t bits;         /* 2, 3 or 4 */
    int32_t head_dim;     /* 128 (multiple of 32 in the format; kernels take 128) */
    int32_t group;        /* must be 32 */
    int32_t hybrid;       /* 0: asymmetric only; 1: per-group sym/asym choice + flag bit */
    int32_t block_tokens; /* must be 128: packed block = flush unit = residual capacity */
} kvq_format;

typedef enum { KVQ_OUT_F32 = 0, KVQ_OUT_F16 = 1 } kvq_out_dtype;

typedef enum { KVQ_SCALE_DIVIDE = 0, KVQ_SCALE_MULTIPLY = 1 } kvq_scale_mode;

/* Per-sequence state of a paged cache with a sliding window (see "Paged cache" below). */
typedef struct {
    int32_t n_packed;   /* tokens in the packed cache */
    int32_t n_res;      /* window slots in use, 0..res_capacity (slots 0..n_res-1) */
    int32_t next_slot;  /* once the window is full: the slot of its oldest recent token,
                           in [n_sink, res_capacity); start it at n_sink */
    int32_t reserved;   /* kept as it is */
} kvq_seq_state;

/* ---- size helpers (header-only) ---- */
static inline int64_t kvq_align64(int64_t v) { return (v + 63) / 64 * 64; }
static inline int64_t kvq_codes_bytes(const kvq_format *f)
{
    return (int64_t)f->block_tokens * f->head_dim * f->bits / 8;
}
static inline int64_t kvq_sz_offset(const kvq_format *f) { return kvq_align64(kvq_codes_bytes(f)); }
static inline int64_t kvq_sz_bytes(const kvq_format *f)
{
    return (int64_t)f->block_tokens * (f->head_dim / f->group) * 4;
}
static inline int64_t kvq_flag_offset(const kvq_format *f)
{
    return kvq_align64(kvq_sz_offset(f) + kvq_sz_bytes(f));
}
static inline int64_t kvq_flag_bytes(const kvq_format *f)
{
    return f->hybrid ? ((int64_t)f->block_tokens * (f->head_dim / f->group) + 7) / 8 : 0;
}
static inline int64_t kvq_block_bytes(const kvq_format *f)
{
    return kvq_align64(kvq_flag_offset(f) + kvq_flag_bytes(f));
}
/* A split count for decode on `cu_count` CUs. When the B*Hkv rows are few (at most half
   as many as CUs) and the sequence short enough that cu_count/rows splits leave each of
   them at most 128 packed 32-token tiles, one split per CU per row: the launch then has
   at most one workgroup per CU and takes the 8-wave kernel, which holds a whole CU's LDS
   (measured best at 32K and 128K tokens x 8 kv-heads, 32 splits). Otherwise enough
   splits that B*Hkv*S workgroups give three 4-wave workgroups per CU while each split
   keeps at least 64 tiles, else two per CU (shorter splits pay the per-workgroup start
   and merge too often; three measured best at 32K x 64 rows). With three per CU the
   packed splits alone fill the CUs and the window's own split comes on top: its
   workgroups are short and run as the first packed ones finish (32K x 64 rows: 13 splits,
   1.5-3% faster than 12). Never fewer than 8 tiles per split, never more than 256
   splits. */
static inline int32_t kvq_suggest_splits(int32_t B, int32_t Hkv, int32_t n_tokens,
                                         int32_t cu_count)
{
    int64_t rows = (int64_t)B * Hkv;
    int64_t tiles = n_tokens / 32;
    int64_t cap = tiles / 8;
    int64_t want;
    if (rows >= 1 && 2 * rows <= cu_count && tiles <= 128LL * (cu_count / rows)) {
        want = cu_count / rows;
    } else {
        want = (3LL * cu_count + rows - 1) / rows;
        if (tiles < 64 * want) want = (2LL * cu_count + rows - 1) / rows;
        else if (want >= 2) want += 1;
    }
    int64_t s = want < cap ? want : cap;
    if (s < 1) s = 1;
    if (s > 256) s = 256;
    return (int32_t)s;
}
/* A split count for kvq_decode_attention_paged over sequences of different lengths: the
   longest sequence sets the critical path, so its splits are made about as long as a
   quarter of one CU's share of all the packed tokens (measured best, 12-16 splits, on 16
   sequences of 1.5K-32K tokens), and no shorter than 8 tiles of 32 tokens.
     total_packed  sum of the sequences' packed tokens; max_packed  the largest of them */
static inline int32_t kvq_suggest_splits_paged(int64_t total_packed, int32_t max_packed,
                                               int32_t Hkv, int32_t cu_count)
{
    if (total_packed < 1 || max_packed < 1) return 1;
    int64_t s = (4LL * cu_count * max_packed + total_packed * Hkv - 1) / (total_packed * Hkv);
    const int64_t cap = (int64_t)max_packed / 32 / 8;
    if (s > cap) s = cap;
    if (s < 1) s = 1;
    if (s > 256) s = 256;
    return (int32_t)s;
}
static inline const char *kvq_status_string(kvq_status s)
{
    switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_NULL: return "null pointer";
    case KVQ_ERR_SHAPE: return "bad shape or stride";
    case KVQ_ERR_UNSUPPORTED: return "unsupported format or shape";
    case KVQ_ERR_ALIGN: return "misaligned pointer or stride";
    case KVQ_ERR_LAUNCH: return "kernel launch failed";
    case KVQ_ERR_TOO_LARGE: return "sizes exceed the fixed scratch of the allocation-free call";
    }
    return "unknown status";
}

/*
 * kvq_quantize_pack -- quantize fp16 tokens and write them as packed blocks.
 * [BitDecoding] sec. 2.1 (scale/zero/round), sec. 3.1 (register-only quantize with a
 * cross-lane min/max reduction); [InnerQ] sec. 2.1-2.2 (groups along head_dim, hybrid
 * mode and flag); [3-bit blog] sec. 2.3 (clip), sec. 3.2 (fp16 K/V -> packed + scale/zero).
 *
 *   src_fp16        fp16 [n_rows][..][head_dim]: token t of row r at
 *                   src + r*src_row_stride + t*src_tok_stride (elements); channels contiguous.
 *                   Strides must be multiples of 8 elements (16-byte token rows).
 *   n_rows          rows to quantize (e.g. B*Hkv for the K or the V cache), >= 1
 *   n_tokens        tokens per row, a positive multiple of 128
 *   dst_packed      packed rows; row r at dst + r*dst_row_stride_bytes
 *   dst_row_stride_bytes  >= (dst_first_block + n_tokens/128) * kvq_block_bytes(fmt),
 *                   multiple of 64
 *   dst_first_block first block written in every row (the flush of a full residual window
 *                   writes block n_packed/128)
 * Writes blocks [dst_first_block, dst_first_block + n_tokens/128) of every row, all bytes
 * of each block (codes, scale/zero, flags). Deterministic: equal inputs give equal bytes.
 */
kvq_status kvq_quantize_pack(const kvq_format *fmt, const void *src_fp16, int64_t n_rows,
                             int32_t n_tokens, int64_t src_row_stride, int64_t src_tok_stride,
                             void *dst_packed, int64_t dst_row_stride_bytes,
                             int32_t dst_first_block, hipStream_t stream);

/*
 * kvq_decode_attention -- split-K partials of one decode step.
 * [BitDecoding] sec. 2.2 (fp16 residual block next to the packed cache), sec. 2.3 (query
 * rows of one GQA group processed together; dequantize while computing); [InnerQ] sec. 3.1
 * (fused dequantize + dot product, scale/zero staged on chip), sec. 2.3 (sink/recent
 * windows at full precision).
 *
 *   q_fp16          [B][Hq][head_dim]; head h reads kv-head h / (Hq/Hkv)
 *   k_packed, v_packed   packed rows [B*Hkv], row b*Hkv + kvh at base + row*packed_row_stride_bytes
 *   n_packed_tokens multiple of 128, >= 0; the row stride must hold n_packed/128 blocks
 *   k_res_fp16, v_res_fp16  [B][Hkv][res_capacity][head_dim] (may be NULL when n_res == 0)
 *   n_res           0..res_capacity; n_packed + n_res must be > 0
 *   sm_scale        softmax scale (1/sqrt(head_dim) for standard attention)
 *   num_splits      S >= 1 (at most 1024); see "Split-K partials" above for the token split
 *   part_o, part_lse  fp32 outputs as described above
 * Supported: bits 2/3/4, head_dim 128, 1 <= Hq/Hkv <= 16.
 */
kvq_status kvq_decode_attention(const kvq_format *fmt, const void *q_fp16, int32_t B,
                                int32_t Hq, int32_t Hkv, const void *k_packed,
                                const void *v_packed, int64_t packed_row_stride_bytes,
                                int32_t n_packed_tokens, const void *k_res_fp16,
                                const void *v_res_fp16, int32_t res_capacity, int32_t n_res,
                                float sm_scale, int32_t num_splits, float *part_o,
                                float *part_lse, hipStream_t stream);

/*
 * kvq_decode_attention_append -- kvq_append_residual of one new token into window slot
 * n_res - 1 followed by kvq_decode_attention, in one launch ([InnerQ] sec. 2.3: the new
 * token enters the fp16 recent window; the decode then attends to it with the rest). The
 * workgroups that process the window read the new token from k_new / v_new, and one of them
 * per (batch, kv-head) stores it into the window, so the window afterwards and the partials
 * equal those of the two separate calls, bit for bit.
 *   k_new_fp16, v_new_fp16  fp16 [B][Hkv][head_dim], 64-byte aligned
 *   k_res_fp16, v_res_fp16  the windows, as for kvq_decode_attention; slot n_res - 1 of
 *                   every row is written by this call (the caller advances its own count
 *                   first: n_res here includes the new token)
 *   n_res           1..res_capacity (KVQ_ERR_SHAPE for 0)
 *   other arguments, validation and outputs: as kvq_decode_attention. A NULL window or new
 *   token is KVQ_ERR_NULL. When the window is full before the step, the caller flushes it
 *   first (kvq_quantize_pack of the 128 window tokens into the next block) and passes
 *   n_res = 1.
 */
kvq_status kvq_decode_attention_append(const kvq_format *fmt, const void *q_fp16, int32_t B,
                                       int32_t Hq, int32_t Hkv, const void *k_packed,
                                       const void *v_packed, int64_t packed_row_stride_bytes,
                                       int32_t n_packed_tokens, void *k_res_fp16,
                                       void *v_res_fp16, int32_t res_capacity, int32_t n_res,
                                       const void *k_new_fp16, const void *v_new_fp16,
                                       float sm_scale, int32_t num_splits, float *part_o,
                                       float *part_lse, hipStream_t stream);

/*
 * ---------------------------------------------------------------------------------
 * Outer-dimension grouping (the comparison the InnerQ page draws: [InnerQ] sec. 1, the
 * conventional KIVI-style grouping along the sequence; sec. 4.1, its timing)
 * ---------------------------------------------------------------------------------
 * A group is the 32 consecutive tokens 32*tg .. 32*tg+31 (tg = 0..3) of one channel of a
 * 128-token block, for K and for V; the quantizer is the asymmetric one above (hybrid is
 * not supported: KVQ_ERR_UNSUPPORTED). The block has the same size and regions as the
 * inner format: the codes sit at the same positions (token-major, 32-channel LSB-first
 * words), and the scale/zero region holds [4 token groups][head_dim channels]
 * {fp16 scale, fp16 zero}. A value decodes as zero(tg, c) + code * scale(tg, c).
 */

/*
 * kvq_quantize_pack_outer -- kvq_quantize_pack with outer-dimension groups. Arguments,
 * validation and errors as kvq_quantize_pack; fmt->hybrid must be 0.
 */
kvq_status kvq_quantize_pack_outer(const kvq_format *fmt, const void *src_fp16, int64_t n_rows,
                                   int32_t n_tokens, int64_t src_row_stride,
                                   int64_t src_tok_stride, void *dst_packed,
                                   int64_t dst_row_stride_bytes, int32_t dst_first_block,
                                   hipStream_t stream);

/*
 * kvq_decode_attention_outer -- kvq_decode_attention over outer-grouped blocks (same
 * arguments, split rule, outputs and limits; fmt->hybrid must be 0). The per-channel
 * scales sit inside the Q K^T contraction and along the P V output channels, so each
 * 32-token tile takes q * scale_k as its MFMA operand and adds scale_v * (P V) + zero_v *
 * sum(p) per channel; this is the cost of the outer grouping the comparison measures.
 */
kvq_status kvq_decode_attention_outer(const kvq_format *fmt, const void *q_fp16, int32_t B,
                                      int32_t Hq, int32_t Hkv, const void *k_packed,
                                      const void *v_packed, int64_t packed_row_stride_bytes,
                                      int32_t n_packed_tokens, const void *k_res_fp16,
                                      const void *v_res_fp16, int32_t res_capacity,
                                      int32_t n_res, float sm_scale, int32_t num_splits,
                                      float *part_o, float *part_lse, hipStream_t stream);

/*
 * kvq_decode_attention_knorm -- kvq_decode_attention for a cache whose keys were
 * key-channel normalized ([InnerQ] sec. 2.4, see kvq_key_norm): every query channel is first
 * multiplied by the norm of its kv-head's row, q'[c] = fp16(q[c] * key_norm[b*Hkv + kvh][c])
 * (binary32 product, round to nearest even), inside the decode kernel as it stages q. The
 * partials are bit for bit those of kvq_channel_scale(q, KVQ_SCALE_MULTIPLY) followed by
 * kvq_decode_attention on q', with no extra launch or q' buffer (the page folds the norm
 * into the query projection for no run-time cost; this is the same for a caller that keeps
 * its projection as is).
 *   key_norm        fp32 [B*Hkv][128], 64-byte aligned (KVQ_ERR_NULL / KVQ_ERR_ALIGN)
 *   other arguments, validation and outputs: as kvq_decode_attention.
 */
kvq_status kvq_decode_attention_knorm(const kvq_format *fmt, const void *q_fp16,
                                      const float *key_norm, int32_t B, int32_t Hq,
                                      int32_t Hkv, const void *k_packed, const void *v_packed,
                                      int64_t packed_row_stride_bytes, int32_t n_packed_tokens,
                                      const void *k_res_fp16, const void *v_res_fp16,
                                      int32_t res_capacity, int32_t n_res, float sm_scale,
                                      int32_t num_splits, float *part_o, float *part_lse,
                                      hipStream_t stream);

/*
 * kvq_decode_attention_valu -- the same partials as kvq_decode_attention (same arguments,
 * validation, errors and output layout; equal within floating-point rounding), computed
 * with VALU dot products only (v_dot2_f32_f16, one query head per wave, no matrix cores).
 * It is the measured comparison for the matrix-core design of kvq_decode_attention, whose
 * use of MFMA for Q K^T and P V at GQA groups of 4 and more is justified by being faster.
 */
kvq_status kvq_decode_attention_valu(const kvq_format *fmt, const void *q_fp16, int32_t B,
                                     int32_t Hq, int32_t Hkv, const void *k_packed,
                                     const void *v_packed, int64_t packed_row_stride_bytes,
                                     int32_t n_packed_tokens, const void *k_res_fp16,
                                     const void *v_res_fp16, int32_t res_capacity,
                                     int32_t n_res, float sm_scale, int32_t num_splits,
                                     float *part_o, float *part_lse, hipStream_t stream);

/*
 * kvq_decode_attention_fp16 -- the split-K partials of one decode step over an
 * uncompressed fp16 K/V cache: the FP16 flash-decoding baseline that the low-bit cache is
 * compared against ([BitDecoding] sec. 4.1-4.2 report speed-ups over FP16 decoding).
 *   q_fp16          [B][Hq][128]; head h reads kv-head h / (Hq/Hkv)
 *   k_fp16, v_fp16  [B*Hkv][row_stride_tokens][128] fp16, token-major; tokens 0..n_tokens-1
 *                   of every row are attended
 *   row_stride_tokens  >= n_tokens, even (rows stay 64-byte aligned)
 *   num_splits      S in 1..1024: with NT = ceil(n_tokens/32) tiles of 32 tokens, split s
 *                   takes tiles [s*NT/S, (s+1)*NT/S); a split with no token has lse = -inf
 *   part_o, part_lse  as for kvq_decode_attention; merge them with kvq_combine
 * Supported: head_dim 128, 1 <= Hq/Hkv <= 16, n_tokens * 256 B < 2^31.
 */
kvq_status kvq_decode_attention_fp16(const void *q_fp16, int32_t B, int32_t Hq, int32_t Hkv,
                                     const void *k_fp16, const void *v_fp16,
                                     int64_t row_stride_tokens, int32_t n_tokens,
                                     float sm_scale, int32_t num_splits, float *part_o,
                                     float *part_lse, hipStream_t stream);

/*
 * kvq_combine -- merge the split partials into the attention output (the log-sum-exp
 * merge of split-K flash-decoding, the FP16 baseline named in [BitDecoding] sec. 4.2):
 *   M = max_s lse_s, w_s = e^(lse_s - M), out = sum_s w_s o_s / sum_s w_s.
 * Splits with lse = -inf weigh 0; a (b, h) whose splits are all empty gets 0.
 *   out             [B][Hq][head_dim], fp32 (KVQ_OUT_F32) or fp16 rounded to nearest even
 *                   from the fp32 result (KVQ_OUT_F16)
 */
kvq_status kvq_combine(const float *part_o, const float *part_lse, int32_t B, int32_t Hq,
                       int32_t head_dim, int32_t num_splits, void *out, int32_t out_dtype,
                       hipStream_t stream);

/*
 * kvq_decode_attention_fused -- one whole decode step in one launch: the split-K partials
 * of kvq_decode_attention (optionally with kvq_decode_attention_knorm's query scaling and
 * kvq_decode_attention_append's new token) merged into the output inside the same launch,
 * by the log-sum-exp rule of kvq_combine ([BitDecoding] sec. 2.2-2.3 for the decode,
 * sec. 4.2 for the split-K merge). The splits of each (batch, kv-head, chunk of up to 4
 * query heads) merge in a tree of fan-in 32 (one level up to 32 splits): every split
 * stores its partial in the workspace and counts itself in its parent's counter, and the
 * last of a parent's children merges them; no workgroup waits for another.
 *   key_norm        NULL, or fp32 [B*Hkv][128] key-channel factors (as kvq_decode_attention_knorm)
 *   k_new_fp16, v_new_fp16  NULL (both), or the new token [B][Hkv][head_dim] that becomes
 *                   window slot n_res - 1, as in kvq_decode_attention_append (the windows are
 *                   then written and n_res >= 1)
 *   workspace       device memory of at least kvq_decode_workspace_bytes(B, Hq, Hkv,
 *                   num_splits) bytes, 256-byte aligned; may be NULL when that size is 0
 *                   (num_splits == 1). It must be zeroed before its first use; every call
 *                   leaves its counters at zero again (each is reset by the workgroup that
 *                   completes it; the records need no clearing), so one zeroed workspace
 *                   serves any sequence of calls of any shape that fits. Calls that share a
 *                   workspace and may overlap (other streams) race; give them separate
 *                   workspaces. A launch that does not complete (a device fault) leaves it
 *                   undefined: zero it again.
 *   out             [B][Hq][head_dim], fp32 (KVQ_OUT_F32) or fp16 (KVQ_OUT_F16: the
 *                   round-to-nearest-even of the fp32 value the kernel computed)
 *   other arguments, the split rule, validation and limits: as kvq_decode_attention.
 *   KVQ_ERR_SHAPE if workspace_bytes is too small; a (b, h) that attends no token gets 0.
 * The result equals kvq_decode_attention + kvq_combine up to floating-point rounding (the
 * merge order differs).
 */
kvq_status kvq_decode_attention_fused(const kvq_format *fmt, const void *q_fp16,
                                      const float *key_norm, int32_t B, int32_t Hq, int32_t Hkv,
                                      const void *k_packed, const void *v_packed,
                                      int64_t packed_row_stride_bytes, int32_t n_packed_tokens,
                                      void *k_res_fp16, void *v_res_fp16, int32_t res_capacity,
                                      int32_t n_res, const void *k_new_fp16,
                                      const void *v_new_fp16, float sm_scale, int32_t num_splits,
                                      void *workspace, int64_t workspace_bytes, void *out,
                                      int32_t out_dtype, hipStream_t stream);

/*
 * kvq_decode_attention_fused_noalloc -- kvq_decode_attention_fused without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation). The split records live in a
 * device array of KVQ_NOALLOC_SCRATCH_BYTES bytes that the library holds on each GPU it
 * runs on until the process ends; the call allocates nothing (no hipMalloc, no allocating
 * library routine). The first call on a device (the current device) looks the array up and
 * enqueues one kernel that zeroes it; every call leaves its counters at zero again.
 *   Arguments, outputs, validation and limits: as kvq_decode_attention_fused without
 *   workspace / workspace_bytes; KVQ_ERR_TOO_LARGE when kvq_decode_workspace_bytes(B, Hq,
 *   Hkv, num_splits) exceeds KVQ_NOALLOC_SCRATCH_BYTES (e.g. 8 rows of 4 query heads take
 *   1.1 MB at 64 splits; 1024 splits need 17.6 MB and are rejected).
 *   Every call on one GPU shares that GPU's array: calls that may overlap on one GPU (other
 *   streams, other threads) race and give undefined results; serialize them, or use
 *   kvq_decode_attention_fused with separate workspaces.
 */
kvq_status kvq_decode_attention_fused_noalloc(const kvq_format *fmt, const void *q_fp16,
                                              const float *key_norm, int32_t B, int32_t Hq,
                                              int32_t Hkv, const void *k_packed,
                                              const void *v_packed,
                                              int64_t packed_row_stride_bytes,
                                              int32_t n_packed_tokens, void *k_res_fp16,
                                              void *v_res_fp16, int32_t res_capacity,
                                              int32_t n_res, const void *k_new_fp16,
                                              const void *v_new_fp16, float sm_scale,
                                              int32_t num_splits, void *out, int32_t out_dtype,
                                              hipStream_t stream);

/*
 * kvq_decode_workspace_bytes -- bytes of workspace kvq_decode_attention_fused and
 * kvq_decode_attention_paged_fused need for these sizes (0 when num_splits == 1; -1 for
 * sizes those calls reject): per chunk of up to 4 query heads of every (batch, kv-head),
 * one 2080-byte slot per node below the root of the fan-in-32 split tree (the node's
 * partial: 4 x 128 fp32 outputs and 4 log-sum-exps; its padding word holds the counter of
 * the parent whose first child it is). Every call lays its slots out from the start of the
 * workspace on the same 2080-byte grid, which is why one zeroed workspace serves calls of
 * any shape.
 */
int64_t kvq_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t num_splits);

/*
 * kvq_append_residual -- write one new fp16 token per (batch, kv-head) into residual slot
 * `slot` of the K and V windows ([InnerQ] sec. 2.3: new tokens always enter the recent
 * window).
 *   k_new, v_new    fp16 [B][Hkv][head_dim]
 *   k_res, v_res    fp16 [B][Hkv][res_capacity][head_dim]
 *   0 <= slot < res_capacity
 */
kvq_status kvq_append_residual(const void *k_new, const void *v_new, void *k_res, void *v_res,
                               int32_t B, int32_t Hkv, int32_t head_dim, int32_t res_capacity,
                               int32_t slot, hipStream_t stream);

/*
 * kvq_key_norm -- key-channel normalization factors ([InnerQ] sec. 2.4): for every row r
 * (one (batch, kv-head) of the K cache) and channel c,
 *     norm[r][c] = sqrt(max_t |K_r[t][c]|)   over tokens t = 0..n_tokens-1 (the prefill keys),
 * 1 where that maximum is 0. The maximum is exact (fp16 magnitudes); the square root is the
 * correctly rounded binary32 one. Keys divided by these factors and queries multiplied by
 * them (kvq_channel_scale, kvq_decode_attention_knorm) leave q . k unchanged up to fp16
 * rounding while the range of outlier channels shrinks to its square root.
 *   k_fp16          token t of row r at k + r*row_stride + t*tok_stride (elements), channels
 *                   contiguous; strides multiples of 8 elements; may be NULL if n_tokens == 0
 *   n_rows >= 1, n_tokens >= 0 (0: every factor is 1), head_dim must be 128
 *   norm            fp32 [n_rows][128], written (also used as the reduction's workspace, so
 *                   it must not alias k)
 * Enqueues three small kernels; results are deterministic (a maximum does not depend on the
 * order of its operands). Non-finite keys give undefined factors.
 */
kvq_status kvq_key_norm(const void *k_fp16, int64_t n_rows, int32_t n_tokens,
                        int64_t row_stride, int64_t tok_stride, int32_t head_dim, float *norm,
                        hipStream_t stream);

/*
 * kvq_channel_scale -- apply key-channel normalization factors ([InnerQ] sec. 2.4) to fp16
 * vectors: for rows r, tokens t and channels c,
 *     y[r][t][c] = fp16(x[r][t][c] / norm[r / rows_per_norm][c])   (KVQ_SCALE_DIVIDE: keys)
 *     y[r][t][c] = fp16(x[r][t][c] * norm[r / rows_per_norm][c])   (KVQ_SCALE_MULTIPLY: queries)
 * one binary32 operation (division correctly rounded) then round to nearest even.
 *   x_fp16, y_fp16  token t of row r at base + r*row_stride + t*tok_stride (elements, per
 *                   buffer); strides multiples of 8 elements. y may be x itself with the
 *                   same strides (in place); any other overlap is undefined. Writing y into
 *                   a residual window slot scales a new key on its way into the window.
 *   n_rows >= 1, n_tokens >= 0 (0: nothing is enqueued), head_dim must be 128
 *   norm            fp32 [n_rows / rows_per_norm rounded up][128] (kvq_key_norm's output)
 *   rows_per_norm   >= 1: query rows [B][Hq] use rows_per_norm = Hq/Hkv so that head h of
 *                   batch b takes the factors of kv-head h / (Hq/Hkv); key rows use 1
 */
kvq_status kvq_channel_scale(const void *x_fp16, int64_t n_rows, int32_t n_tokens,
                             int64_t x_row_stride, int64_t x_tok_stride, int32_t head_dim,
                             const float *norm, int64_t rows_per_norm, int32_t mode,
                             void *y_fp16, int64_t y_row_stride, int64_t y_tok_stride,
                             hipStream_t stream);

/*
 * ---------------------------------------------------------------------------------
 * Paged cache, ragged lengths, per-token sliding window ([InnerQ] sec. 2.3: new tokens
 * always enter the recent window, the oldest recent token is quantized into the main
 * cache when the window is full, the sink window is fixed after prefill; [3-bit blog]
 * sec. 6.1: the packed cache is kept in pages of a byte pool)
 * ---------------------------------------------------------------------------------
 * Packed blocks (the format above) live in a K pool and a V pool of pool_blocks blocks
 * per kv-head. Packed token j of sequence b, kv-head h is token j % 128 of the block
 *     pool + block_table[b][j / 128] * block_stride + h * head_stride      (bytes)
 * block_table is int32 [B][max_blocks]. The strides are multiples of 64 and lay the pool
 * out as [pool_blocks][Hkv][block_bytes] (head_stride >= block_bytes, block_stride >=
 * Hkv * head_stride) or as [Hkv][pool_blocks][block_bytes] (block_stride >= block_bytes,
 * head_stride >= pool_blocks * block_stride); KVQ_ERR_SHAPE otherwise.
 * Each sequence has its own lengths, in a kvq_seq_state [B] array in device memory, and
 * an fp16 window [B][Hkv][res_capacity][128] whose slots 0..n_sink-1 hold the sinks.
 * Table entries, lengths and counts live on the device and are not checked on the host:
 * a table entry outside [0, pool_blocks) or a position past the table makes the kernels
 * skip that write (or read block 0 instead), and lengths are clamped to the table and the
 * window, so bad device data gives wrong results but never an access outside the buffers.
 */

/*
 * kvq_pack_tokens_paged -- quantize and pack tokens t = 0..count[b]-1 of every (b, h) row
 * of src into packed positions start[b] + t of sequence b (prefill, or any bulk move into
 * the paged cache); one token at a time, so a block may be filled in several calls. The
 * bytes of each token equal those kvq_quantize_pack gives it; nothing else is written.
 *   src_fp16        token t of row b*Hkv + h at src + (b*Hkv + h)*src_row_stride +
 *                   t*src_tok_stride (elements, multiples of 8)
 *   count, start    int32 [B] in device memory; max_count >= every count[b] (host bound
 *                   for the grid; counts above it are cut to it)
 *   pool            the K or the V pool
 */
kvq_status kvq_pack_tokens_paged(const kvq_format *fmt, const void *src_fp16, int32_t B,
                                 int32_t Hkv, int64_t src_row_stride, int64_t src_tok_stride,
                                 const int32_t *count, const int32_t *start, int32_t max_count,
                                 void *pool, int64_t pool_blocks, int64_t block_stride_bytes,
                                 int64_t head_stride_bytes, const int32_t *block_table,
                                 int32_t max_blocks, hipStream_t stream);

/*
 * kvq_append_evict -- one decode step's cache update for every sequence b: if
 * n_res < res_capacity the new token takes slot n_res (n_res += 1); otherwise the token in
 * slot next_slot (the oldest recent one) is quantized into packed position n_packed
 * (n_packed += 1), the new token takes that slot, and next_slot moves to the next slot,
 * wrapping from res_capacity - 1 to n_sink. The state is updated on the device, so steps
 * can be enqueued (or captured in a graph) without reading it back.
 *   k_new, v_new    fp16 [B][Hkv][128]
 *   k_res, v_res    fp16 [B][Hkv][res_capacity][128]
 *   0 <= n_sink < res_capacity (the same on every call for a sequence)
 * Calls on one stream apply in order; the decode of a step must follow its update.
 */
kvq_status kvq_append_evict(const kvq_format *fmt, const void *k_new, const void *v_new,
                            void *k_res, void *v_res, int32_t res_capacity, int32_t n_sink,
                            void *k_pool, void *v_pool, int64_t pool_blocks,
                            int64_t block_stride_bytes, int64_t head_stride_bytes,
                            const int32_t *block_table, int32_t max_blocks, kvq_seq_state *state,
                            int32_t B, int32_t Hkv, hipStream_t stream);

/*
 * kvq_decode_attention_paged -- the split-K partials of kvq_decode_attention for a paged
 * cache: sequence b attends its own state[b].n_packed packed tokens (through the table;
 * any number, not only multiples of 128) and its window slots 0..state[b].n_res-1.
 * Split rule per sequence: NT = ceil(n_packed / 32) tiles (the last possibly partial);
 * with num_splits S > 1 and n_res > 0 split S-1 holds the window and splits 0..S-2 share
 * the tiles, otherwise all S share them and split S-1 also takes the window; split s of
 * the Sp sharing splits gets tiles [s*NT/Sp, (s+1)*NT/Sp). Empty splits have lse = -inf
 * and o = 0; kvq_combine gives 0 for a sequence that attends no token.
 *   key_norm        NULL, or the fp32 [B*Hkv][128] key-channel factors of a cache whose keys
 *                   were normalized: q is then multiplied by them as in
 *                   kvq_decode_attention_knorm (64-byte aligned)
 *   Other arguments, outputs and limits: as kvq_decode_attention.
 */
kvq_status kvq_decode_attention_paged(const kvq_format *fmt, const void *q_fp16, int32_t B,
                                      int32_t Hq, int32_t Hkv, const void *k_pool,
                                      const void *v_pool, int64_t pool_blocks,
                                      int64_t block_stride_bytes, int64_t head_stride_bytes,
                                      const int32_t *block_table, int32_t max_blocks,
                                      const kvq_seq_state *state, const void *k_res_fp16,
                                      const void *v_res_fp16, int32_t res_capacity,
                                      const float *key_norm, float sm_scale, int32_t num_splits,
                                      float *part_o, float *part_lse, hipStream_t stream);

/*
 * kvq_decode_attention_paged_append -- one serving step of the paged cache in one call:
 * kvq_append_evict (the new token enters the window; when the window is full the token in
 * slot next_slot is quantized into packed position n_packed and the new token takes its
 * slot; [InnerQ] sec. 2.3) followed by kvq_decode_attention_paged over the updated cache,
 * with the same windows, pool bytes, state and partials as those two calls, bit for bit.
 * The update is applied inside the decode launch: `state` is only read, the updated state
 * is written to `state_out` (the caller alternates the two buffers from step to step).
 * With more than four query heads per kv-head the two calls run as two launches
 * internally (same results).
 *   state, state_out  [B] states, 64-byte aligned, not overlapping
 *   n_sink, k_new, v_new   as kvq_append_evict; k_res_fp16 / v_res_fp16 and the pools are
 *                   written (the new token and the evicted token)
 *   Other arguments, outputs and limits: as kvq_decode_attention_paged.
 */
kvq_status kvq_decode_attention_paged_append(
    const kvq_format *fmt, const void *q_fp16, int32_t B, int32_t Hq, int32_t Hkv, void *k_pool,
    void *v_pool, int64_t pool_blocks, int64_t block_stride_bytes, int64_t head_stride_bytes,
    const int32_t *block_table, int32_t max_blocks, const kvq_seq_state *state,
    kvq_seq_state *state_out, void *k_res_fp16, void *v_res_fp16, int32_t res_capacity,
    int32_t n_sink, const void *k_new, const void *v_new, const float *key_norm, float sm_scale,
    int32_t num_splits, float *part_o, float *part_lse, hipStream_t stream);

/*
 * kvq_decode_attention_paged_fused -- kvq_decode_attention_paged with the split merge in
 * the same launch, as kvq_decode_attention_fused: the output [B][Hq][head_dim] (out_dtype
 * as kvq_combine), the workspace as for kvq_decode_attention_fused. A sequence that attends
 * no token gets 0. Other arguments, validation and limits: as kvq_decode_attention_paged.
 */
kvq_status kvq_decode_attention_paged_fused(const kvq_format *fmt, const void *q_fp16, int32_t B,
                                            int32_t Hq, int32_t Hkv, const void *k_pool,
                                            const void *v_pool, int64_t pool_blocks,
                                            int64_t block_stride_bytes,
                                            int64_t head_stride_bytes, const int32_t *block_table,
                                            int32_t max_blocks, const kvq_seq_state *state,
                                            const void *k_res_fp16, const void *v_res_fp16,
                                            int32_t res_capacity, const float *key_norm,
                                            float sm_scale, int32_t num_splits, void *workspace,
                                            int64_t workspace_bytes, void *out, int32_t out_dtype,
                                            hipStream_t stream);

/*
 * kvq_stream_read -- a measurement reference, not part of the method: read n (1..4) device
 * buffers once, as one streaming pass with plain 16-byte non-temporal loads (every 64 KB
 * piece of a buffer one workgroup of 256 threads, all of a thread's loads in flight at
 * once), and nothing else. Timed over the bytes a decode step reads, it gives the read
 * bandwidth the same memory system delivers to a kernel with no other work.
 *   bufs, bytes     host arrays of n device pointers (16-byte aligned) and byte counts
 *                   (multiples of 16, at least 16 each; at most 2^31 - 1 pieces in all)
 *   sink            device memory of at least 256 bytes; written only in the practically
 *                   impossible case that a workgroup's folded data equals a fixed constant
 */
kvq_status kvq_stream_read(const void *const *bufs, const int64_t *bytes, int32_t n, void *sink,
                           hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
