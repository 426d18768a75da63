/*
 * kvq_oracle.c -- CPU oracle for the low-bit packed KV cache and decode attention.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark load this library. The product path (the HIP library) never
 * includes, links or calls anything here, and nothing here includes the product's
 * headers: the packed format is restated below from the pages' description.
 *
 * What it computes (plain, slow, in the pages' order):
 *   1. the group-wise asymmetric quantizer of the BitDecoding page ("Tensor Core加速的
 *      低比特KV缓存解码系统", sec. 2.1: scale = (max-min)/(2^b-1), q = round((x-min)/scale)),
 *      with the clip to [0, 2^b-1] of the 3-bit blog page ("3-bit KV缓存量化：大模型推理
 *      功耗与带宽优化核心技术", sec. 2.3) and groups of 32 along head_dim as on the InnerQ
 *      page ("KV缓存量化技术InnerQ：提升大模型推理效率", sec. 2.1);
 *   2. the InnerQ hybrid choice between a symmetric and an asymmetric candidate per group,
 *      kept in a 1-bit flag (InnerQ page, sec. 2.2; flag 0 = symmetric, 1 = asymmetric);
 *   3. LSB-first packing of the codes (InnerQ page, sec. 3.2: the 32 values of a group
 *      form one contiguous word; 3-bit blog page, sec. 3.2: code i sits at bit 3*i);
 *   4. decode attention out = softmax(sm * q K^T) V over the dequantized packed tokens
 *      (InnerQ page, sec. 3.1: x = scale * code + zero) plus the fp16 residual / sink
 *      tokens kept at full precision (BitDecoding page, sec. 2.2; InnerQ page, sec. 2.3),
 *      in fp64, with the GQA head mapping of the BitDecoding page, sec. 2.3;
 *   5. the split-K form of the same attention (per-split max / sum / normalised output)
 *      and the log-sum-exp merge of the splits, in fp64;
 *   6. key-channel normalization before quantization (InnerQ page, sec. 2.4): per-channel
 *      norm = sqrt(max |K|) over the prefill keys, keys divided by it, queries multiplied;
 *   7. the paged cache with ragged lengths and the per-token sliding window (InnerQ page,
 *      sec. 2.3; 3-bit blog page, sec. 6.1);
 *   8. the outer-dimension (KIVI-style) grouping the InnerQ page compares against (sec. 1,
 *      sec. 4.1): groups of 32 tokens per channel.
 *
 * Floating point: every quantizer step is one IEEE binary32 operation with round to
 * nearest even (build with -O2 -ffp-contract=off, never -ffast-math). Attention is fp64.
 *
 * Readings where the pages are silent or ambiguous (each is listed in the design notes):
 *   - round() is round-half-away-from-zero, done exactly (for t >= 0 it equals the
 *     3-bit blog's floor(t + 0.5) without the rounding of t + 0.5);
 *   - the scale is rounded to fp16 first, and the codes are computed with that stored
 *     fp16 scale, so that encoding and decoding use the same number;
 *   - zero = min, stored as fp16 (exact); a -0.0 minimum or maximum is taken as +0.0, so
 *     neither the zero nor the scale is ever -0.0;
 *   - a group whose fp16 scale is 0 (constant group, or a range that underflows fp16)
 *     gets all-zero codes; it is reconstructed as zero exactly (no epsilon);
 *   - the symmetric candidate uses the signed grid -(2^(b-1)-1) .. +(2^(b-1)-1) times
 *     s = fp16(max|x| / (2^(b-1)-1)), stored as offset-binary codes u = 2^(b-1) + k with
 *     zero field -2^(b-1) * s, so both modes decode as zero + code * scale;
 *   - the hybrid criterion is the lower sum of squared errors (fp32, fixed pairwise
 *     order over the 32 channels); a tie keeps the asymmetric candidate.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OQ_GROUP 32          /* values per quantization group (InnerQ page, sec. 2.1) */
#define OQ_BLOCK 128         /* tokens per packed block = residual window capacity */
#define OQ_ALIGN 64          /* region alignment inside a block (InnerQ page, sec. 3.2) */

/* ------------------------------------------------------------------------------------ */
/* IEEE 754 binary16 <-> binary32, written from the encoding.                            */
/* ------------------------------------------------------------------------------------ */

float oq_f16_to_f32(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int e = (h >> 10) & 0x1f;
    const int m = h & 0x3ff;
    float mag;
    if (e == 0)
        mag = ldexpf((float)m, -24);                 /* subnormal: m * 2^-24 */
    else if (e == 31)
        mag = m ? NAN : INFINITY;
    else
        mag = ldexpf((float)(m | 0x400), e - 25);    /* 1.m * 2^(e-15) = (1024+m) * 2^(e-25) */
    return sign ? -mag : mag;
}

/* Nearest binary16 value to f, ties to even. */
uint16_t oq_f32_to_f16(float f)
{
    if (isnan(f))
        return 0x7e00;
    const uint16_t sign = signbit(f) ? 0x8000 : 0;
    const double a = fabs((double)f);
    if (a >= 65520.0)                                /* max finite 65504 + half an ulp (16) */
        return sign | 0x7c00;
    if (a < ldexp(1.0, -14)) {                       /* subnormal range: quantum 2^-24 */
        const double n = rint(a / ldexp(1.0, -24));  /* exact division; rint = ties-to-even */
        return sign | (uint16_t)n;                   /* n == 1024 encodes the smallest normal */
    }
    int ex;
    frexp(a, &ex);                                   /* a = fr * 2^ex, fr in [0.5, 1) */
    int E = ex - 1;                                  /* a in [2^E, 2^(E+1)) */
    double n = rint(a / ldexp(1.0, E - 10));         /* significand in units of the quantum */
    if (n == 2048.0) {                               /* rounded up into the next binade */
        n = 1024.0;
        E += 1;
    }
    if (E + 15 >= 31)
        return sign | 0x7c00;
    return sign | (uint16_t)(((E + 15) << 10) | ((int)n - 1024));
}

/* ------------------------------------------------------------------------------------ */
/* Group quantizer.                                                                      */
/* ------------------------------------------------------------------------------------ */

/* Round half away from zero, exactly: the fraction t - trunc(t) is exact in binary32. */
static int round_half_away(float t)
{
    const float k = truncf(fabsf(t));
    const float r = (fabsf(t) - k >= 0.5f) ? k + 1.0f : k;
    return (int)(t < 0.0f ? -r : r);
}

/*
 * Asymmetric candidate (BitDecoding page sec. 2.1; clip from the 3-bit blog sec. 2.3):
 * scale = fp16((max - min) / (2^b - 1)), zero = fp16(min), code = min(N, round((x - zero) / scale)).
 */
void oq_asym_candidate(const uint16_t *x, int bits, uint16_t *scale_out, uint16_t *zero_out,
                       uint8_t *codes)
{
    const int N = (1 << bits) - 1;
    float mn = oq_f16_to_f32(x[0]), mx = mn;
    for (int i = 1; i < OQ_GROUP; i++) {
        const float v = oq_f16_to_f32(x[i]);
        if (v < mn) mn = v;
        if (v > mx) mx = v;
    }
    mn = mn + 0.0f;                                  /* -0.0 -> +0.0 */
    mx = mx + 0.0f;                                  /* so an all -0.0 group gets scale +0.0 */
    const float scale_f = (mx - mn) / (float)N;
    const uint16_t sh = oq_f32_to_f16(scale_f);
    const uint16_t zh = oq_f32_to_f16(mn);           /* exact: mn is an fp16 value */
    const float s = oq_f16_to_f32(sh), z = oq_f16_to_f32(zh);
    for (int i = 0; i < OQ_GROUP; i++) {
        if (s == 0.0f) {
            codes[i] = 0;
            continue;
        }
        const float t = (oq_f16_to_f32(x[i]) - z) / s;   /* t >= 0 */
        int c = round_half_away(t);
        if (c > N) c = N;
        if (c < 0) c = 0;
        codes[i] = (uint8_t)c;
    }
    *scale_out = sh;
    *zero_out = zh;
}

/*
 * Symmetric candidate (the InnerQ page, sec. 2.2, names it without a formula; reading:
 * signed grid k * s, |k| <= 2^(b-1)-1, s = fp16(max|x| / (2^(b-1)-1)), offset-binary code
 * u = 2^(b-1) + k, zero field -2^(b-1) * s). Returns 0 when the zero field would not fit
 * in fp16 (then the candidate cannot be stored and is not eligible).
 */
int oq_sym_candidate(const uint16_t *x, int bits, uint16_t *scale_out, uint16_t *zero_out,
                     uint8_t *codes)
{
    const int Qs = (1 << (bits - 1)) - 1;
    const int off = 1 << (bits - 1);
    float m = 0.0f;
    for (int i = 0; i < OQ_GROUP; i++) {
        const float a = fabsf(oq_f16_to_f32(x[i]));
        if (a > m) m = a;
    }
    const uint16_t sh = oq_f32_to_f16(m / (float)Qs);
    const float s = oq_f16_to_f32(sh);
    const float zf = -((float)off * s) + 0.0f;       /* exact (power-of-two multiple); -0 -> +0 */
    const int eligible = fabsf(zf) <= 65504.0f;
    for (int i = 0; i < OQ_GROUP; i++) {
        int k = 0;
        if (s != 0.0f) {
            k = round_half_away(oq_f16_to_f32(x[i]) / s);
            if (k > Qs) k = Qs;
            if (k < -Qs) k = -Qs;
        }
        codes[i] = (uint8_t)(off + k);
    }
    *scale_out = sh;
    *zero_out = eligible ? oq_f32_to_f16(zf) : 0x7c00;
    return eligible;
}

/*
 * Sum of squared reconstruction errors of one candidate, in binary32:
 * e_i = x_i - fma(code_i, scale, zero), summed as a balanced binary tree in channel order
 * ((e0^2 + e1^2) + (e2^2 + e3^2)) + ... so that the value does not depend on the machine.
 */
float oq_group_sse(const uint16_t *x, const uint8_t *codes, uint16_t scale, uint16_t zero)
{
    const float s = oq_f16_to_f32(scale), z = oq_f16_to_f32(zero);
    float v[OQ_GROUP];
    for (int i = 0; i < OQ_GROUP; i++) {
        const float e = oq_f16_to_f32(x[i]) - fmaf((float)codes[i], s, z);
        v[i] = e * e;
    }
    for (int w = 1; w < OQ_GROUP; w *= 2)
        for (int i = 0; i < OQ_GROUP; i += 2 * w)
            v[i] = v[i] + v[i + w];
    return v[0];
}

/*
 * One group: the asymmetric quantizer, or (hybrid) the InnerQ choice of the candidate
 * with the lower squared error, sym only when strictly lower. flag: 1 = asym, 0 = sym.
 */
void oq_quantize_group(const uint16_t *x, int bits, int hybrid, uint16_t *scale_out,
                       uint16_t *zero_out, uint8_t *codes, int *flag_out)
{
    uint16_t sa, za;
    uint8_t ca[OQ_GROUP];
    oq_asym_candidate(x, bits, &sa, &za, ca);
    int flag = 1;
    if (hybrid) {
        uint16_t ss, zs;
        uint8_t cs[OQ_GROUP];
        const int ok = oq_sym_candidate(x, bits, &ss, &zs, cs);
        if (ok && oq_group_sse(x, cs, ss, zs) < oq_group_sse(x, ca, sa, za)) {
            flag = 0;
            sa = ss;
            za = zs;
            memcpy(ca, cs, sizeof ca);
        }
    }
    memcpy(codes, ca, OQ_GROUP);
    *scale_out = sa;
    *zero_out = za;
    *flag_out = flag;
}

/* ------------------------------------------------------------------------------------ */
/* Bit packing: code i of a group occupies bits [b*i, b*i + b) of the group's            */
/* little-endian 32*b-bit word (16 bytes at 4 bits, 12 at 3 bits, 8 at 2 bits).           */
/* ------------------------------------------------------------------------------------ */

void oq_pack_codes(const uint8_t *codes, int bits, uint8_t *out)
{
    memset(out, 0, (size_t)(OQ_GROUP * bits / 8));
    for (int i = 0; i < OQ_GROUP; i++)
        for (int j = 0; j < bits; j++)
            if ((codes[i] >> j) & 1) {
                const int pos = bits * i + j;
                out[pos / 8] |= (uint8_t)(1u << (pos % 8));
            }
}

void oq_unpack_codes(const uint8_t *in, int bits, uint8_t *codes)
{
    for (int i = 0; i < OQ_GROUP; i++) {
        int c = 0;
        for (int j = 0; j < bits; j++) {
            const int pos = bits * i + j;
            c |= ((in[pos / 8] >> (pos % 8)) & 1) << j;
        }
        codes[i] = (uint8_t)c;
    }
}

/* ------------------------------------------------------------------------------------ */
/* Block layout of one row (the K or the V of one (batch, kv-head)):                     */
/*   codes [128 tokens][head_dim/32 groups][4*b bytes]                                   */
/*   sz    [128 tokens][head_dim/32 groups]{fp16 scale, fp16 zero}   (64-B aligned)       */
/*   flags [128*head_dim/32 bits], bit (token*groups + group), 1 = asym (hybrid only)     */
/* Blocks follow each other; a row of the cache is a sequence of blocks.                  */
/* ------------------------------------------------------------------------------------ */

static int64_t align64(int64_t v) { return (v + OQ_ALIGN - 1) / OQ_ALIGN * OQ_ALIGN; }

int64_t oq_codes_bytes(int bits, int head_dim) { return (int64_t)OQ_BLOCK * head_dim * bits / 8; }
int64_t oq_sz_bytes(int head_dim) { return (int64_t)OQ_BLOCK * (head_dim / OQ_GROUP) * 4; }
int64_t oq_flag_bytes(int head_dim, int hybrid)
{
    return hybrid ? ((int64_t)OQ_BLOCK * (head_dim / OQ_GROUP) + 7) / 8 : 0;
}
int64_t oq_sz_offset(int bits, int head_dim) { return align64(oq_codes_bytes(bits, head_dim)); }
int64_t oq_flag_offset(int bits, int head_dim)
{
    return align64(oq_sz_offset(bits, head_dim) + oq_sz_bytes(head_dim));
}
int64_t oq_block_bytes(int bits, int head_dim, int hybrid)
{
    return align64(oq_flag_offset(bits, head_dim) + oq_flag_bytes(head_dim, hybrid));
}

static void put_u16(uint8_t *p, uint16_t v)
{
    p[0] = (uint8_t)(v & 0xff);
    p[1] = (uint8_t)(v >> 8);
}
static uint16_t get_u16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* Quantize and pack token t of one row into its slot of block `blk`. */
static void quantize_token(const uint16_t *src_tok, int bits, int head_dim, int hybrid,
                           uint8_t *blk, int t_in_block)
{
    const int ng = head_dim / OQ_GROUP;
    const int64_t gbytes = OQ_GROUP * bits / 8;
    for (int g = 0; g < ng; g++) {
        uint16_t s, z;
        uint8_t codes[OQ_GROUP];
        int flag;
        oq_quantize_group(src_tok + g * OQ_GROUP, bits, hybrid, &s, &z, codes, &flag);
        oq_pack_codes(codes, bits, blk + (int64_t)t_in_block * ng * gbytes + g * gbytes);
        uint8_t *sz = blk + oq_sz_offset(bits, head_dim) + ((int64_t)t_in_block * ng + g) * 4;
        put_u16(sz, s);
        put_u16(sz + 2, z);
        if (hybrid) {
            const int bit = t_in_block * ng + g;
            uint8_t *fl = blk + oq_flag_offset(bits, head_dim) + bit / 8;
            if (flag)
                *fl |= (uint8_t)(1u << (bit % 8));
            else
                *fl &= (uint8_t)~(1u << (bit % 8));
        }
    }
}

/* Worker-thread plumbing: a plain loop over [0, n) split into contiguous chunks. */
typedef void (*oq_body)(void *ctx, int64_t i);
typedef struct {
    oq_body fn;
    void *ctx;
    int64_t lo, hi;
} oq_chunk;

static void *oq_chunk_run(void *arg)
{
    oq_chunk *c = (oq_chunk *)arg;
    for (int64_t i = c->lo; i < c->hi; i++)
        c->fn(c->ctx, i);
    return NULL;
}

static void oq_parallel_for(int64_t n, int n_threads, oq_body fn, void *ctx)
{
    if (n_threads < 1) n_threads = 1;
    if (n_threads > 256) n_threads = 256;
    if (n_threads > n) n_threads = (int)(n > 0 ? n : 1);
    pthread_t th[256];
    oq_chunk ch[256];
    for (int k = 0; k < n_threads; k++) {
        ch[k].fn = fn;
        ch[k].ctx = ctx;
        ch[k].lo = n * k / n_threads;
        ch[k].hi = n * (k + 1) / n_threads;
    }
    for (int k = 1; k < n_threads; k++)
        pthread_create(&th[k], NULL, oq_chunk_run, &ch[k]);
    oq_chunk_run(&ch[0]);
    for (int k = 1; k < n_threads; k++)
        pthread_join(th[k], NULL);
}

typedef struct {
    const uint16_t *src;
    int bits, head_dim, hybrid, n_tokens;
    int64_t src_row_stride, src_tok_stride;
    uint8_t *dst;
    int64_t dst_row_stride;
    int first_block;
} qp_ctx;

static void qp_row(void *vctx, int64_t r)
{
    const qp_ctx *c = (const qp_ctx *)vctx;
    const int64_t bb = oq_block_bytes(c->bits, c->head_dim, c->hybrid);
    for (int t = 0; t < c->n_tokens; t++) {
        uint8_t *blk = c->dst + r * c->dst_row_stride + (int64_t)(c->first_block + t / OQ_BLOCK) * bb;
        quantize_token(c->src + r * c->src_row_stride + (int64_t)t * c->src_tok_stride, c->bits,
                       c->head_dim, c->hybrid, blk, t % OQ_BLOCK);
    }
}

/*
 * Quantize n_tokens (a multiple of 128) tokens of each of n_rows rows of fp16 data
 * (channels contiguous; strides in elements) into blocks first_block, first_block+1, ...
 * of each destination row (row stride in bytes). Padding bytes between regions are zeroed.
 */
int oq_quantize_pack(int bits, int head_dim, int hybrid, const uint16_t *src, int64_t n_rows,
                     int n_tokens, int64_t src_row_stride, int64_t src_tok_stride, uint8_t *dst,
                     int64_t dst_row_stride, int first_block, int n_threads)
{
    if (bits < 2 || bits > 4 || head_dim % OQ_GROUP || n_tokens % OQ_BLOCK)
        return -1;
    const int64_t bb = oq_block_bytes(bits, head_dim, hybrid);
    for (int64_t r = 0; r < n_rows; r++)
        memset(dst + r * dst_row_stride + (int64_t)first_block * bb, 0,
               (size_t)(bb * (n_tokens / OQ_BLOCK)));
    qp_ctx c = {src, bits, head_dim, hybrid, n_tokens, src_row_stride, src_tok_stride,
                dst, dst_row_stride, first_block};
    oq_parallel_for(n_rows, n_threads, qp_row, &c);
    return 0;
}

/* Dequantize token t of one packed row into fp64: x = zero + code * scale (InnerQ sec. 3.1). */
static void dequant_token(const uint8_t *row, int bits, int head_dim, int hybrid, int64_t t,
                          double *out)
{
    const int ng = head_dim / OQ_GROUP;
    const int64_t gbytes = OQ_GROUP * bits / 8;
    const uint8_t *blk = row + (t / OQ_BLOCK) * oq_block_bytes(bits, head_dim, hybrid);
    const int tb = (int)(t % OQ_BLOCK);
    for (int g = 0; g < ng; g++) {
        uint8_t codes[OQ_GROUP];
        oq_unpack_codes(blk + (int64_t)tb * ng * gbytes + g * gbytes, bits, codes);
        const uint8_t *sz = blk + oq_sz_offset(bits, head_dim) + ((int64_t)tb * ng + g) * 4;
        const double s = (double)oq_f16_to_f32(get_u16(sz));
        const double z = (double)oq_f16_to_f32(get_u16(sz + 2));
        for (int i = 0; i < OQ_GROUP; i++)
            out[g * OQ_GROUP + i] = z + (double)codes[i] * s;
    }
}

/* Dequantize tokens [0, n_tokens) of n_rows packed rows into out[row][token][head_dim]. */
void oq_dequant(int bits, int head_dim, int hybrid, const uint8_t *packed, int64_t n_rows,
                int64_t n_tokens, int64_t row_stride, double *out)
{
    for (int64_t r = 0; r < n_rows; r++)
        for (int64_t t = 0; t < n_tokens; t++)
            dequant_token(packed + r * row_stride, bits, head_dim, hybrid, t,
                          out + (r * n_tokens + t) * head_dim);
}

/* ------------------------------------------------------------------------------------ */
/* Decode attention in fp64.                                                              */
/* The token sequence of a (batch, kv-head) is: packed tokens 0..n_packed-1, then the     */
/* residual slots 0..n_res-1 (fp16, used as they are). No mask: every token is attended.  */
/* ------------------------------------------------------------------------------------ */

typedef struct {
    int bits, head_dim, hybrid;
    const uint16_t *q;
    int B, Hq, Hkv;
    const uint8_t *kp, *vp;
    int64_t row_stride;
    int n_packed;
    const uint16_t *kres, *vres;
    int res_cap, n_res;
    double sm;
    int S;                 /* number of splits (1 = plain attention) */
    double *out;           /* [B][Hq][d] when S == 0; part_o [B][Hq][S][d] otherwise */
    double *lse;           /* part_lse [B][Hq][S] */
    int outer;             /* 1: blocks hold outer-dimension groups (see below) */
} att_ctx;

static void dequant_token_outer(const uint8_t *row, int bits, int head_dim, int64_t t, double *out);

/* Token j of the sequence of (b, kvh): its key (which = 0) or value (which = 1) in fp64. */
static void load_token(const att_ctx *c, int b, int kvh, int64_t j, int which, double *x)
{
    const int64_t row = (int64_t)b * c->Hkv + kvh;
    if (j < c->n_packed) {
        const uint8_t *base = which ? c->vp : c->kp;
        if (c->outer)
            dequant_token_outer(base + row * c->row_stride, c->bits, c->head_dim, j, x);
        else
            dequant_token(base + row * c->row_stride, c->bits, c->head_dim, c->hybrid, j, x);
    } else {
        const int64_t slot = j - c->n_packed;
        const uint16_t *r = (which ? c->vres : c->kres) + (row * c->res_cap + slot) * c->head_dim;
        for (int d = 0; d < c->head_dim; d++)
            x[d] = (double)oq_f16_to_f32(r[d]);
    }
}

/*
 * Softmax attention of head (b, h) over tokens [lo, hi) of its sequence:
 * writes o = sum_j e^(l_j - m) v_j / sum_j e^(l_j - m) and returns lse = m + ln(sum).
 * An empty range gives o = 0 and lse = -inf.
 */
static double attend_range(const att_ctx *c, int b, int h, int64_t lo, int64_t hi, double *o)
{
    const int d = c->head_dim;
    const int kvh = h / (c->Hq / c->Hkv);
    for (int i = 0; i < d; i++) o[i] = 0.0;
    if (hi <= lo) return -INFINITY;
    const uint16_t *qh = c->q + ((int64_t)b * c->Hq + h) * d;
    double *qd = malloc(sizeof(double) * d);
    double *k = malloc(sizeof(double) * d), *v = malloc(sizeof(double) * d);
    double *logit = malloc(sizeof(double) * (size_t)(hi - lo));
    for (int i = 0; i < d; i++) qd[i] = (double)oq_f16_to_f32(qh[i]);
    double m = -INFINITY;
    for (int64_t j = lo; j < hi; j++) {
        load_token(c, b, kvh, j, 0, k);
        double dot = 0.0;
        for (int i = 0; i < d; i++) dot += qd[i] * k[i];
        logit[j - lo] = c->sm * dot;
        if (logit[j - lo] > m) m = logit[j - lo];
    }
    double l = 0.0;
    for (int64_t j = lo; j < hi; j++) {
        load_token(c, b, kvh, j, 1, v);
        const double p = exp(logit[j - lo] - m);
        l += p;
        for (int i = 0; i < d; i++) o[i] += p * v[i];
    }
    for (int i = 0; i < d; i++) o[i] /= l;
    free(qd);
    free(k);
    free(v);
    free(logit);
    return m + log(l);
}

static void att_head(void *vctx, int64_t bh)
{
    const att_ctx *c = (const att_ctx *)vctx;
    const int b = (int)(bh / c->Hq), h = (int)(bh % c->Hq);
    const int64_t total = (int64_t)c->n_packed + c->n_res;
    attend_range(c, b, h, 0, total, c->out + bh * c->head_dim);
}

/*
 * Split of the token sequence used by the split-K partials (restated from the interface
 * contract): packed tokens form 32-token tiles, NT = n_packed / 32. With S > 1 and a
 * non-empty residual, split S-1 holds the whole residual and splits 0..S-2 share the
 * tiles; otherwise all S splits share the tiles and split S-1 also takes the residual.
 * Split s of the Sp tile-sharing splits gets tiles [s*NT/Sp, (s+1)*NT/Sp).
 */
static void split_range(int n_packed, int n_res, int S, int s, int64_t *lo, int64_t *hi,
                        int *with_res)
{
    const int64_t NT = n_packed / 32;
    const int res_alone = (S > 1 && n_res > 0);
    const int Sp = res_alone ? S - 1 : S;
    *with_res = 0;
    if (res_alone && s == S - 1) {
        *lo = n_packed;
        *hi = (int64_t)n_packed + n_res;
        return;
    }
    *lo = 32 * (s * NT / Sp);
    *hi = 32 * ((s + 1) * NT / Sp);
    if (!res_alone && s == S - 1) {
        *hi = (int64_t)n_packed + n_res;       /* last split runs on into the residual */
        *with_res = 1;
    }
}

static void att_head_split(void *vctx, int64_t bh)
{
    const att_ctx *c = (const att_ctx *)vctx;
    const int b = (int)(bh / c->Hq), h = (int)(bh % c->Hq);
    for (int s = 0; s < c->S; s++) {
        int64_t lo, hi;
        int wr;
        split_range(c->n_packed, c->n_res, c->S, s, &lo, &hi, &wr);
        c->lse[bh * c->S + s] =
            attend_range(c, b, h, lo, hi, c->out + (bh * c->S + s) * c->head_dim);
    }
}

/* out[B][Hq][d] = softmax(sm * q K^T) V over packed + residual tokens, fp64. */
void oq_attention(int bits, int head_dim, int hybrid, const uint16_t *q, int B, int Hq, int Hkv,
                  const uint8_t *kp, const uint8_t *vp, int64_t row_stride, int n_packed,
                  const uint16_t *kres, const uint16_t *vres, int res_cap, int n_res, double sm,
                  double *out, int n_threads)
{
    att_ctx c = {bits, head_dim, hybrid, q, B, Hq, Hkv, kp, vp, row_stride, n_packed,
                 kres, vres, res_cap, n_res, sm, 0, out, NULL, 0};
    oq_parallel_for((int64_t)B * Hq, n_threads, att_head, &c);
}

/* Per-split partials: part_o[B][Hq][S][d] (normalised), part_lse[B][Hq][S] (natural log). */
void oq_split_attention(int bits, int head_dim, int hybrid, const uint16_t *q, int B, int Hq,
                        int Hkv, const uint8_t *kp, const uint8_t *vp, int64_t row_stride,
                        int n_packed, const uint16_t *kres, const uint16_t *vres, int res_cap,
                        int n_res, double sm, int S, double *part_o, double *part_lse,
                        int n_threads)
{
    att_ctx c = {bits, head_dim, hybrid, q, B, Hq, Hkv, kp, vp, row_stride, n_packed,
                 kres, vres, res_cap, n_res, sm, S, part_o, part_lse, 0};
    oq_parallel_for((int64_t)B * Hq, n_threads, att_head_split, &c);
}

/*
 * Merge of split partials (the split-K flash-decoding combine): with M = max_s lse_s and
 * w_s = e^(lse_s - M), out = sum_s w_s o_s / sum_s w_s. Splits with lse = -inf weigh 0.
 */
void oq_combine(const double *part_o, const double *part_lse, int B, int Hq, int head_dim, int S,
                double *out)
{
    for (int64_t bh = 0; bh < (int64_t)B * Hq; bh++) {
        double M = -INFINITY;
        for (int s = 0; s < S; s++)
            if (part_lse[bh * S + s] > M) M = part_lse[bh * S + s];
        double wsum = 0.0;
        double *o = out + bh * head_dim;
        for (int i = 0; i < head_dim; i++) o[i] = 0.0;
        for (int s = 0; s < S; s++) {
            const double ls = part_lse[bh * S + s];
            if (ls == -INFINITY) continue;
            const double w = exp(ls - M);
            wsum += w;
            for (int i = 0; i < head_dim; i++) o[i] += w * part_o[(bh * S + s) * head_dim + i];
        }
        for (int i = 0; i < head_dim; i++) o[i] /= wsum;
    }
}

/* Exposed for the split-range check in the tests. */
void oq_split_range(int n_packed, int n_res, int S, int s, int64_t *lo, int64_t *hi)
{
    int wr;
    split_range(n_packed, n_res, S, s, lo, hi, &wr);
}

/* ------------------------------------------------------------------------------------ */
/* Key-channel normalization (InnerQ page, sec. 2.4): once, over the prefill keys, each  */
/* channel i of a (batch, kv-head) gets norm_i = sqrt(max_t |K[t][i]|); keys are divided */
/* by it and queries multiplied by it, which leaves every q . k, hence the softmax,      */
/* unchanged while squeezing the spread between outlier and ordinary channels.           */
/* Readings: the maximum runs over the tokens given (the prefill), per (row, channel);   */
/* norm is the binary32 square root of that maximum, and 1 for an all-zero channel; the  */
/* scaled value is the binary32 quotient (keys) or product (queries), rounded to fp16.   */
/* ------------------------------------------------------------------------------------ */

void oq_key_norm(const uint16_t *src, int64_t n_rows, int64_t n_tokens, int64_t row_stride,
                 int64_t tok_stride, int head_dim, float *norm_out)
{
    for (int64_t r = 0; r < n_rows; ++r) {
        for (int c = 0; c < head_dim; ++c) {
            float mx = 0.0f;
            for (int64_t t = 0; t < n_tokens; ++t) {
                const float v = fabsf(oq_f16_to_f32(src[r * row_stride + t * tok_stride + c]));
                if (v > mx) mx = v;
            }
            norm_out[r * head_dim + c] = mx > 0.0f ? sqrtf(mx) : 1.0f;
        }
    }
}

/* dst[r][t][c] = fp16(src[r][t][c] / norm[r / rows_per_norm][c])  (multiply == 0, keys)
 *              = fp16(src[r][t][c] * norm[r / rows_per_norm][c])  (multiply != 0, queries) */
void oq_channel_scale(const uint16_t *src, int64_t n_rows, int64_t n_tokens, int64_t row_stride,
                      int64_t tok_stride, int head_dim, const float *norm, int64_t rows_per_norm,
                      int multiply, uint16_t *dst, int64_t dst_row_stride, int64_t dst_tok_stride)
{
    for (int64_t r = 0; r < n_rows; ++r) {
        const float *nr = norm + (r / rows_per_norm) * head_dim;
        for (int64_t t = 0; t < n_tokens; ++t) {
            for (int c = 0; c < head_dim; ++c) {
                const float x = oq_f16_to_f32(src[r * row_stride + t * tok_stride + c]);
                const float y = multiply ? x * nr[c] : x / nr[c];
                dst[r * dst_row_stride + t * dst_tok_stride + c] = oq_f32_to_f16(y);
            }
        }
    }
}

/* ------------------------------------------------------------------------------------ */
/* Paged cache with ragged lengths and a per-token sliding window.                       */
/* InnerQ page sec. 2.3: a new token always enters the recent window; once the window is */
/* full, its oldest token is quantized into the main (packed) cache; the sink window is  */
/* filled at prefill and never changes. 3-bit blog page sec. 6.1: the packed cache is    */
/* kept in pages of a uint8 pool reached through a per-sequence table.                   */
/* Readings: packed token j of sequence b, kv-head h lives in pool block tbl[b][j / 128] */
/* at pool + blk * block_stride + h * head_stride, token j % 128 of that block. Each     */
/* sequence has a state {n_packed, n_res, next_slot, unused}: window slots             */
/* [0, n_res) hold its fp16 tokens, slots [0, n_sink) are the sinks, and next_slot in    */
/* [n_sink, res_cap) is the oldest recent token (the slots after the sinks are used as a */
/* ring once the window is full). Lengths differ per sequence.                           */
/* ------------------------------------------------------------------------------------ */

static uint8_t *paged_block(uint8_t *pool, int64_t block_stride, int64_t head_stride,
                            const int32_t *tbl, int max_blocks, int b, int h, int64_t j)
{
    const int64_t blk = tbl[(int64_t)b * max_blocks + j / OQ_BLOCK];
    return pool + blk * block_stride + (int64_t)h * head_stride;
}

/* Quantize tokens t in [0, count[b]) of every (b, h) row of src into packed positions
 * start[b] + t of sequence b (one token at a time, as the window eviction does). */
void oq_pack_tokens_paged(int bits, int head_dim, int hybrid, const uint16_t *src, int B,
                          int Hkv, int64_t src_row_stride, int64_t src_tok_stride,
                          const int32_t *count, const int32_t *start, uint8_t *pool,
                          int64_t block_stride, int64_t head_stride, const int32_t *tbl,
                          int max_blocks)
{
    for (int b = 0; b < B; b++)
        for (int h = 0; h < Hkv; h++)
            for (int64_t t = 0; t < count[b]; t++) {
                const int64_t j = (int64_t)start[b] + t;
                quantize_token(src + ((int64_t)b * Hkv + h) * src_row_stride + t * src_tok_stride,
                               bits, head_dim, hybrid,
                               paged_block(pool, block_stride, head_stride, tbl, max_blocks, b,
                                           h, j),
                               (int)(j % OQ_BLOCK));
            }
}

/* One decode-step update of every sequence's cache: if the window has a free slot the new
 * token takes slot n_res; otherwise the oldest recent token (slot next_slot) is quantized
 * into packed position n_packed, and the new token takes its slot. */
void oq_append_evict(int bits, int head_dim, int hybrid, const uint16_t *k_new,
                     const uint16_t *v_new, uint16_t *k_res, uint16_t *v_res, int res_cap,
                     int n_sink, uint8_t *k_pool, uint8_t *v_pool, int64_t block_stride,
                     int64_t head_stride, const int32_t *tbl, int max_blocks, int32_t *state,
                     int B, int Hkv)
{
    const int d = head_dim;
    for (int b = 0; b < B; b++) {
        int32_t *st = state + 4 * (int64_t)b;
        int slot;
        if (st[1] < res_cap) {
            slot = st[1];
            st[1] += 1;
        } else {
            slot = st[2];
            for (int h = 0; h < Hkv; h++) {
                const int64_t w = (((int64_t)b * Hkv + h) * res_cap + slot) * d;
                quantize_token(k_res + w, bits, d, hybrid,
                               paged_block(k_pool, block_stride, head_stride, tbl, max_blocks,
                                           b, h, st[0]),
                               st[0] % OQ_BLOCK);
                quantize_token(v_res + w, bits, d, hybrid,
                               paged_block(v_pool, block_stride, head_stride, tbl, max_blocks,
                                           b, h, st[0]),
                               st[0] % OQ_BLOCK);
            }
            st[0] += 1;
            st[2] = slot + 1 < res_cap ? slot + 1 : n_sink;
        }
        for (int h = 0; h < Hkv; h++) {
            const int64_t w = (((int64_t)b * Hkv + h) * res_cap + slot) * d;
            memcpy(k_res + w, k_new + ((int64_t)b * Hkv + h) * d, sizeof(uint16_t) * d);
            memcpy(v_res + w, v_new + ((int64_t)b * Hkv + h) * d, sizeof(uint16_t) * d);
        }
    }
}

typedef struct {
    int bits, head_dim, hybrid;
    const uint16_t *q;
    int B, Hq, Hkv;
    const uint8_t *kpool, *vpool;
    int64_t block_stride, head_stride;
    const int32_t *tbl;
    int max_blocks;
    const int32_t *state;
    const uint16_t *kres, *vres;
    int res_cap;
    double sm;
    int S;
    double *out, *lse;
} patt_ctx;

/* Token j of sequence b's order (packed 0..n_packed-1, then window slots 0..n_res-1). */
static void paged_load_token(const patt_ctx *c, int b, int kvh, int64_t j, int which, double *x)
{
    const int64_t n_packed = c->state[4 * (int64_t)b];
    if (j < n_packed) {
        const uint8_t *blk = paged_block((uint8_t *)(which ? c->vpool : c->kpool),
                                         c->block_stride, c->head_stride, c->tbl, c->max_blocks,
                                         b, kvh, j);
        dequant_token(blk, c->bits, c->head_dim, c->hybrid, j % OQ_BLOCK, x);
    } else {
        const int64_t slot = j - n_packed;
        const uint16_t *r = (which ? c->vres : c->kres) +
                            (((int64_t)b * c->Hkv + kvh) * c->res_cap + slot) * c->head_dim;
        for (int i = 0; i < c->head_dim; i++)
            x[i] = (double)oq_f16_to_f32(r[i]);
    }
}

/* The fp64 softmax attention of head (b, h) over tokens [lo, hi) of its sequence. */
static double paged_attend_range(const patt_ctx *c, int b, int h, int64_t lo, int64_t hi,
                                 double *o)
{
    const int d = c->head_dim;
    const int kvh = h / (c->Hq / c->Hkv);
    for (int i = 0; i < d; i++) o[i] = 0.0;
    if (hi <= lo) return -INFINITY;
    const uint16_t *qh = c->q + ((int64_t)b * c->Hq + h) * d;
    double *qd = malloc(sizeof(double) * d);
    double *k = malloc(sizeof(double) * d), *v = malloc(sizeof(double) * d);
    double *logit = malloc(sizeof(double) * (size_t)(hi - lo));
    for (int i = 0; i < d; i++) qd[i] = (double)oq_f16_to_f32(qh[i]);
    double m = -INFINITY;
    for (int64_t j = lo; j < hi; j++) {
        paged_load_token(c, b, kvh, j, 0, k);
        double dot = 0.0;
        for (int i = 0; i < d; i++) dot += qd[i] * k[i];
        logit[j - lo] = c->sm * dot;
        if (logit[j - lo] > m) m = logit[j - lo];
    }
    double l = 0.0;
    for (int64_t j = lo; j < hi; j++) {
        paged_load_token(c, b, kvh, j, 1, v);
        const double p = exp(logit[j - lo] - m);
        l += p;
        for (int i = 0; i < d; i++) o[i] += p * v[i];
    }
    for (int i = 0; i < d; i++) o[i] /= l;
    free(qd);
    free(k);
    free(v);
    free(logit);
    return m + log(l);
}

/*
 * Split of a ragged sequence (restated from the interface contract): its packed tokens
 * form NT = ceil(n_packed / 32) tiles, the last one possibly partial. With S > 1 and a
 * non-empty window, split S-1 holds the window and splits 0..S-2 share the tiles;
 * otherwise all S splits share the tiles and split S-1 also takes the window. Split s of
 * the Sp sharing splits gets tiles [s*NT/Sp, (s+1)*NT/Sp), cut at n_packed.
 */
static void paged_split_range(int64_t n_packed, int64_t n_res, int S, int s, int64_t *lo,
                              int64_t *hi)
{
    const int64_t NT = (n_packed + 31) / 32;
    const int res_alone = (S > 1 && n_res > 0);
    const int64_t Sp = res_alone ? S - 1 : S;
    if (res_alone && s == S - 1) {
        *lo = n_packed;
        *hi = n_packed + n_res;
        return;
    }
    *lo = 32 * (s * NT / Sp);
    *hi = 32 * ((s + 1) * NT / Sp);
    if (*lo > n_packed) *lo = n_packed;
    if (*hi > n_packed) *hi = n_packed;
    if (!res_alone && s == S - 1) *hi = n_packed + n_res;
}

static void patt_head(void *vctx, int64_t bh)
{
    const patt_ctx *c = (const patt_ctx *)vctx;
    const int b = (int)(bh / c->Hq), h = (int)(bh % c->Hq);
    const int64_t n = (int64_t)c->state[4 * (int64_t)b] + c->state[4 * (int64_t)b + 1];
    paged_attend_range(c, b, h, 0, n, c->out + bh * c->head_dim);
}

static void patt_head_split(void *vctx, int64_t bh)
{
    const patt_ctx *c = (const patt_ctx *)vctx;
    const int b = (int)(bh / c->Hq), h = (int)(bh % c->Hq);
    for (int s = 0; s < c->S; s++) {
        int64_t lo, hi;
        paged_split_range(c->state[4 * (int64_t)b], c->state[4 * (int64_t)b + 1], c->S, s, &lo,
                          &hi);
        c->lse[bh * c->S + s] =
            paged_attend_range(c, b, h, lo, hi, c->out + (bh * c->S + s) * c->head_dim);
    }
}

/* out[B][Hq][d] over each sequence's own tokens (S == 0), or the split partials (S >= 1:
 * part_o[B][Hq][S][d] into out, part_lse[B][Hq][S] into lse), fp64. */
void oq_attention_paged(int bits, int head_dim, int hybrid, const uint16_t *q, int B, int Hq,
                        int Hkv, const uint8_t *k_pool, const uint8_t *v_pool,
                        int64_t block_stride, int64_t head_stride, const int32_t *tbl,
                        int max_blocks, const int32_t *state, const uint16_t *kres,
                        const uint16_t *vres, int res_cap, double sm, int S, double *out,
                        double *lse, int n_threads)
{
    patt_ctx c = {bits, head_dim, hybrid, q, B, Hq, Hkv, k_pool, v_pool, block_stride,
                  head_stride, tbl, max_blocks, state, kres, vres, res_cap, sm, S, out, lse};
    oq_parallel_for((int64_t)B * Hq, n_threads, S ? patt_head_split : patt_head, &c);
}

/* Exposed for the tests: the token range [lo, hi) of split s of a ragged sequence. */
void oq_paged_split_range(int64_t n_packed, int64_t n_res, int S, int s, int64_t *lo,
                          int64_t *hi)
{
    paged_split_range(n_packed, n_res, S, s, lo, hi);
}

/* ------------------------------------------------------------------------------------ */
/* Outer-dimension grouping, the KIVI-style layout the InnerQ page sets against its own  */
/* (sec. 1: the conventional scheme groups the cache along the sequence dimension, so    */
/* the values of one token row belong to different groups and need their own scale and  */
/* zero; sec. 4.1 times it as "KIVI (outer)"). Readings: a group is the 32 consecutive   */
/* tokens 32*tg .. 32*tg+31 of a 128-token block in one channel, for K and for V; the    */
/* quantizer is the same asymmetric one (no hybrid); codes keep the inner layout's        */
/* positions (token t, channel c: word c/32 of token t, bits b*(c%32)), and the          */
/* scale/zero region holds [4 token groups][head_dim channels]{fp16 scale, fp16 zero}    */
/* (the same 2048 bytes at the same offset), so a block has the inner block's size.      */
/* ------------------------------------------------------------------------------------ */

int oq_quantize_pack_outer(int bits, int head_dim, const uint16_t *src, int64_t n_rows,
                           int n_tokens, int64_t src_row_stride, int64_t src_tok_stride,
                           uint8_t *dst, int64_t dst_row_stride, int first_block)
{
    if (bits < 2 || bits > 4 || head_dim % OQ_GROUP || n_tokens % OQ_BLOCK)
        return -1;
    const int64_t bb = oq_block_bytes(bits, head_dim, 0);
    const int ng = head_dim / OQ_GROUP;
    const int64_t gbytes = OQ_GROUP * bits / 8;
    uint8_t *codes = malloc((size_t)OQ_BLOCK * head_dim);
    for (int64_t r = 0; r < n_rows; r++) {
        for (int blk = 0; blk < n_tokens / OQ_BLOCK; blk++) {
            uint8_t *out = dst + r * dst_row_stride + (int64_t)(first_block + blk) * bb;
            memset(out, 0, (size_t)bb);
            const uint16_t *sb = src + r * src_row_stride + (int64_t)blk * OQ_BLOCK * src_tok_stride;
            for (int tg = 0; tg < OQ_BLOCK / OQ_GROUP; tg++) {
                for (int c = 0; c < head_dim; c++) {
                    uint16_t x[OQ_GROUP], sc, z;
                    uint8_t cd[OQ_GROUP];
                    for (int i = 0; i < OQ_GROUP; i++)
                        x[i] = sb[(int64_t)(OQ_GROUP * tg + i) * src_tok_stride + c];
                    oq_asym_candidate(x, bits, &sc, &z, cd);
                    for (int i = 0; i < OQ_GROUP; i++)
                        codes[(OQ_GROUP * tg + i) * head_dim + c] = cd[i];
                    uint8_t *sz = out + oq_sz_offset(bits, head_dim) + ((int64_t)tg * head_dim + c) * 4;
                    put_u16(sz, sc);
                    put_u16(sz + 2, z);
                }
            }
            for (int t = 0; t < OQ_BLOCK; t++)
                for (int g = 0; g < ng; g++)
                    oq_pack_codes(codes + t * head_dim + g * OQ_GROUP, bits,
                                  out + (int64_t)t * ng * gbytes + g * gbytes);
        }
    }
    free(codes);
    return 0;
}

/* Token t of one outer-grouped packed row in fp64: x[c] = zero(tg, c) + code * scale(tg, c). */
static void dequant_token_outer(const uint8_t *row, int bits, int head_dim, int64_t t, double *out)
{
    const int ng = head_dim / OQ_GROUP;
    const int64_t gbytes = OQ_GROUP * bits / 8;
    const uint8_t *blk = row + (t / OQ_BLOCK) * oq_block_bytes(bits, head_dim, 0);
    const int tb = (int)(t % OQ_BLOCK);
    const int tg = tb / OQ_GROUP;
    for (int g = 0; g < ng; g++) {
        uint8_t codes[OQ_GROUP];
        oq_unpack_codes(blk + (int64_t)tb * ng * gbytes + g * gbytes, bits, codes);
        for (int i = 0; i < OQ_GROUP; i++) {
            const int c = g * OQ_GROUP + i;
            const uint8_t *sz = blk + oq_sz_offset(bits, head_dim) + ((int64_t)tg * head_dim + c) * 4;
            const double sc = (double)oq_f16_to_f32(get_u16(sz));
            const double z = (double)oq_f16_to_f32(get_u16(sz + 2));
            out[c] = z + (double)codes[i] * sc;
        }
    }
}

void oq_attention_outer(int bits, int head_dim, const uint16_t *q, int B, int Hq, int Hkv,
                        const uint8_t *kp, const uint8_t *vp, int64_t row_stride, int n_packed,
                        const uint16_t *kres, const uint16_t *vres, int res_cap, int n_res,
                        double sm, double *out, int n_threads)
{
    att_ctx c = {bits, head_dim, 0, q, B, Hq, Hkv, kp, vp, row_stride, n_packed,
                 kres, vres, res_cap, n_res, sm, 0, out, NULL, 1};
    oq_parallel_for((int64_t)B * Hq, n_threads, att_head, &c);
}

void oq_split_attention_outer(int bits, int head_dim, const uint16_t *q, int B, int Hq, int Hkv,
                              const uint8_t *kp, const uint8_t *vp, int64_t row_stride,
                              int n_packed, const uint16_t *kres, const uint16_t *vres,
                              int res_cap, int n_res, double sm, int S, double *part_o,
                              double *part_lse, int n_threads)
{
    att_ctx c = {bits, head_dim, 0, q, B, Hq, Hkv, kp, vp, row_stride, n_packed,
                 kres, vres, res_cap, n_res, sm, S, part_o, part_lse, 1};
    oq_parallel_for((int64_t)B * Hq, n_threads, att_head_split, &c);
}
