/*
 * rq_oracle.c -- plain, slow CPU oracle for the ResidualQuant KV-cache path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load this library.  The product path
 * (the HIP library and its Python binding) never calls it, and it shares no
 * code, header, table or helper with the HIP sources.
 *
 * What it computes, with the passage each step follows.  "ResidualQuant page"
 * is the summary page "ResidualQuant: KV Cache Quantization for Looped
 * Transformers with 2-Bit Residuals" (thelatestinai.com, arXiv 2610.10381).
 *
 *   encode (FP32, bit-exact contract):
 *     - the final loop's KV is the reference and every earlier loop is stored
 *       as a low-precision residual against it            (Abstract; Fig. 1 step 2)
 *     - least-square scaling: alpha = <x,y>/<y,y>, residual x - alpha*y
 *                                                   (Abstract; Fig. 1 step 3; Fig. 2;
 *                                                    Fig. 3 right: alpha = 1 means no LS)
 *     - a rotation of the residual (here the normalized Sylvester Hadamard
 *       matrix over head_dim)                          (Abstract; Fig. 1 step 4; Fig. 6)
 *     - group-wise asymmetric INT2/INT4 quantization with per-group scale and
 *       offset, group size g          (Fig. 1 caption: g=32; Table 8 caption: the
 *                                      bit width counts codes, scales, offsets
 *                                      and LS coefficients)
 *     - loop-wise mixed precision: a bit width per loop        (Table 5; Fig. 1 step 5)
 *   quantized anchor (FP32, bit-exact contract): the final loop itself stored
 *       at INT4 with its own group size, the residuals taken against its
 *       dequantized value                (Fig. 3 caption: Ascending [2,2,2,4];
 *                                          Table 8 caption; Fig. 6 caption)
 *   reconstruct (FP64):  x_hat = a*y + H_n (z + s*q)     (Abstract: the residual
 *                                                          form keeps reconstruction
 *                                                          cheap)
 *   attention (FP64):    softmax(scale * q . x_hat^T) v_hat per loop, one query
 *                        per loop, optionally followed by recent tokens kept
 *                        in BF16                         (Abstract: decode over the
 *                                                          compressed cache;
 *                                                          Table 10: recent BF16
 *                                                          tokens)
 *
 * Where the pages leave a step open, the reading taken is stated at the
 * function.  Where floating point decides an integer code, the FP32 steps are
 * spelled out one IEEE operation at a time (build with -ffp-contract=off), so
 * that a device implementation doing the same operations gets the same bytes.
 *
 * Plane layouts (token-major per (batch, head); all little-endian):
 *   ref    bf16 [B][H][cap][d]
 *   codes  u8   [B][H][cap][d*bits/8]   code i at bits [bits*(i % (8/bits)), +bits)
 *                                        of byte i*bits/8
 *   meta   f16  [B][H][cap][d/g][2]      (scale, zero) per group
 *   alpha  f16  [B][H][cap]
 * With a quantized anchor the final loop has codes and meta planes of its own
 * (its bit width and group size) and no ref plane.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define RQO_MAX_D 256

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

/* bfloat16 bits -> float: the 16 stored bits are the top half of an fp32. */
float rqo_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* IEEE binary16 bits -> float, by the definition of the format. */
float rqo_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int exp = (h >> 10) & 0x1f;
    int man = h & 0x3ff;
    double v;
    if (exp == 0)
        v = ldexp((double)man, -24);            /* subnormal: man * 2^-24 */
    else if (exp == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(man + 1024), exp - 25); /* (1 + man/1024) * 2^(exp-15) */
    return (float)(sign ? -v : v);
}

/* float -> IEEE binary16, round to nearest, ties to even; overflow -> inf.
 * Written as "snap to the grid of representable halves near |x|", which is
 * the definition of round-to-nearest on that grid. */
uint16_t rqo_f32_to_f16(float xf)
{
    if (isnan(xf))
        return 0x7e00;
    uint16_t sign = signbit(xf) ? 0x8000 : 0;
    double a = fabs((double)xf);
    /* Halfway between 65504 (largest finite half) and 65536 is 65520; RNE
     * sends 65520 to the even neighbour 65536, which is out of range. */
    if (a >= 65520.0)
        return sign | 0x7c00;
    double quantum;
    if (a < ldexp(1.0, -14)) {
        quantum = ldexp(1.0, -24);              /* subnormal spacing */
    } else {
        int e;
        frexp(a, &e);                           /* a in [2^(e-1), 2^e) */
        quantum = ldexp(1.0, e - 1 - 10);       /* 10 fraction bits */
    }
    double r = nearbyint(a / quantum) * quantum;  /* exact scaling, RNE */
    if (r == 0.0)
        return sign;
    if (r < ldexp(1.0, -14))
        return sign | (uint16_t)(r / ldexp(1.0, -24));
    int e;
    frexp(r, &e);
    int exp_field = (e - 1) + 15;
    int man = (int)(r / ldexp(1.0, e - 1 - 10)) - 1024;
    return sign | (uint16_t)(exp_field << 10) | (uint16_t)man;
}

/* Storage conversion used by the encoder: RNE, but a result that would be
 * infinite is stored as the largest finite half of that sign (reading: the pages
 * store scales, offsets and LS coefficients in 16 bits and never mention
 * overflow; saturating keeps every stored value finite). */
uint16_t rqo_f32_to_f16_sat(float x)
{
    uint16_t h = rqo_f32_to_f16(x);
    if (!isnan(x) && (h & 0x7fff) == 0x7c00)
        return (h & 0x8000) | 0x7bff;
    return h;
}

/* ------------------------------------------------------------------------ */
/* Encoder steps (FP32 contract)                                             */
/* ------------------------------------------------------------------------ */

/* Pairwise-halving sum of n (a power of two) floats: for m = n/2, n/4, ..., 1
 * a[i] <- a[i] + a[i+m] for i < m.  Destroys a. */
float rqo_tree_sum(float *a, int n)
{
    for (int m = n / 2; m >= 1; m /= 2)
        for (int i = 0; i < m; ++i)
            a[i] = a[i] + a[i + m];
    return a[0];
}

/* Sum of the d (a power of two, >= 8) terms of a dot product, in the order
 * the bit-exact contract fixes (the pages give no arithmetic detail): each
 * block of 8 consecutive terms is summed by pairwise halving (distances 4, 2,
 * 1), then the d/8 block sums are summed by pairwise halving.  Destroys a. */
float rqo_dot_sum(float *a, int d)
{
    float blocks[RQO_MAX_D / 8];
    for (int c = 0; c < d / 8; ++c)
        blocks[c] = rqo_tree_sum(a + 8 * c, 8);
    return rqo_tree_sum(blocks, d / 8);
}

/* Least-square coefficient before storage rounding: the alpha that minimises
 * ||x - alpha*y||^2 is <x,y>/<y,y> (ResidualQuant page, Fig. 2 shows the
 * residual K2 - alpha2*K1; Fig. 3 right compares with alpha = 1).
 * Reading: <y,y> == 0 gives alpha = 0 (nothing to predict from). */
float rqo_alpha_f32_y(const uint16_t *x, const float *y, int d)
{
    float num[RQO_MAX_D], den[RQO_MAX_D];
    for (int i = 0; i < d; ++i) {
        float xf = rqo_bf16_to_f32(x[i]);
        num[i] = xf * y[i];
        den[i] = y[i] * y[i];
    }
    float n = rqo_dot_sum(num, d);
    float s = rqo_dot_sum(den, d);
    return s > 0.0f ? n / s : 0.0f;
}

/* The same with a BF16 reference (products of two BF16 values are exact). */
float rqo_alpha_f32(const uint16_t *x, const uint16_t *y, int d)
{
    float yf[RQO_MAX_D];
    for (int i = 0; i < d; ++i)
        yf[i] = rqo_bf16_to_f32(y[i]);
    return rqo_alpha_f32_y(x, yf, d);
}

/* The scaling coefficients the pages compare (Table 9 columns "Residual",
 * "Norm-ratio", "LS scaling"; Fig. 3 right: alpha = 1 without LS):
 *   mode 0: least squares <x,y>/<y,y>
 *   mode 1: no scaling, alpha = 1
 *   mode 2: norm ratio ||x|| / ||y|| = sqrt(<x,x>) / sqrt(<y,y>)  (0 if y = 0)
 * Dot products sum in the contract order; sqrt and division round to
 * nearest (IEEE). */
float rqo_alpha_mode_f32_y(const uint16_t *x, const float *y, int d, int mode)
{
    if (mode == 1)
        return 1.0f;
    if (mode == 0)
        return rqo_alpha_f32_y(x, y, d);
    float xx[RQO_MAX_D], yy[RQO_MAX_D];
    for (int i = 0; i < d; ++i) {
        float xf = rqo_bf16_to_f32(x[i]);
        xx[i] = xf * xf;
        yy[i] = y[i] * y[i];
    }
    float nx = rqo_dot_sum(xx, d);
    float ny = rqo_dot_sum(yy, d);
    return ny > 0.0f ? sqrtf(nx) / sqrtf(ny) : 0.0f;
}

/* Stored coefficient: one FP16 value per (loop, batch, head, token), for K and
 * V separately.  Reading of the pages' effective-bitwidth accounting, which
 * counts LS coefficients and adds 0.1 bit per value for residual loops over
 * direct ones (Table 5: 2.5 -> 2.6, 3.0 -> 3.1, 4.5 -> 4.6), i.e. 16 bits per
 * head_dim-vector. */
uint16_t rqo_alpha_bits(const uint16_t *x, const uint16_t *y, int d)
{
    return rqo_f32_to_f16_sat(rqo_alpha_f32(x, y, d));
}

/* Normalized Walsh-Hadamard rotation in place: butterflies for
 * h = 1, 2, 4, ..., d/2 on pairs (i, i+h), (u_i, u_{i+h}) <- (u_i + u_{i+h},
 * u_i - u_{i+h}), then one multiplication by c = fp32(1/sqrt(d)).
 * The result is c * H_d * u with H_d the Sylvester-ordered Hadamard matrix.
 * Reading: the pages name their rotation (shared OptR-H; OSCAR) without
 * defining it; the plain orthogonal rotation is the normalized Hadamard
 * matrix, shared by K and V, all loops and heads (Fig. 6 uses one
 * shared rotation). */
void rqo_fwht_f32(float *u, int d)
{
    for (int h = 1; h < d; h *= 2)
        for (int j = 0; j < d; j += 2 * h)
            for (int i = j; i < j + h; ++i) {
                float a = u[i], b = u[i + h];
                u[i] = a + b;
                u[i + h] = a - b;
            }
    float c = (float)(1.0 / sqrt((double)d));
    for (int i = 0; i < d; ++i)
        u[i] = u[i] * c;
}

/* Quantize one group of g values to `bits`-bit codes with an asymmetric
 * min/max grid: scale s = (max - min) / (2^bits - 1), offset z = min, both
 * stored FP16; code = clamp(round_half_even((u - z) * (1/s)), 0, 2^bits - 1).
 * Readings: the offset is a floating-point minimum (not an integer zero
 * point); no clipping; the reciprocal of the stored scale is taken once per
 * group; a zero stored scale (constant group) gives all-zero codes. */
void rqo_quantize_group(const float *u, int g, int bits, uint8_t *codes,
                        uint16_t *s16, uint16_t *z16)
{
    float mn = u[0], mx = u[0];
    for (int i = 1; i < g; ++i) {
        if (u[i] < mn) mn = u[i];
        if (u[i] > mx) mx = u[i];
    }
    float levels = (float)((1 << bits) - 1);
    *s16 = rqo_f32_to_f16_sat((mx - mn) / levels);
    *z16 = rqo_f32_to_f16_sat(mn);
    float s = rqo_f16_to_f32(*s16);
    float z = rqo_f16_to_f32(*z16);
    if (s == 0.0f) {
        memset(codes, 0, (size_t)g);
        return;
    }
    float inv = 1.0f / s;
    for (int i = 0; i < g; ++i) {
        float t = (u[i] - z) * inv;
        t = nearbyintf(t);                      /* ties to even */
        if (t < 0.0f) t = 0.0f;
        if (t > levels) t = levels;
        codes[i] = (uint8_t)t;
    }
}

/* LSB-first packing of `bits`-bit codes into bytes. */
void rqo_pack(const uint8_t *codes, int d, int bits, uint8_t *out)
{
    int per = 8 / bits;
    memset(out, 0, (size_t)(d * bits / 8));
    for (int i = 0; i < d; ++i)
        out[i / per] |= (uint8_t)(codes[i] << (bits * (i % per)));
}

void rqo_unpack(const uint8_t *packed, int d, int bits, uint8_t *codes)
{
    int per = 8 / bits;
    for (int i = 0; i < d; ++i)
        codes[i] = (uint8_t)((packed[i / per] >> (bits * (i % per))) & ((1 << bits) - 1));
}

/* Rotate (optionally), canonicalise -0 to +0, quantize every group and pack:
 * the part of encoding shared by residuals and a quantized anchor. */
static void rqo_quantize_vector(float *u, int d, int g, int bits, int rotate,
                                uint8_t *codes, uint8_t *packed, uint16_t *meta)
{
    if (rotate)
        rqo_fwht_f32(u, d);
    for (int i = 0; i < d; ++i)
        u[i] = u[i] + 0.0f;                     /* -0 -> +0 before min/max */
    for (int k = 0; k < d / g; ++k)
        rqo_quantize_group(u + k * g, g, bits, codes + k * g, meta + 2 * k, meta + 2 * k + 1);
    rqo_pack(codes, d, bits, packed);
}

/* Encode one head_dim vector x of a residual loop against an FP32 reference y
 * (the BF16 final loop, or the dequantized anchor). */
void rqo_encode_vector_ym(const uint16_t *x, const float *y, int d, int g,
                          int bits, int rotate, int alpha_mode, uint8_t *packed,
                          uint16_t *meta, uint16_t *alpha)
{
    float u[RQO_MAX_D];
    uint8_t codes[RQO_MAX_D];
    *alpha = rqo_f32_to_f16_sat(rqo_alpha_mode_f32_y(x, y, d, alpha_mode));
    float a = rqo_f16_to_f32(*alpha);          /* the stored value is what decode sees */
    for (int i = 0; i < d; ++i)
        u[i] = fmaf(-a, y[i], rqo_bf16_to_f32(x[i]));
    rqo_quantize_vector(u, d, g, bits, rotate, codes, packed, meta);
}

/* The same with least-squares scaling. */
void rqo_encode_vector_y(const uint16_t *x, const float *y, int d, int g,
                         int bits, int rotate, uint8_t *packed, uint16_t *meta,
                         uint16_t *alpha)
{
    rqo_encode_vector_ym(x, y, d, g, bits, rotate, 0, packed, meta, alpha);
}

/* Encode one head_dim vector x of a residual loop against the BF16 reference y. */
void rqo_encode_vector(const uint16_t *x, const uint16_t *y, int d, int g,
                       int bits, int rotate, uint8_t *packed, uint16_t *meta,
                       uint16_t *alpha)
{
    float yf[RQO_MAX_D];
    for (int i = 0; i < d; ++i)
        yf[i] = rqo_bf16_to_f32(y[i]);
    rqo_encode_vector_y(x, yf, d, g, bits, rotate, packed, meta, alpha);
}

/* Quantized anchor.  ResidualQuant page, Fig. 3 caption: the "Ascending"
 * precision [2,2,2,4] gives the higher precision to the last loop, i.e. the
 * reference itself is stored at INT4; Table 8 caption: every loop group ends
 * in one INT4 anchor; Fig. 6 caption: INT4 anchors use group size 32 while
 * INT2 residuals use 16.  Readings: the anchor is quantized directly (no
 * reference, no LS coefficient) by the same group quantizer after the same
 * shared rotation; the earlier loops take their residuals against the
 * anchor as decode sees it, the dequantized anchor, so that reconstruction
 * adds back exactly what the encoder subtracted.
 *
 * Dequantized value of a code q of a group with stored scale s and offset
 * z: fmaf(q, s, z) in FP32 (one rounding); un-rotated by the same normalized
 * Hadamard butterflies (c*H is its own inverse).  Writes the packed codes,
 * the (scale, zero) pairs and the FP32 dequantized anchor yhat. */
void rqo_anchor_vector(const uint16_t *y, int d, int g, int bits, int rotate,
                       uint8_t *packed, uint16_t *meta, float *yhat)
{
    float u[RQO_MAX_D];
    uint8_t codes[RQO_MAX_D];
    for (int i = 0; i < d; ++i)
        u[i] = rqo_bf16_to_f32(y[i]);
    rqo_quantize_vector(u, d, g, bits, rotate, codes, packed, meta);
    for (int i = 0; i < d; ++i) {
        int k = i / g;
        yhat[i] = fmaf((float)codes[i], rqo_f16_to_f32(meta[2 * k]), rqo_f16_to_f32(meta[2 * k + 1]));
    }
    if (rotate)
        rqo_fwht_f32(yhat, d);
}

/* Encode tokens [t0, t0+n) of residual loops 0..L-2 of every (b, h).
 *   ref:  bf16 [B][H][cap][d]     (the final loop, already in the cache)
 *   xin:  bf16 [L-1][B][H][n][d]  (the earlier loops' new vectors)
 *   codes[l], meta[l], alpha[l]:  planes of loop l (layouts at the top)  */
void rqo_encode(int L, int B, int H, int d, int g, int cap, int rotate,
                const int *bits, const uint16_t *ref, const uint16_t *xin,
                int t0, int n, uint8_t **codes, uint16_t **meta, uint16_t **alpha,
                int alpha_mode)
{
    float yf[RQO_MAX_D];
    int G = d / g;
    for (int l = 0; l < L - 1; ++l) {
        int nb = d * bits[l] / 8;
        for (int b = 0; b < B; ++b)
            for (int h = 0; h < H; ++h)
                for (int t = 0; t < n; ++t) {
                    size_t bh = (size_t)b * H + h;
                    size_t slot = bh * cap + (size_t)(t0 + t);
                    const uint16_t *x = xin + ((((size_t)l * B + b) * H + h) * n + t) * d;
                    const uint16_t *y = ref + slot * d;
                    for (int i = 0; i < d; ++i)
                        yf[i] = rqo_bf16_to_f32(y[i]);
                    rqo_encode_vector_ym(x, yf, d, g, bits[l], rotate, alpha_mode,
                                         codes[l] + slot * nb, meta[l] + slot * 2 * G,
                                         alpha[l] + slot);
                }
    }
}

/* Encode tokens [t0, t0+n) of all L loops with a quantized anchor:
 *   xin: bf16 [L][B][H][n][d]  (loop L-1 is the anchor's input)
 *   codes[l], meta[l] for l = 0..L-1 (the anchor's at L-1, group ga, abits
 *   bits); alpha[l] for l = 0..L-2.  Per (b, h, token) the anchor is encoded
 *   first and its dequantized value is every residual loop's reference. */
void rqo_encode_anchored(int L, int B, int H, int d, int g, int ga, int abits,
                         int cap, int rotate, const int *bits, const uint16_t *xin,
                         int t0, int n, uint8_t **codes, uint16_t **meta, uint16_t **alpha,
                         int alpha_mode)
{
    int G = d / g, Ga = d / ga, nba = d * abits / 8;
    float yhat[RQO_MAX_D];
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int t = 0; t < n; ++t) {
                size_t bh = (size_t)b * H + h;
                size_t slot = bh * cap + (size_t)(t0 + t);
                const uint16_t *y = xin + ((((size_t)(L - 1) * B + b) * H + h) * n + t) * d;
                rqo_anchor_vector(y, d, ga, abits, rotate, codes[L - 1] + slot * nba,
                                  meta[L - 1] + slot * 2 * Ga, yhat);
                for (int l = 0; l < L - 1; ++l) {
                    int nb = d * bits[l] / 8;
                    const uint16_t *x = xin + ((((size_t)l * B + b) * H + h) * n + t) * d;
                    rqo_encode_vector_ym(x, yhat, d, g, bits[l], rotate, alpha_mode,
                                         codes[l] + slot * nb, meta[l] + slot * 2 * G,
                                         alpha[l] + slot);
                }
            }
}

/* Chained references (RQ page Table 9 "Previous-loop" / "Next-loop"; Fig. 3
 * left): each loop's reference is its neighbour towards the group's root
 * loop, as decode will rebuild it.  After a loop is encoded against y, the
 * next loop's reference is that loop's FP32 reconstruction
 *   y <- fmaf(a, y, r_hat),  r_hat = c*H(fmaf(code, s, z)) (or unrotated)
 * (the reading: closed loop, one rounding per FMA, the butterflies of the
 * rotation in their usual order).  ord lists the group's residual loops from
 * the root outwards; xin holds the loops of the group in loop order. */
void rqo_reconstruct32_vector(const uint8_t *packed, const uint16_t *meta, uint16_t alpha,
                              float *y, int d, int g, int bits, int rotate)
{
    uint8_t codes[RQO_MAX_D];
    float u[RQO_MAX_D];
    rqo_unpack(packed, d, bits, codes);
    for (int i = 0; i < d; ++i) {
        int k = i / g;
        u[i] = fmaf((float)codes[i], rqo_f16_to_f32(meta[2 * k]), rqo_f16_to_f32(meta[2 * k + 1]));
    }
    if (rotate)
        rqo_fwht_f32(u, d);
    float a = rqo_f16_to_f32(alpha);
    for (int i = 0; i < d; ++i)
        y[i] = fmaf(a, y[i], u[i]);
}

/* Encode tokens [t0, t0+n) of one group with chained references.
 *   L: loops in the group; root: the reference loop (index within the group);
 *   ord[0..L-2]: residual loops from the root outwards; abits: 0 = the root is
 *   the BF16 ref plane (ref), else a quantized anchor whose input is xin[root];
 *   xin: bf16 [L][B][H][n][d] when anchored, else [L][B][H][n][d] with the
 *   root's entry unused (the caller passes the group's loops in loop order,
 *   the root's slot may hold anything). */
void rqo_encode_chain(int L, int B, int H, int d, int g, int ga, int abits, int cap,
                      int rotate, int alpha_mode, const int *bits, int root, const int *ord,
                      const uint16_t *ref, const uint16_t *xin, int t0, int n,
                      uint8_t **codes, uint16_t **meta, uint16_t **alpha)
{
    int G = d / g, Ga = d / ga;
    float y[RQO_MAX_D];
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int t = 0; t < n; ++t) {
                size_t bh = (size_t)b * H + h;
                size_t slot = bh * cap + (size_t)(t0 + t);
                if (abits) {
                    const uint16_t *yi = xin + ((((size_t)root * B + b) * H + h) * n + t) * d;
                    rqo_anchor_vector(yi, d, ga, abits, rotate, codes[root] + slot * (d * abits / 8),
                                      meta[root] + slot * 2 * Ga, y);
                } else {
                    for (int i = 0; i < d; ++i)
                        y[i] = rqo_bf16_to_f32(ref[slot * d + i]);
                }
                for (int k = 0; k < L - 1; ++k) {
                    int l = ord[k], nb = d * bits[l] / 8;
                    const uint16_t *x = xin + ((((size_t)l * B + b) * H + h) * n + t) * d;
                    uint8_t *pc = codes[l] + slot * nb;
                    uint16_t *pm = meta[l] + slot * 2 * G;
                    rqo_encode_vector_ym(x, y, d, g, bits[l], rotate, alpha_mode, pc, pm, alpha[l] + slot);
                    rqo_reconstruct32_vector(pc, pm, alpha[l][slot], y, d, g, bits[l], rotate);
                }
            }
}

/* ------------------------------------------------------------------------ */
/* Reconstruction and attention (FP64)                                       */
/* ------------------------------------------------------------------------ */

/* Dequantize a vector in FP64: u = z + s*q per group, then H_d u / sqrt(d)
 * (exact constant) when rotated.  For a residual this is r_hat; for a
 * quantized anchor it is the anchor y_hat. */
void rqo_dequant_f64(const uint8_t *packed, const uint16_t *meta, int d, int g,
                     int bits, int rotate, double *out)
{
    uint8_t codes[RQO_MAX_D];
    double *u = out;
    rqo_unpack(packed, d, bits, codes);
    for (int i = 0; i < d; ++i) {
        int k = i / g;
        double s = rqo_f16_to_f32(meta[2 * k]);
        double z = rqo_f16_to_f32(meta[2 * k + 1]);
        u[i] = z + s * (double)codes[i];
    }
    if (rotate) {
        for (int h = 1; h < d; h *= 2)
            for (int j = 0; j < d; j += 2 * h)
                for (int i = j; i < j + h; ++i) {
                    double a = u[i], b = u[i + h];
                    u[i] = a + b;
                    u[i + h] = a - b;
                }
        double c = 1.0 / sqrt((double)d);
        for (int i = 0; i < d; ++i)
            u[i] *= c;
    }
}

/* x_hat = a*y + H_d (z + s*q) / sqrt(d)  (or without the rotation), y in FP64. */
void rqo_reconstruct_vector_y(const uint8_t *packed, const uint16_t *meta,
                              uint16_t alpha, const double *y, int d, int g,
                              int bits, int rotate, double *out)
{
    double u[RQO_MAX_D];
    rqo_dequant_f64(packed, meta, d, g, bits, rotate, u);
    double a = rqo_f16_to_f32(alpha);
    for (int i = 0; i < d; ++i)
        out[i] = a * y[i] + u[i];
}

/* The same against the BF16 reference y. */
void rqo_reconstruct_vector(const uint8_t *packed, const uint16_t *meta,
                            uint16_t alpha, const uint16_t *y, int d, int g,
                            int bits, int rotate, double *out)
{
    double yd[RQO_MAX_D];
    for (int i = 0; i < d; ++i)
        yd[i] = rqo_bf16_to_f32(y[i]);
    rqo_reconstruct_vector_y(packed, meta, alpha, yd, d, g, bits, rotate, out);
}

/* Reconstruct tokens [t0, t0+n) of residual loop `loop` for every (b, h):
 * out is float64 [B][H][n][d]. */
void rqo_reconstruct(int B, int H, int d, int g, int cap, int rotate, int bits,
                     const uint16_t *ref, const uint8_t *codes,
                     const uint16_t *meta, const uint16_t *alpha, int t0, int n,
                     double *out)
{
    int G = d / g, nb = d * bits / 8;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int t = 0; t < n; ++t) {
                size_t slot = ((size_t)b * H + h) * cap + (size_t)(t0 + t);
                rqo_reconstruct_vector(codes + slot * nb, meta + slot * 2 * G,
                                       alpha[slot], ref + slot * d, d, g, bits,
                                       rotate, out + (((size_t)b * H + h) * n + t) * d);
            }
}

/* Reconstruct tokens [t0, t0+n) of loop `loop` against a quantized anchor
 * (anchor planes ac/am, group ga, abits bits): the dequantized anchor for
 * loop L-1 (pass loop = -1 and NULL residual planes), a*y_hat + r_hat for a
 * residual loop.  out is float64 [B][H][n][d]. */
void rqo_reconstruct_anchored(int B, int H, int d, int g, int ga, int abits, int cap,
                              int rotate, int bits, const uint8_t *ac, const uint16_t *am,
                              const uint8_t *codes, const uint16_t *meta,
                              const uint16_t *alpha, int loop, int t0, int n, double *out)
{
    int G = d / g, nb = d * bits / 8, Ga = d / ga, nba = d * abits / 8;
    double y[RQO_MAX_D];
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int t = 0; t < n; ++t) {
                size_t slot = ((size_t)b * H + h) * cap + (size_t)(t0 + t);
                double *o = out + (((size_t)b * H + h) * n + t) * d;
                rqo_dequant_f64(ac + slot * nba, am + slot * 2 * Ga, d, ga, abits, rotate, y);
                if (loop < 0)
                    memcpy(o, y, sizeof(double) * (size_t)d);
                else
                    rqo_reconstruct_vector_y(codes + slot * nb, meta + slot * 2 * G, alpha[slot],
                                             y, d, g, bits, rotate, o);
            }
}

/* Chain reconstruction in FP64 of one vector of loop ord[upto] (0-based
 * position along the chain from the root): y = root; y = a*y + r_hat for
 * ord[0..upto].  rootv: the root's FP64 vector. */
void rqo_reconstruct_chain_vector(const uint8_t **pc, const uint16_t **pm, const uint16_t **pa,
                                  const int *bits, const int *ord, int upto, const double *rootv,
                                  int d, int g, int rotate, double *out)
{
    double u[RQO_MAX_D];
    memcpy(out, rootv, sizeof(double) * (size_t)d);
    for (int k = 0; k <= upto; ++k) {
        int l = ord[k];
        rqo_dequant_f64(pc[l], pm[l], d, g, bits[l], rotate, u);
        double a = rqo_f16_to_f32(*pa[l]);
        for (int i = 0; i < d; ++i)
            out[i] = a * out[i] + u[i];
    }
}

/* FP64 rows of one (batch*head) bh, tokens [t0, t0+n), of the loop at chain
 * position `upto` (-1: the root itself) of a group with chained references:
 * the root is the BF16 plane `ref` (abits == 0) or the anchor planes ac/am;
 * codes/meta/alpha are indexed by the loop's index within the group.
 * out: float64 [n][d]. */
void rqo_chain_rows(int d, int g, int ga, int abits, int cap, int rotate, const int *bits,
                    const int *ord, int upto, const uint16_t *ref, const uint8_t *ac,
                    const uint16_t *am, const uint8_t **codes, const uint16_t **meta,
                    const uint16_t **alpha, int bh, int t0, int n, double *out)
{
    int G = d / g, Ga = abits ? d / ga : 0;
    double rootv[RQO_MAX_D];
    const uint8_t *pc[RQO_MAX_D];
    const uint16_t *pm[RQO_MAX_D], *pa[RQO_MAX_D];
    for (int t = 0; t < n; ++t) {
        size_t slot = (size_t)bh * cap + (size_t)(t0 + t);
        if (abits)
            rqo_dequant_f64(ac + slot * (d * abits / 8), am + slot * 2 * Ga, d, ga, abits, rotate, rootv);
        else
            for (int i = 0; i < d; ++i)
                rootv[i] = rqo_bf16_to_f32(ref[slot * d + i]);
        for (int k = 0; k <= upto; ++k) {
            int l = ord[k];
            pc[l] = codes[l] + slot * (d * bits[l] / 8);
            pm[l] = meta[l] + slot * 2 * G;
            pa[l] = alpha[l] + slot;
        }
        if (upto < 0)
            memcpy(out + (size_t)t * d, rootv, sizeof(double) * (size_t)d);
        else
            rqo_reconstruct_chain_vector(pc, pm, pa, bits, ord, upto, rootv, d, g, rotate,
                                         out + (size_t)t * d);
    }
}

/* Softmax attention of one query over n keys/values, in FP64:
 * s_t = scale * <q, k_t>, p = softmax(s) (max-subtracted), out = sum_t p_t v_t. */
void rqo_attention(const double *q, const double *k, const double *v, int n,
                   int d, double scale, double *out)
{
    double *s = (double *)malloc(sizeof(double) * (size_t)n);
    double m = -INFINITY;
    for (int t = 0; t < n; ++t) {
        double acc = 0.0;
        for (int i = 0; i < d; ++i)
            acc += q[i] * k[(size_t)t * d + i];
        s[t] = scale * acc;
        if (s[t] > m) m = s[t];
    }
    double den = 0.0;
    for (int i = 0; i < d; ++i)
        out[i] = 0.0;
    for (int t = 0; t < n; ++t) {
        double p = exp(s[t] - m);
        den += p;
        for (int i = 0; i < d; ++i)
            out[i] += p * v[(size_t)t * d + i];
    }
    for (int i = 0; i < d; ++i)
        out[i] /= den;
    free(s);
}

/* One decode row: attention of loop `loop`'s query of (b, h) over tokens
 * [0, n_ctx) of that loop's cache, reconstructed in FP64, followed by n_tail
 * tokens kept in BF16 (the loop's own K/V rows, tk/tv bf16 [n_tail][d]).
 * The final loop (loop == L-1) attends over the reference itself: the BF16
 * plane when abits == 0, else the dequantized anchor (planes kac/kam, vac/vam,
 * group ga, abits bits).  kc/km/ka etc. are loop `loop`'s residual planes
 * (ignored for the final loop); q: bf16 [L][B][H][d]; out: float64 [d].
 * Reading for the tail: the current token's earlier-loop K/V cannot be
 * encoded before its final loop has run, so recent tokens stay in BF16 and
 * are attended as they are (RQ page, Table 10: "Recent 64" BF16 tokens). */
void rqo_decode_row_ex(int L, int B, int H, int d, int g, int cap, int rotate,
                       int bits, const uint16_t *kref, const uint8_t *kc,
                       const uint16_t *km, const uint16_t *ka,
                       const uint16_t *vref, const uint8_t *vc,
                       const uint16_t *vm, const uint16_t *va,
                       int ga, int abits, const uint8_t *kac, const uint16_t *kam,
                       const uint8_t *vac, const uint16_t *vam,
                       const uint16_t *tk, const uint16_t *tv, int n_tail,
                       const uint16_t *q, int loop, int b, int h, int n_ctx,
                       double scale, double *out)
{
    size_t bh = (size_t)b * H + h;
    int n_all = n_ctx + n_tail;
    double *kh = (double *)malloc(sizeof(double) * (size_t)n_all * d);
    double *vh = (double *)malloc(sizeof(double) * (size_t)n_all * d);
    double qd[RQO_MAX_D], yk[RQO_MAX_D], yv[RQO_MAX_D];
    const uint16_t *qrow = q + (((size_t)loop * B + b) * H + h) * d;
    for (int i = 0; i < d; ++i)
        qd[i] = rqo_bf16_to_f32(qrow[i]);
    int G = d / g, nb = d * bits / 8;
    int Ga = abits ? d / ga : 0, nba = d * abits / 8;
    for (int t = 0; t < n_ctx; ++t) {
        size_t slot = bh * cap + (size_t)t;
        if (abits) {
            rqo_dequant_f64(kac + slot * nba, kam + slot * 2 * Ga, d, ga, abits, rotate, yk);
            rqo_dequant_f64(vac + slot * nba, vam + slot * 2 * Ga, d, ga, abits, rotate, yv);
        } else {
            for (int i = 0; i < d; ++i) {
                yk[i] = rqo_bf16_to_f32(kref[slot * d + i]);
                yv[i] = rqo_bf16_to_f32(vref[slot * d + i]);
            }
        }
        double *kt = kh + (size_t)t * d, *vt = vh + (size_t)t * d;
        if (loop == L - 1) {
            memcpy(kt, yk, sizeof(double) * (size_t)d);
            memcpy(vt, yv, sizeof(double) * (size_t)d);
        } else {
            rqo_reconstruct_vector_y(kc + slot * nb, km + slot * 2 * G, ka[slot], yk, d, g,
                                     bits, rotate, kt);
            rqo_reconstruct_vector_y(vc + slot * nb, vm + slot * 2 * G, va[slot], yv, d, g,
                                     bits, rotate, vt);
        }
    }
    for (int t = 0; t < n_tail; ++t)
        for (int i = 0; i < d; ++i) {
            kh[(size_t)(n_ctx + t) * d + i] = rqo_bf16_to_f32(tk[(size_t)t * d + i]);
            vh[(size_t)(n_ctx + t) * d + i] = rqo_bf16_to_f32(tv[(size_t)t * d + i]);
        }
    rqo_attention(qd, kh, vh, n_all, d, scale, out);
    free(kh);
    free(vh);
}

/* rqo_decode_row_ex with the BF16 reference and no tail. */
void rqo_decode_row(int L, int B, int H, int d, int g, int cap, int rotate,
                    int bits, const uint16_t *kref, const uint8_t *kc,
                    const uint16_t *km, const uint16_t *ka,
                    const uint16_t *vref, const uint8_t *vc,
                    const uint16_t *vm, const uint16_t *va, const uint16_t *q,
                    int loop, int b, int h, int n_ctx, double scale,
                    double *out)
{
    rqo_decode_row_ex(L, B, H, d, g, cap, rotate, bits, kref, kc, km, ka, vref, vc, vm, va,
                      g, 0, NULL, NULL, NULL, NULL, NULL, NULL, 0, q, loop, b, h, n_ctx,
                      scale, out);
}
