/*
 * rq.h -- C ABI of librq.so: ResidualQuant KV-cache encoder, reconstruction
 * and fused decode attention on AMD Instinct MI355X (gfx950).
 *
 * The method (ResidualQuant page, "ResidualQuant: KV Cache Quantization for
 * Looped Transformers with 2-Bit Residuals", Abstract and Fig. 1): a looped
 * Transformer keeps one KV cache per loop.  The final loop's K and V are the
 * reference, kept here in BF16; each earlier loop l is stored as a residual
 * against it -- scaled by a least-squares coefficient (Fig. 1 step 3, Fig. 2),
 * rotated (Fig. 1 step 4), and quantized per group of g values to INT2 or
 * INT4 with a per-group scale and offset (Fig. 1, Table 5), with a bit width
 * chosen per loop (loop-wise mixed precision, Table 5).  Decode attends, for
 * every loop, over that loop's cache reconstructed from the reference and its
 * residual (Abstract: the smaller cache is read with less memory traffic).
 *
 * The reference may instead be stored as a quantized anchor: the pages' final
 * configuration keeps the last loop at INT4 too ("Ascending [2,2,2,4]", Fig. 3
 * caption; one INT4 anchor per loop group, Table 8 caption; INT4 anchor at
 * g=32 with INT2 residuals at g=16, Fig. 6 caption).  The earlier loops' residuals
 * are then taken against the dequantized anchor.  Recent tokens whose
 * earlier-loop K/V cannot be encoded yet (their final loop has not run) can be
 * attended from BF16 rows (a "tail", Table 10: recent BF16 tokens), see
 * rq_decode_attn_tail.
 *
 * Conventions for every entry point:
 *   - Loops are numbered 0 .. n_loops-1; loop n_loops-1 is the reference (BF16,
 *     or the quantized anchor when layout.ref_bits > 0).
 *   - All data pointers are DEVICE pointers on the current HIP device, except
 *     the rq_layout / rq_cache structs themselves, which are host memory and
 *     are only read during the call.
 *   - The library allocates nothing and frees nothing; the caller owns every
 *     buffer.  It keeps no state between calls except per-device caches of
 *     the compute-unit count and the decode kernel's occupancy, and is safe to
 *     call from several host threads.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the call returns without waiting for it.
 *   - Arguments are validated on the host before anything is enqueued; on any
 *     error nothing is enqueued and no output is touched.
 *   - Every plane must be 16-byte aligned.  Planes are contiguous and
 *     token-major within one (batch, head): with cap = layout.capacity,
 *       ref    bf16 [batch][heads][cap][head_dim]
 *       codes  u8   [batch][heads][cap][head_dim*bits/8]  code i of a vector at
 *              bits [bits*(i % (8/bits)), +bits) of byte i*bits/8
 *       meta   f16  [batch][heads][cap][head_dim/group][2]   (scale, zero)
 *       alpha  f16  [batch][heads][cap]
 *     A quantized anchor uses codes[L-1] and meta[L-1] (its own bits and group)
 *     and has no alpha plane and no ref plane.
 *   - Non-finite inputs are not supported (results unspecified, no fault).
 *   - Test hook: with RQ_FAULT_INJECT=launch in the environment, every entry
 *     point that enqueues work returns RQ_ERR_DEVICE after validating its
 *     arguments and before any HIP call (read on every call), so callers'
 *     device-error paths can be exercised without a GPU.
 */
#ifndef RQ_H_
#define RQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RQ_OK = 0,
    RQ_ERR_INVALID_ARG = -1,  /* null/misaligned pointer, bad range, empty mask */
    RQ_ERR_UNSUPPORTED = -2,  /* head_dim, group, bits or loop count outside the supported set;
                                 decode: capacity * 2 * head_dim above 2^32 bytes (per
                                 (b, h) plane offsets are 32-bit), likewise a tail's capacity */
    RQ_ERR_WORKSPACE = -3,    /* decode workspace smaller than rq_decode_workspace_bytes */
    RQ_ERR_DEVICE = -4        /* a HIP call or kernel launch reported an error */
} rq_status;

/* 32 loops covers the pages' longest schedules (Table 8: 32-loop Huginn as
 * 2 x [2^15, 4]) and lets one uint32_t mask name every loop. */
#define RQ_MAX_LOOPS 32

/* Shape of one layer's cache.  Host struct, read-only. */
typedef struct {
    int32_t n_loops;             /* L >= 2; loop L-1 is the BF16 reference            */
    int32_t batch;               /* B >= 1                                            */
    int32_t n_heads;             /* H >= 1 (KV heads; one query per KV head per loop) */
    int32_t head_dim;            /* d in {64, 128, 256}                               */
    int32_t group;               /* g in {16, 32}; d % g == 0                         */
    int32_t capacity;            /* token slots per (batch, head) in every plane, >= 1;
                                    decode streams fastest when it is a multiple of
                                    256 tokens (other strides measured 5-10 % slower) */
    int32_t rotate;              /* 1: normalized Hadamard rotation of residuals; 0: none */
    int32_t bits[RQ_MAX_LOOPS];  /* bits[l] in {2, 4} for l < L-1 (entry L-1 unused)  */
    int32_t ref_bits;            /* 0: loop L-1 is the BF16 ref plane; 2 or 4: loop L-1
                                    is a quantized anchor in codes[L-1] / meta[L-1]  */
    int32_t ref_group;           /* the anchor's group size, 16 or 32 (0 = group);
                                    ignored when ref_bits == 0                        */
    int32_t group_loops;         /* loops per anchor group (0 = n_loops: one group).
                                    Loops [k*G, (k+1)*G) form group k; its last loop
                                    is the group's quantized anchor and the others
                                    are residuals against it (Table 8: one INT4
                                    anchor per group of loops).  G >= 2 divides
                                    n_loops; G < n_loops needs ref_bits > 0         */
    int32_t ref_first;           /* 0: each group's LAST loop is its reference (the
                                    Last-loop policy); 1: its FIRST loop (First-loop
                                    policy; Table 1, Table 9)                       */
    int32_t alpha_mode;          /* residual scaling (Table 9 columns): 0 least
                                    squares <x,y>/<y,y>; 1 none (alpha = 1);
                                    2 norm ratio ||x|| / ||y||                      */
    int32_t ref_chain;           /* 1: chained references (Table 9 "Next-loop", or
                                    "Previous-loop" with ref_first): each residual
                                    loop's reference is its neighbour towards the
                                    group's reference loop, as reconstructed
                                    (y <- fma(alpha, y, r_hat) in FP32, r_hat =
                                    c*H_d fma(code, s, z)); decode rebuilds the
                                    chain.  Needs <= 3 residual loops per group and
                                    ref_bits 0 or 4                                 */
} rq_layout;

/* One side (K or V) of one layer's cache: caller-owned device planes.
 * Entries l >= L-1 of the arrays are ignored, except codes[L-1] and meta[L-1]
 * with a quantized anchor.  With several anchor groups, every group's anchor
 * loop a has codes[a] / meta[a] in the anchor format and no alpha[a]. */
typedef struct {
    void *ref;                   /* bf16 [B][H][cap][d], written by the caller;
                                    unused (may be NULL) with a quantized anchor   */
    void *codes[RQ_MAX_LOOPS];   /* u8   [B][H][cap][d*bits[l]/8]; [L-1]: anchor
                                    codes [B][H][cap][d*ref_bits/8]                */
    void *meta[RQ_MAX_LOOPS];    /* f16  [B][H][cap][d/g][2]; [L-1]: anchor
                                    [B][H][cap][d/ref_group][2]                    */
    void *alpha[RQ_MAX_LOOPS];   /* f16  [B][H][cap]                               */
} rq_cache;

/*
 * rq_encode -- write the residual codes of loops 0..L-2 for tokens [t0, t0+n).
 *
 * Follows the ResidualQuant page: residual against the final loop (Fig. 1
 * step 2), least-squares scale (step 3; Fig. 2), rotation (step 4), group
 * quantization with a per-loop bit width (steps 1 and 5; Table 5).  For each
 * (loop l < L-1, batch b, head h, token t) and separately for K and V, with
 * x the loop-l vector and y = ref[b][h][t] (both BF16, widened exactly):
 *   alpha = fp16(<x,y> / <y,y>)   (alpha_mode 0; 0 if <y,y> = 0; alpha_mode 1:
 *                                   1; alpha_mode 2: sqrt(<x,x>) / sqrt(<y,y>),
 *                                   0 if <y,y> = 0; each dot product sums
 *                                   its FP32 terms in blocks of 8 by pairwise
 *                                   halving, then the block sums by pairwise
 *                                   halving; FP16 stores round to nearest
 *                                   even and saturate at +-65504)
 *   r     = fma(-alpha, y, x)                                     (FP32)
 *   u     = fp32(1/sqrt(d)) * H_d r     if rotate (H_d Sylvester Hadamard,
 *                                        butterflies h = 1, 2, ..., d/2)
 *   per group k of g consecutive dims:  s = fp16((max - min) / (2^b - 1)),
 *     z = fp16(min),  code = clamp(rne((u - z) * (1/s)), 0, 2^b - 1)
 *     (u canonicalized to +0 where it is -0; all codes 0 if s = 0)
 * The result is bit-identical to that FP32 definition.
 *
 * With a quantized anchor (ref_bits > 0) the reference vector y (the BF16
 * input of loop L-1) is first quantized the same way -- rotated if rotate,
 * groups of ref_group, ref_bits codes, no alpha -- and the residual loops use
 * its dequantized value instead of y:
 *   y_hat = fp32(1/sqrt(d)) * H_d u_hat (or u_hat without rotation), with
 *   u_hat = fma(code, s, z) per element (FP32, s and z as stored)
 * (the dot products then sum rounded FP32 products).
 *
 *   k, v    caches; with a BF16 reference their ref planes must already hold
 *           tokens [t0, t0+n)
 *   k_in    bf16 [L-1][B][H][n][d] contiguous: the new K vectors of the loops
 *           other than the reference, in loop order; with quantized anchors
 *           [L][B][H][n][d], every loop in loop order (anchors included)
 *   v_in    same for V
 *   t0, n   0 <= t0, 0 <= n, t0 + n <= capacity (n = 0 is a no-op)
 * Writes codes/meta/alpha of loops 0..L-2 (and the anchor's codes/meta) at
 * slots [t0, t0+n); nothing else.
 */
rq_status rq_encode(const rq_layout *layout, const rq_cache *k, const rq_cache *v,
                    const void *k_in, const void *v_in, int32_t t0, int32_t n,
                    void *hip_stream);

/*
 * rq_decode_workspace_bytes -- bytes of scratch rq_decode_attn needs for
 * `n_ctx` tokens and `n_splits` token splits (0 = the split count the library
 * would choose, see rq_decode_splits); also enough for rq_decode_attn_tail.
 * 0 <= n_ctx <= capacity.  Returns 0 for an invalid layout.
 */
size_t rq_decode_workspace_bytes(const rq_layout *layout, int32_t n_ctx, int32_t n_splits);

/* rq_decode_splits -- the token-split count rq_decode_attn uses when asked
 * for 0 splits (a function of the layout, n_ctx and the device); < 0 on an
 * invalid layout or device error.  For tuning, a positive integer in the
 * environment variable RQ_DECODE_SPLITS replaces the choice (capped at
 * n_ctx); it is read on every call. */
int32_t rq_decode_splits(const rq_layout *layout, int32_t n_ctx);

/*
 * rq_decode_attn -- one decode step of one layer: for every loop l in
 * loop_mask and every (b, h),
 *   out[l][b][h] = softmax(sm_scale * q[l][b][h] . K_l^T) V_l
 * over tokens [0, n_ctx), where K_l, V_l are loop l's keys and values
 * reconstructed as alpha*y + H_n (z + s*code) (the reference itself for loop
 * L-1; with a quantized anchor y is the dequantized anchor, and loop L-1
 * attends over it).  ResidualQuant page, Abstract: decode attention over every loop's
 * compressed cache.  The rotation is applied to the query and to the
 * accumulated output instead of to every key and value (H_n is symmetric and
 * orthonormal), and the reference is read once for all loops in the mask.
 *
 *   q          bf16 [L][B][H][d]: one query per loop (rows not in the mask unread)
 *   loop_mask  bit l set = compute loop l; non-zero, no bit >= L
 *   n_ctx      1 <= n_ctx <= capacity
 *   sm_scale   finite softmax scale (1/sqrt(d) for standard attention)
 *   n_splits   token splits (0 = automatic); 1 <= n_splits <= n_ctx otherwise.
 *              How splits map onto workgroups is the library's choice (a
 *              split runs 4 or 8 waves; two splits without a tail may run as
 *              one 8-wave workgroup per (b, h)); results agree to the
 *              tolerance below either way.  For tuning and tests, the
 *              environment variable RQ_DECODE_WAVES=4 or 8 fixes the waves
 *              per split (read on every call)
 *   out        f32 [L][B][H][d]; rows of loops not in the mask are not written
 *   workspace  device scratch of at least rq_decode_workspace_bytes(layout,
 *              n_ctx, n_splits) bytes, 16-byte aligned; no initialisation
 *              needed; calls that may run concurrently need separate ones
 * Results agree with an FP64 evaluation of the same definition to within a
 * few 1e-4 of the row's largest output magnitude.
 */
rq_status rq_decode_attn(const rq_layout *layout, const rq_cache *k, const rq_cache *v,
                         const void *q, uint32_t loop_mask, int32_t n_ctx, float sm_scale,
                         int32_t n_splits, float *out, void *workspace,
                         size_t workspace_bytes, void *hip_stream);

/* Recent tokens kept in BF16, per loop (host struct, read-only).  Loop l's
 * rows are its own K and V, not residuals. */
typedef struct {
    const void *k[RQ_MAX_LOOPS]; /* bf16 [B][H][capacity][d]; NULL for loops not in the mask */
    const void *v[RQ_MAX_LOOPS]; /* same for V                                          */
    int32_t capacity;            /* token slots per (batch, head) of every tail plane   */
    int32_t n;                   /* tail tokens [0, n) attended, 0 <= n <= capacity      */
} rq_tail;

/*
 * rq_decode_attn_tail -- rq_decode_attn over the n_ctx cached tokens followed
 * by tail->n BF16 tokens: for every loop l in the mask and every (b, h),
 *   out[l][b][h] = softmax(sm_scale * q . [K_l ; Kt_l]^T) [V_l ; Vt_l]
 * with Kt_l, Vt_l the tail rows tail->k[l][b][h][0 .. n).  This is the
 * per-loop decode of a looped model: a token's earlier loops run before its
 * final loop, so its own K/V (and those of recent tokens) are not encoded yet
 * and are attended in BF16 (ResidualQuant page, Table 10: recent tokens kept
 * in BF16).  Arguments as for rq_decode_attn, except:
 *   tail       NULL or a tail; tail->n == 0 makes this call rq_decode_attn
 *   n_ctx      0 <= n_ctx <= capacity, n_ctx + tail->n >= 1 (n_ctx = 0: the
 *              tail alone; no cache plane is read)
 * The tail is meant for tens of tokens: the decode kernel attends it, the one
 * workgroup of the (b, h) when a call has one per (b, h) (one split, or two
 * run as one workgroup), otherwise every split an equal share of the tail
 * rows.  With n_ctx = 0 the merge step attends it alone.
 */
rq_status rq_decode_attn_tail(const rq_layout *layout, const rq_cache *k, const rq_cache *v,
                              const rq_tail *tail, const void *q, uint32_t loop_mask,
                              int32_t n_ctx, float sm_scale, int32_t n_splits, float *out,
                              void *workspace, size_t workspace_bytes, void *hip_stream);

/* Device scratch of rq_decode_attn_tail_noalloc, per GPU. */
#define RQ_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * rq_decode_attn_tail_noalloc -- rq_decode_attn_tail without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * The split records live in a scratch array of RQ_NOALLOC_SCRATCH_BYTES
 * compiled into the library: one copy per GPU, held until the process ends,
 * located on the first call on each device.  Nothing is allocated or freed.
 * Arguments and results are those of rq_decode_attn_tail (same kernels,
 * same split choice); the scratch needs no initialisation.
 *   Returns RQ_ERR_WORKSPACE when the call would need more scratch than
 *   RQ_NOALLOC_SCRATCH_BYTES (rq_decode_workspace_bytes(layout, n_ctx,
 *   n_splits) above it), RQ_ERR_DEVICE when the scratch cannot be located.
 * Every call on one GPU shares that GPU's scratch: calls that may overlap on
 * one device (different streams, different host threads) race and must be
 * serialised by the caller.
 */
rq_status rq_decode_attn_tail_noalloc(const rq_layout *layout, const rq_cache *k, const rq_cache *v,
                                      const rq_tail *tail, const void *q, uint32_t loop_mask,
                                      int32_t n_ctx, float sm_scale, int32_t n_splits, float *out,
                                      void *hip_stream);

/*
 * rq_reconstruct -- dequantize loop `loop` (< L-1) for tokens [t0, t0+n):
 *   out[b][h][t - t0] = alpha*y + H_n (z + s*code)          (FP32)
 * ResidualQuant page, Abstract (the residual form keeps reconstruction
 * cheap).  out is f32 [B][H][n][d]; 0 <= t0, 1 <= n, t0 + n <= capacity.
 * With a quantized anchor y is the dequantized anchor, and loop = L-1 is
 * allowed: it returns the dequantized anchor itself.
 */
rq_status rq_reconstruct(const rq_layout *layout, const rq_cache *c, int32_t loop,
                         int32_t t0, int32_t n, float *out, void *hip_stream);

/* Static description of a status code; never NULL. */
const char *rq_status_string(rq_status status);

#ifdef __cplusplus
}
#endif

#endif /* RQ_H_ */
