/*
 * rq_baseline.h -- BF16-KV decode attention in librq.so, the comparison the
 * ResidualQuant page measures against (Fig. 3 left and Fig. 4: decode
 * throughput normalised to BF16 FlashAttention at the same batch; Fig. 1
 * right: peak throughput and largest feasible batch against BF16).
 *
 * Same kernel skeleton as rq_decode_attn (split-K flash decoding, online
 * softmax, 128-bit loads), applied to plain BF16 caches: every loop keeps its
 * own K and V, so a step reads 2 * n_loops * head_dim * 2 bytes per
 * (batch, head, token).  Conventions (device pointers, validation before
 * enqueue, caller-owned buffers, stream semantics, errors) are those of rq.h.
 */
#ifndef RQ_BASELINE_H_
#define RQ_BASELINE_H_

#include "rq.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * rq_bf16_decode_attn -- for every loop l in loop_mask and every (b, h):
 *   out[l][b][h] = softmax(sm_scale * q[l][b][h] . K_l^T) V_l over [0, n_ctx)
 *   layout      a valid rq_layout; only n_loops, batch, n_heads, head_dim and
 *               capacity matter (group, rotate and bits are not used)
 *   k_loops     host array of n_loops device pointers, each bf16 [B][H][cap][d];
 *               entries of loops not in the mask may be NULL
 *   v_loops     same for V
 *   q, loop_mask, n_ctx, sm_scale, n_splits, out, workspace, workspace_bytes:
 *               as for rq_decode_attn; the workspace size is
 *               rq_decode_workspace_bytes(layout, n_ctx, n_splits)
 */
rq_status rq_bf16_decode_attn(const rq_layout *layout, void *const *k_loops, void *const *v_loops,
                              const void *q, uint32_t loop_mask, int32_t n_ctx, float sm_scale,
                              int32_t n_splits, float *out, void *workspace,
                              size_t workspace_bytes, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* RQ_BASELINE_H_ */
