// rq_internal.hpp -- launchers behind the C ABI (host side, arguments already
// validated by rq_api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rq.h"

namespace rq {

// Kernel argument blocks.  Plane pointers are per residual loop.
// Encoder lane mapping: consecutive dims of one vector per lane.
constexpr int kEncodeElemsPerLane = 32;

// One encode launch covers one anchor group: residual loops 0..n_res-1 of the
// launch and, with a quantized anchor, the anchor at index n_res.
struct EncodeSide {
  const uint16_t *ref;               // bf16 [BH][cap][D] (BF16 reference)
  const uint16_t *xin[RQ_MAX_LOOPS]; // bf16 [BH][n][D] input of residual i; [n_res]: the anchor's
  uint8_t *codes[RQ_MAX_LOOPS];      // [n_res]: the anchor's codes
  uint32_t *meta[RQ_MAX_LOOPS];      // (scale | zero << 16) per group; [n_res]: the anchor's
  uint16_t *alpha[RQ_MAX_LOOPS];
};

struct EncodeArgs {
  EncodeSide side[2];                // K, V
  int32_t bits[RQ_MAX_LOOPS];
  int32_t n_res;                     // L - 1
  int32_t bh;                        // B * H
  int32_t cap, t0, n;
  int32_t group;
  int32_t rotate;
  float rot_c;                       // fp32(1/sqrt(D))
  int32_t chunks;                    // ceil(n / vectors per wave)
  int32_t tasks_per_side;            // bh * chunks
  int32_t abits;                     // 0: BF16 reference; 2, 4: quantized anchor
  int32_t agroup;                    // the anchor's group size
  int32_t alpha_mode;                // 0 least squares, 1 alpha = 1, 2 norm ratio
  int32_t chain;                     // residual i+1's reference is residual i's reconstruction
};

struct ReconArgs {
  const uint16_t *ref;               // BF16 reference (abits == 0)
  const uint8_t *acodes;             // quantized anchor (abits > 0)
  const uint32_t *ameta;
  const uint8_t *codes;              // the loop's planes (NULL: the anchor itself)
  const uint32_t *meta;
  const uint16_t *alpha;
  float *out;                        // f32 [BH][n][D]
  int32_t bits, bh, cap, t0, n, group, rotate;
  float rot_c;
  int32_t chunks;
  int32_t abits, agroup;
  // chained references: the loops between the root and this one, root side
  // first, each rebuilt as y = alpha*y + r_hat before this loop's own step
  int32_t npre;
  const uint8_t *pcodes[3];
  const uint32_t *pmeta[3];
  const uint16_t *palpha[3];
  int32_t pbits[3];
};

constexpr int kMaxRes = 3;           // residual loops per decode pass
constexpr int kMaxSlots = 4;         // residual loops + the reference loop

struct DecodeArgs {
  const uint16_t *kref, *vref;       // bf16 [BH][cap][D] (BF16 reference)
  const uint8_t *kac, *vac;          // quantized anchor codes [BH][cap][D*abits/8]
  const uint32_t *kam, *vam;         // and (scale | zero << 16) [BH][cap][D/agroup]
  int32_t agroup;
  int32_t ref_rotated;               // the anchor is stored rotated (anchor and rotate)
  const uint8_t *kc[kMaxRes], *vc[kMaxRes];
  const uint32_t *km[kMaxRes], *vm[kMaxRes];
  const uint16_t *ka[kMaxRes], *va[kMaxRes];
  int32_t bits[kMaxRes];
  const uint16_t *q;                 // bf16 [L][BH][D]
  int32_t qloop[kMaxSlots];          // slot -> loop index (residual slots first)
  float *ws;                         // f32 [S][kMaxSlots][BH][2D+2] split records
  float *out;                        // f32 [L][BH][D]
  const uint16_t *tk[kMaxSlots], *tv[kMaxSlots];   // BF16 tail rows per slot [BH][tcap][D]
  int32_t tcap, n_tail;
  int32_t records;                   // write split records and merge (S > 1 or a tail)
  int32_t wide;                      // run the two splits as one 8-wave workgroup per batch*head,
                                     // no records (two splits, no tail)
  int32_t waves8;                    // 8-wave workgroups per split (else 4)
  int32_t tail_in;                   // the splits attend the BF16 tail, an equal share each
  uint32_t out_mask;                 // loops whose rows are written (a chain pass also
                                     // computes the links between them and the root)
  int32_t bh, cap, n_ctx, n_splits, tps;
  int32_t group, rotate;
  float qscale;                      // sm_scale * log2(e)
  float rot_c;
};

hipError_t launch_encode(const EncodeArgs &a, int head_dim, hipStream_t s);
hipError_t launch_reconstruct(const ReconArgs &a, int head_dim, hipStream_t s);
// One decode pass of n_res residual loops (+ the reference loop if ref);
// anchor_bits 0 for a BF16 reference; chain 0 (independent references), 1
// (chained references, every slot computed) or 2 (chained, slot 0 alone).
// Launches the merge kernel too when a.records is set.
hipError_t launch_decode(const DecodeArgs &a, int head_dim, int n_res, bool ref, int anchor_bits,
                         int chain, hipStream_t s);
template <int D, int AQ, int CHAIN>
hipError_t launch_decode_d(const DecodeArgs &a, int n_res, bool ref, hipStream_t s);
// The split/tail merge for n_slots loop slots, the first n_res of them residual.
hipError_t launch_merge(const DecodeArgs &a, int head_dim, int n_res, int n_slots, hipStream_t s);
// Decode workgroups of this head_dim resident per compute unit at once (the
// occupancy of the main decode kernel), or <= 0 on a HIP error.
int decode_blocks_per_cu(int head_dim);
template <int D>
int decode_blocks_per_cu_d();

}  // namespace rq
