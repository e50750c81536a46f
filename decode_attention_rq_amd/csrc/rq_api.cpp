// rq_api.cpp -- the extern "C" entry points of librq.so: validate on the
// host, fill the kernel argument blocks, enqueue on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "rq.h"
#include "rq_baseline.h"
#include "rq_internal.hpp"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

bool aligned16(const void *p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Layout checks shared by every entry point.
rq_status check_layout(const rq_layout *L) {
  if (L == nullptr) return RQ_ERR_INVALID_ARG;
  if (L->n_loops < 2 || L->n_loops > RQ_MAX_LOOPS) return RQ_ERR_UNSUPPORTED;
  if (L->batch < 1 || L->n_heads < 1 || L->capacity < 1) return RQ_ERR_INVALID_ARG;
  if ((int64_t)L->batch * L->n_heads > 65535) return RQ_ERR_UNSUPPORTED;   // grid y limit
  if (L->head_dim != 64 && L->head_dim != 128 && L->head_dim != 256) return RQ_ERR_UNSUPPORTED;
  if (L->group != 16 && L->group != 32) return RQ_ERR_UNSUPPORTED;
  if (L->head_dim % L->group != 0) return RQ_ERR_UNSUPPORTED;
  if (L->rotate != 0 && L->rotate != 1) return RQ_ERR_INVALID_ARG;
  const int G = L->group_loops ? L->group_loops : L->n_loops;
  if (G < 2 || G > L->n_loops || L->n_loops % G != 0) return RQ_ERR_UNSUPPORTED;
  if (L->ref_first != 0 && L->ref_first != 1) return RQ_ERR_INVALID_ARG;
  if (L->alpha_mode < 0 || L->alpha_mode > 2) return RQ_ERR_UNSUPPORTED;
  if (L->ref_chain != 0 && L->ref_chain != 1) return RQ_ERR_INVALID_ARG;
  // a chain pass reads every link between the root and the loop: at most
  // kMaxRes residual loops per group; anchors of 4 bits or BF16 roots
  if (L->ref_chain && (G - 1 > rq::kMaxRes || L->ref_bits == 2)) return RQ_ERR_UNSUPPORTED;
  const int aof = L->ref_first ? 0 : G - 1;         // the anchor's place in its group
  for (int l = 0; l < L->n_loops; ++l)
    if (l % G != aof && L->bits[l] != 2 && L->bits[l] != 4) return RQ_ERR_UNSUPPORTED;
  if (L->ref_bits != 0 && L->ref_bits != 2 && L->ref_bits != 4) return RQ_ERR_UNSUPPORTED;
  if (G < L->n_loops && L->ref_bits == 0) return RQ_ERR_UNSUPPORTED;   // one BF16 ref plane only
  if (L->ref_bits != 0) {
    const int ga = L->ref_group ? L->ref_group : L->group;
    if (ga != 16 && ga != 32) return RQ_ERR_UNSUPPORTED;
  }
  // token indices are int32 inside the kernels
  if ((int64_t)L->batch * L->n_heads * L->capacity > INT32_MAX) return RQ_ERR_UNSUPPORTED;
  return RQ_OK;
}

// The decode kernels address one (batch, head)'s rows of a plane with 32-bit
// byte offsets; the widest row is a BF16 row of 2*head_dim bytes, so the
// largest offset read is below capacity * 2 * head_dim.
bool rows_fit_u32(int64_t capacity, int head_dim) { return capacity * 2 * head_dim <= ((int64_t)1 << 32); }

int anchor_group(const rq_layout *L) { return L->ref_group ? L->ref_group : L->group; }

// Loops per anchor group, the anchor (reference) loop of loop l's group, and
// whether l is an anchor.
int group_len(const rq_layout *L) { return L->group_loops ? L->group_loops : L->n_loops; }
int anchor_of(const rq_layout *L, int l) {
  const int G = group_len(L);
  return (l / G) * G + (L->ref_first ? 0 : G - 1);
}
bool is_anchor(const rq_layout *L, int l) { return anchor_of(L, l) == l; }

// The residual loops of loop g0's group from the root outwards (the chain
// order; also the encode order).  Returns their number.
int chain_order(const rq_layout *L, int g0, int *ord) {
  const int G = group_len(L);
  int n = 0;
  if (L->ref_first)
    for (int l = g0 + 1; l < g0 + G; ++l) ord[n++] = l;
  else
    for (int l = g0 + G - 2; l >= g0; --l) ord[n++] = l;
  return n;
}

// The reference planes of the group whose anchor is loop a: the BF16 ref
// plane, or the anchor's codes and meta.
bool ref_planes_ok(const rq_layout *L, const rq_cache *c, int a) {
  if (L->ref_bits == 0) return aligned16(c->ref);
  return aligned16(c->codes[a]) && aligned16(c->meta[a]);
}

bool residual_planes_ok(const rq_cache *c, int l) {
  return aligned16(c->codes[l]) && aligned16(c->meta[l]) && aligned16(c->alpha[l]);
}

rq_status check_cache(const rq_layout *L, const rq_cache *c) {
  if (c == nullptr) return RQ_ERR_INVALID_ARG;
  for (int l = 0; l < L->n_loops; ++l) {
    if (is_anchor(L, l) ? !ref_planes_ok(L, c, l) : !residual_planes_ok(c, l)) return RQ_ERR_INVALID_ARG;
  }
  return RQ_OK;
}

float rot_const(int d) { return (float)(1.0 / std::sqrt((double)d)); }

// Test hook: with RQ_FAULT_INJECT=launch in the environment, every entry point
// that enqueues work returns RQ_ERR_DEVICE after validating its arguments and
// before any HIP call, so callers' device-error paths can be exercised
// without a GPU.  Read on every call.
bool launch_fault_injected() {
  const char *v = std::getenv("RQ_FAULT_INJECT");
  return v != nullptr && std::strcmp(v, "launch") == 0;
}

int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
  int n = g_cu_count[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return -1;
  g_cu_count[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Decode workgroups that run at once on the current device, per head_dim
// (64, 128, 256), cached per device.
std::atomic<int> g_slots[kMaxDevices][3];

int decode_slots(int head_dim) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
  const int idx = head_dim == 64 ? 0 : head_dim == 128 ? 1 : 2;
  int n = g_slots[dev][idx].load(std::memory_order_relaxed);
  if (n > 0) return n;
  const int cus = cu_count();
  const int per_cu = rq::decode_blocks_per_cu(head_dim);
  if (cus <= 0 || per_cu <= 0) return -1;
  n = cus * per_cu;
  g_slots[dev][idx].store(n, std::memory_order_relaxed);
  return n;
}

// Token splits for a decode step (in units of 4-wave workgroups; `slots` =
// compute units times resident decode workgroups per unit).
//  * Small batch (bh workgroups leave slots idle): enough splits to fill the
//    slots, but no more than about sqrt(n_ctx / 32): every workgroup runs at
//    once, and the step is one workgroup's chain of tiles plus a merge that
//    grows with the split count (8 splits at 2k, 16 from 8k on; never under
//    256 tokens per split).  When 8 or more splits fit one workgroup per
//    compute unit, the most that fit are taken instead (they then run 8
//    waves each).
//  * Large batch: a decode step is bound by HBM, and a partial last round of
//    workgroups still streams at full rate once it holds half the slots.  So
//    among 1..4 splits take the fewest rounds-equivalent of work, counting a
//    partial round as at least half a round, with 1% for the merge of more
//    than one split.
// Interleaved MI355X timings (batch 1..128, 2k / 8k / 32k, fused and per-loop
// passes) put this rule within 2% of the best count at most points, 5% at
// worst.
int auto_splits(const rq_layout *L, int n_ctx, int slots, int cus) {
  const int64_t bh = (int64_t)L->batch * L->n_heads;
  int64_t max_s = n_ctx / 256 > 0 ? n_ctx / 256 : 1;
  if (max_s > 32) max_s = 32;
  const int64_t fill = (slots + bh - 1) / bh;
  int64_t best = 1;
  if (fill > 1) {
    int64_t lat = (int64_t)std::lround(std::sqrt((double)n_ctx / 32.0));
    if (lat < 1) lat = 1;
    if (lat > 16) lat = 16;
    best = fill < lat ? fill : lat;
    // Workgroups that fit one per compute unit run with 8 waves (see
    // decode_waves); when 8 or more splits fit, take the most that fit, so
    // each 8-wave workgroup has the fewest tiles to chain (batch 1 at 4k,
    // per-loop calls with a tail: 16 splits 7% faster than 11; at 2k the
    // 256-token floor keeps 8, as fast as 16 there).
    if (cus > 0 && cus / bh >= 8) best = cus / bh;
  } else {
    double best_cost = -1.0;
    for (int64_t sp = 1; sp <= 4; ++sp) {
      const int64_t blocks = sp * bh, full = blocks / slots, rem = blocks % slots;
      const double rounds = (double)full + (rem > 0 ? (double)std::max<int64_t>(rem, slots / 2) / slots : 0.0);
      const double cost = rounds * (double)((n_ctx + sp - 1) / sp) * (sp > 1 ? 1.01 : 1.0);
      if (best_cost < 0.0 || cost < best_cost - 1e-9) { best_cost = cost; best = sp; }
    }
  }
  if (best > max_s) best = max_s;
  int64_t s = best;
  if (const char *env = std::getenv("RQ_DECODE_SPLITS")) {
    const int v = std::atoi(env);
    if (v >= 1) s = v < n_ctx ? v : n_ctx;
  }
  return (int)s;
}

// Workgroup shape of a decode call with S token splits over bh batch*heads
// (a kernel with ~250 VGPRs runs at most 8 waves per compute unit):
//  * wide: two splits and bh in (CUs/2, CUs]: the two 4-wave workgroups of
//    each (b, h) run as one 8-wave workgroup over all tokens, with no split
//    records and no merge launch (2-10% faster at batch 16 for fused,
//    per-loop, anchored and chained passes; with bh <= CUs/2 it would leave
//    compute units idle);
//  * waves8: otherwise, when S*bh <= CUs (one workgroup per unit), each
//    split runs 8 waves instead of 4 (2-6% faster at batch 1-2);
//  * else 4-wave workgroups, two per unit.
// For tuning and tests, RQ_DECODE_WAVES=4 forces 4-wave workgroups, and
// RQ_DECODE_WAVES=8 forces 8 (two splits then always run wide).  Read on
// every call.
void decode_waves(int S, int bh, int32_t *wide, int32_t *waves8) {
  int force = 0;
  if (const char *env = std::getenv("RQ_DECODE_WAVES")) {
    const int v = std::atoi(env);
    if (v == 4 || v == 8) force = v;
  }
  const int cus = cu_count();
  if (force == 4) {
    *wide = *waves8 = 0;
  } else if (force == 8) {
    *wide = S == 2 ? 1 : 0;
    *waves8 = 1;
  } else {
    *wide = (S == 2 && cus > 0 && 2 * bh > cus && bh <= cus) ? 1 : 0;
    *waves8 = (cus > 0 && (int64_t)S * bh <= cus) ? 1 : 0;
  }
}

// Workspace: the split records f32 [S][kMaxSlots][BH][2D+2].  A call with
// one workgroup per (b, h) (one split, or the wide form of two) writes no
// records; one split's worth is still asked for, so that a workspace sized
// for any split count is never empty.
size_t workspace_for(const rq_layout *L, int n_splits) {
  const size_t s = n_splits > 1 ? (size_t)n_splits : 1;
  return s * rq::kMaxSlots * (size_t)L->batch * L->n_heads * (size_t)(2 * L->head_dim + 2) *
         sizeof(float);
}

}  // namespace

extern "C" {

const char *rq_status_string(rq_status status) {
  // A C caller may pass any int: read the bytes as one, since loading an
  // out-of-range value through the enum type is undefined in C++.
  int s;
  std::memcpy(&s, &status, sizeof s);
  switch (s) {
    case RQ_OK: return "RQ_OK";
    case RQ_ERR_INVALID_ARG: return "RQ_ERR_INVALID_ARG: null or misaligned pointer, or an argument out of range";
    case RQ_ERR_UNSUPPORTED: return "RQ_ERR_UNSUPPORTED: head_dim, group, bits or loop count outside the supported set";
    case RQ_ERR_WORKSPACE: return "RQ_ERR_WORKSPACE: decode workspace smaller than rq_decode_workspace_bytes";
    case RQ_ERR_DEVICE: return "RQ_ERR_DEVICE: a HIP call or kernel launch failed";
  }
  return "unknown rq_status";
}

rq_status rq_encode(const rq_layout *L, const rq_cache *k, const rq_cache *v, const void *k_in,
                    const void *v_in, int32_t t0, int32_t n, void *hip_stream) {
  rq_status st = check_layout(L);
  if (st != RQ_OK) return st;
  if ((st = check_cache(L, k)) != RQ_OK || (st = check_cache(L, v)) != RQ_OK) return st;
  if (!aligned16(k_in) || !aligned16(v_in)) return RQ_ERR_INVALID_ARG;
  if (t0 < 0 || n < 0 || (int64_t)t0 + n > L->capacity) return RQ_ERR_INVALID_ARG;
  if (n == 0) return RQ_OK;

  const int G = group_len(L);
  const int64_t bh = (int64_t)L->batch * L->n_heads;
  const int vpw = 64 / (L->head_dim / rq::kEncodeElemsPerLane);   // vectors per encode wave
  const int chunks = (n + vpw - 1) / vpw;
  if (bh * chunks * 2 > INT32_MAX - 4) return RQ_ERR_UNSUPPORTED;
  const rq_cache *sides[2] = {k, v};
  const void *ins[2] = {k_in, v_in};
  // Inputs: with a BF16 reference the non-reference loops in loop order; with
  // quantized anchors every loop in loop order.
  const size_t loop_elems = (size_t)bh * n * L->head_dim;
  if (launch_fault_injected()) return RQ_ERR_DEVICE;
  (void)hipGetLastError();
  for (int g0 = 0; g0 < L->n_loops; g0 += G) {
    const int an = anchor_of(L, g0);
    int res[RQ_MAX_LOOPS], nres = 0;                 // this group's residual loops
    if (L->ref_chain) {
      nres = chain_order(L, g0, res);                // root outwards: each refers to the previous
    } else {
      for (int l = g0; l < g0 + G; ++l)
        if (l != an) res[nres++] = l;
    }
    // input index of loop l
    auto in_index = [&](int l) { return L->ref_bits ? l : (l < an ? l : l - 1); };
    rq::EncodeArgs a;
    std::memset(&a, 0, sizeof a);
    for (int s = 0; s < 2; ++s) {
      const uint16_t *base = static_cast<const uint16_t *>(ins[s]);
      a.side[s].ref = static_cast<const uint16_t *>(sides[s]->ref);
      for (int i = 0; i < nres; ++i) {
        const int l = res[i];
        a.side[s].xin[i] = base + (size_t)in_index(l) * loop_elems;
        a.side[s].codes[i] = static_cast<uint8_t *>(sides[s]->codes[l]);
        a.side[s].meta[i] = static_cast<uint32_t *>(sides[s]->meta[l]);
        a.side[s].alpha[i] = static_cast<uint16_t *>(sides[s]->alpha[l]);
      }
      if (L->ref_bits) {
        a.side[s].xin[nres] = base + (size_t)in_index(an) * loop_elems;
        a.side[s].codes[nres] = static_cast<uint8_t *>(sides[s]->codes[an]);
        a.side[s].meta[nres] = static_cast<uint32_t *>(sides[s]->meta[an]);
      }
    }
    for (int i = 0; i < nres; ++i) a.bits[i] = L->bits[res[i]];
    a.abits = L->ref_bits;
    a.agroup = anchor_group(L);
    a.alpha_mode = L->alpha_mode;
    a.chain = L->ref_chain;
    a.n_res = G - 1;
    a.bh = (int32_t)bh;
    a.cap = L->capacity;
    a.t0 = t0;
    a.n = n;
    a.group = L->group;
    a.rotate = L->rotate;
    a.rot_c = rot_const(L->head_dim);
    a.chunks = chunks;
    a.tasks_per_side = (int32_t)(bh * chunks);
    if (rq::launch_encode(a, L->head_dim, static_cast<hipStream_t>(hip_stream)) != hipSuccess)
      return RQ_ERR_DEVICE;
  }
  return RQ_OK;
}

int32_t rq_decode_splits(const rq_layout *L, int32_t n_ctx) {
  if (check_layout(L) != RQ_OK || n_ctx < 0 || n_ctx > L->capacity) return RQ_ERR_INVALID_ARG;
  if (n_ctx == 0) return 1;
  const int slots = decode_slots(L->head_dim);
  if (slots <= 0) return RQ_ERR_DEVICE;
  return auto_splits(L, n_ctx, slots, cu_count());
}

size_t rq_decode_workspace_bytes(const rq_layout *L, int32_t n_ctx, int32_t n_splits) {
  if (check_layout(L) != RQ_OK || n_ctx < 0 || n_ctx > L->capacity || n_splits < 0) return 0;
  int s = n_splits;
  if (s == 0) {
    s = rq_decode_splits(L, n_ctx);
    if (s <= 0) return 0;
  }
  if (s > n_ctx) s = n_ctx;
  return workspace_for(L, s);
}

}  // extern "C"

// Split-record scratch of rq_decode_attn_tail_noalloc: one copy per GPU,
// part of the library's code object.  On the host its name stands for the
// symbol only; its device address (per device) comes from
// hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[RQ_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the current device, looked up on the
// first call with that device current; nullptr on a HIP error.
void *scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

// workspace == nullptr with `noalloc`: the split records go to this
// device's scratch (workspace_bytes is then its size).
rq_status decode_impl(const rq_layout *L, const rq_cache *k, const rq_cache *v, const rq_tail *tail,
                      const void *q, uint32_t loop_mask, int32_t n_ctx, float sm_scale,
                      int32_t n_splits, float *out, void *workspace, size_t workspace_bytes,
                      void *hip_stream, bool noalloc = false) {
  rq_status st = check_layout(L);
  if (st != RQ_OK) return st;
  if (k == nullptr || v == nullptr) return RQ_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(out) || (!noalloc && !aligned16(workspace))) return RQ_ERR_INVALID_ARG;
  if (loop_mask == 0) return RQ_ERR_INVALID_ARG;
  if (L->n_loops < 32 && (loop_mask >> L->n_loops) != 0) return RQ_ERR_INVALID_ARG;
  const int n_tail = tail ? tail->n : 0;
  if (tail && (tail->n < 0 || tail->capacity < tail->n)) return RQ_ERR_INVALID_ARG;
  if (n_ctx < 0 || n_ctx > L->capacity || (int64_t)n_ctx + n_tail < 1) return RQ_ERR_INVALID_ARG;
  if (n_tail > 0 && (int64_t)L->batch * L->n_heads * tail->capacity > INT32_MAX) return RQ_ERR_UNSUPPORTED;
  if (!rows_fit_u32(L->capacity, L->head_dim) || (n_tail > 0 && !rows_fit_u32(tail->capacity, L->head_dim)))
    return RQ_ERR_UNSUPPORTED;
  if (!std::isfinite(sm_scale)) return RQ_ERR_INVALID_ARG;
  if (n_splits < 0 || (n_ctx > 0 && n_splits > n_ctx)) return RQ_ERR_INVALID_ARG;
  for (int l = 0; l < L->n_loops; ++l) {
    if (!((loop_mask >> l) & 1u)) continue;
    if (n_ctx > 0) {
      const int an = anchor_of(L, l);
      if (!ref_planes_ok(L, k, an) || !ref_planes_ok(L, v, an)) return RQ_ERR_INVALID_ARG;
      if (!is_anchor(L, l) && (!residual_planes_ok(k, l) || !residual_planes_ok(v, l)))
        return RQ_ERR_INVALID_ARG;
      if (L->ref_chain && !is_anchor(L, l)) {        // every link between the root and l
        int ord[RQ_MAX_LOOPS];
        const int nc = chain_order(L, (l / group_len(L)) * group_len(L), ord);
        for (int c = 0; c < nc && ord[c] != l; ++c)
          if (!residual_planes_ok(k, ord[c]) || !residual_planes_ok(v, ord[c])) return RQ_ERR_INVALID_ARG;
      }
    }
    if (n_tail > 0 && (!aligned16(tail->k[l]) || !aligned16(tail->v[l]))) return RQ_ERR_INVALID_ARG;
  }
  int S = 0, tps = 0;
  if (n_ctx > 0) {
    S = n_splits;
    if (S == 0) {
      S = rq_decode_splits(L, n_ctx);
      if (S <= 0) return RQ_ERR_DEVICE;
    }
    // every split non-empty
    tps = (n_ctx + S - 1) / S;
    S = (n_ctx + tps - 1) / tps;
  }
  if (workspace_bytes < workspace_for(L, S)) return RQ_ERR_WORKSPACE;

  rq::DecodeArgs a;
  std::memset(&a, 0, sizeof a);
  if (L->ref_bits == 0) {
    a.kref = static_cast<const uint16_t *>(k->ref);
    a.vref = static_cast<const uint16_t *>(v->ref);
  } else {
    a.ref_rotated = L->rotate;
  }
  a.agroup = anchor_group(L);
  a.q = static_cast<const uint16_t *>(q);
  a.ws = static_cast<float *>(workspace);
  a.out = out;
  a.bh = L->batch * L->n_heads;
  a.cap = L->capacity;
  a.n_ctx = n_ctx;
  a.n_splits = S;
  a.tps = tps;
  a.n_tail = n_tail;
  a.tcap = tail ? tail->capacity : 0;
  a.out_mask = loop_mask;
  decode_waves(S, a.bh, &a.wide, &a.waves8);
  // The BF16 tail is attended by the decode kernel: with one workgroup per
  // (b,h) (one split, or the wide form of two) by that workgroup, which
  // finishes the rows; with several splits each split takes an equal share
  // of the tail rows as more tokens of its own, so the merge kernel has no
  // tail to walk.  (Against the first split taking the whole tail, per-loop
  // calls with a 64-row tail: 6-9% faster at batch 1-2, 2k; 4-6% at batch 4,
  // 2k and 8k.)  A call over the tail alone runs the merge kernel only.
  a.tail_in = (n_tail > 0 && S > 0) ? 1 : 0;
  a.records = (S > 1 && !a.wide) ? 1 : 0;
  a.group = L->group;
  a.rotate = L->rotate;
  a.qscale = sm_scale * 1.4426950408889634f;   // exp(x) = exp2(x * log2(e))
  a.rot_c = L->rotate ? rot_const(L->head_dim) : 1.0f;

  const hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  const int G = group_len(L);
  if (launch_fault_injected()) return RQ_ERR_DEVICE;
  if (noalloc) {
    a.ws = static_cast<float *>(scratch_on_current_device());
    if (a.ws == nullptr) return RQ_ERR_DEVICE;
  }
  (void)hipGetLastError();
  for (int g0 = 0; g0 < L->n_loops; g0 += G) {
    const int ref_loop = anchor_of(L, g0);    // this group's reference / anchor
    int res[RQ_MAX_LOOPS], nres = 0;
    if (L->ref_chain) {
      // one pass over the chain from the farthest loop asked for to the root,
      // slots farthest first (each slot's reference is the next slot)
      int ord[RQ_MAX_LOOPS];
      const int nc = chain_order(L, g0, ord);
      int far = -1;
      for (int c = 0; c < nc; ++c)
        if ((loop_mask >> ord[c]) & 1u) far = c;
      for (int c = far; c >= 0; --c) res[nres++] = ord[c];
    } else {
      for (int l = g0; l < g0 + G; ++l)
        if (l != ref_loop && ((loop_mask >> l) & 1u)) res[nres++] = l;
    }
    bool want_ref = (loop_mask >> ref_loop) & 1u;
    if (nres == 0 && !want_ref) continue;
    // A chain pass whose only wanted output is its first slot (a call for
    // one loop) computes that slot alone; the links are read, not attended.
    int chain_mode = 0;
    if (L->ref_chain) {
      chain_mode = want_ref ? 1 : 2;
      for (int i = 1; i < nres; ++i)
        if ((loop_mask >> res[i]) & 1u) chain_mode = 1;
    }
    if (L->ref_bits) {
      a.kac = static_cast<const uint8_t *>(k->codes[ref_loop]);
      a.vac = static_cast<const uint8_t *>(v->codes[ref_loop]);
      a.kam = static_cast<const uint32_t *>(k->meta[ref_loop]);
      a.vam = static_cast<const uint32_t *>(v->meta[ref_loop]);
    }
    // Passes of at most kMaxRes residual loops; the first also computes the
    // reference loop.  Each pass reads the reference once.
    int done = 0;
    do {
      const int cnt = (nres - done) < rq::kMaxRes ? (nres - done) : rq::kMaxRes;
      for (int i = 0; i < rq::kMaxSlots; ++i) a.tk[i] = a.tv[i] = nullptr;
      for (int i = 0; i < cnt; ++i) {
        const int l = res[done + i];
        a.kc[i] = static_cast<const uint8_t *>(k->codes[l]);
        a.vc[i] = static_cast<const uint8_t *>(v->codes[l]);
        a.km[i] = static_cast<const uint32_t *>(k->meta[l]);
        a.vm[i] = static_cast<const uint32_t *>(v->meta[l]);
        a.ka[i] = static_cast<const uint16_t *>(k->alpha[l]);
        a.va[i] = static_cast<const uint16_t *>(v->alpha[l]);
        a.bits[i] = L->bits[l];
        a.qloop[i] = l;
        if (n_tail > 0) {
          a.tk[i] = static_cast<const uint16_t *>(tail->k[l]);
          a.tv[i] = static_cast<const uint16_t *>(tail->v[l]);
        }
      }
      if (want_ref) {
        a.qloop[cnt] = ref_loop;
        if (n_tail > 0) {
          a.tk[cnt] = static_cast<const uint16_t *>(tail->k[ref_loop]);
          a.tv[cnt] = static_cast<const uint16_t *>(tail->v[ref_loop]);
        }
      }
      hipError_t e;
      if (n_ctx > 0)
        e = rq::launch_decode(a, L->head_dim, cnt, want_ref, L->ref_bits, chain_mode, stream);
      else   // the tail alone: the merge kernel attends over it, no split records
        e = rq::launch_merge(a, L->head_dim, cnt, cnt + (want_ref ? 1 : 0), stream);
      if (e != hipSuccess) return RQ_ERR_DEVICE;
      want_ref = false;
      done += cnt;
    } while (done < nres);
  }
  return RQ_OK;
}

}  // namespace

extern "C" {

rq_status rq_decode_attn(const rq_layout *L, const rq_cache *k, const rq_cache *v, const void *q,
                         uint32_t loop_mask, int32_t n_ctx, float sm_scale, int32_t n_splits,
                         float *out, void *workspace, size_t workspace_bytes, void *hip_stream) {
  if (n_ctx < 1) return RQ_ERR_INVALID_ARG;
  return decode_impl(L, k, v, nullptr, q, loop_mask, n_ctx, sm_scale, n_splits, out, workspace,
                     workspace_bytes, hip_stream);
}

rq_status rq_decode_attn_tail(const rq_layout *L, const rq_cache *k, const rq_cache *v,
                              const rq_tail *tail, const void *q, uint32_t loop_mask,
                              int32_t n_ctx, float sm_scale, int32_t n_splits, float *out,
                              void *workspace, size_t workspace_bytes, void *hip_stream) {
  return decode_impl(L, k, v, tail, q, loop_mask, n_ctx, sm_scale, n_splits, out, workspace,
                     workspace_bytes, hip_stream);
}

rq_status rq_decode_attn_tail_noalloc(const rq_layout *L, const rq_cache *k, const rq_cache *v,
                                      const rq_tail *tail, const void *q, uint32_t loop_mask,
                                      int32_t n_ctx, float sm_scale, int32_t n_splits, float *out,
                                      void *hip_stream) {
  return decode_impl(L, k, v, tail, q, loop_mask, n_ctx, sm_scale, n_splits, out, nullptr,
                     RQ_NOALLOC_SCRATCH_BYTES, hip_stream, true);
}

rq_status rq_bf16_decode_attn(const rq_layout *L, void *const *k_loops, void *const *v_loops,
                              const void *q, uint32_t loop_mask, int32_t n_ctx, float sm_scale,
                              int32_t n_splits, float *out, void *workspace, size_t workspace_bytes,
                              void *hip_stream) {
  rq_status st = check_layout(L);
  if (st != RQ_OK) return st;
  if (k_loops == nullptr || v_loops == nullptr) return RQ_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(out) || !aligned16(workspace)) return RQ_ERR_INVALID_ARG;
  if (loop_mask == 0) return RQ_ERR_INVALID_ARG;
  if (L->n_loops < 32 && (loop_mask >> L->n_loops) != 0) return RQ_ERR_INVALID_ARG;
  if (n_ctx < 1 || n_ctx > L->capacity) return RQ_ERR_INVALID_ARG;
  if (!std::isfinite(sm_scale)) return RQ_ERR_INVALID_ARG;
  if (n_splits < 0 || n_splits > n_ctx) return RQ_ERR_INVALID_ARG;
  if (!rows_fit_u32(L->capacity, L->head_dim)) return RQ_ERR_UNSUPPORTED;
  for (int l = 0; l < L->n_loops; ++l)
    if (((loop_mask >> l) & 1u) && (!aligned16(k_loops[l]) || !aligned16(v_loops[l])))
      return RQ_ERR_INVALID_ARG;
  int S = n_splits;
  if (S == 0) {
    S = rq_decode_splits(L, n_ctx);
    if (S <= 0) return RQ_ERR_DEVICE;
  }
  if (workspace_bytes < workspace_for(L, S)) return RQ_ERR_WORKSPACE;
  const int tps = (n_ctx + S - 1) / S;
  S = (n_ctx + tps - 1) / tps;
  rq::DecodeArgs a;
  std::memset(&a, 0, sizeof a);
  a.bh = L->batch * L->n_heads;
  decode_waves(S, a.bh, &a.wide, &a.waves8);   // the same workgroup shapes as rq_decode_attn
  a.records = (S > 1 && !a.wide) ? 1 : 0;
  a.out_mask = 0xffffffffu;
  a.agroup = 32;
  a.ws = static_cast<float *>(workspace);
  a.out = out;
  a.q = static_cast<const uint16_t *>(q);
  a.cap = L->capacity;
  a.n_ctx = n_ctx;
  a.n_splits = S;
  a.tps = tps;
  a.group = 32;
  a.qscale = sm_scale * 1.4426950408889634f;
  a.rot_c = 1.0f;
  if (launch_fault_injected()) return RQ_ERR_DEVICE;
  (void)hipGetLastError();
  // every loop attends over its own BF16 cache: the reference-only kernel
  for (int l = 0; l < L->n_loops; ++l) {
    if (!((loop_mask >> l) & 1u)) continue;
    a.kref = static_cast<const uint16_t *>(k_loops[l]);
    a.vref = static_cast<const uint16_t *>(v_loops[l]);
    a.qloop[0] = l;
    if (rq::launch_decode(a, L->head_dim, 0, true, 0, false, static_cast<hipStream_t>(hip_stream)) !=
        hipSuccess)
      return RQ_ERR_DEVICE;
  }
  return RQ_OK;
}

rq_status rq_reconstruct(const rq_layout *L, const rq_cache *c, int32_t loop, int32_t t0, int32_t n,
                         float *out, void *hip_stream) {
  rq_status st = check_layout(L);
  if (st != RQ_OK) return st;
  if (loop < 0 || loop >= L->n_loops) return RQ_ERR_INVALID_ARG;
  const int ref_loop = anchor_of(L, loop);
  const bool anchor_loop = loop == ref_loop;
  if (anchor_loop && L->ref_bits == 0) return RQ_ERR_INVALID_ARG;   // the BF16 reference itself
  if (c == nullptr || !ref_planes_ok(L, c, ref_loop) || !aligned16(out)) return RQ_ERR_INVALID_ARG;
  if (!anchor_loop && !residual_planes_ok(c, loop)) return RQ_ERR_INVALID_ARG;
  if (t0 < 0 || n < 1 || (int64_t)t0 + n > L->capacity) return RQ_ERR_INVALID_ARG;
  rq::ReconArgs a;
  std::memset(&a, 0, sizeof a);
  if (L->ref_bits == 0) {
    a.ref = static_cast<const uint16_t *>(c->ref);
  } else {
    a.acodes = static_cast<const uint8_t *>(c->codes[ref_loop]);
    a.ameta = static_cast<const uint32_t *>(c->meta[ref_loop]);
  }
  a.abits = L->ref_bits;
  a.agroup = anchor_group(L);
  if (!anchor_loop) {
    a.codes = static_cast<const uint8_t *>(c->codes[loop]);
    a.meta = static_cast<const uint32_t *>(c->meta[loop]);
    a.alpha = static_cast<const uint16_t *>(c->alpha[loop]);
    a.bits = L->bits[loop];
    if (L->ref_chain) {                             // the links between the root and loop
      int ord[RQ_MAX_LOOPS];
      const int nc = chain_order(L, (loop / group_len(L)) * group_len(L), ord);
      for (int q = 0; q < nc && ord[q] != loop; ++q) {
        if (!residual_planes_ok(c, ord[q])) return RQ_ERR_INVALID_ARG;
        a.pcodes[a.npre] = static_cast<const uint8_t *>(c->codes[ord[q]]);
        a.pmeta[a.npre] = static_cast<const uint32_t *>(c->meta[ord[q]]);
        a.palpha[a.npre] = static_cast<const uint16_t *>(c->alpha[ord[q]]);
        a.pbits[a.npre] = L->bits[ord[q]];
        ++a.npre;
      }
    }
  }
  a.out = out;
  a.bh = L->batch * L->n_heads;
  a.cap = L->capacity;
  a.t0 = t0;
  a.n = n;
  a.group = L->group;
  a.rotate = L->rotate;
  a.rot_c = rot_const(L->head_dim);
  const int vpw = 64 / (L->head_dim / 8);
  a.chunks = (n + vpw - 1) / vpw;
  if ((int64_t)a.bh * a.chunks > INT32_MAX - 4) return RQ_ERR_UNSUPPORTED;
  if (launch_fault_injected()) return RQ_ERR_DEVICE;
  (void)hipGetLastError();
  return rq::launch_reconstruct(a, L->head_dim, static_cast<hipStream_t>(hip_stream)) == hipSuccess
             ? RQ_OK : RQ_ERR_DEVICE;
}

}  // extern "C"
