// Internal definitions shared by the libsparsekv translation units (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sparsekv.h"

namespace sk {

constexpr int kHeadDim = 128;
constexpr int kBlock = 16;
constexpr int kTileBytes = kBlock * kHeadDim * 2;  // one (block, kv-head) tile of K or V
constexpr int kMaxGroup = 16;                      // Hq / Hkv handled by one MFMA column block
constexpr int kMaxBatch = 1024;

// Workspace header: [0] error word, [64..] ticket counters, then split partials.
constexpr size_t kWsHeaderBytes = 256;
constexpr int kMaxTickets = kMaxBatch * 16;        // (request, kv-head) pairs
constexpr size_t kTicketBytes = size_t(kMaxTickets) * 4;
constexpr size_t kPartialsOffset = kWsHeaderBytes + kTicketBytes;
// Decode launches use at most this many workgroups, hence work items (split partials),
// plus one per (request, kv-head) for rounding; every item stores G * (128 + 2) floats.
constexpr int kTargetItems = 1024;
constexpr int kWavesPerWG = 8;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

inline int launch_status(hipError_t e) { return e == hipSuccess ? SK_OK : SK_E_LAUNCH_BASE - int(e); }

inline int check_kv(const sk_paged_kv& kv) {
  if (!kv.k_pool || !kv.v_pool || !kv.block_tables || !kv.seq_lens) return SK_E_NULL;
  if (kv.head_dim != kHeadDim || kv.block_size != kBlock) return SK_E_SHAPE;
  if (kv.batch < 1 || kv.batch > kMaxBatch || kv.num_kv_heads < 1 || kv.num_q_heads < 1 ||
      kv.max_blocks < 1 || kv.num_phys_blocks < 1)
    return SK_E_RANGE;
  if (kv.num_q_heads % kv.num_kv_heads != 0) return SK_E_HEADS;
  if (kv.num_q_heads / kv.num_kv_heads > kMaxGroup) return SK_E_SHAPE;
  if (int64_t(kv.batch) * kv.num_kv_heads > kMaxTickets) return SK_E_RANGE;
  if (int64_t(kv.max_blocks) * kBlock > INT32_MAX / 2) return SK_E_RANGE;
  return SK_OK;
}

inline size_t partials_bytes(int batch, int num_q_heads) {
  // A decode launch has at most kTargetItems + batch * Hkv work items, each storing
  // G * (128 + 2) floats; G <= min(Hq, 16) and batch * Hkv * G == batch * Hq.
  size_t g_max = size_t(num_q_heads < kMaxGroup ? num_q_heads : kMaxGroup);
  return (size_t(kTargetItems) * g_max + size_t(batch) * size_t(num_q_heads)) * (kHeadDim + 2) * 4;
}

__device__ inline void set_error(int32_t* err, int bits) {
  if (err) atomicOr(err, bits);
}

}  // namespace sk
