// Paged KV pool maintenance: workspace set-up, token write / read, stand-alone commit.
//
// Commit of the current position's KV into the preserved history follows the
// On-Demand Attention summary page ("Approach": the selected pass's current
// position KV is written into the full history). The tile byte order is the
// one documented in sparsekv.h.
#include <string.h>

#include "sk_internal.h"

namespace sk {

__device__ inline uint32_t k_off(int t, int d) { return (d >> 3) * 256 + t * 16 + (d & 7) * 2; }
__device__ inline uint32_t v_off(int t, int d) {
  return (d >> 5) * 1024 + (t >> 2) * 256 + (d & 15) * 16 + ((d >> 4) & 1) * 8 + (t & 3) * 2;
}

__global__ void ws_clear_kernel(uint32_t* p, size_t words) {
  size_t i = blockIdx.x * size_t(blockDim.x) + threadIdx.x;
  if (i < words) p[i] = 0u;
}

// One thread per (token, kv-head, 8-dim chunk). Direction: write (logical -> pool) or read.
template <bool kWrite>
__global__ __launch_bounds__(256) void kv_copy_kernel(sk_paged_kv kv, int request, int pos0, int count,
                                                      const uint16_t* __restrict__ k_src,
                                                      const uint16_t* __restrict__ v_src,
                                                      uint16_t* __restrict__ k_dst, uint16_t* __restrict__ v_dst,
                                                      int32_t* err) {
  const int Hkv = kv.num_kv_heads;
  int64_t gid = blockIdx.x * int64_t(blockDim.x) + threadIdx.x;
  int64_t total = int64_t(count) * Hkv * 16;
  if (gid >= total) return;
  int chunk = int(gid & 15);
  int64_t th = gid >> 4;
  int g = int(th % Hkv);
  int tok = int(th / Hkv);
  int pos = pos0 + tok;
  int lblock = pos / kBlock, t = pos % kBlock;
  int phys = kv.block_tables[int64_t(request) * kv.max_blocks + lblock];
  int64_t row = (int64_t(tok) * Hkv + g) * kHeadDim + chunk * 8;  // logical element index
  if (phys < 0 || phys >= kv.num_phys_blocks) {
    set_error(err, SK_DEVERR_BLOCK_ID);
    if (!kWrite) {
      *reinterpret_cast<u32x4*>(k_dst + row) = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(v_dst + row) = u32x4{0u, 0u, 0u, 0u};
    }
    return;
  }
  size_t tile = (size_t(phys) * Hkv + g) * kTileBytes;
  uint8_t* kt = reinterpret_cast<uint8_t*>(kv.k_pool) + tile;
  uint8_t* vt = reinterpret_cast<uint8_t*>(kv.v_pool) + tile;
  int d0 = chunk * 8;
  if (kWrite) {
    *reinterpret_cast<u32x4*>(kt + k_off(t, d0)) = *reinterpret_cast<const u32x4*>(k_src + row);
    u32x4 vv = *reinterpret_cast<const u32x4*>(v_src + row);
    uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<uint16_t*>(vt + v_off(t, d0 + i)) = uint16_t(w[i >> 1] >> ((i & 1) * 16));
  } else {
    *reinterpret_cast<u32x4*>(k_dst + row) = *reinterpret_cast<const u32x4*>(kt + k_off(t, d0));
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i)
      w[i >> 1] |= uint32_t(*reinterpret_cast<const uint16_t*>(vt + v_off(t, d0 + i))) << ((i & 1) * 16);
    *reinterpret_cast<u32x4*>(v_dst + row) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// Stand-alone commit: one thread per (request, kv-head, 8-dim chunk).
__global__ __launch_bounds__(256) void kv_append_kernel(sk_paged_kv kv, const uint16_t* __restrict__ k_new,
                                                        const uint16_t* __restrict__ v_new,
                                                        const int32_t* __restrict__ sel, int sel_value,
                                                        int32_t* err) {
  const int Hkv = kv.num_kv_heads;
  int64_t gid = blockIdx.x * int64_t(blockDim.x) + threadIdx.x;
  if (gid >= int64_t(kv.batch) * Hkv * 16) return;
  int chunk = int(gid & 15);
  int g = int((gid >> 4) % Hkv);
  int b = int((gid >> 4) / Hkv);
  if (sel && sel[b] != sel_value) return;
  int n = kv.seq_lens[b];
  if (n < 1 || n > kv.max_blocks * kBlock) {
    set_error(err, SK_DEVERR_SEQ_LEN);
    return;
  }
  int pos = n - 1;
  int phys = kv.block_tables[int64_t(b) * kv.max_blocks + pos / kBlock];
  if (phys < 0 || phys >= kv.num_phys_blocks) {
    set_error(err, SK_DEVERR_BLOCK_ID);
    return;
  }
  int t = pos % kBlock, d0 = chunk * 8;
  size_t tile = (size_t(phys) * Hkv + g) * kTileBytes;
  uint8_t* kt = reinterpret_cast<uint8_t*>(kv.k_pool) + tile;
  uint8_t* vt = reinterpret_cast<uint8_t*>(kv.v_pool) + tile;
  int64_t row = (int64_t(b) * Hkv + g) * kHeadDim + d0;
  *reinterpret_cast<u32x4*>(kt + k_off(t, d0)) = *reinterpret_cast<const u32x4*>(k_new + row);
  u32x4 vv = *reinterpret_cast<const u32x4*>(v_new + row);
  uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<uint16_t*>(vt + v_off(t, d0 + i)) = uint16_t(w[i >> 1] >> ((i & 1) * 16));
}

}  // namespace sk

using namespace sk;

extern "C" {

size_t sk_workspace_bytes(int32_t batch, int32_t num_q_heads) {
  if (batch < 1) batch = 1;
  if (num_q_heads < 1) num_q_heads = 1;
  return kPartialsOffset + partials_bytes(batch, num_q_heads);
}

int sk_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!ws) return SK_E_NULL;
  if (ws_bytes < kPartialsOffset) return SK_E_WORKSPACE;
  size_t words = kPartialsOffset / 4;
  hipLaunchKernelGGL(ws_clear_kernel, dim3(unsigned((words + 255) / 256)), dim3(256), 0, stream,
                     reinterpret_cast<uint32_t*>(ws), words);
  return launch_status(hipGetLastError());
}

int sk_workspace_error(const void* ws, int32_t* err_out, hipStream_t stream) {
  if (!ws || !err_out) return SK_E_NULL;
  hipError_t e = hipMemcpyAsync(err_out, ws, sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  return launch_status(e);
}

const char* sk_status_str(int status) {
  switch (status) {
    case SK_OK: return "ok";
    case SK_E_NULL: return "a required pointer is NULL";
    case SK_E_SHAPE: return "unsupported shape (head_dim must be 128, block_size 16, Hq/Hkv <= 16)";
    case SK_E_HEADS: return "num_q_heads is not a multiple of num_kv_heads";
    case SK_E_RANGE: return "a size or index argument is out of range";
    case SK_E_WORKSPACE: return "workspace too small";
    default: break;
  }
  if (status <= SK_E_LAUNCH_BASE) return "kernel launch failed (status = -(1000 + hipError_t))";
  return "unknown status";
}

static int kv_copy(sk_paged_kv kv, int32_t request, int32_t pos0, int32_t count, const void* k, const void* v,
                   void* ws, hipStream_t stream, bool write) {
  int st = check_kv(kv);
  if (st) return st;
  if (request < 0 || request >= kv.batch || pos0 < 0 || count < 0 ||
      int64_t(pos0) + count > int64_t(kv.max_blocks) * kBlock)
    return SK_E_RANGE;
  if (count == 0) return SK_OK;
  if (!k || !v) return SK_E_NULL;
  int32_t* err = reinterpret_cast<int32_t*>(ws);
  int64_t threads = int64_t(count) * kv.num_kv_heads * 16;
  dim3 grid(unsigned((threads + 255) / 256));
  if (write)
    hipLaunchKernelGGL(kv_copy_kernel<true>, grid, dim3(256), 0, stream, kv, request, pos0, count,
                       reinterpret_cast<const uint16_t*>(k), reinterpret_cast<const uint16_t*>(v),
                       (uint16_t*)nullptr, (uint16_t*)nullptr, err);
  else
    hipLaunchKernelGGL(kv_copy_kernel<false>, grid, dim3(256), 0, stream, kv, request, pos0, count,
                       (const uint16_t*)nullptr, (const uint16_t*)nullptr,
                       reinterpret_cast<uint16_t*>(const_cast<void*>(k)),
                       reinterpret_cast<uint16_t*>(const_cast<void*>(v)), err);
  return launch_status(hipGetLastError());
}

int sk_kv_write(sk_paged_kv kv, int32_t request, int32_t pos0, int32_t count, const void* k, const void* v,
                void* ws, hipStream_t stream) {
  return kv_copy(kv, request, pos0, count, k, v, ws, stream, true);
}

int sk_kv_read(sk_paged_kv kv, int32_t request, int32_t pos0, int32_t count, void* k_out, void* v_out,
               void* ws, hipStream_t stream) {
  return kv_copy(kv, request, pos0, count, k_out, v_out, ws, stream, false);
}

int sk_kv_append(sk_paged_kv kv, const void* k_new, const void* v_new, const int32_t* sel, int32_t sel_value,
                 void* ws, hipStream_t stream) {
  int st = check_kv(kv);
  if (st) return st;
  if (!k_new || !v_new) return SK_E_NULL;
  int64_t threads = int64_t(kv.batch) * kv.num_kv_heads * 16;
  hipLaunchKernelGGL(kv_append_kernel, dim3(unsigned((threads + 255) / 256)), dim3(256), 0, stream, kv,
                     reinterpret_cast<const uint16_t*>(k_new), reinterpret_cast<const uint16_t*>(v_new), sel,
                     sel_value, reinterpret_cast<int32_t*>(ws));
  return launch_status(hipGetLastError());
}

}  // extern "C"
