// Streaming-read probe: the measured bandwidth reference for the rooflines of the
// decode kernels. One launch of one workgroup per CU reads a buffer once: workgroup w
// streams its own contiguous range in rounds of 32 KiB, where each of its 8 waves reads
// 4 consecutive KiB with 16-byte non-temporal loads (a wave instruction reads 1 KiB
// contiguous, four independent loads per lane in flight). The words are folded into one
// XOR checksum per workgroup, which keeps the loads live and lets a test check that every
// word was read. Measured on MI355X, this pattern streams faster than a grid-stride loop,
// whose concurrent accesses all fall a fixed large stride apart.
#include "sk_internal.h"

namespace sk {
namespace {

constexpr int kProbeThreads = 512;
constexpr int kProbeLoads = 4;                                          // per lane per round
constexpr uint64_t kProbeRound = uint64_t(kProbeThreads) * kProbeLoads;  // 16-byte units (32 KiB)

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const u32x4* __restrict__ p, uint64_t n16,
                                                                    uint32_t* __restrict__ sink) {
  __shared__ uint32_t s_x[kProbeThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // range of this workgroup: whole rounds, the last range cut at the end of the buffer
  const uint64_t per = ((n16 + gridDim.x - 1) / gridDim.x + kProbeRound - 1) / kProbeRound * kProbeRound;
  const uint64_t begin = per * blockIdx.x;
  const uint64_t end = begin + per < n16 ? begin + per : n16;
  const uint64_t off = uint64_t(wave) * kProbeLoads * 64 + lane;
  u32x4 a = {0u, 0u, 0u, 0u};
  uint64_t base = begin;
  for (; base + kProbeRound <= end; base += kProbeRound) {
    u32x4 x[kProbeLoads];
#pragma unroll
    for (int c = 0; c < kProbeLoads; ++c) x[c] = __builtin_nontemporal_load(p + base + off + 64 * c);
#pragma unroll
    for (int c = 0; c < kProbeLoads; ++c) a ^= x[c];
  }
  if (base < end) {
#pragma unroll
    for (int c = 0; c < kProbeLoads; ++c) {
      const uint64_t i = base + off + 64 * c;
      if (i < end) a ^= __builtin_nontemporal_load(p + i);
    }
  }
  uint32_t x = (a.x ^ a.y) ^ (a.z ^ a.w);
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
  if (lane == 0) s_x[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int w = 0; w < kProbeThreads / 64; ++w) t ^= s_x[w];
    sink[blockIdx.x] = t;
  }
}

}  // namespace
}  // namespace sk

using namespace sk;

extern "C" {

int sk_stream_read(const void* data, uint64_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!sink || (bytes > 0 && !data)) return SK_E_NULL;
  if (bytes % 16 != 0 || reinterpret_cast<uintptr_t>(data) % 16 != 0) return SK_E_RANGE;
  hipLaunchKernelGGL(stream_read_kernel, dim3(SK_STREAM_READ_GRID), dim3(kProbeThreads), 0, stream,
                     reinterpret_cast<const u32x4*>(data), bytes / 16, sink);
  return launch_status(hipGetLastError());
}

}  // extern "C"
