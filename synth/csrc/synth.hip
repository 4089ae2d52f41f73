// Device side of the synthetic input streams (see synth/rng.py for the definition):
// SplitMix64 output per element index, centred sum of its four 16-bit fields, one
// float32 multiply, optional round-to-nearest-even to bf16. Bit-identical to the
// NumPy implementation. Also the per-step "feed" kernel that stands in for a model's
// projections: it writes the step's query / key / value candidates, recall inputs,
// scores and sequence lengths into fixed buffers, so a captured decode step can be
// replayed with new inputs every step.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ inline uint64_t splitmix_at(uint64_t key, uint64_t i) {
  uint64_t z = key + (i + 1ull) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ inline float normal_at(uint64_t key, uint64_t i, float scale) {
  uint64_t r = splitmix_at(key, i);
  int c = int(r & 0xFFFFull) + int((r >> 16) & 0xFFFFull) + int((r >> 32) & 0xFFFFull) + int(r >> 48) - 131070;
  return __fmul_rn(float(c), scale);
}

__device__ inline uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__global__ void fill_f32_kernel(float* out, int64_t count, uint64_t key, int64_t index0, float scale) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < count; i += int64_t(gridDim.x) * blockDim.x)
    out[i] = normal_at(key, uint64_t(index0 + i), scale);
}

__global__ void fill_bf16_kernel(uint16_t* out, int64_t count, uint64_t key, int64_t index0, float scale) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < count; i += int64_t(gridDim.x) * blockDim.x)
    out[i] = bf16_rne(normal_at(key, uint64_t(index0 + i), scale));
}

struct FeedParams {
  int32_t* state;  // [0] step counter (free-running), [1] ticket
  int32_t* seq_lens;
  const int32_t* H0;
  int B, L, P, Hq, Hkv, num_steps;
  uint64_t key_q, key_k, key_v, key_x, key_score;
  float scale;
  float* q_out;       // [L][P][B][Hq][128]
  uint16_t* k_out;    // [L][P][B][Hkv][128]
  uint16_t* v_out;
  int x_dim;
  float* x_out;       // [B][x_dim] or null
  const float* sched; // [num_steps][B] or null
  float* score_out;   // [B] or null
  const int32_t* decl_table;  // [num_steps][B][4] or null
  int32_t* decl_out;  // [B][4]
  const int32_t* token_table;  // [num_steps][B] or null
  int32_t* token_out;  // [B]
};

// Element indices stay below 2^31 for every workload here (the host checks), so the
// decomposition uses 32-bit arithmetic.
constexpr int kFeedThreads = 1024;  // 16 waves per block: the hash chains are latency-bound
__global__ __launch_bounds__(kFeedThreads) void feed_kernel(FeedParams F) {
  __shared__ int s_last;
  const int t = F.state[0] % F.num_steps;
  const int rq = F.Hq * 128, rkv = F.Hkv * 128;
  const int nq = F.L * F.P * F.B * rq;
  const int nkv = F.L * F.P * F.B * rkv;
  const int nx = F.x_out ? F.B * F.x_dim : 0;
  const int total = nq + nkv + nx + F.B;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += gridDim.x * blockDim.x) {
    if (i < nq) {
      const int e = i % rq;
      int r = i / rq;
      const int b = r % F.B;
      r /= F.B;
      const int p = r % F.P;
      const int l = r / F.P;
      const int pe = (l == 0) ? 0 : p;
      const uint64_t gi = uint64_t(((int64_t(t) * F.L + l) * F.P + pe) * F.B + b) * rq + e;
      F.q_out[i] = normal_at(F.key_q, gi, F.scale);
    } else if (i < nq + nkv) {
      const int j = i - nq;
      const int e = j % rkv;
      int r = j / rkv;
      const int b = r % F.B;
      r /= F.B;
      const int p = r % F.P;
      const int l = r / F.P;
      const int pe = (l == 0) ? 0 : p;
      const uint64_t gi = uint64_t(((int64_t(t) * F.L + l) * F.P + pe) * F.B + b) * rkv + e;
      F.k_out[j] = bf16_rne(normal_at(F.key_k, gi, F.scale));
      F.v_out[j] = bf16_rne(normal_at(F.key_v, gi, F.scale));
    } else if (i < nq + nkv + nx) {
      const int j = i - nq - nkv;
      F.x_out[j] = normal_at(F.key_x, uint64_t(int64_t(t) * F.B * F.x_dim + j), F.scale);
    } else {
      const int b = i - nq - nkv - nx;
      F.seq_lens[b] = F.H0[b] + t + 1;
      if (F.score_out)
        F.score_out[b] = F.sched ? F.sched[int64_t(t) * F.B + b]
                                 : normal_at(F.key_score, uint64_t(int64_t(t) * F.B + b), F.scale);
      if (F.decl_out)
        for (int k = 0; k < 4; ++k) F.decl_out[4 * b + k] = F.decl_table[(int64_t(t) * F.B + b) * 4 + k];
      if (F.token_out) F.token_out[b] = F.token_table[int64_t(t) * F.B + b];
    }
  }
  // every block has read state[0] above; the last block to arrive advances the step
  // (no fence: the outputs only need to be visible after the kernel ends)
  __syncthreads();
  if (threadIdx.x == 0) s_last = (atomicAdd(&F.state[1], 1) == int(gridDim.x) - 1);
  __syncthreads();
  if (s_last && threadIdx.x == 0) {
    F.state[1] = 0;
    F.state[0] = F.state[0] + 1;
  }
}

__global__ void set_step_kernel(int32_t* state, int32_t t) {
  state[0] = t;
  state[1] = 0;
}

int status(hipError_t e) { return e == hipSuccess ? 0 : -(1000 + int(e)); }

}  // namespace

extern "C" {

int synth_fill_f32(float* out, int64_t count, uint64_t key, int64_t index0, float scale, hipStream_t s) {
  if (count <= 0) return 0;
  int64_t blocks = (count + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_f32_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, out, count, key, index0, scale);
  return status(hipGetLastError());
}

int synth_fill_bf16(uint16_t* out, int64_t count, uint64_t key, int64_t index0, float scale, hipStream_t s) {
  if (count <= 0) return 0;
  int64_t blocks = (count + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_bf16_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, out, count, key, index0, scale);
  return status(hipGetLastError());
}

int synth_feed(int32_t* state, int32_t* seq_lens, const int32_t* H0, int B, int L, int P, int Hq, int Hkv,
               int num_steps, uint64_t key_q, uint64_t key_k, uint64_t key_v, uint64_t key_x, uint64_t key_score,
               float scale, float* q_out, uint16_t* k_out, uint16_t* v_out, int x_dim, float* x_out,
               const float* sched, float* score_out, const int32_t* decl_table, int32_t* decl_out,
               const int32_t* token_table, int32_t* token_out, hipStream_t s) {
  const int64_t total = int64_t(L) * P * B * (Hq + Hkv) * 128 + (x_out ? int64_t(B) * x_dim : 0) + B;
  if (total >= (int64_t(1) << 31) || B < 1 || num_steps < 1) return -4;
  FeedParams F{state, seq_lens, H0, B, L, P, Hq, Hkv, num_steps, key_q, key_k, key_v, key_x, key_score, scale,
               q_out, k_out, v_out, x_dim, x_out, sched, score_out, decl_table, decl_out, token_table, token_out};
  // at most 256 blocks (one per CU), so the last-block ticket that advances the step stays cheap
  int64_t blocks = (total + kFeedThreads - 1) / kFeedThreads;
  if (blocks > 256) blocks = 256;
  hipLaunchKernelGGL(feed_kernel, dim3(unsigned(blocks)), dim3(kFeedThreads), 0, s, F);
  return status(hipGetLastError());
}

int synth_set_step(int32_t* state, int32_t t, hipStream_t s) {
  hipLaunchKernelGGL(set_step_kernel, dim3(1), dim3(1), 0, s, state, t);
  return status(hipGetLastError());
}

}  // extern "C"
