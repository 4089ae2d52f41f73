// Recall head, gate and per-request view selection.
//
// On-Demand Attention summary page, "Approach": a recall head maps the three inputs
// available before any global read (previous selected hidden state, current token
// embedding, current Local final hidden state) to one scalar q_t, and the step is
// recomputed with Full attention when q_t > theta (theta = 0 by default).
// "Developer perspective": the head is evaluated in FP32 inside the same GPU
// execution flow as the Local pass and the conditional Full pass, so the decision
// never goes back to the host.
//
// The head here is a two-layer MLP, q = <w2, GELU(W1 x + b1)> + b2 (exact-erf GELU).
// It is a GEMV: each group of four waves keeps one row of W1 (in_dim fp32, a quarter
// each) in registers and dots it with every request's x; no matrix cores are used. Per-workgroup
// partial sums are published with device-coherent stores and added in a fixed order by
// the last workgroup (atomic ticket), so q is deterministic.
#include <math.h>

#include "sk_internal.h"

namespace sk {
namespace {

constexpr int kRecallMaxBatch = 64;
constexpr int kRecallMaxIn = 65536;
// Measured at 6144 -> 512, batch 1 (per call in a graph): 16 waves per workgroup, 4 per
// row (128 workgroups) took 6.6 us; one row per wave in 4-wave workgroups 9.7 us; other
// splits (1, 2 or 8 waves per row; 32 to 512 workgroups, i.e. fewer parallel loads or more
// ticket atomics) 7.0-11.8 us.
constexpr int kRecallWaves = 16;     // waves per workgroup
constexpr int kRecallRowWaves = 4;   // waves sharing one W1 row (each a contiguous quarter of its columns)
constexpr int kRecallRows = kRecallWaves / kRecallRowWaves;  // W1 rows per workgroup
constexpr int kRecallMaxParts = 16384;  // workgroups x batch partial sums the last workgroup stages

__device__ inline float gelu_erf(float a) { return 0.5f * a * (1.0f + erff(a * 0.70710678118654752f)); }

// CHUNKS > 0: the wave's part of its W1 row (CHUNKS float4 per lane) stays in registers
// across requests. CHUNKS == 0: long rows are streamed from memory once per request.
template <int CHUNKS>
__global__ __launch_bounds__(64 * kRecallWaves) void recall_kernel(
    const float* __restrict__ x, const float* __restrict__ W1, const float* __restrict__ b1,
    const float* __restrict__ w2, const float* __restrict__ b2, int B, int in_dim, int hidden, float theta,
    float* __restrict__ q_out, int32_t* __restrict__ gate_out, float* partials, uint32_t* ticket) {
  __shared__ float s_d[kRecallWaves][kRecallMaxBatch];
  __shared__ float s_part[kRecallMaxParts];
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row0 = blockIdx.x * kRecallRows;
  const int row = row0 + wave / kRecallRowWaves;
  // this wave's columns of the row, in float4 units: [c_begin, c_end)
  const int n4 = in_dim / 4;
  const int per = (n4 + kRecallRowWaves - 1) / kRecallRowWaves;
  const int c_begin = (wave % kRecallRowWaves) * per, c_end = min(n4, c_begin + per);
  const f32x4* wrow = reinterpret_cast<const f32x4*>(W1 + size_t(row < hidden ? row : 0) * in_dim);
  // the rows' bias and output weight, requested with the row so that they are in
  // registers when the row sums are finished
  float b1r[kRecallRows], w2r[kRecallRows];
#pragma unroll
  for (int r = 0; r < kRecallRows; ++r) {
    const bool ok = row0 + r < hidden;
    b1r[r] = ok ? b1[row0 + r] : 0.f;
    w2r[r] = ok ? w2[row0 + r] : 0.f;
  }
  constexpr int R = CHUNKS > 0 ? CHUNKS : 1;
  f32x4 w[R];
  if (CHUNKS > 0) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int c = c_begin + lane + 64 * i;
      w[i] = (row < hidden && c < c_end) ? wrow[c] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  for (int b = 0; b < B; ++b) {
    float dot = 0.f;
    const f32x4* xb = reinterpret_cast<const f32x4*>(x + size_t(b) * in_dim);
    if (CHUNKS > 0) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int c = c_begin + lane + 64 * i;
        if (c < c_end) {
          f32x4 v = xb[c];
          dot += w[i].x * v.x + w[i].y * v.y + w[i].z * v.z + w[i].w * v.w;
        }
      }
    } else if (row < hidden) {
      for (int c = c_begin + lane; c < c_end; c += 64) {
        f32x4 v = xb[c], u = wrow[c];
        dot += u.x * v.x + u.y * v.y + u.z * v.z + u.w * v.w;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) dot += __shfl_xor(dot, off);
    if (lane == 0) s_d[wave][b] = dot;
  }
  __syncthreads();
  // Row dots from their parts, then the workgroup's sum of w2 * GELU(W1 x + b1) over its
  // rows. Workgroup sums are published with device-coherent stores; once they have
  // completed, one thread takes the ticket. The last workgroup loads every workgroup's
  // sums in one round of device-coherent loads into LDS and adds them in a fixed order.
  for (int b = tid; b < B; b += blockDim.x) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < kRecallRows; ++r) {
      float d = 0.f;
#pragma unroll
      for (int h = 0; h < kRecallRowWaves; ++h) d += s_d[r * kRecallRowWaves + h][b];
      if (row0 + r < hidden) s += w2r[r] * gelu_erf(d + b1r[r]);
    }
    __hip_atomic_store(&partials[size_t(blockIdx.x) * B + b], s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's stores have completed
  __syncthreads();
  if (tid == 0) s_last = (atomicAdd(ticket, 1u) == gridDim.x - 1);
  __syncthreads();
  if (!s_last) return;
  const int nwg = int(gridDim.x), total = nwg * B;
  for (int e = tid; e < total; e += blockDim.x)
    s_part[e] = __hip_atomic_load(&partials[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  // wave w adds requests w, w + kRecallWaves, ...: lane u the workgroups u, u + 64, ...
  // in order, then a butterfly over the lanes (a fixed order: deterministic)
  for (int b = wave; b < B; b += kRecallWaves) {
    float s = 0.f;
    for (int i = lane; i < nwg; i += 64) s += s_part[i * B + b];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) {
      const float q = s + b2[0];
      q_out[b] = q;
      gate_out[b] = (q > theta) ? 1 : 0;
    }
  }
  if (tid == 0) *ticket = 0u;
}

__global__ void gate_scores_kernel(const float* __restrict__ scores, int B, float theta,
                                   const int32_t* __restrict__ fallback, int32_t* __restrict__ out) {
  int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) out[b] = (scores[b] > theta) ? 1 : (fallback ? fallback[b] : 0);
}

// Bits of mask word w of one request: block blk is kept when it holds a visible position
// (blk < nb) and the declared mode keeps it.
__device__ inline uint32_t keep_word(int mode, int fb, int fe, int ob, int first_local, int nb, int w) {
  uint32_t bits = 0u;
  for (int i = 0; i < 32; ++i) {
    const int blk = 32 * w + i;
    bool keep = false;
    if (blk < nb) {
      if (mode == SK_DA_GLOBAL) keep = true;
      else if (mode == SK_DA_FOCUS) keep = (blk >= fb && blk < fe) || blk >= ob;
      else if (mode == SK_DA_LOCAL) keep = blk >= first_local;
    }
    bits |= uint32_t(keep) << i;
  }
  return bits;
}

__device__ inline int visible_blocks(const sk_paged_kv& kv, int n) {
  return (n >= 1 && n <= kv.max_blocks * kBlock) ? (n + kBlock - 1) / kBlock : 0;
}

__global__ void keep_mask_kernel(const int32_t* __restrict__ decl, sk_paged_kv kv, int local_tokens,
                                 uint32_t* __restrict__ mask) {
  const int words_row = (kv.max_blocks + 31) / 32;
  int64_t gid = blockIdx.x * int64_t(blockDim.x) + threadIdx.x;
  if (gid >= int64_t(kv.batch) * words_row) return;
  const int b = int(gid / words_row), w = int(gid % words_row);
  const int n = kv.seq_lens[b];
  const int first_local = (n > local_tokens ? n - local_tokens : 0) / kBlock;
  mask[gid] = keep_word(decl[4 * b], decl[4 * b + 1], decl[4 * b + 2], decl[4 * b + 3], first_local,
                        visible_blocks(kv, n), w);
}

// One workgroup per request: thread 0 advances the request's declaration parser by this
// step's token, then the workgroup writes the keep mask of the new declaration.
__global__ __launch_bounds__(256) void declare_kernel(const int32_t* __restrict__ tokens, int32_t* __restrict__ state,
                                                      const int32_t* __restrict__ segments, int num_segments,
                                                      const int32_t* __restrict__ output_begin, sk_da_tags tags,
                                                      sk_paged_kv kv, int local_tokens, int32_t* __restrict__ decl,
                                                      uint32_t* __restrict__ mask) {
  __shared__ int s_decl[4];
  const int b = blockIdx.x;
  if (threadIdx.x == 0) {
    int* st = state + 4 * b;
    int mode = st[0], fb = st[1], fe = st[2], pending = st[3];
    const int tok = tokens[b];
    if (tok == tags.global_tag) {
      mode = SK_DA_GLOBAL;
      pending = 0;
    } else if (tok == tags.local_tag) {
      mode = SK_DA_LOCAL;
      pending = 0;
    } else if (tok == tags.focus_tag) {
      pending = 1;
    } else if (pending) {
      pending = 0;
      const int64_t k = int64_t(tok) - tags.segment_base;
      if (k >= 0 && k < num_segments) {
        const int64_t e = (int64_t(b) * num_segments + k) * 2;
        const int begin = max(segments[e], 0), end = segments[e + 1];
        mode = SK_DA_FOCUS;
        fb = begin / kBlock;
        fe = (end > begin) ? (end + kBlock - 1) / kBlock : fb;
      }
    }
    st[0] = mode;
    st[1] = fb;
    st[2] = fe;
    st[3] = pending;
    const int ob = output_begin[b];
    decl[4 * b] = mode;
    decl[4 * b + 1] = fb;
    decl[4 * b + 2] = fe;
    decl[4 * b + 3] = ob;
    s_decl[0] = mode;
    s_decl[1] = fb;
    s_decl[2] = fe;
    s_decl[3] = ob;
  }
  __syncthreads();
  const int words_row = (kv.max_blocks + 31) / 32;
  const int n = kv.seq_lens[b];
  const int first_local = (n > local_tokens ? n - local_tokens : 0) / kBlock;
  const int nb = visible_blocks(kv, n);
  if (mask)
    for (int w = threadIdx.x; w < words_row; w += blockDim.x)
      mask[int64_t(b) * words_row + w] = keep_word(s_decl[0], s_decl[1], s_decl[2], s_decl[3], first_local, nb, w);
}

template <int CHUNKS>
int launch_recall(const float* x, const float* W1, const float* b1, const float* w2, const float* b2, int B,
                  int in_dim, int hidden, float theta, float* q_out, int32_t* gate_out, void* ws,
                  hipStream_t stream) {
  int nwg = (hidden + kRecallRows - 1) / kRecallRows;
  float* partials = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + kPartialsOffset);
  uint32_t* ticket = reinterpret_cast<uint32_t*>(ws) + 1;
  hipLaunchKernelGGL(recall_kernel<CHUNKS>, dim3(nwg), dim3(64 * kRecallWaves), 0, stream, x, W1, b1, w2, b2, B,
                     in_dim, hidden, theta, q_out, gate_out, partials, ticket);
  return launch_status(hipGetLastError());
}

}  // namespace
}  // namespace sk

using namespace sk;

extern "C" {

int oda_recall_score(const float* x, const float* W1, const float* b1, const float* w2, const float* b2,
                     int32_t batch, int32_t in_dim, int32_t hidden, float theta, float* q_out, int32_t* gate_out,
                     void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!x || !W1 || !b1 || !w2 || !b2 || !q_out || !gate_out || !ws) return SK_E_NULL;
  if (batch < 1 || batch > kRecallMaxBatch || in_dim < 4 || in_dim > kRecallMaxIn || (in_dim % 4) || hidden < 1)
    return SK_E_RANGE;
  const size_t parts = size_t((hidden + kRecallRows - 1) / kRecallRows) * batch;
  if (parts > size_t(kRecallMaxParts)) return SK_E_RANGE;
  size_t need = kPartialsOffset + parts * 4;
  if (ws_bytes < need) return SK_E_WORKSPACE;
  const int per = (in_dim / 4 + kRecallRowWaves - 1) / kRecallRowWaves;  // float4 of a wave's part of a row
  const int chunks = (per + 63) / 64;                                     // per lane
  if (chunks <= 8) return launch_recall<8>(x, W1, b1, w2, b2, batch, in_dim, hidden, theta, q_out, gate_out, ws, stream);
  if (chunks <= 12) return launch_recall<12>(x, W1, b1, w2, b2, batch, in_dim, hidden, theta, q_out, gate_out, ws, stream);
  if (chunks <= 16) return launch_recall<16>(x, W1, b1, w2, b2, batch, in_dim, hidden, theta, q_out, gate_out, ws, stream);
  return launch_recall<0>(x, W1, b1, w2, b2, batch, in_dim, hidden, theta, q_out, gate_out, ws, stream);
}

int oda_gate_scores(const float* scores, int32_t batch, float theta, const int32_t* fallback, int32_t* out,
                    hipStream_t stream) {
  if (!scores || !out) return SK_E_NULL;
  if (batch < 1) return SK_E_RANGE;
  hipLaunchKernelGGL(gate_scores_kernel, dim3((batch + 255) / 256), dim3(256), 0, stream, scores, batch, theta,
                     fallback, out);
  return launch_status(hipGetLastError());
}

int da_keep_mask(const int32_t* decl, sk_paged_kv kv, int32_t local_tokens, uint32_t* keep_mask,
                 hipStream_t stream) {
  int st = check_kv(kv);
  if (st) return st;
  if (!decl || !keep_mask) return SK_E_NULL;
  if (local_tokens < 0) return SK_E_RANGE;
  int64_t threads = int64_t(kv.batch) * ((kv.max_blocks + 31) / 32);
  hipLaunchKernelGGL(keep_mask_kernel, dim3(unsigned((threads + 255) / 256)), dim3(256), 0, stream, decl, kv,
                     local_tokens, keep_mask);
  return launch_status(hipGetLastError());
}

int da_declare(const int32_t* tokens, int32_t* state, const int32_t* segments, int32_t num_segments,
               const int32_t* output_begin, sk_da_tags tags, sk_paged_kv kv, int32_t local_tokens, int32_t* decl,
               uint32_t* keep_mask, hipStream_t stream) {
  int st = check_kv(kv);
  if (st) return st;
  if (!tokens || !state || !output_begin || !decl) return SK_E_NULL;
  if (num_segments < 0 || local_tokens < 0) return SK_E_RANGE;
  if (num_segments > 0 && !segments) return SK_E_NULL;
  hipLaunchKernelGGL(declare_kernel, dim3(unsigned(kv.batch)), dim3(256), 0, stream, tokens, state, segments,
                     num_segments, output_begin, tags, kv, local_tokens, decl, keep_mask);
  return launch_status(hipGetLastError());
}

}  // extern "C"
